// C ABI of libsra: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before the first launch of a call.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_err;
thread_local int g_time_which = 0;
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;
thread_local sra::Tuning g_tune;

sra_status fail(sra_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool debug_sync() {
  static const int v = [] {
    const char* e = getenv("SRA_DEBUG");
    return e ? atoi(e) : 0;
  }();
  return v != 0;
}

sra_status hip_done(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return fail(SRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(SRA_ERR_HIP, "%s (sync): %s", what, hipGetErrorString(e));
  }
  return SRA_OK;
}

#define SRA_TRY(expr)                   \
  do {                                  \
    const sra_status st_ = (expr);      \
    if (st_ != SRA_OK) return st_;      \
  } while (0)

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(int dtype) { return dtype == SRA_BF16 ? 2 : 4; }

sra_status check_dtype(int dtype) {
  if (dtype != SRA_BF16 && dtype != SRA_F32) return fail(SRA_ERR_INVALID_ARG, "dtype %d is not SRA_BF16 or SRA_F32", dtype);
  return SRA_OK;
}

sra_status check_ptr(const void* p, bool needed, const char* name) {
  if (!needed) return SRA_OK;
  if (!p) return fail(SRA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!al16(p)) return fail(SRA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return SRA_OK;
}

sra_status check_nm(int64_t rows, int64_t cols, int n, int m) {
  if (rows < 0 || cols < 0) return fail(SRA_ERR_INVALID_ARG, "negative shape");
  if (n < 1 || m < n || (m > 4 && m != 8)) return fail(SRA_ERR_INVALID_ARG, "invalid N:M %d:%d", n, m);
  if (!((n == 2 && m == 4) || (n == 1 && m == 2) || (n == 2 && m == 8)))
    return fail(SRA_ERR_UNSUPPORTED, "only 2:4, 1:2 and 2:8 are implemented (got %d:%d)", n, m);
  if (cols % 32) return fail(SRA_ERR_UNSUPPORTED, "grouped dimension %lld is not a multiple of 32", (long long)cols);
  return SRA_OK;
}

// 1:2 weights run on the 2:4 kernels: each group of four columns holds one entry of each pair, and
// the metadata becomes the 2:4 encoding when every odd field gains 2 (word | 0x88888888).
constexpr uint32_t kMeta12To24 = 0x88888888u;
bool is12(const sra_sparse* S) { return S->format == SRA_FMT_NM && S->n == 1 && S->m == 2; }
bool is28(const sra_sparse* S) { return S->format == SRA_FMT_NM && S->n == 2 && S->m == 8; }
// a 2:8 weight in its streaming layout (sra_nm_tile)
bool is28t(const sra_sparse* S) { return S->format == SRA_FMT_NM_TILED && S->n == 2 && S->m == 8; }
// 2:8 weights for 16 tokens or fewer run the 2:8 decode kernel (one streaming pass over the
// weight, fragments expanded to dense in registers).  Otherwise bf16 N:M weights on the dense-MFMA
// engine run the expanded-fragment products, and 2:8 weights run on the 2:4 kernels: every group
// of four columns of a 2:8 row holds at most two kept entries, so the call rewrites the weight as
// a 2:4 one (the same entries plus +0.0 fillers) in its workspace first.  With few tokens a
// product reads the weight once, and that rewrite would cost more than it saves.
bool use_dec28(const sra_sparse* S, int64_t T) { return (is28(S) || is28t(S)) && T <= 16; }
bool use_xp(const sra_sparse* S, int64_t T) {
  if (S->format != SRA_FMT_NM && S->format != SRA_FMT_NM_TILED) return false;
  return S->dtype == SRA_BF16 && sra::tuning().engine == SRA_ENGINE_DENSE_MFMA && !use_dec28(S, T);
}
// (a 2:8 weight in the streaming layout is rewritten as canonical 2:4 above 16 tokens on either
// engine: the dense engine then runs the expanded-fragment product on that 2:4 form)
bool is28_on24(const sra_sparse* S, int64_t T) {
  return (is28(S) && !use_dec28(S, T) && !use_xp(S, T)) || (is28t(S) && T > 16);
}
size_t meta_bytes(const sra_sparse* S) {
  return (size_t)S->rows * (size_t)sra_nm_meta_words(S->cols, S->n, S->m) * 4;
}

sra_status check_sparse(const sra_sparse* S, const char* name) {
  if (!S) return fail(SRA_ERR_INVALID_ARG, "%s descriptor is NULL", name);
  SRA_TRY(check_dtype(S->dtype));
  if (S->rows < 0 || S->cols < 0) return fail(SRA_ERR_INVALID_ARG, "%s has a negative shape", name);
  const bool any = S->rows > 0 && S->cols > 0;
  if (S->format == SRA_FMT_NM) {
    SRA_TRY(check_nm(S->rows, S->cols, S->n, S->m));
    if (S->m == 8 && S->dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "%s: 2:8 is bf16 only", name);
    SRA_TRY(check_ptr(S->values, any, "values"));
    SRA_TRY(check_ptr(S->meta, any, "meta"));
  } else if (S->format == SRA_FMT_NM_TILED) {
    SRA_TRY(check_nm(S->rows, S->cols, S->n, S->m));
    if (S->n != 2 || (S->m != 4 && S->m != 8))
      return fail(SRA_ERR_UNSUPPORTED, "%s: the streaming layout is 2:4 or 2:8 only", name);
    if (S->dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "%s: the streaming layout is bf16 only", name);
    SRA_TRY(check_ptr(S->values, any, "values"));
    SRA_TRY(check_ptr(S->meta, any, "meta"));
  } else if (S->format == SRA_FMT_ELL) {
    if (S->cols > 32767) return fail(SRA_ERR_INVALID_ARG, "%s: ELL needs cols <= 32767", name);
    if (S->k < 1 || S->k > S->cols) return fail(SRA_ERR_INVALID_ARG, "%s: need 1 <= k <= cols", name);
    if (S->rows * (int64_t)S->k > INT32_MAX) return fail(SRA_ERR_UNSUPPORTED, "%s: rows*k exceeds int32", name);
    SRA_TRY(check_ptr(S->values, any, "values"));
    SRA_TRY(check_ptr(S->index, any, "index"));
  } else if (S->format == SRA_FMT_CSR) {
    if (S->cols > 32767) return fail(SRA_ERR_INVALID_ARG, "%s: CSR column ids are int16 (cols <= 32767)", name);
    if (S->nnz < 0 || S->nnz > INT32_MAX) return fail(SRA_ERR_INVALID_ARG, "%s: bad nnz", name);
    SRA_TRY(check_ptr(S->row_ptr, S->rows > 0, "row_ptr"));
    SRA_TRY(check_ptr(S->values, S->nnz > 0, "values"));
    SRA_TRY(check_ptr(S->index, S->nnz > 0, "index"));
  } else if (S->format == SRA_FMT_FFI_TILED) {
    if (S->dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "%s: the tiled fixed fan-in format is bf16 only", name);
    if (S->cols > 32767) return fail(SRA_ERR_INVALID_ARG, "%s: tiled fixed fan-in needs cols <= 32767", name);
    if (S->nnz < 0 || S->nnz >= ((int64_t)1 << 29)) return fail(SRA_ERR_INVALID_ARG, "%s: bad entry capacity (nnz)", name);
    SRA_TRY(check_ptr(S->values, S->nnz > 0, "values"));
    SRA_TRY(check_ptr(S->meta, true, "meta"));
  } else {
    return fail(SRA_ERR_INVALID_ARG, "%s: unknown format %d", name, S->format);
  }
  return SRA_OK;
}

// Bump allocation inside the caller's workspace (256-byte aligned pieces).
struct Arena {
  size_t used = 0;
  size_t take(size_t bytes) {
    const size_t off = used;
    used += (bytes + 255) & ~(size_t)255;
    return off;
  }
};

sra::F32Sparse f32_view(const sra_sparse* S) {
  sra::F32Sparse v{};
  v.format = S->format;
  v.rows = S->rows;
  v.cols = S->cols;
  v.vals = (const uint32_t*)S->values;
  v.meta = S->meta;
  v.meta_stride = S->format == SRA_FMT_NM ? sra_nm_meta_words(S->cols, S->n, S->m) : 0;
  v.idx = S->index;
  v.row_ptr = S->row_ptr;
  v.k = S->k;
  return v;
}

// ---------------------------------------------------------------- forward plan
struct FwdPlan {
  size_t u_off = 0, u64_off = 0, gemm_off = 0, ffi_off = 0, meta_off = 0, v24_off = 0, total = 0;
  bool own_u = false;
};

sra_status validate_fwd(const sra_sparse* Ws, int64_t T, int32_t r) {
  SRA_TRY(check_sparse(Ws, "Ws"));
  if (Ws->format == SRA_FMT_CSR) return fail(SRA_ERR_INVALID_ARG, "forward takes an N:M or ELL weight, not CSR");
  if (Ws->format == SRA_FMT_FFI_TILED && T > 0 && (Ws->cols == 0 || Ws->cols % 64 != 0))
    return fail(SRA_ERR_UNSUPPORTED, "the tiled fixed fan-in product needs K %% 64 == 0 and K > 0 (K = %lld)",
                (long long)Ws->cols);
  if (T < 0) return fail(SRA_ERR_INVALID_ARG, "T < 0");
  if (Ws->format == SRA_FMT_NM_TILED && !is28t(Ws) && !sra::spmm24_tiled_ok(Ws->cols, T))
    return fail(SRA_ERR_UNSUPPORTED, "the streaming 2:4 layout needs K %% 128 == 0 above 16 tokens (T = %lld)", (long long)T);
  if (Ws->format == SRA_FMT_NM_TILED && Ws->cols == 0)
    return fail(SRA_ERR_UNSUPPORTED, "bf16 2:4 forward needs K > 0");
  if (r < 0 || r > 256) return fail(SRA_ERR_UNSUPPORTED, "rank %d outside [0, 256]", r);
  if (Ws->format == SRA_FMT_NM && Ws->dtype == SRA_BF16 && Ws->cols == 0)
    return fail(SRA_ERR_UNSUPPORTED, "bf16 2:4 forward needs K > 0");
  if (use_xp(Ws, T) && T > 0 && !sra::spmm_xp_ok(Ws->cols))
    return fail(SRA_ERR_UNSUPPORTED, "%s products need K %% 128 == 0 (K = %lld)",
                is28(Ws) ? "2:8" : "dense-MFMA 2:4", (long long)Ws->cols);
  return SRA_OK;
}

size_t fwd_bytes(const sra_sparse* Ws, int64_t T, int32_t r, bool own_u, FwdPlan* plan) {
  Arena a;
  FwdPlan p;
  p.own_u = own_u && r > 0 && Ws->dtype == SRA_BF16;
  if (p.own_u) p.u_off = a.take((size_t)T * r * 4);
  if (Ws->dtype == SRA_F32 && r > 0) p.u64_off = a.take((size_t)T * r * 8);
  if (Ws->dtype == SRA_BF16) {
    size_t g = r > 0 ? sra::adapter_rows_ws(T, Ws->cols, r) : 0;
    if (use_xp(Ws, T))
      g = std::max(g, sra::spmm_xp_ws(Ws->rows, Ws->cols, T));
    else if (Ws->format == SRA_FMT_NM || Ws->format == SRA_FMT_NM_TILED)
      g = std::max(g, sra::spmm24_ws(Ws->rows, Ws->cols, T));
    p.gemm_off = a.take(g);
    if (Ws->format == SRA_FMT_ELL)
      p.ffi_off = a.take(sra::spmm_ffi_ws(Ws->rows, Ws->cols, T, Ws->rows * Ws->k));
  }
  if (is12(Ws)) p.meta_off = a.take(meta_bytes(Ws));  // the 2:4 encoding of the metadata
  if (is28_on24(Ws, T)) {  // the 2:4 form of a 2:8 weight (one metadata word per 32 columns in both)
    p.meta_off = a.take(meta_bytes(Ws));
    p.v24_off = a.take((size_t)Ws->rows * (size_t)(Ws->cols / 2) * 2);
  }

  p.total = a.used;
  if (plan) *plan = p;
  return p.total;
}

// ---------------------------------------------------------------- backward plan
struct BwdPlan {
  bool need_du = false, need_u = false, own_du = false, own_u = false;
  size_t u_off = 0, du_off = 0, u64_off = 0, du64_off = 0, gemm_off = 0, spmm_off = 0, total = 0;
  size_t wt_off = 0, vtu_off = 0, vtdu_off = 0;  // packed B^T, split U^T (dB), split dU^T (dA)
  size_t at_off = 0;                             // packed A^T (dX epilogue)
  size_t meta_off = 0;                           // 1:2 (or 2:8) metadata in the 2:4 encoding
  size_t v24_off = 0;                            // 2:8 values in the 2:4 layout
};

sra_status validate_bwd(const sra_sparse* P, int64_t T, int32_t r, uint32_t flags) {
  SRA_TRY(check_sparse(P, "P"));
  if (P->format == SRA_FMT_ELL)
    return fail(SRA_ERR_INVALID_ARG, "backward takes the double-pruned N:M weight, the CSR transpose or its tiled form");
  if (P->format == SRA_FMT_NM_TILED && !is28t(P) && (flags & SRA_GRAD_DX) && !sra::spmm24_tiled_ok(P->cols, T))
    return fail(SRA_ERR_UNSUPPORTED, "the streaming 2:4 layout needs N %% 128 == 0 above 16 tokens (T = %lld)", (long long)T);
  if (P->format == SRA_FMT_NM_TILED && P->cols == 0 && (flags & SRA_GRAD_DX))
    return fail(SRA_ERR_UNSUPPORTED, "bf16 2:4 backward needs N > 0");
  if (P->format == SRA_FMT_FFI_TILED && (flags & SRA_GRAD_DX) && T > 0 && (P->cols == 0 || P->cols % 64 != 0))
    return fail(SRA_ERR_UNSUPPORTED, "the tiled fixed fan-in dX needs N %% 64 == 0 and N > 0 (N = %lld)",
                (long long)P->cols);
  if (T < 0) return fail(SRA_ERR_INVALID_ARG, "T < 0");
  if (r < 0 || r > 256) return fail(SRA_ERR_UNSUPPORTED, "rank %d outside [0, 256]", r);
  if (flags & ~15u) return fail(SRA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (P->format == SRA_FMT_NM && P->dtype == SRA_BF16 && (flags & SRA_GRAD_DX) && P->cols == 0)
    return fail(SRA_ERR_UNSUPPORTED, "bf16 2:4 dX needs N > 0");
  if (use_xp(P, T) && (flags & SRA_GRAD_DX) && T > 0 && !sra::spmm_xp_ok(P->cols))
    return fail(SRA_ERR_UNSUPPORTED, "%s dX needs N %% 128 == 0 (N = %lld)",
                is28(P) ? "2:8" : "dense-MFMA 2:4", (long long)P->cols);
  return SRA_OK;
}

// dB (over dY, V = U in three parts) and dA (over X, V = dU in three parts, stored transposed) as
// jobs of the merged adapter-gradient launch; pointers are filled in by the caller.
int grad_jobs(sra::AdapterGrad* jobs, bool db, bool da, int64_t N, int64_t K) {
  int n = 0;
  if (db) {
    jobs[n] = sra::AdapterGrad{};
    jobs[n].M = N;
    jobs[n].parts = 3;
    ++n;
  }
  if (da) {
    jobs[n] = sra::AdapterGrad{};
    jobs[n].M = K;
    jobs[n].parts = 3;
    jobs[n].out_t = true;
    ++n;
  }
  return n;
}

size_t bwd_bytes(const sra_sparse* P, int64_t T, int32_t r, uint32_t flags, bool have_u,
                 bool have_du, BwdPlan* plan) {
  BwdPlan p;
  const int64_t K = P->rows, N = P->cols;
  const bool dx = flags & SRA_GRAD_DX, da = flags & SRA_GRAD_DA, db = flags & SRA_GRAD_DB;
  const bool dx_ad = dx && !(flags & SRA_DX_NO_ADAPTER);
  p.need_du = r > 0 && (dx_ad || da || have_du);
  p.need_u = r > 0 && db;
  Arena a;
  if (is12(P) && dx) p.meta_off = a.take(meta_bytes(P));
  if (is28_on24(P, T) && dx) {
    p.meta_off = a.take(meta_bytes(P));
    p.v24_off = a.take((size_t)P->rows * (size_t)(P->cols / 2) * 2);
  }
  if (P->dtype == SRA_F32) {  // fp32: U and dU stay fp64; U is always recomputed
    if (p.need_u) p.u64_off = a.take((size_t)T * r * 8);
    if (p.need_du) p.du64_off = a.take((size_t)T * r * 8);
    p.total = a.used;
    if (plan) *plan = p;
    return p.total;
  }
  p.own_du = p.need_du && !have_du;
  p.own_u = p.need_u && !have_u;
  if (p.own_u) p.u_off = a.take((size_t)T * r * 4);
  if (p.own_du) p.du_off = a.take((size_t)T * r * 4);
  if (p.need_du) p.wt_off = a.take(sra::adapter_wt_bytes(N, r));
  if (dx_ad) p.at_off = a.take(sra::adapter_at_bytes(K, r));
  if (db && r > 0) p.vtu_off = a.take(sra::adapter_vt_bytes(T, r, 3));
  if (da && r > 0) p.vtdu_off = a.take(sra::adapter_vt_bytes(T, r, 3));  // dU (fp32) split for dA
  if (P->dtype == SRA_BF16 && r > 0) {
    size_t g = 0;
    if (p.own_u) g = std::max(g, sra::adapter_rows_ws(T, K, r));
    if (p.need_du) g = std::max(g, sra::adapter_rows_ws(T, N, r));
    if (db) g = std::max(g, sra::adapter_cols_ws(T, N, r));
    if (da) g = std::max(g, sra::adapter_cols_ws(T, K, r));
    sra::AdapterGrad jobs[2];
    const int nj = grad_jobs(jobs, db, da, N, K);
    g = std::max(g, sra::adapter_grads_ws(jobs, nj, T, r));
    p.gemm_off = a.take(g);
  }
  if (P->dtype == SRA_BF16 && use_xp(P, T) && dx)
    p.spmm_off = a.take(sra::spmm_xp_ws(K, N, T));
  else if (P->dtype == SRA_BF16 && (P->format == SRA_FMT_NM || P->format == SRA_FMT_NM_TILED) && dx)
    p.spmm_off = a.take(sra::spmm24_ws(K, N, T));
  if (P->dtype == SRA_BF16 && P->format == SRA_FMT_CSR && dx)
    p.spmm_off = a.take(sra::spmm_ffi_ws(K, N, T, P->nnz));
  p.total = a.used;
  if (plan) *plan = p;
  return p.total;
}

// Every host check of a backward call except the workspace: shapes, flags, pointers.  Fills the
// workspace plan for the U / dU_out choices of the call.
sra_status check_bwd_args(const sra_sparse* P, const void* dY, const void* X, int64_t T,
                          const float* U, const void* A, const void* B, int32_t r, uint32_t flags,
                          const void* dX, const float* dA, const float* dB, const float* dU_out,
                          BwdPlan* plan) {
  SRA_TRY(validate_bwd(P, T, r, flags));
  const int64_t K = P->rows, N = P->cols;
  const bool fdx = flags & SRA_GRAD_DX, fda = (flags & SRA_GRAD_DA) && r > 0,
             fdb = (flags & SRA_GRAD_DB) && r > 0;
  const bool dx_ad = fdx && !(flags & SRA_DX_NO_ADAPTER) && r > 0;
  bwd_bytes(P, T, r, flags, U != nullptr, dU_out != nullptr, plan);
  const bool any = T > 0;
  SRA_TRY(check_ptr(dY, any && N > 0 && (fdx || plan->need_du || fdb), "dY"));
  const bool recompute_u = plan->own_u || (P->dtype == SRA_F32 && plan->need_u);
  SRA_TRY(check_ptr(X, any && K > 0 && (fda || recompute_u), "X"));
  SRA_TRY(check_ptr(A, any && r > 0 && K > 0 && (dx_ad || recompute_u), "A"));
  SRA_TRY(check_ptr(B, any && r > 0 && N > 0 && plan->need_du, "B"));
  SRA_TRY(check_ptr(dX, fdx && any && K > 0, "dX"));
  SRA_TRY(check_ptr(dA, fda && K > 0, "dA"));
  SRA_TRY(check_ptr(dB, fdb && N > 0, "dB"));
  if (U) SRA_TRY(check_ptr(U, true, "U"));
  if (dU_out) SRA_TRY(check_ptr(dU_out, true, "dU_out"));
  return SRA_OK;
}

}  // namespace

namespace sra {
const Tuning& tuning() { return g_tune; }

bool take_timing(int which, hipEvent_t* start, hipEvent_t* stop) {
  if (g_time_which == 0 || g_time_which != which) return false;
  *start = g_time_start;
  *stop = g_time_stop;
  g_time_which = 0;
  return true;
}
}  // namespace sra

extern "C" {

sra_status sra_time_next_kernel(int32_t which, void* start, void* stop) {
  if (which == 0) {
    g_time_which = 0;
    return SRA_OK;
  }
  if (which < SRA_KERNEL_COMPRESS || which > SRA_KERNEL_NM_UPDATE)
    return fail(SRA_ERR_INVALID_ARG, "unknown kernel class %d", which);
  if (!start || !stop) return fail(SRA_ERR_INVALID_ARG, "start and stop events are required");
  g_time_which = which;
  g_time_start = (hipEvent_t)start;
  g_time_stop = (hipEvent_t)stop;
  return SRA_OK;
}


sra_status sra_set_tuning(int32_t key, int32_t value) {
  switch (key) {
    case SRA_TUNE_RESET: g_tune = sra::Tuning{}; return SRA_OK;
    case SRA_TUNE_SPMM_CONFIG:
      if (value < 0 || value > 99) return fail(SRA_ERR_INVALID_ARG, "SpMM configuration %d out of range", value);
      g_tune.spmm_cfg = value;
      return SRA_OK;
    case SRA_TUNE_SPMM_SPLITS:
      if (value < -2 || value == -1 || value > 64) return fail(SRA_ERR_INVALID_ARG, "splits %d out of range", value);
      g_tune.spmm_splits = value;
      return SRA_OK;
    case SRA_TUNE_SPMM_FUSE:
      if (value != 0 && value != 1) return fail(SRA_ERR_INVALID_ARG, "fuse must be 0 or 1");
      g_tune.spmm_fuse = value;
      return SRA_OK;
    case SRA_TUNE_ENGINE:
      if (value != SRA_ENGINE_SMFMAC && value != SRA_ENGINE_DENSE_MFMA)
        return fail(SRA_ERR_INVALID_ARG, "unknown engine %d", value);
      g_tune.engine = value;
      return SRA_OK;
    case SRA_TUNE_DECODE_ROWS:
      if (value != 0 && value != 3 && value != 4 && value != 9)
        return fail(SRA_ERR_INVALID_ARG, "decode row tiles must be 0, 3, 4 or 9");
      g_tune.decode_rows = value;
      return SRA_OK;
    case SRA_TUNE_ROWS_SLICES:
    case SRA_TUNE_GRADS_SLICES:
      if (value < 0 || value > 1024) return fail(SRA_ERR_INVALID_ARG, "slices %d out of range", value);
      (key == SRA_TUNE_ROWS_SLICES ? g_tune.rows_slices : g_tune.grads_slices) = value;
      return SRA_OK;
    default: return fail(SRA_ERR_INVALID_ARG, "unknown tuning key %d", key);
  }
}

int32_t sra_abi_version(void) { return SRA_ABI_VERSION; }

const char* sra_last_error(void) { return g_err.c_str(); }

int64_t sra_nm_meta_words(int64_t cols, int32_t n, int32_t m) {
  if (m <= 0 || n <= 0 || cols < 0) return 0;
  if (m == 8) return (cols / 8 + 3) / 4;  // one byte per 8-column group
  const int64_t fields = cols / m * n;
  return (fields + 15) / 16;
}

sra_status sra_compress(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t n,
                        int32_t m, sra_sparse* out, void* stream) {
  SRA_TRY(check_dtype(dtype));
  SRA_TRY(check_nm(rows, cols, n, m));
  if (m == 8 && dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "2:8 is bf16 only");
  if (!out) return fail(SRA_ERR_INVALID_ARG, "out descriptor is NULL");
  const bool any = rows > 0 && cols > 0;
  SRA_TRY(check_ptr(W, any, "W"));
  SRA_TRY(check_ptr(out->values, any, "out->values"));
  SRA_TRY(check_ptr(out->meta, any, "out->meta"));
  out->format = SRA_FMT_NM;
  out->dtype = dtype;
  out->rows = rows;
  out->cols = cols;
  out->n = n;
  out->m = m;
  const hipStream_t s = (hipStream_t)stream;
  if (m == 8) {
    return hip_done(sra::launch_compress28((const uint16_t*)W, rows, cols, (uint16_t*)out->values,
                                           out->meta, s), s, "compress 2:8");
  }
  if (n == 1)
    return hip_done(sra::launch_compress12(dtype, W, rows, cols, out->values, out->meta, s), s, "compress 1:2");
  return hip_done(sra::launch_compress24(dtype, W, rows, cols, out->values, out->meta, s), s, "compress");
}

sra_status sra_double_prune(const sra_sparse* Ws, sra_sparse* P, void* stream) {
  SRA_TRY(check_sparse(Ws, "Ws"));
  if (Ws->format != SRA_FMT_NM) return fail(SRA_ERR_INVALID_ARG, "double_prune needs an N:M weight");
  SRA_TRY(check_nm(Ws->cols, Ws->rows, Ws->n, Ws->m));  // the second prune groups along rows
  if (!P) return fail(SRA_ERR_INVALID_ARG, "P descriptor is NULL");
  const bool any = Ws->rows > 0 && Ws->cols > 0;
  SRA_TRY(check_ptr(P->values, any, "P->values"));
  SRA_TRY(check_ptr(P->meta, any, "P->meta"));
  P->format = SRA_FMT_NM;
  P->dtype = Ws->dtype;
  P->rows = Ws->cols;
  P->cols = Ws->rows;
  P->n = Ws->n;
  P->m = Ws->m;
  const hipStream_t s = (hipStream_t)stream;
  if (is28(Ws))
    return hip_done(sra::launch_double_prune28((const uint16_t*)Ws->values, Ws->meta, Ws->rows, Ws->cols,
                                               (uint16_t*)P->values, P->meta, s),
                    s, "double_prune 2:8");
  if (is12(Ws))
    return hip_done(sra::launch_double_prune12(Ws->dtype, Ws->values, Ws->meta, Ws->rows, Ws->cols,
                                               P->values, P->meta, s),
                    s, "double_prune 1:2");
  return hip_done(sra::launch_double_prune24(Ws->dtype, Ws->values, Ws->meta, Ws->rows, Ws->cols,
                                             P->values, P->meta, s),
                  s, "double_prune");
}

sra_status sra_compress_pair(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t n,
                             int32_t m, sra_sparse* Ws, sra_sparse* P, void* stream) {
  SRA_TRY(check_dtype(dtype));
  SRA_TRY(check_nm(rows, cols, n, m));
  SRA_TRY(check_nm(cols, rows, n, m));  // the second prune groups along rows
  if (m == 8) return fail(SRA_ERR_UNSUPPORTED, "compress_pair: 2:8 runs as sra_compress + sra_double_prune");
  if (!Ws || !P) return fail(SRA_ERR_INVALID_ARG, "output descriptor is NULL");
  const bool any = rows > 0 && cols > 0;
  SRA_TRY(check_ptr(W, any, "W"));
  SRA_TRY(check_ptr(Ws->values, any, "Ws->values"));
  SRA_TRY(check_ptr(Ws->meta, any, "Ws->meta"));
  SRA_TRY(check_ptr(P->values, any, "P->values"));
  SRA_TRY(check_ptr(P->meta, any, "P->meta"));
  Ws->format = P->format = SRA_FMT_NM;
  Ws->dtype = P->dtype = dtype;
  Ws->rows = rows;
  Ws->cols = cols;
  P->rows = cols;
  P->cols = rows;
  Ws->n = P->n = n;
  Ws->m = P->m = m;
  const hipStream_t s = (hipStream_t)stream;
  if (n == 1) {  // 1:2: the two passes (the one-pass kernel ranks groups of four)
    SRA_TRY(hip_done(sra::launch_compress12(dtype, W, rows, cols, Ws->values, Ws->meta, s), s, "compress 1:2"));
    return hip_done(sra::launch_double_prune12(dtype, Ws->values, Ws->meta, rows, cols, P->values, P->meta, s),
                    s, "double_prune 1:2");
  }
  return hip_done(sra::launch_compress_pair24(dtype, W, rows, cols, Ws->values, Ws->meta, P->values,
                                              P->meta, s),
                  s, "compress_pair");
}

sra_status sra_compress_pair_tiled(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t n,
                                   int32_t m, sra_sparse* Ws, sra_sparse* P, void* stream) {
  SRA_TRY(check_dtype(dtype));
  SRA_TRY(check_nm(rows, cols, n, m));
  SRA_TRY(check_nm(cols, rows, n, m));
  if (dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "the streaming 2:4 layout is bf16 only");
  if (n != 2 || m != 4) return fail(SRA_ERR_UNSUPPORTED, "the streaming layout is 2:4 only");
  if (rows % 128 || cols % 128)
    return fail(SRA_ERR_UNSUPPORTED, "compress_pair_tiled needs rows and cols that are multiples of 128");
  if (!Ws || !P) return fail(SRA_ERR_INVALID_ARG, "output descriptor is NULL");
  const bool any = rows > 0 && cols > 0;
  SRA_TRY(check_ptr(W, any, "W"));
  SRA_TRY(check_ptr(Ws->values, any, "Ws->values"));
  SRA_TRY(check_ptr(Ws->meta, any, "Ws->meta"));
  SRA_TRY(check_ptr(P->values, any, "P->values"));
  SRA_TRY(check_ptr(P->meta, any, "P->meta"));
  Ws->format = P->format = SRA_FMT_NM_TILED;
  Ws->dtype = P->dtype = dtype;
  Ws->rows = rows;
  Ws->cols = cols;
  P->rows = cols;
  P->cols = rows;
  Ws->n = P->n = n;
  Ws->m = P->m = m;
  const hipStream_t s = (hipStream_t)stream;
  return hip_done(sra::launch_compress_pair24_tiled((const uint16_t*)W, rows, cols, Ws->values, Ws->meta,
                                                    P->values, P->meta, s),
                  s, "compress_pair_tiled");
}

sra_status sra_masked_weight_grad(const sra_sparse* S, const void* row_act, const void* col_act,
                                  int64_t T, void* out_values, void* stream) {
  if (!S) return fail(SRA_ERR_INVALID_ARG, "S descriptor is NULL");
  SRA_TRY(check_dtype(S->dtype));
  if (S->format != SRA_FMT_NM) return fail(SRA_ERR_INVALID_ARG, "masked_weight_grad needs a canonical N:M matrix");
  SRA_TRY(check_nm(S->rows, S->cols, S->n, S->m));
  if (S->dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "masked_weight_grad is bf16 only");
  if (is28(S)) return fail(SRA_ERR_UNSUPPORTED, "masked_weight_grad is 2:4 and 1:2 only");
  if (S->rows % 8) return fail(SRA_ERR_UNSUPPORTED, "masked_weight_grad needs rows %% 8 == 0");
  if (T < 0) return fail(SRA_ERR_INVALID_ARG, "T < 0");
  if (!sra::sddmm24_fits(S->rows, S->cols, T))
    return fail(SRA_ERR_UNSUPPORTED, "masked_weight_grad needs T*rows and T*cols below 2^30 elements");
  const bool any = S->rows > 0 && S->cols > 0;
  SRA_TRY(check_ptr(S->meta, any, "meta"));
  SRA_TRY(check_ptr(out_values, any, "out_values"));
  SRA_TRY(check_ptr(row_act, any && T > 0, "row_act"));
  SRA_TRY(check_ptr(col_act, any && T > 0, "col_act"));
  const hipStream_t s = (hipStream_t)stream;
  return hip_done(sra::launch_sddmm24_bf16((const uint16_t*)row_act, (const uint16_t*)col_act, S->meta,
                                           is12(S) ? kMeta12To24 : 0u, S->rows, S->cols, T,
                                           (uint16_t*)out_values, s),
                  s, "masked_weight_grad");
}

sra_status sra_nm_axpby(const void* a_values, float beta, const void* b_values, float gamma,
                        void* out_values, int64_t n_values, int32_t dtype, void* stream) {
  SRA_TRY(check_dtype(dtype));
  if (n_values < 0) return fail(SRA_ERR_INVALID_ARG, "n_values < 0");
  SRA_TRY(check_ptr(a_values, n_values > 0, "a_values"));
  SRA_TRY(check_ptr(b_values, n_values > 0, "b_values"));
  SRA_TRY(check_ptr(out_values, n_values > 0, "out_values"));
  const hipStream_t s = (hipStream_t)stream;
  return hip_done(sra::launch_nm_axpby(dtype, a_values, beta, b_values, gamma, out_values, n_values, s),
                  s, "nm_axpby");
}

sra_status sra_nm_tile_bytes(int64_t rows, int64_t cols, int32_t n, int32_t m, size_t* value_bytes,
                             size_t* meta_bytes) {
  SRA_TRY(check_nm(rows, cols, n, m));
  if (n != 2 || (m != 4 && m != 8)) return fail(SRA_ERR_UNSUPPORTED, "the streaming layout is 2:4 or 2:8 only");
  if (!value_bytes || !meta_bytes) return fail(SRA_ERR_INVALID_ARG, "size pointers are NULL");
  if (m == 8)
    sra::nm28_tile_bytes(rows, cols, value_bytes, meta_bytes);
  else
    sra::nm_tile_bytes(rows, cols, value_bytes, meta_bytes);
  return SRA_OK;
}

sra_status sra_nm_tile(const sra_sparse* Ws, sra_sparse* out, void* stream) {
  SRA_TRY(check_sparse(Ws, "Ws"));
  if (Ws->format != SRA_FMT_NM) return fail(SRA_ERR_INVALID_ARG, "nm_tile needs a canonical N:M weight");
  if (Ws->dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "the streaming layout is bf16 only");
  if (is12(Ws)) return fail(SRA_ERR_UNSUPPORTED, "the streaming layout is 2:4 or 2:8 only");
  if (!out) return fail(SRA_ERR_INVALID_ARG, "out descriptor is NULL");
  const bool any = Ws->rows > 0 && Ws->cols > 0;
  SRA_TRY(check_ptr(out->values, any, "out values"));
  SRA_TRY(check_ptr(out->meta, any, "out meta"));
  out->format = SRA_FMT_NM_TILED;
  out->dtype = Ws->dtype;
  out->rows = Ws->rows;
  out->cols = Ws->cols;
  out->n = Ws->n;
  out->m = Ws->m;
  const hipStream_t s = (hipStream_t)stream;
  if (is28(Ws))
    return hip_done(sra::launch_nm_tile28_bf16((const uint16_t*)Ws->values, Ws->meta, Ws->rows, Ws->cols,
                                               out->values, out->meta, s), s, "nm_tile 2:8");
  return hip_done(sra::launch_nm_tile_bf16((const uint16_t*)Ws->values, Ws->meta, Ws->rows, Ws->cols,
                                           out->values, out->meta, s), s, "nm_tile");
}

sra_status sra_compress_ffi(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t k,
                            sra_sparse* out, void* stream) {
  SRA_TRY(check_dtype(dtype));
  if (rows < 0 || cols < 1 || cols > 32767) return fail(SRA_ERR_INVALID_ARG, "need rows >= 0 and 1 <= cols <= 32767");
  if (k < 1 || k > cols) return fail(SRA_ERR_INVALID_ARG, "need 1 <= k <= cols (k = %d)", k);
  if (rows > UINT32_MAX / 2) return fail(SRA_ERR_UNSUPPORTED, "too many rows");
  if (!out) return fail(SRA_ERR_INVALID_ARG, "out descriptor is NULL");
  SRA_TRY(check_ptr(W, rows > 0, "W"));
  SRA_TRY(check_ptr(out->values, rows > 0, "out->values"));
  SRA_TRY(check_ptr(out->index, rows > 0, "out->index"));
  out->format = SRA_FMT_ELL;
  out->dtype = dtype;
  out->rows = rows;
  out->cols = cols;
  out->k = k;
  const hipStream_t s = (hipStream_t)stream;
  return hip_done(sra::launch_compress_ffi(dtype, W, rows, cols, k, out->values, out->index, s), s,
                  "compress_ffi");
}

sra_status sra_ffi_transpose_workspace(int64_t rows, int64_t cols, int32_t k, size_t* bytes) {
  if (!bytes) return fail(SRA_ERR_INVALID_ARG, "bytes is NULL");
  if (rows < 0 || cols < 1 || cols > 32767 || k < 1 || k > cols) return fail(SRA_ERR_INVALID_ARG, "bad ELL shape");
  *bytes = sra::ffi_transpose_ws(rows, cols);
  return SRA_OK;
}

sra_status sra_ffi_transpose(const sra_sparse* Ws, sra_sparse* WsT, void* ws, size_t ws_bytes,
                             void* stream) {
  SRA_TRY(check_sparse(Ws, "Ws"));
  if (Ws->format != SRA_FMT_ELL) return fail(SRA_ERR_INVALID_ARG, "ffi_transpose needs an ELL weight");
  if (!WsT) return fail(SRA_ERR_INVALID_ARG, "WsT descriptor is NULL");
  const int64_t nnz = Ws->rows * Ws->k;
  if (Ws->rows > 32767) return fail(SRA_ERR_INVALID_ARG, "transpose column ids are int16: rows must be <= 32767");
  SRA_TRY(check_ptr(WsT->row_ptr, true, "WsT->row_ptr"));
  SRA_TRY(check_ptr(WsT->index, nnz > 0, "WsT->index"));
  SRA_TRY(check_ptr(WsT->values, nnz > 0, "WsT->values"));
  const size_t need = sra::ffi_transpose_ws(Ws->rows, Ws->cols);
  if (!ws || ws_bytes < need) return fail(SRA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (!al16(ws)) return fail(SRA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  WsT->format = SRA_FMT_CSR;
  WsT->dtype = Ws->dtype;
  WsT->rows = Ws->cols;
  WsT->cols = Ws->rows;
  WsT->nnz = nnz;
  const hipStream_t s = (hipStream_t)stream;
  return hip_done(sra::launch_ffi_transpose(Ws->dtype, Ws->values, Ws->index, Ws->rows, Ws->cols,
                                            Ws->k, WsT->row_ptr, WsT->index, WsT->values, ws, s),
                  s, "ffi_transpose");
}

sra_status sra_ffi_tile_size(int64_t rows, int64_t cols, int64_t nnz, size_t* entry_bytes,
                             size_t* offset_bytes) {
  if (!entry_bytes || !offset_bytes) return fail(SRA_ERR_INVALID_ARG, "entry_bytes / offset_bytes is NULL");
  if (rows < 0 || cols < 1 || cols > 32767 || nnz < 0 || nnz > rows * cols)
    return fail(SRA_ERR_INVALID_ARG, "need rows >= 0, 1 <= cols <= 32767, 0 <= nnz <= rows * cols");
  sra::ffi_tile_bytes(rows, cols, nnz, entry_bytes, offset_bytes);
  if (*entry_bytes >= ((size_t)1 << 31)) return fail(SRA_ERR_UNSUPPORTED, "tiled format over 2 GiB of entries");
  return SRA_OK;
}

sra_status sra_ffi_tile(const sra_sparse* S, sra_sparse* out, void* stream) {
  SRA_TRY(check_sparse(S, "S"));
  if (S->format != SRA_FMT_ELL && S->format != SRA_FMT_CSR)
    return fail(SRA_ERR_INVALID_ARG, "ffi_tile needs an ELL or CSR matrix");
  if (S->dtype != SRA_BF16) return fail(SRA_ERR_UNSUPPORTED, "ffi_tile: the tiled format is bf16 only");
  if (!out) return fail(SRA_ERR_INVALID_ARG, "out descriptor is NULL");
  const int64_t nnz = S->format == SRA_FMT_ELL ? S->rows * S->k : S->nnz;
  size_t eb, ob;
  SRA_TRY(sra_ffi_tile_size(S->rows, S->cols, nnz, &eb, &ob));
  SRA_TRY(check_ptr(out->values, eb > 0, "out->values"));
  SRA_TRY(check_ptr(out->meta, true, "out->meta"));
  out->format = SRA_FMT_FFI_TILED;
  out->dtype = S->dtype;
  out->rows = S->rows;
  out->cols = S->cols;
  out->nnz = (int64_t)(eb / 4);
  const hipStream_t s = (hipStream_t)stream;
  return hip_done(sra::launch_ffi_tile((const uint16_t*)S->values, S->index,
                                       S->format == SRA_FMT_CSR ? S->row_ptr : nullptr, S->k, S->rows,
                                       S->cols, (uint32_t*)out->values, out->meta, out->nnz, s),
                  s, "ffi_tile");
}

sra_status sra_fwd_workspace(const sra_sparse* Ws, int64_t T, int32_t r, size_t* bytes) {
  SRA_TRY(validate_fwd(Ws, T, r));
  if (!bytes) return fail(SRA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = fwd_bytes(Ws, T, r, /*own_u=*/true, nullptr);
  return SRA_OK;
}

sra_status sra_sparse_lora_fwd(const sra_sparse* Ws, const void* X, int64_t T, const void* A,
                               const void* B, int32_t r, void* Y, float* U_out, void* ws,
                               size_t ws_bytes, void* stream) {
  SRA_TRY(validate_fwd(Ws, T, r));
  const int64_t N = Ws->rows, K = Ws->cols;
  const bool any = T > 0;
  SRA_TRY(check_ptr(X, any && K > 0, "X"));
  SRA_TRY(check_ptr(Y, any && N > 0, "Y"));
  SRA_TRY(check_ptr(A, any && r > 0 && K > 0, "A"));
  SRA_TRY(check_ptr(B, any && r > 0 && N > 0, "B"));
  if (U_out) SRA_TRY(check_ptr(U_out, true, "U_out"));
  FwdPlan plan;
  fwd_bytes(Ws, T, r, U_out == nullptr, &plan);
  if (plan.total > 0 && (!ws || ws_bytes < plan.total))
    return fail(SRA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", plan.total, ws_bytes);
  if (plan.total > 0 && !al16(ws)) return fail(SRA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (T == 0) return SRA_OK;
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* wsb = (uint8_t*)ws;
  float* U = r > 0 ? (U_out ? U_out : (float*)(wsb + plan.u_off)) : nullptr;
  sra_sparse w24;
  if (is12(Ws)) {  // run on the 2:4 kernels with the converted metadata
    w24 = *Ws;
    w24.meta = (uint32_t*)(wsb + plan.meta_off);
    w24.n = 2;
    w24.m = 4;
    SRA_TRY(hip_done(sra::launch_meta_or(Ws->meta, w24.meta, (int64_t)(meta_bytes(Ws) / 4), kMeta12To24, s),
                     s, "fwd 1:2 metadata"));
    Ws = &w24;
  } else if (is28_on24(Ws, T)) {  // run on the 2:4 kernels with the weight rewritten as 2:4
    w24 = *Ws;
    w24.format = SRA_FMT_NM;
    w24.values = wsb + plan.v24_off;
    w24.meta = (uint32_t*)(wsb + plan.meta_off);
    w24.n = 2;
    w24.m = 4;
    SRA_TRY(hip_done(sra::launch_nm28_to24((const uint16_t*)Ws->values, Ws->meta, Ws->rows, Ws->cols,
                                           (uint16_t*)w24.values, w24.meta, s, is28t(Ws)),
                     s, "fwd 2:8 as 2:4"));
    Ws = &w24;
  }

  if (Ws->dtype == SRA_F32) {
    double* U64 = r > 0 ? (double*)(wsb + plan.u64_off) : nullptr;
    if (r > 0)
      SRA_TRY(hip_done(sra::launch_f32_adapter_u((const float*)X, (const float*)A, T, K, r, U64,
                                                 U_out, s), s, "fwd U"));
    const sra::F32Sparse S = f32_view(Ws);
    return hip_done(sra::launch_f32_spmm(S, (const float*)X, T, U64, (const float*)B, r, 1, r,
                                         (float*)Y, s), s, "fwd spmm f32");
  }
  // U = X A^T: computed inside the SpMM when its plan allows, else by the adapter kernel first
  const bool nm24 = Ws->format == SRA_FMT_NM || Ws->format == SRA_FMT_NM_TILED;
  const bool xp = use_xp(Ws, T);
  const bool fuse = r > 0 && nm24 && (xp ? sra::spmm_xp_fuses_adapter(N, K, T, r)
                                         : sra::spmm24_fuses_adapter(N, K, T, r));
  if (r > 0 && !fuse)
    SRA_TRY(hip_done(sra::launch_adapter_rows((const uint16_t*)X, T, K, (const uint16_t*)A, K, r, U,
                                              nullptr, nullptr, wsb + plan.gemm_off, s), s, "fwd U"));
  sra::Epilogue ep;
  ep.U = U;
  ep.E = (const uint16_t*)B;
  ep.e_row_stride = r;
  ep.e_j_stride = 1;
  ep.r = r;
  if (fuse) {
    ep.G = (const uint16_t*)A;
    ep.g_ld = K;
    ep.u_out = U_out;
  }
  if (use_dec28(Ws, T))
    return hip_done(sra::launch_decode28_bf16((const uint16_t*)Ws->values, Ws->meta, N, K,
                                              (const uint16_t*)X, T, ep, (uint16_t*)Y, s, is28t(Ws)),
                    s, "fwd spmm 2:8 (decode)");
  if (xp)
    return hip_done(sra::launch_spmm_xp_bf16(is28(Ws) ? 28 : 24, Ws->format == SRA_FMT_NM_TILED,
                                             (const uint16_t*)Ws->values, Ws->meta, N, K,
                                             (const uint16_t*)X, T, ep, (uint16_t*)Y,
                                             wsb ? wsb + plan.gemm_off : nullptr, s),
                    s, is28(Ws) ? "fwd spmm 2:8" : "fwd spmm 2:4 (dense MFMA)");
  if (Ws->format == SRA_FMT_NM_TILED)
    return hip_done(sra::launch_spmm24_tiled_bf16((const uint16_t*)Ws->values, Ws->meta, N, K,
                                                  (const uint16_t*)X, T, ep, (uint16_t*)Y,
                                                  wsb ? wsb + plan.gemm_off : nullptr, s),
                    s, "fwd spmm 2:4 (streaming layout)");
  if (Ws->format == SRA_FMT_NM)
    return hip_done(sra::launch_spmm24_bf16((const uint16_t*)Ws->values, Ws->meta, N, K,
                                            (const uint16_t*)X, T, ep, (uint16_t*)Y,
                                            wsb ? wsb + plan.gemm_off : nullptr, s),
                    s, "fwd spmm 2:4");
  if (Ws->format == SRA_FMT_FFI_TILED)
    return hip_done(sra::launch_ffi_tiled_bf16((const uint32_t*)Ws->values, Ws->meta, (size_t)Ws->nnz * 4,
                                               N, K, (const uint16_t*)X, T, ep, (uint16_t*)Y, s),
                    s, "fwd spmm ffi (tiled)");
  return hip_done(sra::launch_spmm_ffi_bf16(SRA_FMT_ELL, (const uint16_t*)Ws->values, Ws->index,
                                            nullptr, Ws->k, N, K, (const uint16_t*)X, T, ep,
                                            (uint16_t*)Y, wsb ? wsb + plan.ffi_off : nullptr, s,
                                            Ws->rows * Ws->k),
                  s, "fwd spmm ffi");
}

sra_status sra_bwd_workspace(const sra_sparse* P, int64_t T, int32_t r, uint32_t flags, size_t* bytes) {
  SRA_TRY(validate_bwd(P, T, r, flags));
  if (!bytes) return fail(SRA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_bytes(P, T, r, flags, /*have_u=*/false, /*have_du=*/false, nullptr);
  return SRA_OK;
}

sra_status sra_sparse_lora_bwd(const sra_sparse* P, const void* dY, const void* X, int64_t T,
                               const float* U,
                               const void* A, const void* B, int32_t r, uint32_t flags, void* dX,
                               float* dA, float* dB, float* dU_out, void* ws, size_t ws_bytes,
                               void* stream) {
  BwdPlan plan;
  SRA_TRY(check_bwd_args(P, dY, X, T, U, A, B, r, flags, dX, dA, dB, dU_out, &plan));
  const int64_t K = P->rows, N = P->cols;
  const bool fdx = flags & SRA_GRAD_DX, fda = (flags & SRA_GRAD_DA) && r > 0,
             fdb = (flags & SRA_GRAD_DB) && r > 0;
  const bool dx_ad = fdx && !(flags & SRA_DX_NO_ADAPTER) && r > 0;
  if (plan.total > 0 && (!ws || ws_bytes < plan.total))
    return fail(SRA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", plan.total, ws_bytes);
  if (plan.total > 0 && !al16(ws)) return fail(SRA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    if (fda) SRA_TRY(hip_done(sra::launch_fill_f32(dA, (int64_t)r * K, 0.f, s), s, "zero dA"));
    if (fdb) SRA_TRY(hip_done(sra::launch_fill_f32(dB, N * (int64_t)r, 0.f, s), s, "zero dB"));
    return SRA_OK;
  }
  uint8_t* wsb = (uint8_t*)ws;
  sra_sparse p24;
  if (is12(P) && fdx) {  // run on the 2:4 kernels with the converted metadata
    p24 = *P;
    p24.meta = (uint32_t*)(wsb + plan.meta_off);
    p24.n = 2;
    p24.m = 4;
    SRA_TRY(hip_done(sra::launch_meta_or(P->meta, p24.meta, (int64_t)(meta_bytes(P) / 4), kMeta12To24, s),
                     s, "bwd 1:2 metadata"));
    P = &p24;
  } else if (is28_on24(P, T) && fdx) {  // dX on the 2:4 kernels with P rewritten as 2:4
    p24 = *P;
    p24.format = SRA_FMT_NM;
    p24.values = wsb + plan.v24_off;
    p24.meta = (uint32_t*)(wsb + plan.meta_off);
    p24.n = 2;
    p24.m = 4;
    SRA_TRY(hip_done(sra::launch_nm28_to24((const uint16_t*)P->values, P->meta, P->rows, P->cols,
                                           (uint16_t*)p24.values, p24.meta, s, is28t(P)),
                     s, "bwd 2:8 as 2:4"));
    P = &p24;
  }
  const float* Uv = plan.need_u ? (plan.own_u ? (const float*)(wsb + plan.u_off) : U) : nullptr;
  float* dU = plan.need_du ? (plan.own_du ? (float*)(wsb + plan.du_off) : dU_out) : nullptr;
  void* gws = wsb ? wsb + plan.gemm_off : nullptr;

  if (P->dtype == SRA_F32) {
    double* U64 = plan.need_u ? (double*)(wsb + plan.u64_off) : nullptr;
    double* dU64 = plan.need_du ? (double*)(wsb + plan.du64_off) : nullptr;
    if (plan.need_u)
      SRA_TRY(hip_done(sra::launch_f32_adapter_u((const float*)X, (const float*)A, T, K, r, U64,
                                                 nullptr, s), s, "bwd U"));
    if (plan.need_du)
      SRA_TRY(hip_done(sra::launch_f32_du((const float*)dY, (const float*)B, T, N, r, dU64, dU_out, s),
                       s, "bwd dU"));
    if (fdx)
      SRA_TRY(hip_done(sra::launch_f32_spmm(f32_view(P), (const float*)dY, T, dU64, (const float*)A,
                                            1, K, dx_ad ? r : 0, (float*)dX, s), s, "bwd dX f32"));
    if (fdb)
      SRA_TRY(hip_done(sra::launch_f32_tn((const float*)dY, nullptr, N, nullptr, U64, r, T, N, r,
                                          dB, s), s, "bwd dB"));
    if (fda)
      SRA_TRY(hip_done(sra::launch_f32_tn(nullptr, dU64, r, (const float*)X, nullptr, K, T, r, K,
                                          dA, s), s, "bwd dA"));
    return SRA_OK;
  }
  uint16_t* wt = plan.need_du ? (uint16_t*)(wsb + plan.wt_off) : nullptr;
  uint16_t* vtU = fdb ? (uint16_t*)(wsb + plan.vtu_off) : nullptr;
  uint16_t* vtdU = fda ? (uint16_t*)(wsb + plan.vtdu_off) : nullptr;
  if (plan.own_u)
    SRA_TRY(hip_done(sra::launch_adapter_rows((const uint16_t*)X, T, K, (const uint16_t*)A, K, r,
                                              (float*)Uv, nullptr, nullptr, gws, s), s, "bwd U"));
  uint16_t* at = dx_ad ? (uint16_t*)(wsb + plan.at_off) : nullptr;
  SRA_TRY(hip_done(sra::launch_adapter_bwd_prep((const uint16_t*)B, N, r, wt, (const uint16_t*)A, K,
                                                at, Uv, T, vtU, s), s, "bwd prep"));
  // dU = dY B: computed inside the dX SpMM (which also writes dU_out and dU^T's parts for dA)
  // when its plan allows, else by the adapter kernel first
  const bool nm24 = P->format == SRA_FMT_NM || P->format == SRA_FMT_NM_TILED;
  const bool xp = use_xp(P, T);
  const bool fuse = dx_ad && nm24 && (xp ? sra::spmm_xp_fuses_adapter(K, N, T, r)
                                         : sra::spmm24_fuses_adapter(K, N, T, r));
  if (plan.need_du && !fuse)
    SRA_TRY(hip_done(sra::launch_adapter_rows((const uint16_t*)dY, T, N, wt, sra::packed_wt_ld(N), r,
                                              dU, nullptr, vtdU, gws, s), s, "bwd dU"));
  if (fdx) {
    sra::Epilogue ep;
    ep.U = dU;
    ep.E = at;  // A^T rows: E(k, j) = A[j][k]
    ep.e_row_stride = sra::packed_at_ld(r);
    ep.e_j_stride = 1;
    ep.r = dx_ad ? r : 0;
    if (fuse) {
      ep.G = wt;
      ep.g_ld = sra::packed_wt_ld(N);
      ep.u_out = dU_out;
      ep.vt = vtdU;
      ep.vt_rp = (int)sra::vt_rows(r);
      ep.vt_tp = sra::vt_cols(T);
    }
    if (use_dec28(P, T))
      SRA_TRY(hip_done(sra::launch_decode28_bf16((const uint16_t*)P->values, P->meta, K, N,
                                                 (const uint16_t*)dY, T, ep, (uint16_t*)dX, s, is28t(P)),
                       s, "bwd dX 2:8 (decode)"));
    else if (xp)
      SRA_TRY(hip_done(sra::launch_spmm_xp_bf16(is28(P) ? 28 : 24, P->format == SRA_FMT_NM_TILED,
                                                (const uint16_t*)P->values, P->meta, K, N,
                                                (const uint16_t*)dY, T, ep, (uint16_t*)dX,
                                                wsb ? wsb + plan.spmm_off : nullptr, s),
                       s, is28(P) ? "bwd dX 2:8" : "bwd dX 2:4 (dense MFMA)"));
    else if (P->format == SRA_FMT_NM_TILED)
      SRA_TRY(hip_done(sra::launch_spmm24_tiled_bf16((const uint16_t*)P->values, P->meta, K, N,
                                                     (const uint16_t*)dY, T, ep, (uint16_t*)dX,
                                                     wsb ? wsb + plan.spmm_off : nullptr, s),
                       s, "bwd dX 2:4 (streaming layout)"));
    else if (P->format == SRA_FMT_NM)
      SRA_TRY(hip_done(sra::launch_spmm24_bf16((const uint16_t*)P->values, P->meta, K, N,
                                               (const uint16_t*)dY, T, ep, (uint16_t*)dX,
                                               wsb ? wsb + plan.spmm_off : nullptr, s),
                       s, "bwd dX 2:4"));
    else if (P->format == SRA_FMT_FFI_TILED)
      SRA_TRY(hip_done(sra::launch_ffi_tiled_bf16((const uint32_t*)P->values, P->meta, (size_t)P->nnz * 4,
                                                  K, N, (const uint16_t*)dY, T, ep, (uint16_t*)dX, s),
                       s, "bwd dX ffi (tiled)"));
    else
      SRA_TRY(hip_done(sra::launch_spmm_ffi_bf16(SRA_FMT_CSR, (const uint16_t*)P->values, P->index,
                                                 P->row_ptr, 0, K, N, (const uint16_t*)dY, T, ep,
                                                 (uint16_t*)dX, wsb ? wsb + plan.spmm_off : nullptr, s,
                                                 P->nnz),
                       s, "bwd dX ffi"));
  }
  // dB and dA: one merged launch (and one slice reduction) when the shapes allow
  sra::AdapterGrad jobs[2];
  const int nj = grad_jobs(jobs, fdb, fda, N, K);
  for (int i = 0; i < nj; ++i) {
    const bool is_db = fdb && i == 0;
    jobs[i].act = (const uint16_t*)(is_db ? dY : X);
    jobs[i].vt = is_db ? vtU : vtdU;
    jobs[i].out = is_db ? dB : dA;
  }
  if (nj > 0 && sra::adapter_grads_ok(jobs, nj, T, r)) {
    SRA_TRY(hip_done(sra::launch_adapter_grads(jobs, nj, T, r, gws, s), s, "bwd dB, dA"));
    return SRA_OK;
  }
  if (fdb)
    SRA_TRY(hip_done(sra::launch_adapter_cols((const uint16_t*)dY, T, N, vtU, 3, r, false, dB, gws, s),
                     s, "bwd dB"));
  if (fda)
    SRA_TRY(hip_done(sra::launch_adapter_cols((const uint16_t*)X, T, K, vtdU, 3, r, true, dA, gws, s),
                     s, "bwd dA"));
  return SRA_OK;
}

// ---------------------------------------------------------------- fixed-fan-in adapter factor
// A [r, K] as ELL: densified into the workspace, then the dense-adapter path; dA is gathered at
// A's stored columns from the dense fp32 gradient.
static sra_status check_ffa(const sra_sparse* A, const sra_sparse* S, int64_t K) {
  SRA_TRY(check_sparse(A, "A"));
  if (A->format != SRA_FMT_ELL) return fail(SRA_ERR_INVALID_ARG, "A must be an ELL matrix (fixed fan-in)");
  if (A->dtype != SRA_BF16 || S->dtype != SRA_BF16)
    return fail(SRA_ERR_UNSUPPORTED, "the fixed-fan-in adapter factor is bf16 only");
  if (A->cols != K) return fail(SRA_ERR_INVALID_ARG, "A has %lld columns, the layer has K = %lld",
                                (long long)A->cols, (long long)K);
  if (A->rows < 1 || A->rows > 256) return fail(SRA_ERR_UNSUPPORTED, "adapter rank %lld outside [1, 256]", (long long)A->rows);
  if (K % 8) return fail(SRA_ERR_UNSUPPORTED, "K %% 8 != 0");
  return SRA_OK;
}

static size_t ffa_dense_bytes(const sra_sparse* A) { return ((size_t)A->rows * A->cols * 2 + 255) & ~(size_t)255; }
static size_t ffa_grad_bytes(const sra_sparse* A) { return ((size_t)A->rows * A->cols * 4 + 255) & ~(size_t)255; }

sra_status sra_ffa_fwd_workspace(const sra_sparse* Ws, int64_t T, const sra_sparse* A, size_t* bytes) {
  SRA_TRY(validate_fwd(Ws, T, A ? (int32_t)std::min<int64_t>(A->rows, 256) : 0));
  SRA_TRY(check_ffa(A, Ws, Ws->cols));
  if (!bytes) return fail(SRA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ffa_dense_bytes(A) + fwd_bytes(Ws, T, (int32_t)A->rows, /*own_u=*/true, nullptr);
  return SRA_OK;
}

sra_status sra_sparse_lora_fwd_ffa(const sra_sparse* Ws, const void* X, int64_t T, const sra_sparse* A,
                                   const void* B, void* Y, float* U_out, void* ws, size_t ws_bytes,
                                   void* stream) {
  SRA_TRY(validate_fwd(Ws, T, A ? (int32_t)std::min<int64_t>(A->rows, 256) : 0));
  SRA_TRY(check_ffa(A, Ws, Ws->cols));
  const int32_t r = (int32_t)A->rows;
  const size_t head = ffa_dense_bytes(A);
  const size_t need = head + fwd_bytes(Ws, T, r, U_out == nullptr, nullptr);
  if (!ws || ws_bytes < need)
    return fail(SRA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!al16(ws)) return fail(SRA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const int64_t N = Ws->rows, K = Ws->cols;
  SRA_TRY(check_ptr(X, T > 0 && K > 0, "X"));
  SRA_TRY(check_ptr(Y, T > 0 && N > 0, "Y"));
  SRA_TRY(check_ptr(B, T > 0 && N > 0, "B"));
  if (U_out) SRA_TRY(check_ptr(U_out, true, "U_out"));
  if (T == 0) return SRA_OK;
  const hipStream_t s = (hipStream_t)stream;
  uint16_t* Ad = (uint16_t*)ws;
  SRA_TRY(hip_done(sra::launch_ffi_densify(SRA_FMT_ELL, (const uint16_t*)A->values, A->index, nullptr,
                                           A->k, r, K, Ad, s), s, "fwd A densify"));
  return sra_sparse_lora_fwd(Ws, X, T, Ad, B, r, Y, U_out, (uint8_t*)ws + head, ws_bytes - head, stream);
}

sra_status sra_ffa_bwd_workspace(const sra_sparse* P, int64_t T, const sra_sparse* A, uint32_t flags,
                                 size_t* bytes) {
  SRA_TRY(validate_bwd(P, T, A ? (int32_t)std::min<int64_t>(A->rows, 256) : 0, flags));
  SRA_TRY(check_ffa(A, P, P->rows));
  if (!bytes) return fail(SRA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ffa_dense_bytes(A) + ((flags & SRA_GRAD_DA) ? ffa_grad_bytes(A) : 0) +
           bwd_bytes(P, T, (int32_t)A->rows, flags, /*have_u=*/false, /*have_du=*/false, nullptr);
  return SRA_OK;
}

sra_status sra_sparse_lora_bwd_ffa(const sra_sparse* P, const void* dY, const void* X, int64_t T,
                                   const float* U, const sra_sparse* A, const void* B, uint32_t flags,
                                   void* dX, float* dA_values, float* dB, float* dU_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  SRA_TRY(validate_bwd(P, T, A ? (int32_t)std::min<int64_t>(A->rows, 256) : 0, flags));
  SRA_TRY(check_ffa(A, P, P->rows));
  const int32_t r = (int32_t)A->rows;
  const int64_t K = P->rows;
  const bool fda = flags & SRA_GRAD_DA;
  const size_t head = ffa_dense_bytes(A), gbytes = fda ? ffa_grad_bytes(A) : 0;
  uint16_t* Ad = ws ? (uint16_t*)ws : nullptr;
  float* dA_dense = (ws && fda) ? (float*)((uint8_t*)ws + head) : nullptr;
  BwdPlan plan;
  // every check of the dense-adapter call, with the densified factor and the dense dA in place
  SRA_TRY(check_bwd_args(P, dY, X, T, U, Ad ? Ad : (const void*)16, B, r, flags, dX,
                         fda ? (dA_dense ? dA_dense : (const float*)16) : nullptr, dB, dU_out, &plan));
  SRA_TRY(check_ptr(dA_values, fda, "dA_values"));
  const size_t need = head + gbytes + plan.total;
  if (!ws || ws_bytes < need)
    return fail(SRA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!al16(ws)) return fail(SRA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  if (T > 0)
    SRA_TRY(hip_done(sra::launch_ffi_densify(SRA_FMT_ELL, (const uint16_t*)A->values, A->index, nullptr,
                                             A->k, r, K, Ad, s), s, "bwd A densify"));
  SRA_TRY(sra_sparse_lora_bwd(P, dY, X, T, U, Ad, B, r, flags, dX, dA_dense, dB, dU_out,
                              (uint8_t*)ws + head + gbytes, ws_bytes - head - gbytes, stream));
  if (fda)
    SRA_TRY(hip_done(sra::launch_ell_gather_f32(dA_dense, A->index, A->k, r, K, dA_values, s), s,
                     "bwd dA gather"));
  return SRA_OK;
}

// Allocation-free backward: the workspace is this fixed device array.  In host code its name is
// only a stand-in for the symbol; the device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[SRA_NOALLOC_SCRATCH_BYTES];

sra_status sra_sparse_lora_bwd_noalloc(const sra_sparse* P, const void* dY, const void* X, int64_t T,
                                       const float* U, const void* A, const void* B, int32_t r,
                                       uint32_t flags, void* dX, float* dA, float* dB,
                                       float* dU_out, void* stream) {
  BwdPlan plan;
  SRA_TRY(check_bwd_args(P, dY, X, T, U, A, B, r, flags, dX, dA, dB, dU_out, &plan));
  const size_t need = plan.total;
  if (need > SRA_NOALLOC_SCRATCH_BYTES)
    return fail(SRA_ERR_WORKSPACE, "this call needs %zu bytes of workspace, above the %zu of the "
                "allocation-free entry point (use sra_sparse_lora_bwd)", need,
                (size_t)SRA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    static std::mutex mu;
    static void* dev_ptr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SRA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(SRA_ERR_UNSUPPORTED, "device ordinal %d above 63", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(SRA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      dev_ptr[dev] = p;
    }
    ws = dev_ptr[dev];
  }
  return sra_sparse_lora_bwd(P, dY, X, T, U, A, B, r, flags, dX, dA, dB, dU_out, ws,
                             ws ? (size_t)SRA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"

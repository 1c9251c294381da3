// Adapter products of the low-rank branch (SLoPe paper, section 2.2 "sparse + low-rank adapters";
// LoRA's factorised update):
//   rows kernel:  U  = X A^T   [T x r]   and   dU = dY B   [T x r]
//   cols kernel:  dB = dY^T U  [N x r]   and   dA = dU^T X [r x K]
// For the ranks the method uses these stream X or dY once and do little arithmetic per byte, so
// both kernels are built to keep many loads in flight: every wave issues the next batch of global
// loads before it multiplies the current one, and workgroups are small enough in LDS and
// registers that several share a CU.
//
// rows: Out[t][j] = sum_c Act[t][c] Wt[j][c].  A workgroup owns 16 tokens and 16*JT adapter
//   columns over a slice of the reduction dim c; its four waves take interleaved 32-column steps of
//   the slice (so together they read whole 256-byte stretches of each token row) and are summed
//   through LDS at the end.  Both MFMA operands come straight from global memory as 16-byte
//   fragments: the activation row and a c-contiguous weight row (A as given; B transposed once
//   into the workspace).
// cols: Out[m][j] = sum_t Act[t][m] V[t][j].  The reduction runs over tokens, the slow dim of Act,
//   so each 64-token x 64-column Act tile is staged in LDS as [t][m] and a lane gathers its 8
//   tokens of one column from there.  dB and dA sum thousands of token products whose total can
//   cancel by orders of magnitude, so V's rounding is amplified ~sqrt(T) times: V^T arrives as
//   bf16 parts [part][j][t] -- three parts for fp32 V (U, split by the backward prep kernel; split
//   error below fp32 rounding), four for fp64 dU (written by the rows kernel that produces it) --
//   which read as contiguous 16-byte fragments.
// Both use v_mfma_f32_16x16x32_bf16 and move every 32-step MFMA partial into fp64 registers (fp32
// rounding only acts inside one 32-term dot product); slices write fp64 partials that one more
// kernel sums in a fixed order, so results are independent of scheduling.
#include "common.h"

namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

union Frag {
  u32x4 v;
  uint16_t h[8];
  bf16x8v b;
};

template <int N>
SRA_DEV void flush(f32x4 (&acc)[N], double (&acc64)[N][4]) {
#pragma unroll
  for (int a = 0; a < N; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc64[a][e] += (double)acc[a][e];
      acc[a][e] = 0.f;
    }
}

// 8 consecutive bf16 values p[i .. i+7] with i < lim masking (zeros past lim)
SRA_DEV u32x4 load8(const uint16_t* __restrict__ p, int64_t i, int64_t lim, bool vec) {
  Frag x;
  x.v = u32x4{0, 0, 0, 0};
  if (vec && i + 8 <= lim) {
    x.v = *reinterpret_cast<const u32x4*>(p + i);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (i + q < lim) x.h[q] = p[i + q];
  }
  return x.v;
}

// ------------------------------------------------------------------------------------ rows
// grid: (ceil(T/16), ceil(r/(16 JT)), S); slice z covers c in [z*c_per, min(C, (z+1)*c_per)).
// Wave w takes the 32-column steps w, w+4, w+8, ... of its slice, UB steps per batch.
// When vt is non-null the result is also written as V^T split into four bf16 parts (write_vt4),
// vt[p][j][t] (rows rp, columns Tp; the zero padding is the caller's), ready for the cols kernel.

template <int JT, int UB>
__global__ __launch_bounds__(256) void k_adapter_rows(const uint16_t* __restrict__ act, int64_t T,
                                                      int64_t C, const uint16_t* __restrict__ wt,
                                                      int64_t ldw, int r, int64_t c_per,
                                                      double* __restrict__ part,
                                                      float* __restrict__ out,
                                                      double* __restrict__ out64,
                                                      uint16_t* __restrict__ vt, int rp, int64_t Tp) {
  __shared__ double red[3][JT * 4][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16, t = t0 + lr;
  const int j0 = blockIdx.y * 16 * JT;
  const int64_t cb = (int64_t)blockIdx.z * c_per, ce = min(C, cb + c_per);
  const int64_t nsteps = (ce - cb + 31) / 32;
  const int nb = (int)((nsteps + 4 * UB - 1) / (4 * UB));  // batches (same count for every wave)
  const bool a_vec = (C & 7) == 0, w_vec = (ldw & 7) == 0;
  const bool t_ok = t < T;
  const uint16_t* arow = act + (t_ok ? t : 0) * C;
  const uint16_t* wrow[JT];
  bool j_ok[JT];
#pragma unroll
  for (int a = 0; a < JT; ++a) {
    const int j = j0 + 16 * a + lr;
    j_ok[a] = j < r;
    wrow[a] = wt + (int64_t)(j_ok[a] ? j : 0) * ldw;
  }

  u32x4 fa0[UB], fw0[UB][JT], fa1[UB], fw1[UB][JT];
  auto load = [&](int b, u32x4(&fa)[UB], u32x4(&fw)[UB][JT]) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int64_t st = w + 4 * ((int64_t)b * UB + u);
      const int64_t c = cb + 32 * st + 8 * lg;
      fa[u] = t_ok ? load8(arow, c, ce, a_vec) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int a = 0; a < JT; ++a) fw[u][a] = j_ok[a] ? load8(wrow[a], c, ce, w_vec) : u32x4{0, 0, 0, 0};
    }
  };
  f32x4 acc[JT];
  double acc64[JT][4];
#pragma unroll
  for (int a = 0; a < JT; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[a][e] = 0.f;
      acc64[a][e] = 0.0;
    }
  auto compute = [&](int b, const u32x4(&fa)[UB], const u32x4(&fw)[UB][JT]) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (w + 4 * ((int64_t)b * UB + u) >= nsteps) break;  // wave-uniform
      Frag x;
      x.v = fa[u];
#pragma unroll
      for (int a = 0; a < JT; ++a) {
        Frag y;
        y.v = fw[u][a];
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.b, y.b, acc[a], 0, 0, 0);
      }
      flush(acc, acc64);
    }
  };
  if (nb > 0) load(0, fa0, fw0);
  for (int b = 0; b < nb; b += 2) {
    if (b + 1 < nb) load(b + 1, fa1, fw1);
    compute(b, fa0, fw0);
    if (b + 2 < nb) load(b + 2, fa0, fw0);
    if (b + 1 < nb) compute(b + 1, fa1, fw1);
  }
  // V^T columns T .. Tp-1 (padding to a multiple of 8) must read as zero in the cols kernel
  if (vt && blockIdx.z == 0 && w == 0) {
#pragma unroll
    for (int a = 0; a < JT; ++a) {
      const int j = j0 + 16 * a + lr;
      const int64_t tt = t0 + 4 * lg;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j < r && tt + e >= T && tt + e < Tp)
#pragma unroll
          for (int p = 0; p < 4; ++p) vt[((int64_t)p * rp + j) * Tp + tt + e] = 0;
    }
  }
  // waves 1..3 hand their sums to wave 0, which adds them in wave order
  if (w > 0) {
#pragma unroll
    for (int a = 0; a < JT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[w - 1][a * 4 + e][l] = acc64[a][e];
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int a = 0; a < JT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc64[a][e] += red[k][a * 4 + e][l];
  // D layout: row (token) 4*(l/16)+e of the 16, column j = l%16 of j tile a
#pragma unroll
  for (int a = 0; a < JT; ++a) {
    const int j = j0 + 16 * a + lr;
    if (j >= r) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t tt = t0 + 4 * lg + e;
      if (tt >= T) continue;
      const double s = acc64[a][e];
      if (part) {
        part[(int64_t)blockIdx.z * T * r + tt * r + j] = s;
      } else {
        if (out) out[tt * r + j] = (float)s;
        if (out64) out64[tt * r + j] = s;
        if (vt) write_vt4(vt, rp, Tp, j, tt, s);
      }
    }
  }
}

// Backward prep, one launch for two independent inputs of the adapter gradients:
//   blocks [0, n_pack):  wt[j][c] = B[c][j] (c < C, j < r; rows of stride ldw), a 64 x 64 tile per
//                        block transposed through LDS so reads and writes are coalesced;
//   blocks [n_pack, ..): vt[p][j][t], U^T split into three bf16 parts (j < rp, t < Tp, zero
//                        outside r x T), 256 entries per block.
__global__ void k_bwd_prep(const uint16_t* __restrict__ B, int64_t C, int r, int64_t ldw,
                           uint16_t* __restrict__ wt, int n_pack, int pack_cx,
                           const float* __restrict__ U, int64_t T, int rp, int64_t Tp,
                           uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[64][65];
  const int bid = blockIdx.x;
  if (bid < n_pack) {
    const int64_t c0 = (int64_t)(bid % pack_cx) * 64;
    const int j0 = (bid / pack_cx) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 256 threads: 4 rows at a time
    uint16_t v[16];  // all loads issued before the first LDS store
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int64_t c = c0 + ty + 4 * k;
      const int j = j0 + tx;
      v[k] = (c < C && j < r) ? B[c * r + j] : (uint16_t)0;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[ty + 4 * k][tx] = v[k];
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
      const int j = j0 + i;
      const int64_t c = c0 + tx;
      if (j < r && c < C) wt[(int64_t)j * ldw + c] = tile[tx][i];
    }
    return;
  }
  const int64_t i = (int64_t)(bid - n_pack) * 256 + threadIdx.x;  // i = j * Tp + t
  if (i >= (int64_t)rp * Tp) return;
  const int j = (int)(i / Tp);
  const int64_t t = i - (int64_t)j * Tp;
  uint16_t p[3] = {0, 0, 0};
  if (j < r && t < T) split3_bf16(U[t * r + j], p[0], p[1], p[2]);
  for (int q = 0; q < 3; ++q) vt[((int64_t)q * rp + j) * Tp + t] = p[q];
}

// ------------------------------------------------------------------------------------ cols
constexpr int CS = 64;        // tokens per staged tile
constexpr int ALD = 64 + 8;   // LDS row of the Act tile [t][m] (elements; 144 B keeps 16 B alignment)
constexpr int VLD = CS + 8;   // LDS row of the V^T tile [j][t]

// V^T parts: vt[p][j][t] for j < rp (r rounded up to 16) and t < Tp (T rounded up to 8; columns
// past T are 0).  fp32 V (U) -> 3 parts written by the backward prep kernel, fp64 V (dU) -> 4 parts
// written by the rows kernel (or its slice reduction).

// grid: (ceil(M/64), ceil(r/(16 JT)), S); slice z covers tokens [z*t_per, min(T, (z+1)*t_per)),
// t_per % CS == 0.  Wave w owns columns m0 + 16w .. +15.
template <int JT>
__global__ __launch_bounds__(256) void k_adapter_cols(const uint16_t* __restrict__ act, int64_t T,
                                                      int64_t M, const uint16_t* __restrict__ vt,
                                                      int parts, int r, int rp, int64_t Tp,
                                                      int64_t t_per, bool out_t,
                                                      double* __restrict__ part,
                                                      float* __restrict__ out) {
  constexpr int JR = 16 * JT;  // adapter rows of one pass
  constexpr int NV = (4 * JR * (CS / 8) + 255) / 256;  // V^T vectors per thread (4 parts max)
  __shared__ __attribute__((aligned(16))) uint16_t al[CS * ALD];
  __shared__ __attribute__((aligned(16))) uint16_t vl[4 * JR * VLD];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int j0 = blockIdx.y * JR;
  const int64_t tb = (int64_t)blockIdx.z * t_per, te = min(T, tb + t_per);
  const bool m_vec = (M & 7) == 0;
  const int nvv = parts * JR * (CS / 8);

  // Act tile 64 t x 64 m = 512 vectors of 8: two per thread; V^T tile parts x JR x 64 t
  u32x4 ar[2], vr[NV];
  auto load = [&](int64_t s0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i, tt = v >> 3, mm = (v & 7) * 8;
      const int64_t tk = s0 + tt;
      ar[i] = tk < te ? load8(act + tk * M, m0 + mm, M, m_vec) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + 256 * i;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (v < nvv) {
        const int tv = v & 7, row = v >> 3;  // row = p * JR + jj
        const int p = row / JR, jj = row - p * JR;
        const int64_t tk = s0 + 8 * tv;
        // vt is zero past T up to Tp (a multiple of 8), and te is T or a multiple of CS, so a
        // vector that starts before te lies inside vt and holds zeros for tokens >= te
        if (tk < te && j0 + jj < rp)
          x = *reinterpret_cast<const u32x4*>(vt + ((int64_t)p * rp + j0 + jj) * Tp + tk);
      }
      vr[i] = x;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i, tt = v >> 3, mm = (v & 7) * 8;
      *reinterpret_cast<u32x4*>(&al[tt * ALD + mm]) = ar[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + 256 * i;
      if (v < nvv) {
        const int tv = v & 7, row = v >> 3;
        *reinterpret_cast<u32x4*>(&vl[row * VLD + 8 * tv]) = vr[i];
      }
    }
  };

  f32x4 acc[JT];
  double acc64[JT][4];
#pragma unroll
  for (int a = 0; a < JT; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[a][e] = 0.f;
      acc64[a][e] = 0.0;
    }
  if (tb < te) load(tb);
  for (int64_t s0 = tb; s0 < te; s0 += CS) {
    __syncthreads();  // the previous tile has been consumed
    store();
    __syncthreads();
    if (s0 + CS < te) load(s0 + CS);
#pragma unroll
    for (int k = 0; k < CS / 32; ++k) {
      if (s0 + 32 * k >= te) break;  // workgroup-uniform
      // B fragment: Act[t][m] for t = 32k + 8(l/16) .. +7 and m = 16w + l%16
      Frag bfr;
#pragma unroll
      for (int q = 0; q < 8; ++q) bfr.h[q] = al[(32 * k + 8 * lg + q) * ALD + 16 * w + lr];
#pragma unroll
      for (int a = 0; a < JT; ++a) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (p >= parts) break;
          const bf16x8v af = *reinterpret_cast<const bf16x8v*>(&vl[(p * JR + 16 * a + lr) * VLD + 32 * k + 8 * lg]);
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr.b, acc[a], 0, 0, 0);
        }
      }
      flush(acc, acc64);
    }
  }
  // D layout: row j = 4*(l/16)+e within j tile a, column m = l%16 of this wave's 16
  const int64_t m = m0 + 16 * w + lr;
  if (m >= M) return;
#pragma unroll
  for (int a = 0; a < JT; ++a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + 16 * a + 4 * lg + e;
      if (j >= r) continue;
      const double s = acc64[a][e];
      const int64_t o = out_t ? (int64_t)j * M + m : m * r + j;
      if (part)
        part[(int64_t)blockIdx.z * M * r + o] = s;
      else
        out[o] = (float)s;
    }
  }
}

// out[i] = sum_k part[k][i], summed in slice order
__global__ void k_reduce_parts(const double* __restrict__ part, int S, int64_t n,
                               float* __restrict__ out, double* __restrict__ out64, int r,
                               uint16_t* __restrict__ vt, int rp, int64_t Tp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  int k = 0;
  for (; k + 8 <= S; k += 8) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = part[(int64_t)(k + q) * n + i];
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  for (; k < S; ++k) s += part[(int64_t)k * n + i];
  if (out) out[i] = (float)s;
  if (out64) out64[i] = s;
  if (vt) write_vt4(vt, rp, Tp, (int)(i % r), i / r, s);  // rows output [T][r]
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int pick_jt(int r) { return r <= 16 ? 1 : r <= 32 ? 2 : 4; }

// Slices of the reduction so that about `target` workgroups run, each slice >= min_len long
// (a multiple of `quantum`); returns the slice length.
int64_t slice_len(int64_t blocks, int64_t len, int64_t min_len, int64_t quantum, int64_t target) {
  int64_t S = cdiv(target, blocks < 1 ? 1 : blocks);
  const int64_t max_s = cdiv(len, min_len);
  if (S > max_s) S = max_s;
  if (S > 64) S = 64;
  if (S < 1) S = 1;
  return round_up(cdiv(len, S), quantum);
}

struct RowsPlan {
  int jt, ub, S;
  int64_t c_per;
  size_t part_bytes;
};

// Slices of the reduction: none once the token x adapter blocks fill the GPU; with a medium
// number of blocks, slices of about 1024 columns (each wave then has two batches in flight);
// with few blocks (decode), enough slices for ~512 workgroups.
RowsPlan rows_plan(int64_t T, int64_t C, int r) {
  RowsPlan p;
  p.jt = pick_jt(r);
  p.ub = p.jt >= 4 ? 2 : 4;
  const int64_t quantum = 128 * p.ub;
  const int64_t blocks = cdiv(T, 16) * cdiv(r, 16 * p.jt);
  if (blocks >= 512) {
    p.c_per = round_up(C, quantum);
  } else if (blocks >= 64) {
    const int64_t s1 = cdiv(C, 1024), s2 = cdiv(1024, blocks);
    const int64_t S = s1 < s2 ? s1 : s2;
    p.c_per = round_up(cdiv(C, S < 1 ? 1 : S), quantum);
  } else {
    p.c_per = slice_len(blocks, C, quantum, quantum, 512);
  }
  p.S = (int)cdiv(C, p.c_per);
  p.part_bytes = p.S > 1 ? (size_t)p.S * T * r * sizeof(double) : 0;
  return p;
}

struct ColsPlan {
  int jt, S;
  int64_t t_per;
  size_t part_bytes;
};

ColsPlan cols_plan(int64_t T, int64_t M, int r) {
  ColsPlan p;
  p.jt = pick_jt(r);
  const int64_t blocks = cdiv(M, 64) * cdiv(r, 16 * p.jt);
  p.t_per = slice_len(blocks, T, 128, CS, 512);
  p.S = (int)cdiv(T, p.t_per);
  p.part_bytes = p.S > 1 ? (size_t)p.S * M * r * sizeof(double) : 0;
  return p;
}

template <int JT, int UB>
void rows_launch(dim3 grid, hipStream_t s, const uint16_t* act, int64_t T, int64_t C,
                 const uint16_t* wt, int64_t ldw, int r, int64_t c_per, double* part, float* out,
                 double* out64, uint16_t* vt, int rp, int64_t Tp) {
  sra::launch(SRA_KERNEL_ADAPTER, k_adapter_rows<JT, UB>, grid, dim3(256), 0, s, act, T, C, wt,
              ldw, r, c_per, part, out, out64, vt, rp, Tp);
}

template <int JT>
void cols_launch(dim3 grid, hipStream_t s, const uint16_t* act, int64_t T, int64_t M,
                 const uint16_t* vt, int parts, int r, int rp, int64_t Tp, int64_t t_per,
                 bool out_t, double* part, float* out) {
  sra::launch(SRA_KERNEL_ADAPTER, k_adapter_cols<JT>, grid, dim3(256), 0, s, act, T, M, vt, parts,
              r, rp, Tp, t_per, out_t, part, out);
}

}  // namespace

namespace sra {

int64_t vt_rows(int r) { return round_up(r, 16); }
int64_t vt_cols(int64_t T) { return round_up(T, 8); }
size_t adapter_vt_bytes(int64_t T, int r, int parts) {
  return align256((size_t)parts * vt_rows(r) * vt_cols(T) * 2);
}
int64_t packed_wt_ld(int64_t C) { return round_up(C, 8); }
size_t adapter_wt_bytes(int64_t C, int r) { return align256((size_t)r * packed_wt_ld(C) * 2); }

hipError_t launch_adapter_bwd_prep(const uint16_t* B, int64_t N, int r, uint16_t* wt,
                                   const float* U, int64_t T, uint16_t* vtU, hipStream_t s) {
  if (r == 0 || (!wt && !vtU)) return hipSuccess;
  const int pack_cx = wt ? (int)cdiv(N, 64) : 0;
  const int n_pack = wt ? pack_cx * (int)cdiv(r, 64) : 0;
  const int rp = (int)vt_rows(r);
  const int64_t Tp = vt_cols(T);
  const int n_split = vtU ? (int)cdiv((int64_t)rp * Tp, 256) : 0;
  if (n_pack + n_split == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_prep, dim3((unsigned)(n_pack + n_split)), dim3(256), 0, s, B, N, r,
                     packed_wt_ld(N), wt, n_pack, pack_cx > 0 ? pack_cx : 1, U, T, rp, Tp, vtU);
  return hipGetLastError();
}

size_t adapter_rows_ws(int64_t T, int64_t C, int r) {
  if (T <= 0 || C <= 0 || r <= 0) return 0;
  return rows_plan(T, C, r).part_bytes;
}

hipError_t launch_adapter_rows(const uint16_t* act, int64_t T, int64_t C, const uint16_t* wt,
                               int64_t ldw, int r, float* out, double* out64, uint16_t* vt,
                               void* ws, hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  if (C == 0) {
    if (out64 || vt) return hipErrorInvalidValue;  // callers never ask for fp64 with an empty reduction
    return launch_fill_f32(out, T * r, 0.f, s);
  }
  const RowsPlan p = rows_plan(T, C, r);
  double* part = p.S > 1 ? (double*)ws : nullptr;
  const int rp = (int)vt_rows(r);
  const int64_t Tp = vt_cols(T);
  const dim3 grid((unsigned)cdiv(T, 16), (unsigned)cdiv(r, 16 * p.jt), (unsigned)p.S);
  switch (p.jt) {
    case 1: rows_launch<1, 4>(grid, s, act, T, C, wt, ldw, r, p.c_per, part, out, out64, vt, rp, Tp); break;
    case 2: rows_launch<2, 4>(grid, s, act, T, C, wt, ldw, r, p.c_per, part, out, out64, vt, rp, Tp); break;
    default: rows_launch<4, 2>(grid, s, act, T, C, wt, ldw, r, p.c_per, part, out, out64, vt, rp, Tp); break;
  }
  if (p.S > 1) {
    const int64_t n = T * r;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, part, p.S,
                       n, out, out64, r, vt, rp, Tp);
  }
  return hipGetLastError();
}

size_t adapter_cols_ws(int64_t T, int64_t M, int r) {
  if (T <= 0 || M <= 0 || r <= 0) return 0;
  return cols_plan(T, M, r).part_bytes;
}

hipError_t launch_adapter_cols(const uint16_t* act, int64_t T, int64_t M, const uint16_t* vt,
                               int parts, int r, bool out_transposed, float* out, void* ws,
                               hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  if (T == 0) return launch_fill_f32(out, M * r, 0.f, s);
  const ColsPlan p = cols_plan(T, M, r);
  double* part = p.S > 1 ? (double*)ws : nullptr;
  const int rp = (int)vt_rows(r);
  const int64_t Tp = vt_cols(T);
  const dim3 grid((unsigned)cdiv(M, 64), (unsigned)cdiv(r, 16 * p.jt), (unsigned)p.S);
  switch (p.jt) {
    case 1: cols_launch<1>(grid, s, act, T, M, vt, parts, r, rp, Tp, p.t_per, out_transposed, part, out); break;
    case 2: cols_launch<2>(grid, s, act, T, M, vt, parts, r, rp, Tp, p.t_per, out_transposed, part, out); break;
    default: cols_launch<4>(grid, s, act, T, M, vt, parts, r, rp, Tp, p.t_per, out_transposed, part, out); break;
  }
  if (p.S > 1) {
    const int64_t n = M * r;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, part, p.S,
                       n, out, nullptr, r, nullptr, 0, 0);
  }
  return hipGetLastError();
}

}  // namespace sra

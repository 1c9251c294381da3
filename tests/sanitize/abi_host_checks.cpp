// Host-side checks of libsra under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Drives every argument check and workspace plan of the C ABI over a grid of shapes, ranks, flags,
// formats and tuning settings, with fake device pointers that are never dereferenced.  No call
// here reaches a kernel launch: each either fails validation, is a pure host query, or is a T = 0
// product call that returns before any launch.  A sanitizer report aborts the program; explicit
// expectations print and count their failures.  Exit status 0 with "all checks passed" on success.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "sra.h"

static int g_fail = 0, g_calls = 0;
// an aligned fake device address, convertible to any pointer type (never dereferenced)
struct Fake {
  template <class T>
  operator T*() const { return reinterpret_cast<T*>((uintptr_t)(1u << 20)); }
};
static const Fake FAKE{};

static void expect(bool ok, const char* what, int line) {
  if (!ok) {
    ++g_fail;
    std::printf("FAILED line %d: %s (%s)\n", line, what, sra_last_error());
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

static bool valid_status(sra_status s) {
  ++g_calls;
  return s == SRA_OK || s == SRA_ERR_INVALID_ARG || s == SRA_ERR_UNSUPPORTED || s == SRA_ERR_WORKSPACE;
}

static sra_sparse nm(int64_t rows, int64_t cols, int n, int m, int dtype, int fmt = SRA_FMT_NM) {
  sra_sparse d;
  std::memset(&d, 0, sizeof d);
  d.format = fmt;
  d.dtype = dtype;
  d.rows = rows;
  d.cols = cols;
  d.n = n;
  d.m = m;
  d.values = FAKE;
  d.meta = (uint32_t*)FAKE;
  return d;
}

static sra_sparse ell(int64_t rows, int64_t cols, int k, int dtype) {
  sra_sparse d;
  std::memset(&d, 0, sizeof d);
  d.format = SRA_FMT_ELL;
  d.dtype = dtype;
  d.rows = rows;
  d.cols = cols;
  d.k = k;
  d.values = FAKE;
  d.index = (int16_t*)FAKE;
  return d;
}

static const int64_t kDims[] = {0, 32, 64, 96, 128, 160, 1024, 4096, 5120, 9216, 20480, 36864};
static const int64_t kT[] = {0, 1, 5, 16, 17, 64, 300, 2048, 8192, 10240};
static const int kR[] = {0, 1, 16, 17, 32, 64, 128, 136, 256, 257, -1};

static void grid_queries() {
  const int pats[][2] = {{2, 4}, {1, 2}, {2, 8}, {1, 4}, {3, 8}};
  for (int64_t rows : kDims)
    for (int64_t cols : kDims)
      for (int64_t T : kT)
        for (int r : kR)
          for (const auto& pt : pats)
            for (int dtype = 0; dtype < 2; ++dtype)
              for (int fmt : {SRA_FMT_NM, SRA_FMT_NM_TILED}) {
                sra_sparse W = nm(rows, cols, pt[0], pt[1], dtype, fmt);
                size_t b = 0;
                sra_status s = sra_fwd_workspace(&W, T, r, &b);
                EXPECT(valid_status(s));
                if (s == SRA_OK) EXPECT(b < ((size_t)1 << 50));
                for (uint32_t flags : {1u, 2u, 4u, 7u, 9u, 15u, 16u}) {
                  s = sra_bwd_workspace(&W, T, r, flags, &b);
                  EXPECT(valid_status(s));
                  if (s == SRA_OK) EXPECT(b < ((size_t)1 << 50));
                }
              }
  for (int64_t rows : kDims)
    for (int64_t cols : kDims)
      for (int k : {0, 1, 7, 410, 32767, 40000}) {
        size_t b = 0;
        EXPECT(valid_status(sra_ffi_transpose_workspace(rows, cols, k, &b)));
        sra_sparse E = ell(rows, cols, k, SRA_BF16);
        for (int64_t T : kT) {
          sra_status s = sra_fwd_workspace(&E, T, 16, &b);
          EXPECT(valid_status(s));
          sra_sparse A = ell(32, cols, k, SRA_BF16);
          sra_sparse W = nm(rows, cols, 2, 4, SRA_BF16);
          EXPECT(valid_status(sra_ffa_fwd_workspace(&W, T, &A, &b)));
          sra_sparse P = nm(cols, rows, 2, 4, SRA_BF16);
          EXPECT(valid_status(sra_ffa_bwd_workspace(&P, T, &A, 7, &b)));
        }
      }
  for (int64_t cols = 0; cols <= 40000; cols += 8)
    for (int n = 0; n <= 9; ++n)
      for (int m = 0; m <= 9; ++m) EXPECT(sra_nm_meta_words(cols, n, m) >= 0);
  for (int64_t rows : kDims)
    for (int64_t cols : kDims) {
      size_t vb = 0, mb = 0;
      EXPECT(valid_status(sra_nm_tile_bytes(rows, cols, 2, 4, &vb, &mb)));
    }
}

static void tuning_sweep() {
  const int cfgs[] = {0, 3, 13, 14, 30, 50, 51, 55, 61, 62, 7, 99};
  const int splits[] = {0, 1, 2, 3, -2, 8, 64};
  for (int c : cfgs)
    for (int sp : splits)
      for (int engine = 0; engine < 2; ++engine)
        for (int fuse = 0; fuse < 2; ++fuse) {
          EXPECT(sra_set_tuning(SRA_TUNE_SPMM_CONFIG, c) == SRA_OK);
          EXPECT(sra_set_tuning(SRA_TUNE_SPMM_SPLITS, sp) == SRA_OK);
          EXPECT(sra_set_tuning(SRA_TUNE_ENGINE, engine) == SRA_OK);
          EXPECT(sra_set_tuning(SRA_TUNE_SPMM_FUSE, fuse) == SRA_OK);
          for (int64_t T : kT)
            for (int64_t rows : {128, 1024, 5120, 20480})
              for (int64_t cols : {64, 128, 1024, 5120, 20480})
                for (int r : {0, 8, 16, 128}) {
                  size_t b = 0;
                  sra_sparse W = nm(rows, cols, 2, 4, SRA_BF16);
                  EXPECT(valid_status(sra_fwd_workspace(&W, T, r, &b)));
                  EXPECT(valid_status(sra_bwd_workspace(&W, T, r, 7, &b)));
                  sra_sparse W8 = nm(rows, cols, 2, 8, SRA_BF16);
                  EXPECT(valid_status(sra_fwd_workspace(&W8, T, r, &b)));
                }
        }
  EXPECT(sra_set_tuning(SRA_TUNE_RESET, 0) == SRA_OK);
  for (int key = -1; key <= 9; ++key)
    for (int v : {-3, -2, -1, 0, 1, 2, 3, 4, 9, 100, 2000}) EXPECT(valid_status(sra_set_tuning(key, v)));
  EXPECT(sra_set_tuning(SRA_TUNE_RESET, 0) == SRA_OK);
}

static void rejections() {
  sra_sparse d = nm(64, 128, 2, 4, SRA_BF16);
  sra_sparse p = nm(128, 64, 2, 4, SRA_BF16);
  // compress / double prune / pairs: bad patterns, shapes, pointers
  EXPECT(sra_compress(FAKE, SRA_BF16, 64, 128, 2, 6, &d, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_compress(FAKE, SRA_BF16, 64, 100, 2, 4, &d, nullptr) == SRA_ERR_UNSUPPORTED);
  EXPECT(sra_compress(FAKE, 7, 64, 128, 2, 4, &d, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_compress(nullptr, SRA_BF16, 64, 128, 2, 4, &d, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_compress((char*)FAKE + 2, SRA_BF16, 64, 128, 2, 4, &d, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_compress(FAKE, SRA_BF16, 64, 128, 2, 4, nullptr, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_compress(FAKE, SRA_F32, 64, 128, 2, 8, &d, nullptr) == SRA_ERR_UNSUPPORTED);
  EXPECT(sra_double_prune(nullptr, &p, nullptr) == SRA_ERR_INVALID_ARG);
  sra_sparse bad = nm(-1, 128, 2, 4, SRA_BF16);
  EXPECT(sra_double_prune(&bad, &p, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_compress_pair(FAKE, SRA_BF16, 64, 128, 2, 8, &d, &p, nullptr) == SRA_ERR_UNSUPPORTED);
  EXPECT(sra_compress_pair_tiled(FAKE, SRA_BF16, 96, 128, 2, 4, &d, &p, nullptr) == SRA_ERR_UNSUPPORTED);
  EXPECT(sra_compress_ffi(FAKE, SRA_BF16, 64, 40000, 8, &d, nullptr) == SRA_ERR_INVALID_ARG);
  // products: NULL operands, small workspaces, CSR as a forward weight, T = 0 (no launch)
  size_t need = 0;
  sra_sparse W = nm(4096, 1024, 2, 4, SRA_BF16);
  EXPECT(sra_fwd_workspace(&W, 2048, 16, &need) == SRA_OK);
  EXPECT(sra_sparse_lora_fwd(&W, nullptr, 2048, FAKE, FAKE, 16, FAKE, nullptr, FAKE, need, nullptr) ==
         SRA_ERR_INVALID_ARG);
  EXPECT(need > 0);  // U goes to the workspace when U_out is NULL, so a zero-byte one is refused
  if (need > 0)
    EXPECT(sra_sparse_lora_fwd(&W, FAKE, 2048, FAKE, FAKE, 16, FAKE, nullptr, FAKE, 0, nullptr) ==
           SRA_ERR_WORKSPACE);
  EXPECT(sra_sparse_lora_fwd(&W, FAKE, 0, FAKE, FAKE, 16, FAKE, nullptr, FAKE, need, nullptr) == SRA_OK);
  sra_sparse csr;
  std::memset(&csr, 0, sizeof csr);
  csr.format = SRA_FMT_CSR;
  csr.rows = 1024;
  csr.cols = 4096;
  csr.nnz = 10;
  csr.values = FAKE;
  csr.index = (int16_t*)FAKE;
  csr.row_ptr = (int32_t*)FAKE;
  EXPECT(sra_fwd_workspace(&csr, 8, 4, &need) == SRA_ERR_INVALID_ARG);
  sra_sparse P = nm(1024, 4096, 2, 4, SRA_BF16);
  EXPECT(sra_bwd_workspace(&P, 2048, 16, 7, &need) == SRA_OK);
  EXPECT(sra_sparse_lora_bwd(&P, FAKE, FAKE, 2048, FAKE, FAKE, FAKE, 16, 7, nullptr, FAKE, FAKE, nullptr,
                             FAKE, need, nullptr) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_sparse_lora_bwd(&P, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 16, SRA_GRAD_DX, FAKE, nullptr, nullptr,
                             nullptr, FAKE, need, nullptr) == SRA_OK);
  // the allocation-free backward refuses oversized calls before any HIP call
  sra_sparse P13 = nm(5120, 20480, 2, 4, SRA_BF16);
  EXPECT(sra_sparse_lora_bwd_noalloc(&P13, FAKE, FAKE, 8192, nullptr, FAKE, FAKE, 128, 7, FAKE, FAKE, FAKE,
                                     nullptr, nullptr) == SRA_ERR_WORKSPACE);
  // fixed-fan-in adapter factor
  sra_sparse A = ell(32, 1024, 100, SRA_BF16);
  EXPECT(sra_ffa_fwd_workspace(&W, 2048, &A, &need) == SRA_OK);
  sra_sparse Abad = ell(32, 512, 100, SRA_BF16);
  EXPECT(sra_ffa_fwd_workspace(&W, 2048, &Abad, &need) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_sparse_lora_fwd_ffa(&W, FAKE, 2048, &A, FAKE, FAKE, nullptr, FAKE, 16, nullptr) ==
         SRA_ERR_WORKSPACE);
  // weight gradient / update / streaming layout / profiling hook
  EXPECT(sra_masked_weight_grad(&d, FAKE, FAKE, -1, FAKE, nullptr) == SRA_ERR_INVALID_ARG);
  sra_sparse d8 = nm(64, 128, 2, 8, SRA_BF16);
  EXPECT(sra_masked_weight_grad(&d8, FAKE, FAKE, 16, FAKE, nullptr) == SRA_ERR_UNSUPPORTED);
  EXPECT(sra_nm_axpby(FAKE, 1.f, FAKE, 1.f, FAKE, -5, SRA_BF16, nullptr) == SRA_ERR_INVALID_ARG);
  sra_sparse d12 = nm(64, 128, 1, 2, SRA_BF16);
  EXPECT(sra_nm_tile(&d12, &p, nullptr) == SRA_ERR_UNSUPPORTED);  // the streaming layout is 2:4 or 2:8
  EXPECT(sra_time_next_kernel(77, FAKE, FAKE) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_time_next_kernel(3, nullptr, FAKE) == SRA_ERR_INVALID_ARG);
  EXPECT(sra_time_next_kernel(0, nullptr, nullptr) == SRA_OK);
}

int main() {
  EXPECT(sra_abi_version() == SRA_ABI_VERSION);
  grid_queries();
  tuning_sweep();
  rejections();
  if (g_fail) {
    std::printf("%d check(s) failed of %d calls\n", g_fail, g_calls);
    return 1;
  }
  std::printf("all checks passed (%d calls)\n", g_calls);
  return 0;
}

// 2:4 compression and double pruning (SLoPe paperlayer summary, §2.1 "Double-pruned backward
// pass": a fixed N:M mask chosen at initialisation, then the pruned weight is transposed and
// N:M-pruned again for the backward product; §2.3 keeps compressed forms of both).
//
// Both kernels are memory-bound one-pass rewrites.  Each lane owns whole 4-element groups, so the
// top-2 selection is a rank-by-count over four magnitude keys held in registers (six compares per
// group); no cross-lane traffic is needed for the first prune.  The second prune groups along the
// output dimension, which is strided in memory, so a 128 x 64 tile of the compressed weight is
// decompressed into LDS and each lane then ranks one column's groups.
#include "common.h"

namespace {

// Rank-by-count top-2 of 4 keys; returns positions p0 < p1 of the kept entries.
SRA_DEV void top2_of4(const uint32_t k[4], int& p0, int& p1) {
  int kept[2], nk = 0;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rank += (j != a) && ((k[j] > k[a]) || (k[j] == k[a] && j < a));
    if (rank < 2 && nk < 2) kept[nk++] = a;
  }
  p0 = kept[0];
  p1 = kept[1];
}

// One lane per 32-column block of a row: 8 groups -> 16 kept values + one metadata word.
template <typename T>
__global__ __launch_bounds__(256) void k_compress24(const T* __restrict__ W, int64_t rows,
                                                    int64_t words_per_row, T* __restrict__ vals,
                                                    uint32_t* __restrict__ meta) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte access
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * words_per_row) return;
  const int64_t row = id / words_per_row, w = id - row * words_per_row;
  const int64_t cols = words_per_row * 32;
  union { u32x4 v[32 / VEC]; T e[32]; } x;
  const u32x4* src = reinterpret_cast<const u32x4*>(W + row * cols + w * 32);
#pragma unroll
  for (int i = 0; i < 32 / VEC; ++i) x.v[i] = src[i];
  union { u32x4 v[16 / VEC]; T e[16]; } o;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t k[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) k[a] = mag_key(x.e[4 * g + a]);
    int p0, p1;
    top2_of4(k, p0, p1);
    o.e[2 * g] = x.e[4 * g + p0];
    o.e[2 * g + 1] = x.e[4 * g + p1];
    word |= (uint32_t)(p0 | (p1 << 2)) << (4 * g);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(vals + row * (cols / 2) + w * 16);
#pragma unroll
  for (int i = 0; i < 16 / VEC; ++i) dst[i] = o.v[i];
  meta[id] = word;
}

// Tile: 128 rows (outputs, the second prune's group dim) x 64 columns (inputs).
// Load phase: lane -> (row, 32-column half): decompress into key/value LDS tiles.  Keys are
// (magnitude + 1) for entries kept by the first prune and 0 otherwise, so ineligible entries rank
// below every eligible one and, among themselves, by index: a group with fewer than two eligible
// entries is completed with its lowest unused positions, whose value tile holds +0.0.
// Select phase: lane -> (column, 32-row block): rank the 8 groups of 4 rows, write one 16-value
// slice and one metadata word of P's row.
template <typename T>
__global__ __launch_bounds__(256) void k_double_prune24(const T* __restrict__ vals,
                                                        const uint32_t* __restrict__ meta,
                                                        int64_t rows, int64_t cols,
                                                        T* __restrict__ pv,
                                                        uint32_t* __restrict__ pm) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ uint32_t key[128][65];
  __shared__ T val[128][65];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 128;
  {
    const int lr = tid >> 1, h = tid & 1;
    const int64_t row = r0 + lr, cb = c0 + 32 * h;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      key[lr][32 * h + i] = 0;
      val[lr][32 * h + i] = (T)0;
    }
    if (row < rows && cb < cols) {
      union { u32x4 v[16 / VEC]; T e[16]; } x;
      const u32x4* src = reinterpret_cast<const u32x4*>(vals + row * (cols / 2) + cb / 2);
#pragma unroll
      for (int i = 0; i < 16 / VEC; ++i) x.v[i] = src[i];
      const uint32_t word = meta[row * (cols / 32) + cb / 32];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int p0 = (word >> (4 * g)) & 3, p1 = (word >> (4 * g + 2)) & 3;
        key[lr][32 * h + 4 * g + p0] = mag_key(x.e[2 * g]) + 1;
        val[lr][32 * h + 4 * g + p0] = x.e[2 * g];
        key[lr][32 * h + 4 * g + p1] = mag_key(x.e[2 * g + 1]) + 1;
        val[lr][32 * h + 4 * g + p1] = x.e[2 * g + 1];
      }
    }
  }
  __syncthreads();
  const int c = tid & 63, b = tid >> 6;
  const int64_t prow = c0 + c, ostart = r0 + 32 * b;
  if (prow >= cols || ostart >= rows) return;
  union { u32x4 v[16 / VEC]; T e[16]; } o;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t k[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) k[a] = key[32 * b + 4 * g + a][c];
    int p0, p1;
    top2_of4(k, p0, p1);
    o.e[2 * g] = val[32 * b + 4 * g + p0][c];
    o.e[2 * g + 1] = val[32 * b + 4 * g + p1][c];
    word |= (uint32_t)(p0 | (p1 << 2)) << (4 * g);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(pv + prow * (rows / 2) + ostart / 2);
#pragma unroll
  for (int i = 0; i < 16 / VEC; ++i) dst[i] = o.v[i];
  pm[prow * (rows / 32) + ostart / 32] = word;
}

// Both prunes in one pass over W, for training loops that refresh Ws and P together after each
// weight update: a 128 x 64 tile of W is read once; each lane ranks one row's 32-column block (the
// first prune, written to Ws as in k_compress24) and drops the survivors' keys and values into the
// LDS tiles the second prune reads (as k_double_prune24 builds them from Ws), then each lane ranks
// one column's 32-row block and writes P.  Same selection code, so the bits match the two-kernel
// path exactly.
template <typename T>
__global__ __launch_bounds__(256) void k_compress_pair24(const T* __restrict__ W, int64_t rows,
                                                         int64_t cols, T* __restrict__ vals,
                                                         uint32_t* __restrict__ meta,
                                                         T* __restrict__ pv,
                                                         uint32_t* __restrict__ pm) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ uint32_t key[128][65];
  __shared__ T val[128][65];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 128;
  {
    const int lr = tid >> 1, h = tid & 1;
    const int64_t row = r0 + lr, cb = c0 + 32 * h;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      key[lr][32 * h + i] = 0;
      val[lr][32 * h + i] = (T)0;
    }
    if (row < rows && cb < cols) {
      union { u32x4 v[32 / VEC]; T e[32]; } x;
      const u32x4* src = reinterpret_cast<const u32x4*>(W + row * cols + cb);
#pragma unroll
      for (int i = 0; i < 32 / VEC; ++i) x.v[i] = src[i];
      union { u32x4 v[16 / VEC]; T e[16]; } o;
      uint32_t word = 0;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        uint32_t k[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) k[a] = mag_key(x.e[4 * g + a]);
        int p0, p1;
        top2_of4(k, p0, p1);
        o.e[2 * g] = x.e[4 * g + p0];
        o.e[2 * g + 1] = x.e[4 * g + p1];
        word |= (uint32_t)(p0 | (p1 << 2)) << (4 * g);
        key[lr][32 * h + 4 * g + p0] = k[p0] + 1;
        val[lr][32 * h + 4 * g + p0] = x.e[4 * g + p0];
        key[lr][32 * h + 4 * g + p1] = k[p1] + 1;
        val[lr][32 * h + 4 * g + p1] = x.e[4 * g + p1];
      }
      u32x4* dst = reinterpret_cast<u32x4*>(vals + row * (cols / 2) + cb / 2);
#pragma unroll
      for (int i = 0; i < 16 / VEC; ++i) dst[i] = o.v[i];
      meta[row * (cols / 32) + cb / 32] = word;
    }
  }
  __syncthreads();
  const int c = tid & 63, b = tid >> 6;
  const int64_t prow = c0 + c, ostart = r0 + 32 * b;
  if (prow >= cols || ostart >= rows) return;
  union { u32x4 v[16 / VEC]; T e[16]; } o;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t k[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) k[a] = key[32 * b + 4 * g + a][c];
    int p0, p1;
    top2_of4(k, p0, p1);
    o.e[2 * g] = val[32 * b + 4 * g + p0][c];
    o.e[2 * g + 1] = val[32 * b + 4 * g + p1][c];
    word |= (uint32_t)(p0 | (p1 << 2)) << (4 * g);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(pv + prow * (rows / 2) + ostart / 2);
#pragma unroll
  for (int i = 0; i < 16 / VEC; ++i) dst[i] = o.v[i];
  pm[prow * (rows / 32) + ostart / 32] = word;
}

}  // namespace

namespace sra {

hipError_t launch_compress_pair24(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                                  uint32_t* meta, void* p_vals, uint32_t* p_meta, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 127) / 128));
  if (dtype == SRA_BF16)
    launch(SRA_KERNEL_COMPRESS, k_compress_pair24<uint16_t>, grid, dim3(256), 0, s,
           (const uint16_t*)W, rows, cols, (uint16_t*)vals, meta, (uint16_t*)p_vals, p_meta);
  else
    launch(SRA_KERNEL_COMPRESS, k_compress_pair24<uint32_t>, grid, dim3(256), 0, s,
           (const uint32_t*)W, rows, cols, (uint32_t*)vals, meta, (uint32_t*)p_vals, p_meta);
  return hipGetLastError();
}

hipError_t launch_compress24(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                             uint32_t* meta, hipStream_t s) {
  const int64_t wpr = cols / 32, total = rows * wpr;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == SRA_BF16)
    launch(SRA_KERNEL_COMPRESS, k_compress24<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)W, rows,
                       wpr, (uint16_t*)vals, meta);
  else
    launch(SRA_KERNEL_COMPRESS, k_compress24<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)W, rows,
                       wpr, (uint32_t*)vals, meta);
  return hipGetLastError();
}

hipError_t launch_double_prune24(int dtype, const void* vals, const uint32_t* meta, int64_t rows,
                                 int64_t cols, void* p_vals, uint32_t* p_meta, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 127) / 128));
  if (dtype == SRA_BF16)
    launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune24<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)vals,
                       meta, rows, cols, (uint16_t*)p_vals, p_meta);
  else
    launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune24<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)vals,
                       meta, rows, cols, (uint32_t*)p_vals, p_meta);
  return hipGetLastError();
}

}  // namespace sra

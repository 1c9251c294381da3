// 2:4 compression and double pruning (SLoPe paperlayer summary, §2.1 "Double-pruned backward
// pass": a fixed N:M mask chosen at initialisation, then the pruned weight is transposed and
// N:M-pruned again for the backward product; §2.3 keeps compressed forms of both).
//
// All kernels are memory-bound one-pass rewrites.  Each lane owns whole 4-element groups, so the
// top-2 selection needs no cross-lane traffic for the first prune.  The second prune groups along
// the output dimension, which is strided in memory, so a tile of the first prune's output is
// expanded into LDS and each lane then ranks one column's groups.  bf16 (the training path) runs
// on 128 x 128 tiles with a branch-free selection (top2_net, gather2); fp32 keeps the
// rank-by-count selection on 128 x 64 tiles.
#include <algorithm>

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

// bf16 selection without branches or indexed registers: with the position folded into the low bits of
// each key (lower position = larger tiebreak), the four keys are distinct, a max/min network gives
// the largest and the second largest, their low bits give the positions, and one byte permute
// gathers both kept bf16 values from the group's two 32-bit words.  Same choice as top2_of4.
constexpr uint32_t kPrunedMark = 0xFFFFu;

// positions p0 < p1 of the two largest keys (k < 2^30; ties: the lower position wins)
SRA_DEV void top2_net(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3, uint32_t& p0, uint32_t& p1) {
  const uint32_t K0 = (k0 << 2) | 3u, K1 = (k1 << 2) | 2u, K2 = (k2 << 2) | 1u, K3 = k3 << 2;
  const uint32_t a = max(K0, K1), b = min(K0, K1), c = max(K2, K3), d = min(K2, K3);
  const uint32_t first = max(a, c), second = max(min(a, c), max(b, d));
  const uint32_t pa = 3u - (first & 3u), pb = 3u - (second & 3u);
  p0 = min(pa, pb);
  p1 = max(pa, pb);
}
// the bf16 values at positions p0, p1 of a group held as words lo = (x0, x1), hi = (x2, x3)
SRA_DEV uint32_t gather2(uint32_t lo, uint32_t hi, uint32_t p0, uint32_t p1) {
  const uint32_t sel = (p0 * 0x0202u + 0x0100u) | ((p1 * 0x0202u + 0x0100u) << 16);
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// the group's words with pruned halves replaced by the mark (kept: positions p0, p1)
SRA_DEV void mark_pruned(uint32_t& lo, uint32_t& hi, uint32_t p0, uint32_t p1) {
  const uint32_t m = (1u << p0) | (1u << p1);
  lo |= ((m & 1u) ? 0u : 0x0000FFFFu) | ((m & 2u) ? 0u : 0xFFFF0000u);
  hi |= ((m & 4u) ? 0u : 0x0000FFFFu) | ((m & 8u) ? 0u : 0xFFFF0000u);
}
SRA_DEV uint32_t second_key(uint32_t v) { return v == kPrunedMark ? 0u : (v & 0x7FFFu) + 1u; }


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
  union { u32x4 v[16 / VEC]; T e[16]; uint32_t w[8]; } o;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t lo = x.v[g / 2][2 * (g & 1)], hi = x.v[g / 2][2 * (g & 1) + 1];
      uint32_t p0, p1;
      top2_net(lo & 0x7FFFu, (lo >> 16) & 0x7FFFu, hi & 0x7FFFu, (hi >> 16) & 0x7FFFu, p0, p1);
      o.w[g] = gather2(lo, hi, p0, p1);
      word |= (p0 | (p1 << 2)) << (4 * g);
    } else {
      uint32_t k[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) k[a] = mag_key(x.e[4 * g + a]);
      int p0, p1;
      top2_of4(k, p0, p1);
      o.e[2 * g] = x.e[4 * g + p0];
      o.e[2 * g + 1] = x.e[4 * g + p1];
      word |= (uint32_t)(p0 | (p1 << 2)) << (4 * g);
    }
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
// weight update (fp32 weights; bf16 has the 128 x 128 tile kernel below): a 128 x 64 tile of W is
// read once; each lane ranks one row's 32-column block (the
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


// bf16 pair on 128 x 128 tiles, so that both outputs leave as whole 128-byte row segments: Ws rows
// (64 kept values of the tile's 128 columns) and P rows (64 kept values of its 128 rows).  The LDS
// tile holds the first prune's output in place -- kept values as they are, pruned positions as the
// NaN pattern 0xFFFF (weights are finite) -- and the second prune derives its magnitude keys from
// it (pruned: 0, kept: |w| key + 1), which is what the two-kernel path ranks.
//
// Second prune of a 128 x 128 LDS tile of the first prune's output (kept values, pruned positions
// marked): lane = (column, 64-row half), two 32-row blocks of 8 groups each; writes one 16-value
// slice and one metadata word of P's row per block.
constexpr int kTileLD = 128 + 8;  // LDS row stride (elements), 16-byte multiple

// Streaming 2:4 layout (the decode and streaming SpMM kernels' operand order): 1 KB value blocks per
// (16-row group, 64-column step), chunk 16q + i = stored values 32s + 8q .. +7 of row 16t + i;
// 1 KB metadata blocks per (16-row group, 512-column batch), row i's 16 words at 64i.
// Element offset of the 8 stored values from stored index j (j % 8 == 0) of `row`:
SRA_DEV int64_t tl_val(int64_t row, int64_t j, int64_t nsteps) {
  return (((row >> 4) * nsteps + (j >> 5)) * 64 + 16 * ((j & 31) >> 3) + (row & 15)) * 8;
}
// Word offset of metadata word w of `row`:
SRA_DEV int64_t tl_meta(int64_t row, int64_t w, int64_t nbat) {
  return ((row >> 4) * nbat + (w >> 4)) * 256 + (row & 15) * 16 + (w & 15);
}

template <bool TL>
SRA_DEV void second_prune_tile(const uint16_t* tile, int64_t c0, int64_t r0, int64_t rows,
                               int64_t cols, uint16_t* __restrict__ pv, uint32_t* __restrict__ pm) {
  constexpr int LD = kTileLD;
  const int tid = threadIdx.x;
  const int c = tid & 127, b = tid >> 7;
  const int64_t prow = c0 + c;
  if (prow >= cols) return;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int lr0 = 64 * b + 32 * q;
    const int64_t ostart = r0 + lr0;
    if (ostart >= rows) break;
    union { u32x4 v[2]; uint32_t w[8]; } o;
    uint32_t word = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      uint32_t v[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) v[a] = tile[(lr0 + 4 * g + a) * LD + c];
      uint32_t p0, p1;
      top2_net(second_key(v[0]), second_key(v[1]), second_key(v[2]), second_key(v[3]), p0, p1);
      uint32_t y = gather2(v[0] | (v[1] << 16), v[2] | (v[3] << 16), p0, p1);
      // a group with fewer than two survivors pads with +0.0
      if ((y & 0xFFFFu) == kPrunedMark) y &= 0xFFFF0000u;
      if ((y >> 16) == kPrunedMark) y &= 0x0000FFFFu;
      o.w[g] = y;
      word |= (p0 | (p1 << 2)) << (4 * g);
    }
    if constexpr (TL) {  // P rows have `rows` columns
      const int64_t ns = (rows + 63) / 64, nb = (rows + 511) / 512;
      *reinterpret_cast<u32x4*>(pv + tl_val(prow, ostart / 2, ns)) = o.v[0];
      *reinterpret_cast<u32x4*>(pv + tl_val(prow, ostart / 2 + 8, ns)) = o.v[1];
      pm[tl_meta(prow, ostart / 32, nb)] = word;
    } else {
      u32x4* dst = reinterpret_cast<u32x4*>(pv + prow * (rows / 2) + ostart / 2);
      dst[0] = o.v[0];
      dst[1] = o.v[1];
      pm[prow * (rows / 32) + ostart / 32] = word;
    }
  }
}

// TL: both outputs in the streaming layout (rows and cols multiples of 128).  ST: the W tile first
// crosses into LDS with coalesced row-run loads (faster for large W; for small W the extra pass
// adds latency, so lanes load their blocks directly).
template <bool TL, bool ST>
__global__ __launch_bounds__(256) void k_compress_pair24t(const uint16_t* __restrict__ W,
                                                          int64_t rows, int64_t cols,
                                                          uint16_t* __restrict__ vals,
                                                          uint32_t* __restrict__ meta,
                                                          uint16_t* __restrict__ pv,
                                                          uint32_t* __restrict__ pm) {
  constexpr int LD = kTileLD;
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * LD];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 128, r0 = (int64_t)blockIdx.y * 128;
  {
    // the W tile into LDS with coalesced 16-byte loads (a wave reads four 256-byte row runs;
    // non-temporal, every byte of W is read once); positions past the matrix hold the pruned mark
    if constexpr (ST) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int v = tid + 256 * k, lr = v >> 4, ch = v & 15;
        const int64_t row = r0 + lr, col = c0 + 8 * ch;
        u32x4 x = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
        if (row < rows && col < cols) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + row * cols + col));
        *reinterpret_cast<u32x4*>(&tile[lr * LD + 8 * ch]) = x;
      }
      __syncthreads();
    }
    // first prune: lane = (row, 64-column half), two 32-column blocks
    const int lr = tid >> 1, h = tid & 1;
    const int64_t row = r0 + lr;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int lc = 64 * h + 32 * q;
      const int64_t cb = c0 + lc;
      union { u32x4 v[4]; uint32_t w[16]; } x;
      if (row < rows && cb < cols) {
        if constexpr (ST) {
#pragma unroll
          for (int i = 0; i < 4; ++i) x.v[i] = *reinterpret_cast<const u32x4*>(&tile[lr * LD + lc + 8 * i]);
        } else {
          const u32x4* src = reinterpret_cast<const u32x4*>(W + row * cols + cb);
#pragma unroll
          for (int i = 0; i < 4; ++i) x.v[i] = src[i];
        }
        union { u32x4 v[2]; uint32_t w[8]; } o;
        uint32_t word = 0;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          uint32_t lo = x.w[2 * g], hi = x.w[2 * g + 1], p0, p1;
          top2_net(lo & 0x7FFFu, (lo >> 16) & 0x7FFFu, hi & 0x7FFFu, (hi >> 16) & 0x7FFFu, p0, p1);
          o.w[g] = gather2(lo, hi, p0, p1);
          word |= (p0 | (p1 << 2)) << (4 * g);
          mark_pruned(lo, hi, p0, p1);
          x.w[2 * g] = lo;
          x.w[2 * g + 1] = hi;
        }
        if constexpr (TL) {
          const int64_t ns = (cols + 63) / 64, nb = (cols + 511) / 512;
          *reinterpret_cast<u32x4*>(vals + tl_val(row, cb / 2, ns)) = o.v[0];
          *reinterpret_cast<u32x4*>(vals + tl_val(row, cb / 2 + 8, ns)) = o.v[1];
          meta[tl_meta(row, cb / 32, nb)] = word;
        } else {
          u32x4* dst = reinterpret_cast<u32x4*>(vals + row * (cols / 2) + cb / 2);
          dst[0] = o.v[0];
          dst[1] = o.v[1];
          meta[row * (cols / 32) + cb / 32] = word;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&tile[lr * LD + lc + 8 * i]) = x.v[i];
      } else if constexpr (!ST) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(&tile[lr * LD + lc + 8 * i]) =
              u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
      }
    }
  }
  __syncthreads();
  second_prune_tile<TL>(tile, c0, r0, rows, cols, pv, pm);
}


// bf16 double prune on 128 x 128 tiles of Ws (128 rows x 128 logical columns = 64 stored values,
// one 128-byte run per row): each lane expands one row's 64-column half into the LDS tile (kept
// values at their positions, the mark elsewhere, one byte permute per two positions), then the
// tile goes through the same second prune as the pair kernel.
__global__ __launch_bounds__(256) void k_double_prune24t(const uint16_t* __restrict__ vals,
                                                         const uint32_t* __restrict__ meta,
                                                         int64_t rows, int64_t cols,
                                                         uint16_t* __restrict__ pv,
                                                         uint32_t* __restrict__ pm) {
  constexpr int LD = kTileLD;
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * LD];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 128, r0 = (int64_t)blockIdx.y * 128;
  {
    const int lr = tid >> 1, h = tid & 1;
    const int64_t row = r0 + lr;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int lc = 64 * h + 32 * q;
      const int64_t cb = c0 + lc;
      union { u32x4 v[4]; uint32_t w[16]; } x;
      if (row < rows && cb < cols) {
        union { u32x4 v[2]; uint32_t w[8]; } in;
        const u32x4* src = reinterpret_cast<const u32x4*>(vals + row * (cols / 2) + cb / 2);
        in.v[0] = src[0];
        in.v[1] = src[1];
        const uint32_t word = meta[row * (cols / 32) + cb / 32];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint32_t p0 = (word >> (4 * g)) & 3u, p1 = (word >> (4 * g + 2)) & 3u;
          // byte pairs of {mark, mark : v1, v0}: v0 = 0x0100, v1 = 0x0302, mark = 0x0504
          uint32_t sel[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) sel[a] = a == (int)p0 ? 0x0100u : a == (int)p1 ? 0x0302u : 0x0504u;
          x.w[2 * g] = __builtin_amdgcn_perm(0xFFFFFFFFu, in.w[g], sel[0] | (sel[1] << 16));
          x.w[2 * g + 1] = __builtin_amdgcn_perm(0xFFFFFFFFu, in.w[g], sel[2] | (sel[3] << 16));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) x.v[i] = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&tile[lr * LD + lc + 8 * i]) = x.v[i];
    }
  }
  __syncthreads();
  second_prune_tile<false>(tile, c0, r0, rows, cols, pv, pm);
}

// ------------------------------------------------------------------------------------------------
// 1:2 (SLoPe §2.1 N:M pruning with N = 1, M = 2; its Lemma 2.1 figures cover 1:2).  Same canonical
// format: values [rows, cols/2] in ascending column order, one 2-bit field (the in-pair index) per
// stored value.  A 1:2 row keeps one entry of every column pair, so each group of four columns
// holds exactly two: the 2:4 SMFMAC kernels take it once each odd field gains 2 (the in-quad index
// of the pair's second half), i.e. metadata word | 0x88888888.

// One lane per 32-column block of a row: 16 pairs -> 16 kept values + one metadata word.
template <typename T>
__global__ __launch_bounds__(256) void k_compress12(const T* __restrict__ W, int64_t rows,
                                                    int64_t words_per_row, T* __restrict__ vals,
                                                    uint32_t* __restrict__ meta) {
  constexpr int VEC = 16 / sizeof(T);
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
  for (int g = 0; g < 16; ++g) {
    // larger magnitude first; equal magnitudes keep the lower index
    const uint32_t p = mag_key(x.e[2 * g + 1]) > mag_key(x.e[2 * g]) ? 1u : 0u;
    o.e[g] = x.e[2 * g + p];
    word |= p << (2 * g);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(vals + row * (cols / 2) + w * 16);
#pragma unroll
  for (int i = 0; i < 16 / VEC; ++i) dst[i] = o.v[i];
  meta[id] = word;
}

// Double prune of a 1:2 Ws (rows = N outputs, cols = K): P row k, pairs of output rows
// (2g, 2g+1): the eligible entries are those Ws keeps at column k (in-pair field == k & 1, value
// at stored index k/2); the larger eligible magnitude is kept (the lower row on ties); a pair with
// none eligible stores its first position with +0.0.  One lane per (stored index j, 32 output
// rows) writes both P rows k = 2j and 2j+1: a row's stored value at j belongs to exactly one of
// them, so each row is read once, 2 bytes per lane (128 bytes per wave load).
template <typename T>
__global__ __launch_bounds__(256) void k_double_prune12(const T* __restrict__ vals,
                                                        const uint32_t* __restrict__ meta,
                                                        int64_t rows, int64_t cols,
                                                        T* __restrict__ pv, uint32_t* __restrict__ pm) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= cols / 2) return;
  const int64_t n0 = (int64_t)blockIdx.y * 32;
  const int64_t mw = cols / 32;
  const int shift = (int)(2 * (j & 15));
  union { u32x4 v[16 / VEC]; T e[16]; } o[2];
  uint32_t word[2] = {0, 0};
#pragma unroll 4
  for (int g = 0; g < 16; ++g) {
    int f[2];
    T v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t n = n0 + 2 * g + e;
      f[e] = (int)((meta[n * mw + (j >> 4)] >> shift) & 3u);  // 0: row keeps column 2j, 1: 2j+1
      v[e] = vals[n * (cols / 2) + j];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // P row k = 2j + h
      const bool k0 = f[0] == h, k1 = f[1] == h;
      uint32_t p = 0;
      if (k0 && k1) p = mag_key(v[1]) > mag_key(v[0]) ? 1u : 0u;
      else if (k1) p = 1;
      o[h].e[g] = (p ? k1 : k0) ? v[p] : (T)0;
      word[h] |= p << (2 * g);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t k = 2 * j + h;
    u32x4* dst = reinterpret_cast<u32x4*>(pv + k * (rows / 2) + n0 / 2);
#pragma unroll
    for (int i = 0; i < 16 / VEC; ++i) dst[i] = o[h].v[i];
    pm[k * (rows / 32) + n0 / 32] = word[h];
  }
}

__global__ void k_meta_or(const uint32_t* __restrict__ in, uint32_t* __restrict__ out, int64_t n,
                          uint32_t bits) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = in[i] | bits;
}

// ---------------------------------------------------------------- 2:8 (bf16)
// Each 8-column group keeps its two largest magnitudes (ties: the lower position); positions are
// 3-bit fields, the two of a group in one byte (first at bits 0-2, second at 3-5), 4 groups per
// metadata word, values in ascending position order.

// positions p0 < p1 of the two largest of eight keys (k < 2^28; ties: the lower position wins)
SRA_DEV void top2_of8(const uint32_t k[8], uint32_t& p0, uint32_t& p1) {
  uint32_t K[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) K[j] = (k[j] << 3) | (uint32_t)(7 - j);  // distinct folded keys
  uint32_t first = K[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) first = max(first, K[j]);
  uint32_t second = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) second = max(second, K[j] == first ? 0u : K[j]);
  const uint32_t pa = 7u - (first & 7u), pb = 7u - (second & 7u);
  p0 = min(pa, pb);
  p1 = max(pa, pb);
}

// the word of a group's four words w[0..3] that holds position p (branch-free select)
SRA_DEV uint32_t word_at(const uint32_t w[4], uint32_t p) {
  const uint32_t q = p >> 1;
  const uint32_t a = (q & 1u) ? w[1] : w[0], b = (q & 1u) ? w[3] : w[2];
  return (q & 2u) ? b : a;
}

// One lane per 32-column block of a row: 4 groups -> 8 kept values (16 bytes) + one metadata word.
__global__ __launch_bounds__(256) void k_compress28(const uint16_t* __restrict__ W, int64_t rows,
                                                    int64_t words_per_row, uint16_t* __restrict__ vals,
                                                    uint32_t* __restrict__ meta) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * words_per_row) return;
  const int64_t row = id / words_per_row, w = id - row * words_per_row;
  const int64_t cols = words_per_row * 32;
  union { u32x4 v[4]; uint32_t w[16]; } x;
  const u32x4* src = reinterpret_cast<const u32x4*>(W + row * cols + w * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) x.v[i] = src[i];
  union { u32x4 v; uint32_t w[4]; } o;
  uint32_t word = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t* gw = &x.w[4 * g];
    uint32_t key[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) key[a] = (gw[a >> 1] >> (16 * (a & 1))) & 0x7FFFu;
    uint32_t p0, p1;
    top2_of8(key, p0, p1);
    const uint32_t lo = word_at(gw, p0), hi = word_at(gw, p1);
    const uint32_t sel = ((p0 & 1u) * 0x0202u + 0x0100u) | (((p1 & 1u) * 0x0202u + 0x0504u) << 16);
    o.w[g] = __builtin_amdgcn_perm(hi, lo, sel);
    word |= (p0 | (p1 << 3)) << (8 * g);
  }
  *reinterpret_cast<u32x4*>(vals + row * (cols / 4) + w * 8) = o.v;
  meta[row * words_per_row + w] = word;
}

// The second prune at 2:8 on 128-row x 64-column tiles of Ws: the tile's first-prune output is
// expanded into LDS (positions the first prune dropped hold the mark 0xFFFF), then each lane ranks
// four 8-row groups of one input column.  Keys: 0 for a dropped position, |w| + 1 for a kept one,
// with the position folded in as for the first prune, so the two largest are the kept entries by
// (|w| desc, row asc) and, when fewer than two were kept, the lowest unused positions (stored as
// +0.0).  P row k receives, per tile, 4 lanes x (8 values, 1 metadata word).
constexpr int kDp28Rows = 128, kDp28Cols = 64, kDp28Ld = kDp28Cols + 2;
__global__ __launch_bounds__(256) void k_double_prune28(const uint16_t* __restrict__ vals,
                                                        const uint32_t* __restrict__ meta, int64_t rows,
                                                        int64_t cols, uint16_t* __restrict__ p_vals,
                                                        uint32_t* __restrict__ p_meta) {
  __shared__ uint16_t t[kDp28Rows * kDp28Ld];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kDp28Rows, c0 = (int64_t)blockIdx.x * kDp28Cols;
  {  // expand: lane -> (row r0 + tid / 2, 32 columns from c0 + 32 (tid & 1))
    const int lr = tid >> 1, h = tid & 1;
    uint16_t* dst = t + lr * kDp28Ld + 32 * h;
#pragma unroll
    for (int e = 0; e < 32; ++e) dst[e] = (uint16_t)kPrunedMark;
    const int64_t row = r0 + lr, cb = c0 + 32 * h;
    if (row < rows && cb < cols) {
      union { u32x4 v; uint16_t h[8]; } x;
      x.v = *reinterpret_cast<const u32x4*>(vals + row * (cols / 4) + cb / 4);
      const uint32_t mw = meta[row * (cols / 32) + cb / 32];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t b = (mw >> (8 * g)) & 0xFFu;
        dst[8 * g + (b & 7u)] = x.h[2 * g];
        dst[8 * g + ((b >> 3) & 7u)] = x.h[2 * g + 1];
      }
    }
  }
  __syncthreads();
  const int lc = tid >> 2, q = tid & 3;
  const int64_t k = c0 + lc, g0 = r0 + 32 * q;  // input column; first output row of 4 groups
  if (k >= cols || g0 >= rows) return;
  union { u32x4 v; uint16_t h[8]; } o;
  uint32_t word = 0;
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    const uint16_t* col = t + (32 * q + 8 * gg) * kDp28Ld + lc;
    uint32_t key[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const uint32_t v = col[a * kDp28Ld];
      key[a] = v == kPrunedMark ? 0u : (v & 0x7FFFu) + 1u;
    }
    uint32_t p0, p1;
    top2_of8(key, p0, p1);
    const uint32_t v0 = col[p0 * kDp28Ld], v1 = col[p1 * kDp28Ld];
    o.h[2 * gg] = (uint16_t)(v0 == kPrunedMark ? 0u : v0);
    o.h[2 * gg + 1] = (uint16_t)(v1 == kPrunedMark ? 0u : v1);
    word |= (p0 | (p1 << 3)) << (8 * gg);
  }
  *reinterpret_cast<u32x4*>(p_vals + k * (rows / 4) + g0 / 4) = o.v;
  p_meta[k * (rows / 32) + g0 / 32] = word;
}

// 2:8 rows as 2:4 rows.  A 2:8 row keeps two entries of every eight columns, so each group of four
// holds at most two of them: the row is a 2:4 row once each four-column half is filled up to two
// stored values with +0.0 at its lowest unused positions (the zeros add nothing to any product).
// One lane per 32-column block: 8 values and one 2:8 metadata word in, 16 values and one 2:4
// metadata word out (both formats keep one word per 32 columns).
// Rows are whole metadata words, so metadata word i covers 2:8 values [8i, 8i + 8) and 2:4
// values [16i, 16i + 16) of the flat arrays: one lane per word, no row arithmetic. The 2:8 arrays
// are read once per call and not again by the product, so their loads bypass the caches.
// TL: the 2:8 weight is in its streaming layout (16-row x 256-column blocks: 2 KB of values, lane
// l = 16 q + i holding row i's chunk c at 1024 c + 16 l, and 512 bytes of metadata, lane l's two
// words at 8 l), where word w of row r is chunk / word w % 2 of lane 16 ((w % 8) / 2) + r % 16 in
// block (r / 16, w / 8); the 2:4 output is canonical either way.
template <bool TL>
__global__ __launch_bounds__(256) void k_nm28_to24(const uint16_t* __restrict__ v8,
                                                   const uint32_t* __restrict__ m8, int64_t words,
                                                   int64_t words_per_row,
                                                   uint16_t* __restrict__ v4,
                                                   uint32_t* __restrict__ m4) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= words) return;
  int64_t vi = id, mi = id;  // 16-byte value chunk and metadata word of this lane's input
  if constexpr (TL) {
    const int64_t row = id / words_per_row, w = id - row * words_per_row, nb = (words_per_row + 7) / 8;
    const int64_t blk = (row / 16) * nb + w / 8;
    const int l = (int)(16 * ((w & 7) >> 1) + (row & 15)), c = (int)(w & 1);
    vi = blk * 128 + 64 * c + l;
    mi = blk * 128 + 2 * l + c;
  }
  union { u32x4 v; uint16_t h[8]; } in;
  in.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v8) + vi);
  const uint32_t word8 = __builtin_nontemporal_load(m8 + mi);
  union { u32x4 v[2]; uint16_t h[16]; } out;
  uint32_t word4 = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t byte = (word8 >> (8 * g)) & 0xFFu, p0 = byte & 7u, p1 = (byte >> 3) & 7u;
    const uint16_t a = in.h[2 * g], b = in.h[2 * g + 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t lo = 4u * h;
      const bool k0 = p0 >= lo && p0 < lo + 4, k1 = p1 >= lo && p1 < lo + 4;
      uint32_t q0, q1;
      uint16_t x0, x1;
      if (k0 && k1) {
        q0 = p0 - lo; q1 = p1 - lo; x0 = a; x1 = b;
      } else if (k0 || k1) {
        const uint32_t q = (k0 ? p0 : p1) - lo, z = q == 0 ? 1u : 0u;
        const uint16_t v = k0 ? a : b;
        if (z < q) { q0 = z; q1 = q; x0 = 0; x1 = v; }
        else { q0 = q; q1 = z; x0 = v; x1 = 0; }
      } else {
        q0 = 0; q1 = 1; x0 = 0; x1 = 0;
      }
      const int grp = 2 * g + h;  // four-column group of the block
      out.h[2 * grp] = x0;
      out.h[2 * grp + 1] = x1;
      word4 |= (q0 | (q1 << 2)) << (4 * grp);
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(v4) + 2 * id;
  dst[0] = out.v[0];
  dst[1] = out.v[1];
  m4[id] = word4;
}

}  // namespace

namespace sra {

hipError_t launch_nm28_to24(const uint16_t* v8, const uint32_t* m8, int64_t rows, int64_t cols,
                            uint16_t* v4, uint32_t* m4, hipStream_t s, bool tiled) {
  const int64_t wpr = cols / 32, total = rows * wpr;
  if (total == 0) return hipSuccess;
  if (cols % 32) return hipErrorInvalidValue;
  if (tiled)
    launch(SRA_KERNEL_COMPRESS, k_nm28_to24<true>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
           v8, m8, total, wpr, v4, m4);
  else
    launch(SRA_KERNEL_COMPRESS, k_nm28_to24<false>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
           v8, m8, total, wpr, v4, m4);
  return hipGetLastError();
}

hipError_t launch_compress28(const uint16_t* W, int64_t rows, int64_t cols, uint16_t* vals, uint32_t* meta,
                             hipStream_t s) {
  const int64_t wpr = cols / 32, total = rows * wpr;
  if (total == 0) return hipSuccess;
  if (cols % 32) return hipErrorInvalidValue;
  launch(SRA_KERNEL_COMPRESS, k_compress28, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W,
         rows, wpr, vals, meta);
  return hipGetLastError();
}

hipError_t launch_double_prune28(const uint16_t* vals, const uint32_t* meta, int64_t rows, int64_t cols,
                                 uint16_t* p_vals, uint32_t* p_meta, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows % 32 || cols % 32) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols + kDp28Cols - 1) / kDp28Cols), (unsigned)((rows + kDp28Rows - 1) / kDp28Rows));
  launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune28, grid, dim3(256), 0, s, vals, meta, rows, cols, p_vals,
         p_meta);
  return hipGetLastError();
}

// W elements from which the pair kernel stages its tile through LDS first (OPT-13B-sized weights,
// 105M elements, gain; OPT-350M-sized ones, 4M, do not)
constexpr int64_t kPairStageElems = (int64_t)1 << 25;

hipError_t launch_compress_pair24(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                                  uint32_t* meta, void* p_vals, uint32_t* p_meta, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (dtype == SRA_BF16) {
    const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
    if (rows * cols >= kPairStageElems)
      launch(SRA_KERNEL_COMPRESS, k_compress_pair24t<false, true>, grid, dim3(256), 0, s, (const uint16_t*)W,
             rows, cols, (uint16_t*)vals, meta, (uint16_t*)p_vals, p_meta);
    else
      launch(SRA_KERNEL_COMPRESS, k_compress_pair24t<false, false>, grid, dim3(256), 0, s, (const uint16_t*)W,
             rows, cols, (uint16_t*)vals, meta, (uint16_t*)p_vals, p_meta);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 127) / 128));
  launch(SRA_KERNEL_COMPRESS, k_compress_pair24<uint32_t>, grid, dim3(256), 0, s,
         (const uint32_t*)W, rows, cols, (uint32_t*)vals, meta, (uint32_t*)p_vals, p_meta);
  return hipGetLastError();
}

hipError_t launch_compress_pair24_tiled(const uint16_t* W, int64_t rows, int64_t cols, void* vals,
                                        uint32_t* meta, void* p_vals, uint32_t* p_meta, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows % 128 != 0 || cols % 128 != 0) return hipErrorInvalidValue;
  // metadata words past a row's end inside its last 512-column batch are not written by the
  // kernel: clear them first (only when a batch is partial)
  if (cols % 512 != 0) {
    const hipError_t e = launch_fill_f32((float*)meta, rows / 16 * ((cols + 511) / 512) * 256, 0.f, s);
    if (e != hipSuccess) return e;
  }
  if (rows % 512 != 0) {
    const hipError_t e = launch_fill_f32((float*)p_meta, cols / 16 * ((rows + 511) / 512) * 256, 0.f, s);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128));
  if (rows * cols < kPairStageElems)
    launch(SRA_KERNEL_COMPRESS, k_compress_pair24t<true, false>, grid, dim3(256), 0, s, W, rows, cols,
           (uint16_t*)vals, meta, (uint16_t*)p_vals, p_meta);
  else
    launch(SRA_KERNEL_COMPRESS, k_compress_pair24t<true, true>, grid, dim3(256), 0, s, W, rows, cols,
           (uint16_t*)vals, meta, (uint16_t*)p_vals, p_meta);
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
  if (dtype == SRA_BF16) {
    const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
    launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune24t, grid, dim3(256), 0, s, (const uint16_t*)vals,
           meta, rows, cols, (uint16_t*)p_vals, p_meta);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 127) / 128));
  launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune24<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)vals,
         meta, rows, cols, (uint32_t*)p_vals, p_meta);
  return hipGetLastError();
}

hipError_t launch_compress12(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                             uint32_t* meta, hipStream_t s) {
  const int64_t wpr = cols / 32, total = rows * wpr;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == SRA_BF16)
    launch(SRA_KERNEL_COMPRESS, k_compress12<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)W, rows,
           wpr, (uint16_t*)vals, meta);
  else
    launch(SRA_KERNEL_COMPRESS, k_compress12<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)W, rows,
           wpr, (uint32_t*)vals, meta);
  return hipGetLastError();
}

hipError_t launch_double_prune12(int dtype, const void* vals, const uint32_t* meta, int64_t rows,
                                 int64_t cols, void* p_vals, uint32_t* p_meta, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows % 32 || cols % 32) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols / 2 + 255) / 256), (unsigned)(rows / 32));
  if (dtype == SRA_BF16)
    launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune12<uint16_t>, grid, dim3(256), 0, s,
           (const uint16_t*)vals, meta, rows, cols, (uint16_t*)p_vals, p_meta);
  else
    launch(SRA_KERNEL_DOUBLE_PRUNE, k_double_prune12<uint32_t>, grid, dim3(256), 0, s,
           (const uint32_t*)vals, meta, rows, cols, (uint32_t*)p_vals, p_meta);
  return hipGetLastError();
}

hipError_t launch_meta_or(const uint32_t* in, uint32_t* out, int64_t n, uint32_t bits, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_meta_or, dim3(grid), dim3(256), 0, s, in, out, n, bits);
  return hipGetLastError();
}

}  // namespace sra

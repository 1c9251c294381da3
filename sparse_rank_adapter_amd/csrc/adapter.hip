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
//   bf16 parts [part][j][t] -- three parts of an fp32 V, an exact split (U, split by the backward
//   prep kernel; dU, summed in fp64 by the rows kernel that produces it and rounded once to fp32,
//   the dU the call returns) -- which read as contiguous 16-byte fragments.
// Both use v_mfma_f32_16x16x32_bf16 and move every 32-step MFMA partial into fp64 registers (fp32
// rounding only acts inside one 32-term dot product); slices write fp64 partials that one more
// kernel sums in a fixed order, so results are independent of scheduling.
#include <cstdlib>

#include "common.h"

namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

union Frag {
  u32x4 v;
  uint16_t h[8];
  bf16x8v b;
};

// s_waitcnt vmcnt(N) only (expcnt / lgkmcnt left at their maxima), gfx9 encoding
template <int N>
SRA_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// With n stages of L transfers each in flight (1 <= n <= D), wait for the oldest stage.
template <int L, int D>
SRA_DEV void wait_inflight(int n) {
  if constexpr (D > 1) {
    if (n >= D) {
      wait_vm<((D - 1) * L < 63 ? (D - 1) * L : 63)>();
      return;
    }
    wait_inflight<L, D - 1>(n);
  } else {
    wait_vm<0>();
  }
}

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
// When vt is non-null the result is also written as V^T split into three bf16 parts (write_vt3),
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
          for (int p = 0; p < 3; ++p) vt[((int64_t)p * rp + j) * Tp + tt + e] = 0;
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
        if (vt) write_vt3(vt, rp, Tp, j, tt, s);
      }
    }
  }
}

// dst[y][x] = src[x][y] for a 64 x 64 tile (src rows x < X of Y elements, dst rows of stride ld),
// transposed through LDS so reads and writes are coalesced; 256 threads.
SRA_DEV void transpose_tile(const uint16_t* __restrict__ src, int64_t X, int64_t Y,
                            uint16_t* __restrict__ dst, int64_t ld, int64_t x0, int64_t y0,
                            uint16_t (*tile)[65]) {
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 4 rows at a time
  uint16_t v[16];  // all loads issued before the first LDS store
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t x = x0 + ty + 4 * k, y = y0 + tx;
    v[k] = (x < X && y < Y) ? src[x * Y + y] : (uint16_t)0;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) tile[ty + 4 * k][tx] = v[k];
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t y = y0 + i, x = x0 + tx;
    if (y < Y && x < X) dst[y * ld + x] = tile[tx][i];
  }
}

// Backward prep, one launch for the independent inputs of the adapter products:
//   blocks [0, nb):        wt[j][c] = B[c][j] (c < C, j < r; rows of stride ldw), the dU operand;
//   blocks [nb, nb + na):  at[k][j] = A[j][k] (k < K, j < r; rows of stride lda), the dX epilogue's
//                          E operand as 16-byte rows;
//   blocks [nb + na, ..):  vt[p][j][t], U^T split into three bf16 parts (j < rp, t < Tp, zero
//                          outside r x T), 256 entries per block.
struct PrepArgs {
  const uint16_t* B;
  int64_t C, ldw;
  uint16_t* wt;
  int nb, b_cx;  // B^T tiles, tiles along C
  const uint16_t* A;
  int64_t K, lda;
  uint16_t* at;
  int na, a_cx;  // A^T tiles, tiles along K
  const float* U;
  int64_t T, Tp;
  int r, rp;
  uint16_t* vt;
};
__global__ void k_bwd_prep(PrepArgs pa) {
  __shared__ uint16_t tile[64][65];
  const int bid = blockIdx.x;
  if (bid < pa.nb) {
    transpose_tile(pa.B, pa.C, pa.r, pa.wt, pa.ldw, (int64_t)(bid % pa.b_cx) * 64,
                   (int64_t)(bid / pa.b_cx) * 64, tile);
    return;
  }
  if (bid < pa.nb + pa.na) {
    const int b = bid - pa.nb;
    transpose_tile(pa.A, pa.r, pa.K, pa.at, pa.lda, (int64_t)(b / pa.a_cx) * 64,
                   (int64_t)(b % pa.a_cx) * 64, tile);
    return;
  }
  const int64_t i = (int64_t)(bid - pa.nb - pa.na) * 256 + threadIdx.x;  // i = j * Tp + t
  if (i >= (int64_t)pa.rp * pa.Tp) return;
  const int j = (int)(i / pa.Tp);
  const int64_t t = i - (int64_t)j * pa.Tp;
  uint16_t p[3] = {0, 0, 0};
  if (j < pa.r && t < pa.T) split3_bf16(pa.U[t * pa.r + j], p[0], p[1], p[2]);
  for (int q = 0; q < 3; ++q) pa.vt[((int64_t)q * pa.rp + j) * pa.Tp + t] = p[q];
}

// ------------------------------------------------------------------------------------ cols
constexpr int CS = 64;        // tokens per staged tile
constexpr int ALD = 64 + 8;   // LDS row of the Act tile [t][m] (elements; 144 B keeps 16 B alignment)
constexpr int VLD = CS + 8;   // LDS row of the V^T tile [j][t]

// V^T parts: vt[p][j][t] for j < rp (r rounded up to 16) and t < Tp (T rounded up to 8; columns
// past T are 0).  U -> 3 parts written by the backward prep kernel, dU -> 3 parts of its fp32 value
// written by the rows kernel (or its slice reduction).  The kernels take 1 to 4 parts.

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
// U = Act G^T for a few tokens (T <= 16), in one launch: workgroup (j0 / 4, t) computes
// U[t][j0 .. j0+3] over the whole reduction.  Each thread takes 16-byte chunks c = tid, tid + 256,
// ... of the token's row and of the four G rows, accumulates exact products in fp64, and the
// workgroup sums the 256 partials through LDS in a fixed tree order (deterministic).  Columns
// j0 + jj >= r accumulate a clamped row and are never written.  A split of
// the reduction over workgroups would need a second launch for the sum; with few tokens both
// launches are latency-bound, so this one reads the token row once per four adapter columns
// instead.  Needs C % 8 == 0, 16-byte aligned rows (ldw % 8 == 0).
constexpr int kFewJ = 4;
__global__ __launch_bounds__(256) void k_adapter_rows_few(const uint16_t* __restrict__ act, int64_t C,
                                                         const uint16_t* __restrict__ wt, int64_t ldw,
                                                         int r, float* __restrict__ out) {
  __shared__ double red[kFewJ][256];
  const int tid = threadIdx.x;
  // grid (column groups, tokens): consecutive workgroup ids go to different XCDs, so with a
  // multiple of 8 column groups every token of one group runs on the same XCD and its G rows
  // come from that XCD's L2 after the first read
  const int64_t t = blockIdx.y;
  const int j0 = blockIdx.x * kFewJ;
  const uint16_t* xrow = act + t * C;
  double acc[kFewJ] = {0.0, 0.0, 0.0, 0.0};
  // every load of a block of NCH chunks is issued before the first product, so the reduction
  // costs one memory round trip per 256 * NCH chunks instead of one per chunk
  constexpr int NCH = 5;
  const int64_t nch = C / 8;
  for (int64_t base = 0; base < nch; base += 256 * NCH) {
    u32x4 xv[NCH], gv[NCH][kFewJ];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int64_t c = base + tid + 256 * k;
      const bool in = c < nch;
      xv[k] = in ? *reinterpret_cast<const u32x4*>(xrow + 8 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < kFewJ; ++jj) {
        const int j = min(j0 + jj, r - 1);  // columns past r: a valid row, never accumulated
        gv[k][jj] = in ? *reinterpret_cast<const u32x4*>(wt + (int64_t)j * ldw + 8 * c) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int jj = 0; jj < kFewJ; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __uint_as_float(xv[k][e] << 16), x1 = __uint_as_float(xv[k][e] & 0xffff0000u);
          const float g0 = __uint_as_float(gv[k][jj][e] << 16), g1 = __uint_as_float(gv[k][jj][e] & 0xffff0000u);
          acc[jj] += (double)(x0 * g0);  // bf16 x bf16 is exact in fp32
          acc[jj] += (double)(x1 * g1);
        }
  }
#pragma unroll
  for (int jj = 0; jj < kFewJ; ++jj) red[jj][tid] = acc[jj];
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) {
#pragma unroll
      for (int jj = 0; jj < kFewJ; ++jj) red[jj][tid] += red[jj][tid + h];
    }
    __syncthreads();
  }
  if (tid < kFewJ && j0 + tid < r) out[t * r + j0 + tid] = (float)red[tid][0];
}

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
  if (vt) write_vt3(vt, rp, Tp, (int)(i % r), i / r, s);  // rows output [T][r]
}

// The same sum for a block of 32 tokens x 64 ranks when V^T's parts are written too: the partials
// are read and out / out64 written along the ranks, the fp32 sums go through LDS, and each part
// row of V^T is written along the tokens (the per-element kernel above writes those parts
// T columns apart, two bytes at a time).
__global__ __launch_bounds__(256) void k_reduce_parts_vt(const double* __restrict__ part, int S, int64_t T,
                                                         int r, float* __restrict__ out,
                                                         double* __restrict__ out64,
                                                         uint16_t* __restrict__ vt, int rp, int64_t Tp) {
  __shared__ float tile[64][33];  // [rank][token]
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 32, n = T * r;
  const int j0 = blockIdx.y * 64;
  // eight elements per thread, all of their loads of four slices in flight before the adds (the
  // sums keep the slice order of the per-element kernel)
  const int jj = tid & 63, j = j0 + jj;
  int64_t idx[8];
  bool ok[8];
  double sum[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t t = t0 + (tid >> 6) + 4 * q;
    ok[q] = t < T && j < r;
    idx[q] = ok[q] ? t * r + j : 0;
    sum[q] = 0.0;
  }
  for (int k = 0; k < S; k += 4) {
    double v[8][4];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) v[q][u] = k + u < S ? part[(int64_t)(k + u) * n + idx[q]] : 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k + u < S) sum[q] += v[q][u];
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if (ok[q]) {
      if (out) out[idx[q]] = (float)sum[q];
      if (out64) out64[idx[q]] = sum[q];
      tile[jj][(tid >> 6) + 4 * q] = (float)sum[q];
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int tt = tid & 31, jj = (tid >> 5) + 8 * q;
    const int64_t t = t0 + tt;
    const int j = j0 + jj;
    if (t < T && j < r) {
      uint16_t p3[3];
      split3_bf16(tile[jj][tt], p3[0], p3[1], p3[2]);
#pragma unroll
      for (int p = 0; p < 3; ++p) vt[((int64_t)p * rp + j) * Tp + t] = p3[p];
    }
  }
}

// Sum of the S fp64 slice partials of a [T][r] adapter product: per element, or tiled when V^T's
// parts are written as well.
void reduce_parts(const double* part, int S, int64_t T, int r, float* out, double* out64, uint16_t* vt,
                  int rp, int64_t Tp, hipStream_t s) {
  const int64_t n = T * r;
  if (vt)
    hipLaunchKernelGGL(k_reduce_parts_vt, dim3((unsigned)((T + 31) / 32), (unsigned)((r + 63) / 64)), dim3(256),
                       0, s, part, S, T, r, out, out64, vt, rp, Tp);
  else
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, S, n, out,
                       out64, r, vt, rp, Tp);
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


// ------------------------------------------------------------------------------------ grads
// Both adapter gradients of the backward in one launch: each "job" is a cols product
// Out[m][j] = sum_t Act[t][m] V[t][j] (dB: Act = dY, V = U; dA: Act = X, V = dU, transposed out).
// A workgroup owns 64 columns m x 16*JT adapter rows j x one slice of tokens; grid.x runs over the
// column blocks of the first job, then the second.  Tokens stream through an LDS ring of NS stages
// of ST = 32*KG tokens, filled by buffer -> LDS DMA: every token row of the Act tile (128 bytes)
// and every V^T row (part p, row j; 2*ST bytes) of a stage is one run, and rows past the slice or
// past T read as zeros.  The 4*KG waves split a stage into 4 column fragments x KG 32-token groups,
// so each wave's MFMA chain per stage is short and every SIMD holds KG waves; the KG partial sums
// of a fragment are added in a fixed order through LDS at the end.
// Swizzles (16-byte chunk c of LDS row x holds source chunk c ^ s(x)): Act rows s = 2((x>>3)&3), so
// the four 8-token groups of a transposed 2-byte read fall on different banks; V^T rows
// s = x & (2*KG*... ) as below, so 16 consecutive rows of a 16-byte fragment read do.
template <int JT, int KG>
struct GradTile {
  static constexpr int JR = 16 * JT, NW = 4 * KG, ST = 32 * KG;
  static constexpr int VROW = 2 * ST, VCH = VROW / 16;           // V^T row bytes, 16-byte chunks
  static constexpr int A_BYTES = ST * 128, V_BYTES = 4 * JR * VROW, STAGE = A_BYTES + V_BYTES;
  static constexpr int NS = (160 * 1024 - 4096) / STAGE < 8 ? (160 * 1024 - 4096) / STAGE : 8;
  static constexpr int LA = A_BYTES / 1024 / NW, LV = V_BYTES / 1024 / NW, L = LA + LV;
  static_assert(A_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0, "whole transfers per wave");
  static_assert(NS >= 2, "two stages fit");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int JT, int KG>
SRA_DEV void adapter_grads_body(const sra::AdapterGradArgs& ga) {
  using GT = GradTile<JT, KG>;
  constexpr int JR = GT::JR, NS = GT::NS, L = GT::L, ST = GT::ST, VCH = GT::VCH;
  constexpr int RED = (KG - 1) * 4 * JT * 4 * 64 * 8;  // k-group partials handed over at the end
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * GT::STAGE > RED ? NS * GT::STAGE : RED];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), cf = w & 3, kg = w >> 2;
  const bool second = (int)blockIdx.x >= ga.job[0].nmb;
  const sra::AdapterGrad job = second ? ga.job[1] : ga.job[0];
  const int mb = (int)blockIdx.x - (second ? ga.job[0].nmb : 0);
  const int64_t M = job.M, m0 = (int64_t)mb * 64;
  const int j0 = blockIdx.y * JR;
  const int64_t tb = (int64_t)blockIdx.z * ga.t_per, te = min(ga.T, tb + ga.t_per);
  const int n_st = (int)((te - tb + ST - 1) / ST);

  // Act rows [tb, te) seen from column m0; V^T parts whole
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(job.act + tb * M + m0), 0, (int)((te - tb) * M * 2 - m0 * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)job.vt, 0, (int)((int64_t)job.parts * ga.rp * ga.Tp * 2), 0x00020000);
  uint32_t a_off[GT::LA], v_off[GT::LV];
  int a_dst[GT::LA], v_dst[GT::LV];
#pragma unroll
  for (int k = 0; k < GT::LA; ++k) {  // 1 KB = 8 token rows of 128 bytes
    const int b = k * GT::NW + w, x = 8 * b + (lane >> 3), c = (lane & 7) ^ (((x >> 3) & 3) << 1);
    a_off[k] = (uint32_t)((x * M + c * 8) * 2);
    a_dst[k] = b * 1024;
  }
#pragma unroll
  for (int k = 0; k < GT::LV; ++k) {  // 1 KB = 64 / VCH rows of 2 ST bytes
    const int b = k * GT::NW + w, x = b * (64 / VCH) + lane / VCH;
    const int c = (lane % VCH) ^ ((x >> (VCH == 8 ? 1 : 0)) & (VCH - 1));
    const int p = min(x / JR, job.parts - 1), jj = x % JR;  // parts past the job's repeat its last
    v_off[k] = (uint32_t)((((int64_t)p * ga.rp + j0 + jj) * ga.Tp + tb + c * 8) * 2);
    v_dst[k] = GT::A_BYTES + b * 1024;
  }
  auto issue = [&](int st, int buf) {
    uint8_t* base = smem + buf * GT::STAGE;
#pragma unroll
    for (int k = 0; k < GT::LA; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + a_dst[k]), 16,
                                               a_off[k] + (uint32_t)(st * ST * M * 2), 0, 0, 0);
#pragma unroll
    for (int k = 0; k < GT::LV; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(base + v_dst[k]), 16,
                                               v_off[k] + (uint32_t)(st * ST * 2), 0, 0, 0);
  };

  // two accumulator sets, alternating by stage: the other (previous stage's) set moves to fp64
  // while this stage's MFMAs run
  f32x4 acc[2][JT];
  double acc64[JT][4];
#pragma unroll
  for (int a = 0; a < JT; ++a) {
    acc[0][a] = acc[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc64[a][e] = 0.0;
  }
  // the set's next stage starts its products from zero (the first MFMA's accumulator input), so
  // a flushed set needs no clearing
  auto to64 = [&](const f32x4 (&x)[JT]) {
#pragma unroll
    for (int a = 0; a < JT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc64[a][e] += (double)x[a][e];
  };
  const int m = 16 * cf + l16, mc = m >> 3, mo = m & 7;
  auto compute = [&](int buf, f32x4 (&cur)[JT], f32x4 (&prev)[JT]) {
    const uint8_t* A = smem + buf * GT::STAGE;
    const uint8_t* V = A + GT::A_BYTES;
    // B: Act[t][m] for this wave's 32 tokens t = 32kg + 8(l/16) .. +7 (one column per lane);
    // A: V^T rows, the same 8 tokens
    Frag bf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 32 * kg + 8 * q4 + e, c = mc ^ (((t >> 3) & 3) << 1);
      bf.h[e] = *reinterpret_cast<const uint16_t*>(A + t * 128 + c * 16 + mo * 2);
    }
    bf16x8v af[JT][4];
#pragma unroll
    for (int a = 0; a < JT; ++a)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int x = p * JR + 16 * a + l16;
        const int c = (4 * kg + q4) ^ ((x >> (VCH == 8 ? 1 : 0)) & (VCH - 1));
        af[a][p] = *reinterpret_cast<const bf16x8v*>(V + x * GT::VROW + c * 16);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < JT; ++a)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (p < job.parts)
          cur[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a][p], bf.b,
                                                           p == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : cur[a], 0, 0, 0);
    to64(prev);
  };

  constexpr int D = NS - 1;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < n_st) issue(d, d);
  auto step = [&](int st, f32x4 (&cur)[JT], f32x4 (&prev)[JT]) {
    wait_inflight<L, D>(min(D, n_st - st));
    ring_barrier();
    if (st + D < n_st) issue(st + D, (st + D) % NS);
    compute(st % NS, cur, prev);
  };
  // two stages per iteration, so each accumulator set keeps its registers; stage 0 flushes the
  // zero-initialised second set
  int st = 0;
  for (; st + 1 < n_st; st += 2) {
    step(st, acc[0], acc[1]);
    step(st + 1, acc[1], acc[0]);
  }
  if (st < n_st) {
    step(st, acc[0], acc[1]);
    to64(acc[0]);
  } else if (n_st > 0) {
    to64(acc[1]);
  }

  // k-groups 1 .. KG-1 hand their sums to k-group 0, which adds them in k-group order
  if constexpr (KG > 1) {
    __syncthreads();  // the ring is no longer read
    double* red = reinterpret_cast<double*>(smem);
    if (kg > 0) {
#pragma unroll
      for (int a = 0; a < JT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((((kg - 1) * 4 + cf) * JT + a) * 4 + e) * 64 + lane] = acc64[a][e];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g)
#pragma unroll
      for (int a = 0; a < JT; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc64[a][e] += red[((((g - 1) * 4 + cf) * JT + a) * 4 + e) * 64 + lane];
  }

  // D layout: rows j = 4(l/16) + e of adapter tile a, column m = l%16 of this fragment
  const int64_t mg = m0 + m;
  if (mg >= M) return;
#pragma unroll
  for (int a = 0; a < JT; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + 16 * a + 4 * q4 + e;
      if (j >= ga.r) continue;
      const int64_t o = job.out_t ? (int64_t)j * M + mg : mg * ga.r + j;
      if (ga.S > 1)
        job.part[(int64_t)blockIdx.z * M * ga.r + o] = acc64[a][e];
      else
        job.out[o] = (float)acc64[a][e];
    }
}

// one kernel per adapter-row tile width (the body is a device template: the buffer-resource
// builtins it uses have no host form)
constexpr int kGradKG[3] = {4, 4, 2};  // k-groups (waves / 4) for 16, 32, 64 adapter rows
__global__ __launch_bounds__(256 * kGradKG[0]) void k_adapter_grads16(sra::AdapterGradArgs ga) { adapter_grads_body<1, kGradKG[0]>(ga); }
__global__ __launch_bounds__(256 * kGradKG[1]) void k_adapter_grads32(sra::AdapterGradArgs ga) { adapter_grads_body<2, kGradKG[1]>(ga); }
__global__ __launch_bounds__(256 * kGradKG[2]) void k_adapter_grads64(sra::AdapterGradArgs ga) { adapter_grads_body<4, kGradKG[2]>(ga); }

// Wide tiles of the merged gradients, for ranks above 32.  With 64 x 64 tiles the V^T parts of a
// stage (3 parts x 64 rows) are three times the Act tile and are re-read by every column block, and
// Act itself is re-read once per 64 adapter rows.  Here each of the 8 waves owns 2 column
// fragments x 4 adapter-row fragments, and the waves tile either 128 columns x 128 adapter rows
// (WJ = 2) or 256 columns x 64 adapter rows (WJ = 1).  Stages are 32 tokens: the Act tile as
// 2*MW-byte token rows, the V^T tile as P*JR rows of 64 bytes, both by buffer -> LDS DMA with the
// same zero-reads past the slice and past T as the narrow kernel.  P is the part count of V^T (3:
// U for dB and dU for dA, both fp32 split exactly).
// Swizzles: Act row t keeps 16-byte chunk c in slot c ^ 2((t >> 3) & 3) (the four 8-token groups
// of a transposed 2-byte read land on different banks); V^T row x keeps chunk c in slot
// c ^ ((x >> 2) & 3) (16 consecutive 64-byte rows of a 16-byte fragment read cover all banks once).
template <int WJ, int P>
struct GradWide {
  static constexpr int WM = 8 / WJ, MW = 32 * WM, JR = 64 * WJ, ST = 32, NW = 8;
  static constexpr int CPR = MW / 8;                            // 16-byte chunks per Act row
  static constexpr int A_BYTES = ST * MW * 2, V_BYTES = P * JR * 64, STAGE = A_BYTES + V_BYTES;
  static constexpr int NS = (150 * 1024) / STAGE < 4 ? (150 * 1024) / STAGE : 4;
  static constexpr int LA = A_BYTES / 1024 / NW;                // Act transfers per wave
  static constexpr int NV = V_BYTES / 1024, LVM = (NV + NW - 1) / NW;
  static_assert(A_BYTES % (1024 * NW) == 0, "whole Act transfers per wave");
  static_assert(NS >= 3, "three stages fit");
};
constexpr int kGradWideLds = 128 * 1024;

template <int WJ, int P>
SRA_DEV void adapter_grads_wide_body(const sra::AdapterGradArgs& ga, const sra::AdapterGrad& job,
                                     int mb, uint8_t* smem) {
  using GW = GradWide<WJ, P>;
  static_assert(GW::NS * GW::STAGE <= kGradWideLds, "ring fits the shared buffer");
  constexpr int NS = GW::NS, NW = GW::NW, ST = GW::ST, JR = GW::JR, MW = GW::MW;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w % GW::WM, wj = w / GW::WM;
  const int64_t M = job.M, m0 = (int64_t)mb * MW;
  const int j0 = blockIdx.y * JR;
  const int64_t tb = (int64_t)blockIdx.z * ga.t_per, te = min(ga.T, tb + ga.t_per);
  const int n_st = (int)((te - tb + ST - 1) / ST);

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(job.act + tb * M + m0), 0, (int)((te - tb) * M * 2 - m0 * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)job.vt, 0, (int)((int64_t)P * ga.rp * ga.Tp * 2), 0x00020000);
  uint32_t a_off[GW::LA], v_off[GW::LVM];
  int a_dst[GW::LA], v_dst[GW::LVM];
#pragma unroll
  for (int k = 0; k < GW::LA; ++k) {  // 1 KB = 64 / CPR token rows of 2 MW bytes
    const int b = k * NW + w, x = b * (64 / GW::CPR) + lane / GW::CPR;
    const int c = (lane % GW::CPR) ^ (((x >> 3) & 3) << 1);
    a_off[k] = (uint32_t)((x * M + c * 8) * 2);
    a_dst[k] = b * 1024;
  }
  // waves w < NV - NW (LVM - 1) issue LVM V^T transfers per stage, the others LVM - 1
  const bool full_v = w < GW::NV - NW * (GW::LVM - 1);
#pragma unroll
  for (int k = 0; k < GW::LVM; ++k) {  // 1 KB = 16 rows of 64 bytes
    const int b = min(k * NW + w, GW::NV - 1), x = 16 * b + (lane >> 2);
    const int c = (lane & 3) ^ ((x >> 2) & 3);
    const int p = x / JR, jj = x % JR;
    v_off[k] = (uint32_t)((((int64_t)p * ga.rp + j0 + jj) * ga.Tp + tb + c * 8) * 2);
    v_dst[k] = GW::A_BYTES + b * 1024;
  }
  auto issue = [&](int st, int buf) {
    uint8_t* base = smem + buf * GW::STAGE;
#pragma unroll
    for (int k = 0; k < GW::LA; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + a_dst[k]), 16,
                                               a_off[k] + (uint32_t)(st * ST * M * 2), 0, 0, 0);
#pragma unroll
    for (int k = 0; k < GW::LVM; ++k)
      if (k < GW::LVM - 1 || full_v)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(base + v_dst[k]), 16,
                                                 v_off[k] + (uint32_t)(st * ST * 2), 0, 0, 0);
  };

  f32x4 acc[2][2][4];
  double acc64[2][4][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      acc[0][f][a] = acc[1][f][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc64[f][a][e] = 0.0;
    }
  // the set's next stage starts its products from zero (the first MFMA's accumulator input), so
  // a flushed set needs no clearing
  auto to64 = [&](const f32x4 (&x)[2][4]) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc64[f][a][e] += (double)x[f][a][e];
  };
  auto compute = [&](int buf, f32x4 (&cur)[2][4], f32x4 (&prev)[2][4]) {
    const uint8_t* A = smem + buf * GW::STAGE;
    const uint8_t* V = A + GW::A_BYTES;
    // B operand: Act[t][m] for tokens t = 8(l/16) .. +7 of the stage, one column m per lane
    Frag bf[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int m = 32 * wm + 16 * f + l16, mc = m >> 3, mo = m & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 8 * q4 + e, c = mc ^ (((t >> 3) & 3) << 1);
        bf[f].h[e] = *reinterpret_cast<const uint16_t*>(A + t * (2 * MW) + c * 16 + mo * 2);
      }
    }
    // A operand: V^T rows (part p, adapter row 64 wj + 16 a + l%16), the same 8 tokens
    bf16x8v vf[4][P];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int x = p * JR + 64 * wj + 16 * a + l16;
        vf[a][p] = *reinterpret_cast<const bf16x8v*>(V + x * 64 + ((q4 ^ ((x >> 2) & 3)) << 4));
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int p = 0; p < P; ++p)
          cur[f][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[a][p], bf[f].b,
                                                              p == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : cur[f][a], 0, 0, 0);
    to64(prev);
  };

  constexpr int D = NS - 1;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < n_st) issue(d, d);
  auto step = [&](int st, f32x4 (&cur)[2][4], f32x4 (&prev)[2][4]) {
    if (full_v) wait_inflight<GW::LA + GW::LVM, D>(min(D, n_st - st));
    else wait_inflight<GW::LA + GW::LVM - 1, D>(min(D, n_st - st));
    ring_barrier();
    if (st + D < n_st) issue(st + D, (st + D) % NS);
    compute(st % NS, cur, prev);
  };
  // two stages per iteration, so each accumulator set keeps its registers (alternating the roles
  // inside one loop body made the compiler copy both sets every stage)
  // (stage 0 flushes the zero-initialised second set)
  int st = 0;
  for (; st + 1 < n_st; st += 2) {
    step(st, acc[0], acc[1]);
    step(st + 1, acc[1], acc[0]);
  }
  if (st < n_st) {
    step(st, acc[0], acc[1]);
    to64(acc[0]);
  } else if (n_st > 0) {
    to64(acc[1]);
  }

  // D layout: adapter rows 4(l/16) + e of fragment (wj, a), column l%16 of fragment (wm, f)
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t mg = m0 + 32 * wm + 16 * f + l16;
    if (mg >= M) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 64 * wj + 16 * a + 4 * q4 + e;
        if (j >= ga.r) continue;
        const int64_t o = job.out_t ? (int64_t)j * M + mg : mg * ga.r + j;
        if (ga.S > 1)
          job.part[(int64_t)blockIdx.z * M * ga.r + o] = acc64[f][a][e];
        else
          job.out[o] = (float)acc64[f][a][e];
      }
  }
}

template <int WJ>
SRA_DEV void adapter_grads_wide(const sra::AdapterGradArgs& ga) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kGradWideLds];
  const bool second = (int)blockIdx.x >= ga.job[0].nmb;
  const sra::AdapterGrad job = second ? ga.job[1] : ga.job[0];
  const int mb = (int)blockIdx.x - (second ? ga.job[0].nmb : 0);
  adapter_grads_wide_body<WJ, 3>(ga, job, mb, smem);
}
__global__ __launch_bounds__(512) void k_adapter_grads_w64(sra::AdapterGradArgs ga) { adapter_grads_wide<1>(ga); }
__global__ __launch_bounds__(512) void k_adapter_grads_w128(sra::AdapterGradArgs ga) { adapter_grads_wide<2>(ga); }

// out = sum over the S slices of each job's partials, in slice order (one thread per element of
// the first job's output, then of the second's)
__global__ void k_reduce_grads(sra::AdapterGradArgs ga) {
  const int64_t n0 = ga.job[0].M * ga.r;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = i >= n0;
  const sra::AdapterGrad job = second ? ga.job[1] : ga.job[0];
  if (second) i -= n0;
  const int64_t n = job.M * ga.r;
  if (i >= n) return;
  double s = 0.0;
  for (int z = 0; z < ga.S; ++z) s += job.part[(int64_t)z * n + i];
  job.out[i] = (float)s;
}

// ------------------------------------------------------------------------------ rows, ring
// The rows product for ranks above 32 at training token counts.  The small-tile rows kernel reads
// the whole weight operand once per 16 tokens, which at r = 128 and C = 20480 (dU = dY B) is
// gigabytes of L2 / Infinity Cache traffic; here a workgroup owns 128 tokens x JR = 16 JT adapter
// columns over a slice of c, and both operands stream through an NS-deep LDS ring of 64-column
// stages filled by buffer -> LDS DMA (one 128-byte run per row; token rows past T and adapter rows
// past r read as zeros through the buffer range checks).  Wave w owns tokens 16w .. 16w+15 and all
// JR columns: per stage 2 x JT mfma_f32_16x16x32_bf16 into one of two fp32 accumulator sets, the
// other (previous stage's) set moving into fp64 meanwhile, so fp32 rounding only acts inside one
// stage's 64-term dot products.
// LDS rows are 128 bytes; 16-byte chunk k of row x sits in slot k ^ ((x >> 1) & 7), so the 16 rows
// of one fragment read spread over the banks.
// Requires C % 64 == 0, c_per % 64 == 0, ldw % 8 == 0 and 16-byte aligned act / wt.
template <int JT>
struct RowsRing {
  static constexpr int TT = 128, JR = 16 * JT, NW = 8;
  static constexpr int A_BYTES = TT * 128, G_BYTES = JR * 128, STAGE = A_BYTES + G_BYTES;
  static constexpr int NS = 4;
  static constexpr int LA = A_BYTES / 1024 / NW, LG = G_BYTES / 1024 / NW, L = LA + LG;
  static_assert(A_BYTES % (1024 * NW) == 0 && G_BYTES % (1024 * NW) == 0, "whole transfers per wave");
  static_assert(NS * STAGE <= 160 * 1024, "ring fits in LDS");
};

SRA_DEV int rows_swz(int x) { return (x >> 1) & 7; }

template <int JT>
SRA_DEV void adapter_rows_ring_body(const uint16_t* __restrict__ act, int64_t T, int64_t C,
                                    const uint16_t* __restrict__ wt, int64_t ldw, int r,
                                    int64_t c_per, double* __restrict__ part,
                                    float* __restrict__ out, double* __restrict__ out64,
                                    uint16_t* __restrict__ vt, int rp, int64_t Tp) {
  using RR = RowsRing<JT>;
  constexpr int NS = RR::NS, L = RR::L, NW = RR::NW;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * RR::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * RR::TT;
  const int j0 = blockIdx.y * RR::JR;
  const int64_t cb = (int64_t)blockIdx.z * c_per, ce = min(C, cb + c_per);
  const int n_st = (int)((ce - cb) / 64);

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(act + t0 * C + cb), 0, (int)(((T - t0) * C - cb) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wt + (int64_t)j0 * ldw + cb), 0, (int)(((int64_t)(r - j0) * ldw - cb) * 2), 0x00020000);
  uint32_t a_off[RR::LA], g_off[RR::LG];
  int a_dst[RR::LA], g_dst[RR::LG];
#pragma unroll
  for (int k = 0; k < RR::LA; ++k) {  // 1 KB = 8 rows of 128 bytes
    const int b = k * NW + w, x = 8 * b + (lane >> 3), c = (lane & 7) ^ rows_swz(x);
    a_off[k] = (uint32_t)((x * C + c * 8) * 2);
    a_dst[k] = b * 1024;
  }
#pragma unroll
  for (int k = 0; k < RR::LG; ++k) {
    const int b = k * NW + w, x = 8 * b + (lane >> 3), c = (lane & 7) ^ rows_swz(x);
    g_off[k] = (uint32_t)((x * ldw + c * 8) * 2);
    g_dst[k] = RR::A_BYTES + b * 1024;
  }
  auto issue = [&](int st, int buf) {
    uint8_t* base = smem + buf * RR::STAGE;
#pragma unroll
    for (int k = 0; k < RR::LA; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + a_dst[k]), 16,
                                               a_off[k] + (uint32_t)(st * 128), 0, 0, 0);
#pragma unroll
    for (int k = 0; k < RR::LG; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_ptr_t)(base + g_dst[k]), 16,
                                               g_off[k] + (uint32_t)(st * 128), 0, 0, 0);
  };

  f32x4 acc[2][JT];
  double acc64[JT][4];
#pragma unroll
  for (int a = 0; a < JT; ++a) {
    acc[0][a] = acc[1][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc64[a][e] = 0.0;
  }
  // the set's next stage starts its products from zero (the first MFMA's accumulator input), so
  // a flushed set needs no clearing
  auto to64 = [&](const f32x4 (&x)[JT]) {
#pragma unroll
    for (int a = 0; a < JT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc64[a][e] += (double)x[a][e];
  };
  const int xa = 16 * w + l16;  // this lane's token row of the stage
  auto compute = [&](int buf, f32x4 (&cur)[JT], f32x4 (&prev)[JT]) {
    const uint8_t* Ab = smem + buf * RR::STAGE;
    const uint8_t* Gb = Ab + RR::A_BYTES;
    bf16x8v af[2], gf[2][JT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int k = 4 * ks + q4;
      af[ks] = *reinterpret_cast<const bf16x8v*>(Ab + xa * 128 + ((k ^ rows_swz(xa)) << 4));
#pragma unroll
      for (int a = 0; a < JT; ++a) {
        const int x = 16 * a + l16;
        gf[ks][a] = *reinterpret_cast<const bf16x8v*>(Gb + x * 128 + ((k ^ rows_swz(x)) << 4));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < JT; ++a)
        cur[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], gf[ks][a],
                                                         ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : cur[a], 0, 0, 0);
    to64(prev);
  };

  constexpr int D = NS - 1;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < n_st) issue(d, d);
  auto step = [&](int st, f32x4 (&cur)[JT], f32x4 (&prev)[JT]) {
    wait_inflight<L, D>(min(D, n_st - st));
    ring_barrier();
    if (st + D < n_st) issue(st + D, (st + D) % NS);
    compute(st % NS, cur, prev);
  };
  // two stages per iteration, so each accumulator set keeps its registers; stage 0 flushes the
  // zero-initialised second set
  int st = 0;
  for (; st + 1 < n_st; st += 2) {
    step(st, acc[0], acc[1]);
    step(st + 1, acc[1], acc[0]);
  }
  if (st < n_st) {
    step(st, acc[0], acc[1]);
    to64(acc[0]);
  } else if (n_st > 0) {
    to64(acc[1]);
  }

  // D layout: tokens 16w + 4(l/16) + e, column j = 16a + l%16
#pragma unroll
  for (int a = 0; a < JT; ++a) {
    const int j = j0 + 16 * a + l16;
    if (j >= r) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t tt = t0 + 16 * w + 4 * q4 + e;
      if (tt >= T) {
        // V^T columns T .. Tp-1 (padding to a multiple of 8) must read as zero in the cols kernel
        if (vt && blockIdx.z == 0 && tt < Tp)
#pragma unroll
          for (int p = 0; p < 3; ++p) vt[((int64_t)p * rp + j) * Tp + tt] = 0;
        continue;
      }
      const double s = acc64[a][e];
      if (part) {
        part[(int64_t)blockIdx.z * T * r + tt * r + j] = s;
      } else {
        if (out) out[tt * r + j] = (float)s;
        if (out64) out64[tt * r + j] = s;
        if (vt) write_vt3(vt, rp, Tp, j, tt, s);
      }
    }
  }
}

__global__ __launch_bounds__(512) void k_adapter_rows_ring64(
    const uint16_t* __restrict__ act, int64_t T, int64_t C, const uint16_t* __restrict__ wt,
    int64_t ldw, int r, int64_t c_per, double* __restrict__ part, float* __restrict__ out,
    double* __restrict__ out64, uint16_t* __restrict__ vt, int rp, int64_t Tp) {
  adapter_rows_ring_body<4>(act, T, C, wt, ldw, r, c_per, part, out, out64, vt, rp, Tp);
}
__global__ __launch_bounds__(512) void k_adapter_rows_ring128(
    const uint16_t* __restrict__ act, int64_t T, int64_t C, const uint16_t* __restrict__ wt,
    int64_t ldw, int r, int64_t c_per, double* __restrict__ part, float* __restrict__ out,
    double* __restrict__ out64, uint16_t* __restrict__ vt, int rp, int64_t Tp) {
  adapter_rows_ring_body<8>(act, T, C, wt, ldw, r, c_per, part, out, out64, vt, rp, Tp);
}

}  // namespace

namespace sra {

int64_t vt_rows(int r) { return round_up(r, 16); }
int64_t vt_cols(int64_t T) { return round_up(T, 8); }
size_t adapter_vt_bytes(int64_t T, int r, int parts) {
  return align256((size_t)parts * vt_rows(r) * vt_cols(T) * 2);
}
int64_t packed_wt_ld(int64_t C) { return round_up(C, 8); }
int64_t packed_at_ld(int r) { return round_up(r, 8); }
size_t adapter_at_bytes(int64_t K, int r) { return align256((size_t)K * packed_at_ld(r) * 2); }
size_t adapter_wt_bytes(int64_t C, int r) { return align256((size_t)r * packed_wt_ld(C) * 2); }

hipError_t launch_adapter_bwd_prep(const uint16_t* B, int64_t N, int r, uint16_t* wt,
                                   const uint16_t* A, int64_t K, uint16_t* at, const float* U,
                                   int64_t T, uint16_t* vtU, hipStream_t s) {
  if (r == 0 || (!wt && !at && !vtU)) return hipSuccess;
  PrepArgs pa{};
  pa.B = B;
  pa.C = N;
  pa.ldw = packed_wt_ld(N);
  pa.wt = wt;
  pa.b_cx = (int)cdiv(N, 64);
  pa.nb = wt ? pa.b_cx * (int)cdiv(r, 64) : 0;
  pa.A = A;
  pa.K = K;
  pa.lda = packed_at_ld(r);
  pa.at = at;
  pa.a_cx = (int)cdiv(K, 64);
  pa.na = at ? pa.a_cx * (int)cdiv(r, 64) : 0;
  pa.U = U;
  pa.T = T;
  pa.r = r;
  pa.rp = (int)vt_rows(r);
  pa.Tp = vt_cols(T);
  pa.vt = vtU;
  const int n_split = vtU ? (int)cdiv((int64_t)pa.rp * pa.Tp, 256) : 0;
  const int blocks = pa.nb + pa.na + n_split;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_prep, dim3((unsigned)blocks), dim3(256), 0, s, pa);
  return hipGetLastError();
}

namespace {
// The ring kernel: ranks above 32 with at least two 128-token tiles, whole 64-column stages and
// 32-bit buffer offsets; the grid gets as many reduction slices (of whole stages, at least 4 per
// slice) as keep it near 256 workgroups, one per CU.
struct RingPlan {
  bool ok;
  int jr, S;
  int64_t c_per;
  size_t part_bytes;
};
RingPlan ring_plan(int64_t T, int64_t C, int r) {
  RingPlan p{};
  if (r <= 32 || T < 256 || C % 64 != 0 || T * C * 2 >= ((int64_t)1 << 31)) return p;
  p.ok = true;
  p.jr = r <= 64 ? 64 : 128;
  const int64_t blocks = cdiv(T, 128) * cdiv(r, p.jr);
  int64_t S = cdiv(256, blocks);
  if (tuning().rows_slices > 0) S = tuning().rows_slices;
  const int64_t max_s = C / 256 > 0 ? C / 256 : 1;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  p.c_per = round_up(cdiv(C, S), 64);
  p.S = (int)cdiv(C, p.c_per);
  p.part_bytes = p.S > 1 ? (size_t)p.S * T * r * sizeof(double) : 0;
  return p;
}
bool ring_usable(const RingPlan& p, const uint16_t* act, const uint16_t* wt, int64_t ldw, int r) {
  return p.ok && ldw % 8 == 0 && (int64_t)r * ldw * 2 < ((int64_t)1 << 31) &&
         ((uintptr_t)act & 15) == 0 && ((uintptr_t)wt & 15) == 0;
}
}  // namespace

size_t adapter_rows_ws(int64_t T, int64_t C, int r) {
  if (T <= 0 || C <= 0 || r <= 0) return 0;
  // the ring kernel may fall back to the register kernel at launch (operand alignment): room for both
  const size_t a = rows_plan(T, C, r).part_bytes, b = ring_plan(T, C, r).part_bytes;
  return a > b ? a : b;
}

hipError_t launch_adapter_rows(const uint16_t* act, int64_t T, int64_t C, const uint16_t* wt,
                               int64_t ldw, int r, float* out, double* out64, uint16_t* vt,
                               void* ws, hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  if (C == 0) {
    if (out64 || vt) return hipErrorInvalidValue;  // callers never ask for fp64 with an empty reduction
    return launch_fill_f32(out, T * r, 0.f, s);
  }
  if (T <= 16 && !out64 && !vt && C % 8 == 0 && ldw % 8 == 0 && (((uintptr_t)act | (uintptr_t)wt) & 15) == 0) {
    launch(SRA_KERNEL_ADAPTER, k_adapter_rows_few, dim3((unsigned)cdiv(r, kFewJ), (unsigned)T),
           dim3(256), 0, s, act, C, wt, ldw, r, out);
    return hipGetLastError();
  }
  const int rp = (int)vt_rows(r);
  const int64_t Tp = vt_cols(T);
  const RingPlan q = ring_plan(T, C, r);
  if (ring_usable(q, act, wt, ldw, r)) {
    double* part = q.S > 1 ? (double*)ws : nullptr;
    const dim3 grid((unsigned)cdiv(T, 128), (unsigned)cdiv(r, q.jr), (unsigned)q.S);
    if (q.jr == 64)
      launch(SRA_KERNEL_ADAPTER, k_adapter_rows_ring64, grid, dim3(512), 0, s, act, T, C, wt, ldw,
             r, q.c_per, part, out, out64, vt, rp, Tp);
    else
      launch(SRA_KERNEL_ADAPTER, k_adapter_rows_ring128, grid, dim3(512), 0, s, act, T, C, wt, ldw,
             r, q.c_per, part, out, out64, vt, rp, Tp);
    if (q.S > 1) reduce_parts(part, q.S, T, r, out, out64, vt, rp, Tp, s);
    return hipGetLastError();
  }
  const RowsPlan p = rows_plan(T, C, r);
  double* part = p.S > 1 ? (double*)ws : nullptr;
  const dim3 grid((unsigned)cdiv(T, 16), (unsigned)cdiv(r, 16 * p.jt), (unsigned)p.S);
  switch (p.jt) {
    case 1: rows_launch<1, 4>(grid, s, act, T, C, wt, ldw, r, p.c_per, part, out, out64, vt, rp, Tp); break;
    case 2: rows_launch<2, 4>(grid, s, act, T, C, wt, ldw, r, p.c_per, part, out, out64, vt, rp, Tp); break;
    default: rows_launch<4, 2>(grid, s, act, T, C, wt, ldw, r, p.c_per, part, out, out64, vt, rp, Tp); break;
  }
  if (p.S > 1) reduce_parts(part, p.S, T, r, out, out64, vt, rp, Tp, s);
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


// ---- merged adapter gradients
namespace {
struct GradsPlan {
  int jt, njb, S;
  int wj;   // wide tiles: 1 (256 columns x 64 adapter rows) or 2 (128 x 128); 0 for 64 x 64
  int mw;   // columns per workgroup
  int64_t t_per;
};
GradsPlan grads_plan(const AdapterGrad* g, int n, int64_t T, int r) {
  GradsPlan p;
  p.jt = pick_jt(r);
  bool wide = r > 32;
  // (three parts; the per-lane offsets of a 32-token stage stay below 2^31)
  for (int i = 0; i < n; ++i)
    wide = wide && g[i].parts == 3 && g[i].M * 64 < ((int64_t)1 << 31);
  p.wj = wide ? (r <= 64 ? 1 : 2) : 0;
  p.mw = wide ? 256 / p.wj : 64;
  p.njb = (int)cdiv(r, wide ? 64 * p.wj : 16 * p.jt);
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) blocks += cdiv(g[i].M, p.mw) * p.njb;
  // one workgroup per CU (the ring takes most of the LDS).  Narrow tiles: as many slices as keep
  // the grid within 256 workgroups.  Wide tiles: the slice count (<= 8) that minimises whole
  // waves of 256 workgroups per slice plus about 4% per extra slice for the partials' traffic.
  // Each slice is at least 256 tokens.
  int64_t S = 256 / (blocks < 1 ? 1 : blocks);
  if (wide) {
    double best = 1e30;
    for (int64_t c = 1; c <= 8; ++c) {
      const double cost = (double)cdiv(blocks * c, 256) / (double)c + 0.04 * (double)(c - 1);
      if (cost < best - 1e-9) best = cost, S = c;
    }
  }
  if (tuning().grads_slices > 0) S = tuning().grads_slices;
  const int64_t max_s = cdiv(T, 256);
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  p.t_per = round_up(cdiv(T, S), 64);
  p.S = (int)cdiv(T, p.t_per);
  return p;
}
}  // namespace

bool adapter_grads_ok(const AdapterGrad* g, int n, int64_t T, int r) {
  if (n < 1 || n > 2 || T <= 0 || r <= 0) return false;
  const int64_t Tp = vt_cols(T), rp = vt_rows(r);
  for (int i = 0; i < n; ++i) {
    if (g[i].M <= 0 || g[i].M % 8 != 0 || g[i].parts < 1 || g[i].parts > 4) return false;
    // 32-bit buffer offsets
    if (T * g[i].M * 2 >= (int64_t)1 << 31 || (int64_t)g[i].parts * (rp + 64) * (Tp + 64) * 2 >= (int64_t)1 << 31)
      return false;
  }
  return true;
}

size_t adapter_grads_ws(const AdapterGrad* g, int n, int64_t T, int r) {
  if (!adapter_grads_ok(g, n, T, r)) return 0;
  const GradsPlan p = grads_plan(g, n, T, r);
  if (p.S <= 1) return 0;
  size_t b = 0;
  for (int i = 0; i < n; ++i) b += align256((size_t)p.S * g[i].M * r * sizeof(double));
  return b;
}

hipError_t launch_adapter_grads(const AdapterGrad* g, int n, int64_t T, int r, void* ws,
                                hipStream_t s) {
  if (!adapter_grads_ok(g, n, T, r)) return hipErrorInvalidValue;
  const GradsPlan p = grads_plan(g, n, T, r);
  AdapterGradArgs ga{};
  uint8_t* w = (uint8_t*)ws;
  int nmb = 0;
  for (int i = 0; i < n; ++i) {
    ga.job[i] = g[i];
    ga.job[i].nmb = (int)cdiv(g[i].M, p.mw);
    nmb += ga.job[i].nmb;
    if (p.S > 1) {
      ga.job[i].part = (double*)w;
      w += align256((size_t)p.S * g[i].M * r * sizeof(double));
    }
  }
  if (n == 1) ga.job[1] = ga.job[0], ga.job[1].M = 0;  // no second job: never reached
  ga.T = T;
  ga.Tp = vt_cols(T);
  ga.t_per = p.t_per;
  ga.r = r;
  ga.rp = (int)vt_rows(r);
  ga.S = p.S;
  const dim3 grid((unsigned)nmb, (unsigned)p.njb, (unsigned)p.S);
  switch (p.wj ? 4 + p.wj : p.jt) {
    case 5: launch(SRA_KERNEL_ADAPTER, k_adapter_grads_w64, grid, dim3(512), 0, s, ga); break;
    case 6: launch(SRA_KERNEL_ADAPTER, k_adapter_grads_w128, grid, dim3(512), 0, s, ga); break;
    case 1: launch(SRA_KERNEL_ADAPTER, k_adapter_grads16, grid, dim3(256 * kGradKG[0]), 0, s, ga); break;
    case 2: launch(SRA_KERNEL_ADAPTER, k_adapter_grads32, grid, dim3(256 * kGradKG[1]), 0, s, ga); break;
    default: launch(SRA_KERNEL_ADAPTER, k_adapter_grads64, grid, dim3(256 * kGradKG[2]), 0, s, ga); break;
  }
  if (p.S > 1) {
    int64_t tot = 0;
    for (int i = 0; i < n; ++i) tot += g[i].M * r;
    hipLaunchKernelGGL(k_reduce_grads, dim3((unsigned)cdiv(tot, 256)), dim3(256), 0, s, ga);
  }
  return hipGetLastError();
}

}  // namespace sra

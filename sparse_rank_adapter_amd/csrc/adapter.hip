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
//   cancel by orders of magnitude, so V's rounding is amplified ~sqrt(T) times: a pre-pass stores
//   V^T as bf16 parts [part][j][t] -- three parts for fp32 V (U; split error below fp32 rounding),
//   four for the fp64 dU that the rows kernel hands over for dA -- which then read as contiguous
//   16-byte fragments.
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
template <int JT, int UB>
__global__ __launch_bounds__(256) void k_adapter_rows(const uint16_t* __restrict__ act, int64_t T,
                                                      int64_t C, const uint16_t* __restrict__ wt,
                                                      int64_t ldw, int r, int64_t c_per,
                                                      double* __restrict__ part,
                                                      float* __restrict__ out,
                                                      double* __restrict__ out64) {
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
      }
    }
  }
}

// wt[j][c] = src[j*sj + c*sc] for j < r, c < C, rows of stride ldw >= C (a 64 x 64 tile per
// workgroup, transposed through LDS so that B [C x r] (sj = 1) is read and written coalesced).
__global__ void k_pack_w(const uint16_t* __restrict__ src, int64_t C, int r, int64_t sj, int64_t sc,
                         int64_t ldw, uint16_t* __restrict__ wt) {
  __shared__ uint16_t tile[64][65];
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int j0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 256 threads: 4 rows at a time
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i;
    const int j = j0 + tx;
    tile[i][tx] = (c < C && j < r) ? src[(int64_t)j * sj + c * sc] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int j = j0 + i;
    const int64_t c = c0 + tx;
    if (j < r && c < C) wt[(int64_t)j * ldw + c] = tile[tx][i];
  }
}

// ------------------------------------------------------------------------------------ cols
constexpr int CS = 64;        // tokens per staged tile
constexpr int ALD = 64 + 8;   // LDS row of the Act tile [t][m] (elements; 144 B keeps 16 B alignment)
constexpr int VLD = CS + 8;   // LDS row of the V^T tile [j][t]

// V^T parts: vt[p][j][t] for j < rp (r rounded up to 16; rows past r are 0) and t < Tp (T rounded
// up to 8; columns past T are 0).  fp32 V -> 3 parts, fp64 V -> 4 parts.
__global__ void k_split_vt(const float* __restrict__ V32, const double* __restrict__ V64, int64_t T,
                           int r, int rp, int64_t Tp, uint16_t* __restrict__ vt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // i = j * Tp + t (t fastest)
  if (i >= (int64_t)rp * Tp) return;
  const int j = (int)(i / Tp);
  const int64_t t = i - (int64_t)j * Tp;
  uint16_t p[4] = {0, 0, 0, 0};
  if (j < r && t < T) {
    if (V64) split4_bf16(V64[t * r + j], p);
    else split3_bf16(V32[t * r + j], p[0], p[1], p[2]);
  }
  const int parts = V64 ? 4 : 3;
  for (int q = 0; q < parts; ++q) vt[((int64_t)q * rp + j) * Tp + t] = p[q];
}

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
                               float* __restrict__ out, double* __restrict__ out64) {
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
  int jt, ub;
  int64_t c_per, ldw;
  int S;
  bool pack;  // weight needs transposing into the workspace
  size_t w_bytes, part_bytes;
};

RowsPlan rows_plan(int64_t T, int64_t C, int r, int64_t wt_sj, int64_t wt_sc, const void* wt) {
  RowsPlan p;
  p.jt = pick_jt(r);
  p.ub = p.jt >= 4 ? 2 : 4;
  // used in place when its rows are c-contiguous, 16-byte aligned and (for r > 1) 8-aligned apart
  p.pack = !(wt_sc == 1 && (r == 1 || (wt_sj & 7) == 0) && (((uintptr_t)wt) & 15) == 0);
  p.ldw = p.pack || r == 1 ? round_up(C, 8) : wt_sj;
  p.w_bytes = p.pack ? align256((size_t)r * p.ldw * 2) : 0;
  const int64_t blocks = cdiv(T, 16) * cdiv(r, 16 * p.jt);
  p.c_per = slice_len(blocks, C, 128 * p.ub, 128 * p.ub, 512);
  p.S = (int)cdiv(C, p.c_per);
  p.part_bytes = p.S > 1 ? (size_t)p.S * T * r * sizeof(double) : 0;
  return p;
}

struct ColsPlan {
  int jt, S, rp;
  int64_t t_per, Tp;
  size_t vt_bytes, part_bytes;
};

ColsPlan cols_plan(int64_t T, int64_t M, int r) {
  ColsPlan p;
  p.jt = pick_jt(r);
  const int64_t blocks = cdiv(M, 64) * cdiv(r, 16 * p.jt);
  p.t_per = slice_len(blocks, T, 128, CS, 512);
  p.S = (int)cdiv(T, p.t_per);
  p.Tp = round_up(T, 8);
  p.rp = (int)round_up(r, 16);
  p.vt_bytes = align256((size_t)4 * p.rp * p.Tp * 2);
  p.part_bytes = p.S > 1 ? (size_t)p.S * M * r * sizeof(double) : 0;
  return p;
}

template <int JT, int UB>
void rows_launch(dim3 grid, hipStream_t s, const uint16_t* act, int64_t T, int64_t C,
                 const uint16_t* wt, int64_t ldw, int r, int64_t c_per, double* part, float* out,
                 double* out64) {
  sra::launch(SRA_KERNEL_ADAPTER, k_adapter_rows<JT, UB>, grid, dim3(256), 0, s, act, T, C, wt,
              ldw, r, c_per, part, out, out64);
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

// The workspace size depends on the weight's strides only through whether it must be packed;
// the query assumes it must (the larger case).
size_t adapter_rows_ws(int64_t T, int64_t C, int r) {
  if (T <= 0 || C <= 0 || r <= 0) return 0;
  const RowsPlan p = rows_plan(T, C, r, 1, r, nullptr);  // partial sizes do not depend on wt
  return align256((size_t)r * round_up(C, 8) * 2) + p.part_bytes;
}

hipError_t launch_adapter_rows(const uint16_t* act, int64_t T, int64_t C, const uint16_t* wt,
                               int64_t wt_sj, int64_t wt_sc, int r, float* out, double* out64,
                               void* ws, hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  if (C == 0) {
    if (out64) return hipErrorInvalidValue;  // callers never ask for fp64 with an empty reduction
    return launch_fill_f32(out, T * r, 0.f, s);
  }
  const RowsPlan p = rows_plan(T, C, r, wt_sj, wt_sc, wt);
  uint8_t* wsb = (uint8_t*)ws;
  const uint16_t* w = wt;
  if (p.pack) {
    uint16_t* wp = (uint16_t*)wsb;
    const dim3 tg((unsigned)cdiv(C, 64), (unsigned)cdiv(r, 64));
    hipLaunchKernelGGL(k_pack_w, tg, dim3(256), 0, s, wt, C, r, wt_sj, wt_sc, p.ldw, wp);
    w = wp;
  }
  double* part = p.S > 1 ? (double*)(wsb + align256((size_t)r * round_up(C, 8) * 2)) : nullptr;
  const dim3 grid((unsigned)cdiv(T, 16), (unsigned)cdiv(r, 16 * p.jt), (unsigned)p.S);
  switch (p.jt) {
    case 1: rows_launch<1, 4>(grid, s, act, T, C, w, p.ldw, r, p.c_per, part, out, out64); break;
    case 2: rows_launch<2, 4>(grid, s, act, T, C, w, p.ldw, r, p.c_per, part, out, out64); break;
    default: rows_launch<4, 2>(grid, s, act, T, C, w, p.ldw, r, p.c_per, part, out, out64); break;
  }
  if (p.S > 1) {
    const int64_t n = T * r;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, part, p.S,
                       n, out, out64);
  }
  return hipGetLastError();
}

size_t adapter_cols_ws(int64_t T, int64_t M, int r) {
  if (T <= 0 || M <= 0 || r <= 0) return 0;
  const ColsPlan p = cols_plan(T, M, r);
  return p.vt_bytes + p.part_bytes;
}

hipError_t launch_adapter_cols(const uint16_t* act, int64_t T, int64_t M, const float* V32,
                               const double* V64, int r, bool out_transposed, float* out, void* ws,
                               hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  if (T == 0) return launch_fill_f32(out, M * r, 0.f, s);
  const ColsPlan p = cols_plan(T, M, r);
  uint16_t* vt = (uint16_t*)ws;
  double* part = p.S > 1 ? (double*)((uint8_t*)ws + p.vt_bytes) : nullptr;
  const int parts = V64 ? 4 : 3;
  const int64_t nvt = (int64_t)p.rp * p.Tp;
  hipLaunchKernelGGL(k_split_vt, dim3((unsigned)cdiv(nvt, 256)), dim3(256), 0, s, V32, V64, T, r,
                     p.rp, p.Tp, vt);
  const dim3 grid((unsigned)cdiv(M, 64), (unsigned)cdiv(r, 16 * p.jt), (unsigned)p.S);
  switch (p.jt) {
    case 1: cols_launch<1>(grid, s, act, T, M, vt, parts, r, p.rp, p.Tp, p.t_per, out_transposed, part, out); break;
    case 2: cols_launch<2>(grid, s, act, T, M, vt, parts, r, p.rp, p.Tp, p.t_per, out_transposed, part, out); break;
    default: cols_launch<4>(grid, s, act, T, M, vt, parts, r, p.rp, p.Tp, p.t_per, out_transposed, part, out); break;
  }
  if (p.S > 1) {
    const int64_t n = M * r;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, part, p.S,
                       n, out, nullptr);
  }
  return hipGetLastError();
}

}  // namespace sra

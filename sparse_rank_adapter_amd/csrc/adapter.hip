// Adapter products of the low-rank branch (SLoPe paperlayer summary §2.2; LoRA):
//   rows kernel:  U  = X A^T   [T x r]   and   dU = dY B   [T x r]
//   cols kernel:  dB = dY^T U  [N x r]   and   dA = dU^T X [r x K]
// With r <= 256 these are skinny, bandwidth-bound products: the point is to stream X or dY once
// with wide, coalesced loads and keep the small operand in LDS.
//
// rows: Out[t][j] = sum_c Act[t][c] Wt(j, c).  A workgroup owns 64 tokens (16 per wave) and up to
//   64 adapter columns, over one slice of the reduction dim c (slices are split over workgroups to
//   fill the GPU).  Per 256-column block the weight slice Wt(j, c) is staged in LDS as [j][c]
//   (from a c-contiguous source such as A, or a j-contiguous one such as B, both with 16-byte
//   loads); each wave then takes 16-byte activation fragments straight from global memory.
// cols: Out[m][j] = sum_t Act[t][m] V[t][j] with V fp32.  A workgroup owns 64 columns m (16 per
//   wave) and up to 64 adapter columns j over a slice of tokens.  Per 32-token chunk both tiles are
//   read with coalesced 16-byte loads and written to LDS transposed ([m][t] and [j][t]), so every
//   MFMA fragment is one 128-bit LDS read.  dB and dA sum thousands of token products whose total
//   can cancel by five orders of magnitude, so V's rounding error is amplified ~sqrt(T) times:
//   an fp32 V (U from the forward) enters as a bf16 hi + mid + lo triple (split error below fp32
//   rounding); for dA the rows kernel hands over dU in fp64, which enters as four bf16 parts.
// Both use v_mfma_f32_16x16x32_bf16 and move every 32-step MFMA partial into fp64 registers (so
// fp32 rounding acts only inside one 32-term dot product), and write fp64 partials per slice that
// one more kernel sums in a fixed order, so results are independent of scheduling.
#include "common.h"

namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

constexpr int kJ = 64;      // adapter columns per workgroup pass
constexpr int kFlush = 32;   // reduction steps between fp64 flushes

SRA_DEV bf16x8v as_bf16x8(const uint16_t h[8]) {
  union { uint16_t h[8]; bf16x8v v; } u;
#pragma unroll
  for (int q = 0; q < 8; ++q) u.h[q] = h[q];
  return u.v;
}

// ------------------------------------------------------------------------------------ rows
constexpr int RB = 256;            // reduction columns per LDS block
constexpr int RLD = RB + 8;        // padded LDS row (elements)

// grid: (ceil(T/64), ceil(r/64), S); slice z covers c in [z*c_per, (z+1)*c_per), c_per % RB == 0
__global__ __launch_bounds__(256) void k_adapter_rows(const uint16_t* __restrict__ act, int64_t T,
                                                      int64_t C, const uint16_t* __restrict__ wt,
                                                      int64_t wt_sj, int64_t wt_sc, int r,
                                                      int64_t c_per, double* __restrict__ part,
                                                      float* __restrict__ out,
                                                      double* __restrict__ out64) {
  __shared__ __attribute__((aligned(16))) uint16_t wl[kJ * RLD];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int64_t t = (int64_t)blockIdx.x * 64 + w * 16 + lr;  // this lane's A-fragment token
  const int j0 = blockIdx.y * kJ;
  const int jt_n = min(4, (r - j0 + 15) / 16);
  const int64_t cb = (int64_t)blockIdx.z * c_per, ce = min(C, cb + c_per);
  f32x4 acc[4];
  double acc64[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[a][e] = 0.f;
      acc64[a][e] = 0.0;
    }
  int steps = 0;
  const bool a_vec = (C & 7) == 0;                                   // 16-byte aligned rows
  const bool w_vec = wt_sc == 1 ? (wt_sj & 7) == 0 : (wt_sc & 7) == 0;
  for (int64_t c0 = cb; c0 < ce; c0 += RB) {
    __syncthreads();
    // ---- stage Wt(j0 .. j0+63, c0 .. c0+255) as wl[j][c]
    if (wt_sc == 1) {  // c contiguous: lane -> (j, 8 consecutive c); 64 x 32 vectors
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = tid + 256 * i, jj = v >> 5, cc = (v & 31) * 8;
        const int j = j0 + jj;
        const int64_t c = c0 + cc;
        union { u32x4 v; uint16_t h[8]; } x;
        x.v = u32x4{0, 0, 0, 0};
        if (j < r) {
          if (w_vec && c + 8 <= ce) {
            x.v = *reinterpret_cast<const u32x4*>(wt + (int64_t)j * wt_sj + c);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (c + q < ce) x.h[q] = wt[(int64_t)j * wt_sj + c + q];
          }
        }
        *reinterpret_cast<u32x4*>(&wl[jj * RLD + cc]) = x.v;
      }
    } else {  // j contiguous (wt_sj == 1): lane -> (8 consecutive j, c), transposed into wl
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = tid + 256 * i, cc = v >> 3, jj = (v & 7) * 8;
        const int j = j0 + jj;
        const int64_t c = c0 + cc;
        union { u32x4 v; uint16_t h[8]; } x;
        x.v = u32x4{0, 0, 0, 0};
        if (c < ce) {
          if (w_vec && j + 8 <= r) {
            x.v = *reinterpret_cast<const u32x4*>(wt + c * wt_sc + j);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (j + q < r) x.h[q] = wt[c * wt_sc + j + q];
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) wl[(jj + q) * RLD + cc] = x.h[q];
      }
    }
    __syncthreads();
    // ---- 8 chunks of 32 columns
    for (int k = 0; k < RB; k += 32) {
      const int64_t cl = c0 + k + 8 * lg;  // this lane's 8 reduction indices
      if (cl >= ce && c0 + k >= ce) break;
      uint16_t ah[8];
      if (a_vec && t < T && cl + 8 <= ce) {
        union { u32x4 v; uint16_t h[8]; } x;
        x.v = *reinterpret_cast<const u32x4*>(act + t * C + cl);
#pragma unroll
        for (int q = 0; q < 8; ++q) ah[q] = x.h[q];
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) ah[q] = (t < T && cl + q < ce) ? act[t * C + cl + q] : (uint16_t)0;
      }
      const bf16x8v af = as_bf16x8(ah);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (a >= jt_n) break;
        const bf16x8v bfv = *reinterpret_cast<const bf16x8v*>(&wl[(a * 16 + lr) * RLD + k + 8 * lg]);
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfv, acc[a], 0, 0, 0);
      }
      if (++steps == kFlush / 32) {
        steps = 0;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc64[a][e] += (double)acc[a][e];
            acc[a][e] = 0.f;
          }
      }
    }
  }
  // D layout: row (token) 4*(l/16)+e of this wave's 16, column j = l%16
  for (int a = 0; a < jt_n; ++a) {
    const int j = j0 + a * 16 + lr;
    if (j >= r) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t tt = (int64_t)blockIdx.x * 64 + w * 16 + 4 * lg + e;
      if (tt >= T) continue;
      const double s = acc64[a][e] + (double)acc[a][e];
      if (part) {
        part[(int64_t)blockIdx.z * T * r + tt * r + j] = s;
      } else {
        if (out) out[tt * r + j] = (float)s;
        if (out64) out64[tt * r + j] = s;
      }
    }
  }
}

// ------------------------------------------------------------------------------------ cols
constexpr int CT = 32;           // tokens per chunk
constexpr int CLD = CT + 8;      // padded LDS row (elements)

// grid: (ceil(M/64), ceil(r/64), S); slice z covers tokens [z*t_per, (z+1)*t_per), t_per % 32 == 0
__global__ __launch_bounds__(256) void k_adapter_cols(const uint16_t* __restrict__ act, int64_t T,
                                                      int64_t M, const float* __restrict__ V32,
                                                      const double* __restrict__ V64, int r,
                                                      int64_t t_per, bool out_t,
                                                      double* __restrict__ part,
                                                      float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t al[64 * CLD];      // Act^T: [m][t]
  __shared__ __attribute__((aligned(16))) uint16_t vl[4][kJ * CLD];   // V^T split parts: [j][t]
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int j0 = blockIdx.y * kJ;
  const int jt_n = min(4, (r - j0 + 15) / 16);
  const int64_t tb = (int64_t)blockIdx.z * t_per, te = min(T, tb + t_per);
  f32x4 acc[4];
  double acc64[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[a][e] = 0.f;
      acc64[a][e] = 0.0;
    }
  int steps = 0;
  const bool m_vec = (M & 7) == 0, r_vec = (r & 3) == 0;
  const int parts = V64 ? 4 : 3;
  for (int64_t t0 = tb; t0 < te; t0 += CT) {
    __syncthreads();
    {  // Act tile: 32 tokens x 64 columns, lane -> (token, 8 consecutive m), written as [m][t]
      const int tt = tid >> 3, mm = (tid & 7) * 8;
      const int64_t t = t0 + tt, m = m0 + mm;
      union { u32x4 v; uint16_t h[8]; } x;
      x.v = u32x4{0, 0, 0, 0};
      if (t < te) {
        if (m_vec && m + 8 <= M) {
          x.v = *reinterpret_cast<const u32x4*>(act + t * M + m);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (m + q < M) x.h[q] = act[t * M + m + q];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) al[(mm + q) * CLD + tt] = x.h[q];
    }
    // V tile: 32 tokens x 64 adapter columns, lane -> (token, 4 consecutive j), as [j][t] parts
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i, tt = v >> 4, jj = (v & 15) * 4;
      const int64_t t = t0 + tt;
      const int j = j0 + jj;
      double f[4] = {0.0, 0.0, 0.0, 0.0};
      if (t < te) {
        if (V64) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (j + q < r) f[q] = V64[t * r + j + q];
        } else if (r_vec && j + 4 <= r) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(V32 + t * r + j);
#pragma unroll
          for (int q = 0; q < 4; ++q) f[q] = (double)x[q];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (j + q < r) f[q] = (double)V32[t * r + j + q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t pp[4];
        if (V64) {
          split4_bf16(f[q], pp);
        } else {
          split3_bf16((float)f[q], pp[0], pp[1], pp[2]);
          pp[3] = 0;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) vl[p][(jj + q) * CLD + tt] = pp[p];
      }
    }
    __syncthreads();
    // D[j][m] += V^T[j][t] Act[t][m]: A = V^T rows j (k = t), B = Act^T rows m (k = t)
    const bf16x8v bf = *reinterpret_cast<const bf16x8v*>(&al[(w * 16 + lr) * CLD + 8 * lg]);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (a >= jt_n) break;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p >= parts) break;
        const bf16x8v af = *reinterpret_cast<const bf16x8v*>(&vl[p][(a * 16 + lr) * CLD + 8 * lg]);
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[a], 0, 0, 0);
      }
    }
    if (++steps == kFlush / CT) {
      steps = 0;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc64[a][e] += (double)acc[a][e];
          acc[a][e] = 0.f;
        }
    }
  }
  // D layout: row j = 4*(l/16)+e within the j tile, column m = l%16 of this wave's 16
  const int64_t m = m0 + w * 16 + lr;
  if (m >= M) return;
  for (int a = 0; a < jt_n; ++a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + a * 16 + 4 * lg + e;
      if (j >= r) continue;
      const double s = acc64[a][e] + (double)acc[a][e];
      const int64_t o = out_t ? (int64_t)j * M + m : m * r + j;
      if (part)
        part[(int64_t)blockIdx.z * M * r + o] = s;
      else
        out[o] = (float)s;
    }
  }
}

__global__ void k_reduce_parts(const double* __restrict__ part, int S, int64_t n,
                               float* __restrict__ out, double* __restrict__ out64) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int k = 0; k < S; ++k) s += part[(int64_t)k * n + i];
  if (out) out[i] = (float)s;
  if (out64) out64[i] = s;
}

// Number of reduction slices: enough workgroups for the GPU (~512), each slice >= `min_len`.
int n_slices(int64_t blocks, int64_t len, int64_t min_len) {
  if (blocks <= 0 || len <= 0) return 1;
  int64_t S = (512 + blocks - 1) / blocks;
  const int64_t max_s = (len + min_len - 1) / min_len;
  if (S > max_s) S = max_s;
  if (S > 64) S = 64;
  return (int)(S < 1 ? 1 : S);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

namespace sra {

size_t adapter_rows_ws(int64_t T, int64_t C, int r) {
  const int64_t blocks = ((T + 63) / 64) * ((r + kJ - 1) / kJ);
  const int S = n_slices(blocks, C, 512);
  return S > 1 ? (size_t)S * T * r * sizeof(double) : 0;
}

hipError_t launch_adapter_rows(const uint16_t* act, int64_t T, int64_t C, const uint16_t* wt,
                               int64_t wt_sj, int64_t wt_sc, int r, float* out, double* out64,
                               void* ws, hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  if (C == 0) {
    if (out64) return hipErrorInvalidValue;  // callers never ask for fp64 with an empty reduction
    return launch_fill_f32(out, T * r, 0.f, s);
  }
  const int64_t blocks = ((T + 63) / 64) * ((r + kJ - 1) / kJ);
  const int S = n_slices(blocks, C, 512);
  const int64_t c_per = round_up((C + S - 1) / S, RB);
  const int Seff = (int)((C + c_per - 1) / c_per);
  double* part = Seff > 1 ? (double*)ws : nullptr;
  const dim3 grid((unsigned)((T + 63) / 64), (unsigned)((r + kJ - 1) / kJ), (unsigned)Seff);
  launch(SRA_KERNEL_ADAPTER, k_adapter_rows, grid, dim3(256), 0, s, act, T, C, wt, wt_sj, wt_sc,
         r, c_per, part, out, out64);
  if (Seff > 1) {
    const int64_t n = T * r;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       Seff, n, out, out64);
  }
  return hipGetLastError();
}

size_t adapter_cols_ws(int64_t T, int64_t M, int r) {
  const int64_t blocks = ((M + 63) / 64) * ((r + kJ - 1) / kJ);
  const int S = n_slices(blocks, T, 256);
  return S > 1 ? (size_t)S * M * r * sizeof(double) : 0;
}

hipError_t launch_adapter_cols(const uint16_t* act, int64_t T, int64_t M, const float* V32,
                               const double* V64, int r, bool out_transposed, float* out, void* ws,
                               hipStream_t s) {
  if (M == 0 || r == 0) return hipSuccess;
  if (T == 0) return launch_fill_f32(out, M * r, 0.f, s);
  const int64_t blocks = ((M + 63) / 64) * ((r + kJ - 1) / kJ);
  const int S = n_slices(blocks, T, 256);
  const int64_t t_per = round_up((T + S - 1) / S, CT);
  const int Seff = (int)((T + t_per - 1) / t_per);
  double* part = Seff > 1 ? (double*)ws : nullptr;
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((r + kJ - 1) / kJ), (unsigned)Seff);
  launch(SRA_KERNEL_ADAPTER, k_adapter_cols, grid, dim3(256), 0, s, act, T, M, V32, V64, r,
         t_per, out_transposed, part, out);
  if (Seff > 1) {
    const int64_t n = M * r;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       Seff, n, out, nullptr);
  }
  return hipGetLastError();
}

}  // namespace sra

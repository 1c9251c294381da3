// Adapter products of the low-rank branch (SLoPe paperlayer summary §2.2; LoRA):
//   U  = X A^T   [T x r]      dU = dY B   [T x r]
//   dB = dY^T U  [N x r]      dA = dU^T X [r x K]
// all as  Out[m][n] = sum_c P(m, c) Q(n, c)  with arbitrary (row, reduction) strides, bf16 or fp32
// operands and an fp32 result.
//
// One 64 x 64 output tile per workgroup (4 waves of 32 x 32, dense v_mfma_f32_32x32x16_bf16),
// 32 reduction steps per LDS stage.  fp32 operands (U, dU) enter as a bf16 hi + mid + lo triple
// (three MFMAs; the split error is below fp32 rounding), because dB and dA sum thousands of
// token products whose total can cancel by five orders of magnitude, and a two-way split's
// 2^-17 error then shows.  After every stage the fp32 MFMA accumulators are flushed into fp64
// registers; a reduction split over workgroups (for parallelism) writes fp64 partials that one
// more kernel sums in a fixed order, so results do not depend on scheduling.
#include "common.h"

namespace {

constexpr int BM = 64, BN = 64, BCA = 32;
constexpr int LD = 80;  // bytes per LDS row: 32 bf16 + 16 pad
constexpr int kFlushSteps = 32;

struct __align__(16) ASmem {
  uint8_t p[3][BM * LD];  // hi, mid, lo
  uint8_t q[3][BN * LD];
};

// Load a 64 x 32 tile of operand O (rows [r0, r0+64), reduction [c0, c0+32)) into LDS
// hi / mid / lo tiles (mid and lo only for fp32 operands).
SRA_DEV void load_tile(const sra::Operand& O, int64_t rows, int64_t C, int64_t r0, int64_t c0,
                       uint8_t* const* tiles) {
  const int tid = threadIdx.x;
  const bool need_lo = O.f32;
  uint16_t hv[8], mv[8], lv[8];
  int lr, lc;          // tile coordinates of the first of the 8 elements
  bool along_red;      // the 8 elements run along the reduction index (else along rows)
  if (O.s_red == 1) {  // reduction contiguous: lane -> (row, 8 consecutive c)
    lr = tid >> 2;
    lc = (tid & 3) * 8;
    along_red = true;
  } else {  // row index contiguous (or general): lane -> (8 consecutive rows, c)
    lr = (tid >> 5) * 8;
    lc = tid & 31;
    along_red = false;
  }
  const int64_t gr = r0 + lr, gc = c0 + lc;
  const int64_t step = along_red ? O.s_red : O.s_row;
  const int64_t base = gr * O.s_row + gc * O.s_red;
  const bool full = along_red ? (gr < rows && gc + 8 <= C) : (gr + 8 <= rows && gc < C);
  if (O.f32) {
    const float* p = (const float*)O.ptr;
    float v[8];
    if (full && step == 1 && (base & 3) == 0) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(p + base);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(p + base + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = a0[q];
        v[q + 4] = a1[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t r = along_red ? gr : gr + q, c = along_red ? gc + q : gc;
        v[q] = (r < rows && c < C) ? p[r * O.s_row + c * O.s_red] : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) split3_bf16(v[q], hv[q], mv[q], lv[q]);
  } else {
    const uint16_t* p = (const uint16_t*)O.ptr;
    if (full && step == 1 && (base & 7) == 0) {
      union { u32x4 v; uint16_t h[8]; } x;
      x.v = *reinterpret_cast<const u32x4*>(p + base);
#pragma unroll
      for (int q = 0; q < 8; ++q) hv[q] = x.h[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t r = along_red ? gr : gr + q, c = along_red ? gc + q : gc;
        hv[q] = (r < rows && c < C) ? p[r * O.s_row + c * O.s_red] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) mv[q] = lv[q] = 0;
  }
  const uint16_t* parts[3] = {hv, mv, lv};
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (t > 0 && !need_lo) break;
    if (along_red) {
      union { u32x4 v; uint16_t h[8]; } x;
#pragma unroll
      for (int q = 0; q < 8; ++q) x.h[q] = parts[t][q];
      *reinterpret_cast<u32x4*>(tiles[t] + lr * LD + lc * 2) = x.v;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        *reinterpret_cast<uint16_t*>(tiles[t] + (lr + q) * LD + lc * 2) = parts[t][q];
    }
  }
}

__global__ __launch_bounds__(256) void k_adapter_gemm(sra::Operand P, sra::Operand Q, int64_t M,
                                                      int64_t Nn, int64_t C, int64_t c_per_split,
                                                      double* __restrict__ part,
                                                      float* __restrict__ out, int n_tn) {
  __shared__ ASmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = blockIdx.x / n_tn, tn = blockIdx.x - tm * n_tn;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t cb = (int64_t)blockIdx.y * c_per_split, ce = min(C, cb + c_per_split);
  f32x16 acc;
  double acc64[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc[e] = 0.f;
    acc64[e] = 0.0;
  }
  int since_flush = 0;
  for (int64_t c0 = cb; c0 < ce; c0 += BCA) {
    {
      uint8_t* pt[3] = {sm.p[0], sm.p[1], sm.p[2]};
      uint8_t* qt[3] = {sm.q[0], sm.q[1], sm.q[2]};
      load_tile(P, M, ce, m0, c0, pt);
      load_tile(Q, Nn, ce, n0, c0, qt);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int off = (ks * 16 + 8 * g) * 2;
      const bf16x8 ph = *reinterpret_cast<const bf16x8*>(sm.p[0] + (wm * 32 + li) * LD + off);
      const bf16x8 qh = *reinterpret_cast<const bf16x8*>(sm.q[0] + (wn * 32 + li) * LD + off);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, qh, acc, 0, 0, 0);
      if (P.f32) {
#pragma unroll
        for (int t = 1; t < 3; ++t) {
          const bf16x8 pl = *reinterpret_cast<const bf16x8*>(sm.p[t] + (wm * 32 + li) * LD + off);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, qh, acc, 0, 0, 0);
        }
      }
      if (Q.f32) {
#pragma unroll
        for (int t = 1; t < 3; ++t) {
          const bf16x8 ql = *reinterpret_cast<const bf16x8*>(sm.q[t] + (wn * 32 + li) * LD + off);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, ql, acc, 0, 0, 0);
        }
      }
    }
    __syncthreads();
    since_flush += BCA;
    if (since_flush >= kFlushSteps) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc64[e] += (double)acc[e];
        acc[e] = 0.f;
      }
      since_flush = 0;
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) acc64[e] += (double)acc[e];
  const int64_t n = n0 + wn * 32 + li;
  if (n >= Nn) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t m = m0 + wm * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
    if (m >= M) continue;
    if (part)
      part[(int64_t)blockIdx.y * M * Nn + m * Nn + n] = acc64[e];
    else
      out[m * Nn + n] = (float)acc64[e];
  }
}

__global__ void k_reduce_parts(const double* __restrict__ part, int S, int64_t n,
                               float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int k = 0; k < S; ++k) s += part[(int64_t)k * n + i];
  out[i] = (float)s;
}

int n_splits(int64_t M, int64_t Nn, int64_t C) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((Nn + BN - 1) / BN);
  if (tiles == 0 || C <= 0) return 1;
  int64_t S = (512 + tiles - 1) / tiles;
  const int64_t max_s = C / 256 > 1 ? C / 256 : 1;
  if (S > max_s) S = max_s;
  if (S > 64) S = 64;
  return (int)(S > 1 ? S : 1);
}

}  // namespace

namespace sra {

size_t adapter_gemm_ws(int64_t M, int64_t Nn, int64_t C) {
  const int S = n_splits(M, Nn, C);
  return S > 1 ? (size_t)S * M * Nn * sizeof(double) : 0;
}

hipError_t launch_adapter_gemm(const Operand& P, const Operand& Q, int64_t M, int64_t Nn, int64_t C,
                               float* out, void* ws, hipStream_t s) {
  if (M == 0 || Nn == 0) return hipSuccess;
  if (C == 0) return launch_fill_f32(out, M * Nn, 0.f, s);
  const int S = n_splits(M, Nn, C);
  int64_t cps = (C + S - 1) / S;
  cps = (cps + BCA - 1) / BCA * BCA;
  const int Seff = (int)((C + cps - 1) / cps);
  const int n_tm = (int)((M + BM - 1) / BM), n_tn = (int)((Nn + BN - 1) / BN);
  double* part = Seff > 1 ? (double*)ws : nullptr;
  launch(SRA_KERNEL_ADAPTER, k_adapter_gemm, dim3((unsigned)(n_tm * n_tn), (unsigned)Seff), dim3(256), 0,
                     s, P, Q, M, Nn, C, cps, part, out, n_tn);
  if (Seff > 1) {
    const int64_t n = M * Nn;
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       Seff, n, out);
  }
  return hipGetLastError();
}

}  // namespace sra

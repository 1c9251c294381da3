// bf16 2:4 SpMM with a fused low-rank epilogue on gfx950 structured-sparse MFMA (SMFMAC).
//
//   Out[t][row] = sum_c Act[t][c] * S[row][c]  +  sum_j U[t][j] * E(row, j)
//
// forward:  S = Ws (rows = N outputs, c = K),  Act = X,  U = X A^T,  E(n, j) = B[n][j]
// backward: S = P  (rows = K,          c = N),  Act = dY, U = dU,     E(k, j) = A[j][k]
// (SLoPe paperlayer summary §2.1: the double-pruned transpose keeps the backward product N:M;
//  §2.4 and App. D: the adapter product is fused with the following addition.)
//
// The sparse weight is the SMFMAC "A" operand, so each 32x32 accumulator is an Out^T tile
// (rows = weight rows, columns = tokens).  The canonical 2:4 layout feeds SMFMAC directly: a lane
// holding 16 logical columns (8 stored values, 16 contiguous bytes) takes its 4 groups' 2-bit
// fields from one 16-bit half of a metadata word.  The activation lane layout of
// v_smfmac_f32_32x32x32_bf16 is two 8-element runs, at 8g and 8g+16 of the 32-column step
// (g = lane / 32), both plain 16-byte LDS reads.
//
// Tiling: 128 weight rows x 128 tokens per workgroup, 4 waves of 64 x 64 (2 x 2 accumulators),
// 64 logical columns per stage (C % 32 == 0; a final half stage is zero-filled).  Stages are double-buffered in LDS with register prefetch; LDS
// rows are padded by 16 bytes so the 128-bit fragment reads of 16 consecutive lanes hit 16
// distinct 4-bank groups.  The epilogue adds U E^T with dense 32x32x16 MFMAs on the same
// accumulators; U stays fp32 through a bf16 hi + lo split.  Workgroup ids are remapped so that
// tiles sharing weight rows land on the same XCD (and its L2).
#include "common.h"

namespace {

constexpr int BR = 128, BT = 128, BC = 64;
constexpr int A_LD = 80;   // bytes per compressed row in LDS (32 bf16 + pad)
constexpr int B_LD = 144;  // bytes per activation row in LDS (64 bf16 + pad)

struct __align__(16) Smem {
  uint8_t a[2][BR * A_LD];
  uint32_t m[2][BR * 2];
  uint8_t b[2][BT * B_LD];
};

struct Prefetch {
  u32x4 a[2];
  u32x2 m;
  u32x4 b[4];
};

SRA_DEV int xcd_remap(int bid, int nblocks) {
  // Hardware dispatches consecutive workgroup ids round-robin over the 8 XCDs; give each XCD a
  // contiguous range of logical tiles instead.
  const int full = nblocks & ~7;
  if (bid >= full) return bid;
  const int per = full >> 3;
  return (bid & 7) * per + (bid >> 3);
}

__global__ __launch_bounds__(256, 2) void k_spmm24(const uint16_t* __restrict__ s_vals,
                                                   const uint32_t* __restrict__ s_meta, int64_t R,
                                                   int64_t C, const uint16_t* __restrict__ act,
                                                   int64_t T, sra::Epilogue ep,
                                                   uint16_t* __restrict__ out, int n_rt,
                                                   int n_tt) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, n_rt * n_tt);
  const int rt = tile / n_tt, tt = tile - rt * n_tt;
  const int64_t row0 = (int64_t)rt * BR, t0 = (int64_t)tt * BT;
  const int64_t cv = C / 2, cm = C / 32;  // stored values / meta words per weight row
  const int nC = (int)((C + BC - 1) / BC);

  // The last stage may be half full (C % 64 == 32): its upper 32 columns load as zeros.
  auto load = [&](int c, Prefetch& p) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, r = q >> 2, part = q & 3;
      const int64_t row = row0 + r, off = (int64_t)c * 32 + part * 8;
      p.a[i] = (row < R && off < cv) ? *reinterpret_cast<const u32x4*>(s_vals + row * cv + off)
                                     : u32x4{0, 0, 0, 0};
    }
    if (tid < BR) {
      const int64_t row = row0 + tid, w = (int64_t)c * 2;
      p.m = u32x2{0, 0};
      if (row < R) {
        p.m[0] = s_meta[row * cm + w];
        if (w + 1 < cm) p.m[1] = s_meta[row * cm + w + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, tk = q >> 3, part = q & 7;
      const int64_t t = t0 + tk, off = (int64_t)c * BC + part * 8;
      p.b[i] = (t < T && off < C) ? *reinterpret_cast<const u32x4*>(act + t * C + off)
                                  : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf, const Prefetch& p) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, r = q >> 2, part = q & 3;
      *reinterpret_cast<u32x4*>(&sm.a[buf][r * A_LD + part * 16]) = p.a[i];
    }
    if (tid < BR) *reinterpret_cast<u32x2*>(&sm.m[buf][tid * 2]) = p.m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, tk = q >> 3, part = q & 7;
      *reinterpret_cast<u32x4*>(&sm.b[buf][tk * B_LD + part * 16]) = p.b[i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int wr = wave >> 1, wt = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[2];
      int idx[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wr * 64 + i * 32 + li;
        af[i] = *reinterpret_cast<const bf16x8*>(&sm.a[buf][r * A_LD + 32 * s + 16 * g]);
        idx[i] = (int)(sm.m[buf][r * 2 + s] >> (16 * g));
      }
      bf16x16 bfr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tk = wt * 64 + j * 32 + li;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(&sm.b[buf][tk * B_LD + 64 * s + 16 * g]);
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&sm.b[buf][tk * B_LD + 64 * s + 32 + 16 * g]);
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[i], bfr[j], acc[i][j], idx[i], 0, 0);
    }
  };

  {
    Prefetch p;
    load(0, p);
    store(0, p);
  }
  __syncthreads();
  for (int c = 0; c < nC; ++c) {
    Prefetch p;
    const bool more = c + 1 < nC;
    if (more) load(c + 1, p);
    compute(c & 1);
    if (more) store((c + 1) & 1, p);
    __syncthreads();
  }

  // ---- fused low-rank epilogue: acc += E(rows, :) U(tokens, :)^T
  if (ep.r > 0) {
    const bool e_vec = ep.e_j_stride == 1 && (ep.r & 7) == 0;
    const bool u_vec = (ep.r & 7) == 0;
    for (int jj = 0; jj < ep.r; jj += 16) {
      const int jb = jj + 8 * g;
      bf16x8 ef[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t row = row0 + wr * 64 + i * 32 + li;
        union { u32x4 v; uint16_t h[8]; bf16x8 b; } x;
        x.v = u32x4{0, 0, 0, 0};
        if (row < R) {
          if (e_vec && jb + 8 <= ep.r) {
            x.v = *reinterpret_cast<const u32x4*>(ep.E + row * ep.e_row_stride + jb);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (jb + q < ep.r) x.h[q] = ep.E[row * ep.e_row_stride + (int64_t)(jb + q) * ep.e_j_stride];
          }
        }
        ef[i] = x.b;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t t = t0 + wt * 64 + j * 32 + li;
        float u[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = 0.f;
        if (t < T) {
          const float* up = ep.U + t * ep.r + jb;
          if (u_vec && jb + 8 <= ep.r) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(up);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(up + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              u[q] = a0[q];
              u[q + 4] = a1[q];
            }
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (jb + q < ep.r) u[q] = up[q];
          }
        }
        union { uint16_t h[8]; bf16x8 b; } hi, lo;
#pragma unroll
        for (int q = 0; q < 8; ++q) split_bf16(u[q], hi.h[q], lo.h[q]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[i], hi.b, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[i], lo.b, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- store: lane holds, for token (col) li, rows 8a + 4g + {0..3}
  const bool r4 = (R & 3) == 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t t = t0 + wt * 64 + j * 32 + li;
      if (t >= T) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int64_t rb = row0 + wr * 64 + i * 32 + 8 * a + 4 * g;
        uint16_t* o = out + t * R + rb;
        if (r4 && rb + 3 < R) {
          u32x2 v;
          v[0] = pack_bf16x2(acc[i][j][4 * a + 0], acc[i][j][4 * a + 1]);
          v[1] = pack_bf16x2(acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]);
          *reinterpret_cast<u32x2*>(o) = v;
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (rb + b < R) o[b] = f32_to_bf16(acc[i][j][4 * a + b]);
        }
      }
    }
}

}  // namespace

namespace sra {

hipError_t launch_spmm24_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                              const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                              hipStream_t s) {
  if (T == 0 || R == 0) return hipSuccess;
  const int n_rt = (int)((R + BR - 1) / BR), n_tt = (int)((T + BT - 1) / BT);
  launch(SRA_KERNEL_SPMM24, k_spmm24, dim3((unsigned)(n_rt * n_tt)), dim3(256), 0, s, s_vals, s_meta, R,
                     C, act, T, ep, out, n_rt, n_tt);
  return hipGetLastError();
}

}  // namespace sra

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
// Tiling (template): each of the 4 waves owns FR x FT accumulators of 32x32 (a wave tile of
// 32FR rows x 32FT tokens); the waves form a WR x WT grid.  Per SMFMAC cycle a wave reads
// 1024/(32FT) bytes of weights and 2048/(32FR) bytes of activations from LDS, so larger wave tiles
// cut LDS traffic; larger workgroup tiles cut L2 re-reads; small problems need small tiles (or a
// split of the reduction) to occupy 256 CUs.  64 logical columns per stage (C % 32 == 0; a final
// half stage is zero-filled), double-buffered LDS with register prefetch, rows padded by 16
// bytes so the 128-bit fragment reads of 16 consecutive lanes hit distinct bank groups.
// The epilogue adds U E^T with dense 32x32x16 MFMAs on the same accumulators; U stays fp32
// through a bf16 hi + lo split.  A split of the reduction over S workgroups writes fp32 partial
// tiles (the first split adds the epilogue) that a second kernel sums in a fixed order, so the
// result is deterministic.  Workgroup ids are remapped so each XCD runs a contiguous range of
// tiles, ordered in groups of 8 row tiles so concurrent workgroups share both operands in L2.



#include "common.h"
#include "spmm_q.h"

namespace {

constexpr int A_LD = 80;   // bytes per compressed row in LDS (32 bf16 + pad)
constexpr int B_LD = 144;  // bytes per activation row in LDS (64 bf16 + pad)

// Eight consecutive adapter entries E(row, jb .. jb+7) as an MFMA operand (zero past r or R).
SRA_DEV bf16x8 load_e8(const sra::Epilogue& ep, int64_t row, int64_t R, int jb) {
  union { u32x4 v; uint16_t h[8]; bf16x8 b; } x;
  x.v = u32x4{0, 0, 0, 0};
  if (row < R) {
    if (ep.e_j_stride == 1 && (ep.r & 7) == 0 && jb + 8 <= ep.r) {
      x.v = *reinterpret_cast<const u32x4*>(ep.E + row * ep.e_row_stride + jb);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (jb + q < ep.r) x.h[q] = ep.E[row * ep.e_row_stride + (int64_t)(jb + q) * ep.e_j_stride];
    }
  }
  return x.b;
}

template <int FR, int FT, int WR, int WT>
struct Tile {
  static constexpr int BR = 32 * FR * WR, BT = 32 * FT * WT;
  static constexpr int NA = BR * 4 / 256;             // 16-byte value chunks per lane
  static constexpr int NB = BT * 8 / 256;             // 16-byte activation chunks per lane
  static constexpr int OCC = (FR * FT >= 8) ? 1 : 2;  // workgroups per CU the registers allow
  struct __align__(16) Smem {
    uint8_t a[2][BR * A_LD];
    uint32_t m[2][BR * 2];
    uint8_t b[2][BT * B_LD];
  };
  struct Prefetch {
    u32x4 a[NA];
    u32x2 m;
    u32x4 b[NB];
  };
};

template <int FR, int FT, int WR, int WT>
__global__ __launch_bounds__(256, (Tile<FR, FT, WR, WT>::OCC)) void k_spmm24(
    const uint16_t* __restrict__ s_vals, const uint32_t* __restrict__ s_meta, int64_t R, int64_t C,
    const uint16_t* __restrict__ act, int64_t T, sra::Epilogue ep, uint16_t* __restrict__ out,
    float* __restrict__ part, int n_rt, int n_tt, int stages_per_split) {
  using TL = Tile<FR, FT, WR, WT>;
  constexpr int BR = TL::BR, BT = TL::BT, NA = TL::NA, NB = TL::NB;
  static_assert(WR * WT == 4, "4 waves");
  static_assert(NA >= 1 && NB >= 1, "tile too small for the loaders");
  using Smem = typename TL::Smem;
  using Prefetch = typename TL::Prefetch;
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  int rt, tt;
  tile_coords(xcd_remap(blockIdx.x, n_rt * n_tt), n_rt, n_tt, rt, tt);
  const int64_t row0 = (int64_t)rt * BR, t0 = (int64_t)tt * BT;
  const int64_t cv = C / 2, cm = C / 32;  // stored values / meta words per weight row
  const int nC_all = (int)((C + BC - 1) / BC);
  const int z = blockIdx.y;
  const int c_beg = z * stages_per_split;
  const int c_end = min(nC_all, c_beg + stages_per_split);

  // The last stage may be half full (C % 64 == 32): its upper 32 columns load as zeros.
  auto load = [&](int c, Prefetch& p) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + 256 * i, r = q >> 2, part_ = q & 3;
      const int64_t row = row0 + r, off = (int64_t)c * 32 + part_ * 8;
      p.a[i] = (row < R && off < cv) ? *reinterpret_cast<const u32x4*>(s_vals + row * cv + off)
                                     : u32x4{0, 0, 0, 0};
    }
    p.m = u32x2{0, 0};
    if (tid < BR) {
      const int64_t row = row0 + tid, w = (int64_t)c * 2;
      if (row < R) {
        p.m[0] = s_meta[row * cm + w];
        if (w + 1 < cm) p.m[1] = s_meta[row * cm + w + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = tid + 256 * i, tk = q >> 3, part_ = q & 7;
      const int64_t t = t0 + tk, off = (int64_t)c * BC + part_ * 8;
      p.b[i] = (t < T && off < C) ? *reinterpret_cast<const u32x4*>(act + t * C + off)
                                  : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf, const Prefetch& p) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + 256 * i, r = q >> 2, part_ = q & 3;
      *reinterpret_cast<u32x4*>(&sm.a[buf][r * A_LD + part_ * 16]) = p.a[i];
    }
    if (tid < BR) *reinterpret_cast<u32x2*>(&sm.m[buf][tid * 2]) = p.m;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = tid + 256 * i, tk = q >> 3, part_ = q & 7;
      *reinterpret_cast<u32x4*>(&sm.b[buf][tk * B_LD + part_ * 16]) = p.b[i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int wr = wave / WT, wt = wave % WT;
  f32x16 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[FR];
      int idx[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 32 * FR + i * 32 + li;
        af[i] = *reinterpret_cast<const bf16x8*>(&sm.a[buf][r * A_LD + 32 * s + 16 * g]);
        idx[i] = (int)(sm.m[buf][r * 2 + s] >> (16 * g));
      }
      bf16x16 bfr[FT];
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tk = wt * 32 * FT + j * 32 + li;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(&sm.b[buf][tk * B_LD + 64 * s + 16 * g]);
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&sm.b[buf][tk * B_LD + 64 * s + 32 + 16 * g]);
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[i], bfr[j], acc[i][j], idx[i], 0, 0);
    }
  };

  if (c_beg < c_end) {
    {
      Prefetch p;
      load(c_beg, p);
      store(0, p);
    }
    __syncthreads();
    for (int c = c_beg; c < c_end; ++c) {
      Prefetch p;
      const bool more = c + 1 < c_end;
      if (more) load(c + 1, p);
      compute((c - c_beg) & 1);
      if (more) store((c + 1 - c_beg) & 1, p);
      __syncthreads();
    }
  }

  // ---- fused low-rank epilogue (first split only): acc += E(rows, :) U(tokens, :)^T
  if (ep.r > 0 && z == 0) {
    const bool e_vec = ep.e_j_stride == 1 && (ep.r & 7) == 0;
    const bool u_vec = (ep.r & 7) == 0;
    for (int jj = 0; jj < ep.r; jj += 16) {
      const int jb = jj + 8 * g;
      bf16x8 ef[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int64_t row = row0 + wr * 32 * FR + i * 32 + li;
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
      for (int j = 0; j < FT; ++j) {
        const int64_t t = t0 + wt * 32 * FT + j * 32 + li;
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
        for (int i = 0; i < FR; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[i], hi.b, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[i], lo.b, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- store: lane holds, for token (col) li, rows 8a + 4g + {0..3}
  const bool r4 = (R & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int64_t t = t0 + wt * 32 * FT + j * 32 + li;
      if (t >= T) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int64_t rb = row0 + wr * 32 * FR + i * 32 + 8 * a + 4 * g;
        if (part) {  // fp32 partial of split z, in the output's [t][row] layout
          float* o = part + ((int64_t)z * T + t) * R + rb;
          if (r4 && rb + 3 < R) {
            *reinterpret_cast<f32x4*>(o) = f32x4{acc[i][j][4 * a], acc[i][j][4 * a + 1],
                                                 acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]};
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (rb + b < R) o[b] = acc[i][j][4 * a + b];
          }
          continue;
        }
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

// ---------------------------------------------------------------------------------------------
// Pipelined variant (C % 64 == 0): operands move global -> LDS with global_load_lds (no register
// staging) into a ring of NS stage buffers, issued NS-1 stages ahead of the MFMAs.  Every wave
// issues the same number L of 1 KB (dwordx4) / 256 B (dword, metadata) transfers per stage, so
// "stage c has landed" is a compile-time vmcnt.  A DMA writes lane i's 16 bytes at slot i of its
// 1 KB block, so each lane chooses which global chunk to fetch: LDS rows are XOR-swizzled
// (chunk ^ f(row)) instead of padded, and the 128-bit fragment reads of 16 consecutive lanes
// still hit 16 distinct bank groups.  Rows / tokens past the edge read a clamped valid address
// and their results are never stored.
// UG > 0: UG adapter rows G (Epilogue::G) ride along as rows BT .. BT+UG-1 of each stage's
// activation region (same 128-byte rows and swizzle as the tokens), in GT 1 KB transfers per
// stage spread over the waves (GW each, one more for the first GX waves).
template <int FR, int FT, int WR, int WT, int NS, int UG = 0>
struct PTile {
  static constexpr int BR = 32 * FR * WR, BT = 32 * FT * WT;
  static constexpr int LA = BR / 64, LM = BR / 128, LB = BT / 32;  // transfers per wave per stage
  static constexpr int GT = UG / 8, GW = GT / 4, GX = GT % 4;
  static constexpr int L = LA + LM + LB + GW;  // waves >= GX
  static constexpr int L1 = L + (GX ? 1 : 0);  // waves < GX
  static constexpr int A_BYTES = BR * 64, M_BYTES = BR * 8, B_BYTES = (BT + UG) * 128;
  static constexpr int STAGE = A_BYTES + M_BYTES + B_BYTES;
  static constexpr int LDS = NS * STAGE;
  static constexpr int OCC = (FR * FT >= 8 || 2 * LDS > 160 * 1024) ? 1 : 2;
};

template <int FR, int FT, int WR, int WT, int NS, int UG = 0>
__global__ __launch_bounds__(256, (PTile<FR, FT, WR, WT, NS, UG>::OCC)) void k_spmm24_pipe(
    const uint16_t* __restrict__ s_vals, const uint32_t* __restrict__ s_meta, int64_t R, int64_t C,
    const uint16_t* __restrict__ act, int64_t T, sra::Epilogue ep, uint16_t* __restrict__ out,
    float* __restrict__ part, int n_rt, int n_tt, int stages_per_split) {
  using TL = PTile<FR, FT, WR, WT, NS, UG>;
  using AD = AdapterRows<TL::BT, (UG > 0 ? UG : 16), 4>;
  static_assert(UG == 0 || AD::ULD * 4 * TL::BT <= TL::LDS, "U tile fits in LDS");
  constexpr int BR = TL::BR, BT = TL::BT, L = TL::L;
  static_assert(WR * WT == 4, "4 waves");
  static_assert(BR % 128 == 0 && BT % 32 == 0, "transfer counts must be whole per wave");
  __shared__ __attribute__((aligned(16))) uint8_t smem[TL::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  int rt, tt;
  tile_coords(xcd_remap(blockIdx.x, n_rt * n_tt), n_rt, n_tt, rt, tt);
  const int64_t row0 = (int64_t)rt * BR, t0 = (int64_t)tt * BT;
  const int64_t cv = C / 2, cm = C / 32;
  const int nC_all = (int)(C / BC);
  const int z = blockIdx.y;
  const int c_beg = z * stages_per_split;
  const int c_end = min(nC_all, c_beg + stages_per_split);

  // Operands through buffer resources based at the tile: each lane's offset is fixed and the stage
  // moves an SGPR offset (c*64 bytes of values, c*8 of metadata, c*128 of activations and adapter
  // rows), so issuing a stage costs no vector address arithmetic; rows past R, T or r are out of
  // range and read as zeros.
  const int rows_here = (int)min((int64_t)BR, R - row0), toks_here = (int)min((int64_t)BT, T - t0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(s_vals + row0 * cv), 0, rows_here * (int)C, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(s_meta + row0 * cm), 0, rows_here * (int)cm * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(act + t0 * C), 0, toks_here * (int)C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ep.G, 0, UG > 0 ? ep.r * (int)ep.g_ld * 2 : 0, 0x00020000);
  uint32_t a_off[TL::LA], m_off[TL::LM], b_off[TL::LB];
  int a_dst[TL::LA], m_dst[TL::LM], b_dst[TL::LB];
#pragma unroll
  for (int k = 0; k < TL::LA; ++k) {
    const int b = k * 4 + wave, row = 16 * b + (lane >> 2), pos = lane & 3;
    const int ch = pos ^ ((row >> 2) & 3);
    a_off[k] = (uint32_t)(row * C + ch * 16);
    a_dst[k] = b * 1024;
  }
#pragma unroll
  for (int k = 0; k < TL::LM; ++k) {
    const int b = k * 4 + wave, row = 32 * b + (lane >> 1);
    m_off[k] = (uint32_t)((row * cm + (lane & 1)) * 4);
    m_dst[k] = TL::A_BYTES + b * 256;
  }
#pragma unroll
  for (int k = 0; k < TL::LB; ++k) {
    const int b = k * 4 + wave, tk = 8 * b + (lane >> 3), pos = lane & 7;
    const int ch = pos ^ ((tk >> 1) & 7);
    b_off[k] = (uint32_t)((tk * C + ch * 8) * 2);
    b_dst[k] = TL::A_BYTES + TL::M_BYTES + b * 1024;
  }
  // adapter rows: transfer k*4 + wave (< GT) moves rows BT + 8(k*4 + wave) .. +7 of the region
  constexpr int NG = TL::GW + (TL::GX ? 1 : 0);
  uint32_t g_off[NG ? NG : 1];
  int g_dst[NG ? NG : 1];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int b = k * 4 + wave, tk = BT + 8 * b + (lane >> 3), pos = lane & 7;
    const int ch = pos ^ ((tk >> 1) & 7);
    g_off[k] = (uint32_t)(((tk - BT) * ep.g_ld + ch * 8) * 2);
    g_dst[k] = TL::A_BYTES + TL::M_BYTES + (BT / 8 + b) * 1024;
  }
  auto issue = [&](int c, int buf) {
    uint8_t* base = smem + buf * TL::STAGE;
#pragma unroll
    for (int k = 0; k < TL::LA; ++k) bdma(ra, base + a_dst[k], 16, a_off[k], c * 64);
#pragma unroll
    for (int k = 0; k < TL::LM; ++k) bdma(rm, base + m_dst[k], 4, m_off[k], c * 8);
#pragma unroll
    for (int k = 0; k < TL::LB; ++k) bdma(rb, base + b_dst[k], 16, b_off[k], c * 128);
#pragma unroll
    for (int k = 0; k < NG; ++k)
      if (k < TL::GW || wave < TL::GX) bdma(rg, base + g_dst[k], 16, g_off[k], c * 128);
  };
  AD ad;
  if constexpr (UG > 0) ad.zero();

  f32x16 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int wr = wave / WT, wt = wave % WT;
  // One stage: every fragment read first (one LDS round trip), then the adapter-row MFMAs (which
  // do not depend on the accumulators), then the sparse products.
  auto compute = [&](int buf) {
    const uint8_t* A = smem + buf * TL::STAGE;
    const uint32_t* M = reinterpret_cast<const uint32_t*>(A + TL::A_BYTES);
    const uint8_t* B = A + TL::A_BYTES + TL::M_BYTES;
    if constexpr (UG > 0) ad.flush();
    bf16x8 af[2][FR];
    int idx[2][FR];
    bf16x16 bfr[2][FT];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 32 * FR + i * 32 + li;
        af[s][i] = *reinterpret_cast<const bf16x8*>(A + r * 64 + (((2 * s + g) ^ ((r >> 2) & 3)) << 4));
        idx[s][i] = (int)(M[r * 2 + s] >> (16 * g));
      }
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tk = wt * 32 * FT + j * 32 + li, sw = (tk >> 1) & 7;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 * s + g) ^ sw) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 * s + 2 + g) ^ sw) << 4));
        bfr[s][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
    }
    if constexpr (UG > 0) ad.read(B, wave, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
    if constexpr (UG > 0) ad.mma(wave);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[s][i], bfr[s][j], acc[i][j], idx[s][i], 0, 0);
  };

  constexpr int D = NS - 1;  // stages in flight ahead of the one being computed
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (c_beg + d < c_end) issue(c_beg + d, d);
  // Steady state, unrolled by the ring depth so that every buffer index (LDS addresses, DMA
  // destinations) is a constant: D stages in flight at each wait.
  int c = c_beg;
  for (; c + NS + D <= c_end; c += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (TL::GX && wave < TL::GX) wait_vm<((D - 1) * TL::L1 < 63 ? (D - 1) * TL::L1 : 63)>();
      else wait_vm<((D - 1) * L < 63 ? (D - 1) * L : 63)>();
      ring_barrier();  // stage c+u visible to all waves; stage c+u-1 consumed
      issue(c + u + D, (u + D) % NS);
      compute(u);
    }
  }
  for (; c < c_end; ++c) {
    const int in_flight = min(D, c_end - c);  // stages c .. c+in_flight-1 were issued
    if (TL::GX && wave < TL::GX) wait_stages<TL::L1>(in_flight);
    else wait_stages<L>(in_flight);
    ring_barrier();
    if (c + D < c_end) issue(c + D, (c - c_beg + D) % NS);
    compute((c - c_beg) % NS);
  }
  if constexpr (UG > 0) ad.flush();

  // ---- in-kernel U: hand the tile over through LDS (and write U / V^T from the first row tile)
  float* const ut = reinterpret_cast<float*>(smem);
  if constexpr (UG > 0) {
    __syncthreads();  // every wave is done with the operand ring
    ad.hand_over(ut, wave, lane, rt == 0, t0, T, ep);
    __syncthreads();
  }

  // ---- fused low-rank epilogue (first split only): acc += E(rows, :) U(tokens, :)^T
  if (ep.r > 0 && z == 0) {
    const bool u_vec = (ep.r & 7) == 0;
    for (int jj = 0; jj < ep.r; jj += 16) {
      const int jb = jj + 8 * g;
      bf16x8 ef[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i) ef[i] = load_e8(ep, row0 + wr * 32 * FR + i * 32 + li, R, jb);
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tl = wt * 32 * FT + j * 32 + li;
        const int64_t t = t0 + tl;
        float u[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = 0.f;
        if (UG > 0 && t < T) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (jb + q < ep.r) u[q] = ut[tl * AD::ULD + jb + q];
        } else if (t < T) {
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
        for (int i = 0; i < FR; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[i], hi.b, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[i], lo.b, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- store: lane holds rows 8a+4g .. +3 of token li in each 32x32 accumulator
  using OB = OutStage<BR, false>;
  using OP = OutStage<BR, true>;
  constexpr bool stage_bf16 = OB::template bytes<BT>() <= TL::LDS;
  constexpr bool stage_f32 = OP::template bytes<BT>() <= TL::LDS;
  if ((part && stage_f32) || (!part && stage_bf16)) {
    __syncthreads();  // every wave is done with the operand ring
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int tok = wt * 32 * FT + j * 32 + li, row = wr * 32 * FR + i * 32 + 8 * a + 4 * g;
          const f32x16& c = acc[i][j];
          if (part) OP::put(smem, tok, row, c[4 * a], c[4 * a + 1], c[4 * a + 2], c[4 * a + 3]);
          else OB::put(smem, tok, row, c[4 * a], c[4 * a + 1], c[4 * a + 2], c[4 * a + 3]);
        }
    __syncthreads();
    if (part) OP::template flush<BT>(smem, part + (int64_t)z * T * R, row0, t0, R, T);
    else OB::template flush<BT>(smem, out, row0, t0, R, T);
    return;
  }
  const bool r4 = (R & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int64_t t = t0 + wt * 32 * FT + j * 32 + li;
      if (t >= T) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int64_t rb = row0 + wr * 32 * FR + i * 32 + 8 * a + 4 * g;
        if (part) {
          float* o = part + ((int64_t)z * T + t) * R + rb;
          if (r4 && rb + 3 < R) {
            *reinterpret_cast<f32x4*>(o) = f32x4{acc[i][j][4 * a], acc[i][j][4 * a + 1],
                                                 acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]};
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (rb + b < R) o[b] = acc[i][j][4 * a + b];
          }
          continue;
        }
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

// register-staged (any C % 32 == 0): 3 = 128x128 (2x2 accumulators per wave)
// LDS-DMA pipelined on 32x32x32 SMFMAC (C % 64 == 0): 13 = 128x128 (3 stages), 14 = 128x64 (4)
// eight waves (512 threads) on 16x16x64 SMFMAC, 64-column stages:
//   50 = 256x128 (4x2 waves of 64x64, 4 stages), 51 = 256x256 (4x2 waves of 64x128, 3)
// the same with metadata in super-stages (C % 128 == 0): 55 = 256x128 (8-stage super-stages,
//   4 stages), 61 = 256x256 (4-stage super-stages, 32-byte runs, so three stages fit)
// ping-pong (waves 0-3 and 4-7 half a stage apart, reads of one group beside the products of the
// other): 62 = 61 so scheduled
// streaming decode kernel (T <= 16, one 16-token column tile, weight read once from HBM):
//   30 = 48 to 144 weight rows per workgroup (decode24.hip)
constexpr Cfg kCfgs[] = {{3, 128, 128, false}, {13, 128, 128, true}, {14, 128, 64, true},
                         {30, 64, 16, false}, {50, 256, 128, true}, {51, 256, 256, true},
                         {55, 256, 128, true, 64, true}, {61, 256, 256, true, 64, true},
                         {62, 256, 256, true, 64, true}};

Cfg cfg_by_id(int id) {
  for (const Cfg& c : kCfgs)
    if (c.id == id) return c;
  return kCfgs[0];
}

Plan plan_for(int64_t R, int64_t C, int64_t T) {
  const bool pipe_ok = C % 64 == 0, wide_ok = C % 128 == 0;
  Plan p{cfg_by_id(pipe_ok ? 13 : 3), 1, 1};
  if (T <= 0 || R <= 0 || C <= 0) return p;
  const sra::Tuning& tu = sra::tuning();
  if (T <= 16) {
    p.cfg = cfg_by_id(30);  // few tokens: bound by reading the weight once (a forced tile is ignored)
  } else if (tu.spmm_cfg > 0) {
    Cfg c = cfg_by_id(tu.spmm_cfg);
    if (c.super && !wide_ok) c = cfg_by_id(pipe_ok ? 13 : 3);
    if (c.pipe && !pipe_ok) c = cfg_by_id(3);
    if (c.id == 30) c = cfg_by_id(pipe_ok ? 13 : 3);
    p.cfg = c;
    p.splits = tu.spmm_splits == -2 ? 2 : tu.spmm_splits > 1 ? tu.spmm_splits : 1;
    p.tail = tu.spmm_splits == -2;  // split only the last wave's tiles
  } else {
    // Measured on MI355X (2:4, bf16): once 256x256 tiles fill the GPU twice, eight-wave 256x256
    // tiles with three stages and 4-stage metadata super-stages (C % 128 == 0; else per-stage
    // metadata, or 256x128 with four stages for long reductions, C >= 2R); eight-wave 256x128
    // once those fill the GPU; 128x64 for long reductions that would otherwise need a split;
    // otherwise 128x128 (two workgroups per CU), splitting the reduction when even those leave
    // CUs idle.
    auto tiles = [&](int br, int bt) { return ((R + br - 1) / br) * ((T + bt - 1) / bt); };
    if (pipe_ok && tiles(256, 256) >= 512) {
      p.cfg = cfg_by_id(wide_ok ? 61 : C >= 2 * R ? 50 : 51);
      // long reductions whose tiles leave the last wave of 256 workgroups at most half full: the
      // tiles of that wave are split in two over the reduction (8-stage aligned), which fills it
      // with half-length workgroups; the others run whole
      const int64_t t = tiles(256, 256);
      if (wide_ok && C >= 2 * R && C % 1024 == 0 && t % 256 != 0 && t % 256 <= 128) {
        p.splits = 2;
        p.tail = true;
      }
    } else if (pipe_ok && tiles(256, 128) >= 240) {
      p.cfg = cfg_by_id(wide_ok ? 55 : 50);
    } else if (pipe_ok && tiles(128, 64) >= 240 && C >= 2048) {
      p.cfg = cfg_by_id(14);  // long reductions: 128x64 tiles beat 128x128 split plus its reduction
    } else {
      p.cfg = cfg_by_id(pipe_ok ? 13 : 3);
      const int64_t t = tiles(128, 128);
      if (t < 240) {
        const int nC = (int)((C + p.cfg.width - 1) / p.cfg.width);
        int s = (int)((256 + t - 1) / t);
        if (s > nC / 8) s = nC / 8;  // keep >= 8 stages per split
        p.splits = s < 1 ? 1 : s;
      }
    }
  }
  const int nC = (int)((C + p.cfg.width - 1) / p.cfg.width);
  // Metadata super-stages allow a split of the reduction when every split starts on a
  // super-stage boundary (the 256x256 tile's 4-stage super-stages, 8-stage splits).
  const bool super_split = p.cfg.id == 61 && p.splits > 1 && nC % (8 * p.splits) == 0;
  if (p.splits < 1 || p.cfg.id == 30 || (p.cfg.super && !super_split)) p.splits = 1;
  if (p.splits != 2 || p.cfg.id != 61) p.tail = false;  // the 256x256 tiling of finish_split
  if (p.splits > nC) p.splits = nC;
  p.stages_per_split = (nC + p.splits - 1) / p.splits;
  p.splits = (nC + p.stages_per_split - 1) / p.stages_per_split;
  return p;
}

template <int FR, int FT, int WR, int WT>
void launch_cfg(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                const uint16_t* act, int64_t T, const sra::Epilogue& ep, uint16_t* out, float* part,
                const Plan& p, hipStream_t s) {
  using TL = Tile<FR, FT, WR, WT>;
  const int n_rt = (int)((R + TL::BR - 1) / TL::BR), n_tt = (int)((T + TL::BT - 1) / TL::BT);
  sra::launch(SRA_KERNEL_SPMM24, k_spmm24<FR, FT, WR, WT>,
              dim3((unsigned)(n_rt * n_tt), (unsigned)p.splits), dim3(256), 0, s, s_vals, s_meta, R,
              C, act, T, ep, out, part, n_rt, n_tt, p.stages_per_split);
}

template <int FR, int FT, int WR, int WT, int NS, int UG = 0>
void launch_pipe(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                 const uint16_t* act, int64_t T, const sra::Epilogue& ep, uint16_t* out,
                 float* part, const Plan& p, hipStream_t s) {
  using TL = PTile<FR, FT, WR, WT, NS, UG>;
  const int n_rt = (int)((R + TL::BR - 1) / TL::BR), n_tt = (int)((T + TL::BT - 1) / TL::BT);
  sra::launch(SRA_KERNEL_SPMM24, k_spmm24_pipe<FR, FT, WR, WT, NS, UG>,
              dim3((unsigned)(n_rt * n_tt), (unsigned)p.splits), dim3(256), 0, s, s_vals, s_meta, R,
              C, act, T, ep, out, part, n_rt, n_tt, p.stages_per_split);
}

// In-kernel adapter rows (Epilogue::G): ranks up to 16, one reduction pass (no split), and the
// configurations that keep their occupancy and registers with the 2 KB of adapter rows added to
// each stage (the 256x128 eight-wave tile drops to 3 stages for it; the 256x256 one would spill).
// The tuning knob SRA_TUNE_SPMM_FUSE = 0 turns it off.
constexpr int kFuseRank = 16;
bool fuse_ok(const Plan& p, int64_t C, int r) {
  if (r <= 0 || r > kFuseRank || C % 64 != 0 || p.splits != 1 || !sra::tuning().spmm_fuse) return false;
  return p.cfg.id == 14 || (p.cfg.id == 55 && C % 128 == 0);
}

}  // namespace

namespace sra {

// The fixed fan-in product on the tiled entry lists of sra_ffi_tile: the dense-weight (DN) tiles
// of the SpMM kernel, with each stage's A tile written from the entries in LDS instead of
// transferred (C % 64 == 0).
// Lists of up to 256 entries per 32 rows and stage ride the ring (longer ones finish from memory);
// denser weights (more than 216 words per list on average: at 10.5% density a list of 2048
// cells holds 215 +- 14 entries, so 256 covers all but a few) take the four-wave tile with
// 1024-entry slots.
hipError_t launch_ffi_tiled_bf16(const uint32_t* ent, const uint32_t* offs, size_t ent_bytes, int64_t R,
                                 int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                 uint16_t* out, hipStream_t s) {
  if (T == 0 || R == 0) return hipSuccess;
  if (C <= 0 || C % 64 != 0 || ep.G || !epilogue_ok(ep, R) || ent_bytes >= ((size_t)1 << 31))
    return hipErrorInvalidValue;
  Plan p{cfg_by_id(13), 1, (int)(C / 64)};
  const auto* v = reinterpret_cast<const uint16_t*>(ent);
  const uint32_t eb = (uint32_t)ent_bytes;
  const int64_t lists = ((R + 31) / 32) * (C / 64);
  const int64_t huge = ((R + 255) / 256) * ((T + 255) / 256), big = ((R + 255) / 256) * ((T + 127) / 128);
  constexpr int K = SRA_KERNEL_SPMM_FFI;
  if ((int64_t)(ent_bytes / 4) > 216 * lists)  // four waves, 128x64 tiles, 3 stages, 1024-entry slots
    launch_q<4, 2, 2, 2, 3, 0, 0, true, false, false, 0, 1024>(v, offs, R, C, act, T, ep, out, nullptr, p, s, K, eb);
  else if (huge >= 240)  // eight waves, 256x256 tiles, 2 stages of 32 KB + 8 KB of entries
    launch_q<4, 8, 4, 2, 2, 0, 0, true, false, false, 0, 256>(v, offs, R, C, act, T, ep, out, nullptr, p, s, K, eb);
  else if (big >= 240)   // eight waves, 256x128 tiles, 3 stages of 16 KB + 8 KB
    launch_q<4, 4, 4, 2, 3, 0, 0, true, false, false, 0, 256>(v, offs, R, C, act, T, ep, out, nullptr, p, s, K, eb);
  else                   // four waves, 128x64 tiles, 3 stages of 8 KB + 4 KB, two workgroups per CU
    launch_q<4, 2, 2, 2, 3, 0, 0, true, false, false, 0, 256>(v, offs, R, C, act, T, ep, out, nullptr, p, s, K, eb);
  return hipGetLastError();
}

bool spmm24_fuses_adapter(int64_t R, int64_t C, int64_t T, int r) {
  if (T <= 0 || R <= 0) return false;
  return fuse_ok(plan_for(R, C, T), C, r);
}

size_t spmm24_ws(int64_t R, int64_t C, int64_t T) {
  const Plan p = plan_for(R, C, T);
  return p.splits > 1 ? (size_t)p.splits * T * R * sizeof(float) : 0;
}

// The same product on the streaming layout (sra_nm_tile).  T <= 16 goes to the decode kernel;
// otherwise the metadata super-stage kernels read the 1 KB blocks: the tile shape follows the
// canonical plan (256x256, 256x128 or a 128-row tile), never split, C % 128 == 0.
bool spmm24_tiled_ok(int64_t C, int64_t T) { return T <= 16 || C % 128 == 0; }

hipError_t launch_spmm24_tiled_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R,
                                    int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                    uint16_t* out, void* ws, hipStream_t s) {
  if (T == 0 || R == 0) return hipSuccess;
  if (T <= 16) return launch_decode24_bf16(s_vals, s_meta, R, C, act, T, ep, out, s, /*tiled=*/true);
  if (C % 128 != 0 || !epilogue_ok(ep, R)) return hipErrorInvalidValue;
  Plan p = plan_for(R, C, T);
  const int id = p.cfg.id;
  const bool fuse = ep.G != nullptr;
  if (fuse && (!fuse_ok(p, C, ep.r) || ep.g_ld % 8 != 0)) return hipErrorInvalidValue;
  // only the 256x256 tile splits (8-stage aligned, the plan's own split); others run whole
  if (!(id == 61 && p.splits > 1 && !fuse && ws)) {
    p.splits = 1;
    p.tail = false;
    p.stages_per_split = (int)((C + 63) / 64);
  }
  float* part = p.splits > 1 ? (float*)ws : nullptr;
  const bool wide = id == 51 || id == 61;  // 256x256
  const bool mid = id == 50 || id == 55;   // 256x128
  if (fuse) {
    if (id == 55) launch_q<4, 4, 4, 2, 3, 8, 16, false, true>(s_vals, s_meta, R, C, act, T, ep, out, nullptr, p, s);
    else launch_q<2, 2, 4, 2, 4, 8, 16, false, true>(s_vals, s_meta, R, C, act, T, ep, out, nullptr, p, s);
  } else if (id == 62) {
    launch_q<4, 8, 4, 2, 3, 4, 0, false, true, true>(s_vals, s_meta, R, C, act, T, ep, out, nullptr, p, s);
  } else if (wide) {
    launch_q<4, 8, 4, 2, 3, 4, 0, false, true>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s);
  } else if (mid) {
    launch_q<4, 4, 4, 2, 4, 8, 0, false, true>(s_vals, s_meta, R, C, act, T, ep, out, nullptr, p, s);
  } else {
    launch_q<2, 2, 4, 2, 4, 8, 0, false, true>(s_vals, s_meta, R, C, act, T, ep, out, nullptr, p, s);
  }
  if (part) finish_split(p, part, R, T, out, s);
  return hipGetLastError();
}

hipError_t launch_spmm24_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                              const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                              void* ws, hipStream_t s) {
  if (T == 0 || R == 0) return hipSuccess;
  if (!epilogue_ok(ep, R)) return hipErrorInvalidValue;
  const Plan p = plan_for(R, C, T);
  float* part = p.splits > 1 ? (float*)ws : nullptr;
  const bool fuse = ep.G != nullptr;
  if (fuse && (!fuse_ok(p, C, ep.r) || ep.g_ld % 8 != 0)) return hipErrorInvalidValue;
  if (fuse) {
    switch (p.cfg.id) {
      case 14: launch_pipe<2, 1, 2, 2, 4, 16>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
      case 55: launch_q<4, 4, 4, 2, 3, 8, 16>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (p.cfg.id) {
    case 30: return launch_decode24_bf16(s_vals, s_meta, R, C, act, T, ep, out, s);
    case 55: launch_q<4, 4, 4, 2, 4, 8>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 61: launch_q<4, 8, 4, 2, 3, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 62: launch_q<4, 8, 4, 2, 3, 4, 0, false, false, true>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 50: launch_q<4, 4, 4, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 51: launch_q<4, 8, 4, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 13: launch_pipe<2, 2, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 14: launch_pipe<2, 1, 2, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    default: launch_cfg<2, 2, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
  }
  if (p.splits > 1) finish_split(p, part, R, T, out, s);
  return hipGetLastError();
}

}  // namespace sra

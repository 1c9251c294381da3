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
#include <cstdlib>
#include <cstring>

#include "common.h"

namespace {

constexpr int BC = 64;
constexpr int A_LD = 80;   // bytes per compressed row in LDS (32 bf16 + pad)
constexpr int B_LD = 144;  // bytes per activation row in LDS (64 bf16 + pad)

SRA_DEV int xcd_remap(int bid, int nblocks) {
  // Hardware dispatches consecutive workgroup ids round-robin over the 8 XCDs; give each XCD a
  // contiguous range of logical tiles instead.
  const int full = nblocks & ~7;
  if (bid >= full) return bid;
  const int per = full >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Logical tile id -> (row tile, token tile) in groups of 8 row tiles: consecutive ids (which run
// concurrently on one XCD) sweep 8 row tiles for each token tile, so the XCD's L2 serves both
// operands to ~8 workgroups each instead of re-streaming activations once per row tile.
SRA_DEV void tile_coords(int L, int n_rt, int n_tt, int& rt, int& tt) {
  constexpr int G = 8;
  const int per_group = G * n_tt;
  const int group = L / per_group, first = group * G;
  const int gsize = min(G, n_rt - first);
  const int in = L - group * per_group;
  rt = first + in % gsize;
  tt = in / gsize;
}


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

// Output tile staged through LDS so that global stores are whole 16-byte vectors along a token's
// row of Y (consecutive weight rows): the MFMA accumulator layout gives each lane 4 rows of one
// token, which written directly would be 8-byte pieces 2R bytes apart.  Layout [token][row] with a
// 16-byte pad per token row; bf16 for the final output, fp32 for split-K partials.
template <int BR, bool F32>
struct OutStage {
  static constexpr int LD = BR + (F32 ? 4 : 8);  // elements per staged token row
  static constexpr int EV = F32 ? 4 : 8;         // elements per 16-byte vector
  template <int BT>
  static constexpr int bytes() { return BT * LD * (F32 ? 4 : 2); }
  // four consecutive rows (row .. row+3) of token tok
  static SRA_DEV void put(uint8_t* smem, int tok, int row, float v0, float v1, float v2, float v3) {
    if constexpr (F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(smem) + tok * LD + row) = f32x4{v0, v1, v2, v3};
    } else {
      u32x2 p;
      p[0] = pack_bf16x2(v0, v1);
      p[1] = pack_bf16x2(v2, v3);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(smem) + tok * LD + row) = p;
    }
  }
  // copy the staged BT x BR tile to dst[(t0 + tok) * R + row0 + row], inside T x R
  template <int BT>
  static SRA_DEV void flush(const uint8_t* smem, void* dst, int64_t row0, int64_t t0, int64_t R,
                            int64_t T) {
    constexpr int VPR = BR / EV;
    const bool vec = R % EV == 0;
    for (int v = threadIdx.x; v < BT * VPR; v += blockDim.x) {
      const int tok = v / VPR, ch = v - tok * VPR;
      const int64_t t = t0 + tok, row = row0 + (int64_t)ch * EV;
      if (t >= T || row >= R) continue;
      if constexpr (F32) {
        const float* src = reinterpret_cast<const float*>(smem) + tok * LD + ch * EV;
        float* o = reinterpret_cast<float*>(dst) + t * R + row;
        if (vec && row + EV <= R) {
          *reinterpret_cast<f32x4*>(o) = *reinterpret_cast<const f32x4*>(src);
        } else {
          for (int e = 0; e < EV && row + e < R; ++e) o[e] = src[e];
        }
      } else {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(smem) + tok * LD + ch * EV;
        uint16_t* o = reinterpret_cast<uint16_t*>(dst) + t * R + row;
        if (vec && row + EV <= R) {
          *reinterpret_cast<u32x4*>(o) = *reinterpret_cast<const u32x4*>(src);
        } else {
          for (int e = 0; e < EV && row + e < R; ++e) o[e] = src[e];
        }
      }
    }
  }
};

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

SRA_DEV void dma16(const void* g, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_block, 16, 0, 0);
}
SRA_DEV void dma4(const void* g, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_block, 4, 0, 0);
}
// buffer -> LDS transfer of `size` bytes per lane at lane offset `voff` + wave-uniform `soff`
SRA_DEV void bdma(__amdgpu_buffer_rsrc_t rs, uint8_t* lds_block, int size, uint32_t voff, int soff) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds_block, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds_block, 4, voff, soff, 0, 0);
}
// s_waitcnt vmcnt(N) only (expcnt / lgkmcnt left at their maxima), gfx9 encoding
template <int N>
SRA_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// With `in_flight` stages issued (the oldest is the one about to be computed) and L transfers per
// stage, wait until at most the newer stages' transfers are outstanding.
template <int L>
SRA_DEV void wait_stages(int in_flight) {
  if (in_flight >= 4) wait_vm<(3 * L < 63 ? 3 * L : 63)>();
  else if (in_flight == 3) wait_vm<2 * L>();
  else if (in_flight == 2) wait_vm<L>();
  else wait_vm<0>();
}

// In-kernel adapter rows (UG > 0): per stage, U^T[j][t] += G[j][c] Act[t][c] over the stage's 64
// columns for the 16-token fragments f = wave, wave + NW, ..., with dense v_mfma_f32_16x16x32_bf16
// (A = G rows j, lane: j = l%16, columns 8(l/16)..+7; B = tokens, lane: token l%16, same columns)
// from the stage's activation region `rows` (128-byte rows, chunk c of row x at (c ^ ((x>>1)&7))).
// Each stage's fp32 result is added to fp64 sums one stage later (so the wave never waits on these
// MFMAs), and U keeps full fp32 accuracy over long C.
template <int BT, int UG, int NW>
struct AdapterRows {
  static constexpr int NTF = BT / 16, NFW = (NTF + NW - 1) / NW, NJ = UG / 16;
  static constexpr int ULD = UG + 4;  // floats per token row of the U tile handed over in LDS
  double u[NFW][NJ][4];
  f32x4 d[NFW][NJ];  // the last stage's products, not yet in u
  SRA_DEV void zero() {
#pragma unroll
    for (int i = 0; i < NFW; ++i)
#pragma unroll
      for (int jf = 0; jf < NJ; ++jf) {
        d[i][jf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) u[i][jf][e] = 0.0;
      }
  }
  SRA_DEV void flush() {
#pragma unroll
    for (int i = 0; i < NFW; ++i)
#pragma unroll
      for (int jf = 0; jf < NJ; ++jf)
#pragma unroll
        for (int e = 0; e < 4; ++e) u[i][jf][e] += (double)d[i][jf][e];
  }
  bf16x8 tb0[NFW], tb1[NFW], g0[NJ], g1[NJ];  // the stage's operand fragments
  // fragment reads of one stage (issued together with the main product's reads)
  SRA_DEV void read(const uint8_t* rows, int wave, int lane) {
    const int q4 = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int i = 0; i < NFW; ++i) {
      const int f = min(wave + NW * i, NTF - 1);
      const int tk = f * 16 + l16, sw = (tk >> 1) & 7;
      tb0[i] = *reinterpret_cast<const bf16x8*>(rows + tk * 128 + ((q4 ^ sw) << 4));
      tb1[i] = *reinterpret_cast<const bf16x8*>(rows + tk * 128 + (((4 + q4) ^ sw) << 4));
    }
#pragma unroll
    for (int jf = 0; jf < NJ; ++jf) {
      const int gr = BT + jf * 16 + l16, sg = (gr >> 1) & 7;
      g0[jf] = *reinterpret_cast<const bf16x8*>(rows + gr * 128 + ((q4 ^ sg) << 4));
      g1[jf] = *reinterpret_cast<const bf16x8*>(rows + gr * 128 + (((4 + q4) ^ sg) << 4));
    }
  }
  SRA_DEV void mma(int wave) {
#pragma unroll
    for (int i = 0; i < NFW; ++i) {
      if (NTF % NW != 0 && wave + NW * i >= NTF) continue;
#pragma unroll
      for (int jf = 0; jf < NJ; ++jf) {
        const f32x4 x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g0[jf], tb0[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        d[i][jf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g1[jf], tb1[i], x, 0, 0, 0);
      }
    }
  }
  // U tile -> LDS ut[t][j] (fp32); the first row tile also writes U and its V^T parts out.
  SRA_DEV void hand_over(float* ut, int wave, int lane, bool first_row_tile, int64_t t0, int64_t T,
                         const sra::Epilogue& ep) const {
    const int q4 = lane >> 4, l16 = lane & 15;
    const bool u_vec = (ep.r & 3) == 0;
#pragma unroll
    for (int i = 0; i < NFW; ++i) {
      const int f = wave + NW * i;
      if (NTF % NW != 0 && f >= NTF) continue;
      const int tl = f * 16 + l16;
      const int64_t tg = t0 + tl;
#pragma unroll
      for (int jf = 0; jf < NJ; ++jf) {
        const int j = jf * 16 + 4 * q4;
        const f32x4 v = f32x4{(float)u[i][jf][0], (float)u[i][jf][1], (float)u[i][jf][2],
                              (float)u[i][jf][3]};
        *reinterpret_cast<f32x4*>(ut + tl * ULD + j) = v;
        if (!first_row_tile) continue;
        if (tg < T) {
          if (ep.u_out) {
            if (u_vec && j + 4 <= ep.r) {
              *reinterpret_cast<f32x4*>(ep.u_out + tg * ep.r + j) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (j + e < ep.r) ep.u_out[tg * ep.r + j + e] = v[e];
            }
          }
          if (ep.vt) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j + e < ep.r) write_vt4(ep.vt, ep.vt_rp, ep.vt_tp, j + e, tg, u[i][jf][e]);
          }
        } else if (ep.vt && tg < ep.vt_tp) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < ep.r)
#pragma unroll
              for (int p = 0; p < 4; ++p) ep.vt[((int64_t)p * ep.vt_rp + j + e) * ep.vt_tp + tg] = 0;
        }
      }
    }
  }
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

// ---------------------------------------------------------------------------------------------
// Pipelined variant on v_smfmac_f32_16x16x64_bf16, which moves stored (non-zero) work ~20% faster
// on gfx950 than the 32x32x32 form.  Same LDS ring, DMA transfers and swizzles as above; per
// 64-column stage one SMFMAC per (16 weight rows, 16 tokens) pair.  Lane l of an A fragment holds
// row l%16 and logical columns 16(l/16)..+15 (16 contiguous bytes = swizzled chunk l/16 of the
// row); its metadata is the (l/16)&1 half of word (l/16)/2.  Lane l of a B fragment holds token
// l%16 and columns 8(l/16)..+7 and 32+8(l/16)..+7 (chunks l/16 and 4 + l/16).  Accumulator lane l
// holds rows 4(l/16)..+3 of token l%16.
// MS > 0: metadata is not part of a stage but fetched in super-stages of MS stages (8 B per row per
// stage, so MS = 8 gives 64-byte runs instead of 8-byte ones, which LDS-DMA moves ~7x faster per
// byte; MS = 4 gives 32-byte runs in half the LDS) into a double buffer of its own, one
// super-stage ahead; needs C % 128 == 0, and a split of the reduction must start on an 8-stage
// boundary (the planner splits only the 256x256 tile, so).
// UG > 0: adapter rows in the activation region as in PTile (GT transfers over NW waves).
// DN: the weight is dense (rows of C bf16, 128 bytes per row and stage, no metadata) and the
// products are pairs of dense v_mfma_f32_16x16x32_bf16 -- the fixed fan-in layer's densified
// weight.
template <int FR, int FT, int WR, int WT, int NS, int MS = 0, int UG = 0, bool DN = false>
struct QTile {
  static_assert(!(DN && (MS || UG)), "dense weights have no metadata or adapter rows");
  static constexpr int NW = WR * WT;  // waves per workgroup: 4 or 8
  static constexpr int BR = 16 * FR * WR, BT = 16 * FT * WT;
  static constexpr int LA = BR / ((DN ? 8 : 16) * NW), LM = (MS || DN) ? 0 : BR / (32 * NW);
  static constexpr int LB = BT / (8 * NW);
  static constexpr int GT = UG / 8, GW = GT / NW, GX = GT % NW;
  static constexpr int L = LA + LM + LB + GW;  // waves >= GX
  static constexpr int L1 = L + (GX ? 1 : 0);  // waves < GX
  static constexpr int A_BYTES = BR * (DN ? 128 : 64), M_BYTES = (MS || DN) ? 0 : BR * 8;
  static constexpr int B_BYTES = (BT + UG) * 128;
  static constexpr int STAGE = A_BYTES + M_BYTES + B_BYTES;
  static constexpr int MSB = MS ? BR * MS * 8 : 0;            // one metadata super-stage buffer
  static constexpr int LMS = MS ? MSB / (1024 * NW) : 0;      // its 1 KB transfers per wave
  static constexpr int LDS = NS * STAGE + 2 * MSB;
  static constexpr int OCC = (NW == 8 || FR * FT >= 32 || 2 * LDS > 160 * 1024) ? 1 : 2;
};

// TLAY: the weight is in the streaming 2:4 layout (1 KB blocks per 16-row group and 64-column stage,
// metadata in 1 KB blocks per 16-row group and 512 columns; see decode24.hip), so every transfer of
// the values reads 1 KB contiguously instead of 64-byte runs per row, and a super-stage of
// metadata reads 64-byte (MS = 8) or 32-byte (MS = 4) pieces of those blocks.  Same LDS layout and
// products; needs MS > 0.
template <int FR, int FT, int WR, int WT, int NS, int MS = 0, int UG = 0, bool DN = false, bool TLAY = false,
          bool PP = false>
__global__ __launch_bounds__(64 * WR * WT, (QTile<FR, FT, WR, WT, NS, MS, UG, DN>::OCC)) void k_spmm24_q(
    const uint16_t* __restrict__ s_vals, const uint32_t* __restrict__ s_meta, int64_t R, int64_t C,
    const uint16_t* __restrict__ act, int64_t T, sra::Epilogue ep, uint16_t* __restrict__ out,
    float* __restrict__ part, int n_rt, int n_tt, int stages_per_split, int n_whole) {
  using TL = QTile<FR, FT, WR, WT, NS, MS, UG, DN>;
  constexpr int BR = TL::BR, BT = TL::BT, L = TL::L;
  constexpr int NW = TL::NW;
  using AD = AdapterRows<BT, (UG > 0 ? UG : 16), NW>;
  static_assert(!TLAY || (MS > 0 && !DN), "the streaming layout is read with metadata super-stages");
  static_assert(UG == 0 || AD::ULD * 4 * BT <= TL::LDS, "U tile fits in LDS");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(BR % (16 * NW) == 0 && (MS || DN || BR % (32 * NW) == 0) && BT % (8 * NW) == 0,
                "transfer counts must be whole per wave");
  static_assert(MS == 0 || ((MS == 8 || MS == 4) && TL::MSB % (1024 * NW) == 0),
                "metadata super-stages of 4 or 8");
  static_assert(!PP || (NW == 8 && MS > 0 && UG == 0 && !DN), "ping-pong: eight waves, super-stages");
  __shared__ __attribute__((aligned(16))) uint8_t smem[TL::LDS];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q4 = lane >> 4, l16 = lane & 15;
  // n_whole < 0: blockIdx.x is the tile, blockIdx.y the split of the reduction.  n_whole >= 0
  // (tail split): the first n_whole workgroups run whole tiles and store bf16; each remaining
  // tile is split in two (workgroups n_whole + 2i + z) into fp32 partials.
  int rt, tt, z = blockIdx.y;
  float* part_w = part;  // where this workgroup's partial goes (nullptr: the output itself)
  bool whole = false;
  if (n_whole < 0) {
    tile_coords(xcd_remap(blockIdx.x, n_rt * n_tt), n_rt, n_tt, rt, tt);
  } else if ((int)blockIdx.x < n_whole) {
    tile_coords(xcd_remap(blockIdx.x, n_whole), n_rt, n_tt, rt, tt);
    z = 0;
    part_w = nullptr;
    whole = true;
  } else {
    const int k = (int)blockIdx.x - n_whole;
    tile_coords(n_whole + (k >> 1), n_rt, n_tt, rt, tt);
    z = k & 1;
  }
  const int64_t row0 = (int64_t)rt * BR, t0 = (int64_t)tt * BT;
  const int64_t cv = C / 2, cm = C / 32;
  const int nC_all = (int)(C / BC);
  const int c_beg = z * stages_per_split;
  const int c_end = whole ? nC_all : min(nC_all, c_beg + stages_per_split);

  // operands through buffer resources based at the tile (fixed lane offsets, the stage offset in
  // an SGPR; rows past R, T or r read as zeros), as in k_spmm24_pipe
  const int rows_here = (int)min((int64_t)BR, R - row0), toks_here = (int)min((int64_t)BT, T - t0);
  constexpr int A_ROW = TLAY ? 1024 : DN ? 128 : 64;  // stage offset of the weight operand (bytes)
  // streaming layout: 16-row groups of nsteps 1 KB value blocks and nbat 1 KB metadata blocks
  const int nsteps = (int)((C + 63) / 64), nbat = (int)((C + 511) / 512), ngrp = (rows_here + 15) / 16;
  const __amdgpu_buffer_rsrc_t ra =
      TLAY ? __builtin_amdgcn_make_buffer_rsrc((void*)(s_vals + (row0 / 16) * nsteps * 512), 0,
                                               ngrp * nsteps * 1024, 0x00020000)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(s_vals + row0 * (DN ? C : cv)), 0,
                                               rows_here * (int)C * (DN ? 2 : 1), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      TLAY ? __builtin_amdgcn_make_buffer_rsrc((void*)(s_meta + (row0 / 16) * nbat * 256), 0,
                                               ngrp * nbat * 1024, 0x00020000)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(DN ? nullptr : s_meta + row0 * cm), 0,
                                               DN ? 0 : rows_here * (int)cm * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(act + t0 * C), 0, toks_here * (int)C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ep.G, 0, UG > 0 ? ep.r * (int)ep.g_ld * 2 : 0, 0x00020000);
  uint32_t a_off[TL::LA];
  int a_dst[TL::LA];
#pragma unroll
  for (int k = 0; k < TL::LA; ++k) {
    const int b = k * NW + wave;
    if constexpr (DN) {  // 8 rows of 128 bytes, chunk swizzle (row >> 1) & 7 as for tokens
      const int row = 8 * b + (lane >> 3), ch = (lane & 7) ^ ((row >> 1) & 7);
      a_off[k] = (uint32_t)((row * C + ch * 8) * 2);
    } else {             // 16 rows of 64 bytes
      const int row = 16 * b + (lane >> 2), ch = (lane & 3) ^ ((row >> 2) & 3);
      // streaming layout: chunk ch of row i of group b sits at (16 ch + i) * 16 in its block
      a_off[k] = TLAY ? (uint32_t)(b * nsteps * 1024 + (16 * ch + (lane >> 2)) * 16)
                      : (uint32_t)(row * C + ch * 16);
    }
    a_dst[k] = b * 1024;
  }
  uint32_t m_off[TL::LM ? TL::LM : 1];
  int m_dst[TL::LM ? TL::LM : 1];
#pragma unroll
  for (int k = 0; k < TL::LM; ++k) {
    const int b = k * NW + wave, row = 32 * b + (lane >> 1);
    m_off[k] = (uint32_t)((row * cm + (lane & 1)) * 4);
    m_dst[k] = TL::A_BYTES + b * 256;
  }
  // super-stage metadata: row r holds MS*8 bytes, 16-byte chunk ch = stages 2ch and 2ch+1 of the
  // super-stage, stored in slot ch ^ ms_swz(r); a 1 KB transfer b covers 16 rows (MS = 8, lane:
  // row lane/4, slot lane%4) or 32 rows (MS = 4, lane: row lane/2, slot lane%2)
  // slot swizzle of a super-stage row: the 16 rows of a fragment's 4-byte reads spread over the banks
  auto ms_swz = [](int r) { return MS == 4 ? (r >> 2) & 1 : (r >> 2) & 3; };
  uint32_t ms_row[TL::LMS ? TL::LMS : 1];
  int ms_ch[TL::LMS ? TL::LMS : 1], ms_dst[TL::LMS ? TL::LMS : 1];
#pragma unroll
  for (int k = 0; k < TL::LMS; ++k) {
    constexpr int SL = MS / 2;  // 16-byte slots per row
    const int b = k * NW + wave, row = (1024 / (8 * MS)) * b + lane / SL, pos = lane % SL;
    ms_ch[k] = pos ^ ms_swz(row);
    ms_row[k] = (uint32_t)row;
    ms_dst[k] = b * 1024;
  }
  uint8_t* const msbuf = smem + NS * TL::STAGE;
  auto issue_meta = [&](int g) {
    uint8_t* base = msbuf + (g & 1) * TL::MSB;
#pragma unroll
    for (int k = 0; k < TL::LMS; ++k) {
      if constexpr (TLAY) {
        // super-stage g covers columns 64 (c_beg + MS g) ..: block (row / 16, that / 512), row
        // (row % 16)'s 64 bytes at 64 (row % 16), this super-stage's MS*8 of them from 8 MS (g % (8/MS));
        // a split starts on a 512-column batch (c_beg % 8 == 0)
        const int row = (int)ms_row[k];
        bdma(rm, base + ms_dst[k], 16,
             (uint32_t)((row >> 4) * nbat * 1024 + 64 * (row & 15) + 16 * ms_ch[k]),
             (c_beg / 8 + g / (8 / MS)) * 1024 + 8 * MS * (g % (8 / MS)));
      } else {
        int w = 2 * (c_beg + MS * g) + 4 * ms_ch[k];  // two words per stage
        if (w > (int)cm - 4) w = (int)cm - 4;  // past the row's end: clamped, never read
        bdma(rm, base + ms_dst[k], 16, ms_row[k] * (uint32_t)cm * 4 + (uint32_t)w * 4, 0);
      }
    }
  };
  uint32_t b_off[TL::LB];
  int b_dst[TL::LB];
#pragma unroll
  for (int k = 0; k < TL::LB; ++k) {
    const int b = k * NW + wave, tk = 8 * b + (lane >> 3), pos = lane & 7;
    const int ch = pos ^ ((tk >> 1) & 7);
    b_off[k] = (uint32_t)((tk * C + ch * 8) * 2);
    b_dst[k] = TL::A_BYTES + TL::M_BYTES + b * 1024;
  }
  constexpr int NG = TL::GW + (TL::GX ? 1 : 0);
  uint32_t g_off[NG ? NG : 1];
  int g_dst[NG ? NG : 1];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int b = k * NW + wave, tk = BT + 8 * b + (lane >> 3), pos = lane & 7;
    const int ch = pos ^ ((tk >> 1) & 7);
    g_off[k] = (uint32_t)(((tk - BT) * ep.g_ld + ch * 8) * 2);
    g_dst[k] = TL::A_BYTES + TL::M_BYTES + (BT / 8 + b) * 1024;
  }
  auto issue = [&](int c, int buf) {
    uint8_t* base = smem + buf * TL::STAGE;
#pragma unroll
    for (int k = 0; k < TL::LA; ++k) bdma(ra, base + a_dst[k], 16, a_off[k], c * A_ROW);
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

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wr = wave / WT, wt = wave % WT;
  auto compute = [&](int buf, int rel) {
    const uint8_t* A = smem + buf * TL::STAGE;
    const uint32_t* M = reinterpret_cast<const uint32_t*>(A + TL::A_BYTES);
    const uint8_t* MS_buf = msbuf + (MS ? ((rel / (MS ? MS : 1)) & 1) * TL::MSB : 0);
    const int u = MS ? rel % (MS ? MS : 1) : 0;
    const uint8_t* B = A + TL::A_BYTES + TL::M_BYTES;
    if constexpr (UG > 0) ad.flush();
    bf16x16 bfr[FT];
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int tk = wt * 16 * FT + j * 16 + l16, sw = (tk >> 1) & 7;
      const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 128 + ((q4 ^ sw) << 4));
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 + q4) ^ sw) << 4));
      bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
    if constexpr (DN) {
      // dense weight rows: columns 8(l/16)..+7 and 32+8(l/16)..+7 of the stage, one dense MFMA each
      bf16x8 alo[FR], ahi[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 16 * FR + i * 16 + l16, sw = (r >> 1) & 7;
        alo[i] = *reinterpret_cast<const bf16x8*>(A + r * 128 + ((q4 ^ sw) << 4));
        ahi[i] = *reinterpret_cast<const bf16x8*>(A + r * 128 + (((4 + q4) ^ sw) << 4));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          const bf16x8 blo = __builtin_shufflevector(bfr[j], bfr[j], 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 bhi = __builtin_shufflevector(bfr[j], bfr[j], 8, 9, 10, 11, 12, 13, 14, 15);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[i], blo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[i], bhi, acc[i][j], 0, 0, 0);
        }
      return;
    }
    bf16x8 af[FR];
    uint32_t mword[FR];
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int r = wr * 16 * FR + i * 16 + l16;
      af[i] = *reinterpret_cast<const bf16x8*>(A + r * 64 + ((q4 ^ ((r >> 2) & 3)) << 4));
      if constexpr (MS > 0) {
        const int chunk = (u >> 1) ^ ms_swz(r);
        mword[i] = *reinterpret_cast<const uint32_t*>(MS_buf + r * (MS * 8) + (chunk << 4) +
                                                      4 * (2 * (u & 1) + (q4 >> 1)));
      } else {
        mword[i] = M[r * 2 + (q4 >> 1)];
      }
    }
    if constexpr (UG > 0) ad.read(B, wave, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
    if constexpr (UG > 0) ad.mma(wave);
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int idx = (int)(mword[i] >> (16 * (q4 & 1)));
#pragma unroll
      for (int j = 0; j < FT; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[i], bfr[j], acc[i][j], idx, 0, 0);
    }
  };

  constexpr int D = NS - 1;
  if constexpr (PP) {
    // Ping-pong: waves 0-3 and 4-7 (one of each per SIMD) run the same read / multiply sequence
    // half a stage apart: the late group passes one extra barrier first (and the early group one
    // at the end), so between two workgroup barriers one group reads fragments from LDS while the
    // other runs the SMFMACs on the fragments it read in the previous phase, and each SIMD's
    // matrix core and the LDS work at once instead of in turn.  Barriers k -> k+1: early reads
    // stage c at k = 2(c - c_beg), multiplies it at k + 1; late reads it at k + 1, multiplies at
    // k + 2.  Stage c+1 must be visible at barrier 2(c - c_beg) + 2, so each wave waits for its own
    // transfers of it before that barrier (the late group's is the one after its read phase).  A
    // stage's buffer is free once the late group's read phase ends (reads drained by lgkmcnt(0)),
    // so each group issues stage c + D into the buffer of stage c-1 as it starts stage c.
    struct Frags {
      bf16x16 b[FT];
      bf16x8 a[FR];
      uint32_t m[FR];
    };
    auto pp_read = [&](int buf, int rel, Frags& f) {
      const uint8_t* A = smem + buf * TL::STAGE;
      const uint8_t* B = A + TL::A_BYTES;
      const uint8_t* MS_buf = msbuf + ((rel / MS) & 1) * TL::MSB;
      const int u = rel % MS;
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tk = wt * 16 * FT + j * 16 + l16, sw = (tk >> 1) & 7;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 128 + ((q4 ^ sw) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 + q4) ^ sw) << 4));
        f.b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 16 * FR + i * 16 + l16;
        f.a[i] = *reinterpret_cast<const bf16x8*>(A + r * 64 + ((q4 ^ ((r >> 2) & 3)) << 4));
        const int chunk = (u >> 1) ^ ms_swz(r);
        f.m[i] = *reinterpret_cast<const uint32_t*>(MS_buf + r * (MS * 8) + (chunk << 4) +
                                                    4 * (2 * (u & 1) + (q4 >> 1)));
      }
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0): the reads are done
    };
    auto pp_mma = [&](const Frags& f) {
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int idx = (int)(f.m[i] >> (16 * (q4 & 1)));
#pragma unroll
        for (int j = 0; j < FT; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(f.a[i], f.b[j], acc[i][j], idx, 0, 0);
      }
    };
    const bool late = wave >= NW / 2;
    Frags f;
    if (c_beg < c_end) issue_meta(0);
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (c_beg + d < c_end) issue(c_beg + d, d);
    wait_stages<L>(min(D, c_end - c_beg));
    ring_barrier();  // stage c_beg visible
    if (late) ring_barrier();
    for (int c = c_beg; c < c_end; ++c) {
      const int rel = c - c_beg;
      if (rel % MS == 0 && c + MS < c_end) issue_meta(rel / MS + 1);
      if (c + D < c_end) issue(c + D, (rel + D) % NS);
      pp_read(rel % NS, rel, f);
      if (late && c + 1 < c_end) wait_stages<L>(min(D, c_end - (c + 1)));
      ring_barrier();
      pp_mma(f);
      if (!late && c + 1 < c_end) wait_stages<L>(min(D, c_end - (c + 1)));
      ring_barrier();
    }
    if (!late) ring_barrier();
  } else {
  if constexpr (MS > 0) {
    if (c_beg < c_end) issue_meta(0);
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (c_beg + d < c_end) issue(c_beg + d, d);
  // waiting for at most (in_flight-1)*L outstanding transfers completes stage c and every older
  // one, including the metadata of stage c's super-stage (issued before stage c's own loads).
  // Steady state unrolled by the ring depth: constant buffer indices, D stages in flight (not for
  // the largest wave tiles, whose registers are spoken for).
  constexpr bool kUnroll = FR * FT < 32;
  int c = c_beg;
  for (; kUnroll && c + NS + D <= c_end; c += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (TL::GX && wave < TL::GX) wait_vm<((D - 1) * TL::L1 < 63 ? (D - 1) * TL::L1 : 63)>();
      else wait_vm<((D - 1) * L < 63 ? (D - 1) * L : 63)>();
      ring_barrier();
      const int rel = c + u - c_beg;
      if constexpr (MS > 0) {
        if (rel % MS == 0 && c + u + MS < c_end) issue_meta(rel / MS + 1);
      }
      issue(c + u + D, (u + D) % NS);
      compute(u, rel);
    }
  }
  for (; c < c_end; ++c) {
    const int in_flight = min(D, c_end - c);
    if (TL::GX && wave < TL::GX) wait_stages<TL::L1>(in_flight);
    else wait_stages<L>(in_flight);
    ring_barrier();
    const int rel = c - c_beg;
    if constexpr (MS > 0) {
      if (rel % MS == 0 && c + MS < c_end) issue_meta(rel / MS + 1);
    }
    if (c + D < c_end) issue(c + D, (rel + D) % NS);
    compute(rel % NS, rel);
  }
  }
  if constexpr (UG > 0) ad.flush();

  // ---- in-kernel U: hand the tile over through LDS (and write U / V^T from the first row tile)
  float* const ut = reinterpret_cast<float*>(smem);
  if constexpr (UG > 0) {
    __syncthreads();  // every wave is done with the operand ring
    ad.hand_over(ut, wave, lane, rt == 0, t0, T, ep);
    __syncthreads();
  }

  // ---- fused low-rank epilogue (first split only), dense v_mfma_f32_16x16x32_bf16:
  //      A operand = E rows (lane: row l%16, j = 8(l/16)..+7), B operand = U^T (token l%16)
  // With U from memory, the tile's U rows go through LDS once per 128 adapter columns (LDS-DMA
  // when r % 4 == 0, no registers held), so each U element crosses from L2 once per workgroup
  // and all of a block's transfers are in flight together, instead of every wave reading its
  // tokens' U in four dependent rounds per block (the WR waves of one token column read the same
  // rows).  Staged fp32 rows of 512 bytes, 16-byte chunk c of token t at slot c ^ (t % 32) so the
  // 16 tokens of a fragment read spread over the banks; each wave splits its fragments into bf16
  // hi + lo itself.
  constexpr bool kStageU = UG == 0 && BT * 512 <= TL::LDS && BT % (2 * NW) == 0;
  if constexpr (kStageU) {
  if (ep.r > 0 && z == 0) {
    // E rows are contiguous in j (e_j_stride == 1, checked by the launchers): one 16-byte load
    // per fragment (eight 2-byte ones when rows are not 16-byte aligned) through a resource over
    // E's rows R, so rows past R read as zero; entries past r (the next row's, or padding) are
    // cleared after the load.
    const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ep.E, 0, (int)(R * ep.e_row_stride * 2), 0x00020000);
    const bool e_al = (ep.e_row_stride & 7) == 0;  // 16-byte aligned fragments
    auto load_e = [&](int64_t row, int j0) {
      union { u32x4 v; uint16_t h[8]; } x;
      const uint32_t off = (uint32_t)((row * ep.e_row_stride + j0) * 2);
      if (e_al) {
        x.v = __builtin_amdgcn_raw_buffer_load_b128(re, off, 0, 0);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) x.h[q] = __builtin_amdgcn_raw_buffer_load_b16(re, off + 2 * q, 0, 0);
      }
      if (j0 + 8 > ep.r) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (j0 + q >= ep.r) x.h[q] = 0;
      }
      return x.v;
    };
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ep.U + t0 * ep.r), 0, toks_here * ep.r * 4, 0x00020000);
    for (int jb0 = 0; jb0 < ep.r; jb0 += 128) {
      __syncthreads();  // the operand ring (or the previous block's U) is no longer read
      if ((ep.r & 3) == 0) {
#pragma unroll
        for (int k = 0; k < BT / (2 * NW); ++k) {  // 1 KB = two token rows per transfer
          const int b = k * NW + wave, tok = 2 * b + (lane >> 5), c = (lane & 31) ^ (tok & 31);
          const int j = jb0 + 4 * c;
          bdma(ru, smem + b * 1024, 16, j < ep.r ? (uint32_t)((tok * ep.r + j) * 4) : 0x80000000u, 0);
        }
      } else {  // U rows not 16-byte aligned: 4-byte transfers, 64 floats (256 B) each
#pragma unroll 1
        for (int k = 0; k < 2 * BT / NW; ++k) {
          const int b = k * NW + wave, f = 64 * b + lane, tok = f >> 7, p = f & 127;
          const int j = jb0 + 4 * ((p >> 2) ^ (tok & 31)) + (p & 3);
          bdma(ru, smem + b * 256, 4, j < ep.r ? (uint32_t)((tok * ep.r + j) * 4) : 0x80000000u, 0);
        }
      }
      wait_vm<0>();
      __syncthreads();
      const int nj = min(128, ep.r - jb0);
      for (int jj = 0; jj < nj; jj += 32) {
        const int c0 = (jj + 8 * q4) >> 2;
        union { u32x4 v; bf16x8 b; } e[FR];
#pragma unroll
        for (int i = 0; i < FR; ++i) e[i].v = load_e(row0 + wr * 16 * FR + i * 16 + l16, jb0 + jj + 8 * q4);
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          const int tl = wt * 16 * FT + j * 16 + l16, sw = tl & 31;
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(smem + tl * 512 + 16 * (c0 ^ sw));
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(smem + tl * 512 + 16 * ((c0 + 1) ^ sw));
          union { uint16_t h[8]; bf16x8 b; } uhi, ulo;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            split_bf16(u0[q], uhi.h[q], ulo.h[q]);
            split_bf16(u1[q], uhi.h[4 + q], ulo.h[4 + q]);
          }
#pragma unroll
          for (int i = 0; i < FR; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e[i].b, uhi.b, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e[i].b, ulo.b, acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }
  } else {
  if (ep.r > 0 && z == 0) {
    const bool e_vec = ep.e_j_stride == 1 && (ep.r & 7) == 0;
    const bool u_vec = (ep.r & 7) == 0;
    for (int jj = 0; jj < ep.r; jj += 32) {
      const int jb = jj + 8 * q4;
      union UH { uint16_t h[8]; bf16x8 b; };
      UH uhi[FT], ulo[FT];
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tl = wt * 16 * FT + j * 16 + l16;
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
#pragma unroll
        for (int q = 0; q < 8; ++q) split_bf16(u[q], uhi[j].h[q], ulo[j].h[q]);
      }
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int64_t row = row0 + wr * 16 * FR + i * 16 + l16;
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
        const bf16x8 e = x.b;
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e, uhi[j].b, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e, ulo[j].b, acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  }

  // ---- store: lane holds rows 4(l/16)..+3 of token l%16
  using OB = OutStage<BR, false>;
  using OP = OutStage<BR, true>;
  constexpr bool stage_bf16 = OB::template bytes<BT>() <= TL::LDS;
  constexpr bool stage_f32 = OP::template bytes<BT>() <= TL::LDS;
  if ((part_w && stage_f32) || (!part_w && stage_bf16)) {
    __syncthreads();  // every wave is done with the operand ring
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tok = wt * 16 * FT + j * 16 + l16, row = wr * 16 * FR + i * 16 + 4 * q4;
        const f32x4& c = acc[i][j];
        if (part_w) OP::put(smem, tok, row, c[0], c[1], c[2], c[3]);
        else OB::put(smem, tok, row, c[0], c[1], c[2], c[3]);
      }
    __syncthreads();
    if (part_w) OP::template flush<BT>(smem, part_w + (int64_t)z * T * R, row0, t0, R, T);
    else OB::template flush<BT>(smem, out, row0, t0, R, T);
    return;
  }
  const bool r4 = (R & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int64_t t = t0 + wt * 16 * FT + j * 16 + l16;
      if (t >= T) continue;
      const int64_t rb = row0 + wr * 16 * FR + i * 16 + 4 * q4;
      if (part_w) {
        float* o = part_w + ((int64_t)z * T + t) * R + rb;
        if (r4 && rb + 3 < R) {
          *reinterpret_cast<f32x4*>(o) = acc[i][j];
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (rb + b < R) o[b] = acc[i][j][b];
        }
        continue;
      }
      uint16_t* o = out + t * R + rb;
      if (r4 && rb + 3 < R) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        v[1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(o) = v;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (rb + b < R) o[b] = f32_to_bf16(acc[i][j][b]);
      }
    }
}

// Wide-stage variant (C % 128 == 0) on v_smfmac_f32_16x16x64_bf16.  Global -> LDS transfer
// throughput of LDS-DMA on gfx950 depends on the length of the contiguous run each row
// contributes: 128-byte runs move ~1.6x more per second than 64-byte runs and ~12x more than the
// 8-byte metadata runs of a 64-column stage.  So a stage here is 128 logical columns (128 B of
// stored values per weight row, 256 B per token) and metadata is fetched in super-stages of MS
// stages (16 B per row per stage, MS*16-byte runs) into a double buffer of its own, one super-stage
// ahead.  Swizzles: value rows chunk ^ (row & 7) (8 chunks of 16 B), token rows chunk ^ (t & 15)
// (16 chunks), metadata rows chunk ^ ((row >> 2) & 3) (MS = 4 chunks); each keeps the 16 lanes of
// a fragment read on distinct banks.  Operand lane layouts are the 16x16x64 ones above.
template <int FR, int FT, int NS, int MS>
struct WTile {
  static constexpr int WR = 2, WT = 2;
  static constexpr int BR = 16 * FR * WR, BT = 16 * FT * WT;
  static constexpr int LA = BR / 32, LB = BT / 16;    // 1 KB transfers per wave per stage
  static constexpr int LM = BR * MS * 16 / 4096;      // per wave per super-stage
  static constexpr int L = LA + LB;
  static constexpr int A_BYTES = BR * 128, B_BYTES = BT * 256, STAGE = A_BYTES + B_BYTES;
  static constexpr int M_BYTES = BR * MS * 16;        // one metadata buffer
  static constexpr int LDS = NS * STAGE + 2 * M_BYTES;
};
constexpr int BCW = 128;  // logical columns per wide stage

template <int FR, int FT, int NS, int MS>
__global__ __launch_bounds__(256, 1) void k_spmm24_w(
    const uint16_t* __restrict__ s_vals, const uint32_t* __restrict__ s_meta, int64_t R, int64_t C,
    const uint16_t* __restrict__ act, int64_t T, sra::Epilogue ep, uint16_t* __restrict__ out,
    float* __restrict__ part, int n_rt, int n_tt, int stages_per_split) {
  using TL = WTile<FR, FT, NS, MS>;
  constexpr int BR = TL::BR, BT = TL::BT, L = TL::L, WT = TL::WT, NW = 4;
  static_assert(MS == 4, "metadata chunk swizzle assumes 4 chunks per row");
  static_assert(TL::LDS <= 160 * 1024, "LDS");
  static_assert((BR * MS * 16) % 4096 == 0, "metadata transfers must be whole per wave");
  __shared__ __attribute__((aligned(16))) uint8_t smem[TL::LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, q4 = lane >> 4, l16 = lane & 15;
  int rt, tt;
  tile_coords(xcd_remap(blockIdx.x, n_rt * n_tt), n_rt, n_tt, rt, tt);
  const int64_t row0 = (int64_t)rt * BR, t0 = (int64_t)tt * BT;
  const int64_t cv = C / 2, cm = C / 32;
  const int nC_all = (int)(C / BCW);
  const int z = blockIdx.y;
  const int c_beg = z * stages_per_split;
  const int c_end = min(nC_all, c_beg + stages_per_split);

  // values: 1 KB block b = 8 rows x 128 B; lane -> row 8b + lane/8, slot lane%8 holds chunk slot^(row&7)
  const uint16_t* a_src[TL::LA];
  int a_dst[TL::LA];
#pragma unroll
  for (int k = 0; k < TL::LA; ++k) {
    const int b = k * NW + wave, row = 8 * b + (lane >> 3), pos = lane & 7;
    const int ch = pos ^ (row & 7);
    const int64_t grow = min(row0 + row, R - 1);
    a_src[k] = s_vals + grow * cv + ch * 8;
    a_dst[k] = b * 1024;
  }
  // tokens: 1 KB block b = 4 tokens x 256 B; slot lane%16 holds chunk slot^(t&15)
  const uint16_t* b_src[TL::LB];
  int b_dst[TL::LB];
#pragma unroll
  for (int k = 0; k < TL::LB; ++k) {
    const int b = k * NW + wave, tk = 4 * b + (lane >> 4), pos = lane & 15;
    const int ch = pos ^ (tk & 15);
    const int64_t gt = min(t0 + tk, T - 1);
    b_src[k] = act + gt * C + ch * 8;
    b_dst[k] = TL::A_BYTES + b * 1024;
  }
  // metadata: 1 KB block b = 16 rows x 64 B (4 stages of 16 B); slot lane%4 holds chunk
  // slot^((row>>2)&3); chunk = stage within the super-stage
  const uint32_t* m_row[TL::LM];
  int m_ch[TL::LM], m_dst[TL::LM];
#pragma unroll
  for (int k = 0; k < TL::LM; ++k) {
    const int b = k * NW + wave, row = 16 * b + (lane >> 2), pos = lane & 3;
    m_ch[k] = pos ^ ((row >> 2) & 3);
    const int64_t grow = min(row0 + row, R - 1);
    m_row[k] = s_meta + grow * cm;
    m_dst[k] = b * 1024;
  }
  uint8_t* const mbuf = smem + NS * TL::STAGE;
  auto issue = [&](int c, int buf) {
    uint8_t* base = smem + buf * TL::STAGE;
#pragma unroll
    for (int k = 0; k < TL::LA; ++k) dma16(a_src[k] + (int64_t)c * 64, base + a_dst[k]);
#pragma unroll
    for (int k = 0; k < TL::LB; ++k) dma16(b_src[k] + (int64_t)c * BCW, base + b_dst[k]);
  };
  // super-stage g covers stages c_beg + MS*g .. +MS-1; 4 metadata words per stage.  Words past
  // the row end (a partial last super-stage) are clamped to the row's last 16 bytes and unused.
  auto issue_meta = [&](int g) {
    uint8_t* base = mbuf + (g & 1) * TL::M_BYTES;
#pragma unroll
    for (int k = 0; k < TL::LM; ++k) {
      int64_t w = 4 * ((int64_t)c_beg + MS * g + m_ch[k]);
      if (w > cm - 4) w = cm - 4;
      dma16(m_row[k] + w, base + m_dst[k]);
    }
  };

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wr = wave / WT, wt = wave % WT;
  auto compute = [&](int buf, int c) {
    const uint8_t* A = smem + buf * TL::STAGE;
    const uint8_t* B = A + TL::A_BYTES;
    const int u = (c - c_beg) % MS;
    const uint32_t* M = reinterpret_cast<const uint32_t*>(mbuf + (((c - c_beg) / MS) & 1) * TL::M_BYTES);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x16 bfr[FT];
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tk = wt * 16 * FT + j * 16 + l16, sw = tk & 15;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 256 + (((8 * s + q4) ^ sw) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 256 + (((8 * s + 4 + q4) ^ sw) << 4));
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 16 * FR + i * 16 + l16;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(A + r * 128 + (((4 * s + q4) ^ (r & 7)) << 4));
        const int word = ((u ^ ((r >> 2) & 3)) << 2) + 2 * s + (q4 >> 1);
        const int idx = (int)(M[r * (MS * 4) + word] >> (16 * (q4 & 1)));
#pragma unroll
        for (int j = 0; j < FT; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af, bfr[j], acc[i][j], idx, 0, 0);
      }
    }
  };

  constexpr int D = NS - 1;
  if (c_beg < c_end) issue_meta(0);
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (c_beg + d < c_end) issue(c_beg + d, d);
  for (int c = c_beg; c < c_end; ++c) {
    // stages c .. c+in_flight-1 and every earlier transfer (metadata included) are issued; waiting
    // for at most (in_flight-1)*L outstanding completes stage c and all older metadata
    const int in_flight = min(D, c_end - c);
    if (in_flight >= 3) wait_vm<(2 * L < 63 ? 2 * L : 63)>();
    else if (in_flight == 2) wait_vm<L>();
    else wait_vm<0>();
    ring_barrier();  // stage c visible; stage c-1 and its super-stage reads done
    const int rel = c - c_beg;
    if (rel % MS == 0 && c + MS < c_end) issue_meta(rel / MS + 1);
    if (c + D < c_end) issue(c + D, (rel + D) % NS);
    compute(rel % NS, c);
  }

  // ---- fused low-rank epilogue (first split only), dense v_mfma_f32_16x16x32_bf16:
  //      A operand = E rows (lane: row l%16, j = 8(l/16)..+7), B operand = U^T (token l%16)
  if (ep.r > 0 && z == 0) {
    const bool e_vec = ep.e_j_stride == 1 && (ep.r & 7) == 0;
    const bool u_vec = (ep.r & 7) == 0;
    for (int jj = 0; jj < ep.r; jj += 32) {
      const int jb = jj + 8 * q4;
      union UH { uint16_t h[8]; bf16x8 b; };
      UH uhi[FT], ulo[FT];
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int64_t t = t0 + wt * 16 * FT + j * 16 + l16;
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
#pragma unroll
        for (int q = 0; q < 8; ++q) split_bf16(u[q], uhi[j].h[q], ulo[j].h[q]);
      }
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int64_t row = row0 + wr * 16 * FR + i * 16 + l16;
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
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.b, uhi[j].b, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.b, ulo[j].b, acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // ---- store: lane holds rows 4(l/16)..+3 of token l%16
  using OB = OutStage<BR, false>;
  using OP = OutStage<BR, true>;
  constexpr bool stage_bf16 = OB::template bytes<BT>() <= TL::LDS;
  constexpr bool stage_f32 = OP::template bytes<BT>() <= TL::LDS;
  if ((part && stage_f32) || (!part && stage_bf16)) {
    __syncthreads();  // every wave is done with the operand ring
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tok = wt * 16 * FT + j * 16 + l16, row = wr * 16 * FR + i * 16 + 4 * q4;
        const f32x4& c = acc[i][j];
        if (part) OP::put(smem, tok, row, c[0], c[1], c[2], c[3]);
        else OB::put(smem, tok, row, c[0], c[1], c[2], c[3]);
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
      const int64_t t = t0 + wt * 16 * FT + j * 16 + l16;
      if (t >= T) continue;
      const int64_t rb = row0 + wr * 16 * FR + i * 16 + 4 * q4;
      if (part) {
        float* o = part + ((int64_t)z * T + t) * R + rb;
        if (r4 && rb + 3 < R) {
          *reinterpret_cast<f32x4*>(o) = acc[i][j];
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (rb + b < R) o[b] = acc[i][j][b];
        }
        continue;
      }
      uint16_t* o = out + t * R + rb;
      if (r4 && rb + 3 < R) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        v[1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(o) = v;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (rb + b < R) o[b] = f32_to_bf16(acc[i][j][b]);
      }
    }
}

// Fixed-order sum of the S fp32 partials, rounded once to bf16.
// The two fp32 partials of each tail-split tile (tiles n_whole .. of a BR x BT tiling, in the
// SpMM's tile order) summed in split order and stored as bf16: gridDim.y workgroups per tile,
// each over its share of the tile's tokens.
__global__ void k_tail_reduce(const float* __restrict__ part, int64_t T, int64_t R, int n_whole,
                              int n_rt, int n_tt, int BR, int BT, uint16_t* __restrict__ out) {
  int rt, tt;
  tile_coords(n_whole + (int)blockIdx.x, n_rt, n_tt, rt, tt);
  const int64_t row0 = (int64_t)rt * BR, t0 = (int64_t)tt * BT, n = T * R;
  const bool vec = (R & 3) == 0;
  const int tpw = BT / (int)gridDim.y;  // tokens per workgroup
  for (int v = threadIdx.x; v < tpw * (BR / 4); v += blockDim.x) {
    const int tok = (int)blockIdx.y * tpw + v / (BR / 4), c = v % (BR / 4);
    const int64_t t = t0 + tok, row = row0 + 4 * c;
    if (t >= T || row >= R) continue;
    const int64_t i = t * R + row;
    if (vec && row + 4 <= R) {
      const f32x4 s = *reinterpret_cast<const f32x4*>(part + i) + *reinterpret_cast<const f32x4*>(part + n + i);
      u32x2 o;
      o[0] = pack_bf16x2(s[0], s[1]);
      o[1] = pack_bf16x2(s[2], s[3]);
      *reinterpret_cast<u32x2*>(out + i) = o;
    } else {
      for (int e = 0; e < 4 && row + e < R; ++e) out[i + e] = f32_to_bf16(part[i + e] + part[n + i + e]);
    }
  }
}

__global__ void k_splitk_reduce(const float* __restrict__ part, int S, int64_t n,
                                uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
    for (int k = 1; k < S; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)k * n + i);
      s += v;
    }
    u32x2 o;
    o[0] = pack_bf16x2(s[0], s[1]);
    o[1] = pack_bf16x2(s[2], s[3]);
    *reinterpret_cast<u32x2*>(out + i) = o;
  } else {
    for (int64_t e = i; e < n; ++e) {
      float s = part[e];
      for (int k = 1; k < S; ++k) s += part[(int64_t)k * n + e];
      out[e] = f32_to_bf16(s);
    }
  }
}

struct Cfg {
  int id, br, bt;
  bool pipe;
  int width = 64;      // logical columns per stage
  bool super = false;  // metadata in super-stages: C % 128 == 0 and no split of the reduction
};
// register-staged (any C % 32 == 0):
//   0 = 256x256 (4x4 accumulators per wave), 1 = 256x128 (4x2), 2 = 128x256 (2x4),
//   3 = 128x128 (2x2), 4 = 128x64 (2x1), 5 = 64x128 (1x2)
// LDS-DMA pipelined (C % 64 == 0):
//   10 = 256x256 (3 stages), 11 = 256x128 (4), 12 = 128x256 (3), 13 = 128x128 (3), 14 = 128x64 (4)
// LDS-DMA pipelined on 16x16x64 SMFMAC (C % 64 == 0):
//   20 = 256x128 (waves 128x64, 4 stages), 21 = 128x256 (waves 64x128, 3), 22 = 256x256 (3),
//   23 = 128x128 (waves 64x64, 3), 24 = 128x64 (waves 64x32, 4)
// wide stages (128 columns, C % 128 == 0) on 16x16x64 SMFMAC, metadata in 4-stage super-stages:
//   40 = 256x128 (waves 128x64, 2 stages), 41 = 128x128 (waves 64x64, 3), 44 = 256x64 (waves 128x32, 2)
// eight waves (512 threads) on 16x16x64 SMFMAC, 64-column stages:
//   50 = 256x128 (4x2 waves of 64x64, 4 stages), 51 = 256x256 (4x2 waves of 64x128, 3)
// the same with metadata in 8-stage super-stages (C % 128 == 0, no split):
//   55 = 256x128 (8 waves, 4 stages), 56 = 128x64 (4 waves, 4), 57 = 128x128 (4 waves, 3),
//   58 = 256x256 (8 waves, 2), 60 = 128x64 (8 waves of 32x32, 4)
// metadata in 4-stage super-stages (32-byte runs, half the LDS), so 256x256 keeps three stages:
//   61 = 256x256 (8 waves, 3)
// ping-pong (waves 0-3 and 4-7 half a stage apart, reads of one group beside the products of the
// other): 62 = 61 so scheduled
// streaming decode kernel (T <= 16, one 16-token column tile, weight read once from HBM):
//   30 = 64 weight rows per workgroup (decode24.hip)
constexpr Cfg kCfgs[] = {{0, 256, 256, false}, {1, 256, 128, false}, {2, 128, 256, false},
                         {3, 128, 128, false}, {4, 128, 64, false},  {5, 64, 128, false},
                         {10, 256, 256, true}, {11, 256, 128, true}, {12, 128, 256, true},
                         {13, 128, 128, true}, {14, 128, 64, true},
                         {20, 256, 128, true}, {21, 128, 256, true}, {22, 256, 256, true},
                         {23, 128, 128, true}, {24, 128, 64, true},  {30, 64, 16, false},
                         {40, 256, 128, true, 128}, {41, 128, 128, true, 128},
                         {44, 256, 64, true, 128}, {50, 256, 128, true}, {51, 256, 256, true},
                         {55, 256, 128, true, 64, true}, {56, 128, 64, true, 64, true},
                         {57, 128, 128, true, 64, true}, {58, 256, 256, true, 64, true},
                         {60, 128, 64, true, 64, true}, {61, 256, 256, true, 64, true},
                         {62, 256, 256, true, 64, true}};

Cfg cfg_by_id(int id) {
  for (const Cfg& c : kCfgs)
    if (c.id == id) return c;
  return kCfgs[3];
}

struct Plan {
  Cfg cfg;
  int splits;
  int stages_per_split;
  bool tail = false;  // splits == 2 for the tiles past the last whole wave of 256 only
};

Plan plan_for(int64_t R, int64_t C, int64_t T) {
  const bool pipe_ok = C % 64 == 0, wide_ok = C % 128 == 0;
  Plan p{cfg_by_id(pipe_ok ? 13 : 3), 1, 1};
  if (T <= 0 || R <= 0 || C <= 0) return p;
  const char* env = getenv("SRA_SPMM24_CFG");  // tuning override: "<cfg id>[,<splits>]"
  if (env && *env) {
    Cfg c = cfg_by_id(atoi(env));
    if ((c.width == 128 || c.super) && !wide_ok) c = cfg_by_id(pipe_ok ? 13 : 3);
    if (c.pipe && !pipe_ok) c = cfg_by_id(3);
    if (c.id == 30 && T > 16) c = cfg_by_id(3);
    p.cfg = c;
    const char* comma = strchr(env, ',');
    p.splits = comma ? atoi(comma + 1) : 1;
    p.tail = comma && strchr(comma, 't') != nullptr;  // "61,2t": split only the last wave's tiles
  } else {
    // Measured on MI355X (2:4, bf16): once 256x256 tiles fill the GPU twice, eight-wave 256x256
    // tiles with three stages and 4-stage metadata super-stages (C % 128 == 0; else per-stage
    // metadata, or 256x128 with four stages for long reductions, C >= 2R); eight-wave 256x128
    // once those fill the GPU; 128x64 for long reductions that would otherwise need a split;
    // otherwise 128x128 (two workgroups per CU), splitting the reduction when even those leave
    // CUs idle.
    auto tiles = [&](int br, int bt) { return ((R + br - 1) / br) * ((T + bt - 1) / bt); };
    if (T <= 16) {
      p.cfg = cfg_by_id(30);  // few tokens: bound by reading the weight once
    } else if (pipe_ok && tiles(256, 256) >= 512) {
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

template <int FR, int FT, int WR, int WT, int NS, int MS = 0, int UG = 0, bool DN = false, bool TLAY = false,
          bool PP = false>
void launch_q(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
              const uint16_t* act, int64_t T, const sra::Epilogue& ep, uint16_t* out, float* part,
              const Plan& p, hipStream_t s, int which = SRA_KERNEL_SPMM24) {
  using TL = QTile<FR, FT, WR, WT, NS, MS, UG, DN>;
  const int n_rt = (int)((R + TL::BR - 1) / TL::BR), n_tt = (int)((T + TL::BT - 1) / TL::BT);
  const int n = n_rt * n_tt, n_whole = p.tail ? n - n % 256 : -1;
  const dim3 grid = p.tail ? dim3((unsigned)(n_whole + 2 * (n - n_whole))) : dim3((unsigned)n, (unsigned)p.splits);
  sra::launch(which, k_spmm24_q<FR, FT, WR, WT, NS, MS, UG, DN, TLAY, PP>, grid, dim3(64 * TL::NW), 0, s,
              s_vals, s_meta, R, C, act, T, ep, out, part, n_rt, n_tt, p.stages_per_split, n_whole);
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

template <int FR, int FT, int NS, int MS>
void launch_w(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
              const uint16_t* act, int64_t T, const sra::Epilogue& ep, uint16_t* out, float* part,
              const Plan& p, hipStream_t s) {
  using TL = WTile<FR, FT, NS, MS>;
  const int n_rt = (int)((R + TL::BR - 1) / TL::BR), n_tt = (int)((T + TL::BT - 1) / TL::BT);
  sra::launch(SRA_KERNEL_SPMM24, k_spmm24_w<FR, FT, NS, MS>,
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
// SRA_SPMM24_FUSE=0 turns it off.
constexpr int kFuseRank = 16;
// Sum of a split product's fp32 partials into bf16 out: every element (k_splitk_reduce), or only
// the tail-split tiles of the 256x256 tiling (k_tail_reduce; the rest was stored whole).
void finish_split(const Plan& p, const float* part, int64_t R, int64_t T, uint16_t* out, hipStream_t s) {
  if (p.tail) {
    const int n_rt = (int)((R + 255) / 256), n_tt = (int)((T + 255) / 256), n = n_rt * n_tt;
    const int n_whole = n - n % 256;
    hipLaunchKernelGGL(k_tail_reduce, dim3((unsigned)(n - n_whole), 8), dim3(256), 0, s, part, T, R,
                       n_whole, n_rt, n_tt, 256, 256, out);
    return;
  }
  const int64_t n = T * R;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n / 4 + 255) / 256 + 1)), dim3(256), 0, s,
                     part, p.splits, n, out);
}

// The adapter epilogue reads E through a buffer resource: rows contiguous in j, and R rows of
// e_row_stride elements addressable with 32-bit byte offsets.
bool epilogue_ok(const sra::Epilogue& ep, int64_t R) {
  return ep.r <= 0 || (ep.e_j_stride == 1 && R * ep.e_row_stride * 2 < ((int64_t)1 << 31));
}
bool fuse_ok(const Plan& p, int64_t C, int r) {
  if (r <= 0 || r > kFuseRank || C % 64 != 0 || p.splits != 1) return false;
  const char* env = getenv("SRA_SPMM24_FUSE");
  if (env && env[0] == '0') return false;
  return p.cfg.id == 14 || p.cfg.id == 55 || p.cfg.id == 56 || p.cfg.id == 60;
}

}  // namespace

namespace sra {

hipError_t launch_dense_bf16(const uint16_t* Wd, int64_t R, int64_t C, const uint16_t* act, int64_t T,
                             const Epilogue& ep, uint16_t* out, hipStream_t s) {
  if (T == 0 || R == 0) return hipSuccess;
  if (C % 64 != 0 || ep.G || !epilogue_ok(ep, R)) return hipErrorInvalidValue;
  Plan p{cfg_by_id(13), 1, (int)(C / 64)};
  const int64_t big = ((R + 255) / 256) * ((T + 127) / 128);
  if (big >= 240)  // eight waves, 256x128 tiles, 3 stages of 48 KB
    launch_q<4, 4, 4, 2, 3, 0, 0, true>(Wd, nullptr, R, C, act, T, ep, out, nullptr, p, s, SRA_KERNEL_SPMM_FFI);
  else             // four waves, 128x64 tiles, 4 stages of 24 KB
    launch_q<4, 2, 2, 2, 4, 0, 0, true>(Wd, nullptr, R, C, act, T, ep, out, nullptr, p, s, SRA_KERNEL_SPMM_FFI);
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
  const bool wide = id == 0 || id == 10 || id == 22 || id == 51 || id == 58 || id == 61;  // 256x256
  const bool mid = id == 1 || id == 11 || id == 20 || id == 50 || id == 55;    // 256x128
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
      case 56: launch_q<4, 2, 2, 2, 3, 8, 16>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
      case 60: launch_q<2, 2, 4, 2, 4, 8, 16>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (p.cfg.id) {
    case 30: return launch_decode24_bf16(s_vals, s_meta, R, C, act, T, ep, out, s);
    case 55: launch_q<4, 4, 4, 2, 4, 8>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 56: launch_q<4, 2, 2, 2, 4, 8>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 60: launch_q<2, 2, 4, 2, 4, 8>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 57: launch_q<4, 4, 2, 2, 3, 8>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 58: launch_q<4, 8, 4, 2, 2, 8>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 61: launch_q<4, 8, 4, 2, 3, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 62: launch_q<4, 8, 4, 2, 3, 4, 0, false, false, true>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 50: launch_q<4, 4, 4, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 51: launch_q<4, 8, 4, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 40: launch_w<8, 4, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 41: launch_w<4, 4, 3, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 44: launch_w<8, 2, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 20: launch_q<8, 4, 2, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 21: launch_q<4, 8, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 22: launch_q<8, 8, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 23: launch_q<4, 4, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 24: launch_q<4, 2, 2, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 10: launch_pipe<4, 4, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 11: launch_pipe<4, 2, 2, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 12: launch_pipe<2, 4, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 13: launch_pipe<2, 2, 2, 2, 3>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 14: launch_pipe<2, 1, 2, 2, 4>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 0: launch_cfg<4, 4, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 1: launch_cfg<4, 2, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 2: launch_cfg<2, 4, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 4: launch_cfg<2, 1, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    case 5: launch_cfg<1, 2, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
    default: launch_cfg<2, 2, 2, 2>(s_vals, s_meta, R, C, act, T, ep, out, part, p, s); break;
  }
  if (p.splits > 1) finish_split(p, part, R, T, out, s);
  return hipGetLastError();
}

}  // namespace sra

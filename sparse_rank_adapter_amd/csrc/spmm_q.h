// The pipelined 2:4 SpMM on v_smfmac_f32_16x16x64_bf16 (k_spmm24_q) and the pieces it shares with
// the other product kernels: tile order, output staging, LDS-DMA transfers, in-kernel adapter
// rows, split-reduction sums.  Included by spmm24.hip (SMFMAC products) and spmm_xp.hip (the same
// pipeline with the weight fragments expanded to dense bf16 for dense MFMA: 2:8 weights, and 2:4
// weights on the dense engine).  Everything here is internal (anonymous namespace).
#pragma once

#include "common.h"

namespace {

constexpr int BC = 64;

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
              if (j + e < ep.r) write_vt3(ep.vt, ep.vt_rp, ep.vt_tp, j + e, tg, u[i][jf][e]);
          }
        } else if (ep.vt && tg < ep.vt_tp) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < ep.r)
#pragma unroll
              for (int p = 0; p < 3; ++p) ep.vt[((int64_t)p * ep.vt_rp + j + e) * ep.vt_tp + tg] = 0;
        }
      }
    }
  }
};

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
// DN: the weight tile is dense (rows of 128 bytes per stage, no metadata) and the products are
// pairs of dense v_mfma_f32_16x16x32_bf16; the tile is written in LDS from the fixed fan-in entry
// lists (FE > 0, below).
// NM = 24 / 28: the weight is 2:4 / 2:8 and each fragment is expanded to dense bf16 before the same
// pairs of dense MFMAs (expand24 / expand28).  2:8 rows carry 32 bytes of stored values per
// 64-column stage (two 16-byte chunks, slot = chunk ^ ((row >> 3) & 1)) and the same 8 bytes of
// metadata per stage as 2:4 (one byte per 8-column group), so the metadata transfers are 2:4's.
// FE > 0 (with DN): the fixed fan-in weight arrives in the tiled entry lists of sra_ffi_tile
// instead of dense rows.  Each wave owns 32 rows of the tile; per 64-column stage it copies up to
// FE of its rows' entries into LDS (LDS-DMA, with the activations), and one stage ahead of the
// products it clears its 32 rows of a dense 128-byte-row A tile and writes each entry's value at
// its (row, column).  The A tile is double-buffered apart from the ring (it is written with
// ordinary LDS stores one stage ahead, not transferred); the entry lists ride the ring.
template <int FR, int FT, int WR, int WT, int NS, int MS = 0, int UG = 0, bool DN = false, int NM = 0,
          int FE = 0>
struct QTile {
  static_assert(!(DN && (MS || UG)), "dense weights have no metadata or adapter rows");
  static_assert(NM == 0 || NM == 24 || NM == 28, "2:4 SMFMAC, or 2:4 / 2:8 expanded to dense");
  static_assert(FE == 0 || (DN && FE % 256 == 0), "fixed fan-in entry lists: dense products, whole 1 KB transfers");
  static_assert(!DN || FE > 0, "dense products take their weight tile from the entry lists");
  static constexpr int NW = WR * WT;  // waves per workgroup: 4 or 8
  static constexpr int BR = 16 * FR * WR, BT = 16 * FT * WT;
  static_assert(FE == 0 || BR == 32 * NW, "fixed fan-in: 32 weight rows per wave");
  static constexpr int VB = NM == 28 ? 32 : 64;  // stored-value bytes per weight row and stage
  static constexpr int LA = FE ? 0 : BR / ((NM == 28 ? 32 : 16) * NW);
  static constexpr int LM = (MS || DN) ? 0 : BR / (32 * NW);
  static constexpr int LB = BT / (8 * NW);
  static constexpr int LE = FE / 256;  // 1 KB entry transfers per wave and stage
  static constexpr int GT = UG / 8, GW = GT / NW, GX = GT % NW;
  static constexpr int L = LA + LM + LB + GW + LE;  // waves >= GX
  static constexpr int L1 = L + (GX ? 1 : 0);       // waves < GX
  static constexpr int A_BYTES = FE ? 0 : BR * VB, M_BYTES = (MS || DN) ? 0 : BR * 8;
  static constexpr int B_BYTES = (BT + UG) * 128;
  static constexpr int STAGE = A_BYTES + M_BYTES + B_BYTES;
  static constexpr int MSB = MS ? BR * MS * 8 : 0;            // one metadata super-stage buffer
  static constexpr int LMS = MS ? MSB / (1024 * NW) : 0;      // its 1 KB transfers per wave
  static constexpr int ABUF = FE ? 2 * BR * 128 : 0;          // the two scattered A tiles
  static constexpr int EBUF = NS * NW * FE * 4;               // entry lists, one per wave and ring slot
  static constexpr int OTAB = FE ? NW * 512 * 4 : 0;          // each wave's list offsets (<= 511 stages)
  static constexpr int LDS = NS * STAGE + 2 * MSB + ABUF + EBUF + OTAB;
  static constexpr int OCC = (NW == 8 || FR * FT >= 32 || 2 * LDS > 160 * 1024) ? 1 : 2;
};

// TLAY: the weight is in the streaming 2:4 layout (1 KB blocks per 16-row group and 64-column stage,
// metadata in 1 KB blocks per 16-row group and 512 columns; see decode24.hip), so every transfer of
// the values reads 1 KB contiguously instead of 64-byte runs per row, and a super-stage of
// metadata reads 64-byte (MS = 8) or 32-byte (MS = 4) pieces of those blocks.  Same LDS layout and
// products; needs MS > 0.
// FE > 0: s_vals holds the tiled fixed fan-in entries (ent_bytes bytes) and s_meta their list
// offsets (sra_ffi_tile); C % 64 == 0, no splits.
template <int FR, int FT, int WR, int WT, int NS, int MS = 0, int UG = 0, bool DN = false, bool TLAY = false,
          bool PP = false, int NM = 0, int FE = 0>
__global__ __launch_bounds__(64 * WR * WT, (QTile<FR, FT, WR, WT, NS, MS, UG, DN, NM, FE>::OCC)) void k_spmm24_q(
    const uint16_t* __restrict__ s_vals, const uint32_t* __restrict__ s_meta, int64_t R, int64_t C,
    const uint16_t* __restrict__ act, int64_t T, sra::Epilogue ep, uint16_t* __restrict__ out,
    float* __restrict__ part, int n_rt, int n_tt, int stages_per_split, int n_whole,
    uint32_t ent_bytes) {
  using TL = QTile<FR, FT, WR, WT, NS, MS, UG, DN, NM, FE>;
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
  static_assert(!PP || (NW == 8 && MS > 0 && UG == 0 && !DN && NM == 0), "ping-pong: eight waves, super-stages");
  static_assert(NM == 0 || !DN, "an expanded N:M weight is not a dense one");
  static_assert(NM != 28 || (!TLAY && BR % (32 * NW) == 0), "2:8: canonical arrays, whole transfers");
  static_assert(FE == 0 || (!TLAY && !PP), "fixed fan-in entry lists: their own schedule");
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
  const int64_t cv = NM == 28 ? C / 4 : C / 2, cm = C / 32;  // stored values, metadata words per row
  const int nC_all = (int)(C / BC);
  const int c_beg = z * stages_per_split;
  const int c_end = whole ? nC_all : min(nC_all, c_beg + stages_per_split);

  // operands through buffer resources based at the tile (fixed lane offsets, the stage offset in
  // an SGPR; rows past R, T or r read as zeros), as in k_spmm24_pipe
  const int rows_here = (int)min((int64_t)BR, R - row0), toks_here = (int)min((int64_t)BT, T - t0);
  constexpr int A_ROW = TLAY ? 1024 : TL::VB;  // stage offset of the weight operand (bytes)
  // streaming layout: 16-row groups of nsteps 1 KB value blocks and nbat 1 KB metadata blocks
  const int nsteps = (int)((C + 63) / 64), nbat = (int)((C + 511) / 512), ngrp = (rows_here + 15) / 16;
  const __amdgpu_buffer_rsrc_t ra =
      TLAY ? __builtin_amdgcn_make_buffer_rsrc((void*)(s_vals + (row0 / 16) * nsteps * 512), 0,
                                               ngrp * nsteps * 1024, 0x00020000)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(DN ? nullptr : s_vals + row0 * cv), 0,
                                               DN ? 0 : rows_here * (int)cv * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      TLAY ? __builtin_amdgcn_make_buffer_rsrc((void*)(s_meta + (row0 / 16) * nbat * 256), 0,
                                               ngrp * nbat * 1024, 0x00020000)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(DN ? nullptr : s_meta + row0 * cm), 0,
                                               DN ? 0 : rows_here * (int)cm * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(act + t0 * C), 0, toks_here * (int)C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ep.G, 0, UG > 0 ? ep.r * (int)ep.g_ld * 2 : 0, 0x00020000);
  uint32_t a_off[TL::LA ? TL::LA : 1];
  int a_dst[TL::LA ? TL::LA : 1];
#pragma unroll
  for (int k = 0; k < TL::LA; ++k) {
    const int b = k * NW + wave;
    if constexpr (NM == 28) {  // 32 rows of 32 bytes, chunk swizzle (row >> 3) & 1
      const int row = 32 * b + (lane >> 1), ch = (lane & 1) ^ ((row >> 3) & 1);
      a_off[k] = (uint32_t)(row * (C / 2) + ch * 16);
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
    constexpr int SL = MS ? MS / 2 : 1;  // 16-byte slots per row
    const int b = k * NW + wave, row = (1024 / (8 * (MS ? MS : 1))) * b + lane / SL, pos = lane % SL;
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
  // fixed fan-in: this wave's 32-row group, the entry lists' ring slots, the two A tiles after the
  // operand ring, and the group's list offsets (stage x: words otab[x] .. otab[x+1]) copied to LDS
  // once, so that reading them waits only on the wave's own earlier LDS work
  const int nst = (int)(C >> 6);
  const int64_t g_w = (row0 >> 5) + wave;
  const bool g_in = FE > 0 && g_w * 32 < R;
  const __amdgpu_buffer_rsrc_t rent = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(FE ? s_vals : nullptr), 0, FE ? (int)ent_bytes : 0, 0x00020000);
  uint8_t* const abuf = smem + NS * TL::STAGE + 2 * TL::MSB;
  uint8_t* const ebuf = abuf + TL::ABUF;
  uint32_t* const otab = reinterpret_cast<uint32_t*>(ebuf + TL::EBUF) + wave * 512;
  if constexpr (FE > 0) {
    const uint32_t* og = s_meta + (g_in ? g_w * nst : 0);
    for (int i = lane; i <= nst; i += 64) otab[i] = g_in ? og[i] : 0u;
  }
  auto fe_start = [&](int x) -> uint32_t { return otab[x]; };
  auto eslot = [&](int slot) { return ebuf + (slot * NW + wave) * FE * 4; };
  auto fe_tile = [&](int rel) { return abuf + (rel & 1) * (TL::BR * 128); };
  // one entry into the wave's rows of A tile `at`: bf16 value in the low half, in the high half
  // its byte offset in the group's 32 rows of 128 bytes (the tile's swizzle, chunk c of row i at
  // c ^ ((i >> 1) & 7), already applied; row 32 w + i of the tile has the same swizzle as row i);
  // padding entries (offset >= 4096) are skipped
  auto fe_put = [&](uint8_t* at, uint32_t e) {
    const uint32_t off = e >> 16;
    if (off < 4096) *reinterpret_cast<uint16_t*>(at + wave * 4096 + off) = (uint16_t)e;
  };
  auto fe_clear = [&](uint8_t* at) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(at + wave * 4096 + i * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
  };
  // entries q .. n-1 of a list starting at word e0, straight from memory (four per lane at a time)
  auto fe_from_memory = [&](uint8_t* at, uint32_t e0, uint32_t q, uint32_t n) {
    for (; q < n; q += 256) {
      const uint32_t q0 = q + (uint32_t)lane * 4;
      if (q0 < n) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rent, (e0 + q0) * 4, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (q0 + i < n) fe_put(at, v[i]);
      }
    }
  };
  // the first stage's A tile, all from memory
  auto fe_scatter_direct = [&](int rel) {
    uint8_t* at = fe_tile(rel);
    fe_clear(at);
    const uint32_t e0 = __builtin_amdgcn_readfirstlane(fe_start(c_beg + rel));
    const uint32_t n = min(__builtin_amdgcn_readfirstlane(fe_start(c_beg + rel + 1)) - e0, 2048u);
    fe_from_memory(at, e0, 0, n);
  };
  // later stages in two steps between the products of the stage before: (1) clear the A tile's
  // rows, read the list's bounds, its first FE words from the ring slot and the start of the list
  // the next transfer brings in; (2) a few products later, write the entries (a list holds at most
  // 32 * 64 words; past FE they come from memory)
  u32x4 fe_ev[TL::LE ? TL::LE : 1];
  uint32_t fe_lo = 0, fe_hi = 0, fe_dma = 0;
  // (step 1 runs whether or not the stage exists, with its table reads clamped, so that nothing
  // waits for these reads before step 2 uses them; the tile it clears is not read again)
  auto fe_step1 = [&](int rel) {  // during the products of stage c_beg + rel
    const int x = c_beg + rel + 1;
    fe_clear(fe_tile(rel + 1));
    fe_lo = fe_start(min(x, nst));
    fe_hi = fe_start(min(x + 1, nst));
    fe_dma = fe_start(min(x + NS - 1, nst));  // the list the next transfer brings in
    const uint8_t* es = eslot((rel + 1) % NS);
#pragma unroll
    for (int k = 0; k < TL::LE; ++k) fe_ev[k] = *reinterpret_cast<const u32x4*>(es + (k * 256 + lane * 4) * 4);
  };
  auto fe_step2 = [&](int rel) {
    const int x = c_beg + rel + 1;
    if (x < c_end) {
      uint8_t* at = fe_tile(rel + 1) + wave * 4096;
      const uint32_t e0 = __builtin_amdgcn_readfirstlane(fe_lo);
      const uint32_t n = min(__builtin_amdgcn_readfirstlane(fe_hi) - e0, 2048u);
#pragma unroll
      for (int k = 0; k < TL::LE; ++k) {
        const uint32_t q0 = (uint32_t)(k * 256 + lane * 4);
        if (q0 < n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t e = fe_ev[k][i], off = e >> 16;
            if (q0 + i < n && off < 4096) *reinterpret_cast<uint16_t*>(at + off) = (uint16_t)e;
          }
        }
      }
      if (n > (uint32_t)FE) fe_from_memory(fe_tile(rel + 1), e0, FE, n);
    }
  };
  auto issue = [&](int c, int buf) {
    uint8_t* base = smem + buf * TL::STAGE;
    // the entry list of stage c + 1 goes first (ring slot buf + 1), so that waiting for stage c's
    // transfers also covers it
    const uint32_t e_start = FE ? __builtin_amdgcn_readfirstlane(fe_dma) : 0u;  // list of stage c + 1
#pragma unroll
    for (int k = 0; k < TL::LE; ++k)
      bdma(rent, eslot((buf + 1) % NS) + k * 1024, 16, (uint32_t)(k * 1024 + lane * 16), e_start * 4);
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
  constexpr bool kIlv = UG == 0 && NM == 0 && !DN && !PP;
  constexpr int kIlvAhead = 2;  // column fragments read ahead of their products
  // compute(buf, rel, post): the products of the stage in buffer buf; post() issues the transfers
  // of a later stage and runs before the products, or between them in the interleaved schedule
  auto compute = [&](int buf, int rel, auto&& post) {
    if constexpr (!kIlv && !DN) post();
    const uint8_t* A = FE ? fe_tile(rel) : smem + buf * TL::STAGE;
    const uint32_t* M = reinterpret_cast<const uint32_t*>(smem + buf * TL::STAGE + TL::A_BYTES);
    const uint8_t* MS_buf = msbuf + (MS ? ((rel / (MS ? MS : 1)) & 1) * TL::MSB : 0);
    const int u = MS ? rel % (MS ? MS : 1) : 0;
    const uint8_t* B = smem + buf * TL::STAGE + TL::A_BYTES + TL::M_BYTES;
    if constexpr (UG > 0) ad.flush();
    bf16x16 bfr[FT];
    if constexpr (kIlv) {
      // Interleaved schedule (SMFMAC, no in-kernel adapter rows): the wave's row fragments and
      // their metadata first, then one column fragment at a time, each used by the FR products of
      // its column before the next is needed; column fragments are read two columns ahead and the
      // later stage's transfers are issued after the second column's first product.  The LDS reads
      // spread evenly over the stage's products instead of coming all at once, and a product waits
      // only for its own operands.
      bf16x8 af[FR];
      uint32_t mword[FR];
      auto read_row = [&](int i) {
        const int r = wr * 16 * FR + i * 16 + l16;
        af[i] = *reinterpret_cast<const bf16x8*>(A + r * 64 + ((q4 ^ ((r >> 2) & 3)) << 4));
        const int chunk = (u >> 1) ^ ms_swz(r);
        mword[i] = MS > 0 ? *reinterpret_cast<const uint32_t*>(MS_buf + r * (MS * 8) + (chunk << 4) +
                                                                4 * (2 * (u & 1) + (q4 >> 1)))
                          : M[r * 2 + (q4 >> 1)];
      };
      auto read_col = [&](int j) {
        const int tk = wt * 16 * FT + j * 16 + l16, sw = (tk >> 1) & 7;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 128 + ((q4 ^ sw) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 + q4) ^ sw) << 4));
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      };
      constexpr int CA = kIlvAhead < FT ? kIlvAhead : FT;  // column fragments read ahead
#pragma unroll
      for (int i = 0; i < FR; ++i) read_row(i);
#pragma unroll
      for (int j = 0; j < CA; ++j) read_col(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < FR * FT; ++k) {
        const int j = k / FR, i = k % FR;
        const int idx = (int)(mword[i] >> (16 * (q4 & 1)));
        acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[i], bfr[j], acc[i][j], idx, 0, 0);
        if (i == 0 && j + CA < FT) read_col(j + CA);
        if (k == (FT > 1 ? FR : 0)) post();
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    if constexpr (DN) {
      // dense weight rows: columns 8(l/16)..+7 and 32+8(l/16)..+7 of the stage, one dense MFMA
      // each.  The same interleaved order as the SMFMAC schedule: the wave's row fragments first,
      // then one column fragment at a time (read two columns ahead), the later stage's transfers
      // issued after the second column's first products.
      bf16x8 alo[FR], ahi[FR];
      auto read_col = [&](int j) {
        const int tk = wt * 16 * FT + j * 16 + l16, sw = (tk >> 1) & 7;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 128 + ((q4 ^ sw) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 + q4) ^ sw) << 4));
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      };
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 16 * FR + i * 16 + l16, sw = (r >> 1) & 7;
        alo[i] = *reinterpret_cast<const bf16x8*>(A + r * 128 + ((q4 ^ sw) << 4));
        ahi[i] = *reinterpret_cast<const bf16x8*>(A + r * 128 + (((4 + q4) ^ sw) << 4));
      }
      constexpr int CA = kIlvAhead < FT ? kIlvAhead : FT;
#pragma unroll
      for (int j = 0; j < CA; ++j) read_col(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < FR * FT; ++k) {
        const int j = k / FR, i = k % FR;
        const bf16x8 blo = __builtin_shufflevector(bfr[j], bfr[j], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 bhi = __builtin_shufflevector(bfr[j], bfr[j], 8, 9, 10, 11, 12, 13, 14, 15);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[i], blo, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[i], bhi, acc[i][j], 0, 0, 0);
        if (i == 0 && j + CA < FT) read_col(j + CA);
        // the later stage's transfers after the second column's first products; with entry lists,
        // step 1 there and step 2 with the transfers (which need the list start step 1 read)
        // four products later
        constexpr int kS1 = FT > 1 ? FR : 0, kS2 = 2 * FR < FR * FT - 1 ? 2 * FR : FR * FT - 1;
        if (k == kS1) {
          if constexpr (FE > 0) fe_step1(rel);
          else post();
        }
        if (FE > 0 && k == kS2) {
          fe_step2(rel);
          post();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int tk = wt * 16 * FT + j * 16 + l16, sw = (tk >> 1) & 7;
      const bf16x8 lo = *reinterpret_cast<const bf16x8*>(B + tk * 128 + ((q4 ^ sw) << 4));
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(B + tk * 128 + (((4 + q4) ^ sw) << 4));
      bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
    if constexpr (NM != 0) {
      // Expanded N:M: per weight fragment the stored values and both metadata words of the row's
      // stage are read first (behind one scheduling barrier with the activation reads); each
      // fragment is then expanded to the dense columns of the lane's A operand (lo: 8 q4 .. +7,
      // hi: 32 + 8 q4 .. +7) and multiplied with dense MFMAs, the layout of the activation
      // fragments above.
      constexpr int NV = NM == 28 ? 2 : 4;
      uint32_t sv[FR][NV];
      u32x2 mw[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int r = wr * 16 * FR + i * 16 + l16;
        if constexpr (MS > 0) {
          mw[i] = *reinterpret_cast<const u32x2*>(MS_buf + r * (MS * 8) + (((u >> 1) ^ ms_swz(r)) << 4) +
                                                  8 * (u & 1));
        } else {
          mw[i] = *reinterpret_cast<const u32x2*>(M + r * 2);
        }
        if constexpr (NM == 24) {  // stored 4 q4 .. +3 (lo) and 16 + 4 q4 .. +3 (hi): 8 bytes each
          const int sw = (r >> 2) & 3, h = 8 * (q4 & 1);
          const u32x2 lo = *reinterpret_cast<const u32x2*>(A + r * 64 + (((q4 >> 1) ^ sw) << 4) + h);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(A + r * 64 + (((2 + (q4 >> 1)) ^ sw) << 4) + h);
          sv[i][0] = lo[0];
          sv[i][1] = lo[1];
          sv[i][2] = hi[0];
          sv[i][3] = hi[1];
        } else {  // groups q4 (lo) and 4 + q4 (hi): their two stored values, 4 bytes each
          const int sw = (r >> 3) & 1;
          sv[i][0] = *reinterpret_cast<const uint32_t*>(A + r * 32 + (sw << 4) + 4 * q4);
          sv[i][1] = *reinterpret_cast<const uint32_t*>(A + r * 32 + ((1 ^ sw) << 4) + 4 * q4);
        }
      }
      if constexpr (UG > 0) ad.read(B, wave, lane);
      __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
      if constexpr (UG > 0) ad.mma(wave);
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const uint32_t mlo = (mw[i][0] >> (8 * q4)) & 255u, mhi = (mw[i][1] >> (8 * q4)) & 255u;
        bf16x8 alo, ahi;
        if constexpr (NM == 24) {
          alo = expand24(sv[i][0], sv[i][1], mlo);
          ahi = expand24(sv[i][2], sv[i][3], mhi);
        } else {
          alo = expand28(sv[i][0], mlo);
          ahi = expand28(sv[i][1], mhi);
        }
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          const bf16x8 blo = __builtin_shufflevector(bfr[j], bfr[j], 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 bhi = __builtin_shufflevector(bfr[j], bfr[j], 8, 9, 10, 11, 12, 13, 14, 15);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, blo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi, acc[i][j], 0, 0, 0);
        }
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
  // waiting for at most (in_flight-1)*L outstanding transfers completes stage c and every older
  // one, including the metadata of stage c's super-stage (issued before stage c's own loads).
  // Steady state unrolled by the ring depth: constant buffer indices, D stages in flight (not for
  // the largest wave tiles, whose registers are spoken for).
  constexpr bool kUnroll = FR * FT < 32;
  if constexpr (MS > 0) {
    if (c_beg < c_end) issue_meta(0);
  }
  // fixed fan-in: the first stage's A tile from memory; later ones one stage ahead from the ring
  if constexpr (FE > 0) {
    if (c_beg < c_end) fe_scatter_direct(0);
  }
  // the scattered A tile is written with LDS stores, which the bare barrier does not wait for
  auto stage_barrier = [&] {
    if constexpr (FE > 0) __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
    ring_barrier();
  };
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (c_beg + d < c_end) {
      if constexpr (FE > 0) fe_dma = fe_start(c_beg + d + 1);
      issue(c_beg + d, d);
    }
  int c = c_beg;
  for (; kUnroll && c + NS + D <= c_end; c += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (TL::GX && wave < TL::GX) wait_vm<((D - 1) * TL::L1 < 63 ? (D - 1) * TL::L1 : 63)>();
      else wait_vm<((D - 1) * L < 63 ? (D - 1) * L : 63)>();
      stage_barrier();
      const int rel = c + u - c_beg;
      compute(u, rel, [&] {
        if constexpr (MS > 0) {
          if (rel % MS == 0 && c + u + MS < c_end) issue_meta(rel / MS + 1);
        }
        issue(c + u + D, (u + D) % NS);
      });
    }
  }
  for (; c < c_end; ++c) {
    const int in_flight = min(D, c_end - c);
    if (TL::GX && wave < TL::GX) wait_stages<TL::L1>(in_flight);
    else wait_stages<L>(in_flight);
    stage_barrier();
    const int rel = c - c_beg;
    compute(rel % NS, rel, [&] {
      if constexpr (MS > 0) {
        if (rel % MS == 0 && c + MS < c_end) issue_meta(rel / MS + 1);
      }
      if (c + D < c_end) issue(c + D, (rel + D) % NS);
    });
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

struct Plan {
  Cfg cfg;
  int splits;
  int stages_per_split;
  bool tail = false;  // splits == 2 for the tiles past the last whole wave of 256 only
};

template <int FR, int FT, int WR, int WT, int NS, int MS = 0, int UG = 0, bool DN = false, bool TLAY = false,
          bool PP = false, int NM = 0, int FE = 0>
void launch_q(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
              const uint16_t* act, int64_t T, const sra::Epilogue& ep, uint16_t* out, float* part,
              const Plan& p, hipStream_t s, int which = SRA_KERNEL_SPMM24, uint32_t ent_bytes = 0) {
  using TL = QTile<FR, FT, WR, WT, NS, MS, UG, DN, NM, FE>;
  const int n_rt = (int)((R + TL::BR - 1) / TL::BR), n_tt = (int)((T + TL::BT - 1) / TL::BT);
  const int n = n_rt * n_tt, n_whole = p.tail ? n - n % 256 : -1;
  const dim3 grid = p.tail ? dim3((unsigned)(n_whole + 2 * (n - n_whole))) : dim3((unsigned)n, (unsigned)p.splits);
  sra::launch(which, k_spmm24_q<FR, FT, WR, WT, NS, MS, UG, DN, TLAY, PP, NM, FE>, grid, dim3(64 * TL::NW), 0, s,
              s_vals, s_meta, R, C, act, T, ep, out, part, n_rt, n_tt, p.stages_per_split, n_whole,
              ent_bytes);
}

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

}  // namespace

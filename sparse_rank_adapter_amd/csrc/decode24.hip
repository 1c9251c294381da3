// Decode-shaped 2:4 SpMM with the fused low-rank epilogue, for T <= 16 tokens:
//   Out[t][row] = sum_c Act[t][c] S[row][c] + sum_j U[t][j] E(row, j)
// (SLoPe paper, section 2.2 and its inference results: with few tokens the layer is bound by
// reading the compressed weight, and 2:4 halves those bytes; values plus 2-bit metadata are
// 9/16 of the dense bf16 weight.)  The 2:8 decode kernel (k_decode28, further below) computes the
// same for 2:8 weights, 5/16 of the dense bytes, sharing the epilogue (DecodeTail).
//
// Design: one pass over S straight from HBM into registers, no LDS staging.  All tokens fit in
// one v_smfmac_f32_16x16x64_bf16 column tile (tokens past T are zero), so the instruction's
// B operand (Act, 295 KB at the largest shape, L2-resident) is shared by every weight row tile.
// A workgroup owns 16 FR weight rows (FR 16-row tiles, FR = 3, 4 or 9 picked per shape so the
// workgroups split evenly over the CUs) and its NW waves (4, or 8 for FR = 9) split the
// reduction: batch b covers 64-column steps 8b .. 8b+7 and wave w takes the 8/NW steps from
// 8b + (8/NW)w, so the workgroup reads each row in 512-byte runs.  Each wave loads batch b+1 while
// multiplying batch b.  The NW partial tiles are summed through LDS in wave order
// (deterministic), and wave i % NW finishes row tile i: adapter epilogue on
// v_mfma_f32_16x16x32_bf16 (U as bf16 hi + lo) and a bf16 store.
//
// Operand layouts (gfx950, lane l, l16 = l % 16, q = l / 16):
//   A (weight)  row l16, logical columns 16q .. 16q+15 of the step = stored values 8q .. 8q+7,
//               metadata = half (q & 1) of word 2s + (q >> 1) of the row
//   B (tokens)  token l16, columns 8q .. 8q+7 and 32+8q .. 32+8q+7 of the step
//   D           rows 4q .. 4q+3 of token l16
//
// Streaming layout (TL = true, built by launch_nm_tile_bf16 from the canonical arrays): the
// canonical rows are C bytes apart, so a 16-row tile is 16 separate streams and a wave's 1 KB load
// is 16 pieces of 64 B.  In the streaming layout every (16-row tile, 64-column step) A fragment is
// one 1 KB block in lane order (lane 16q + i = row 16t + i, stored values 32s + 8q .. +7), blocks
// ordered by tile then step, and every (tile, 512-column batch) metadata block is 1 KB (row i's 16
// words at 64i).  Each load instruction then reads 1 KB contiguously and a workgroup walks its
// tiles' memory front to back.  Rows past R and steps past C are zero in the layout.
#include <algorithm>
#include <cstdlib>

#include "common.h"

namespace {

// Cache policy of the weight stream's loads on the streaming layout: non-temporal (gfx950's nt
// bit), since every weight byte is read once, so the activation block, which every workgroup
// re-reads, stays cached.  Measured at OPT-66B FFN: 67.3 -> 59.5 us at T = 1, 70.0 -> 62.8 us at
// T = 16.  The canonical arrays keep the default: there a 128-byte line is read as two 64-byte
// pieces by different loads, and a non-temporal line is dropped between them (72.9 -> 82.1 us).
constexpr int kStreamPolicy = 2;
// Buffer resource word 3 for untyped loads on gfx9-family GPUs (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
// Offsets stay below 2^31 (every resource is smaller), so setting bit 31 moves an access past the
// resource's end, where it reads zero.  Arithmetic rather than a select keeps the loads
// unconditional.
SRA_DEV uint32_t oob_unless(bool in, uint32_t off) { return off | ((uint32_t)!in << 31); }

// Per-thread register share of one batch (eight 64-column steps = 512 logical columns):
// SPW = 8 / NW steps of every row tile for this wave, MC metadata chunks and XC Act chunks
// (16 bytes each) of the workgroup's cooperative LDS staging.
template <int FR, int NW>
struct Batch {
  static constexpr int SPW = 8 / NW, MC = (FR + NW - 1) / NW, XC = 16 / NW;
  u32x4 a[FR][SPW];
  u32x4 m[MC];
  u32x4 x[XC];
};

constexpr int MLD = 20;       // LDS row of the metadata block: 16 words + 4 (16-byte rows, reads spread over banks)
constexpr int XLD = 512 + 8;  // LDS row of the Act block: 512 columns + 8 (bank spread)

// LDS of one workgroup: the double-buffered staging during the pass, then the NW x FR partial
// tiles of the reduction (which may be larger; both share one array).
template <int FR, int NW>
struct DecLds {
  static constexpr int RB = 16 * FR;
  static constexpr int ML = 2 * RB * MLD * 4, XL = 2 * 16 * XLD * 2, RED = NW * FR * 64 * 16;
  static constexpr int BYTES = ML + XL > RED ? ML + XL : RED;
};

// Adapter epilogue of both decode kernels.  Lane (l16, q) takes E(row rt + l16, j = jb .. jb+7) and
// U(token l16, j = jb .. jb+7) for jb = jj + 8q.  The first 64 adapter columns of the first row
// tile a wave finishes are loaded at construction, before the weight stream, so their latency is
// hidden behind it instead of following it (not for 64-row tiles, which have no registers to
// spare).  finish_tile() adds U E^T to row tile i's sums on v_mfma_f32_16x16x32_bf16 (U as bf16
// hi + lo) and stores bf16 rows 4q .. 4q+3 of token l16; finish() first sums the NW waves' partial
// tiles through LDS in wave order (deterministic), and row tile i is finished by wave i % NW.
template <int FR, int NW, int PF = FR == 4 ? 0 : 2>
struct DecodeTail {
  const sra::Epilogue& ep;
  const int64_t R, T, row0;
  const int w, l, l16, q;
  const bool tok_ok, e_vec, pf;
  u32x4 pf_e[2];
  float pf_u[2][8];

  SRA_DEV DecodeTail(const sra::Epilogue& ep_, int64_t R_, int64_t T_, int64_t row0_, int w_, int l_)
      : ep(ep_), R(R_), T(T_), row0(row0_), w(w_), l(l_), l16(l_ & 15), q(l_ >> 4), tok_ok(l16 < T_),
        e_vec(ep_.e_j_stride == 1 && (ep_.r & 7) == 0 && (ep_.e_row_stride & 7) == 0),
        pf(PF > 0 && ep_.r > 0 && w_ < FR && row0_ + 16 * w_ < R_) {
    if (pf) {
#pragma unroll
      for (int c = 0; c < PF; ++c) {
        pf_e[c] = load_e(row0 + 16 * w + l16, 32 * c + 8 * q);
        load_u(32 * c + 8 * q, pf_u[c]);
      }
    }
  }
  SRA_DEV u32x4 load_e(int64_t erow, int jb) const {
    union { u32x4 v; uint16_t h[8]; } x;
    x.v = u32x4{0, 0, 0, 0};
    if (erow < R) {
      if (e_vec && jb + 8 <= ep.r) {
        x.v = *reinterpret_cast<const u32x4*>(ep.E + erow * ep.e_row_stride + jb);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (jb + e < ep.r) x.h[e] = ep.E[erow * ep.e_row_stride + (int64_t)(jb + e) * ep.e_j_stride];
      }
    }
    return x.v;
  }
  SRA_DEV void load_u(int jb, float (&u)[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = tok_ok && jb + e < ep.r ? ep.U[(int64_t)l16 * ep.r + jb + e] : 0.f;
  }
  // call after the last use of the staging LDS by any wave (a barrier)
  SRA_DEV void finish(const f32x4 (&acc)[FR], unsigned char* lds, uint16_t* __restrict__ out) {
    f32x4* red = reinterpret_cast<f32x4*>(lds);  // [wave][tile][lane]
#pragma unroll
    for (int i = 0; i < FR; ++i) red[(w * FR + i) * 64 + l] = acc[i];
    __syncthreads();
    for (int i = w; i < FR; i += NW) {
      if (row0 + 16 * i >= R) break;
      f32x4 y = red[i * 64 + l];
#pragma unroll
      for (int k = 1; k < NW; ++k) y += red[(k * FR + i) * 64 + l];
      finish_tile(y, i, out);
    }
  }
  SRA_DEV void finish_tile(f32x4 y, int i, uint16_t* __restrict__ out) {
    const int64_t rt = row0 + 16 * i;
    if (rt >= R) return;
    // ---- adapter epilogue: A operand = E rows (row l16, j = 8q..), B operand = U^T (token l16)
    if (ep.r > 0) {
      const bool first = pf && i == w;  // the prefetched tile
      for (int jj = 0; jj < ep.r; jj += 32) {
        const int jb = jj + 8 * q;
        union { u32x4 v; bf16x8 b; } x;
        float u[8];
        if (first && jj < 32 * PF) {
          const int c = jj / 32;
          x.v = c == 0 ? pf_e[0] : pf_e[1];
#pragma unroll
          for (int e = 0; e < 8; ++e) u[e] = c == 0 ? pf_u[0][e] : pf_u[1][e];
        } else {
          x.v = load_e(rt + l16, jb);
          load_u(jb, u);
        }
        union UH { uint16_t h[8]; bf16x8 b; } uhi, ulo;
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(u[e], uhi.h[e], ulo.h[e]);
        y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.b, uhi.b, y, 0, 0, 0);
        y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.b, ulo.b, y, 0, 0, 0);
      }
    }

    // ---- store rows rt + 4q .. +3 of token l16
    if (!tok_ok) return;
    const int64_t n = rt + 4 * q;
    uint16_t* o = out + (int64_t)l16 * R + n;
    if ((R & 3) == 0 && n + 4 <= R) {
      u32x2 v;
      v[0] = pack_bf16x2(y[0], y[1]);
      v[1] = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<u32x2*>(o) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < R) o[e] = f32_to_bf16(y[e]);
    }
  }
};

// FR 16-row tiles per workgroup, NW waves splitting each batch's 8 steps (SPW each), OCC
// workgroups per CU.  (3, 4): 48 rows, 3 per CU; (4, 4): 64 rows; (9, 8): 144 rows, one per CU,
// which reads the Act block a third as often per weight byte.
template <int FR, int NW, int OCC, bool TL>
__global__ __launch_bounds__(64 * NW, OCC) void k_decode24(const uint16_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ meta, int64_t R,
                                                          int64_t C, const uint16_t* __restrict__ act,
                                                          int64_t T, sra::Epilogue ep,
                                                          uint16_t* __restrict__ out) {
  using BT = Batch<FR, NW>;
  using L = DecLds<FR, NW>;
  constexpr int RB = L::RB;  // weight rows per workgroup
  constexpr int SPW = BT::SPW, MC = BT::MC, XC = BT::XC, NT = 64 * NW;
  // Per batch the workgroup stages the metadata of its RB rows (64 B per row) and the Act block
  // (T x 512) in LDS with coalesced 16-byte loads; each wave streams its own steps of every row
  // tile's values into registers.
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];
  uint32_t(*ml)[RB * MLD] = reinterpret_cast<uint32_t(*)[RB * MLD]>(lds);
  uint16_t(*xl)[16 * XLD] = reinterpret_cast<uint16_t(*)[16 * XLD]>(lds + L::ML);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, q = l >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int64_t vstride = C / 2, mstride = C / 32;  // stored values / metadata words per row
  const int nb = (int)((C + 511) / 512);            // batches
  const int c32 = (int)C;                           // buffer offsets limit C to 32 bits anyway
  // Every operand goes through a buffer resource: 32-bit offsets, and an offset past the end
  // reads as zero, so no load needs a branch and a whole batch stays in flight.
  const int64_t nrows = min((int64_t)RB, R - row0);
  // streaming layout: 1 KB blocks per (tile, step) and per (tile, batch), this workgroup's FR tiles
  const int64_t nsteps = (C + 63) / 64, ntl = (nrows + 15) / 16, tile0 = row0 / 16;
  const __amdgpu_buffer_rsrc_t vres =
      TL ? __builtin_amdgcn_make_buffer_rsrc((void*)(vals + tile0 * nsteps * 512), (short)0,
                                             (int)(ntl * nsteps * 1024), kRsrcWord3)
         : __builtin_amdgcn_make_buffer_rsrc((void*)(vals + row0 * vstride), (short)0,
                                             (int)(nrows * vstride * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mres =
      TL ? __builtin_amdgcn_make_buffer_rsrc((void*)(meta + tile0 * nb * 256), (short)0,
                                             (int)(ntl * nb * 1024), kRsrcWord3)
         : __builtin_amdgcn_make_buffer_rsrc((void*)(meta + row0 * mstride), (short)0,
                                             (int)(nrows * mstride * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)act, (short)0, (int)(T * C * 2), kRsrcWord3);
  const uint32_t v_lane = TL ? (uint32_t)(16 * l) : (uint32_t)(l16 * vstride * 2 + 16 * q);  // bytes
  // metadata chunk c = tid + NT * k (k < MC): row c/4, words 4*(c%4) .. +3 of the batch's 16 (in
  // the streaming layout byte 16*(c%64) of tile c/64's block); chunks past RB rows are not staged

  auto load = [&](int b, BT& B) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int s = 8 * b + SPW * w + u;              // this wave's step
      const bool a_in = TL ? s < nsteps : 64 * s + 16 * q < c32;  // this lane's columns exist
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const uint32_t off = TL ? oob_unless(a_in, v_lane + (uint32_t)((i * nsteps + s) * 1024))
                                : oob_unless(a_in, v_lane + (uint32_t)((16 * i * vstride + 32 * s) * 2));
        B.a[i][u] = __builtin_amdgcn_raw_buffer_load_b128(vres, off, 0, TL ? kStreamPolicy : 0);
      }
    }
    // words past the row's end belong to steps whose values are zero; only the buffer end matters
#pragma unroll
    for (int k = 0; k < MC; ++k) {
      const int c = tid + NT * k, m_row = c >> 2, m_chunk = c & 3;
      const bool m_in = c < 4 * RB && (TL ? b < nb : 16 * b + 4 * m_chunk < (int)mstride);
      const uint32_t off = TL ? (uint32_t)((c >> 6) * nb * 1024 + 16 * (c & 63) + 1024 * b)
                              : (uint32_t)((m_row * mstride + 4 * m_chunk) * 4 + 64 * b);
      B.m[k] = __builtin_amdgcn_raw_buffer_load_b128(mres, oob_unless(m_in, off), 0, TL ? kStreamPolicy : 0);
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
      const int v = tid + NT * k, tok = v >> 6, col = 512 * b + 8 * (v & 63);
      const bool in = tok < T && col < c32;
      B.x[k] = __builtin_amdgcn_raw_buffer_load_b128(xres, oob_unless(in, (uint32_t)((tok * C + col) * 2)), 0, 0);
    }
  };
  auto stage = [&](int buf, const BT& B) {
#pragma unroll
    for (int k = 0; k < MC; ++k) {
      const int c = tid + NT * k;
      if (c < 4 * RB) *reinterpret_cast<u32x4*>(&ml[buf][(c >> 2) * MLD + 4 * (c & 3)]) = B.m[k];
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {
      const int v = tid + NT * k, tok = v >> 6, c = 8 * (v & 63);
      *reinterpret_cast<u32x4*>(&xl[buf][tok * XLD + c]) = B.x[k];
    }
  };

  f32x4 acc[FR];
#pragma unroll
  for (int i = 0; i < FR; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int hsh = 16 * (q & 1);
  auto compute = [&](int buf, const BT& B) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int j = SPW * w + u;  // step within the batch
      union { u32x4 v[2]; bf16x16 b; } xb;
      xb.v[0] = *reinterpret_cast<const u32x4*>(&xl[buf][l16 * XLD + 64 * j + 8 * q]);
      xb.v[1] = *reinterpret_cast<const u32x4*>(&xl[buf][l16 * XLD + 64 * j + 32 + 8 * q]);
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int idx = (int)(ml[buf][(16 * i + l16) * MLD + 2 * j + (q >> 1)] >> hsh);
        union { u32x4 v; bf16x8 b; } af;
        af.v = B.a[i][u];
        acc[i] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af.b, xb.b, acc[i], idx, 0, 0);
      }
    }
  };

  DecodeTail<FR, NW> tail(ep, R, T, row0, w, l);

  // Ping-pong over register batches; batches past the end are all-zero loads.  sched_barrier
  // keeps the compiler from sinking a batch's loads down to their first use.
  BT b0, b1;
  load(0, b0);
  for (int b = 0; b < nb; b += 2) {
    load(b + 1, b1);
    __builtin_amdgcn_sched_barrier(0);
    stage(0, b0);
    __syncthreads();
    compute(0, b0);
    __builtin_amdgcn_sched_barrier(0);
    load(b + 2, b0);
    __builtin_amdgcn_sched_barrier(0);
    stage(1, b1);
    __syncthreads();
    compute(1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // the reduction reuses the staging LDS
  tail.finish(acc, lds, out);
}

// 2:8 weights at T <= 16 (canonical arrays; SLoPe paper, section 2.1, N:M sparsity with M = 8).
// The pass reads 5/8 of a byte per weight entry (a quarter of the values plus 3-bit positions).
// Each 8-column group is fed to v_smfmac_f32_16x16x64_bf16 as two 2:4 groups, formed in
// registers: the half of positions 0-3 takes the pair (first value if its position is below 4,
// else 0; second value likewise) and the half of positions 4-7 the complementary pair, both with
// 2-bit indices (position % 4) of the first and the second value.  A value that is zeroed in a half
// keeps its index there (it may then name the same column as the other value, adding a zero
// product).  That is about 9 instructions per group; expanding to dense bf16 for dense MFMA took
// 19 and made the pass bound by them.  The layout differs from the 2:4 kernel's to keep more waves
// in flight and fewer bytes besides the weight:
//   - each of the NW waves owns FW whole 16-row tiles (tile w + NW f), so there is no reduction
//     over waves, and a 256-column batch of a tile is one contiguous run per row: lane (l16, q) reads
//     row l16's groups 8q .. 8q+7 of the batch, 32 bytes of values and its 2 metadata words (8 bytes)
//     straight into registers (one batch ahead);
//   - the Act batch (T x 256) is staged once per workgroup in LDS and shared by its 16 NW FW rows;
//   - SMFMAC step j of a batch takes the lane's groups 2j and 2j + 1 (of its 8: groups 8q .. 8q+7
//     of the batch) as its 16 logical columns 16q .. 16q+15 (the reduction order permuted the same
//     way on both operands).  Lane (token l16, q) of the B operand holds logical rows 8q .. 8q+7,
//     which are group 8 (q / 2) + 2j + q % 2 of the batch, and rows 32 + 8q .. +7, group
//     8 (2 + q / 2) + 2j + q % 2.  Each 64-column block of a staged Act row is followed by 16 bytes
//     of padding, which spreads the lanes' 16-byte reads over the banks.
// LDS row of a staged Act batch of BW columns: each 64-column block plus 8 columns of padding, and
// 8 more so that consecutive tokens start on different banks
template <int BW>
constexpr int d28_xld() { return BW + BW / 8 + 8; }
SRA_DEV int d28_col(int c) { return c + 8 * (c >> 6); }

// One BW-column batch of a wave: CL = BW / 128 chunks of 16 bytes (4 groups, one 32-bit word
// each) per row tile and lane, the lane's CL metadata words, and its share of the Act staging.
template <int NW, int FW, int BW>
struct Batch28 {
  static constexpr int CL = BW / 128, XC = (2 * BW + 64 * NW - 1) / (64 * NW);
  u32x4 v[FW][CL];
  uint32_t m[FW][CL];
  u32x4 x[XC];
};

// TL: the 2:8 streaming layout (launch_nm_tile28_bf16, 256-column batches): every (16-row tile,
// batch) block is 2 KB of values, chunk c of lane l at 1024 c + 16 l, then 512 bytes of metadata,
// lane l's two words at 8 l, so each wave load reads 1 KB (or 512 bytes) contiguously and
// non-temporally, and rows past R and columns past C hold zeros.
template <int NW, int FW, int BW, int OCC, bool TL>
__global__ __launch_bounds__(64 * NW, OCC) void k_decode28(const uint16_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ meta, int64_t R,
                                                          int64_t C, const uint16_t* __restrict__ act,
                                                          int64_t T, sra::Epilogue ep,
                                                          uint16_t* __restrict__ out) {
  using BT = Batch28<NW, FW, BW>;
  constexpr int FR = NW * FW, RB = 16 * FR, NT = 64 * NW, CL = BT::CL, XC = BT::XC;
  constexpr int XLD = d28_xld<BW>(), XCH = 2 * BW;  // Act chunks per batch (16 tokens x BW / 8)
  static_assert(CL == 2 || CL == 4, "256- or 512-column batches");
  static_assert(!TL || BW == 256, "the streaming layout has 256-column batches");
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][16 * XLD];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, q = l >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int64_t vstride = C / 4, mstride = C / 32;  // stored values / metadata words per row
  const int nb = (int)((C + BW - 1) / BW);          // batches
  const int c32 = (int)C;
  const int64_t nrows = min((int64_t)RB, R - row0);
  const int64_t tile0 = row0 / 16, ntl = (nrows + 15) / 16;  // streaming layout: this workgroup's tiles
  const __amdgpu_buffer_rsrc_t vres =
      TL ? __builtin_amdgcn_make_buffer_rsrc((void*)(vals + tile0 * nb * 1024), (short)0,
                                             (int)(ntl * nb * 2048), kRsrcWord3)
         : __builtin_amdgcn_make_buffer_rsrc((void*)(vals + row0 * vstride), (short)0,
                                             (int)(nrows * vstride * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mres =
      TL ? __builtin_amdgcn_make_buffer_rsrc((void*)(meta + tile0 * nb * 128), (short)0,
                                             (int)(ntl * nb * 512), kRsrcWord3)
         : __builtin_amdgcn_make_buffer_rsrc((void*)(meta + row0 * mstride), (short)0,
                                             (int)(nrows * mstride * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)act, (short)0, (int)(T * C * 2), kRsrcWord3);

  auto load = [&](int b, BT& B) {
    if constexpr (TL) {
#pragma unroll
      for (int f = 0; f < FW; ++f) {  // tiles past the workgroup's last read zero (past the resource)
        const uint32_t blk = (uint32_t)(((w + NW * f) * nb + b) * 2048);
#pragma unroll
        for (int c = 0; c < CL; ++c)
          B.v[f][c] = __builtin_amdgcn_raw_buffer_load_b128(vres, blk + 1024 * c + 16 * l, 0, kStreamPolicy);
        const u32x2 m = __builtin_amdgcn_raw_buffer_load_b64(mres, blk / 4 + 8 * l, 0, kStreamPolicy);
        B.m[f][0] = m[0];
        B.m[f][1] = m[1];
      }
    } else {
#pragma unroll
    for (int f = 0; f < FW; ++f) {
      const int row = 16 * (w + NW * f) + l16;  // rows past nrows read zero (past the resource)
#pragma unroll
      for (int c = 0; c < CL; ++c) {  // groups 4c .. 4c+3 of the lane: columns BW b + (BW/4) q + 32 c ..
        const bool in = BW * b + (BW / 4) * q + 32 * c < c32;
        const uint32_t off = (uint32_t)((row * vstride + (BW / 4) * b + (BW / 16) * q + 8 * c) * 2);
        B.v[f][c] = __builtin_amdgcn_raw_buffer_load_b128(vres, oob_unless(in, off), 0, 0);
      }
      // words past the row's end pair with zero values; past the resource they read zero
      const uint32_t moff = (uint32_t)((row * mstride + (BW / 32) * b + CL * q) * 4);
      if constexpr (CL == 2) {
        const u32x2 m = __builtin_amdgcn_raw_buffer_load_b64(mres, moff, 0, 0);
        B.m[f][0] = m[0];
        B.m[f][1] = m[1];
      } else {
        const u32x4 m = __builtin_amdgcn_raw_buffer_load_b128(mres, moff, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) B.m[f][c] = m[c];
      }
    }
    }
#pragma unroll
    for (int k = 0; k < XC; ++k) {  // chunk v: token v / (BW/8), columns 8 (v % (BW/8)) .. +7 of the batch
      const int v = tid + NT * k, tok = v / (BW / 8), col = BW * b + 8 * (v % (BW / 8));
      const bool in = v < XCH && tok < T && col < c32;
      B.x[k] = __builtin_amdgcn_raw_buffer_load_b128(xres, oob_unless(in, (uint32_t)((tok * C + col) * 2)), 0, 0);
    }
  };
  auto stage = [&](int buf, const BT& B) {
#pragma unroll
    for (int k = 0; k < XC; ++k) {
      const int v = tid + NT * k, tok = v / (BW / 8), c = 8 * (v % (BW / 8));
      if (v < XCH) *reinterpret_cast<u32x4*>(&xl[buf][tok * XLD + d28_col(c)]) = B.x[k];
    }
  };

  f32x4 acc[FW];
#pragma unroll
  for (int f = 0; f < FW; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // group g of the lane (pair s, metadata word mw, byte g % 4) as two 2:4 groups: values of the
  // low and the high half, and the 4-bit index field both halves share
  auto as24 = [](uint32_t s, uint32_t mw, int g, uint32_t& lo, uint32_t& hi) {
    const int sh = 8 * (g & 3);
    // all ones over the first / second value's 16 bits when its position is 4-7
    const uint32_t hmask = (((uint32_t)((int32_t)(mw << (29 - sh)) >> 31)) & 0xFFFFu) |
                           (((uint32_t)((int32_t)(mw << (26 - sh)) >> 31)) & 0xFFFF0000u);
    lo = s & ~hmask;
    hi = s & hmask;
    return ((mw >> sh) & 3u) | (((mw >> (sh + 3)) & 3u) << 2);
  };
  auto compute = [&](int buf, const BT& B) {
#pragma unroll
    for (int j = 0; j < 2 * CL; ++j) {
      union { u32x4 v[2]; bf16x16 b; } xb;
      const int ga = 8 * (q >> 1) + 2 * j + (q & 1);
      xb.v[0] = *reinterpret_cast<const u32x4*>(&xl[buf][l16 * XLD + d28_col(8 * ga)]);
      xb.v[1] = *reinterpret_cast<const u32x4*>(&xl[buf][l16 * XLD + d28_col(8 * (ga + 16))]);
#pragma unroll
      for (int f = 0; f < FW; ++f) {
        union { uint32_t u[4]; bf16x8 b; } af;
        const int g0 = 2 * j, g1 = 2 * j + 1;
        const uint32_t n0 = as24(B.v[f][g0 >> 2][g0 & 3], B.m[f][g0 >> 2], g0, af.u[0], af.u[1]);
        const uint32_t n1 = as24(B.v[f][g1 >> 2][g1 & 3], B.m[f][g1 >> 2], g1, af.u[2], af.u[3]);
        const uint32_t idx = (n0 | (n1 << 8)) * 0x11u;
        acc[f] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af.b, xb.b, acc[f], (int)idx, 0, 0);
      }
    }
  };

  DecodeTail<FR, NW, FW == 1 ? 0 : 2> tail(ep, R, T, row0, w, l);

  // ping-pong over register batches, as in the 2:4 kernel
  BT b0, b1;
  load(0, b0);
  for (int b = 0; b < nb; b += 2) {
    load(b + 1, b1);
    __builtin_amdgcn_sched_barrier(0);
    stage(0, b0);
    __syncthreads();
    compute(0, b0);
    __builtin_amdgcn_sched_barrier(0);
    load(b + 2, b0);
    __builtin_amdgcn_sched_barrier(0);
    stage(1, b1);
    __syncthreads();
    compute(1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int f = 0; f < FW; ++f) tail.finish_tile(acc[f], w + NW * f, out);
}

// Canonical 2:8 arrays -> the 2:8 streaming layout (see k_decode28).  One thread per 16-byte chunk:
// value chunks first (tiles x batches x 128: chunk c = g / 64 of lane g % 64), then metadata chunks
// (tiles x batches x 32: lanes 2h and 2h + 1).  C is a multiple of 32, so a value chunk (8 stored
// values, 4 groups) is wholly inside a row or past its end.
__global__ void k_nm_tile28(const uint16_t* __restrict__ vals, const uint32_t* __restrict__ meta,
                            int64_t R, int64_t C, u32x4* __restrict__ tvals, u32x4* __restrict__ tmeta) {
  const int64_t ntiles = (R + 15) / 16, nb = (C + 255) / 256;
  const int64_t nv = ntiles * nb * 128, nm = ntiles * nb * 32;
  const int64_t vstride = C / 4, mstride = C / 32;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < nv + nm;
       g += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (g < nv) {
      const int64_t blk = g >> 7, t = blk / nb, b = blk - t * nb;
      const int c = (int)((g >> 6) & 1), l = (int)(g & 63), i = l & 15, q = l >> 4;
      const int64_t row = 16 * t + i, col = 64 * b + 16 * q + 8 * c;  // stored-value column
      if (row < R && col < vstride) v = *reinterpret_cast<const u32x4*>(vals + row * vstride + col);
      tvals[g] = v;
    } else {
      const int64_t h = g - nv, blk = h >> 5, t = blk / nb, b = blk - t * nb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // lane 2 (h % 32) + e / 2, its word e % 2
        const int l = (int)(2 * (h & 31) + (e >> 1)), i = l & 15, q = l >> 4;
        const int64_t row = 16 * t + i, word = 8 * b + 2 * q + (e & 1);
        if (row < R && word < mstride) v[e] = meta[row * mstride + word];
      }
      tmeta[h] = v;
    }
  }
}

// Canonical 2:4 arrays -> streaming layout (see the header comment).  One thread per 16-byte
// chunk of the output: value chunks first (tiles x steps x 64), then metadata chunks
// (tiles x batches x 64).  Values move as whole 16-byte chunks (C/2 is a multiple of 16, so a
// chunk is either inside a row or past its end); metadata rows are C/32 words, not always a
// multiple of four, so those move word by word.
__global__ void k_nm_tile(const uint16_t* __restrict__ vals, const uint32_t* __restrict__ meta,
                          int64_t R, int64_t C, u32x4* __restrict__ tvals, u32x4* __restrict__ tmeta) {
  const int64_t ntiles = (R + 15) / 16, nsteps = (C + 63) / 64, nbat = (C + 511) / 512;
  const int64_t nv = ntiles * nsteps * 64, nm = ntiles * nbat * 64;
  const int64_t vstride = C / 2, mstride = C / 32;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < nv + nm;
       g += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (g < nv) {
      const int64_t blk = g >> 6, t = blk / nsteps, s = blk - t * nsteps;
      const int l = (int)(g & 63), i = l & 15, q = l >> 4;
      const int64_t row = 16 * t + i, col = 32 * s + 8 * q;
      if (row < R && col < vstride) v = *reinterpret_cast<const u32x4*>(vals + row * vstride + col);
      tvals[g] = v;
    } else {
      const int64_t h = g - nv, blk = h >> 6, t = blk / nbat, b = blk - t * nbat;
      const int l = (int)(h & 63), i = l >> 2, c = l & 3;
      const int64_t row = 16 * t + i, w0 = 16 * b + 4 * c;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (row < R && w0 + e < mstride) v[e] = meta[row * mstride + w0 + e];
      tmeta[h] = v;
    }
  }
}

}  // namespace

namespace sra {

size_t spmm24_decode_ws(int64_t, int64_t, int64_t) { return 0; }

void nm_tile_bytes(int64_t R, int64_t C, size_t* value_bytes, size_t* meta_bytes) {
  const int64_t ntiles = (R + 15) / 16;
  *value_bytes = (size_t)(ntiles * ((C + 63) / 64) * 1024);
  *meta_bytes = (size_t)(ntiles * ((C + 511) / 512) * 1024);
}

void nm28_tile_bytes(int64_t R, int64_t C, size_t* value_bytes, size_t* meta_bytes) {
  const int64_t blocks = ((R + 15) / 16) * ((C + 255) / 256);
  *value_bytes = (size_t)(blocks * 2048);
  *meta_bytes = (size_t)(blocks * 512);
}

hipError_t launch_nm_tile28_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                                 void* t_vals, void* t_meta, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if ((C & 31) != 0) return hipErrorInvalidValue;
  const int64_t chunks = ((R + 15) / 16) * ((C + 255) / 256) * 160;
  const unsigned grid = (unsigned)std::min<int64_t>((chunks + 255) / 256, 8192);
  hipLaunchKernelGGL(k_nm_tile28, dim3(grid), dim3(256), 0, s, s_vals, s_meta, R, C, (u32x4*)t_vals,
                     (u32x4*)t_meta);
  return hipGetLastError();
}

hipError_t launch_nm_tile_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                               void* t_vals, void* t_meta, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if ((C & 31) != 0) return hipErrorInvalidValue;
  const int64_t ntiles = (R + 15) / 16;
  const int64_t chunks = ntiles * ((C + 63) / 64) * 64 + ntiles * ((C + 511) / 512) * 64;
  const unsigned grid = (unsigned)std::min<int64_t>((chunks + 255) / 256, 8192);
  hipLaunchKernelGGL(k_nm_tile, dim3(grid), dim3(256), 0, s, s_vals, s_meta, R, C, (u32x4*)t_vals,
                     (u32x4*)t_meta);
  return hipGetLastError();
}

hipError_t launch_decode24_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R,
                                int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                uint16_t* out, hipStream_t s, bool tiled) {
  if (T <= 0 || R <= 0) return hipSuccess;
  if (T > 16 || (C & 31) != 0) return hipErrorInvalidValue;
  // Rows per workgroup: the CU with the most workgroups sets the time of a weight-streaming pass,
  // so pick the tile count whose busiest CU streams the fewest rows; ties go to the earlier
  // candidate.  On the canonical arrays the 144-row workgroups (one per CU) measured faster than
  // three 48-row ones at every T <= 16 (fewer Act re-reads, longer runs per row); on the streaming
  // layout the 48-row workgroups were faster (more waves in flight per CU).
  static constexpr int kCanon[3] = {9, 4, 3}, kTiled[2] = {4, 3};
  const int* cand = tiled ? kTiled : kCanon;
  const int ncand = tiled ? 2 : 3;
  int fr = cand[0];
  int64_t best = -1;
  for (int c = 0; c < ncand; ++c) {
    const int f = cand[c];
    const int64_t nwg = (R + 16 * f - 1) / (16 * f), per_cu = (nwg + 255) / 256 * 16 * f;
    if (best < 0 || per_cu < best) best = per_cu, fr = f;
  }
  if (tuning().decode_rows) fr = tuning().decode_rows;  // 3, 4 or 9 row tiles
  const unsigned grid = (unsigned)((R + 16 * fr - 1) / (16 * fr));
#define SRA_DECODE_LAUNCH(F, NW, OCC, TLV)                                                     \
  launch(SRA_KERNEL_DECODE24, k_decode24<F, NW, OCC, TLV>, dim3(grid), dim3(64 * NW), 0, s, s_vals, \
         s_meta, R, C, act, T, ep, out)
  if (tiled) {
    if (fr == 3) SRA_DECODE_LAUNCH(3, 4, 3, true);
    else if (fr == 4) SRA_DECODE_LAUNCH(4, 4, 3, true);
    else SRA_DECODE_LAUNCH(9, 8, 1, true);
  } else {
    if (fr == 3) SRA_DECODE_LAUNCH(3, 4, 3, false);
    else if (fr == 4) SRA_DECODE_LAUNCH(4, 4, 3, false);
    else SRA_DECODE_LAUNCH(9, 8, 1, false);
  }
#undef SRA_DECODE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode28_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R,
                                int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                uint16_t* out, hipStream_t s, bool tiled) {
  if (T <= 0 || R <= 0) return hipSuccess;
  if (T > 16 || (C & 31) != 0) return hipErrorInvalidValue;
  // Workgroup shapes (waves x row tiles per wave): 9 x 1 (144 rows), 4 x 2 (128), 4 x 1 (64) and
  // 3 x 1 (48).  As in the 2:4 kernel, the shape whose busiest CU streams the fewest rows wins,
  // ties going to the larger workgroup (fewer Act re-reads per weight byte).
  static constexpr int kShapes[4][2] = {{9, 1}, {4, 2}, {4, 1}, {3, 1}};
  int pick = 0;
  int64_t best = -1;
  for (int c = 0; c < 4; ++c) {
    const int rows = 16 * kShapes[c][0] * kShapes[c][1];
    const int64_t nwg = (R + rows - 1) / rows, per_cu = (nwg + 255) / 256 * rows;
    if (best < 0 || per_cu < best) best = per_cu, pick = c;
  }
  if (tuning().decode_rows == 9) pick = 0;  // forced: 9 tiles (144 rows), 4, or 3
  else if (tuning().decode_rows == 4) pick = 2;
  else if (tuning().decode_rows == 3) pick = 3;
  const int rows = 16 * kShapes[pick][0] * kShapes[pick][1];
  const unsigned grid = (unsigned)((R + rows - 1) / rows);
#define SRA_D28(NWV, FWV, BWV, OCCV)                                                             \
  do {                                                                                             \
    if (tiled)                                                                                     \
      launch(SRA_KERNEL_DECODE24, k_decode28<NWV, FWV, BWV, OCCV, true>, dim3(grid), dim3(64 * NWV), \
             0, s, s_vals, s_meta, R, C, act, T, ep, out);                                           \
    else                                                                                           \
      launch(SRA_KERNEL_DECODE24, k_decode28<NWV, FWV, BWV, OCCV, false>, dim3(grid), dim3(64 * NWV), \
             0, s, s_vals, s_meta, R, C, act, T, ep, out);                                           \
  } while (0)
  // (512-column batches, twice the bytes in flight per wave, measured no faster at the OPT-66B
  // FFN shape: 44.4 / 50.2 us against 44.1 / 49.6 us at T = 1 / 16)
  switch (pick) {
    case 0: SRA_D28(9, 1, 256, 1); break;
    case 1: SRA_D28(4, 2, 256, 3); break;
    case 2: SRA_D28(4, 1, 256, 3); break;
    default: SRA_D28(3, 1, 256, 4); break;
  }
#undef SRA_D28
  return hipGetLastError();
}

}  // namespace sra

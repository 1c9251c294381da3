// Decode-shaped 2:4 SpMM with the fused low-rank epilogue, for T <= 16 tokens:
//   Out[t][row] = sum_c Act[t][c] S[row][c] + sum_j U[t][j] E(row, j)
// (SLoPe paper, section 2.2 and its inference results: with few tokens the layer is bound by
// reading the compressed weight, and 2:4 halves those bytes; values plus 2-bit metadata are
// 9/16 of the dense bf16 weight.)
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

  // Adapter operands of the epilogue: lane (l16, q) takes E(row rt + l16, j = jb .. jb+7) and
  // U(token l16, j = jb .. jb+7) for jb = jj + 8q.  The first 64 adapter columns of the first row
  // tile this wave finishes are loaded here, before the weight stream, so their latency is hidden
  // behind it instead of following it.
  const bool tok_ok = l16 < T;
  const bool e_vec = ep.e_j_stride == 1 && (ep.r & 7) == 0 && (ep.e_row_stride & 7) == 0;
  auto load_e = [&](int64_t erow, int jb) {
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
  };
  auto load_u = [&](int jb, float (&u)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = tok_ok && jb + e < ep.r ? ep.U[(int64_t)l16 * ep.r + jb + e] : 0.f;
  };
  // prefetched 32-column adapter blocks (none for 64-row tiles, which have no registers to spare)
  constexpr int PF = FR == 4 ? 0 : 2;
  u32x4 pf_e[2];
  float pf_u[2][8];
  const bool pf = PF > 0 && ep.r > 0 && w < FR && row0 + 16 * w < R;
  if (pf) {
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      pf_e[c] = load_e(row0 + 16 * w + l16, 32 * c + 8 * q);
      load_u(32 * c + 8 * q, pf_u[c]);
    }
  }

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
  __syncthreads();  // the reduction below reuses the staging LDS

  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [wave][tile][lane]
#pragma unroll
  for (int i = 0; i < FR; ++i) red[(w * FR + i) * 64 + l] = acc[i];
  __syncthreads();
  // row tile i is finished by wave i % NW: partials summed in wave order (deterministic), adapter
  // epilogue, bf16 store
  for (int i = w; i < FR; i += NW) {
    const int64_t rt = row0 + 16 * i;
    if (rt >= R) break;
    f32x4 y = red[i * 64 + l];
#pragma unroll
    for (int k = 1; k < NW; ++k) y += red[(k * FR + i) * 64 + l];

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
    if (!tok_ok) continue;
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

}  // namespace sra

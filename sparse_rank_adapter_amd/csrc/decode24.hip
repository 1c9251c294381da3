// Decode-shaped 2:4 SpMM with the fused low-rank epilogue, for T <= 16 tokens:
//   Out[t][row] = sum_c Act[t][c] S[row][c] + sum_j U[t][j] E(row, j)
// (SLoPe paper, section 2.2 and its inference results: with few tokens the layer is bound by
// reading the compressed weight, and 2:4 halves those bytes; values plus 2-bit metadata are
// 9/16 of the dense bf16 weight.)
//
// Design: one pass over S straight from HBM into registers, no LDS staging.  All tokens fit in
// one v_smfmac_f32_16x16x64_bf16 column tile (tokens past T are zero), so the instruction's
// B operand (Act, 295 KB at the largest shape, L2-resident) is shared by every weight row tile.
// A workgroup owns 16 FR weight rows (FR 16-row tiles per wave, FR = 3 or 4 picked per shape so
// the workgroups split evenly over the CUs) and its four waves split the reduction: batch b covers 64-column steps 8b .. 8b+7 and wave w takes steps 8b+2w and
// 8b+2w+1, so the workgroup reads each row in 512-byte runs.  Each wave loads batch b+1 while
// multiplying batch b.  The four partial tiles are summed through LDS in wave order (deterministic), and
// wave w < FR finishes row tile w: adapter epilogue on v_mfma_f32_16x16x32_bf16 (U as bf16 hi + lo)
// and a bf16 store.
//
// Operand layouts (gfx950, lane l, l16 = l % 16, q = l / 16):
//   A (weight)  row l16, logical columns 16q .. 16q+15 of the step = stored values 8q .. 8q+7,
//               metadata = half (q & 1) of word 2s + (q >> 1) of the row
//   B (tokens)  token l16, columns 8q .. 8q+7 and 32+8q .. 32+8q+7 of the step
//   D           rows 4q .. 4q+3 of token l16
#include <cstdlib>

#include "common.h"

namespace {

// Buffer resource word 3 for untyped loads on gfx9-family GPUs (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
// Offsets stay below 2^31 (every resource is smaller), so setting bit 31 moves an access past the
// resource's end, where it reads zero.  Arithmetic rather than a select keeps the loads
// unconditional.
SRA_DEV uint32_t oob_unless(bool in, uint32_t off) { return off | ((uint32_t)!in << 31); }

template <int FR>
struct Batch {
  u32x4 a[FR][2];  // this wave's stored values, per row tile and step
  u32x4 m;         // cooperative share of the workgroup's metadata for the batch
  u32x4 x[4];      // cooperative share of the batch's Act columns
};

constexpr int MLD = 20;       // LDS row of the metadata block: 16 words + 4 (16-byte rows, reads spread over banks)
constexpr int XLD = 512 + 8;  // LDS row of the Act block: 512 columns + 8 (bank spread)

template <int FR>
__global__ __launch_bounds__(256, 3) void k_decode24(const uint16_t* __restrict__ vals,
                                                     const uint32_t* __restrict__ meta, int64_t R,
                                                     int64_t C, const uint16_t* __restrict__ act,
                                                     int64_t T, sra::Epilogue ep,
                                                     uint16_t* __restrict__ out) {
  constexpr int RB = 16 * FR;  // weight rows per workgroup
  // Per batch (eight 64-column steps = 512 logical columns) the workgroup stages the metadata of
  // its RB rows (64 B per row) and the Act block (T x 512) in LDS with one coalesced 16-byte
  // load per thread and vector; each wave streams its own rows' values into registers.
  __shared__ __attribute__((aligned(16))) uint32_t ml[2][RB * MLD];
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][16 * XLD];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, q = l >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * RB;
  const int64_t vstride = C / 2, mstride = C / 32;  // stored values / metadata words per row
  const int nb = (int)((C + 511) / 512);            // batches
  const int c32 = (int)C;                           // buffer offsets limit C to 32 bits anyway
  // Every operand goes through a buffer resource: 32-bit offsets, and an offset past the end
  // reads as zero, so no load needs a branch and a whole batch stays in flight.
  const int64_t nrows = min((int64_t)RB, R - row0);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vals + row0 * vstride), (short)0, (int)(nrows * vstride * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t mres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(meta + row0 * mstride), (short)0, (int)(nrows * mstride * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)act, (short)0, (int)(T * C * 2), kRsrcWord3);
  const uint32_t v_lane = (uint32_t)(l16 * vstride * 2 + 16 * q);  // bytes
  // metadata share: row tid/4, words 4*(tid%4) .. +3 of the batch's 16
  const int m_row = tid >> 2, m_chunk = tid & 3;
  const uint32_t m_lane = (uint32_t)((m_row * mstride + 4 * m_chunk) * 4);

  auto load = [&](int b, Batch<FR>& B) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int s = 8 * b + 2 * w + u;                // this wave's step
      const bool a_in = 64 * s + 16 * q < c32;        // this lane's 16 logical columns exist
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const uint32_t off = oob_unless(a_in, v_lane + (uint32_t)((16 * i * vstride + 32 * s) * 2));
        B.a[i][u] = __builtin_amdgcn_raw_buffer_load_b128(vres, off, 0, 0);
      }
    }
    // words past the row's end belong to steps whose values are zero; only the buffer end matters
    const bool m_in = 16 * b + 4 * m_chunk < (int)mstride;
    B.m = __builtin_amdgcn_raw_buffer_load_b128(mres, oob_unless(m_in, m_lane + (uint32_t)(64 * b)), 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = tid + 256 * k, tok = v >> 6, col = 512 * b + 8 * (v & 63);
      const bool in = tok < T && col < c32;
      B.x[k] = __builtin_amdgcn_raw_buffer_load_b128(xres, oob_unless(in, (uint32_t)((tok * C + col) * 2)), 0, 0);
    }
  };
  auto stage = [&](int buf, const Batch<FR>& B) {
    if (m_row < RB) *reinterpret_cast<u32x4*>(&ml[buf][m_row * MLD + 4 * m_chunk]) = B.m;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = tid + 256 * k, tok = v >> 6, c = 8 * (v & 63);
      *reinterpret_cast<u32x4*>(&xl[buf][tok * XLD + c]) = B.x[k];
    }
  };

  f32x4 acc[FR];
#pragma unroll
  for (int i = 0; i < FR; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int hsh = 16 * (q & 1);
  auto compute = [&](int buf, const Batch<FR>& B) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * w + u;  // step within the batch
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

  // Ping-pong over register batches; batches past the end are all-zero loads.  sched_barrier
  // keeps the compiler from sinking a batch's loads down to their first use.
  Batch<FR> b0, b1;
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
  __syncthreads();  // the reduction below reuses the Act block's LDS

  f32x4* red = reinterpret_cast<f32x4*>(&xl[0][0]);  // [wave][tile][lane]
#pragma unroll
  for (int i = 0; i < FR; ++i) red[(w * FR + i) * 64 + l] = acc[i];
  __syncthreads();
  if (w >= FR) return;  // FR row tiles, one per finishing wave
  f32x4 y = red[(0 * FR + w) * 64 + l];
#pragma unroll
  for (int k = 1; k < 4; ++k) y += red[(k * FR + w) * 64 + l];
  const int64_t rt = row0 + 16 * w;  // this wave's row tile
  if (rt >= R) return;
  const bool tok_ok = l16 < T;

  // ---- adapter epilogue: A operand = E rows (row l16, j = 8q..), B operand = U^T (token l16)
  if (ep.r > 0) {
    const bool e_vec = ep.e_j_stride == 1 && (ep.r & 7) == 0 && (ep.e_row_stride & 7) == 0;
    const int64_t erow = rt + l16;
    for (int jj = 0; jj < ep.r; jj += 32) {
      const int jb = jj + 8 * q;
      union UH { uint16_t h[8]; bf16x8 b; } uhi, ulo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float u = tok_ok && jb + e < ep.r ? ep.U[(int64_t)l16 * ep.r + jb + e] : 0.f;
        split_bf16(u, uhi.h[e], ulo.h[e]);
      }
      union { u32x4 v; uint16_t h[8]; bf16x8 b; } x;
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

}  // namespace

namespace sra {

size_t spmm24_decode_ws(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_decode24_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R,
                                int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                uint16_t* out, hipStream_t s) {
  if (T <= 0 || R <= 0) return hipSuccess;
  if (T > 16 || (C & 31) != 0) return hipErrorInvalidValue;
  // Rows per workgroup: the CU with the most workgroups sets the time of a weight-streaming pass,
  // so pick the tile count whose busiest CU streams the fewest rows (ties: the larger tile).
  int fr = 4;
  int64_t best = -1;
  for (int f = 4; f >= 3; --f) {
    const int64_t nwg = (R + 16 * f - 1) / (16 * f), per_cu = (nwg + 255) / 256 * 16 * f;
    if (best < 0 || per_cu < best) best = per_cu, fr = f;
  }
  const char* env = getenv("SRA_DECODE_FR");  // tuning override
  if (env && (*env == '3' || *env == '4')) fr = *env - '0';
  const unsigned grid = (unsigned)((R + 16 * fr - 1) / (16 * fr));
  if (fr == 3)
    launch(SRA_KERNEL_DECODE24, k_decode24<3>, dim3(grid), dim3(256), 0, s, s_vals, s_meta, R, C, act, T, ep, out);
  else
    launch(SRA_KERNEL_DECODE24, k_decode24<4>, dim3(grid), dim3(256), 0, s, s_vals, s_meta, R, C, act, T, ep, out);
  return hipGetLastError();
}

}  // namespace sra

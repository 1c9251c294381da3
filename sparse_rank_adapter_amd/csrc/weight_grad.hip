// Gradient of the stored values of a compressed 2:4 matrix (a sampled dense-dense product):
//
//   Out[row][i] = sum_t RowAct[t][row] * ColAct[t][c_i(row)]
//
// where c_i(row) is the column of the row's i-th stored entry.  For the forward weight Ws
// (rows = N outputs, cols = K) RowAct = dY and ColAct = X, so Out = (dY^T X) o mask1 in Ws's value
// order: the weight gradient of SLoPe's sparse training (SLoPe paperlayer summary, §2.1 -- the mask
// is fixed, only stored entries learn; §2.3 -- both compressed forms are kept).
//
// Design: the dense 64 x 128 block of RowAct^T ColAct is computed with v_mfma_f32_16x16x32_bf16 and
// only its stored half leaves.  The reduction (tokens) runs along the rows of both operands in
// memory, while an MFMA lane needs 8 consecutive reduction elements, so each 32-token stage is
// loaded coalesced along the rows (16-byte chunks) and written to LDS transposed ([row][t] and
// [col][t], 2-byte stores); fragments are then single 16-byte LDS reads.  Stages are double
// buffered with the next stage's global loads in flight during the products.  Each stage's MFMA
// starts from zero and its fp32 result is added to fp64 sums one stage later, so fp32 rounding acts
// only inside a 32-token partial (the outputs are sums of thousands of signed terms and can cancel
// to near zero).  The epilogue stages the block in LDS (fp32) and each thread picks the 16 stored
// values of one metadata word (2 of every 4 columns), rounds them to bf16 and writes 32 bytes.
#include "common.h"

namespace {

constexpr int SD_BM = 64, SD_BC = 128, SD_BT = 32;  // rows, logical columns, tokens per stage
constexpr int SD_LD = SD_BT + 8;                    // LDS row stride of the transposed tiles (bf16)
constexpr int SD_DLD = SD_BC + 4;                   // LDS row stride of the fp32 output block

__global__ __launch_bounds__(256) void k_sddmm24(const uint16_t* __restrict__ ra,
                                                 const uint16_t* __restrict__ ca,
                                                 const uint32_t* __restrict__ meta, int64_t R,
                                                 int64_t C, int64_t T, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t as[2][SD_BM * SD_LD];
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][SD_BC * SD_LD];
  __shared__ __attribute__((aligned(16))) float ds[SD_BM * SD_DLD];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, q4 = l >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * SD_BC, r0 = (int64_t)blockIdx.y * SD_BM;
  const int nst = (int)((T + SD_BT - 1) / SD_BT);

  // staging shares: one 8-row chunk of RowAct and two 8-column chunks of ColAct per thread
  const int a_t = tid >> 3, a_m = (tid & 7) * 8;
  const bool a_in = r0 + a_m < R;
  int b_t[2], b_c[2];
  bool b_in[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 256 * k;
    b_t[k] = idx >> 4;
    b_c[k] = (idx & 15) * 8;
    b_in[k] = c0 + b_c[k] < C;
  }
  u32x4 ga, gb[2];
  auto load = [&](int s) {
    const int64_t t = (int64_t)s * SD_BT;
    ga = (a_in && t + a_t < T) ? *reinterpret_cast<const u32x4*>(ra + (t + a_t) * R + r0 + a_m)
                               : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k)
      gb[k] = (b_in[k] && t + b_t[k] < T)
                  ? *reinterpret_cast<const u32x4*>(ca + (t + b_t[k]) * C + c0 + b_c[k])
                  : u32x4{0, 0, 0, 0};
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      as[buf][(a_m + 2 * e) * SD_LD + a_t] = (uint16_t)(ga[e] & 0xffffu);
      as[buf][(a_m + 2 * e + 1) * SD_LD + a_t] = (uint16_t)(ga[e] >> 16);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bs[buf][(b_c[k] + 2 * e) * SD_LD + b_t[k]] = (uint16_t)(gb[k][e] & 0xffffu);
        bs[buf][(b_c[k] + 2 * e + 1) * SD_LD + b_t[k]] = (uint16_t)(gb[k][e] >> 16);
      }
  };

  // wave w: rows 16w .. 16w+15 of the block against its 8 column fragments
  f32x4 d[8];
  double acc[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    d[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[j][e] = 0.0;
  }
  auto compute = [&](int buf) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&as[buf][(16 * w + l16) * SD_LD + 8 * q4]);
    bf16x8 b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(&bs[buf][(16 * j + l16) * SD_LD + 8 * q4]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] += (double)d[j][e];  // the previous stage's partial
      d[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
  };

  if (nst > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    if (s + 1 < nst) load(s + 1);
    compute(s & 1);
    if (s + 1 < nst) store((s + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[j][e] += (double)d[j][e];

  // dense block -> LDS: lane holds rows 16w + 4 q4 + e of column 16 j + l16
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[(16 * w + 4 * q4 + e) * SD_DLD + 16 * j + l16] = (float)acc[j][e];
  __syncthreads();

  // stored values: thread = (row m, 32-column group q) -> one metadata word, 16 values
  const int m = tid >> 2, q = tid & 3;
  const int64_t row = r0 + m, cg = c0 + 32 * q;
  if (row >= R || cg >= C) return;
  const uint32_t word = meta[row * (C / 32) + cg / 32];
  union { u32x4 v[2]; uint32_t w[8]; } o;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int p0 = (word >> (4 * g)) & 3, p1 = (word >> (4 * g + 2)) & 3;
    const float v0 = ds[m * SD_DLD + 32 * q + 4 * g + p0], v1 = ds[m * SD_DLD + 32 * q + 4 * g + p1];
    o.w[g] = pack_bf16x2(v0, v1);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * (C / 2) + cg / 2);
  dst[0] = o.v[0];
  dst[1] = o.v[1];
}

}  // namespace

namespace sra {

hipError_t launch_sddmm24_bf16(const uint16_t* row_act, const uint16_t* col_act, const uint32_t* meta,
                               int64_t R, int64_t C, int64_t T, uint16_t* out, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (R % 8 != 0 || C % 32 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((C + SD_BC - 1) / SD_BC), (unsigned)((R + SD_BM - 1) / SD_BM));
  launch(SRA_KERNEL_WEIGHT_GRAD, k_sddmm24, grid, dim3(256), 0, s, row_act, col_act, meta, R, C, T, out);
  return hipGetLastError();
}

}  // namespace sra

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
// memory, while an MFMA lane needs 8 consecutive reduction elements.  So a 64-token stage is
// loaded as 8 x 8 blocks (8 tokens x 8 rows or columns, eight coalesced 16-byte loads), each
// transposed in registers with byte permutes and written to LDS as eight 16-byte rows of 8
// tokens ([row][t] and [col][t]); fragments are then single 16-byte LDS reads.  Stages are double
// buffered with the next stage's loads in flight during the products.  Each stage's products start
// from zero in fp32 and are added to fp64 sums one stage later, so fp32 rounding acts only inside
// a 64-token partial (the outputs are sums of thousands of signed terms and can cancel to near
// zero).  The epilogue stages the fp32 block in LDS (over the operand buffers) and each thread
// picks the 16 stored values of one metadata word (2 of every 4 columns), rounds them to bf16 and
// writes 32 bytes.
#include <algorithm>

#include "common.h"

namespace {

constexpr int SD_BM = 64, SD_BC = 128, SD_BT = 64;  // rows, logical columns, tokens per stage
constexpr int SD_LD = SD_BT + 8;                    // LDS row stride of the transposed tiles (bf16)
constexpr int SD_DLD = SD_BC + 4;                   // LDS row stride of the fp32 output block
constexpr int SD_AB = SD_BM * SD_LD, SD_BB = SD_BC * SD_LD;  // elements per stage buffer
constexpr int SD_LDS = 2 * (SD_AB + SD_BB) * 2;              // bytes: two stages of both operands
static_assert(SD_BM * SD_DLD * 4 <= SD_LDS, "the output block fits over the operand buffers");

// 8 x 8 bf16 transpose: in[i] holds row i (8 elements), out[j] receives column j.
SRA_DEV void transpose8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      out[j][k] = __builtin_amdgcn_perm(in[2 * k + 1][j >> 1], in[2 * k][j >> 1],
                                        (j & 1) ? 0x07060302u : 0x05040100u);
}

__global__ __launch_bounds__(256, 2) void k_sddmm24(const uint16_t* __restrict__ ra,
                                                    const uint16_t* __restrict__ ca,
                                                    const uint32_t* __restrict__ meta, uint32_t meta_or,
                                                    int64_t R, int64_t C, int64_t T,
                                                    uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[SD_LDS];
  uint16_t* const as0 = reinterpret_cast<uint16_t*>(lds);
  uint16_t* const bs0 = as0 + 2 * SD_AB;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, q4 = l >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * SD_BC, r0 = (int64_t)blockIdx.y * SD_BM;
  const int nst = (int)((T + SD_BT - 1) / SD_BT);

  // staging: threads 0..127 own one 8 x 8 block of ColAct (16 column blocks x 8 token blocks),
  // threads 128..191 one of RowAct (8 row blocks x 8 token blocks); consecutive threads take
  // consecutive 16-byte chunks of a token row
  const bool is_b = tid < 128, is_a = tid >= 128 && tid < 192;
  const int blk = is_b ? tid : tid - 128;
  const int bx = is_b ? (blk & 15) : (blk & 7), bt = is_b ? (blk >> 4) : (blk >> 3);
  const uint16_t* src = is_b ? ca + c0 + 8 * bx : ra + r0 + 8 * bx;
  const int64_t ld = is_b ? C : R;
  const bool x_in = (is_b && c0 + 8 * bx < C) || (is_a && r0 + 8 * bx < R);
  u32x4 g[8];
  auto load = [&](int s) {
    const int64_t t = (int64_t)s * SD_BT + 8 * bt;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      g[i] = (x_in && t + i < T) ? *reinterpret_cast<const u32x4*>(src + (t + i) * ld) : u32x4{0, 0, 0, 0};
  };
  auto store = [&](int buf) {
    if (!is_a && !is_b) return;
    u32x4 tr[8];
    transpose8(g, tr);
    uint16_t* dst = is_b ? bs0 + buf * SD_BB : as0 + buf * SD_AB;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(dst + (8 * bx + j) * SD_LD + 8 * bt) = tr[j];
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
    const uint16_t* as = as0 + buf * SD_AB;
    const uint16_t* bs = bs0 + buf * SD_BB;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] += (double)d[j][e];  // the previous stage's partial
#pragma unroll
    for (int kk = 0; kk < SD_BT / 32; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(as + (16 * w + l16) * SD_LD + 32 * kk + 8 * q4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(bs + (16 * j + l16) * SD_LD + 32 * kk + 8 * q4);
        d[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, kk ? d[j] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
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

  // dense block -> LDS (over the operand buffers, free after the last barrier): lane holds rows
  // 16w + 4 q4 + e of column 16 j + l16
  float* const ds = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) ds[(16 * w + 4 * q4 + e) * SD_DLD + 16 * j + l16] = (float)acc[j][e];
  __syncthreads();

  // stored values: thread = (row m, 32-column group q) -> one metadata word, 16 values
  const int m = tid >> 2, q = tid & 3;
  const int64_t row = r0 + m, cg = c0 + 32 * q;
  if (row >= R || cg >= C) return;
  const uint32_t word = meta[row * (C / 32) + cg / 32] | meta_or;  // 1:2 read as its 2:4 encoding
  union { u32x4 v[2]; uint32_t w[8]; } o;
#pragma unroll
  for (int g8 = 0; g8 < 8; ++g8) {
    const int p0 = (word >> (4 * g8)) & 3, p1 = (word >> (4 * g8 + 2)) & 3;
    const float v0 = ds[m * SD_DLD + 32 * q + 4 * g8 + p0], v1 = ds[m * SD_DLD + 32 * q + 4 * g8 + p1];
    o.w[g8] = pack_bf16x2(v0, v1);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * (C / 2) + cg / 2);
  dst[0] = o.v[0];
  dst[1] = o.v[1];
}

// beta * A + gamma * B on the value arrays of two compressed matrices that share one N:M pattern
// (SLoPe §2.3's sparse addition; §2.1: the mask is fixed, so the metadata is unchanged): weight
// decay and the update step of sparse training, e.g. Ws <- (1 - lr wd) Ws - lr dWs with dWs from
// k_sddmm24.  Bandwidth-bound: 16 bytes per lane and operand, fp32 arithmetic (one fma), one
// rounding to the storage type.  `out` may be `a` (in place).
template <bool BF16>
__global__ __launch_bounds__(256) void k_nm_axpby(const void* __restrict__ a, float beta,
                                                  const void* __restrict__ b, float gamma,
                                                  void* out, int64_t n) {
  constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte chunk
  constexpr int U = 4;             // chunks per thread and iteration, all loads issued first
  const int64_t nch = n / E;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  auto combine = [&](const u32x4& va, const u32x4& vb) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (BF16) {
        const float a0 = __uint_as_float(va[k] << 16), a1 = __uint_as_float(va[k] & 0xffff0000u);
        const float b0 = __uint_as_float(vb[k] << 16), b1 = __uint_as_float(vb[k] & 0xffff0000u);
        r[k] = pack_bf16x2(fmaf(beta, a0, gamma * b0), fmaf(beta, a1, gamma * b1));
      } else {
        r[k] = __float_as_uint(fmaf(beta, __uint_as_float(va[k]), gamma * __uint_as_float(vb[k])));
      }
    }
    return r;
  };
  const u32x4* pa = reinterpret_cast<const u32x4*>(a);
  const u32x4* pb = reinterpret_cast<const u32x4*>(b);
  u32x4* po = reinterpret_cast<u32x4*>(out);
  // workgroup tiles of U x 256 consecutive chunks: the U loads of a wave read adjacent 1 KB runs
  const int64_t full = nch / (U * 256);
  for (int64_t tile = blockIdx.x; tile < full; tile += gridDim.x) {
    const int64_t i = tile * (U * 256) + threadIdx.x;
    u32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      va[u] = pa[i + 256 * u];
      vb[u] = pb[i + 256 * u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) po[i + 256 * u] = combine(va[u], vb[u]);
  }
  for (int64_t i = full * (U * 256) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nch; i += stride)
    po[i] = combine(pa[i], pb[i]);
  // tail (n % E < E elements), one thread each
  const int64_t t = nch * E + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) {
    if constexpr (BF16) {
      const float av = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(a)[t] << 16);
      const float bv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(b)[t] << 16);
      reinterpret_cast<uint16_t*>(out)[t] = f32_to_bf16(fmaf(beta, av, gamma * bv));
    } else {
      reinterpret_cast<float*>(out)[t] =
          fmaf(beta, reinterpret_cast<const float*>(a)[t], gamma * reinterpret_cast<const float*>(b)[t]);
    }
  }
}

}  // namespace

namespace sra {

hipError_t launch_sddmm24_bf16(const uint16_t* row_act, const uint16_t* col_act, const uint32_t* meta,
                               uint32_t meta_or, int64_t R, int64_t C, int64_t T, uint16_t* out,
                               hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (R % 8 != 0 || C % 32 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((C + SD_BC - 1) / SD_BC), (unsigned)((R + SD_BM - 1) / SD_BM));
  launch(SRA_KERNEL_WEIGHT_GRAD, k_sddmm24, grid, dim3(256), 0, s, row_act, col_act, meta, meta_or, R, C,
         T, out);
  return hipGetLastError();
}

hipError_t launch_nm_axpby(int dtype, const void* a, float beta, const void* b, float gamma, void* out,
                          int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t nch = n / (dtype == SRA_BF16 ? 8 : 4);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((nch + 1023) / 1024, 2048));
  if (dtype == SRA_BF16)
    launch(SRA_KERNEL_NM_UPDATE, k_nm_axpby<true>, dim3(grid), dim3(256), 0, s, a, beta, b, gamma, out, n);
  else
    launch(SRA_KERNEL_NM_UPDATE, k_nm_axpby<false>, dim3(grid), dim3(256), 0, s, a, beta, b, gamma, out, n);
  return hipGetLastError();
}

}  // namespace sra

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
// memory, while an MFMA lane needs 8 consecutive reduction elements.  Each 64-token stage is copied
// as it lies (rows of tokens) from global memory to LDS by buffer -> LDS transfers into a three-
// stage ring, and the fragments are read with ds_read_b64_tr_b16, gfx950's transposing LDS read:
// within a group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// i / 4 + 4 r (r = 0..3).  So lane j (r = j / 4, s = j % 4) of lane group g addresses row
// t = 8 g + 4 h + r and columns m0 + 4 s .. +3, and lane i gets column m0 + i at tokens
// 8 g + 4 h .. +3: half (h) of an MFMA fragment.  Rows are XOR-swizzled by 16-byte chunk so the 16
// rows of one read spread over the LDS banks.  Each stage's products start from zero in fp32 and are
// added to fp64 sums one stage later, so fp32 rounding acts only inside a 64-token partial (the
// outputs are sums of thousands of signed terms and can cancel to near zero).  The epilogue stages
// the fp32 block in LDS (over the ring) and each thread picks the 16 stored values of one metadata
// word (2 of every 4 columns), rounds them to bf16 and writes 32 bytes.
#include <algorithm>

#include "common.h"

namespace {

constexpr int SD_BM = 64, SD_BC = 128, SD_BT = 64;  // rows, logical columns, tokens per stage
constexpr int SD_NS = 3;                            // ring stages
constexpr int SD_AROW = SD_BM * 2, SD_BROW = SD_BC * 2;        // bytes per token row of each tile
constexpr int SD_ASTG = SD_BT * SD_AROW, SD_BSTG = SD_BT * SD_BROW;
constexpr int SD_STAGE = SD_ASTG + SD_BSTG;                    // 24 KB
constexpr int SD_DLD = SD_BC + 4;                              // LDS row stride of the fp32 block
constexpr int SD_LA = SD_ASTG / (1024 * 4), SD_LB = SD_BSTG / (1024 * 4);  // 1 KB transfers per wave
static_assert(SD_BM * SD_DLD * 4 <= SD_NS * SD_STAGE, "the output block fits over the ring");

typedef __attribute__((address_space(3))) void* sd_lds_t;
typedef short sd_v4s __attribute__((ext_vector_type(4)));

// chunk swizzles (16-byte chunks, even values keep chunk pairs together): over the 16 rows one
// transposing read touches, the 32-byte windows land in 8 distinct bank windows, twice each
SRA_DEV int swz_a(int t) { return 2 * (((t >> 1) ^ (t >> 3)) & 3); }
SRA_DEV int swz_b(int t) { return 2 * ((t & 3) | (((t >> 3) & 1) << 2)); }

SRA_DEV void sd_dma(__amdgpu_buffer_rsrc_t rs, uint8_t* lds_block, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (sd_lds_t)lds_block, 16, voff, soff, 0, 0);
}
template <int N>
SRA_DEV void sd_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// half of an MFMA fragment (4 tokens of 16 rows or columns) by one transposing read
SRA_DEV sd_v4s sd_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) sd_v4s*)p);
}

__global__ __launch_bounds__(256, 2) void k_sddmm24(const uint16_t* __restrict__ ra,
                                                    const uint16_t* __restrict__ ca,
                                                    const uint32_t* __restrict__ meta, uint32_t meta_or,
                                                    int64_t R, int64_t C, int64_t T,
                                                    uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[SD_NS * SD_STAGE];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, q4 = l >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * SD_BC, r0 = (int64_t)blockIdx.y * SD_BM;
  const int nst = (int)((T + SD_BT - 1) / SD_BT);

  // buffer resources based at the tile's first column; rows past T are past the range (zeros),
  // columns past R or C get an offset with bit 31 set (past the range too)
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ra + r0), (short)0, (int)((T * R - r0) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ca + c0), (short)0, (int)((T * C - c0) * 2), 0x00020000);
  // transfer k of this wave: A block q = k * 4 + w covers tile rows 8q .. 8q+7 (lane: row 8q + l/8,
  // physical chunk l % 8); B block q covers rows 4q .. 4q+3 (row 4q + l/16, chunk l % 16).  The
  // lane fetches the logical chunk that its slot holds under the swizzle.
  uint32_t a_off[SD_LA], b_off[SD_LB];
#pragma unroll
  for (int k = 0; k < SD_LA; ++k) {
    const int q = k * 4 + w, t = 8 * q + (l >> 3), lc = (l & 7) ^ swz_a(t);
    const bool in = r0 + 8 * lc < R;
    a_off[k] = (uint32_t)((t * R + 8 * lc) * 2) | ((uint32_t)!in << 31);
  }
#pragma unroll
  for (int k = 0; k < SD_LB; ++k) {
    const int q = k * 4 + w, t = 4 * q + (l >> 4), lc = (l & 15) ^ swz_b(t);
    const bool in = c0 + 8 * lc < C;
    b_off[k] = (uint32_t)((t * C + 8 * lc) * 2) | ((uint32_t)!in << 31);
  }
  auto issue = [&](int st, int buf) {
    uint8_t* base = lds + buf * SD_STAGE;
    const int soff_a = (int)((int64_t)st * SD_BT * R * 2), soff_b = (int)((int64_t)st * SD_BT * C * 2);
#pragma unroll
    for (int k = 0; k < SD_LA; ++k) sd_dma(rsa, base + (k * 4 + w) * 1024, a_off[k], soff_a);
#pragma unroll
    for (int k = 0; k < SD_LB; ++k) sd_dma(rsb, base + SD_ASTG + (k * 4 + w) * 1024, b_off[k], soff_b);
  };

  // fragment read addresses: lane (group g = q4, j = l16: r = j/4, s = j%4), half h, K-step kk
  const int fr = l16 >> 2, fs = l16 & 3;
  auto frag = [&](const uint8_t* tile, int rowb, bool is_a, int m0, int kk) {
    union { sd_v4s h[2]; bf16x8 v; } u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 32 * kk + 8 * q4 + 4 * h + fr, col = m0 + 4 * fs;
      const int pc = (col >> 3) ^ (is_a ? swz_a(t) : swz_b(t));
      u.h[h] = sd_tr(tile + t * rowb + pc * 16 + (col & 7) * 2);
    }
    return u.v;
  };

  // wave w: rows 32 (w / 2) .. +31 (two row fragments) against columns 64 (w % 2) .. +63 (four
  // column fragments): six fragment reads per 32-token step for eight products
  const int wr = 32 * (w >> 1), wc = 64 * (w & 1);
  f32x4 d[2][4];
  double acc[2][4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0;
    }
  auto flush = [&]() {  // the previous stage's partials into the fp64 sums
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] += (double)d[i][j][e];
  };
  auto compute = [&](int buf) {
    const uint8_t* at = lds + buf * SD_STAGE;
    const uint8_t* bt = at + SD_ASTG;
    flush();
#pragma unroll
    for (int kk = 0; kk < SD_BT / 32; ++kk) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = frag(at, SD_AROW, true, wr + 16 * i, kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = frag(bt, SD_BROW, false, wc + 16 * j, kk);
      __builtin_amdgcn_sched_barrier(0);  // every read of the step ahead of its products
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], kk ? d[i][j] : f32x4{0.f, 0.f, 0.f, 0.f},
                                                            0, 0, 0);
    }
  };

  // ring: stage c sits in buffer c % NS; NS - 1 stages are in flight ahead of the products
  constexpr int L = SD_LA + SD_LB;
#pragma unroll
  for (int c = 0; c < SD_NS - 1; ++c)
    if (c < nst) issue(c, c);
  for (int c = 0; c < nst; ++c) {
    if (c + 1 < nst) sd_wait_vm<L>();  // stage c + 1's transfers may still be in flight
    else sd_wait_vm<0>();
    ring_barrier();                    // every wave's stage c is in LDS; stage c - 1 is consumed
    if (c + SD_NS - 1 < nst) issue(c + SD_NS - 1, (c + SD_NS - 1) % SD_NS);
    compute(c % SD_NS);
  }
  flush();
  __syncthreads();  // the ring is free

  // dense block -> LDS: lane holds rows wr + 16 i + 4 q4 + e of column wc + 16 j + l16
  float* const ds = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ds[(wr + 16 * i + 4 * q4 + e) * SD_DLD + wc + 16 * j + l16] = (float)acc[i][j][e];
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
  // workgroup tiles of U x 256 consecutive chunks: the U loads of a wave read adjacent 1 KB runs;
  // every byte is read or written once, so the loads and stores are non-temporal
  const int64_t full = nch / (U * 256);
  for (int64_t tile = blockIdx.x; tile < full; tile += gridDim.x) {
    const int64_t i = tile * (U * 256) + threadIdx.x;
    u32x4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      va[u] = __builtin_nontemporal_load(pa + i + 256 * u);
      vb[u] = __builtin_nontemporal_load(pb + i + 256 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(combine(va[u], vb[u]), po + i + 256 * u);
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

bool sddmm24_fits(int64_t R, int64_t C, int64_t T) {
  return T * R * 2 < ((int64_t)1 << 31) && T * C * 2 < ((int64_t)1 << 31);
}

hipError_t launch_sddmm24_bf16(const uint16_t* row_act, const uint16_t* col_act, const uint32_t* meta,
                               uint32_t meta_or, int64_t R, int64_t C, int64_t T, uint16_t* out,
                               hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (R % 8 != 0 || C % 32 != 0) return hipErrorInvalidValue;
  if (!sddmm24_fits(R, C, T)) return hipErrorInvalidValue;  // 32-bit buffer offsets
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

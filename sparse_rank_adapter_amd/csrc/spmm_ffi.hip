// bf16 fixed fan-in SpMM with the low-rank epilogue (SQuAsh project update: fixed fan-in sparse
// weights, applied with the activations resident in LDS and a per-row loop over (index, value)
// pairs; SLoPe paperlayer summary §2.3 keeps the weight and its transpose).
//   forward  (ELL, rows = N):  Y[t][n]  = sum_j X[t][col(n,j)] val(n,j) + sum_j U[t][j] B[n][j]
//   backward (CSR, rows = K):  dX[t][k] = sum_e dY[t][row(e)] val(e)    + sum_j dU[t][j] A[j][k]
//
// With ~10% of the columns kept at arbitrary positions there is no dense sub-block for MFMA, and
// every product needs one activation value picked by the stored index: the kernel is bound by
// those picks (LDS) and by the VALU.  A workgroup owns 64 tokens (one per lane) and 64 sparse rows
// (16 per wave).  The activations of its tokens are staged in LDS one 256-column chunk at a time
// as [column][token], so the pick for a stored index is one 128-byte row read by the whole wave
// without bank conflicts; the LDS footprint stays small so that several workgroups share a CU.  A row's (index, value) pairs are fetched 64 at a time, one per lane,
// and broadcast with v_readlane; indices ascend within a row, so each row keeps a cursor into its
// list from chunk to chunk.  Accumulation is fp32; the adapter term is added in fp32 from the fp32
// U, and the output tile goes out through LDS as contiguous row segments of Y.
#include "common.h"

namespace {

constexpr int TT = 64;     // tokens per workgroup (one per lane)
constexpr int RPW = 16;    // sparse rows per wave
constexpr int RB = 4 * RPW;
constexpr int KC = 256;    // activation columns per LDS chunk (32 KB)

__global__ __launch_bounds__(256) void k_spmm_ffi(int format, const uint16_t* __restrict__ vals,
                                                  const int16_t* __restrict__ idx,
                                                  const int32_t* __restrict__ row_ptr, int k,
                                                  int64_t R, int64_t C,
                                                  const uint16_t* __restrict__ act, int64_t T,
                                                  sra::Epilogue ep, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[KC * TT];  // [column][token]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: row addresses go scalar
  const int64_t t0 = (int64_t)blockIdx.x * TT, rw0 = (int64_t)blockIdx.y * RB + w * RPW;
  const int64_t t = t0 + lane;
  const bool c_vec = (C & 7) == 0;

  // per-row state: running sums in registers (one per row and token), cursor and end of each row's
  // list (wave-uniform, so scalar registers); the row loop is unrolled
  float acc[RPW];
  int cur[RPW], fin[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int64_t row = rw0 + i;
    acc[i] = 0.f;
    int b = 0, e = 0;
    if (row < R) {
      if (format == SRA_FMT_ELL) {
        b = (int)(row * k);
        e = b + k;
      } else {
        b = row_ptr[row];
        e = row_ptr[row + 1];
      }
    }
    cur[i] = b;
    fin[i] = e;
  }

  for (int64_t c0 = 0; c0 < C; c0 += KC) {
    __syncthreads();  // the previous chunk has been consumed
    // stage X[t0 .. t0+63][c0 .. c0+KC) as xs[c][t]: lane -> (token, 8 consecutive columns);
    // consecutive lanes take consecutive tokens, so the transposing 2-byte LDS writes of a wave
    // fall on distinct banks
    for (int v = tid; v < TT * (KC / 8); v += 256) {
      const int tok = v % TT, cc = (v / TT) * 8;
      union { u32x4 v; uint16_t h[8]; } x;
      x.v = u32x4{0, 0, 0, 0};
      const int64_t tg = t0 + tok, cg = c0 + cc;
      if (tg < T && cg < C) {
        const uint16_t* p = act + tg * C + cg;
        if (c_vec && cg + 8 <= C) {
          x.v = *reinterpret_cast<const u32x4*>(p);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (cg + q < C) x.h[q] = p[q];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) xs[(cc + q) * TT + tok] = x.h[q];
    }
    __syncthreads();
    const int cend = (int)(C - c0 < KC ? C - c0 : KC);  // columns of this chunk
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      int e = cur[i];
      const int ee = fin[i];
      float a = acc[i];
      while (e < ee) {
        // pairs e .. e+63, one per lane: index in the low half, bf16 value in the high half
        const int ej = e + lane;
        const uint32_t pk = ej < ee ? (uint32_t)(uint16_t)idx[ej] | ((uint32_t)vals[ej] << 16) : 0u;
        const int n = ee - e < 64 ? ee - e : 64;
        int j = 0;
        // four pairs at a time while the fourth still lies in this chunk (indices ascend), so
        // four LDS picks are in flight together
        for (; j + 4 <= n; j += 4) {
          const uint32_t e3 = __builtin_amdgcn_readlane(pk, j + 3);
          if ((int)(e3 & 0xFFFFu) - (int)c0 >= cend) break;
          uint32_t en[4];
          en[0] = __builtin_amdgcn_readlane(pk, j);
          en[1] = __builtin_amdgcn_readlane(pk, j + 1);
          en[2] = __builtin_amdgcn_readlane(pk, j + 2);
          en[3] = e3;
          float x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = bf16_to_f32(xs[((int)(en[q] & 0xFFFFu) - (int)c0) * TT + lane]);
#pragma unroll
          for (int q = 0; q < 4; ++q) a += x[q] * __uint_as_float(en[q] & 0xFFFF0000u);
        }
        for (; j < n; ++j) {
          const uint32_t ent = __builtin_amdgcn_readlane(pk, j);
          const int col = (int)(ent & 0xFFFFu) - (int)c0;
          if (col >= cend) break;  // the rest of the row lies in later chunks
          a += bf16_to_f32(xs[col * TT + lane]) * __uint_as_float(ent & 0xFFFF0000u);
        }
        e += j;
        if (j < n) break;
      }
      acc[i] = a;
      cur[i] = e;
    }
  }

  // adapter term: acc[i] += sum_j U[t][j] E(row_i, j), two adapter columns at a time (E is read
  // as scalars: 2 x 16 per step)
  if (ep.r > 0) {
    const bool t_ok = t < T;
#pragma unroll 1
    for (int j0 = 0; j0 < ep.r; j0 += 2) {
      float u[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) u[q] = (t_ok && j0 + q < ep.r) ? ep.U[t * ep.r + j0 + q] : 0.f;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int64_t row = rw0 + i;
        if (row >= R) continue;
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (j0 + q < ep.r)
            acc[i] += u[q] * bf16_to_f32(ep.E[row * ep.e_row_stride + (int64_t)(j0 + q) * ep.e_j_stride]);
      }
    }
  }

  // store through LDS: tile [token][row] bf16, then each token's 64 rows as one 128-byte segment
  __syncthreads();
  uint16_t* ot = xs;  // [TT][RB + 8]
  constexpr int OLD = RB + 8;
#pragma unroll
  for (int i = 0; i < RPW; ++i) ot[lane * OLD + w * RPW + i] = f32_to_bf16(acc[i]);
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.y * RB;
  const bool r_vec = (R & 7) == 0;
  for (int v = tid; v < TT * (RB / 8); v += 256) {
    const int tok = v / (RB / 8), rr = (v % (RB / 8)) * 8;
    const int64_t tg = t0 + tok, row = r0 + rr;
    if (tg >= T || row >= R) continue;
    uint16_t* o = out + tg * R + row;
    const uint16_t* src = ot + tok * OLD + rr;
    if (r_vec && row + 8 <= R) {
      union { u32x4 v; uint16_t h[8]; } x;
#pragma unroll
      for (int q = 0; q < 8; ++q) x.h[q] = src[q];
      *reinterpret_cast<u32x4*>(o) = x.v;
    } else {
      for (int q = 0; q < 8 && row + q < R; ++q) o[q] = src[q];
    }
  }
}

// Densify one sparse row per workgroup: the row is cleared and its (index, value) pairs scattered
// in LDS, then written out as C contiguous bf16 (C % 8 == 0; indices within a row are distinct).
__global__ __launch_bounds__(256) void k_ffi_densify(int format, const uint16_t* __restrict__ vals,
                                                     const int16_t* __restrict__ idx,
                                                     const int32_t* __restrict__ row_ptr, int k,
                                                     int64_t C, uint16_t* __restrict__ Wd) {
  extern __shared__ __attribute__((aligned(16))) uint16_t rowbuf[];  // C elements
  const int64_t n = blockIdx.x;
  for (int64_t c = threadIdx.x * 8; c < C; c += 256 * 8)
    *reinterpret_cast<u32x4*>(&rowbuf[c]) = u32x4{0, 0, 0, 0};
  __syncthreads();
  const int64_t b = format == SRA_FMT_ELL ? n * k : row_ptr[n];
  const int64_t e = format == SRA_FMT_ELL ? b + k : row_ptr[n + 1];
  for (int64_t i = b + threadIdx.x; i < e; i += 256) rowbuf[idx[i]] = vals[i];
  __syncthreads();
  for (int64_t c = threadIdx.x * 8; c < C; c += 256 * 8)
    *reinterpret_cast<u32x4*>(&Wd[n * C + c]) = *reinterpret_cast<const u32x4*>(&rowbuf[c]);
}

// The stored entries of an ELL pattern read out of a dense fp32 matrix, one thread per entry.
__global__ __launch_bounds__(256) void k_ell_gather_f32(const float* __restrict__ dense,
                                                        const int16_t* __restrict__ idx, int k,
                                                        int64_t C, int64_t n, float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  out[e] = dense[(e / k) * C + idx[e]];
}

// The tiled product (matrix cores on a dense A tile written from the entries in LDS) pays one
// pass building the tiled format; worth it once the token tile is wide enough to reuse each weight
// row many times.
bool use_tiled(int64_t R, int64_t C, int64_t T) { return T >= 128 && C % 64 == 0 && R > 0; }

}  // namespace

namespace sra {

size_t spmm_ffi_ws(int64_t R, int64_t C, int64_t T, int64_t nnz) {
  if (!use_tiled(R, C, T)) return 0;
  size_t eb, ob;
  ffi_tile_bytes(R, C, nnz, &eb, &ob);
  return ((eb + 255) & ~(size_t)255) + ob;
}

hipError_t launch_ffi_densify(int format, const uint16_t* vals, const int16_t* idx,
                              const int32_t* row_ptr, int k, int64_t R, int64_t C, uint16_t* out,
                              hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  launch(SRA_KERNEL_FFI_DENSIFY, k_ffi_densify, dim3((unsigned)R), dim3(256), (size_t)C * 2, s,
         format, vals, idx, row_ptr, k, C, out);
  return hipGetLastError();
}

hipError_t launch_ell_gather_f32(const float* dense, const int16_t* idx, int k, int64_t R, int64_t C,
                                 float* out, hipStream_t s) {
  const int64_t n = R * k;
  if (n == 0) return hipSuccess;
  launch(0, k_ell_gather_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dense, idx, k, C,
         n, out);
  return hipGetLastError();
}

hipError_t launch_spmm_ffi_bf16(int format, const uint16_t* vals, const int16_t* idx,
                                const int32_t* row_ptr, int k, int64_t R, int64_t C,
                                const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                                void* ws, hipStream_t s, int64_t nnz) {
  if (T == 0 || R == 0) return hipSuccess;
  if (use_tiled(R, C, T)) {
    if (!ws) return hipErrorInvalidValue;
    size_t eb, ob;
    ffi_tile_bytes(R, C, nnz, &eb, &ob);
    uint32_t* ent = (uint32_t*)ws;
    uint32_t* offs = (uint32_t*)((char*)ws + ((eb + 255) & ~(size_t)255));
    hipError_t e = launch_ffi_tile(vals, idx, format == SRA_FMT_ELL ? nullptr : row_ptr, k, R, C, ent, offs,
                                   (int64_t)(eb / 4), s);
    if (e != hipSuccess) return e;
    return launch_ffi_tiled_bf16(ent, offs, eb, R, C, act, T, ep, out, s);
  }
  const dim3 grid((unsigned)((T + TT - 1) / TT), (unsigned)((R + RB - 1) / RB));
  launch(SRA_KERNEL_SPMM_FFI, k_spmm_ffi, grid, dim3(256), 0, s, format, vals, idx, row_ptr, k, R,
         C, act, T, ep, out);
  return hipGetLastError();
}

}  // namespace sra

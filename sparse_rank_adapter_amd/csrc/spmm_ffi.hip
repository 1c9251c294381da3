// bf16 fixed fan-in SpMM with the low-rank epilogue (SQuAsh project update: fixed fan-in sparse
// weights; SLoPe paperlayer summary §2.3 keeps the weight and its transpose).
//   forward  (ELL, rows = N):  Y[t][n]  = sum_j X[t][col(n,j)] val(n,j) + sum_j U[t][j] B[n][j]
//   backward (CSR, rows = K):  dX[t][k] = sum_e dY[t][row(e)] val(e)    + sum_j dU[t][j] A[j][k]
// Gather form: one lane per output element, fp32 accumulation.
#include "common.h"

namespace {

__global__ __launch_bounds__(256) void k_spmm_ffi_gather(int format, const uint16_t* __restrict__ vals,
                                                         const int16_t* __restrict__ idx,
                                                         const int32_t* __restrict__ row_ptr, int k,
                                                         int64_t R, int64_t C,
                                                         const uint16_t* __restrict__ act, int64_t T,
                                                         sra::Epilogue ep, uint16_t* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= T * R) return;
  const int64_t t = id / R, row = id - t * R;
  const uint16_t* a = act + t * C;
  float acc = 0.f;
  int64_t b, e;
  if (format == SRA_FMT_ELL) {
    b = row * k;
    e = b + k;
  } else {
    b = row_ptr[row];
    e = row_ptr[row + 1];
  }
  for (int64_t q = b; q < e; ++q) acc += bf16_to_f32(a[idx[q]]) * bf16_to_f32(vals[q]);
  for (int j = 0; j < ep.r; ++j)
    acc += ep.U[t * ep.r + j] * bf16_to_f32(ep.E[row * ep.e_row_stride + (int64_t)j * ep.e_j_stride]);
  out[id] = f32_to_bf16(acc);
}

}  // namespace

namespace sra {

hipError_t launch_spmm_ffi_bf16(int format, const uint16_t* vals, const int16_t* idx,
                                const int32_t* row_ptr, int k, int64_t R, int64_t C,
                                const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                                hipStream_t s) {
  const int64_t n = T * R;
  if (n == 0) return hipSuccess;
  launch(SRA_KERNEL_SPMM_FFI, k_spmm_ffi_gather, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, format,
                     vals, idx, row_ptr, k, R, C, act, T, ep, out);
  return hipGetLastError();
}

}  // namespace sra

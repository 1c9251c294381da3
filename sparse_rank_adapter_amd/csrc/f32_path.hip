// fp32 layer path: every output element accumulates in fp64 and is rounded once to fp32, and the
// adapter intermediates U and dU stay fp64 between kernels (only their optional fp32 outputs are
// rounded).  This path exists for fp32 weights, where an fp32 accumulator -- or one fp32 rounding
// of U reused across all tokens -- can exceed a 1e-5 relative budget near zero; it favours
// exactness over speed (one lane per output).
#include "common.h"

namespace {

// Visits the (column, value) pairs of one sparse row in ascending column order.
template <typename F>
SRA_DEV void for_row(const sra::F32Sparse& S, int64_t row, F&& f) {
  if (S.format == SRA_FMT_NM) {
    const int64_t nv = S.cols / 2;
    const uint32_t* mrow = S.meta + row * S.meta_stride;
    const uint32_t* vrow = S.vals + row * nv;
    for (int64_t w = 0; w < S.meta_stride; ++w) {
      const uint32_t bits = mrow[w];
      for (int fi = 0; fi < 16; ++fi) {
        const int64_t field = w * 16 + fi;
        if (field >= nv) break;
        const int64_t c = (field >> 1) * 4 + ((bits >> (2 * fi)) & 3u);
        f(c, (double)__uint_as_float(vrow[field]));
      }
    }
  } else if (S.format == SRA_FMT_ELL) {
    const int16_t* irow = S.idx + row * S.k;
    const uint32_t* vrow = S.vals + row * S.k;
    for (int j = 0; j < S.k; ++j) f((int64_t)irow[j], (double)__uint_as_float(vrow[j]));
  } else {
    for (int64_t e = S.row_ptr[row]; e < S.row_ptr[row + 1]; ++e)
      f((int64_t)S.idx[e], (double)__uint_as_float(S.vals[e]));
  }
}

// U64 = X A^T in fp64 (kept unrounded for reuse); U32 (optional) receives it rounded to fp32.
__global__ void k_f32_u(const float* __restrict__ X, const float* __restrict__ A, int64_t T,
                        int64_t K, int r, double* __restrict__ U64, float* __restrict__ U32) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= T * r) return;
  const int64_t t = id / r, j = id - t * r;
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) acc += (double)X[t * K + k] * (double)A[j * K + k];
  U64[id] = acc;
  if (U32) U32[id] = (float)acc;
}

// Out[t][row] = sum_c Act[t][c] S[row][c] + sum_j U64[t][j] E(row, j)
__global__ void k_f32_spmm(sra::F32Sparse S, const float* __restrict__ Act, int64_t T,
                           const double* __restrict__ U64, const float* __restrict__ E,
                           int64_t e_rs, int64_t e_js, int r, float* __restrict__ Out) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= T * S.rows) return;
  const int64_t t = id / S.rows, row = id - t * S.rows;
  const float* a = Act + t * S.cols;
  double acc = 0.0;
  for_row(S, row, [&](int64_t c, double v) { acc += (double)a[c] * v; });
  for (int j = 0; j < r; ++j) acc += U64[t * r + j] * (double)E[row * e_rs + j * e_js];
  Out[id] = (float)acc;
}

__global__ void k_f32_du(const float* __restrict__ dY, const float* __restrict__ B, int64_t T,
                         int64_t N, int r, double* __restrict__ dU64, float* __restrict__ dU32) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= T * r) return;
  const int64_t t = id / r, j = id - t * r;
  double acc = 0.0;
  for (int64_t n = 0; n < N; ++n) acc += (double)dY[t * N + n] * (double)B[n * r + j];
  dU64[id] = acc;
  if (dU32) dU32[id] = (float)acc;
}

// Out[m][n] = sum_t P[t][m] Q[t][n]; each operand is fp32 (*f) or fp64 (*d), whichever is set.
__global__ void k_f32_tn(const float* __restrict__ Pf, const double* __restrict__ Pd, int64_t ldp,
                         const float* __restrict__ Qf, const double* __restrict__ Qd, int64_t ldq,
                         int64_t T, int64_t M, int64_t Nn, float* __restrict__ Out) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= M * Nn) return;
  const int64_t m = id / Nn, n = id - m * Nn;
  double acc = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const double p = Pd ? Pd[t * ldp + m] : (double)Pf[t * ldp + m];
    const double q = Qd ? Qd[t * ldq + n] : (double)Qf[t * ldq + n];
    acc += p * q;
  }
  Out[id] = (float)acc;
}

__global__ void k_fill_f32(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

inline dim3 grid_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

}  // namespace

namespace sra {

hipError_t launch_f32_adapter_u(const float* X, const float* A, int64_t T, int64_t K, int r,
                                double* U64, float* U32, hipStream_t s) {
  if (T * r == 0) return hipSuccess;
  hipLaunchKernelGGL(k_f32_u, grid_for(T * r), dim3(256), 0, s, X, A, T, K, r, U64, U32);
  return hipGetLastError();
}

hipError_t launch_f32_spmm(const F32Sparse& S, const float* Act, int64_t T, const double* U64,
                           const float* E, int64_t e_row_stride, int64_t e_j_stride, int r,
                           float* Out, hipStream_t s) {
  if (T * S.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_f32_spmm, grid_for(T * S.rows), dim3(256), 0, s, S, Act, T, U64, E,
                     e_row_stride, e_j_stride, r, Out);
  return hipGetLastError();
}

hipError_t launch_f32_du(const float* dY, const float* B, int64_t T, int64_t N, int r,
                         double* dU64, float* dU32, hipStream_t s) {
  if (T * r == 0) return hipSuccess;
  hipLaunchKernelGGL(k_f32_du, grid_for(T * r), dim3(256), 0, s, dY, B, T, N, r, dU64, dU32);
  return hipGetLastError();
}

hipError_t launch_f32_tn(const float* Pf, const double* Pd, int64_t ldp, const float* Qf,
                         const double* Qd, int64_t ldq, int64_t T, int64_t M, int64_t Nn,
                         float* Out, hipStream_t s) {
  if (M * Nn == 0) return hipSuccess;
  hipLaunchKernelGGL(k_f32_tn, grid_for(M * Nn), dim3(256), 0, s, Pf, Pd, ldp, Qf, Qd, ldq, T, M,
                     Nn, Out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, grid_for(n), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace sra

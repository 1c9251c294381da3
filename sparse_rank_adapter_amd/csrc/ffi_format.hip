// Fixed fan-in format: per-row top-k selection and the exact transpose.
// (SQuAsh project update: fixed fan-in keeps the same number of inputs for every output row;
//  SLoPe paperlayer summary §2.3: formats are kept for a weight and for its transpose.)
//
// compress_ffi: one workgroup per row.  The k-th largest magnitude key is found by an MSD radix
// select over 8-bit digits (2 passes for bf16, 4 for fp32) with LDS histograms; the kept set is
// then every key above the threshold plus the lowest-column entries equal to it, written in
// column order by two block-wide scans (equal-key ranks, then output slots).
//
// ffi_transpose: rows are cut into 64-row chunks.  Counting per (chunk, column) and a scan over
// chunks give every chunk a private output cursor per column; a chunk's rows are then scattered
// in row order by one workgroup, so CSR rows come out sorted by original row without a sort.
#include "common.h"

namespace {

constexpr int kChunkRows = 64;

// Block-wide exclusive scan over 256 lanes.  Returns the exclusive prefix; *total gets the sum.
SRA_DEV uint32_t block_exclusive_scan256(uint32_t v, uint32_t* sm, uint32_t* total) {
  const int tid = threadIdx.x;
  sm[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = tid >= off ? sm[tid - off] : 0u;
    __syncthreads();
    sm[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = sm[tid];
  *total = sm[255];
  __syncthreads();
  return incl - v;
}

template <typename T>
__global__ __launch_bounds__(256) void k_compress_ffi(const T* __restrict__ W, int cols, int k,
                                                      T* __restrict__ vals,
                                                      int16_t* __restrict__ idx) {
  constexpr int KEYBITS = sizeof(T) == 2 ? 16 : 32;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_sm[256];
  __shared__ uint32_t s_digit, s_need;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const T* w = W + row * (int64_t)cols;

  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  for (int shift = KEYBITS - 8; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cols; i += 256) {
      const uint32_t key = mag_key(w[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t acc = 0;
      int v = 255;
      for (; v > 0; --v) {
        if (acc + hist[v] >= need) break;
        acc += hist[v];
      }
      s_digit = (uint32_t)v;
      s_need = need - acc;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    need = s_need;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // the k-th largest key; `need` entries equal to it are kept

  const int seg = (cols + 255) / 256;
  const int beg = min(cols, tid * seg), end = min(cols, beg + seg);
  uint32_t n_eq = 0;
  for (int i = beg; i < end; ++i) n_eq += mag_key(w[i]) == tau;
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan256(n_eq, scan_sm, &tot);
  uint32_t n_sel = 0, e = eq_before;
  for (int i = beg; i < end; ++i) {
    const uint32_t key = mag_key(w[i]);
    if (key > tau) ++n_sel;
    else if (key == tau) n_sel += (e++ < need);
  }
  uint32_t pos = block_exclusive_scan256(n_sel, scan_sm, &tot);
  e = eq_before;
  T* vo = vals + row * (int64_t)k;
  int16_t* io = idx + row * (int64_t)k;
  for (int i = beg; i < end; ++i) {
    const T x = w[i];
    const uint32_t key = mag_key(x);
    bool take = key > tau;
    if (key == tau) take = (e++ < need);
    if (take && pos < (uint32_t)k) {  // the select guarantees exactly k; the guard keeps writes in bounds
      vo[pos] = x;
      io[pos] = (int16_t)i;
      ++pos;
    }
  }
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_ffi_count(const int16_t* __restrict__ idx, int64_t entries, int k, int cols,
                            int32_t* __restrict__ counts) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= entries) return;
  const int64_t row = e / k;
  atomicAdd(&counts[(row / kChunkRows) * cols + idx[e]], 1);
}

// per column: exclusive prefix over chunks (in place) and the column total into row_ptr[c + 1]
__global__ void k_ffi_colscan(int32_t* __restrict__ counts, int n_chunks, int cols,
                              int32_t* __restrict__ row_ptr) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c > cols) return;
  if (c == cols) {
    row_ptr[0] = 0;
    return;
  }
  int32_t run = 0;
  for (int ch = 0; ch < n_chunks; ++ch) {
    const int32_t v = counts[(int64_t)ch * cols + c];
    counts[(int64_t)ch * cols + c] = run;
    run += v;
  }
  row_ptr[c + 1] = run;
}

// inclusive scan of row_ptr[1..cols] in place (single workgroup of 256 lanes)
__global__ __launch_bounds__(256) void k_ffi_rowptr_scan(int32_t* __restrict__ row_ptr, int cols) {
  __shared__ uint32_t sm[256];
  const int tid = threadIdx.x;
  const int seg = (cols + 255) / 256;
  const int beg = min(cols, tid * seg), end = min(cols, beg + seg);
  uint32_t s = 0;
  for (int i = beg; i < end; ++i) s += (uint32_t)row_ptr[1 + i];
  uint32_t tot;
  uint32_t run = block_exclusive_scan256(s, sm, &tot);
  for (int i = beg; i < end; ++i) {
    run += (uint32_t)row_ptr[1 + i];
    row_ptr[1 + i] = (int32_t)run;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_ffi_scatter(const T* __restrict__ vals,
                                                     const int16_t* __restrict__ idx, int64_t rows,
                                                     int cols, int k,
                                                     const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ row_ptr,
                                                     int16_t* __restrict__ t_idx,
                                                     T* __restrict__ t_vals, int64_t nnz) {
  extern __shared__ uint16_t run[];  // per-column cursor inside this chunk (<= 64)
  const int tid = threadIdx.x;
  const int64_t ch = blockIdx.x;
  for (int c = tid; c < cols; c += 256) run[c] = 0;
  __syncthreads();
  const int32_t* base = counts + ch * cols;
  const int64_t r_end = min(rows, (ch + 1) * kChunkRows);
  for (int64_t row = ch * kChunkRows; row < r_end; ++row) {
    for (int j = tid; j < k; j += 256) {
      const int64_t e = row * k + j;
      const int c = idx[e];
      const int64_t pos = (int64_t)row_ptr[c] + base[c] + run[c];
      run[c] += 1;  // columns of one row are distinct: no two lanes share c
      if (pos < nnz) {
        t_idx[pos] = (int16_t)row;
        t_vals[pos] = vals[e];
      }
    }
    __syncthreads();
  }
}

}  // namespace

namespace sra {

hipError_t launch_compress_ffi(int dtype, const void* W, int64_t rows, int64_t cols, int k,
                               void* vals, int16_t* idx, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype == SRA_BF16)
    hipLaunchKernelGGL(k_compress_ffi<uint16_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       (const uint16_t*)W, (int)cols, k, (uint16_t*)vals, idx);
  else
    hipLaunchKernelGGL(k_compress_ffi<uint32_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       (const uint32_t*)W, (int)cols, k, (uint32_t*)vals, idx);
  return hipGetLastError();
}

size_t ffi_transpose_ws(int64_t rows, int64_t cols) {
  const int64_t n_chunks = (rows + kChunkRows - 1) / kChunkRows;
  return (size_t)(n_chunks * cols * sizeof(int32_t) + 256);
}

hipError_t launch_ffi_transpose(int dtype, const void* vals, const int16_t* idx, int64_t rows,
                                int64_t cols, int k, int32_t* row_ptr, int16_t* t_idx,
                                void* t_vals, void* ws, hipStream_t s) {
  const int64_t n_chunks = (rows + kChunkRows - 1) / kChunkRows;
  int32_t* counts = (int32_t*)ws;
  const int64_t nc = n_chunks * cols;
  if (nc > 0)
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, counts,
                       nc, 0);
  const int64_t entries = rows * k;
  if (entries > 0)
    hipLaunchKernelGGL(k_ffi_count, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, s, idx,
                       entries, k, (int)cols, counts);
  hipLaunchKernelGGL(k_ffi_colscan, dim3((unsigned)((cols + 1 + 255) / 256)), dim3(256), 0, s,
                     counts, (int)n_chunks, (int)cols, row_ptr);
  hipLaunchKernelGGL(k_ffi_rowptr_scan, dim3(1), dim3(256), 0, s, row_ptr, (int)cols);
  if (n_chunks > 0) {
    const size_t lds = (size_t)cols * sizeof(uint16_t);
    if (dtype == SRA_BF16)
      hipLaunchKernelGGL(k_ffi_scatter<uint16_t>, dim3((unsigned)n_chunks), dim3(256), lds, s,
                         (const uint16_t*)vals, idx, rows, (int)cols, k, counts, row_ptr, t_idx,
                         (uint16_t*)t_vals, entries);
    else
      hipLaunchKernelGGL(k_ffi_scatter<uint32_t>, dim3((unsigned)n_chunks), dim3(256), lds, s,
                         (const uint32_t*)vals, idx, rows, (int)cols, k, counts, row_ptr, t_idx,
                         (uint32_t*)t_vals, entries);
  }
  return hipGetLastError();
}

}  // namespace sra

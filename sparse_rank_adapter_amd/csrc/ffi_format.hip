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
//
// ffi_tile: the product's layout of an ELL or CSR matrix.  Rows are cut into 32-row groups and
// columns into 64-column stages; list (group g, stage x) holds the group's entries in that stage
// as 32-bit words, ordered by row and then column, padded to a multiple of four words with
// 0xffffffff.  A word holds the bf16 value in the low half and, in the high half, the entry's
// byte offset in the group's 32 rows of 64 bf16 as the products lay them out in LDS: with
// i = row - 32 g and c = column - 64 x, i * 128 + ((c / 8) ^ ((i / 2) % 8)) * 16 + (c % 8) * 2.
// Lists follow each other group by group, stage by stage; offsets[g * stages + x] is the first
// word of list (g, x), and the word count plus three more copies of it close the array.  Counting
// per list, one scan over the lists, then per group a count per (row, stage) turns into each
// entry's rank: the entries of earlier rows in the same stage plus the entry's place in its row's
// run of that stage (a row's columns ascend, so a stage's entries are one run of the row).
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

// list sizes of one 32-row group, padded to whole 16-byte words (row_ptr == nullptr: ELL)
__global__ __launch_bounds__(256) void k_ffi_tile_count(const int16_t* __restrict__ idx,
                                                        const int32_t* __restrict__ row_ptr, int k,
                                                        int64_t R, int nst, uint32_t* __restrict__ offs) {
  extern __shared__ uint32_t cnt[];  // nst
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x, r0 = g * 32, r1 = min(R, r0 + 32);
  for (int x = tid; x < nst; x += 256) cnt[x] = 0;
  __syncthreads();
  const int64_t b = row_ptr ? row_ptr[r0] : r0 * k, e = row_ptr ? row_ptr[r1] : r1 * k;
#pragma unroll 4
  for (int64_t i = b + tid; i < e; i += 256) atomicAdd(&cnt[idx[i] >> 6], 1u);
  __syncthreads();
  for (int x = tid; x < nst; x += 256) offs[g * nst + x] = (cnt[x] + 3u) & ~3u;
}

// exclusive scan of the n list sizes in place; the total goes to offs[n .. n+3]
__global__ __launch_bounds__(1024) void k_ffi_tile_scan(uint32_t* __restrict__ offs, int64_t n) {
  __shared__ uint32_t sm[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024, b = min(n, tid * per), e = min(n, b + per);
  uint32_t sum = 0;
  for (int64_t i = b; i < e; ++i) sum += offs[i];
  sm[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint32_t add = tid >= off ? sm[tid - off] : 0u;
    __syncthreads();
    sm[tid] += add;
    __syncthreads();
  }
  uint32_t run = sm[tid] - sum;
  const uint32_t total = sm[1023];
  for (int64_t i = b; i < e; ++i) {
    const uint32_t v = offs[i];
    offs[i] = run;
    run += v;
  }
  if (tid < 4) offs[n + tid] = total;
}

// one 32-row group: every entry written at its list's offset plus its rank, then the padding
__global__ __launch_bounds__(256) void k_ffi_tile_fill(const uint16_t* __restrict__ vals,
                                                       const int16_t* __restrict__ idx,
                                                       const int32_t* __restrict__ row_ptr, int k,
                                                       int64_t R, int nst, const uint32_t* __restrict__ offs,
                                                       uint32_t* __restrict__ ent, int64_t cap) {
  extern __shared__ uint32_t sm[];
  // per half group of 16 rows: cnt[i][x] (entries of row i in stage x, then the entries of the
  // group's earlier rows in stage x), pre[i][x] (entries of row i in earlier stages), both 16-bit;
  // run[x] (entries of the group's rows so far in stage x), base[x] (list offset), part[256]
  uint32_t* cntw = sm;
  uint16_t* cnt = reinterpret_cast<uint16_t*>(cntw);
  uint16_t* pre = cnt + 16 * nst;
  uint32_t* run = sm + 16 * nst;
  uint32_t* base = run + nst;
  uint32_t* part = base + nst;
  __shared__ int64_t rowb[17];  // the half group's row starts (entry indices) and its end
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  for (int x = tid; x < nst; x += 256) {
    run[x] = 0;
    base[x] = offs[g * nst + x];
  }
  auto row_beg = [&](int64_t row) -> int64_t { return row_ptr ? row_ptr[row] : row * k; };
  // the row of an entry of the half group: the last row start at or before it (16 rows, 4 steps)
  auto row_of = [&](int64_t q) {
    int lo = 0;
#pragma unroll
    for (int step = 8; step >= 1; step >>= 1)
      if (rowb[lo + step] <= q) lo += step;
    return lo;
  };
  for (int h = 0; h < 2; ++h) {
    const int64_t r0 = g * 32 + 16 * h;
    for (int w = tid; w < 8 * nst; w += 256) cntw[w] = 0;
    if (tid <= 16) rowb[tid] = row_beg(min(r0 + tid, R));
    __syncthreads();
    // every entry of the half group's 16 rows in one pass (their entries are contiguous)
    const int64_t hb = rowb[0], he = rowb[16];
#pragma unroll 4
    for (int64_t q = hb + tid; q < he; q += 256) {
      const int j = row_of(q) * nst + (idx[q] >> 6);
      atomicAdd(&cntw[j >> 1], 1u << (16 * (j & 1)));  // counts stay <= 64: no carry between halves
    }
    __syncthreads();
    // pre: per row, an exclusive scan over the stages (16 lanes per row, each a run of stages)
    {
      const int i = tid >> 4, p = tid & 15, seg = (nst + 15) / 16;
      const int xb = min(nst, p * seg), xe = min(nst, xb + seg);
      uint32_t sum = 0;
      for (int x = xb; x < xe; ++x) sum += cnt[i * nst + x];
      part[tid] = sum;
      __syncthreads();
      uint32_t acc = 0;
      for (int q = 0; q < p; ++q) acc += part[i * 16 + q];
      for (int x = xb; x < xe; ++x) {
        pre[i * nst + x] = (uint16_t)acc;
        acc += cnt[i * nst + x];
      }
    }
    __syncthreads();
    // cnt -> entries of the group's earlier rows in the stage
    for (int x = tid; x < nst; x += 256) {
      uint32_t r = run[x];
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = cnt[i * nst + x];
        cnt[i * nst + x] = (uint16_t)r;
        r += c;
      }
      run[x] = r;
    }
    __syncthreads();
#pragma unroll 4
    for (int64_t q = hb + tid; q < he; q += 256) {
      {
        const int i = row_of(q);
        const int64_t b = rowb[i];
        const int col = idx[q], x = col >> 6;
        const uint32_t pos = base[x] + cnt[i * nst + x] + ((uint32_t)(q - b) - pre[i * nst + x]);
        const int row = 16 * h + i, cc = col & 63;
        const uint32_t off = (uint32_t)(row * 128 + (((cc >> 3) ^ ((row >> 1) & 7)) << 4) + (cc & 7) * 2);
        if (pos < cap) ent[pos] = (uint32_t)vals[q] | (off << 16);
      }
    }
    __syncthreads();
  }
  for (int x = tid; x < nst; x += 256) {
    const uint32_t end = (uint32_t)min((int64_t)offs[g * nst + x + 1], cap);
    for (uint32_t q = base[x] + run[x]; q < end; ++q) ent[q] = 0xffffffffu;
  }
}

}  // namespace

namespace sra {

void ffi_tile_bytes(int64_t R, int64_t C, int64_t nnz, size_t* ent_bytes, size_t* off_bytes) {
  const int64_t lists = ((R + 31) / 32) * ((C + 63) / 64);
  *ent_bytes = (size_t)(nnz + 3 * lists) * 4;
  *off_bytes = (size_t)(lists + 4) * 4;
}

hipError_t launch_ffi_tile(const uint16_t* vals, const int16_t* idx, const int32_t* row_ptr, int k,
                           int64_t R, int64_t C, uint32_t* ent, uint32_t* offs, int64_t cap, hipStream_t s) {
  const int64_t groups = (R + 31) / 32, nst = (C + 63) / 64, lists = groups * nst;
  if (lists > 0)
    hipLaunchKernelGGL(k_ffi_tile_count, dim3((unsigned)groups), dim3(256), (size_t)nst * 4, s, idx,
                       row_ptr, k, R, (int)nst, offs);
  hipLaunchKernelGGL(k_ffi_tile_scan, dim3(1), dim3(1024), 0, s, offs, lists);
  if (lists > 0)
    hipLaunchKernelGGL(k_ffi_tile_fill, dim3((unsigned)groups), dim3(256), (size_t)(18 * nst + 256) * 4, s,
                       vals, idx, row_ptr, k, R, (int)nst, offs, ent, cap);
  return hipGetLastError();
}

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

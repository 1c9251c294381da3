// Internal helpers shared by the HIP sources of libsra (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sra.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SRA_DEV __device__ __forceinline__

// ---- bf16 bit helpers (values travel as raw uint16_t; arithmetic is fp32 or wider)
SRA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// round-to-nearest-even fp32 -> bf16 (inputs are finite)
SRA_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
SRA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---- N:M fragments expanded to dense bf16 (zeros at the pruned positions) for dense MFMA.  A group's
// kept values sit in one 32-bit word as (first, second) bf16, at ascending in-group positions
// f_a < f_b.  Per group a code byte per position marks which value goes there (2: the first, 4:
// the second, 0: none); each dense output word (positions 2k, 2k + 1) then takes three byte
// permutes: the code bytes spread to [c, c + 1, c', c' + 1], those index a table of byte selects
// (0x0C gives a zero byte), and the selects gather the value bytes.

// one dense word from the code bytes x (spread: the permute that picks its two code bytes twice),
// the select table {thi, tlo} and the value words {hi, lo}
SRA_DEV uint32_t dense_word(uint32_t x, uint32_t spread, uint32_t tlo, uint32_t thi, uint32_t hi, uint32_t lo) {
  const uint32_t idx = __builtin_amdgcn_perm(x, x, spread) | 0x01000100u;
  return __builtin_amdgcn_perm(hi, lo, __builtin_amdgcn_perm(thi, tlo, idx));
}

// 2:4: values (v0, v1) of group 0 in s01 and (v2, v3) of group 1 in s23, positions in m (2 bits
// each, least significant first: v0, v1, v2, v3) -> the groups' 8 dense columns
SRA_DEV bf16x8 expand24(uint32_t s01, uint32_t s23, uint32_t m) {
  const uint32_t x0 = (2u << ((m & 3u) << 3)) | (4u << (((m >> 2) & 3u) << 3));
  const uint32_t x1 = (2u << (((m >> 4) & 3u) << 3)) | (4u << (((m >> 6) & 3u) << 3));
  union { u32x4 v; bf16x8 b; } d;
  // group 0's values are bytes 0-3 of {s23, s01}, group 1's bytes 4-7
  d.v[0] = dense_word(x0, 0x01010000u, 0x01000C0Cu, 0x00000302u, s23, s01);
  d.v[1] = dense_word(x0, 0x03030202u, 0x01000C0Cu, 0x00000302u, s23, s01);
  d.v[2] = dense_word(x1, 0x01010000u, 0x05040C0Cu, 0x00000706u, s23, s01);
  d.v[3] = dense_word(x1, 0x03030202u, 0x05040C0Cu, 0x00000706u, s23, s01);
  return d.b;
}

// 2:8: the group's two values in s, positions in m (3 bits each: first at bits 0-2, second at 3-5)
// -> its 8 dense columns.  Each value moves to its position inside the 64-bit half that holds it
// (a shift by 16 (f % 4) bits) and lands in the low (f < 4) or the high half, selected by masks
// sign-extended from bit 2 of each position: about 19 instructions per group, 30% fewer than
// byte permutes with computed selectors.
SRA_DEV bf16x8 expand28(uint32_t s, uint32_t m) {
  // all ones when the first / second position is 4-7 (bits 2 and 5 of m, sign-extended)
  const uint32_t ha = (uint32_t)((int32_t)(m << 29) >> 31), hb = (uint32_t)((int32_t)(m << 26) >> 31);
  const uint64_t va = (uint64_t)(s & 0xFFFFu) << ((m & 3u) << 4);
  const uint64_t vb = (uint64_t)(s >> 16) << (((m >> 3) & 3u) << 4);
  const uint32_t a0 = (uint32_t)va, a1 = (uint32_t)(va >> 32), b0 = (uint32_t)vb, b1 = (uint32_t)(vb >> 32);
  union { u32x4 v; bf16x8 b; } d;
  d.v[0] = (a0 & ~ha) | (b0 & ~hb);  // positions 0-3
  d.v[1] = (a1 & ~ha) | (b1 & ~hb);
  d.v[2] = (a0 & ha) | (b0 & hb);    // positions 4-7
  d.v[3] = (a1 & ha) | (b1 & hb);
  return d.b;
}

// Magnitude key: the value's bits with the sign cleared, compared as an unsigned integer.
// For finite IEEE values this orders by |w| exactly, with +0 == -0.
SRA_DEV uint32_t mag_key(uint16_t b) { return (uint32_t)(b & 0x7FFFu); }
SRA_DEV uint32_t mag_key(uint32_t b) { return b & 0x7FFFFFFFu; }

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static SRA_DEV double to_f64(uint16_t b) { return (double)bf16_to_f32(b); } };
template <> struct Elem<uint32_t> { static SRA_DEV double to_f64(uint32_t b) { return (double)__uint_as_float(b); } };

SRA_DEV double load_f64(const uint16_t* p, int64_t i) { return (double)bf16_to_f32(p[i]); }
SRA_DEV double load_f64(const uint32_t* p, int64_t i) { return (double)__uint_as_float(p[i]); }

// Split an fp32 value into bf16 hi + lo with x ~= hi + lo (|x - hi - lo| <= 2^-17 |x|).
SRA_DEV void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}
// Three-way split x ~= hi + mid + lo (|x - hi - mid - lo| <= 2^-26 |x|, below fp32 rounding);
// each difference is exact in fp32.
SRA_DEV void split3_bf16(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(x);
  const float r1 = x - bf16_to_f32(hi);
  mid = f32_to_bf16(r1);
  lo = f32_to_bf16(r1 - bf16_to_f32(mid));
}
// V^T in three bf16 parts, vt[p][j][t] (rp rows per part, Tp columns), the operand layout of the
// adapter-gradient kernel: v (an fp64 sum) is rounded once to fp32, the value the call returns,
// and split exactly (hi + mid + lo carry all 24 bits of the fp32 significand).
SRA_DEV void write_vt3(uint16_t* __restrict__ vt, int rp, int64_t Tp, int j, int64_t t, double v) {
  uint16_t p3[3];
  split3_bf16((float)v, p3[0], p3[1], p3[2]);
#pragma unroll
  for (int p = 0; p < 3; ++p) vt[((int64_t)p * rp + j) * Tp + t] = p3[p];
}

// Workgroup barrier of the LDS-DMA rings: a bare s_barrier (no memory fence, so it does not wait
// for the transfers still in flight), fenced for the compiler's scheduler on both sides, so that
// no LDS read of the next stage is hoisted above it (nor one of the previous stage sunk below it).
SRA_DEV void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// ---- host-side launchers implemented in the kernel sources (internal C++ linkage)
namespace sra {

// Tuning knobs of the calling thread (sra_set_tuning); zero / default values mean the planners'
// own choices.
struct Tuning {
  int spmm_cfg = 0;     // forced 2:4 SpMM configuration id (T > 16)
  int spmm_splits = 0;  // its reduction splits; -2 = tail split in two
  int spmm_fuse = 1;    // in-kernel U / dU allowed
  int engine = 0;       // SRA_ENGINE_SMFMAC or SRA_ENGINE_DENSE_MFMA
  int decode_rows = 0;  // decode row tiles per workgroup (3, 4 or 9)
  int rows_slices = 0;  // reduction slices of the rank > 32 rows kernel
  int grads_slices = 0; // token slices of the adapter gradient kernel
};
const Tuning& tuning();

// Profiling hook (sra_time_next_kernel): returns true, and the events, exactly once after the
// calling thread armed kernel class `which`.
bool take_timing(int which, hipEvent_t* start, hipEvent_t* stop);

// Launch through hipExtLaunchKernelGGL with the armed events when this kernel class is armed.
template <typename K, typename... Args>
inline void launch(int which, K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                   Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (take_timing(which, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

hipError_t launch_compress24(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                             uint32_t* meta, hipStream_t s);
hipError_t launch_compress_pair24(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                                  uint32_t* meta, void* p_vals, uint32_t* p_meta, hipStream_t s);
// Out[row][i] = sum_t row_act[t][row] col_act[t][c_i(row)] over the stored slots of a 2:4 matrix
// (canonical metadata), bf16 out; R % 8 == 0, C % 32 == 0
// (meta_or = 0x88888888 reads 1:2 metadata as its 2:4 encoding); needs T*R and T*C below 2^30
bool sddmm24_fits(int64_t R, int64_t C, int64_t T);
hipError_t launch_sddmm24_bf16(const uint16_t* row_act, const uint16_t* col_act, const uint32_t* meta,
                               uint32_t meta_or, int64_t R, int64_t C, int64_t T, uint16_t* out,
                               hipStream_t s);
// out = beta a + gamma b over n values (bf16 or fp32), out may alias a
hipError_t launch_nm_axpby(int dtype, const void* a, float beta, const void* b, float gamma, void* out,
                          int64_t n, hipStream_t s);
// 1:2 compress and double prune (canonical format), and the metadata conversion to the 2:4
// encoding the SpMM kernels read (word | 0x88888888)
hipError_t launch_compress12(int dtype, const void* W, int64_t rows, int64_t cols, void* vals,
                             uint32_t* meta, hipStream_t s);
hipError_t launch_double_prune12(int dtype, const void* vals, const uint32_t* meta, int64_t rows,
                                 int64_t cols, void* p_vals, uint32_t* p_meta, hipStream_t s);
hipError_t launch_meta_or(const uint32_t* in, uint32_t* out, int64_t n, uint32_t bits, hipStream_t s);
// 2:8 (bf16): one 3-bit field per kept value, the two of a group in one byte, 4 groups per word
// 2:8 canonical arrays (values [rows][cols/4], one byte of two 3-bit positions per 8-column
// group) rewritten as 2:4 canonical arrays (values [rows][cols/2], 2-bit fields) holding the same
// entries plus +0.0 fillers, for the 2:4 products (cols % 32 == 0)
hipError_t launch_nm28_to24(const uint16_t* v8, const uint32_t* m8, int64_t rows, int64_t cols,
                            uint16_t* v4, uint32_t* m4, hipStream_t s, bool tiled = false);
hipError_t launch_compress28(const uint16_t* W, int64_t rows, int64_t cols, uint16_t* vals, uint32_t* meta,
                             hipStream_t s);
hipError_t launch_double_prune28(const uint16_t* vals, const uint32_t* meta, int64_t rows, int64_t cols,
                                 uint16_t* p_vals, uint32_t* p_meta, hipStream_t s);
// bf16 compress + double prune with both outputs in the streaming layout (rows, cols % 128 == 0)
hipError_t launch_compress_pair24_tiled(const uint16_t* W, int64_t rows, int64_t cols, void* vals,
                                        uint32_t* meta, void* p_vals, uint32_t* p_meta, hipStream_t s);
hipError_t launch_double_prune24(int dtype, const void* vals, const uint32_t* meta, int64_t rows,
                                 int64_t cols, void* p_vals, uint32_t* p_meta, hipStream_t s);
hipError_t launch_compress_ffi(int dtype, const void* W, int64_t rows, int64_t cols, int k,
                               void* vals, int16_t* idx, hipStream_t s);
size_t ffi_transpose_ws(int64_t rows, int64_t cols);
hipError_t launch_ffi_transpose(int dtype, const void* vals, const int16_t* idx, int64_t rows,
                                int64_t cols, int k, int32_t* row_ptr, int16_t* t_idx, void* t_vals,
                                void* ws, hipStream_t s);

// fp32 path (fp64 accumulation)
struct F32Sparse {  // a row-iterable sparse matrix: rows x cols, reduced over cols
  int format;
  int64_t rows, cols;
  const uint32_t* vals;   // fp32 bits
  const uint32_t* meta;   // NM 2:4
  int64_t meta_stride;    // words per row
  const int16_t* idx;     // ELL / CSR
  const int32_t* row_ptr; // CSR
  int k;                  // ELL
};
hipError_t launch_f32_adapter_u(const float* X, const float* A, int64_t T, int64_t K, int r,
                                double* U64, float* U32, hipStream_t s);
hipError_t launch_f32_spmm(const F32Sparse& S, const float* Act, int64_t T, const double* U64,
                           const float* E, int64_t e_row_stride, int64_t e_j_stride, int r,
                           float* Out, hipStream_t s);
hipError_t launch_f32_du(const float* dY, const float* B, int64_t T, int64_t N, int r,
                         double* dU64, float* dU32, hipStream_t s);
hipError_t launch_f32_tn(const float* Pf, const double* Pd, int64_t ldp, const float* Qf,
                         const double* Qd, int64_t ldq, int64_t T, int64_t M, int64_t Nn,
                         float* Out, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);

// bf16 2:4 SpMM with fused low-rank epilogue:
//   Out[t][row] = sum_c Act[t][c] * S[row][c] + sum_j U[t][j] * E(row, j)
struct Epilogue {
  const float* U = nullptr;     // [T][r] fp32
  const uint16_t* E = nullptr;  // bf16, element (row, j) at E[row*e_row_stride + j*e_j_stride]
                                // (the bf16 2:4 and dense SpMM launchers require e_j_stride == 1)
  int64_t e_row_stride = 0, e_j_stride = 0;
  int r = 0;
  // When G is set the SpMM computes U = Act G^T itself (G: r rows of C bf16, row j at G + j*g_ld)
  // and does not read U; its first row tile then writes U to u_out ([T][r] fp32) and, when vt is
  // set, U^T in three bf16 parts (vt[p][j][t], vt_rp rows, vt_tp columns, zeros for t >= T).
  const uint16_t* G = nullptr;
  int64_t g_ld = 0;
  float* u_out = nullptr;
  uint16_t* vt = nullptr;
  int vt_rp = 0;
  int64_t vt_tp = 0;
};
// True when launch_spmm24_bf16 for this shape computes the adapter rows U itself (Epilogue::G);
// the caller then skips the separate U kernel.
bool spmm24_fuses_adapter(int64_t R, int64_t C, int64_t T, int r);
size_t spmm24_ws(int64_t R, int64_t C, int64_t T);
// The same products with the weight fragments expanded to dense bf16 for dense MFMA (spmm_xp.hip):
// nm = 28 (2:8, canonical arrays) or 24 (2:4, canonical or streaming layout); C % 128 == 0.
bool spmm_xp_ok(int64_t C);
bool spmm_xp_fuses_adapter(int64_t R, int64_t C, int64_t T, int r);
size_t spmm_xp_ws(int64_t R, int64_t C, int64_t T);
hipError_t launch_spmm_xp_bf16(int nm, bool tiled, const uint16_t* s_vals, const uint32_t* s_meta,
                               int64_t R, int64_t C, const uint16_t* act, int64_t T,
                               const Epilogue& ep, uint16_t* out, void* ws, hipStream_t s);
hipError_t launch_spmm24_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                              const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                              void* ws, hipStream_t s);
// the same product with the weight in the streaming layout (sra_nm_tile): any T when C % 128 == 0,
// else T <= 16 only; ws holds the fp32 partials when the plan splits the reduction (spmm24_ws
// bytes; without it the product runs unsplit)
bool spmm24_tiled_ok(int64_t C, int64_t T);
hipError_t launch_spmm24_tiled_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R,
                                    int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                    uint16_t* out, void* ws, hipStream_t s);
size_t spmm24_decode_ws(int64_t R, int64_t C, int64_t T);
// 2:8 canonical arrays, T <= 16 (C % 32 == 0); no workspace
hipError_t launch_decode28_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                                const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                                hipStream_t s, bool tiled);
// 2:8 canonical arrays -> the 2:8 streaming layout (value and metadata blocks of 16 rows x 256 columns)
void nm28_tile_bytes(int64_t R, int64_t C, size_t* value_bytes, size_t* meta_bytes);
hipError_t launch_nm_tile28_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                                 void* t_vals, void* t_meta, hipStream_t s);
hipError_t launch_decode24_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R,
                                int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                uint16_t* out, hipStream_t s, bool tiled = false);
// canonical 2:4 bf16 arrays -> the decode kernel's streaming layout (1 KB blocks per 16-row tile
// and 64-column step, metadata per tile and 512-column batch)
void nm_tile_bytes(int64_t R, int64_t C, size_t* value_bytes, size_t* meta_bytes);
hipError_t launch_nm_tile_bf16(const uint16_t* s_vals, const uint32_t* s_meta, int64_t R, int64_t C,
                               void* t_vals, void* t_meta, hipStream_t s);
// The tiled fixed fan-in format (sra_ffi_tile) of an ELL matrix (row_ptr == nullptr, k entries
// per row) or a CSR one: entry lists per 32-row group and 64-column stage, and their offsets.
void ffi_tile_bytes(int64_t R, int64_t C, int64_t nnz, size_t* ent_bytes, size_t* off_bytes);
hipError_t launch_ffi_tile(const uint16_t* vals, const int16_t* idx, const int32_t* row_ptr, int k,
                           int64_t R, int64_t C, uint32_t* ent, uint32_t* offs, int64_t cap, hipStream_t s);
// Out[t][row] = sum over the row's entries of Act[t][col] val + epilogue, from the tiled format
// (C % 64 == 0, ent_bytes < 2^31); no workspace
hipError_t launch_ffi_tiled_bf16(const uint32_t* ent, const uint32_t* offs, size_t ent_bytes, int64_t R,
                                 int64_t C, const uint16_t* act, int64_t T, const Epilogue& ep,
                                 uint16_t* out, hipStream_t s);
// fixed fan-in bf16 SpMM (ELL forward / CSR backward) with the same epilogue; with enough tokens
// it writes the weight's tiled format into the workspace (spmm_ffi_ws bytes, O(nnz)) and runs
// the tiled product
size_t spmm_ffi_ws(int64_t R, int64_t C, int64_t T, int64_t nnz);
// An ELL (or CSR) matrix written out as R dense bf16 rows of C (C % 8 == 0, C <= 32767): the
// fixed fan-in adapter factor's dense copy.
hipError_t launch_ffi_densify(int format, const uint16_t* vals, const int16_t* idx,
                              const int32_t* row_ptr, int k, int64_t R, int64_t C, uint16_t* out,
                              hipStream_t s);
// out[e] = dense[(e / k) * C + idx[e]] for the R * k entries of an ELL pattern (fp32).
hipError_t launch_ell_gather_f32(const float* dense, const int16_t* idx, int k, int64_t R, int64_t C,
                                 float* out, hipStream_t s);
hipError_t launch_spmm_ffi_bf16(int format, const uint16_t* vals, const int16_t* idx,
                                const int32_t* row_ptr, int k, int64_t R, int64_t C,
                                const uint16_t* act, int64_t T, const Epilogue& ep, uint16_t* out,
                                void* ws, hipStream_t s, int64_t nnz);

// Adapter products (fp32 results):
//   rows: out[t][j] = sum_c act[t][c] * wt[j*ldw + c]                              (U, dU)
//   cols: out[m][j] = sum_t act[t][m] * V[t][j], written as [m][j] or transposed [j][m] (dB, dA)
// rows also writes an fp64 copy (out64) and/or V^T split into three bf16 parts (vt) when non-null;
// cols reads V^T as `parts` bf16 parts vt[p][j][t], rows vt_rows(r), columns vt_cols(T), zero past
// T.  The backward prep kernel packs B^T for the dU product (wt [r][packed_wt_ld(N)]) and A^T for
// the dX epilogue, and splits U^T into three parts for dB; any output may be null.
int64_t vt_rows(int r);
int64_t vt_cols(int64_t T);
size_t adapter_vt_bytes(int64_t T, int r, int parts);
int64_t packed_wt_ld(int64_t C);
size_t adapter_wt_bytes(int64_t C, int r);
// at [K][packed_at_ld(r)] = A^T, rows of r adapter entries (16-byte aligned) for the dX epilogue
int64_t packed_at_ld(int r);
size_t adapter_at_bytes(int64_t K, int r);
hipError_t launch_adapter_bwd_prep(const uint16_t* B, int64_t N, int r, uint16_t* wt,
                                   const uint16_t* A, int64_t K, uint16_t* at, const float* U,
                                   int64_t T, uint16_t* vtU, hipStream_t s);
size_t adapter_rows_ws(int64_t T, int64_t C, int r);
hipError_t launch_adapter_rows(const uint16_t* act, int64_t T, int64_t C, const uint16_t* wt,
                               int64_t ldw, int r, float* out, double* out64, uint16_t* vt,
                               void* ws, hipStream_t s);
size_t adapter_cols_ws(int64_t T, int64_t M, int r);
hipError_t launch_adapter_cols(const uint16_t* act, int64_t T, int64_t M, const uint16_t* vt,
                               int parts, int r, bool out_transposed, float* out, void* ws,
                               hipStream_t s);
// One or two cols products in one launch (dB and dA of the backward), each
//   out[m][j] (or out[j][m] when out_t) = sum_t act[t][m] V[t][j],  V^T as `parts` bf16 parts;
// needs M % 8 == 0 (adapter_grads_ok).  nmb and part are filled in by the launcher.
struct AdapterGrad {
  const uint16_t* act = nullptr;
  const uint16_t* vt = nullptr;
  float* out = nullptr;
  double* part = nullptr;
  int64_t M = 0;
  int parts = 0, nmb = 0;
  bool out_t = false;
};
struct AdapterGradArgs {
  AdapterGrad job[2];
  int64_t T, Tp, t_per;
  int r, rp, S;
};
bool adapter_grads_ok(const AdapterGrad* g, int n, int64_t T, int r);
size_t adapter_grads_ws(const AdapterGrad* g, int n, int64_t T, int r);
hipError_t launch_adapter_grads(const AdapterGrad* g, int n, int64_t T, int r, void* ws,
                                hipStream_t s);

}  // namespace sra

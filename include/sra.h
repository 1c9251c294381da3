/*
 * sra.h -- C ABI of libsra, a structured-sparse plus low-rank linear layer for AMD MI355X (gfx950).
 *
 * The layer (SLoPe paperlayer summary, §2.2 "Lazy low-rank adapters"; LoRA as described in
 * "efficient training for the gpu-poor", section PEFT):
 *
 *     forward   U  = X A^T                      (fp32)
 *               Y  = X Ws^T + U B^T
 *     backward  dU = dY B                       (fp32)
 *               dB = dY^T U,  dA = dU^T X       (fp32)
 *               dX = dY P^T + dU A              (P = double-pruned Ws^T for N:M weights,
 *                                                the exact transpose for fixed fan-in weights)
 *
 * Shapes: X [T,K], Ws [N,K] (N outputs, K inputs), A [r,K], B [N,r], Y/dY [T,N], dX [T,K].
 * Ws is either N:M sparse along K (2:4: every 4 consecutive inputs keep 2; SLoPe §2.1) or fixed
 * fan-in (every output row keeps exactly k inputs at arbitrary columns; SQuAsh project update).
 *
 * Conventions for every call:
 *   - Matrices are row-major and contiguous.  Pointers are device pointers unless marked "host".
 *     Device pointers must be 16-byte aligned.
 *   - Ownership: the caller allocates and frees every buffer, including outputs and the
 *     workspace; the library allocates no device memory and keeps no pointer after a call returns.
 *     The one exception is the fixed per-GPU array of sra_sparse_lora_bwd_noalloc, which lives in
 *     the library's code object (no allocating call) until the process ends.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; a call returns after launching.  Calls on different streams may overlap.
 *   - Errors: every call returns an sra_status.  All argument checks happen on the host before any
 *     launch, so a non-OK status means nothing was enqueued, except SRA_ERR_HIP, which reports a
 *     launch failure (some earlier kernels of the same call may have been enqueued).
 *     sra_last_error() returns a message for the last failing call of the calling thread.
 *   - Inputs must be finite.  Values of dtype X (bf16 or fp32) are: X, dY, A, B, Y, dX and the
 *     compressed values; U, dU, dA and dB are always fp32.
 *   - Tie rule for every magnitude selection: larger |w| first; equal magnitudes go to the lower
 *     index; +0 and -0 are equal.
 */
#ifndef SRA_H
#define SRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SRA_ABI_VERSION 1

typedef enum {
  SRA_OK = 0,
  SRA_ERR_INVALID_ARG = -1, /* null pointer, bad shape, misaligned pointer, inconsistent descriptor */
  SRA_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels implement (e.g. N:M other than 2:4) */
  SRA_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than the *_workspace query returned */
  SRA_ERR_HIP = -4          /* a HIP launch failed; see sra_last_error() */
} sra_status;

typedef enum { SRA_BF16 = 0, SRA_F32 = 1 } sra_dtype;

typedef enum {
  SRA_FMT_NM = 0,  /* N:M along cols: values [rows, cols*n/m], meta [rows, sra_nm_meta_words] */
  SRA_FMT_ELL = 1, /* fixed fan-in: values [rows, k], index int16 [rows, k], columns ascending */
  SRA_FMT_CSR = 2, /* transpose of an ELL matrix: row_ptr int32 [rows+1], index int16 [nnz],
                      values [nnz], column ids ascending inside each row */
  SRA_FMT_NM_TILED = 3, /* 2:4 or 2:8 bf16 in the streaming layout of sra_nm_tile */
  SRA_FMT_FFI_TILED = 4 /* fixed fan-in bf16 in the tiled entry lists of sra_ffi_tile */
} sra_format;

/*
 * Description of a compressed sparse matrix (caller-owned; the library only reads it, except that
 * sra_double_prune / sra_ffi_transpose fill the shape fields of their output descriptor).
 *
 * rows x cols is the logical dense shape; every row is reduced over its cols.  For the forward the
 * matrix is Ws (rows = N outputs, cols = K); for the backward it is P (rows = K, cols = N).
 *
 * N:M canonical format (SLoPe §2.1 N:M prune, layout of this library): row i keeps, in each group
 * of m consecutive columns, n entries.  values[i, :] holds the kept entries in ascending column
 * order.  meta[i, :] holds each kept entry's position inside its group as a 2-bit field, fields in
 * kept order, packed least-significant first, 16 fields per uint32 word; the unused high fields of
 * the last word are zero.  Word count per row: sra_nm_meta_words(cols, n, m).
 */
typedef struct sra_sparse {
  int32_t format;   /* sra_format */
  int32_t dtype;    /* sra_dtype of values */
  int64_t rows;
  int64_t cols;
  int32_t n, m;     /* SRA_FMT_NM */
  int32_t k;        /* SRA_FMT_ELL: entries per row */
  int64_t nnz;      /* SRA_FMT_CSR: stored entries (= rows_of_ELL * k) */
  void* values;
  uint32_t* meta;   /* SRA_FMT_NM */
  int16_t* index;   /* SRA_FMT_ELL / SRA_FMT_CSR */
  int32_t* row_ptr; /* SRA_FMT_CSR */
} sra_sparse;

/* ABI version of the loaded library (SRA_ABI_VERSION when it matches this header). */
int32_t sra_abi_version(void);

/* Message for the last non-OK status returned on the calling thread (host string, owned by the
 * library, valid until the next call on that thread).  Empty string if none. */
const char* sra_last_error(void);

/* Number of uint32 metadata words per row for an N:M row of `cols` columns: ceil(cols*n/m/16). */
int64_t sra_nm_meta_words(int64_t cols, int32_t n, int32_t m);

/*
 * compress(W, N, M) -- first N:M prune (SLoPe §2.1; the mask is chosen once and kept fixed).
 * W [rows, cols] dense (dtype) -> out->values [rows, cols*n/m], out->meta [rows, meta_words].
 * In each group of m consecutive columns the n entries of largest magnitude are kept.
 * Supported: 2:4 and 1:2 (same format: one 2-bit in-group field per stored value), cols % 32 == 0.
 * Every call that takes a canonical N:M matrix accepts 1:2 as well; the products run it on the
 * 2:4 kernels (a 1:2 row keeps two entries of every four columns, one per pair), converting the
 * metadata into the workspace.  Also 2:8 (bf16, cols % 32 == 0): values [rows, cols/4] in
 * ascending column order, and per 8-column group one metadata byte holding the two in-group
 * positions (bits 0-2 and 3-5, the rest zero), four group bytes per uint32 word, so cols/32
 * words per row.  The products rewrite a 2:8 weight as a 2:4 one in their workspace above 16
 * tokens (see SRA_TUNE_ENGINE) and stream it through their decode kernel at 16 tokens or fewer;
 * 2:8 has no pair kernel or masked gradient.  sra_nm_tile takes 2:4 and 2:8 (each its own
 * streaming layout); sra_compress_pair_tiled is 2:4 only.  The caller sets out->values and out->meta; the call
 * fills the remaining descriptor fields (format, dtype, rows, cols, n, m).
 */
sra_status sra_compress(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t n,
                        int32_t m, sra_sparse* out /* host */, void* stream);

/*
 * double_prune -- P = prune_NM(Ws^T) (SLoPe §1 and §2.1: the N:M-pruned weight is transposed and
 * N:M-pruned again along the other dimension, so the backward product is also N:M).
 * Ws: SRA_FMT_NM, rows = N outputs, cols = K.  P: caller sets P->values [K, N*n/m] and
 * P->meta [K, meta_words(N)]; the call fills the other fields (rows = K, cols = N).
 * In each group of m consecutive outputs of one input column, only entries kept by Ws are
 * eligible; the n largest eligible are kept.  A group with fewer than n eligible entries is padded
 * with its lowest unused positions holding +0.0, so every group stores exactly n.
 * Supported: 2:4, 1:2 and 2:8 (bf16), Ws->rows % 32 == 0, Ws->cols % 32 == 0.
 */
sra_status sra_double_prune(const sra_sparse* Ws /* host */, sra_sparse* P /* host */, void* stream);

/*
 * compress_pair -- sra_compress followed by sra_double_prune in one pass over W, with bit-identical
 * results: for training loops that refresh both compressed forms of a weight after every update
 * (SLoPe §2.3 keeps compressed formats of the weight and of its transpose; the masks stay fixed).
 * Ws receives compress(W) (rows x cols), P receives double_prune(Ws) (cols x rows); the caller
 * sets the values and meta pointers of both, the call fills the other fields.
 * Supported: 2:4, rows % 32 == 0, cols % 32 == 0.
 */
sra_status sra_compress_pair(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t n,
                             int32_t m, sra_sparse* Ws /* host */, sra_sparse* P /* host */,
                             void* stream);

/*
 * nm_tile -- the same 2:4 or 2:8 weight in a streaming layout for memory-bound forwards of few tokens
 * (SLoPe §3 inference results: with few tokens the layer is bound by reading the compressed
 * weight once; the compressed form is prepared once and reused, SLoPe §2.3).  The content is that
 * of the canonical arrays, permuted so that the decode kernel reads every block contiguously:
 *   values: for row tile t (16 rows) and step s (64 columns = 32 stored values), a 1 KB block at
 *           byte (t * ceil(cols/64) + s) * 1024; its 16-byte chunk l = 16 q + i holds stored values
 *           32 s + 8 q .. 32 s + 8 q + 7 of row 16 t + i.
 *   meta:   for row tile t and batch b (512 columns = 16 words), a 1 KB block at byte
 *           (t * ceil(cols/512) + b) * 1024; bytes 64 i .. 64 i + 63 hold words 16 b .. 16 b + 15
 *           of row 16 t + i.
 * 2:8 (blocks shaped for the 2:8 decode kernel, whose wave owns whole row tiles): for row tile t
 * and batch b (256 columns = 64 stored values and 8 metadata words per row), a 2 KB value block at
 * byte (t * ceil(cols/256) + b) * 2048 whose 16-byte chunk 64 c + l (c = 0, 1; l = 16 q + i) holds
 * stored values 64 b + 16 q + 8 c .. +7 of row 16 t + i, and a 512-byte metadata block at byte
 * (t * ceil(cols/256) + b) * 512 whose bytes 8 l .. 8 l + 7 hold words 8 b + 2 q and 8 b + 2 q + 1
 * of that row.
 * Entries past the last row or column are zero.  Sizes: sra_nm_tile_bytes.
 * Ws: canonical SRA_FMT_NM, bf16, 2:4 or 2:8.  out: the caller sets values and meta (16-byte aligned,
 * value_bytes and meta_bytes long); the call fills the other fields (format SRA_FMT_NM_TILED, same
 * dtype, rows, cols, n, m).  An SRA_FMT_NM_TILED weight is accepted by sra_sparse_lora_fwd (as
 * Ws) and sra_sparse_lora_bwd (as P) for T <= 16, and for any T when cols % 128 == 0 (else
 * SRA_ERR_UNSUPPORTED); the results equal the canonical arrays' bit for bit when neither path
 * splits the reduction.  A 2:8 one is accepted for any T: above 16 tokens the call rewrites it as
 * canonical 2:4 in its workspace, as for canonical 2:8 arrays.
 */
sra_status sra_nm_tile_bytes(int64_t rows, int64_t cols, int32_t n, int32_t m,
                             size_t* value_bytes /* host */, size_t* meta_bytes /* host */);
sra_status sra_nm_tile(const sra_sparse* Ws /* host */, sra_sparse* out /* host */, void* stream);

/*
 * compress_pair_tiled -- sra_compress_pair with both outputs written in the streaming layout of
 * sra_nm_tile (SLoPe §2.3: a training loop refreshes both compressed forms after every update; in
 * this layout the forward and backward products read their sparse operand in 1 KB runs).  The
 * content equals sra_nm_tile applied to sra_compress_pair's outputs, bit for bit.
 * Ws: values / meta of sra_nm_tile_bytes(rows, cols) bytes; P: of sra_nm_tile_bytes(cols, rows).
 * The call fills the other fields (format SRA_FMT_NM_TILED, dtype, shapes, n, m).
 * Supported: bf16, 2:4, rows % 128 == 0, cols % 128 == 0 (else SRA_ERR_UNSUPPORTED).
 */
sra_status sra_compress_pair_tiled(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t n,
                                   int32_t m, sra_sparse* Ws /* host */, sra_sparse* P /* host */,
                                   void* stream);

/*
 * compress_ffi(W, k) -- fixed fan-in selection (SQuAsh project update): every row of W
 * [rows, cols] keeps its k largest-magnitude entries.  out->values [rows, k] and out->index
 * (int16) [rows, k] with columns ascending; set by the caller, other fields filled by the call.
 * Needs 1 <= k <= cols <= 32767.
 */
sra_status sra_compress_ffi(const void* W, int32_t dtype, int64_t rows, int64_t cols, int32_t k,
                            sra_sparse* out /* host */, void* stream);

/* Workspace bytes for sra_ffi_transpose of an ELL matrix with `rows` rows and `cols` columns. */
sra_status sra_ffi_transpose_workspace(int64_t rows, int64_t cols, int32_t k, size_t* bytes /* host */);

/*
 * ffi_transpose -- exact transpose of a fixed fan-in weight for the backward (SLoPe §2.3 keeps
 * sparse formats for a weight and its transpose).  Ws: SRA_FMT_ELL [rows, cols].  WsT: caller
 * sets row_ptr [cols+1], index [rows*k], values [rows*k]; the call fills the other fields
 * (format CSR, rows = Ws->cols, cols = Ws->rows, nnz).  Entries of each CSR row are ordered by
 * ascending original row.
 */
sra_status sra_ffi_transpose(const sra_sparse* Ws /* host */, sra_sparse* WsT /* host */, void* ws,
                             size_t ws_bytes, void* stream);

/* Buffer sizes of sra_ffi_tile for a matrix of `rows` x `cols` with nnz stored entries:
 * *entry_bytes for out->values, *offset_bytes for out->meta.  1 <= cols <= 32767. */
sra_status sra_ffi_tile_size(int64_t rows, int64_t cols, int64_t nnz, size_t* entry_bytes /* host */,
                             size_t* offset_bytes /* host */);

/*
 * ffi_tile -- the products' layout of a fixed fan-in matrix (SQuAsh project update: fixed fan-in
 * weights; SLoPe paperlayer summary §2.3: a format for the weight and one for its transpose),
 * built once per mask like sra_nm_tile.  S: SRA_FMT_ELL (the forward weight) or SRA_FMT_CSR (its
 * transpose from sra_ffi_transpose), bf16.  Rows are cut into 32-row groups and columns into
 * 64-column stages; list (g, x) holds the entries of group g in stage x as uint32 words, the
 * bf16 value in the low 16 bits and in the high 16 bits the entry's byte offset in the group's
 * 32 x 64 bf16 block as the products hold it in LDS: with i = row - 32 g and c = column - 64 x,
 * i * 128 + ((c / 8) XOR ((i / 2) % 8)) * 16 + (c % 8) * 2 (128-byte rows, 16-byte chunks
 * swizzled).  Words are ordered by row, then column, padded to a multiple of 4 words with
 * 0xffffffff.  Lists follow
 * each other by group, then stage.  out->values: the words (entry_bytes of sra_ffi_tile_size,
 * 16-byte aligned); out->meta: uint32 offsets, meta[g * stages + x] = first word of list (g, x),
 * then the total word count 4 times (offset_bytes).  The caller sets out->values and out->meta;
 * the call fills format (SRA_FMT_FFI_TILED), dtype, rows, cols and nnz (the capacity of
 * out->values in words).  sra_sparse_lora_fwd takes the tiled ELL weight, sra_sparse_lora_bwd the
 * tiled CSR transpose; both need the reduction (cols) to be a multiple of 64 and use no
 * workspace for the product.  Errors: SRA_ERR_INVALID_ARG (format, shapes, pointers),
 * SRA_ERR_UNSUPPORTED (fp32, over 2 GiB of entries).
 */
sra_status sra_ffi_tile(const sra_sparse* S /* host */, sra_sparse* out /* host */, void* stream);

/* Workspace bytes for sra_sparse_lora_fwd (T tokens, rank r). */
sra_status sra_fwd_workspace(const sra_sparse* Ws /* host */, int64_t T, int32_t r,
                             size_t* bytes /* host */);

/*
 * sparse_lora_fwd -- Y = X Ws^T + (X A^T) B^T (SLoPe §2.2; the adapter product is fused into the
 * sparse product's epilogue, cf. SLoPe §2.4 and App. D, so Y is written once).
 * Ws: SRA_FMT_NM (2:4), SRA_FMT_NM_TILED (2:4, see sra_nm_tile), SRA_FMT_ELL or SRA_FMT_FFI_TILED
 * (fixed fan-in, see sra_ffi_tile; K % 64 == 0), rows = N, cols = K.  With 128 or more tokens an
 * ELL weight is first tiled into the workspace (O(nnz) bytes).
 * X [T,K], A [r,K], B [N,r], Y [T,N].
 * U_out [T,r] fp32 receives U = X A^T when non-NULL (keep it for the backward).
 * r = 0 means no adapter (A, B, U_out ignored).  T = 0 is a no-op.  Y has dtype Ws->dtype.
 * bf16 accumulates in fp32 (U is kept in fp32); fp32 accumulates in fp64.
 * Supported: 0 <= r <= 256 (2:4 weights need K % 32 == 0, as for sra_compress).
 */
sra_status sra_sparse_lora_fwd(const sra_sparse* Ws /* host */, const void* X, int64_t T,
                               const void* A, const void* B, int32_t r, void* Y, float* U_out,
                               void* ws, size_t ws_bytes, void* stream);

enum {
  SRA_GRAD_DX = 1,       /* compute dX */
  SRA_GRAD_DA = 2,       /* compute dA */
  SRA_GRAD_DB = 4,       /* compute dB */
  SRA_DX_NO_ADAPTER = 8  /* dX without the dU A term (sparse product only) */
};

/* Workspace bytes for sra_sparse_lora_bwd. */
sra_status sra_bwd_workspace(const sra_sparse* P /* host */, int64_t T, int32_t r, uint32_t flags,
                             size_t* bytes /* host */);

/*
 * sparse_lora_bwd -- double-pruned backward (SLoPe §1, §2.1; the output gradient dY is never
 * pruned, SLoPe App. J).
 * P: for N:M weights the output of sra_double_prune (rows = K, cols = N; canonical, or in the
 * streaming layout of sra_nm_tile / sra_compress_pair_tiled); for fixed fan-in weights
 * the CSR of sra_ffi_transpose (rows = K, cols = N) or its sra_ffi_tile form (N % 64 == 0).
 * dY [T,N], X [T,K], A [r,K], B [N,r] (dtype P->dtype); T tokens.  U [T,r] fp32 from the forward, or NULL
 * to recompute it from X and A.  Outputs (each only if its flag is set): dX [T,K] (dtype),
 * dA [r,K] fp32, dB [N,r] fp32.  dU_out [T,r] fp32 receives dU = dY B when non-NULL and r > 0.
 * Flags without r > 0 (dA, dB) are ignored.
 * dA and dB reduce over all T tokens in a fixed order (results do not depend on the stream).
 * fp32 weights keep U and dU in fp64 inside the call (U is recomputed from X and A; the U
 * argument is not read).
 * T = 0 writes zeros to dA and dB.
 */
sra_status sra_sparse_lora_bwd(const sra_sparse* P /* host */, const void* dY, const void* X,
                               int64_t T, const float* U, const void* A, const void* B, int32_t r,
                               uint32_t flags, void* dX, float* dA, float* dB, float* dU_out,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Fixed-fan-in adapter factor (SQuAsh project update, first paragraph: one factor of the low-rank
 * product is itself pruned with fixed fan-in, so that a higher-rank adapter fits the memory of a
 * lower-rank dense one).  The pruned factor is the down-projection A [r,K], given as an ELL matrix
 * (SRA_FMT_ELL, rows = r, cols = K, k entries per row at ascending columns, as sra_compress_ffi
 * writes it); B [N,r] stays dense.  With A_s = A scattered to its columns:
 *     forward   U = X A_s^T,  Y = X Ws^T + U B^T
 *     backward  dU = dY B,  dB = dY^T U,  dX = dY P^T + dU A_s,
 *               dA_values[j][i] = sum_t dU[t][j] X[t][col(j, i)]   (fp32, A's ELL order: only the
 *               stored entries learn, their mask is fixed)
 * Ws / P as for sra_sparse_lora_fwd / sra_sparse_lora_bwd (N:M or its streaming layout); bf16 only;
 * A->dtype == the weight's dtype, A->cols == K, 1 <= A->rows <= 256, K % 8 == 0.  The workspace
 * holds A_s densified (r x K bf16) and, for dA, the dense fp32 r x K gradient before its gather;
 * sizes from sra_ffa_fwd_workspace / sra_ffa_bwd_workspace.  Flags as for sra_sparse_lora_bwd
 * (SRA_GRAD_DA selects dA_values).  Errors as for the dense-adapter calls.
 */
sra_status sra_ffa_fwd_workspace(const sra_sparse* Ws /* host */, int64_t T,
                                 const sra_sparse* A /* host */, size_t* bytes /* host */);
sra_status sra_sparse_lora_fwd_ffa(const sra_sparse* Ws /* host */, const void* X, int64_t T,
                                   const sra_sparse* A /* host */, const void* B, void* Y,
                                   float* U_out, void* ws, size_t ws_bytes, void* stream);
sra_status sra_ffa_bwd_workspace(const sra_sparse* P /* host */, int64_t T,
                                 const sra_sparse* A /* host */, uint32_t flags,
                                 size_t* bytes /* host */);
sra_status sra_sparse_lora_bwd_ffa(const sra_sparse* P /* host */, const void* dY, const void* X,
                                   int64_t T, const float* U, const sra_sparse* A /* host */,
                                   const void* B, uint32_t flags, void* dX, float* dA_values,
                                   float* dB, float* dU_out, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * sparse_lora_bwd_noalloc -- sra_sparse_lora_bwd with no workspace argument and no allocation,
 * for callers that cannot allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc).  Same arguments, same kernels and the same
 * results as sra_sparse_lora_bwd bit for bit; the workspace that call would take is a fixed
 * device array inside the library instead, SRA_NOALLOC_SCRATCH_BYTES long, one per GPU, held
 * until the process ends.
 *   - The GPU is the calling thread's current device; `stream` must belong to it.
 *   - A call whose workspace (sra_bwd_workspace with the same U / dU_out choices) exceeds
 *     SRA_NOALLOC_SCRATCH_BYTES returns SRA_ERR_WORKSPACE before any launch; use
 *     sra_sparse_lora_bwd with a caller workspace for such shapes.
 *   - Every call on one GPU shares that GPU's array: calls on one stream run one after another,
 *     but calls that can overlap on one GPU (different streams, or different threads) race on it
 *     and give undefined results.  Nothing in the array needs to start at zero; a call writes
 *     every part it reads.
 *   - The first call on a device looks up the array's device address (no allocation); errors
 *     there return SRA_ERR_HIP.
 */
#define SRA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sra_status sra_sparse_lora_bwd_noalloc(const sra_sparse* P /* host */, const void* dY,
                                       const void* X, int64_t T, const float* U, const void* A,
                                       const void* B, int32_t r, uint32_t flags, void* dX,
                                       float* dA, float* dB, float* dU_out, void* stream);

/*
 * masked_weight_grad -- gradient of the stored values of a compressed N:M matrix (SLoPe §2.1: in
 * sparse training the mask is fixed and only the stored entries learn; §2.3 keeps compressed
 * forms of the weight and its transpose).  For S (rows x cols, N:M along cols):
 *     out_values[row][i] = sum_t row_act[t][row] * col_act[t][c_i(row)]
 * with c_i(row) the column of the row's i-th stored entry (the order of S->values).  For the
 * forward weight Ws (rows = N, cols = K): row_act = dY [T,N], col_act = X [T,K], giving
 * dWs = (dY^T X) o mask1 in Ws's value order.  For P (rows = K, cols = N): row_act = X,
 * col_act = dY (P's padding slots receive the dense gradient at their positions).
 * S: SRA_FMT_NM canonical, bf16, 2:4 (S->values is not read; S->meta is).  out_values
 * [rows, cols/2] bf16, caller-owned.  fp32 accumulation of 32-token partials summed in fp64, one
 * rounding to bf16.  T = 0 writes zeros.  Supported: bf16, 2:4 or 1:2, rows % 8 == 0,
 * T*rows and T*cols below 2^30 elements (else SRA_ERR_UNSUPPORTED).
 */
sra_status sra_masked_weight_grad(const sra_sparse* S /* host */, const void* row_act,
                                  const void* col_act, int64_t T, void* out_values, void* stream);

/*
 * nm_axpby -- out = beta * A + gamma * B for two compressed matrices that share one N:M pattern,
 * on their value arrays (SLoPe §2.3: a sparse addition of matrices with the same pattern, for
 * weight decay and the update step; §2.1: the mask is fixed, so the metadata stays valid and is
 * not touched).  With B = the masked weight gradient (sra_masked_weight_grad) this is the sparse
 * SGD step with decoupled weight decay, Ws <- (1 - lr wd) Ws - lr dWs; afterwards
 * sra_double_prune (or sra_compress_pair from the dense weight) refreshes the transpose form.
 * a_values, b_values, out_values: n_values elements of `dtype` (out may equal a or b).  fp32
 * arithmetic (one fused multiply-add per element), one rounding to the storage type.
 * The caller guarantees the shared pattern (the call sees values only).
 */
sra_status sra_nm_axpby(const void* a_values, float beta, const void* b_values, float gamma,
                        void* out_values, int64_t n_values, int32_t dtype, void* stream);

/*
 * Tuning knobs of the calling thread, for benchmarks and tests (not needed for computing anything;
 * every knob's default is the library's own choice, and results stay within the stated tolerance
 * under any setting).  Returns SRA_ERR_INVALID_ARG for an unknown key or a value out of range.
 *   SRA_TUNE_RESET         every knob back to its default (value ignored)
 *   SRA_TUNE_SPMM_CONFIG   bf16 2:4 SpMM tile configuration for T > 16 (0 = the planner's); the
 *                          decode path (T <= 16) ignores it.  Ids: 3 register-staged 128x128;
 *                          13 and 14 LDS-DMA 128x128 and 128x64 (32x32x32 SMFMAC); 50, 51 eight-wave
 *                          256x128, 256x256; 55 and 61 the same with metadata super-stages
 *                          (C % 128 == 0); 62 = 61 in a ping-pong schedule.  A configuration the
 *                          shape cannot take falls back to one it can.
 *   SRA_TUNE_SPMM_SPLITS   splits of the reduction for a forced configuration (0 or 1: none;
 *                          -2: only the 256x256 tiles past the last whole wave of 256, in two)
 *   SRA_TUNE_SPMM_FUSE     1 (default): U / dU of ranks <= 16 inside the SpMM where the plan
 *                          allows; 0: always in a separate kernel
 *   SRA_TUNE_ENGINE        SRA_ENGINE_SMFMAC (default): 2:4 products on the structured-sparse
 *                          matrix instructions; SRA_ENGINE_DENSE_MFMA: the same pipeline with each
 *                          weight fragment expanded to dense bf16 (zeros at the pruned positions)
 *                          for dense MFMA (bf16, K % 128 == 0 for the forward, N % 128 == 0 for
 *                          the backward).  2:8 weights: 16 tokens or fewer always take the 2:8
 *                          decode kernel on SMFMAC; above that, on SMFMAC, a 2:8 weight is
 *                          rewritten in the call's workspace as a 2:4 one (each four columns of a
 *                          2:8 row hold at most two kept entries; +0.0 fills the rest) and runs on
 *                          the 2:4 kernels, and on the dense engine its fragments are expanded
 *                          (the streaming layout's after the same 2:4 rewrite)
 *   SRA_TUNE_DECODE_ROWS   decode workgroup row tiles of 16 rows: 3, 4 or 9 (0 = the planner's)
 *   SRA_TUNE_ROWS_SLICES   reduction slices of the rank > 32 U / dU kernel (0 = the planner's)
 *   SRA_TUNE_GRADS_SLICES  token slices of the dA / dB kernel (0 = the planner's)
 */
enum {
  SRA_TUNE_RESET = 0,
  SRA_TUNE_SPMM_CONFIG = 1,
  SRA_TUNE_SPMM_SPLITS = 2,
  SRA_TUNE_SPMM_FUSE = 3,
  SRA_TUNE_ENGINE = 4,
  SRA_TUNE_DECODE_ROWS = 5,
  SRA_TUNE_ROWS_SLICES = 6,
  SRA_TUNE_GRADS_SLICES = 7
};
enum { SRA_ENGINE_SMFMAC = 0, SRA_ENGINE_DENSE_MFMA = 1 };
sra_status sra_set_tuning(int32_t key, int32_t value);

/* Kernel classes for sra_time_next_kernel. */
enum {
  SRA_KERNEL_COMPRESS = 1,     /* 2:4 compression (sra_compress, sra_compress_pair) */
  SRA_KERNEL_DOUBLE_PRUNE = 2, /* sra_double_prune */
  SRA_KERNEL_SPMM24 = 3,       /* bf16 2:4 SpMM + fused adapter epilogue (forward Y, backward dX) */
  SRA_KERNEL_ADAPTER = 4,      /* adapter products U, dU, dB, dA (one launch each) */
  SRA_KERNEL_DECODE24 = 5,     /* bf16 2:4 decode SpMM (forward with T <= 16) */
  SRA_KERNEL_SPMM_FFI = 6,     /* bf16 fixed fan-in SpMM (forward Y, backward dX) */
  SRA_KERNEL_FFI_DENSIFY = 7,  /* bf16 fixed fan-in adapter factor expanded to dense rows */
  SRA_KERNEL_WEIGHT_GRAD = 8,  /* bf16 masked weight gradient (sra_masked_weight_grad) */
  SRA_KERNEL_NM_UPDATE = 9     /* beta A + gamma B on shared-pattern values (sra_nm_axpby) */
};

/*
 * Profiling hook for benchmarks (not needed for computing anything).  Arms the calling thread so
 * that the next launch of a kernel of class `which` records `start` and `stop` (hipEvent_t,
 * created by the caller with timing enabled) immediately around that one kernel, through
 * hipExtLaunchKernelGGL.  One kernel class can be armed at a time; arming again replaces the
 * previous request, and which = 0 disarms.  The events must not be used while a stream is being
 * captured into a graph.
 */
sra_status sra_time_next_kernel(int32_t which, void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* SRA_H */

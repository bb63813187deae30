/*
 * mi_bitmask.h -- C ABI of the packed-bitmask apply for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (XGrammar "Bitmask Operations", apply_token_bitmask_inplace;
 * Modular MAX "apply_packed_bitmask"):
 *
 *   for every processed row r and every token v < V:
 *       word = (uint32) mask[r, v / 32]
 *       if bit (v % 32) of word is 0:  logits[r, v] = fill
 *
 * A set bit keeps the token, a clear bit masks it.  Words are int32 in
 * memory (kept as int32 because old PyTorch had no uint32, XGrammar
 * allocate_token_bitmask) and are read as uint32.
 *
 * Shared conventions of every entry point
 * ---------------------------------------
 * Memory.  Every pointer except the ``out`` parameters of the host helpers
 * is DEVICE memory, borrowed from the caller, and must stay valid until the
 * work enqueued on ``stream`` has finished.  A buffer with no elements (zero
 * rows or zero columns) may be NULL.  The library allocates nothing,
 * keeps no state between calls and never synchronises: each call validates
 * on the host, enqueues its kernel(s) on ``stream`` (0 = the null stream)
 * and returns.  Calls are therefore legal under HIP graph capture.
 *
 * Layout.  logits is [rows, cols] of ``dtype`` with a contiguous last
 * dimension and a row pitch of ``logits_row_stride`` ELEMENTS
 * (>= cols).  mask is int32 [mask_rows, mask_cols] with a pitch of
 * ``mask_row_stride`` WORDS (>= mask_cols).  logits must be aligned to its
 * element size, mask and indices to 4 bytes.  Row pitches may break
 * 16-byte alignment; the kernels handle any row start.
 *
 * Vocab size (XGrammar "Bitmask Operations", Notes: Padding).  vocab_size
 * = -1 selects the default V = min(cols, 32 * mask_cols).  An explicit V
 * must satisfy 0 <= V <= min(cols, 32 * mask_cols).  Only columns [0, V)
 * and words [0, ceil(V/32)) are touched; bits past V in the last word and
 * later words are never used (Modular MAX "apply_packed_bitmask": padding
 * bits are never read).  Columns >= V of a processed row are never written
 * in place.
 *
 * Rows (XGrammar "Bitmask Operations", Notes: Indices).  indices == NULL
 * processes rows 0..rows-1 and needs mask_rows >= rows (extra mask rows are
 * ignored) and num_indices == 0.  Otherwise indices is a device int32 array
 * of num_indices row numbers; each r selects logits row r AND mask row r.
 * They should be unique (duplicates only repeat identical writes) and lie
 * in [0, min(rows, mask_rows)); the host cannot see device memory, so an
 * out-of-range value is skipped by the kernel (that slot writes nothing).
 * num_indices == 0 with a non-NULL pointer processes no row.
 *
 * Fill.  fill_value is rounded once, to nearest-even, into the dtype
 * (overflow gives +-inf; NaN gives a quiet NaN with the input's sign).
 * Kept elements are never rewritten with a different bit pattern: NaN
 * payloads, -0.0 and subnormals survive exactly.
 *
 * Errors.  Every entry point returns a status and never throws or aborts.
 * All argument checks run on the host before any HIP call, so a failing
 * call enqueues nothing.  MI_ERR_HIP reports a launch failure; the HIP
 * error text is then in mi_last_error_message().  The message is
 * thread-local and valid until the thread's next call into the library.
 */
#ifndef MI_BITMASK_H
#define MI_BITMASK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mi_dtype {
    MI_DTYPE_F32 = 0,   /* IEEE binary32 */
    MI_DTYPE_F16 = 1,   /* IEEE binary16 */
    MI_DTYPE_BF16 = 2   /* bfloat16 */
} mi_dtype_t;

typedef enum mi_status {
    MI_OK = 0,
    MI_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
    MI_ERR_BAD_DTYPE = 2,      /* dtype is not one of mi_dtype_t */
    MI_ERR_BAD_SHAPE = 3,      /* negative size, pitch < width, too few mask rows, size limits */
    MI_ERR_BAD_VOCAB = 4,      /* vocab_size < -1 or above min(cols, 32 * mask_cols) */
    MI_ERR_BAD_INDICES = 5,    /* num_indices < 0 or too large */
    MI_ERR_ALIAS = 6,          /* an output overlaps an input it must not overlap */
    MI_ERR_HIP = 7,            /* the HIP runtime refused the launch */
    MI_ERR_MISALIGNED = 8,     /* a pointer is not aligned to its element size */
    MI_ERR_BAD_VARIANT = 9     /* unknown variant, or one the operation does not have */
} mi_status_t;

/* Kernel variants (the *_ex entry points).  All give bit-identical results. */
typedef enum mi_variant {
    MI_VARIANT_AUTO = 0,    /* the library's choice for the dtype and operation */
    MI_VARIANT_SCALAR = 1,  /* one thread per element */
    MI_VARIANT_VEC = 2,     /* 16-byte vectors: all-masked vectors are stored without a
                               read, mixed ones read-select-write, all-kept ones skipped */
    MI_VARIANT_WRONLY = 3,  /* in place only: one lane per element, the store of the fill
                               predicated by the mask bit; logits are never read */
    MI_VARIANT_VEC_RESIDENT = 4  /* in place only: the 16-byte-vector kernel shaped for logits
                               that are still in the GPU's caches (just written by the
                               producing kernel): write-back stores, 16 vectors per lane.
                               AUTO is shaped for logits that must come from HBM. */
} mi_variant_t;

/*
 * In-place apply: logits[r, v] = fill for every processed row r and v < V
 * whose mask bit is 0 (XGrammar "Bitmask Operations",
 * apply_token_bitmask_inplace, with fill_value = -INFINITY for that page's
 * semantics).  mask may not overlap logits; indices may not overlap logits.
 * No work is enqueued when V == 0 or no row is processed.
 */
mi_status_t mi_apply_bitmask_inplace(
    void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int32_t *indices, int64_t num_indices,
    double fill_value, hipStream_t stream);

/*
 * Out-of-place apply (Modular MAX "apply_packed_bitmask": one fused pass,
 * output = logit where the bit is set, else fill_value).  out is [rows, cols]
 * of the same dtype with pitch out_row_stride elements (>= cols).  Every
 * element of out's [rows, cols] window is written: processed rows get the
 * masked copy over [0, V) and a plain copy over [V, cols); rows outside an
 * index list are plain copies.  out == logits with equal pitch is the
 * in-place apply; any other overlap of out with logits, mask or indices is
 * MI_ERR_ALIAS.  One kernel, one pass over every row, without an index list
 * or with one of at most 1024 entries (each block looks for its row in the
 * list); with a longer list, two kernels (a copy, then the in-place apply of
 * the listed rows on out).
 */
mi_status_t mi_apply_bitmask_out(
    void *out, int64_t out_row_stride,
    const void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int32_t *indices, int64_t num_indices,
    double fill_value, hipStream_t stream);

/*
 * Gated in-place apply with a per-row report (TensorRT-Edge-LLM "Guided
 * Decoder": the apply kernel leaves a row whose per-row flag is zero alone;
 * a row whose mask admits no token is unsatisfiable, rowHasAnyToken).
 * Rows 0..rows-1 as without indices (mask_rows >= rows).  Leading logits
 * dimensions such as [activeBatchSize, rowsPerSlot] are flattened rows.
 *
 * row_needs_mask: device int8 [rows], or NULL for every row; a zero entry
 *   leaves that logits row untouched.
 * row_any_allowed: device uint8 [rows] output, or NULL.  Entry r becomes 1
 *   when row r still admits at least one of its first V tokens after the
 *   call -- for a gated-off row that is V > 0; for the others, whether any
 *   of mask bits [0, V) is set (bits past V never count) -- else 0.  Every
 *   entry is written; no initialisation is needed.
 * Neither may overlap logits, mask or each other (MI_ERR_ALIAS).
 */
mi_status_t mi_apply_bitmask_rows(
    void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int8_t *row_needs_mask, uint8_t *row_any_allowed,
    double fill_value, hipStream_t stream);

/* As above, with an explicit kernel variant (MI_VARIANT_WRONLY: in place only). */
mi_status_t mi_apply_bitmask_inplace_ex(
    void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int32_t *indices, int64_t num_indices,
    double fill_value, mi_variant_t variant, hipStream_t stream);

mi_status_t mi_apply_bitmask_out_ex(
    void *out, int64_t out_row_stride,
    const void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int32_t *indices, int64_t num_indices,
    double fill_value, mi_variant_t variant, hipStream_t stream);

/*
 * Fused apply + sample: one token per row (logits-processor page, "Ops:
 * sample" and "How it works").  Per row: z = logit / temperature; top-k,
 * top-p and min-p each keep the largest-probability tokens above a cutoff
 * (k <= 0, p >= 1, m <= 0 disable them; ties at a cutoff are kept) and the
 * kept set is their intersection; one token is drawn from it with
 * probability proportional to its softmax probability (Gumbel-max).
 * A temperature that is not positive (<= 0, or NaN) takes the argmax
 * (lowest index on ties).  top_p <= 0 keeps only the largest value and its
 * ties.
 *
 * Candidates are the tokens v < V whose logit is finite and, when mask is
 * not NULL, whose bit v % 32 of word mask[row, v / 32] is set -- the apply
 * is folded into the reads and the logits are not modified; a masked token
 * is never drawn.  With a mask the vocab-size rule and mask_rows >= rows
 * are those of the apply; without one (mask == NULL, mask_* ignored)
 * V = vocab_size, or cols when vocab_size == -1.  A row with no candidate
 * gets token -1.  V above 2^28 is rejected with MI_ERR_BAD_SHAPE.
 *
 * Randomness: Philox4x32-10 (Salmon et al., SC 2011) with key (seed low,
 * seed high) and, for token v of row r, counter (v / 4, r, offset low,
 * offset high), word v % 4; u = (floor(x / 2^9) + 1/2) / 2^23; Gumbel
 * variate -ln(-ln u).  The same (seed, offset) replays the same tokens;
 * advance offset (or seed) per decoding step.
 *
 * params: HOST struct.  Each per-row array is a device array of `rows`
 * entries, or NULL to use the matching *_all value for every row.
 * tokens: device int64 [rows] output (8-byte aligned; may not overlap logits
 * or mask).  Asynchronous on `stream` like the apply calls.  It uses no
 * device memory beyond its arguments: its working space is on chip (when
 * a row may use top-k or top-p, an LDS histogram of 131 KB per 1024-thread
 * block, one block per compute unit, or, for bf16 and fp16 batches of more
 * than 256 rows of at most 65536 tokens, of 66 KB per 512-thread block, two
 * blocks per compute unit).  With few rows and no
 * top-k, top-p or min-p it splits each row over several blocks that merge
 * their answers in `tokens` itself (three kernels on `stream`; `tokens`
 * holds intermediate values until the last one has run).
 */
typedef struct mi_sample_params {
    const float *temperature;     /* device [rows] or NULL */
    const int32_t *top_k;         /* device [rows] or NULL */
    const float *top_p;           /* device [rows] or NULL */
    const float *min_p;           /* device [rows] or NULL */
    float temperature_all;
    int32_t top_k_all;
    float top_p_all;
    float min_p_all;
    uint64_t seed;
    uint64_t offset;
} mi_sample_params_t;

mi_status_t mi_apply_bitmask_sample(
    const void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const mi_sample_params_t *params, int64_t *tokens, hipStream_t stream);

/*
 * As mi_apply_bitmask_sample (same page and section), with a device
 * workspace that lets a small batch spread its filtered rows over many
 * compute units.  Without it, each row with top-k, top-p or min-p is drawn
 * by one block, so a batch of a few such rows leaves most of the GPU idle.
 * With it, a batch of at most 32 bf16 or fp16 rows of at least 8192 tokens
 * splits each such row into segments: one kernel counts every segment's
 * allowed tokens under their 16-bit keys into the row's histogram in the
 * workspace, one finds the row's cut from it, and one draws over the
 * segments, which merge their picks in `tokens` (five kernels on `stream`
 * in all; `tokens` holds intermediate values until the last has run).  The
 * tokens are the same as without the workspace: the cut comes from the same
 * counts and the draw from the same Gumbel keys.
 *
 * The workspace also serves large batches: with a mask and a filter in
 * force for some row (top-p or min-p for rows of at most 65536 tokens, any
 * of the three for longer ones), a batch of 257 to 8192 bf16 or fp16 rows
 * of more than 16384 tokens hands out its dense rows first.  One kernel
 * marks, in one bit per row, each row whose mask allows more than 4096
 * tokens below V; the draw's blocks then take those rows first, in row
 * order, then the rest.  A dense row costs several sparse ones, and in a
 * batch that mixes them at random some compute units would otherwise get
 * two dense rows at once, or one late, and end the launch last.  The
 * tokens do not depend on the order.
 *
 * workspace: device memory of workspace_bytes bytes, 16-byte aligned, not
 * overlapping logits, mask, tokens or the per-row parameter arrays; its
 * contents on entry do not matter and are overwritten.  It is used only when
 * workspace_bytes >= mi_sample_workspace_bytes(dtype, rows, V) > 0, V being
 * the vocab size the call resolves; otherwise (NULL included) the call runs
 * as mi_apply_bitmask_sample.  Calls that share a workspace must not
 * overlap in time.  Errors as mi_apply_bitmask_sample, plus
 * MI_ERR_MISALIGNED and MI_ERR_ALIAS for a workspace that is used.
 */
mi_status_t mi_apply_bitmask_sample_ws(
    const void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const mi_sample_params_t *params, int64_t *tokens, void *workspace,
    int64_t workspace_bytes, hipStream_t stream);

/*
 * As mi_apply_bitmask_sample_ws, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace argument; the split path's
 * workspace is a device array inside the library (8 393 216 bytes, enough
 * for 32 rows), which each GPU the library runs on holds until the process
 * ends.  The array used is that of the GPU the stream runs on (the current
 * device for the null stream); its address is looked up once per device
 * (hipGetSymbolAddress with that device current, switching to it and back
 * if the stream's device is not current); the call itself allocates
 * nothing and frees nothing.
 *
 * The array holds the workspace of the largest batch that splits (32 bf16
 * or fp16 rows) and the row flags of the largest batch that orders its
 * rows (8192), so every batch runs as mi_apply_bitmask_sample_ws would with
 * a workspace, with the same tokens.  A batch that would need more than the
 * array (none under these limits) is rejected with MI_ERR_BAD_SHAPE and
 * enqueues nothing.
 *
 * All calls on one GPU share its array, and each clears what it uses on its
 * own stream before using it: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race on it and must be
 * ordered by the caller.  Errors as mi_apply_bitmask_sample, plus MI_ERR_HIP
 * when the array's address cannot be had.
 */
mi_status_t mi_apply_bitmask_sample_noalloc(
    const void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const mi_sample_params_t *params, int64_t *tokens, hipStream_t stream);

/*
 * Workspace bytes mi_apply_bitmask_sample_ws uses for `rows` rows of `vocab`
 * tokens (the resolved vocab size) of `dtype`: rows * 262288 (a histogram of
 * 65536 32-bit counts, a 128-byte map of its nonzero runs and 16 bytes of
 * results per row) when the batch can split its filtered rows; one bit
 * per row, rounded up to 256 bytes, when it can order its rows dense first
 * (bf16 or fp16, 257 to 8192 rows of more than 16384 tokens); else 0 (no
 * workspace is used).  0 for invalid arguments.  Pure host arithmetic; no
 * HIP call.
 */
int64_t mi_sample_workspace_bytes(mi_dtype_t dtype, int64_t rows, int64_t vocab);

/*
 * Host-memory apply, for logits and masks that live on the CPU (XGrammar
 * "Bitmask Operations", Notes: Device: CPU tensors get a CPU
 * implementation).  Same arguments, rules and results as the device entry
 * points, except that every pointer is HOST memory, the call runs
 * synchronously on up to `num_threads` threads, the calling thread among
 * them (<= 0: half the hardware threads; at most 256; inputs below 2^20
 * elements run on the calling thread alone; rows a worker thread could not
 * be started for run on the calling thread), and -- since the host can read
 * the index list -- an index outside [0, min(rows, mask_rows)) is
 * MI_ERR_BAD_INDICES before anything is written.  They allocate nothing,
 * never touch a GPU and are never used for device memory.
 */
mi_status_t mi_apply_bitmask_inplace_host(
    void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int32_t *indices, int64_t num_indices,
    double fill_value, int num_threads);

mi_status_t mi_apply_bitmask_out_host(
    void *out, int64_t out_row_stride,
    const void *logits, mi_dtype_t dtype, int64_t rows, int64_t cols, int64_t logits_row_stride,
    const int32_t *mask, int64_t mask_rows, int64_t mask_cols, int64_t mask_row_stride,
    int64_t vocab_size, const int32_t *indices, int64_t num_indices,
    double fill_value, int num_threads);

/*
 * Host helpers (no device access, usable without a GPU).
 *
 * mi_resolve_vocab_size: the V the apply calls use (XGrammar "Bitmask
 * Operations", Notes: Padding); *vocab_out receives it.  MI_ERR_BAD_VOCAB
 * or MI_ERR_BAD_SHAPE as for the apply calls.
 *
 * mi_fill_value_bits: the bit pattern the apply calls store for fill_value
 * in dtype (rounded once to nearest-even), in the low 16 or 32 bits of
 * *bits_out.
 */
mi_status_t mi_resolve_vocab_size(int64_t cols, int64_t mask_cols, int64_t vocab_size,
                                  int64_t *vocab_out);
mi_status_t mi_fill_value_bits(double fill_value, mi_dtype_t dtype, uint32_t *bits_out);

/* Static text for a status code ("MI_OK", ...); never NULL. */
const char *mi_status_string(mi_status_t status);

/* Detail of this thread's last non-OK return ("" if none yet). */
const char *mi_last_error_message(void);

/*
 * Which loop the host-memory entry points run, fixed for the process:
 * "avx512" (one masked vector store per mask word, on x86 with AVX-512 F and
 * BW) or "portable" (one store per masked token).  The environment variable
 * MI_BITMASK_HOST_ISA=portable, read at the first host call, selects the
 * portable loop.  Static text; never NULL.
 */
const char *mi_host_isa(void);

#ifdef __cplusplus
}
#endif

#endif /* MI_BITMASK_H */

/*
 * lora_mi355x.h -- C ABI of the segmented-gather multi-LoRA library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow three vLLM API documentation pages:
 *   - "lora_kernel_metadata": class LoRAKernelMeta (make, _reset,
 *     prepare_tensors, meta_args);
 *   - "punica_gpu": class PunicaWrapperGPU (add_shrink, add_expand,
 *     add_lora_linear);
 *   - "punica_tpu": class PunicaWrapperTPU (add_expand's running column
 *     offset, _apply_bias).
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers unless marked "host".
 *   - Every call is asynchronous on `stream` (NULL = the null stream); none
 *     allocates memory, synchronizes the device, or keeps state between calls,
 *     so prepare + shrink + expand on fixed buffers can be captured in a HIP
 *     graph.  Calls that overlap on the same buffers race.
 *   - The caller owns every buffer.
 *   - Return value: LORA_OK (0) or a negative lora_status_t, decided on the
 *     host before anything is launched (nothing is launched on error), or
 *     LORA_ERR_LAUNCH if the HIP runtime refused a launch.
 *   - Element types: token ids and metadata int32; x, y, weights and bias
 *     bfloat16 (raw 16-bit patterns); the shrink buffer float32.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum lora_status {
    LORA_OK = 0,
    LORA_ERR_NULL = -1,          /* a required pointer is NULL */
    LORA_ERR_NUM_TOKENS = -2,    /* N < 0, N > max_num_tokens, or N differs from the prepared N */
    LORA_ERR_SHAPE = -3,         /* hidden / rank / slice widths / leading dims out of range */
    LORA_ERR_MAX_LORAS = -4,     /* max_loras outside [1, LORA_MAX_LORAS] */
    LORA_ERR_BUFFER = -5,        /* metadata region too small or misaligned */
    LORA_ERR_ALIGN = -6,         /* a bf16 / fp32 operand is not 16-byte aligned as required */
    LORA_ERR_SLICES = -7,        /* num_slices outside [1, LORA_MAX_SLICES] */
    LORA_ERR_LAUNCH = -8,        /* the HIP runtime rejected a kernel launch or copy */
    LORA_ERR_ID_RANGE = -9,      /* device-side only: written to meta->status by prepare */
    LORA_ERR_SYNC = -10,         /* device-side only: a device wait of a shrink timed out (meta->status) */
    LORA_ERR_SCRATCH = -11       /* lora_shrink_expand_noalloc: the buffer would exceed the library's array */
} lora_status_t;

#define LORA_MAX_LORAS 1023      /* ids 0 .. 1022; -1 = no LoRA */
#define LORA_MAX_SLICES 8
#define LORA_MAX_RANK 128
#define LORA_MAX_TOKENS 2097152  /* tokens per batch */

/*
 * Per-batch kernel metadata (LoRAKernelMeta on the "lora_kernel_metadata"
 * page).  All arrays are views into ONE caller-owned device region bound by
 * lora_meta_bind(); sizes are those make() gives:
 *   token_lora_mapping     int32[max_num_tokens]  copy of the batch's ids
 *   token_indices_sorted   int32[max_num_tokens]  token indices, stable-sorted by id
 *   active_lora_ids        int32[max_loras + 1]   distinct ids present, ascending,
 *                                                 -1 first when present; padding -1
 *   num_tokens_per_lora    int32[max_loras + 1]   tokens per active id; padding 0
 *   lora_token_start_loc   int32[max_loras + 2]   0, then running sums; padding 0
 *   no_lora_flag           int32[1]   1 when every id is -1 (or N == 0)
 *   status                 int32[1]   0, or LORA_ERR_ID_RANGE when some id was
 *                                     outside [-1, max_loras) (such ids count as -1)
 *   sync                   int32[128 * (ceil(T / 16) + min(max_loras + 1, T) + 1)]
 *                          followed by float32[64 * T] and float32[1024 * min(T, 2048)],
 *                          T = min(max_num_tokens, 24576): counters, accumulation
 *                                     area and part slots of the one-launch calls;
 *                          then, when max_num_tokens >= 1024, int32[1024] and
 *                          float32[8 << 20]: counters and part slots of the
 *                          stream-K shrink (library-owned)
 * The struct itself lives in host memory; lora_prepare_meta() records
 * num_tokens in it.
 */
typedef struct lora_meta {
    int32_t *token_lora_mapping;
    int32_t *token_indices_sorted;
    int32_t *active_lora_ids;
    int32_t *num_tokens_per_lora;
    int32_t *lora_token_start_loc;
    int32_t *no_lora_flag;
    int32_t *status;
    int32_t *sync;           /* work counters, fp32 accumulation area and part slots of the
                                one-launch calls and of the stream-K shrink (library-owned
                                part of the region): the counters and the accumulation area
                                are zeroed by lora_prepare_meta for batches that can use
                                them and left zero by every call that completes without
                                LORA_ERR_SYNC; the part slots need no clearing */
    int32_t *host_no_lora;   /* optional host pinned word (NULL = none): prepare copies
                                no_lora_flag into it asynchronously on its stream */
    int32_t max_loras;
    int32_t max_num_tokens;
    int32_t num_tokens;      /* set by lora_prepare_meta; -1 before the first prepare */
} lora_meta_t;

/* Bytes of device memory lora_meta_bind() needs for these maximum sizes
 * (the allocation make() performs, as one region).  0 if the sizes are out
 * of range. */
size_t lora_meta_bytes(int max_loras, int max_num_tokens);

/* Carve the metadata arrays out of `dev` (device pointer, 256-byte aligned,
 * at least lora_meta_bytes() bytes) and fill `out` (host).  No device work
 * is done: the arrays hold garbage until the first lora_prepare_meta().
 * host_no_lora is set to NULL; the caller may point it at pinned host memory. */
int lora_meta_bind(void *dev, size_t bytes, int max_loras, int max_num_tokens, lora_meta_t *out);
/* (max_num_tokens above LORA_MAX_TOKENS is rejected with LORA_ERR_NUM_TOKENS.) */

/*
 * LoRAKernelMeta._reset + prepare_tensors for one batch
 * ("lora_kernel_metadata" page).  mapping: int32[num_tokens] token -> LoRA id
 * (-1 = none), device memory.  On device, in one launch:
 *   reset active ids to -1, counts and start_loc to 0; set no_lora_flag to
 *   all(mapping == -1); if set, stop there (the sorted indices are left as
 *   they were, as the pages' early return does, and so is the mapping copy
 *   for batches of up to 16384 tokens; larger batches use it as scratch);
 *   otherwise copy
 *   the mapping, stable-sort token indices by id (ascending, ties in token
 *   order), write the distinct ids with their counts, and the segment starts.
 * Ids outside [-1, max_loras) are treated as -1 and reported in meta->status.
 * The result is deterministic and bit-exact.  Records meta->num_tokens.
 */
int lora_prepare_meta(const int32_t *mapping, int num_tokens, lora_meta_t *meta, hipStream_t stream);

/*
 * lora_shrink (PunicaWrapperGPU.add_shrink on the "punica_gpu" page; the
 * fp32 buffer of add_lora_linear): for each slice i < num_slices and each
 * token t whose id m is not -1,
 *     buf[i][t][j] += scale * sum_k x[t][k] * lora_a[i][m][j][k]   (j < rank)
 * accumulated in float32.  Rows of tokens with id -1 are not touched; when
 * the no-LoRA flag is set nothing is touched.
 *   x       bf16 [num_tokens][ldx], rows 16-byte aligned (ldx % 8 == 0)
 *   lora_a  host array [num_slices] of device pointers, each bf16
 *           [max_loras][rank][hidden] (hidden contiguous), 16-byte aligned
 *   buf     float32 [num_slices][num_tokens][rank], 16-byte aligned
 *   hidden % 8 == 0, rank % 8 == 0, 8 <= rank <= LORA_MAX_RANK
 * num_tokens must equal the N of the last lora_prepare_meta() on `meta`,
 * whose results must be complete in stream order.
 * Batches of at least 1024 tokens whose segments are long enough for the
 * LDS-staged kernel may be split by K steps over the workgroups (stream-K):
 * the workgroups that start a tile in the middle store their partial sums
 * in part slots of meta->sync and count them, and the workgroup holding the
 * tile's first K steps waits on the device for that count, adds the slots
 * in order and writes buf (deterministic).  Calls sharing one metadata
 * region must then not overlap (on one stream they never do).  A wait that
 * never ends (not expected: the parts it waits for start before anything
 * that waits) gives up after about 0.1 s and sets meta->status to
 * LORA_ERR_SYNC; buf and the stream-K counters are then unspecified, and a
 * lora_prepare_meta must run before the next call.  Other shapes may split
 * K with float atomics into buf, whose last bits may then vary between runs.
 */
int lora_shrink(const void *x, int64_t ldx, int num_tokens, int hidden,
                const void *const *lora_a, int num_slices, int rank,
                float *buf, const lora_meta_t *meta, float scale, hipStream_t stream);

/*
 * lora_expand with the per-slice bias folded in (PunicaWrapperGPU.add_expand
 * on the "punica_gpu" page; the running offset of PunicaWrapperTPU.add_expand
 * and the bias rule of PunicaWrapperTPU._apply_bias on the "punica_tpu"
 * page): slice i covers columns [off_i, off_i + slice_widths[i]) of y with
 * off_0 = offset_start and off_{i+1} = off_i + slice_widths[i]; for each token
 * t whose id m is not -1 and each column c of slice i,
 *     v = sum_j buf[i][t][j] * lora_b[i][m][c - off_i][j] (+ bias[i][m][c - off_i])
 *     y[t][c] = bf16_rne((add_inputs ? y[t][c] : 0) + v)
 * accumulated in float32 with a single rounding to bfloat16.  Rows of tokens
 * with id -1 are not touched (no bias either); with the no-LoRA flag set
 * nothing is touched.
 *   buf          float32 [num_slices][num_tokens][rank], 16-byte aligned
 *   lora_b       host array [num_slices] of device pointers, bf16
 *                [max_loras][slice_widths[i]][rank] (rank contiguous)
 *   bias         NULL, or host array [num_slices] of (NULL | device bf16
 *                [max_loras][slice_widths[i]])
 *   slice_widths host int[num_slices], each > 0 and % 8 == 0
 *   y            bf16 [num_tokens][ldy], ldy % 8 == 0, offset_start % 8 == 0,
 *                offset_start + sum(slice_widths) <= ldy
 * num_tokens must equal the prepared N, as for lora_shrink.
 */
int lora_expand(const float *buf, int num_tokens, int rank,
                const void *const *lora_b, const void *const *bias,
                const int *slice_widths, int num_slices,
                void *y, int64_t ldy, int offset_start, int add_inputs,
                const lora_meta_t *meta, hipStream_t stream);

/*
 * PunicaWrapperGPU.add_lora_linear on the "punica_gpu" page in one call: that
 * method allocates a zeroed fp32 buffer, runs add_shrink into it and then
 * add_expand from it.  Here `buf` is that buffer, supplied by the caller:
 *     buf[i][t][j] = scale * sum_k x[t][k] * lora_a[i][m][j][k]    (j < rank)
 *     then y as lora_expand(buf, ...) computes it,
 * for every token t whose id m is not -1.  buf's contents on entry are
 * ignored ("=" where lora_shrink has "+=": the same result on the freshly
 * zeroed buffer of add_lora_linear, so the caller needs no clearing pass);
 * rows of tokens with id -1 are not touched, and with the no-LoRA flag set
 * nothing is.  Arguments, layouts and errors are those of lora_shrink and
 * lora_expand.
 * For batches of short segments (decode-like: expected tokens per LoRA below
 * 24, S * rank <= 64, rank <= 64) both steps run in one launch: workgroups
 * run K chunks ("parts") of a tile's shrink, adding their partial sums with
 * float atomics into the accumulation area of meta->sync, count each part
 * done, and the tile's expand waits on the device until every part is done
 * (a waiter that sees no progress runs the parts nobody has started, so the
 * wait needs no co-residency).  With at least 4 tokens per LoRA id, at most
 * 2048 tokens, at most 16 parts of 512 (hidden <= 8192) and every role
 * resident at once, the launch is laid out by LoRA id instead, reading the
 * prepared id copy (token_lora_mapping) rather than the sorted indices; its
 * parts store their sums in part slots of meta->sync and the expand adds them
 * up in part order, so buf is deterministic in that layout.
 * Other shapes launch the separate kernels (lora_shrink with buf written, not
 * accumulated, then lora_expand; a shrink split over K with float atomics
 * zeroes the active rows of buf first).  The one-launch kernels use meta->sync: calls
 * sharing one metadata region must not overlap (they are ordered on one
 * stream in normal use), and meta must have been prepared at least once since
 * it was bound; every call that completes normally leaves the counters and
 * the accumulation area zero.
 * A device-side wait that never ends (not expected: every wait is on a
 * running workgroup) gives up after about 0.1 s and sets meta->status to
 * LORA_ERR_SYNC.  After that, y, buf and the counters and accumulation area
 * of meta->sync are unspecified: the call's results must be discarded, and
 * a lora_prepare_meta must run before the next call (it clears the counters
 * and the area).  The same holds for the stream-K shrink's wait.
 */
int lora_shrink_expand(const void *x, int64_t ldx, int num_tokens, int hidden,
                       const void *const *lora_a, const void *const *lora_b, const void *const *bias,
                       const int *slice_widths, int num_slices, int rank, float *buf,
                       void *y, int64_t ldy, int offset_start, int add_inputs,
                       const lora_meta_t *meta, float scale, hipStream_t stream);

/*
 * lora_prepare_meta followed by lora_shrink_expand: a batch's metadata and its
 * first LoRA layer (LoRAKernelMeta.prepare_tensors on the "lora_kernel_metadata"
 * page, then PunicaWrapperGPU.add_lora_linear on the "punica_gpu" page), with
 * the arguments and results of those two calls.  For batches of at most 2048
 * tokens in the fused call's range it is one launch.  With at least 4 tokens
 * per LoRA id (and every role resident at once) the launch is laid out by
 * LoRA id: each workgroup picks its id's tokens out of the mapping itself
 * (no sort; the tokens come in batch order, the stable sort's order within a
 * segment) and the metadata arrays are written piecewise by each id's first
 * expander.  Otherwise every workgroup sorts the mapping in its own LDS (the
 * same stable counting sort as lora_prepare_meta) and workgroup 0 writes the
 * metadata arrays.  Outside the range the two calls are made.  buf is
 * written as by lora_shrink_expand ("=", a fresh buffer).  As for
 * lora_shrink_expand, the counters and the accumulation area in meta->sync
 * must start at zero: meta must have been prepared since it was bound with at
 * least as many tokens (or its region zeroed once when allocated); every call
 * leaves them zero.  LORA_ERR_SYNC in meta->status leaves y, buf, the
 * metadata arrays and meta->sync unspecified, as for lora_shrink_expand.
 * Records meta->num_tokens and copies the no-LoRA flag to meta->host_no_lora
 * when that is set.
 */
int lora_prepare_shrink_expand(const int32_t *mapping, int num_tokens, const void *x, int64_t ldx, int hidden,
                               const void *const *lora_a, const void *const *lora_b, const void *const *bias,
                               const int *slice_widths, int num_slices, int rank, float *buf, void *y,
                               int64_t ldy, int offset_start, int add_inputs, lora_meta_t *meta, float scale,
                               hipStream_t stream);

/*
 * lora_shrink_expand for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and errors without `buf`; the fp32 buffer of
 * the call lives in a device array of the library, 32 MiB (8388608 floats) per
 * GPU, held by each GPU the library runs on until the process ends.  Calls
 * needing num_slices * num_tokens * rank > 8388608 floats are rejected with
 * LORA_ERR_SCRATCH before anything is launched.  Every call on one GPU uses
 * that GPU's array (the device current at the call), so calls that overlap on
 * one GPU -- on different streams, or from several threads -- race; calls
 * ordered on one stream do not.  Nothing in the array needs clearing between
 * calls (the buffer is written as a fresh one).  Allocates nothing: the array's
 * address is looked up once per device on its first call.
 */
int lora_shrink_expand_noalloc(const void *x, int64_t ldx, int num_tokens, int hidden,
                               const void *const *lora_a, const void *const *lora_b, const void *const *bias,
                               const int *slice_widths, int num_slices, int rank, void *y, int64_t ldy,
                               int offset_start, int add_inputs, const lora_meta_t *meta, float scale,
                               hipStream_t stream);

/*
 * Kernel launches that lora_shrink_expand (with_prepare = 0) or
 * lora_prepare_shrink_expand (with_prepare != 0) makes for a layer of a batch
 * of num_tokens >= 1 tokens, input width `hidden`, rank `rank` and
 * num_slices slices, with the metadata sized for max_loras: 1 when the call is
 * one launch (the fused kernels' range: fewer than 24 tokens per LoRA id on
 * average, num_slices * rank <= 64, rank <= 64, and with the prepare at most
 * 2048 tokens), else the separate calls' count: prepare (with_prepare), the
 * zeroing of buf's active rows when the shrink is split over K chunks, shrink
 * and expand (prepare: lora_prepare_meta_launches).  A batch whose every id
 * is -1 still makes these launches (they
 * touch nothing).  Host only: no device work, no HIP call.  Negative
 * lora_status for arguments the calls themselves would reject.  A measurement
 * aid: it tells which kernel durations make up a call.
 */
int lora_shrink_expand_launches(int num_tokens, int max_loras, int hidden, int num_slices, int rank,
                                int with_prepare);

/* Kernel launches lora_prepare_meta makes for a batch of num_tokens tokens
 * with the metadata sized for max_loras: 2 when several workgroups sort it
 * (at least 4096 tokens, and enough of them for the id width that one
 * workgroup would take longer: one launch ranks the tokens of each chunk, the
 * next places them), else 1.  Host only.  LORA_ERR_NUM_TOKENS /
 * LORA_ERR_MAX_LORAS for arguments out of range.  A measurement aid. */
int lora_prepare_meta_launches(int num_tokens, int max_loras);

/* Static description of a status code. */
const char *lora_status_string(int status);

/*
 * Measurement aids (not part of the method; bench.py times them next to the
 * calls above as practical ceilings).
 *
 * lora_probe_read: one launch of `workgroups` workgroups of 256 threads that
 * reads `bytes` (> 0, a multiple of 16) of device memory at `src` (16-byte
 * aligned) once, with streaming 16-byte loads, each workgroup a contiguous
 * share.  `sink` is a device float[workgroups] the kernel may write (it never
 * does for data whose 16-byte words do not fold to one particular pattern).
 * lora_probe_empty: one launch of `workgroups` workgroups of 256 threads that
 * do nothing.  Both are asynchronous on `stream`; LORA_ERR_NULL /
 * LORA_ERR_SHAPE / LORA_ERR_ALIGN for bad arguments, checked on the host.
 */
int lora_probe_read(const void *src, size_t bytes, int workgroups, float *sink, hipStream_t stream);
int lora_probe_empty(int workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */

/*
 * pa_decode.h -- C ABI of the paged split-KV decode attention library for
 * AMD Instinct MI355X (gfx950).  Library: libpa_decode.so.
 *
 * What the library computes.  One decode step of paged attention: for every
 * sequence b and query head h, the softmax-weighted sum of the V rows of the
 * context_lens[b] cached tokens, with weights softmax_t(scale * <q[b,h], K_t>).
 * K_t / V_t are gathered through a block table from a paged KV cache.
 * Sources (cited by page title and section):
 *   - project_6 commit 96f4baf ("Dockerfile" commit page), V2 plan:
 *     "Phase 1" per-(sequence, head, partition) attention storing a partial
 *     output, an exp-sum and a max logit; "Phase 2" log-sum-exp merge; the
 *     512-token partition size; V1 as a single pass over the whole context.
 *   - project_6 optimizations/prefix_prefill_patch.py (commit fee8f1b),
 *     "_PARTITION_SIZE inconsistency": both phases must use one partition size.
 *     Here it is a single run-time argument, so they cannot disagree.
 *   - project_6 commit a2a5dd8 ("computility-run.yaml" commit page), decode
 *     path summary: V1 for contexts up to 8192 tokens, V2 above (available as
 *     a setting; the default rule is the one measured on MI355X, see
 *     pa_set_v1_max_context).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * All tensor pointers are DEVICE pointers, owned by the caller; the library
 * never frees or retains them past the call.  Logical shapes:
 *   q, out          [S, Hq, D]          element type = dims->dtype
 *   k_cache,v_cache [NB, Hkv, 16, D]    element type = dims->dtype
 *   block_tables    [S, MB]   int32     physical block ids into the pool
 *   context_lens    [S]       int32     tokens cached per sequence
 * Memory layout: row-major by default; the stride fields of pa_dims_t describe
 * strided views (q or out inside a fused QKV / output buffer, K and V
 * interleaved per block, a block table that is a column slice of a wider one).
 * The innermost (head-dim) stride must be 1 and each 16-token block of one KV
 * head must be contiguous ([16, D] dense).
 * Token t of sequence b is slot (t % 16) of physical block
 * block_tables[b][t / 16].  Query head h reads KV head h / (Hq / Hkv).
 * q, out, k_cache and v_cache must be 16-byte aligned, and so must every q / out
 * row and every cache block (strides times element size multiples of 16 bytes);
 * block_tables and context_lens 4-byte aligned.  PA_ERR_ALIGN otherwise.
 * out must not alias any input; it is fully overwritten (a sequence with no
 * tokens gets 0).  out takes the element type of q, rounded to nearest even
 * from the fp32 accumulator.
 *
 * Supported: dtype in {PA_F32, PA_F16, PA_BF16}; D in {128, 256};
 * block_size == 16; G = Hq / Hkv in {1, 2, 4, 8, 16}.  partition_size must be
 * a positive multiple of 16.
 *
 * Every call validates its arguments on the host before touching the GPU and
 * returns a pa_status_t; pa_last_error() gives a message for the calling
 * thread.  No host synchronisation happens: work is enqueued on `stream`
 * (a hipStream_t; NULL means the default stream) and context_lens is only
 * read on the device.  Block ids outside [0, NB) are read as block 0 and a
 * context length above MB*16 is clamped to MB*16: such inputs give
 * unspecified results but never an access outside the caller's buffers.
 *
 * Scheduling (performance only; results never depend on it).  With 2..512
 * sequences the V2 kernel dispatches only the partitions that exist,
 * contiguously, and V1 on the four-wave matrix-core shape (at least 256
 * (sequence, KV head) pairs, tables over 1024 tokens) takes sequences longest
 * context first.  Each work-group derives its item from all S context lengths
 * on the device.  Above 512 sequences both kernels take their items in grid
 * order: V2 launches every partition slot and the empty ones return at once.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_DTYPE = -2,       /* unknown element type */
  PA_ERR_SHAPE = -3,       /* inconsistent or non-positive sizes */
  PA_ERR_ALIGN = -4,       /* a tensor pointer or row is not 16-byte aligned */
  PA_ERR_PARTITION = -5,   /* partition_size <= 0 or not a multiple of block_size */
  PA_ERR_UNSUPPORTED = -6, /* valid but not built: D, block_size, G, too many partitions */
  PA_ERR_WORKSPACE = -7,   /* caller workspace NULL or smaller than pa_workspace_bytes() */
  PA_ERR_HIP = -8,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_INTERNAL = -9,
  PA_ERR_STRIDE = -10      /* a stride the kernels cannot take (innermost != 1, overlap) */
} pa_status_t;

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype_t;

/* Decode-path selector for pa_decode_ex. */
enum { PA_PATH_AUTO = 0, PA_PATH_V1 = 1, PA_PATH_V2 = 2 };

/* Problem sizes and strides, passed by pointer to every entry point.  Plain
 * integers.  Strides are in elements of the tensor's own type; 0 selects the
 * row-major value (given in brackets), so a zero-initialised stride block
 * describes dense tensors.  Rules (checked on the host, before any HIP call):
 *   q / out: *_stride_dim must be 0 or 1 (PA_ERR_STRIDE otherwise); the head and
 *     sequence strides must be positive and below 2^31, with every row start
 *     16-byte aligned (PA_ERR_ALIGN).  out rows must not overlap:
 *     out_stride_head >= D and out_stride_seq >= (Hq - 1) * out_stride_head + D
 *     (PA_ERR_STRIDE).  q rows may overlap (q is only read).
 *   kv_stride_block: distance between consecutive blocks of k_cache and of
 *     v_cache (the same for both), >= Hkv*16*D, 16-byte multiple; within a block
 *     the layout is [Hkv, 16, D] dense.  Setting it to 2*Hkv*16*D describes K and V
 *     interleaved per block ([NB, 2, Hkv, 16, D] with k_cache = &kv[0][0] and
 *     v_cache = &kv[0][1]).
 *   bt_stride_seq: int32 entries between block-table rows, >= MB. */
typedef struct pa_dims {
  int32_t num_seqs;           /* S   (0 is allowed: nothing to do) */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;           /* D */
  int32_t block_size;         /* tokens per cache block; must be 16 */
  int32_t num_blocks;         /* NB: blocks in the KV pool */
  int32_t max_blocks_per_seq; /* MB: block_tables row length */
  int32_t dtype;              /* pa_dtype_t of q, k_cache, v_cache and out */
  int64_t q_stride_seq;       /* [Hq*D] */
  int64_t q_stride_head;      /* [D] */
  int64_t q_stride_dim;       /* [1]; must be 0 or 1 */
  int64_t out_stride_seq;     /* [Hq*D] */
  int64_t out_stride_head;    /* [D] */
  int64_t out_stride_dim;     /* [1]; must be 0 or 1 */
  int64_t kv_stride_block;    /* [Hkv*16*D] */
  int64_t bt_stride_seq;      /* [MB] */
} pa_dims_t;

/*
 * pa_decode -- one decode step, path chosen by context length.
 * The context bound used for planning is MB*16 (the block-table capacity); the
 * path follows pa_set_v1_max_context's rule (V1, or V2 with partitions of
 * partition_size tokens).  V2 uses a library-owned
 * workspace that grows on demand (hipMalloc on the first call that needs
 * more) and is kept per device; calls that overlap on one device from
 * different streams must use pa_decode_ex with their own workspaces.
 * With the library's workspace, V2 can run as ONE launch (see pa_set_fused): the
 * phase-1 work-groups publish their partials and the merge work-groups of the same
 * grid fold them once every partition of their (sequence, KV head) is in.  The
 * result equals the two-launch V2 to rounding (same partials, the same log-sum-exp
 * merge, a different summation tree).
 * Returns PA_OK or an error status; on error nothing was enqueued.
 */
pa_status_t pa_decode(const pa_dims_t* dims, void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, int32_t partition_size,
                      void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory
 * (code under stream/graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, path rule and result as pa_decode, but the V2
 * workspace is a static device array of PA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library (one per device, held until the process ends) instead of hipMalloc'd
 * memory: the call makes no allocating HIP or library call.  A call whose
 * workspace (pa_workspace_bytes with max_context_len 0) exceeds that size returns
 * PA_ERR_WORKSPACE and enqueues nothing.  Every call on a device shares that
 * device's array: calls that overlap on one device (different streams, or host
 * threads) race and give undefined results.  The array needs no initialisation
 * (every value read was written earlier in the same call).
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status_t pa_decode_noalloc(const pa_dims_t* dims, void* out, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, int32_t partition_size, void* stream);

/*
 * pa_workspace_bytes -- bytes of device workspace a V2 call needs.
 * max_context_len <= 0 means MB*16.  Layout (all fp32, 256-byte aligned
 * sections), with Pmax = ceil(max_context_len / partition_size):
 *   tmp_out     [S, Hq, Pmax, D]  normalised partial output of each partition
 *   max_logits  [S, Hq, Pmax]     max over the partition of scale*q.k
 *   exp_sums    [S, Hq, Pmax]     sum over the partition of exp(logit - max)
 * followed by the piece area of the work split (see pa_set_work_split), with
 * slots = min(1024, S*Hkv*Pmax*2^s) where 2^s (at most 16) is the largest number
 * of equal pieces of a multiple of 64 tokens that partition_size divides into
 * (0 slots if that is 1), G = Hq/Hkv:
 *   piece_out   [slots, G, D]     normalised partial output of each piece
 *   piece_max   [slots, G]        max over the piece of scale*q.k
 *   piece_sum   [slots, G]        sum over the piece of exp(logit - max)
 * pa_workspace_layout() returns the offsets.  The contents need no
 * initialisation.  Returns 0 when the arguments are invalid (see pa_last_error()).
 */
size_t pa_workspace_bytes(const pa_dims_t* dims, int64_t max_context_len,
                          int32_t partition_size);

/* Workspace layout for these arguments, written to layout[0..PA_LAYOUT_FIELDS-1]:
 * Pmax; the byte offsets of tmp_out, max_logits and exp_sums; the number of
 * piece slots; the byte offsets of piece_out, piece_max and piece_sum; the
 * total bytes. */
#define PA_LAYOUT_FIELDS 9
pa_status_t pa_workspace_layout(const pa_dims_t* dims, int64_t max_context_len,
                                int32_t partition_size, int64_t* layout);

/*
 * pa_decode_ex -- pa_decode with caller-chosen path, context bound and
 * workspace.  path: PA_PATH_AUTO (pa_choose_path's rule), PA_PATH_V1 or PA_PATH_V2.
 * max_context_len: upper bound on every context_lens[b] (<= 0: MB*16); it
 * sizes the partition grid, so a smaller bound means fewer idle work-groups.
 * It must not exceed MB*16.  A context longer than the bound is attended only
 * over a prefix: its first ceil(max_context_len / partition_size) *
 * partition_size tokens on V2, its first max_context_len rounded up to a
 * multiple of 16 on V1.
 * workspace: device memory of >= pa_workspace_bytes(dims, max_context_len,
 * partition_size) bytes, needed only when the path taken is V2 (may be NULL
 * for V1).  V2 enqueues two launches, phase 1 then phase 2; after the call the
 * workspace holds the phase-1 partials (layout above) of every partition of a
 * sequence with more than one partition, except the partitions the work split
 * cut into pieces: their partial states are in their pieces' slots.  Calls that
 * overlap on the same workspace race.
 */
pa_status_t pa_decode_ex(const pa_dims_t* dims, void* out, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, int32_t partition_size,
                         void* stream, void* workspace, size_t workspace_bytes,
                         int64_t max_context_len, int32_t path);

/*
 * pa_decode_profiled -- pa_decode_ex that also times the attention kernel (the
 * phase-1 kernel of V2, or the V1 kernel): attn_start_event / attn_stop_event
 * (hipEvent_t created by the caller, or NULL) are recorded by the runtime when
 * that kernel starts and ends, without adding queue packets between kernels.
 * workspace == NULL selects the library-owned workspace as in pa_decode.
 * For measurement harnesses; results are identical to pa_decode_ex.
 */
pa_status_t pa_decode_profiled(const pa_dims_t* dims, void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               float scale, int32_t partition_size, void* stream, void* workspace,
                               size_t workspace_bytes, int64_t max_context_len, int32_t path,
                               void* attn_start_event, void* attn_stop_event);

/*
 * pa_v2_partition -- V2 phase 1 as its own launch (project_6 commit 96f4baf page,
 * "Phase 1: Per-partition attention").  One work-group per (partition, KV
 * head, sequence) computes, for every query head of the group, the partial
 * output, exp-sum and max logit of its partition and writes them to the
 * workspace (layout in pa_workspace_bytes).  A sequence whose context fits
 * in one partition gets its final result written straight to out instead,
 * and a sequence with no tokens gets out = 0.
 */
pa_status_t pa_v2_partition(const pa_dims_t* dims, void* out, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int32_t partition_size, int64_t max_context_len,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_v2_reduce -- V2 phase 2 as its own launch (project_6 commit 96f4baf page, "Phase 2:
 * Cross-partition reduction (log-sum-exp)").  For each (sequence, query
 * head) with more than one partition: M = max_p max_logits[p],
 * r_p = exp(max_logits[p] - M) * exp_sums[p], out = sum_p r_p tmp_out[p] /
 * sum_p r_p.  Reads the workspace written by pa_v2_partition with the same
 * dims, partition_size and max_context_len.
 */
pa_status_t pa_v2_reduce(const pa_dims_t* dims, void* out, const int32_t* context_lens,
                         int32_t partition_size, int64_t max_context_len,
                         const void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_v1 -- V1: one pass over the whole context per (KV head, sequence), the
 * single-launch path (project_6 commit 96f4baf page, V1 limitation note).
 * Same arithmetic as phase 1 with one partition spanning max_context_len
 * (<= 0: MB*16) tokens; writes out directly; needs no workspace.
 */
pa_status_t pa_v1(const pa_dims_t* dims, void* out, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_tables,
                  const int32_t* context_lens, float scale, int64_t max_context_len,
                  void* stream);

/* Path pa_decode / PA_PATH_AUTO would take for this context bound (<= 0:
 * MB*16) and partition size: PA_PATH_V1 or PA_PATH_V2, or a negative
 * pa_status_t for invalid dims. */
int32_t pa_choose_path(const pa_dims_t* dims, int64_t max_context_len, int32_t partition_size);

/* V1/V2 rule.  tokens >= 0: the pages' context-length rule, V1 iff the context
 * bound <= tokens (project_6 commit a2a5dd8 page, decode paths: 8192); 0 means
 * never V1.  tokens < 0 (the default): the rule measured on MI355X (GPU-side step
 * times) -- V1 iff the bound is at most 256 tokens, or S*Hkv >= 256 so that the
 * one-work-group-per-(sequence, KV head) V1 grid already fills the 256 compute
 * units; V2 otherwise (with fewer sequences V2's work split reaches more units).
 * The environment variable PA_V1_MAX_CONTEXT sets the initial value.  The getter
 * returns -1 for the measured rule.  Process-wide; safe from any thread. */
void pa_set_v1_max_context(int64_t tokens);
int64_t pa_get_v1_max_context(void);

/* ceil(n / partition_size) for n >= 0 (0 for n == 0); -1 for invalid input. */
int64_t pa_num_partitions(int64_t n, int32_t partition_size);

/* Message describing the last non-OK status returned on this thread. */
const char* pa_last_error(void);

/* Frees the library-owned workspaces (all devices).  Must not overlap with
 * a running pa_decode call. */
void pa_release(void);

/* Library version string, e.g. "pa_decode 0.1.0 gfx950". */
const char* pa_version(void);

/* Single-launch V2 of pa_decode, pa_decode_noalloc and pa_decode_profiled with
 * the library's workspace.  mode 0 (default): two launches.  mode 1: one launch
 * whenever the shape allows it (S*Hkv <= 256; S*Hq*8 merge work-groups no more than
 * the phase-1 work-groups and at most 4096; at most 4096 partial states per head;
 * workspace below 2 GiB), two launches otherwise.  On MI355X one launch measured
 * slower on a 100K-token context and equal on a mixed batch, hence the default.
 * pa_decode_ex (caller workspace) and the phase entry points always use two
 * launches.  Env PA_FUSED sets the initial value.  Process-wide.  Returns
 * PA_ERR_UNSUPPORTED for another mode. */
pa_status_t pa_set_fused(int32_t mode);
int32_t pa_get_fused(void);
/* 1 if V2 on the library's workspace (pa_decode, pa_decode_noalloc, or
 * pa_decode_profiled with no workspace, whenever they take V2) runs as one launch
 * for these dims and partition size under the current settings, 0 if it takes two
 * launches, or a negative pa_status_t.  Reads the device's compute-unit count
 * (PA_ERR_HIP without a device). */
int32_t pa_fused_applies(const pa_dims_t* dims, int32_t partition_size);

/* Tuning knob for the fp16/bf16 kernel with G >= 4: work-group shape
 *   0 = 2 waves per (partition, KV head, sequence), 3-deep (D=128) / 2-deep
 *       (D=256) register pipeline per wave
 *   1 = 1 wave, 2-deep pipeline
 *   2 = 4 waves, 2-deep pipeline
 *   3 = 1 wave, 5-deep / 3-deep pipeline
 *  -1 = automatic (the default): 2 when a work-group covers more than 1024
 *       tokens, else for grids of >= 512 work-groups 1 (V2) or 3 (V1),
 *       else 0.
 * All variants compute the same result (to rounding).  The environment
 * variable PA_MFMA_VARIANT sets the initial value.  Process-wide; do not
 * change it while another thread is launching.  Returns PA_ERR_UNSUPPORTED
 * for an unknown variant. */
pa_status_t pa_set_mfma_variant(int32_t variant);
int32_t pa_get_mfma_variant(void);

/*
 * Work split of the V2 path of pa_decode / pa_decode_ex / pa_decode_profiled (a
 * load-balancing choice of this implementation; the pages fix the partials per
 * partition, not how the work-groups that produce them are cut).  Phase-1
 * items are (partition, KV head, sequence), linear index
 * p + Pmax*(h + Hkv*b), dispatched in that order.  A cut item runs as 2^s
 * work-groups, piece c covering tokens [p*P + c*P/2^s, p*P + (c+1)*P/2^s), each
 * writing its (max, exp-sum, normalised output) to a piece slot; phase 2 folds
 * a cut partition's non-empty pieces in place of its partial (same log-sum-exp
 * rule, so the output agrees to rounding).  pa_v2_partition / pa_v2_reduce /
 * pa_v1 never cut.
 * pieces: -1 automatic (default): with C compute units and W items, cut
 *            every item into the most pieces that keep W*pieces <= 2C when
 *            W < C; else cut the last r = W mod C items (if 0 < r <= C/2)
 *            into the fewest pieces >= 2 that make r*pieces a multiple of C,
 *            or, if none does, into the most pieces allowed;
 *          0 or 1: never cut;
 *          2, 4, 8, 16: cut every item from first_item on into that many pieces.
 * The number of pieces is lowered to what partition_size allows (pieces of
 * a multiple of 64 tokens); if the cut items' pieces exceed the workspace's piece
 * slots, only the last items that fit are cut.  first_item is used only with a
 * fixed number of pieces.  Process-wide; returns PA_ERR_UNSUPPORTED for another
 * pieces value and PA_ERR_SHAPE for a negative first_item.
 */
pa_status_t pa_set_work_split(int32_t pieces, int64_t first_item);
/* Current setting: returns pieces, writes first_item if the pointer is non-NULL. */
int32_t pa_get_work_split(int64_t* first_item);
/* Split a V2 call with these arguments would use under the current setting,
 * written to plan[0..3]: items W, first cut item (W if none), pieces per cut
 * item (1 if none), phase-1 work-groups.  The automatic setting reads the
 * current device's compute-unit count (PA_ERR_HIP without a device). */
pa_status_t pa_split_plan(const pa_dims_t* dims, int64_t max_context_len, int32_t partition_size,
                          int64_t* plan);

/*
 * pa_copy_blocks -- KV-cache block copy of prefix caching (copy-on-write of a
 * shared block).  Source: project_6_baseline5 GROUND_TRUTH_STATUS_v2.md, section
 * "路径 3" (prefix caching on; its cache copy kernel named as not optimised).
 * For each pair i of block_pairs ([num_pairs][2] int32 on the device: src, dst),
 * block dst of k_cache (and of v_cache) becomes a bitwise copy of block src.
 * A block of one pool is block_bytes contiguous bytes (Hkv*16*D*element bytes
 * in the [num_blocks, Hkv, 16, D] layout); num_blocks bounds both ids.
 * v_cache may be NULL (K pool only).  Pointers: device memory owned by the
 * caller; k_cache / v_cache 16-byte aligned, block_pairs 4-byte aligned.
 * A pair with an id outside [0, num_blocks) is skipped (nothing is written).
 * Pairs are copied in parallel: destinations must be distinct and must not be
 * among the sources (identity pairs aside), otherwise the result is
 * unspecified (but nothing outside the listed dst blocks is written).
 * Asynchronous on stream; num_pairs == 0 is a no-op.  Returns PA_ERR_SHAPE for
 * block_bytes not a positive multiple of 16 (or >= 2^31), num_blocks outside
 * [1, 2^31) or num_pairs < 0; PA_ERR_NULL / PA_ERR_ALIGN for pointers;
 * PA_ERR_HIP if the launch fails.
 */
pa_status_t pa_copy_blocks(void* k_cache, void* v_cache, int64_t block_bytes, int64_t num_blocks,
                           const int32_t* block_pairs, int64_t num_pairs, void* stream);
/* pa_copy_blocks plus start / stop timestamps (hipEvent_t, may be NULL) recorded by the
 * runtime when the copy kernel starts and ends. */
pa_status_t pa_copy_blocks_profiled(void* k_cache, void* v_cache, int64_t block_bytes,
                                    int64_t num_blocks, const int32_t* block_pairs,
                                    int64_t num_pairs, void* stream, void* start_event,
                                    void* stop_event);

/*
 * Paged prefix-prefill attention.  Source: project_6
 * optimizations/prefix_prefill_patch.py (commit fee8f1b), docstring: the
 * prefix_prefill kernel, Flash-Attention style over query tiles and K/V tiles,
 * fp16/bf16, head_dim 128 (256 less often), GQA; and the "Dockerfile" commit page (project_6 commit
 * 96f4baf), "What CAN be optimized", items 1-2 (the same kernel; prefill chunks).
 * What it computes (the plainest reading of the pages): sequence b has a prefix of
 * c_b = context_lens[b] tokens in the paged cache (block_tables as in decode) and a
 * chunk of L_b = query_start[b+1] - query_start[b] new tokens, packed over the batch
 * in q [T, Hq, D], k_new / v_new [T, Hkv, D].  New token i attends, with decode's
 * softmax attention, to the c_b prefix tokens and to new tokens 0..i (causal):
 *   out[query_start[b] + i, h, :] = sum_j softmax_j(scale * <q, k_j>) v_j.
 * The new tokens' K/V are read from k_new / v_new only (writing them into the cache
 * is a separate step).  Layouts and dtypes as in decode; out [T, Hq, D] in q's dtype.
 * Built: fp16 and bf16, head_dim 128 and 256, block_size 16, Hq/Hkv in {1, 2, 4, 8, 16}
 * (others: PA_ERR_UNSUPPORTED).  query_start must be non-decreasing from 0 with
 * query_start[S] <= T (rows past T are not read or written); a context length is
 * clamped to MB*16.  max_query_len bounds every L_b and sizes the grid (<= 0: T);
 * a longer chunk is computed only for its first max_query_len tokens.  A prefix
 * block id outside [0, NB) reads its 16 tokens as zero keys and zero values (each
 * still takes a softmax weight, with logit 0): no access leaves the caller's buffers.
 */
typedef struct pa_prefill_dims {
  int32_t num_seqs;            /* S */
  int32_t num_tokens;          /* T: rows of q, k_new, v_new and out */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv */
  int32_t head_dim;            /* D */
  int32_t block_size;          /* 16 */
  int32_t num_blocks;          /* NB of the cache pools */
  int32_t max_blocks_per_seq;  /* MB: block_tables row length */
  int32_t dtype;               /* pa_dtype_t of q, k_new, v_new, caches and out */
  int32_t max_query_len;       /* bound on L_b (<= 0: num_tokens) */
} pa_prefill_dims_t;

pa_status_t pa_prefill(const pa_prefill_dims_t* dims, void* out, const void* q,
                       const void* k_new, const void* v_new, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start, float scale,
                       void* stream);
/* pa_prefill plus start / stop timestamps (hipEvent_t, may be NULL) recorded by the
 * runtime when the prefill kernel starts and when the call's last kernel ends (bf16 in
 * mode 0: the recompute launch, see pa_set_prefill_mode). */
pa_status_t pa_prefill_profiled(const pa_prefill_dims_t* dims, void* out, const void* q,
                                const void* k_new, const void* v_new, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start,
                                float scale, void* stream, void* start_event, void* stop_event);

/* pa_prefill with a caller-provided workspace instead of the library's (for calls that
 * overlap on one device from different streams: each needs a workspace of its own).
 * workspace_bytes must be at least pa_prefill_workspace_bytes(dims) under the settings
 * in force at the call (0: workspace may be NULL); the workspace is 256-byte aligned, and
 * its first 320 KiB (a counter region) must be zero before its first use; every call
 * leaves them zero.  PA_ERR_WORKSPACE if it is NULL or too small where one is needed,
 * PA_ERR_ALIGN if it is misaligned. */
pa_status_t pa_prefill_ex(const pa_prefill_dims_t* dims, void* out, const void* q,
                          const void* k_new, const void* v_new, const void* k_cache,
                          const void* v_cache, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes a prefill with these dims needs under the current settings (the planned
 * schedule's item list, partial states and counter region; 0 when the call takes the grid
 * schedule), or a negative pa_status_t.  Reads the device's compute-unit count (PA_ERR_HIP
 * without a device).  The library's own prefill workspace is separate from pa_decode's,
 * so a decode and a prefill call may overlap on two streams. */
int64_t pa_prefill_workspace_bytes(const pa_prefill_dims_t* dims);

/* How pa_prefill feeds the probabilities P to the PV products (the matrix cores take
 * 16-bit operands).  Process-wide; env PA_PREFILL_MODE sets the initial value.
 *   0 (default): P as one fp16 value (11 significant bits) and V as fp16; bf16 V is
 *     converted when staged, exactly for |v| < 65536 (below fp16's normal range the
 *     absolute error is at most 2^-25).  For bf16 each call then makes a second
 *     launch that returns at once unless the first one ended with a non-finite
 *     accumulator somewhere (a V value beyond fp16's range becomes an infinity there;
 *     non-finite inputs do the same); in that case it recomputes the whole call as in
 *     mode 1.
 *   1: P as a 16-bit high part plus a 16-bit low part in the input type (about 16
 *     significant bits), V as given; twice the PV products.
 * Both meet |out - ref| <= 2e-3 + 1e-2 |ref| against exact attention for N(0, 1)
 * inputs at scales up to 0.5; P rounded to bf16 alone does not.  The overflow marks
 * of mode 0 live in 1024 words of static device memory, one per call (round robin):
 * a call's mark can be lost only if 1024 later bf16 calls on the same device are
 * enqueued before its recompute launch runs.  Returns PA_ERR_UNSUPPORTED for another
 * mode. */
pa_status_t pa_set_prefill_mode(int32_t mode);
int32_t pa_get_prefill_mode(void);

/* Load balance of pa_prefill in mode 0 with 1..512 sequences (process-wide; env
 * PA_PREFILL_SPLIT sets the initial value).  A row block (positions p0 .. p0+P-1 of one
 * sequence and KV head, P = 256 / G query positions at head_dim 128, 128 / G at 256)
 * attends to its keys in 64-key tiles, t of them.  -1 (default): a plan kernel reads the
 * context and chunk lengths on the device, cuts every row block of more than C tiles
 * into ceil(t / C) chunks (C = max(16, ceil(5W / 4N)) for W tiles in the call and N
 * compute units: only row blocks longer than 1.25 units' fair share are cut), and lists the items (chunks and whole row blocks, per KV head) largest
 * first; the prefill kernel takes them in that order, and the last chunk of a row block
 * to finish folds its chunks with the log-sum-exp rule (the same statistics as decode's
 * Phase 2, over key ranges instead of partitions).  k in 4 .. 2^20: chunks of at most k
 * tiles, the same otherwise (results then do not depend on the rest of the batch).  0:
 * no plan: one work-group per row block in a (position block, KV head, sequence) grid,
 * sequences most keys first; -1 takes this grid too when no row block can exceed 16
 * tiles (prefix plus chunk bound by the table width and max_query_len: 1024 keys).
 * The plan and the chunks' partial states use the library-owned prefill workspace
 * (grown on demand, kept per device, about 0.2 GB at most at 256 compute units; prefill
 * calls that overlap on one device from different streams race: give them pa_prefill_ex
 * workspaces) or pa_prefill_ex's.  Returns PA_ERR_UNSUPPORTED for another value. */
pa_status_t pa_set_prefill_split(int32_t chunk_tiles);
int32_t pa_get_prefill_split(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PA_DECODE_H */

/*
 * rpa.h -- C ABI of the ragged paged attention library (librpa.so, gfx950 only).
 *
 * What it computes.  Causal grouped-query attention over a ragged batch that
 * mixes decode sequences (a few new tokens) and chunked-prefill sequences (many
 * new tokens).  K and V are read in place from a paged cache through
 * per-sequence block tables, and the new tokens' K/V rows can be scattered into
 * their pages in the same call.  This follows the method of "Ragged Paged
 * Attention: A High-Performance and Flexible LLM Inference Kernel for TPU"
 * (summary card, "Key ideas": ragged paged KV, cache writes fused with
 * attention, separate decode / prefill / mixed kernels) and the interface
 * conventions of ONNX Runtime PR 31727, "[WebGPU] Optimized PagedAttention
 * implementation (2/n)" (packed varlen Q with cumulative lengths, block tables,
 * in-place cache update, token_count == 0 is a no-op).  The block-union variant
 * follows "CompactAttention: Accelerating Chunked Prefill with Block-Union KV
 * Selection" ("Core claim", Figures 3 and 4).
 *
 * Conventions shared by every entry point.
 *   - bf16 means bfloat16 storage; all accumulation is fp32.
 *   - All arrays are row-major and densely packed.  Pointers named d_* or
 *     passed as tensor data are DEVICE pointers; h_* pointers are HOST pointers.
 *   - kv_len of a sequence counts all of its keys INCLUDING the new tokens; the
 *     new tokens are the last q_len positions: token t sits at position
 *     past + t (past = kv_len - q_len) and attends to keys 0 .. past + t
 *     (bottom-right causal alignment, the seqlens_q fix of the ONNX Runtime PR).
 *   - Query head h reads KV head h / (Hq / Hkv).
 *   - Every buffer belongs to the caller.  The library allocates no device
 *     memory: scratch space is the caller's workspace.  Caches are updated in
 *     place.  q, out, k_new and v_new must not alias the caches or each other.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream).  Host arrays are read only during the call.
 *   - No call aborts or throws.  A non-zero status comes with a message from
 *     rpa_last_error() (thread-local).  Device contents are preconditions that
 *     are NOT checked on the host: block-table entries of every block a sequence
 *     uses must lie in [0, num_pages), and slots written for different sequences
 *     must be disjoint.  The kernels never store through an entry outside
 *     [0, num_pages) (the new K/V of such a block are dropped) and never read
 *     outside the caches through one (the keys read for it are unspecified, so
 *     the rows that see them are); entries past a sequence's blocks are not read.
 */
#ifndef RPA_H
#define RPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rpa_status {
  RPA_OK = 0,
  RPA_ERR_INVALID_ARGUMENT = 1,   /* malformed shape, lengths, pointers or scale */
  RPA_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, device, group size */
  RPA_ERR_WORKSPACE_TOO_SMALL = 3,
  RPA_ERR_HIP = 4                 /* a HIP runtime call failed (message names it) */
} rpa_status;

/* Cache layouts.
 *   SEQ_MAJOR  (the ONNX Runtime op's paged layout): k_cache, v_cache
 *              [num_pages][page_size][Hkv][D]; one block table row per sequence
 *              block_tables[B][max_pages_per_seq]; kv_lens[B].
 *   HEAD_MAJOR (the KV-head-major layout of CompactAttention, Figure 4: each
 *              page holds one KV head, so every KV head has its own table):
 *              k_cache, v_cache [num_pages][page_size][D];
 *              block_tables[B][Hkv][max_pages_per_seq]; kv_lens[B][Hkv]. */
enum { RPA_LAYOUT_SEQ_MAJOR = 0, RPA_LAYOUT_HEAD_MAJOR = 1 };

/* Kernel selection.  AUTO picks from the batch composition: every sequence
 * decode-class -> DECODE, every one prefill-class -> PREFILL, both -> MIXED
 * (a sequence is decode-class when q_len * (Hq / Hkv) <= 16).  The forced
 * kinds exist for cross-checks; each kernel is correct for any batch. */
enum { RPA_KERNEL_AUTO = 0, RPA_KERNEL_DECODE = 1, RPA_KERNEL_PREFILL = 2, RPA_KERNEL_MIXED = 3 };

/* Cache element types.  The ONNX Runtime PR defers a quantized KV cache ("Quantized
 * KV cache (T_CACHE)") without fixing a format; the one built here is:
 *   BF16      caches of bf16 values (2 bytes an element).
 *   FP8_E4M3  caches of 1-byte codes in the OCP FP8 E4M3 format (bias 7, no
 *             infinities, largest finite 448, S.1111.111 NaN) with one scale per
 *             cache: a cached K value is code value * k_scale, a V value code
 *             value * v_scale.  A new value x is stored as the code of
 *             float(x) * float(1 / scale) clamped to +-448, rounded to nearest
 *             even; attention over new keys sees those stored codes.  Element
 *             strides are those of the bf16 layouts, in bytes. */
enum { RPA_KV_BF16 = 0, RPA_KV_FP8_E4M3 = 1 };

typedef struct rpa_shape {
  int32_t num_seqs;           /* B >= 0 */
  int32_t total_q;            /* T = cu_q_lens[B] */
  int32_t num_q_heads;        /* Hq, a multiple of Hkv */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t page_size;          /* S: a power of two in [16, 1024] (the PR's block_size rule,
                                 capped at the largest size the kernels are tested on) */
  int32_t num_pages;          /* P: pages in each cache */
  int32_t max_pages_per_seq;  /* row length of the block table */
  int32_t layout;             /* RPA_LAYOUT_* */
  int32_t kernel;             /* RPA_KERNEL_* (AUTO in normal use) */
  const int32_t *h_cu_q_lens; /* host mirror of cu_q_lens, [B + 1] */
  const int32_t *h_kv_lens;   /* host mirror of kv_lens, [B] or [B][Hkv] */
  int32_t kv_dtype;           /* RPA_KV_*: element type of k_cache and v_cache */
  float k_scale, v_scale;     /* FP8_E4M3: the caches' scales (finite, > 0); else ignored */
} rpa_shape;

/*
 * rpa_write_kv -- scatter the new tokens' K/V rows into their pages.
 * Defined by the scatter program of the ONNX Runtime PR (Phase 1b.1 commit
 * note): for token t of sequence b and KV head g, pos = past_b + t,
 * page = table(b, g)[pos / page_size], slot = pos % page_size, and the D values
 * of k_new[cu_q_lens[b] + t][g] (likewise v_new) are copied into that slot.
 *   k_new, v_new  device bf16 [T][Hkv][D]
 *   k_cache, v_cache  device caches of shape->kv_dtype, layout per shape->layout,
 *                 written in place
 *   block_tables, cu_q_lens, kv_lens  device int32 copies of the table and of
 *                 the host mirrors in *shape
 * Bit-exact copy (FP8 caches: the codes defined at RPA_KV_FP8_E4M3); no other
 * cache byte is touched.  T == 0 returns RPA_OK.
 */
rpa_status rpa_write_kv(const rpa_shape *shape, const void *k_new, const void *v_new,
                        void *k_cache, void *v_cache, const int32_t *block_tables,
                        const int32_t *cu_q_lens, const int32_t *kv_lens, void *stream);

/*
 * Rotary embedding of the new tokens, fused with the scatter.  The ONNX Runtime
 * PR rotates Q and K before scattering K/V (its rotary program, Phase 1b.2 commit
 * note: position = past + local token, dims from rotary_dim on copied, V not
 * rotated, interleaved or split pairs) and splits packed QKV first (its
 * packed-QKV commit: per token Hq*D columns of Q, then Hkv*D of K, then Hkv*D of
 * V).  Pair (x1, x2) at position p, pair index i becomes
 *     (fmaf(x1, c, -(x2 * s)), fmaf(x2, c, x1 * s)),  c = cos_cache[p][i], s = sin_cache[p][i],
 * in fp32, each rounded to bf16 (nearest even); interleaved pairs are dims
 * (2i, 2i+1), split pairs (i, i + rotary_dim/2).
 */
typedef struct rpa_rotary {
  const float *cos_cache;     /* device fp32 [max_position][rotary_dim / 2] */
  const float *sin_cache;
  int32_t max_position;       /* rows of the tables: every past + t must be below it */
  int32_t rotary_dim;         /* 0 (no rotation) or a multiple of 16, <= head_dim */
  int32_t interleaved;        /* 1: pairs (2i, 2i+1); 0: pairs (i, i + rotary_dim/2) */
} rpa_rotary;

/*
 * rpa_rotary_write_kv -- rotate the new rows of Q and K and scatter K and V.
 *   q, k, v       device bf16: row t of head h at q + t*q_row_stride + h*D
 *                 (likewise k, v with kv_row_stride).  Packed QKV [T][(Hq+2Hkv)*D]
 *                 is q = qkv, k = qkv + Hq*D, v = qkv + (Hq+Hkv)*D, both strides
 *                 (Hq + 2*Hkv)*D; separate tensors have strides Hq*D and Hkv*D.
 *                 Pointers and strides must be multiples of 8 elements.
 *   rotary        NULL or rotary_dim 0: no rotation (a packed split + scatter)
 *   q_out         device bf16 [T][Hq][D], the rotated Q (must not overlap q)
 *   k_cache, v_cache, block_tables, cu_q_lens, kv_lens  as in rpa_write_kv: the
 *                 rotated K and the V rows go to their page slots (FP8 caches
 *                 store codes as defined at RPA_KV_FP8_E4M3).
 * Position of token t of sequence b: kv_len - q_len_b + t.  For the KV-head-major
 * layout every KV head of a rotated sequence must have the same kv_len (checked on
 * the host mirrors).  Afterwards rpa_attention(q_out, ..., k_new = v_new = NULL)
 * attends over the updated caches.  T == 0 returns RPA_OK.
 */
rpa_status rpa_rotary_write_kv(const rpa_shape *shape, const void *q, const void *k,
                               const void *v, int64_t q_row_stride, int64_t kv_row_stride,
                               const rpa_rotary *rotary, void *q_out, void *k_cache,
                               void *v_cache, const int32_t *block_tables,
                               const int32_t *cu_q_lens, const int32_t *kv_lens, void *stream);

/* Bytes of device workspace rpa_attention needs for this shape (split-K
 * partials).  0 is a valid answer.  Returns (size_t)-1 on an invalid shape. */
size_t rpa_attention_workspace_size(const rpa_shape *shape);

/* The kernel rpa_attention will run for this shape (RPA_KERNEL_DECODE /
 * PREFILL / MIXED), or -1 on an invalid shape.  Host-only, no device call. */
int32_t rpa_select_kernel(const rpa_shape *shape);

/*
 * rpa_attention -- ragged paged causal GQA attention.
 *   q             device bf16 [T][Hq][D]
 *   k_cache, v_cache  device caches of shape->kv_dtype (layout per shape->layout)
 *   block_tables  device int32, see the layouts above; unused entries may be -1
 *   cu_q_lens     device int32 [B + 1], non-decreasing from 0 to T
 *   kv_lens       device int32 [B] (or [B][Hkv] for HEAD_MAJOR)
 *   scale         softmax scale applied to q.k (finite, > 0), e.g. 1/sqrt(D)
 *   k_new, v_new  NULL, or device bf16 [T][Hkv][D]: when given, they are first
 *                 scattered into the caches exactly as rpa_write_kv does, on
 *                 the same stream, and the attention sees them
 *   out           device bf16 [T][Hq][D], fully written
 *   workspace     device scratch of >= rpa_attention_workspace_size(shape) bytes
 *                 (may be NULL when that size is 0); its contents on entry do
 *                 not matter and are clobbered
 * For each row: out = softmax(scale * q K^T over keys 0 .. past + t) V, fp32
 * accumulate, rounded to bf16 (round to nearest even); K and V are the cached
 * values (FP8: code values times the scales).  Sequences with
 * q_len == 0 are skipped; T == 0 returns RPA_OK without a launch.
 * Not capturable: the kernel choice, split sizes and the split-merge tag are fixed on
 * the host per call, so a replayed capture would merge nothing.  A call on a stream
 * that is being captured into a HIP graph returns RPA_ERR_UNSUPPORTED and enqueues
 * nothing; graphs use rpa_graph_attention.
 */
rpa_status rpa_attention(const rpa_shape *shape, const void *q, void *k_cache, void *v_cache,
                         const int32_t *block_tables, const int32_t *cu_q_lens,
                         const int32_t *kv_lens, float scale, const void *k_new,
                         const void *v_new, void *out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * rpa_attention_noalloc -- rpa_attention for callers that cannot allocate device memory
 * at all (code that must not call hipMalloc: under HIP graph capture set-up, in tight
 * serving loops, in harnesses that forbid it), not even a workspace once.
 *   Arguments, results and errors as rpa_attention, without the workspace: the split
 *   partials and arrival counters live in a static device array of
 *   RPA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 *   process ends (its address is looked up once per device, on the first call there).
 *   A batch whose partials need more (rpa_attention_workspace_size(shape) bytes) returns
 *   RPA_ERR_WORKSPACE_TOO_SMALL without a launch.  The call allocates nothing and needs
 *   nothing cleared: counters carry a per-call tag, so what an earlier call left behind
 *   reads as stale.  Every call on one GPU shares that GPU's array, so calls that overlap
 *   in time on one GPU (different streams, threads or processes' contexts) race and give
 *   wrong results; calls ordered on one stream are safe.  Kernels and plan are those of
 *   rpa_attention, so the output is bit-identical to it.  Not capturable (as
 *   rpa_attention).
 */
#define RPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rpa_status rpa_attention_noalloc(const rpa_shape *shape, const void *q, void *k_cache,
                                 void *v_cache, const int32_t *block_tables,
                                 const int32_t *cu_q_lens, const int32_t *kv_lens, float scale,
                                 const void *k_new, const void *v_new, void *out, void *stream);

/*
 * Graph-capturable attention: the same computation as rpa_attention, planned on the
 * device.  rpa_attention reads the batch's lengths on the host to choose the kernel, the
 * KV split sizes and the grid; that ties every call to host data and keeps it out of a
 * captured HIP graph (the ONNX Runtime PR lists graph capture among its deferred items).
 * Here the host sees only bounds, fixed for the life of a graph.  One persistent kernel,
 * with a grid that depends only on the device (two workgroups per compute unit), does it
 * all: every workgroup reads cu_q_lens / kv_lens from device memory and derives the plan
 * (split sizes, work-item counts) by the host planner's rules, runs its first work item and
 * then takes items from a queue in the workspace; the last workgroup to finish resets the
 * queue and advances the split-merge tag kept there.  The launch and its arguments are
 * identical from call to call, so it can be captured once and replayed with new device
 * contents.
 */
typedef struct rpa_graph_shape {
  int32_t max_seqs;           /* B_max >= 1: cu_q_lens has B_max + 1 entries, kv_lens B_max
                                 (x Hkv for HEAD_MAJOR); sequences past the live batch carry
                                 q_len 0 (repeated cu_q_lens) and are skipped */
  int32_t max_tokens;         /* T_max >= 1: rows of q, out, k_new, v_new; cu_q_lens[B_max]
                                 must not exceed it */
  int32_t max_splits;         /* 1 .. 64: most KV splits of one sequence; the workspace holds
                                 max_splits partial outputs per row */
  int32_t num_q_heads;        /* as in rpa_shape */
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;
  int32_t max_pages_per_seq;
  int32_t layout;
  int32_t kv_dtype;           /* as in rpa_shape */
  float k_scale, v_scale;
} rpa_graph_shape;

/* Bytes of workspace rpa_graph_attention needs (plan, queue, split partials and
 * counters), or (size_t)-1 on an invalid shape.  Unlike rpa_attention's workspace it
 * carries state from call to call (the split-merge tag): zero it once (any all-zero fill)
 * before the first call, then keep it for every call with this shape. */
size_t rpa_graph_workspace_size(const rpa_graph_shape *shape);

/*
 * rpa_graph_attention -- rpa_attention with device-side planning (see above).
 *   Arguments as in rpa_attention, with the bounds of *shape in place of the host
 *   mirrors; q, out, k_new, v_new have max_tokens rows (rows past cu_q_lens[B_max] are
 *   neither read nor written).  Always one launch on `stream`, also for an empty batch,
 *   so the call can be captured.  Calls that share a workspace must not overlap (they are
 *   ordered when made on one stream).
 * Device data that break the preconditions (a decreasing cu_q_lens, kv_len < q_len, more
 * blocks than max_pages_per_seq, cu_q_lens[B_max] > max_tokens) make the kernel skip the
 * whole batch (out and the caches are left untouched) and set the 32-bit status word at
 * byte offset 0 of the workspace to a non-zero value (0 after a valid batch).
 */
rpa_status rpa_graph_attention(const rpa_graph_shape *shape, const void *q, void *k_cache,
                               void *v_cache, const int32_t *block_tables,
                               const int32_t *cu_q_lens, const int32_t *kv_lens, float scale,
                               const void *k_new, const void *v_new, void *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * rpa_build_union_tables -- per-KV-head block tables of one sequence's chunk
 * from a per-head 2D block mask (CompactAttention, "Core claim" and Figure 3:
 * union over query blocks, then over the query heads of each GQA group).
 *   mask          device uint8 [Hq][num_q_blocks][num_kv_blocks]; nonzero =
 *                 query block qb of head h selects KV block kb
 *   base_tables   device int32 [Hkv][num_kv_blocks]: physical page of every
 *                 logical block of each KV head (KV-head-major pages)
 *   past, kv_len  the chunk covers positions [past, kv_len)
 *   out_tables    device int32 [Hkv][num_kv_blocks]: selected blocks' pages in
 *                 ascending block order, then -1
 *   out_counts    device int32 [Hkv]: number of selected blocks
 *   out_kv_lens   device int32 [Hkv]: keys of the compacted sequence
 * The chunk's own blocks [past / page_size, (kv_len - 1) / page_size] are always
 * selected and blocks at or beyond ceil(kv_len / page_size) never are, so the
 * chunk's queries are the last (kv_len - past) positions of every compacted
 * sequence and rpa_attention (HEAD_MAJOR, out_tables, out_kv_lens) runs causal
 * attention over the selected pages in place.  Deterministic and bit-exact.
 */
rpa_status rpa_build_union_tables(const uint8_t *mask, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t num_q_blocks, int32_t num_kv_blocks,
                                  const int32_t *base_tables, int32_t past, int32_t kv_len,
                                  int32_t page_size, int32_t *out_tables, int32_t *out_counts,
                                  int32_t *out_kv_lens, void *stream);

/* Human-readable message for the last non-OK status on this thread ("" if none). */
const char *rpa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H */

// Host-visible launch entry points of the gfx950 kernels (used by the C ABI in capi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rpa {

struct AttnArgs;

struct WriteArgs {
  const uint16_t *k_new;  // [T][Hkv][D] bf16
  const uint16_t *v_new;
  uint16_t *k_cache;
  uint16_t *v_cache;
  const int32_t *tables;
  const int32_t *cu_q_lens;
  const int32_t *kv_lens;
  int32_t B, T, Hkv;
  int32_t page_shift;
  int32_t num_pages;         // a table entry outside [0, num_pages) is never stored through
  int64_t page_stride, slot_stride, head_stride;
  int32_t bt_seq_stride, bt_head_stride;
  int32_t kvl_seq_stride, kvl_head_stride;
  int32_t kv8;               // caches of FP8 E4M3 codes (else bf16)
  float k_inv, v_inv;        // FP8: 1 / k_scale, 1 / v_scale
};

struct RotaryArgs {
  const uint16_t *q, *k, *v;        // new rows, bf16; row t of head h at base + t*stride + h*D
  int64_t q_stride, kv_stride;      // elements between consecutive tokens' rows
  uint16_t *q_out;                  // [T][Hq][D] bf16
  uint16_t *k_cache, *v_cache;
  const int32_t *tables, *cu_q_lens, *kv_lens;
  const float *cos_cache, *sin_cache;  // [max_position][rotary_dim / 2] fp32
  int32_t B, T, Hq, Hkv;
  int32_t rotary_dim, interleaved;  // rotary_dim: 0 or a multiple of 16, <= D
  int32_t page_shift;
  int32_t num_pages;                // a table entry outside [0, num_pages) is never stored through
  int64_t page_stride, slot_stride, head_stride;
  int32_t bt_seq_stride, bt_head_stride;
  int32_t kvl_seq_stride, kvl_head_stride;
  int32_t kv8;
  float k_inv, v_inv;
};

hipError_t launch_rotary_write(const RotaryArgs &r, int D, hipStream_t stream);

enum class AttnKernel { kDecode = 1, kPrefill = 2, kMixed = 3 };

hipError_t launch_write_kv(const WriteArgs &a, int D, hipStream_t stream);

// The sequences of one class whose items a launch hands out, built on the host from the
// length mirrors, with the first item of each.  Decode-class sequences are listed by
// decreasing item length (longest first, so the launch ends on its shortest items);
// prefill-class sequences of a prefill launch in sequence order (each one's items already run
// heaviest query tile first).  Passed as a kernel argument; n = 0 maps items in sequence
// order with the in-kernel scan instead (batches with more sequences of the class than fit,
// the prefill items of a mixed launch, and the graph-capturable call).  Each listed sequence
// also carries its start, length and longest kv_len, so an item needs no load before its
// query and table loads.
constexpr int kMaxOrderedSeqs = 160;  // keeps the kernel arguments under 4 KB
struct SeqOrder {
  int32_t n;
  // prefill launch whose listed sequences all have the same q_len and kv_len: items run q-tile
  // rank by rank across the sequences (every sequence's heaviest tiles first), not sequence
  // by sequence, so that the launch ends on the lightest items of every sequence
  int32_t interleave;
  int32_t first[kMaxOrderedSeqs + 1];  // first[n] = number of items
  int32_t seq[kMaxOrderedSeqs];
  int32_t q0[kMaxOrderedSeqs];         // cu_q_lens[seq]
  int32_t q_len[kMaxOrderedSeqs];
  int32_t kv[kMaxOrderedSeqs];         // longest kv_len over the sequence's KV heads
};

// Runs the attention kernel of the given kind on n_blocks workgroups (the prefill items,
// then the decode stream's workgroups); the order lists the decode-class sequences of a
// decode or mixed launch and the prefill-class ones of a prefill launch.
hipError_t launch_attention(const AttnArgs &a, const SeqOrder &order, int D, AttnKernel kind,
                            int n_blocks, hipStream_t stream);

struct GraphPlan;

struct GraphPlanArgs {
  const int32_t *cu_q_lens;  // [B + 1]
  const int32_t *kv_lens;
  GraphPlan *plan;
  int32_t B, T_max, Hkv, G;
  int32_t page_size, max_pages;
  int32_t kvl_seq_stride, kvl_head_stride;
  int32_t pf_tokens, max_splits;
  // the host planner's item targets: decode-only batch; decode and prefill shares of a mixed
  // batch; prefill-only batch
  int32_t decode_only_items, mixed_dec_items, mixed_pf_items, prefill_only_items;
};

// Persistent attention of a graph-capturable call on n_workgroups workgroups: each derives
// the call's plan from the lengths on the device, then the workgroups share out the items.
hipError_t launch_graph_attention(const AttnArgs &a, const GraphPlanArgs &p, int D,
                                  int n_workgroups, hipStream_t stream);

struct UnionArgs {
  const uint8_t *mask;       // [Hq][nQB][nKB]
  const int32_t *base;       // [Hkv][nKB]
  int32_t *out_tables;       // [Hkv][nKB]
  int32_t *out_counts;       // [Hkv]
  int32_t *out_kv_lens;      // [Hkv]
  int32_t Hq, Hkv, nQB, nKB;
  int32_t past, kv_len, page_size;
};

// Largest num_kv_blocks the builder accepts (its compaction pass keeps one flag byte per
// block in LDS).
constexpr int kMaxUnionKvBlocks = 32768;

hipError_t launch_union_tables(const UnionArgs &a, hipStream_t stream);

}  // namespace rpa

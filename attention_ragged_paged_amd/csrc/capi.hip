// C ABI of librpa: validation, batch classification, dispatch and launches.
//
// Conventions follow ONNX Runtime PR 31727 ("[WebGPU] Optimized PagedAttention
// implementation (2/n)"): specific error messages per check, token_count == 0 returns OK
// without a launch, caches updated in place, block sizes are powers of two >= 16, and the
// kernel is chosen by a pure function of the batch shape ("distribution-aware" dispatch of
// the Ragged Paged Attention card, "Key ideas": separate decode, prefill and mixed kernels).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <random>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/rpa.h"
#include "rpa_device.h"
#include "rpa_launch.h"

namespace {

thread_local std::string g_last_error;

rpa_status fail(rpa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rpa_status ok() {
  g_last_error.clear();
  return RPA_OK;
}

// Tag of one rpa_attention call, in bits 24..63 of the split-merge counters.  Tags grow by
// one per call from a random start, so counters left by earlier calls or by anything else
// in the workspace never carry the current tag.
unsigned long long next_call_tag() {
  static std::atomic<unsigned long long> next{[] {
    std::random_device rd;
    return ((unsigned long long)rd() << 20) ^ (unsigned long long)rd();
  }()};
  const unsigned long long id = next.fetch_add(1, std::memory_order_relaxed);
  return (id & ((1ull << 40) - 1)) << 24;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

int cdiv(long long x, long long y) { return (int)((x + y - 1) / y); }

// Decode-class threshold in query rows (q_len * G): one 16-row MFMA tile.
constexpr int kDecodeRowsMax = 16;
// Largest number of KV splits of one sequence (one merge wave holds one split per lane).
constexpr int kMaxSplits = 64;
// Work items the split sizes aim for: a few workgroups per compute unit of the 256-CU chip.
// Fewer, longer items amortise each item's fixed cost (work lookup, first loads, combine,
// split merge); even splits keep the tail short.  Measured on one MI355X:
// - a decode-only batch: llama3_decode 768 items 2-3% faster than 512, 896 or 1024 (bf16 and
//   FP8 caches);
#ifndef RPA_DECODE_ONLY_ITEMS
#define RPA_DECODE_ONLY_ITEMS 768
#endif
constexpr long long kDecodeOnlyItems = RPA_DECODE_ONLY_ITEMS;
// - the decode share of a mixed batch, whose decode items run beside long prefill items:
//   mixed_chunked 1280 items 1.2% faster than 1024 (1536: bf16 faster still, FP8 slower);
#ifndef RPA_MIXED_DEC_ITEMS
#define RPA_MIXED_DEC_ITEMS 1280
#endif
constexpr long long kMixedDecodeItems = RPA_MIXED_DEC_ITEMS;
// - the prefill share of a mixed batch: those items run beside the decode items, which keep
//   the memory system busy; splitting them further only adds partial traffic and merges, and
//   when they outnumber a fraction of the workgroup slots they crowd the decode items out
//   (mixed_chunked: 128 items 375 us, 192 items 404 us; mixed_chunked_fp8: 128 items 240 us,
//   160 or 192 items 278 us);
#ifndef RPA_MIXED_PF_ITEMS
#define RPA_MIXED_PF_ITEMS 128
#endif
constexpr long long kMixedPrefillItems = RPA_MIXED_PF_ITEMS;
// - a prefill-only batch, compute-bound, is split only when it has too few items to fill the
//   chip (one 512-token chunk at context 8192, alone: 128 items 210 us, 256 items 129 us,
//   512 items 102 us, 1024 items 136 us).
#ifndef RPA_PREFILL_ONLY_ITEMS
#define RPA_PREFILL_ONLY_ITEMS 512
#endif
constexpr long long kPrefillOnlyItems = RPA_PREFILL_ONLY_ITEMS;

int kv_len_at(const rpa_shape *s, int b, int g) {
  return s->layout == RPA_LAYOUT_SEQ_MAJOR ? s->h_kv_lens[b]
                                           : s->h_kv_lens[(long long)b * s->num_kv_heads + g];
}

int max_kv_len_host(const rpa_shape *s, int b) {
  int m = kv_len_at(s, b, 0);
  if (s->layout == RPA_LAYOUT_HEAD_MAJOR)
    for (int g = 1; g < s->num_kv_heads; ++g) m = std::max(m, kv_len_at(s, b, g));
  return m;
}

rpa_status validate_kv_dtype(int32_t kv_dtype, float k_scale, float v_scale) {
  if (kv_dtype != RPA_KV_BF16 && kv_dtype != RPA_KV_FP8_E4M3)
    return fail(RPA_ERR_INVALID_ARGUMENT, "kv_dtype %d is not a RPA_KV_* value", kv_dtype);
  if (kv_dtype == RPA_KV_FP8_E4M3 &&
      !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f &&
        std::isfinite(1.f / k_scale) && std::isfinite(1.f / v_scale)))
    return fail(RPA_ERR_INVALID_ARGUMENT,
                "FP8 cache scales k_scale %g and v_scale %g must be finite and > 0 (with finite "
                "reciprocals)", (double)k_scale, (double)v_scale);
  return RPA_OK;
}

// Fields of the kernels' arguments that depend on the cache type.
template <class Args>
void fill_kv_dtype(Args &a, int32_t kv_dtype, float k_scale, float v_scale) {
  const bool kv8 = kv_dtype == RPA_KV_FP8_E4M3;
  a.kv8 = kv8 ? 1 : 0;
  a.k_inv = kv8 ? 1.f / k_scale : 1.f;
  a.v_inv = kv8 ? 1.f / v_scale : 1.f;
}

rpa_status validate(const rpa_shape *s, bool need_lens) {
  if (!s) return fail(RPA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->num_seqs < 0) return fail(RPA_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", s->num_seqs);
  if (s->total_q < 0) return fail(RPA_ERR_INVALID_ARGUMENT, "total_q %d < 0", s->total_q);
  if (s->num_kv_heads <= 0 || s->num_q_heads <= 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "num_q_heads %d and num_kv_heads %d must be > 0",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                s->num_q_heads, s->num_kv_heads);
  if (s->head_dim <= 0 || s->head_dim % 8 != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "head_dim %d must be a positive multiple of 8",
                s->head_dim);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RPA_ERR_UNSUPPORTED, "head_dim %d is not built (64 and 128 are)", s->head_dim);
  if (s->num_q_heads / s->num_kv_heads > rpa::kPrefillRows)
    return fail(RPA_ERR_UNSUPPORTED, "group size %d exceeds %d query heads per KV head",
                s->num_q_heads / s->num_kv_heads, rpa::kPrefillRows);
  if (!is_pow2(s->page_size) || s->page_size < 16 || s->page_size > 1024)
    return fail(RPA_ERR_INVALID_ARGUMENT, "page_size %d must be a power of two in [16, 1024]",
                s->page_size);
  if (s->num_pages <= 0) return fail(RPA_ERR_INVALID_ARGUMENT, "num_pages %d <= 0", s->num_pages);
  if (s->max_pages_per_seq <= 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "max_pages_per_seq %d <= 0", s->max_pages_per_seq);
  if (s->layout != RPA_LAYOUT_SEQ_MAJOR && s->layout != RPA_LAYOUT_HEAD_MAJOR)
    return fail(RPA_ERR_INVALID_ARGUMENT, "layout %d unknown", s->layout);
  if (s->kernel < RPA_KERNEL_AUTO || s->kernel > RPA_KERNEL_MIXED)
    return fail(RPA_ERR_INVALID_ARGUMENT, "kernel %d unknown", s->kernel);
  {
    const rpa_status st = validate_kv_dtype(s->kv_dtype, s->k_scale, s->v_scale);
    if (st != RPA_OK) return st;
  }
  if (!need_lens) return RPA_OK;
  if (!s->h_cu_q_lens || (s->num_seqs > 0 && !s->h_kv_lens))
    return fail(RPA_ERR_INVALID_ARGUMENT, "host mirrors of cu_q_lens / kv_lens are NULL");
  if (s->h_cu_q_lens[0] != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "cu_q_lens[0] = %d, expected 0", s->h_cu_q_lens[0]);
  const int Hkv_rows = s->layout == RPA_LAYOUT_HEAD_MAJOR ? s->num_kv_heads : 1;
  for (int b = 0; b < s->num_seqs; ++b) {
    const int q_len = s->h_cu_q_lens[b + 1] - s->h_cu_q_lens[b];
    if (q_len < 0)
      return fail(RPA_ERR_INVALID_ARGUMENT, "cu_q_lens decreases at sequence %d", b);
    for (int g = 0; g < Hkv_rows; ++g) {
      const int kv = kv_len_at(s, b, g);
      if (kv < q_len)
        return fail(RPA_ERR_INVALID_ARGUMENT,
                    "sequence %d (kv head %d): kv_len %d < q_len %d (kv_len counts the new tokens)",
                    b, g, kv, q_len);
      if (cdiv(kv, s->page_size) > s->max_pages_per_seq)
        return fail(RPA_ERR_INVALID_ARGUMENT,
                    "sequence %d: kv_len %d needs %d pages > max_pages_per_seq %d", b, kv,
                    cdiv(kv, s->page_size), s->max_pages_per_seq);
    }
  }
  if (s->h_cu_q_lens[s->num_seqs] != s->total_q)
    return fail(RPA_ERR_INVALID_ARGUMENT, "cu_q_lens[B] = %d != total_q %d",
                s->h_cu_q_lens[s->num_seqs], s->total_q);
  return RPA_OK;
}

rpa_status check_device() {
  static int arch_ok[64];  // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(RPA_ERR_HIP, "hipGetDevice: %s (no usable GPU?)", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(RPA_ERR_UNSUPPORTED, "device index %d", dev);
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess)
      return fail(RPA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    arch_ok[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (arch_ok[dev] != 1)
    return fail(RPA_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X); no code object for it", dev);
  return RPA_OK;
}

// rpa_attention fixes the split-merge tag and the plan in its kernel arguments on the host.
// A captured call would replay with the same tag, find its counters already at the final
// count and merge nothing, leaving split rows stale: such a call is refused (the device-
// planned rpa_graph_attention exists for graphs).
rpa_status refuse_capture(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // the query's error is reported here, not by the next call
    return fail(RPA_ERR_UNSUPPORTED,
                "rpa_attention: the stream cannot be used while a graph is being captured "
                "(hipStreamIsCapturing: %s); use rpa_graph_attention in graphs",
                hipGetErrorString(e));
  }
  if (cs != hipStreamCaptureStatusNone)
    return fail(RPA_ERR_UNSUPPORTED,
                "rpa_attention cannot be captured in a HIP graph (its plan and split-merge tag "
                "are fixed on the host per call); use rpa_graph_attention, which plans on the "
                "device");
  return RPA_OK;
}

struct Plan {
  int kind = 0;         // RPA_KERNEL_DECODE / PREFILL / MIXED
  int dec_rows_max = 0;
  int split_dec = 1 << 30;
  int split_pf = 1 << 30;
  int pf_tokens = 1;
  int n_dec_items = 0;  // decode work items (one workgroup each)
  int n_pf_items = 0;   // prefill work items (one workgroup each)
  int max_nsplit = 1;   // most KV splits of any sequence
};

bool decode_class(const Plan &p, int q_len, int G) { return (long long)q_len * G <= p.dec_rows_max; }

int splits_of(const Plan &p, int q_len, int G, int maxkv) {
  const int split = decode_class(p, q_len, G) ? p.split_dec : p.split_pf;
  return std::max(1, cdiv(maxkv, split));
}

// A split size in keys (a multiple of 64) that cuts `units` 64-key units into about
// `target` items, never giving one sequence more than kMaxSplits splits.
int choose_split(long long units, int longest_kv, int min_keys, long long target) {
  long long per_item = std::max<long long>(1, (units + target - 1) / target);
  long long split = std::max<long long>(per_item * 64, min_keys);
  const long long floor_for_cap = (long long)cdiv(cdiv(longest_kv, 64), kMaxSplits) * 64;
  split = std::max(split, floor_for_cap);
  return (int)std::min<long long>(split, 1 << 30);
}

Plan make_plan(const rpa_shape *s) {
  Plan p;
  const int G = s->num_q_heads / s->num_kv_heads;
  p.pf_tokens = std::max(1, rpa::kPrefillRows / G);
  bool any_dec = false, any_pf = false;
  for (int b = 0; b < s->num_seqs; ++b) {
    const int q_len = s->h_cu_q_lens[b + 1] - s->h_cu_q_lens[b];
    if (q_len == 0) continue;
    if ((long long)q_len * G <= kDecodeRowsMax)
      any_dec = true;
    else
      any_pf = true;
  }
  int kind = s->kernel;
  if (kind == RPA_KERNEL_AUTO)
    kind = any_dec && any_pf ? RPA_KERNEL_MIXED : (any_pf ? RPA_KERNEL_PREFILL : RPA_KERNEL_DECODE);
  p.kind = kind;
  p.dec_rows_max = kind == RPA_KERNEL_DECODE ? (1 << 30)
                   : kind == RPA_KERNEL_PREFILL ? 0
                                                : kDecodeRowsMax;
  // Work in 64-key units of each class, to size the splits.
  long long dec_units = 0, pf_units = 0;
  int dec_longest = 0, pf_longest = 0;
  for (int b = 0; b < s->num_seqs; ++b) {
    const int q_len = s->h_cu_q_lens[b + 1] - s->h_cu_q_lens[b];
    if (q_len == 0) continue;
    const int kv = max_kv_len_host(s, b);
    if (decode_class(p, q_len, G)) {
      dec_units += (long long)s->num_kv_heads * cdiv((long long)q_len * G, rpa::kDecodeRows) * cdiv(kv, 64);
      dec_longest = std::max(dec_longest, kv);
    } else {
      pf_units += (long long)s->num_kv_heads * cdiv(q_len, p.pf_tokens) * cdiv(kv, 64);
      pf_longest = std::max(pf_longest, kv);
    }
  }
  if (dec_units > 0)
    p.split_dec = choose_split(dec_units, dec_longest, 256,
                               pf_units == 0 ? kDecodeOnlyItems : kMixedDecodeItems);
  if (pf_units > 0) {
    p.split_pf = kind == RPA_KERNEL_PREFILL
                     ? choose_split(pf_units, pf_longest, 1024, kPrefillOnlyItems)
                     : choose_split(pf_units, pf_longest, 512, kMixedPrefillItems);
  }
  for (int b = 0; b < s->num_seqs; ++b) {
    const int q_len = s->h_cu_q_lens[b + 1] - s->h_cu_q_lens[b];
    if (q_len == 0) continue;
    const int ns = splits_of(p, q_len, G, max_kv_len_host(s, b));
    p.max_nsplit = std::max(p.max_nsplit, ns);
    if (decode_class(p, q_len, G))
      p.n_dec_items += s->num_kv_heads * cdiv((long long)q_len * G, rpa::kDecodeRows) * ns;
    else
      p.n_pf_items += s->num_kv_heads * cdiv(q_len, p.pf_tokens) * ns;
  }
  return p;
}

struct WorkspaceLayout {
  size_t part_o = 0, part_ml = 0, counters = 0, pf_counter_base = 0, total = 0;
};

// Split partials [max_nsplit][T][Hq][D] + [..][2] fp32, then arrival counters: decode row
// groups at (q0*G + 16*rt)*Hkv + g, prefill row groups after them at (q0 + t0)*Hkv + g.
WorkspaceLayout workspace_layout(const rpa_shape *s, const Plan &p) {
  WorkspaceLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  const size_t rows = p.max_nsplit > 1 ? (size_t)p.max_nsplit * s->total_q * s->num_q_heads : 0;
  w.part_o = take(rows * s->head_dim * sizeof(float));
  w.part_ml = take(rows * 2 * sizeof(float));
  const int G = s->num_q_heads / s->num_kv_heads;
  const size_t dec_ctr = p.max_nsplit > 1 ? ((size_t)s->total_q * G + rpa::kDecodeRows) * s->num_kv_heads : 0;
  const size_t pf_ctr = p.max_nsplit > 1 ? (size_t)s->total_q * s->num_kv_heads : 0;
  w.pf_counter_base = dec_ctr;
  w.counters = take((dec_ctr + pf_ctr) * sizeof(unsigned long long));
  w.total = off;
  return w;
}

size_t workspace_bytes_for(const rpa_shape *s, const Plan &p) {
  return workspace_layout(s, p).total;
}

void fill_layout(const rpa_shape *s, int64_t &page_stride, int64_t &slot_stride,
                 int64_t &head_stride, int32_t &bt_seq, int32_t &bt_head, int32_t &kvl_seq,
                 int32_t &kvl_head) {
  const int64_t D = s->head_dim, S = s->page_size, Hkv = s->num_kv_heads;
  if (s->layout == RPA_LAYOUT_SEQ_MAJOR) {
    page_stride = S * Hkv * D;
    slot_stride = Hkv * D;
    head_stride = D;
    bt_seq = s->max_pages_per_seq;
    bt_head = 0;
    kvl_seq = 1;
    kvl_head = 0;
  } else {
    page_stride = S * D;
    slot_stride = D;
    head_stride = 0;
    bt_seq = (int32_t)(Hkv * s->max_pages_per_seq);
    bt_head = s->max_pages_per_seq;
    kvl_seq = (int32_t)Hkv;
    kvl_head = 1;
  }
}

rpa_status write_kv_impl(const rpa_shape *s, const void *k_new, const void *v_new, void *k_cache,
                         void *v_cache, const int32_t *tables, const int32_t *cu, const int32_t *kvl,
                         hipStream_t stream) {
  rpa::WriteArgs w{};
  w.k_new = static_cast<const uint16_t *>(k_new);
  w.v_new = static_cast<const uint16_t *>(v_new);
  w.k_cache = static_cast<uint16_t *>(k_cache);
  w.v_cache = static_cast<uint16_t *>(v_cache);
  w.tables = tables;
  w.cu_q_lens = cu;
  w.kv_lens = kvl;
  w.B = s->num_seqs;
  w.T = s->total_q;
  w.Hkv = s->num_kv_heads;
  w.page_shift = ilog2(s->page_size);
  w.num_pages = s->num_pages;
  fill_layout(s, w.page_stride, w.slot_stride, w.head_stride, w.bt_seq_stride, w.bt_head_stride,
              w.kvl_seq_stride, w.kvl_head_stride);
  fill_kv_dtype(w, s->kv_dtype, s->k_scale, s->v_scale);
  hipError_t e = rpa::launch_write_kv(w, s->head_dim, stream);
  if (e != hipSuccess) return fail(RPA_ERR_HIP, "write_kv launch: %s", hipGetErrorString(e));
  return RPA_OK;
}

}  // namespace

extern "C" {

rpa_status rpa_write_kv(const rpa_shape *shape, const void *k_new, const void *v_new,
                        void *k_cache, void *v_cache, const int32_t *block_tables,
                        const int32_t *cu_q_lens, const int32_t *kv_lens, void *stream) {
  rpa_status st = validate(shape, true);
  if (st != RPA_OK) return st;
  if (shape->total_q == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !cu_q_lens || !kv_lens)
    return fail(RPA_ERR_INVALID_ARGUMENT, "rpa_write_kv: a device pointer is NULL");
  st = check_device();
  if (st != RPA_OK) return st;
  st = write_kv_impl(shape, k_new, v_new, k_cache, v_cache, block_tables, cu_q_lens, kv_lens,
                     static_cast<hipStream_t>(stream));
  return st == RPA_OK ? ok() : st;
}

rpa_status rpa_rotary_write_kv(const rpa_shape *shape, const void *q, const void *k,
                               const void *v, int64_t q_row_stride, int64_t kv_row_stride,
                               const rpa_rotary *rotary, void *q_out, void *k_cache,
                               void *v_cache, const int32_t *block_tables,
                               const int32_t *cu_q_lens, const int32_t *kv_lens, void *stream) {
  rpa_status st = validate(shape, true);
  if (st != RPA_OK) return st;
  const int Hq = shape->num_q_heads, Hkv = shape->num_kv_heads, D = shape->head_dim;
  const int rd = rotary ? rotary->rotary_dim : 0;
  if (rd < 0 || rd > D || rd % 16 != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "rotary_dim %d must be 0 or a multiple of 16 <= head_dim %d",
                rd, D);
  if (rd > 0 && (!rotary->cos_cache || !rotary->sin_cache || rotary->max_position < 1))
    return fail(RPA_ERR_INVALID_ARGUMENT, "rotary tables are NULL or max_position %d < 1",
                rotary->max_position);
  if (q_row_stride < (int64_t)Hq * D || kv_row_stride < (int64_t)Hkv * D ||
      q_row_stride % 8 != 0 || kv_row_stride % 8 != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT,
                "row strides %lld (q) and %lld (k, v) must be multiples of 8 covering %d and %d "
                "elements", (long long)q_row_stride, (long long)kv_row_stride, Hq * D, Hkv * D);
  if (shape->total_q == 0) return ok();
  if (!q || !k || !v || !q_out || !k_cache || !v_cache || !block_tables || !cu_q_lens || !kv_lens)
    return fail(RPA_ERR_INVALID_ARGUMENT, "rpa_rotary_write_kv: a device pointer is NULL");
  for (const void *p : {q, k, v, static_cast<const void *>(q_out)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return fail(RPA_ERR_INVALID_ARGUMENT, "q, k, v and q_out must be 16-byte aligned");
  {  // q_out must not overlap q's rows (a split pair reads its partner from q)
    const char *qb = static_cast<const char *>(q), *ob = static_cast<const char *>(q_out);
    const int64_t T = shape->total_q;
    const char *qe = qb + ((T - 1) * q_row_stride + (int64_t)Hq * D) * 2;
    const char *oe = ob + T * (int64_t)Hq * D * 2;
    if (qb < oe && ob < qe) return fail(RPA_ERR_INVALID_ARGUMENT, "q_out overlaps q");
  }
  for (int b = 0; b < shape->num_seqs; ++b) {
    const int q_len = shape->h_cu_q_lens[b + 1] - shape->h_cu_q_lens[b];
    if (q_len == 0) continue;
    const int kv0 = kv_len_at(shape, b, 0);
    if (shape->layout == RPA_LAYOUT_HEAD_MAJOR && rd > 0)
      for (int g = 1; g < Hkv; ++g)
        if (kv_len_at(shape, b, g) != kv0)
          return fail(RPA_ERR_INVALID_ARGUMENT,
                      "sequence %d: KV heads have different kv_lens; a rotated sequence needs one "
                      "position per token", b);
    if (rd > 0 && kv0 > rotary->max_position)
      return fail(RPA_ERR_INVALID_ARGUMENT, "sequence %d reaches position %d >= max_position %d",
                  b, kv0 - 1, rotary->max_position);
  }
  st = check_device();
  if (st != RPA_OK) return st;
  rpa::RotaryArgs r{};
  r.q = static_cast<const uint16_t *>(q);
  r.k = static_cast<const uint16_t *>(k);
  r.v = static_cast<const uint16_t *>(v);
  r.q_stride = q_row_stride;
  r.kv_stride = kv_row_stride;
  r.q_out = static_cast<uint16_t *>(q_out);
  r.k_cache = static_cast<uint16_t *>(k_cache);
  r.v_cache = static_cast<uint16_t *>(v_cache);
  r.tables = block_tables;
  r.cu_q_lens = cu_q_lens;
  r.kv_lens = kv_lens;
  r.cos_cache = rd > 0 ? rotary->cos_cache : nullptr;
  r.sin_cache = rd > 0 ? rotary->sin_cache : nullptr;
  r.B = shape->num_seqs;
  r.T = shape->total_q;
  r.Hq = Hq;
  r.Hkv = Hkv;
  r.rotary_dim = rd;
  r.interleaved = rd > 0 && rotary->interleaved ? 1 : 0;
  r.page_shift = ilog2(shape->page_size);
  r.num_pages = shape->num_pages;
  fill_layout(shape, r.page_stride, r.slot_stride, r.head_stride, r.bt_seq_stride,
              r.bt_head_stride, r.kvl_seq_stride, r.kvl_head_stride);
  fill_kv_dtype(r, shape->kv_dtype, shape->k_scale, shape->v_scale);
  const hipError_t e = rpa::launch_rotary_write(r, D, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RPA_ERR_HIP, "rotary write launch: %s", hipGetErrorString(e));
  return ok();
}

size_t rpa_attention_workspace_size(const rpa_shape *shape) {
  if (validate(shape, true) != RPA_OK) return (size_t)-1;
  if (shape->total_q == 0) return 0;
  return workspace_bytes_for(shape, make_plan(shape));
}

int32_t rpa_select_kernel(const rpa_shape *shape) {
  if (validate(shape, true) != RPA_OK) return -1;
  return make_plan(shape).kind;
}

}  // extern "C"

namespace {

// Checks shared by the attention entry points; on success *p is the call's plan.
rpa_status check_attention_call(const rpa_shape *shape, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_tables,
                                const int32_t *cu_q_lens, const int32_t *kv_lens, float scale,
                                const void *k_new, const void *v_new, const void *out,
                                const char *name, Plan *p) {
  rpa_status st = validate(shape, true);
  if (st != RPA_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(RPA_ERR_INVALID_ARGUMENT, "scale %g must be finite and > 0", (double)scale);
  if (shape->total_q == 0) return RPA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !cu_q_lens || !kv_lens || !out)
    return fail(RPA_ERR_INVALID_ARGUMENT, "%s: a device pointer is NULL", name);
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(RPA_ERR_INVALID_ARGUMENT, "k_new and v_new must both be given or both be NULL");
  *p = make_plan(shape);
  return RPA_OK;
}

// The launch of a checked call with its plan, over a workspace of the plan's size.
rpa_status launch_planned(const rpa_shape *shape, const Plan &p, const void *q, void *k_cache,
                          void *v_cache, const int32_t *block_tables, const int32_t *cu_q_lens,
                          const int32_t *kv_lens, float scale, const void *k_new,
                          const void *v_new, void *out, void *workspace, hipStream_t hs) {
  const size_t need = workspace_bytes_for(shape, p);
  const rpa::AttnKernel kind = static_cast<rpa::AttnKernel>(p.kind);
  const WorkspaceLayout wl = workspace_layout(shape, p);
  char *ws = static_cast<char *>(workspace);
  rpa::AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k_cache = static_cast<const uint16_t *>(k_cache);
  a.v_cache = static_cast<const uint16_t *>(v_cache);
  a.out = static_cast<uint16_t *>(out);
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  a.tables = block_tables;
  a.cu_q_lens = cu_q_lens;
  a.kv_lens = kv_lens;
  a.part_o = need ? reinterpret_cast<float *>(ws + wl.part_o) : nullptr;
  a.part_ml = need ? reinterpret_cast<float *>(ws + wl.part_ml) : nullptr;
  a.counters = need ? reinterpret_cast<unsigned long long *>(ws + wl.counters) : nullptr;
  a.call_tag = next_call_tag();
  a.B = shape->num_seqs;
  a.T = shape->total_q;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.G = shape->num_q_heads / shape->num_kv_heads;
  a.page_shift = ilog2(shape->page_size);
  a.num_pages = shape->num_pages;
  fill_layout(shape, a.page_stride, a.slot_stride, a.head_stride, a.bt_seq_stride,
              a.bt_head_stride, a.kvl_seq_stride, a.kvl_head_stride);
  fill_kv_dtype(a, shape->kv_dtype, shape->k_scale, shape->v_scale);
  // FP8 caches hold code values: K's scale joins the softmax scale, V's the output.
  a.scale_log2 = scale * 1.4426950408889634f * (a.kv8 ? shape->k_scale : 1.f);
  a.out_scale = a.kv8 ? shape->v_scale : 1.f;
  a.dec_rows_max = p.dec_rows_max;
  a.split_dec = p.split_dec;
  a.split_pf = p.split_pf;
  a.pf_tokens = p.pf_tokens;
  a.n_pf_items = p.n_pf_items;
  a.pf_counter_base = (int32_t)wl.pf_counter_base;
  // Decode items longest first (a launch that ends on its shortest items has the shortest tail);
  // a prefill launch's sequences in their own order (the in-kernel scan's numbering), so that
  // its items load no lengths before their query and table loads.
  rpa::SeqOrder order;
  order.n = 0;
  order.interleave = 0;
  if (kind == rpa::AttnKernel::kPrefill) {
    const int G = a.G;
    int n = 0, first = 0;
    for (int b = 0; b < shape->num_seqs; ++b) {
      const int q_len = shape->h_cu_q_lens[b + 1] - shape->h_cu_q_lens[b];
      if (q_len == 0 || decode_class(p, q_len, G)) continue;
      if (n == rpa::kMaxOrderedSeqs) {
        n = 0;  // too many: the in-kernel scan
        break;
      }
      const int maxkv = max_kv_len_host(shape, b);
      order.seq[n] = b;
      order.q0[n] = shape->h_cu_q_lens[b];
      order.q_len[n] = q_len;
      order.kv[n] = maxkv;
      order.first[n] = first;
      first += shape->num_kv_heads * cdiv(q_len, p.pf_tokens) * splits_of(p, q_len, G, maxkv);
      ++n;
    }
    order.first[n] = first;
    order.n = n;
    bool same = n > 1;
    for (int i = 1; i < n && same; ++i)
      same = order.q_len[i] == order.q_len[0] && order.kv[i] == order.kv[0];
    order.interleave = same ? 1 : 0;
  } else if (p.n_dec_items > 0) {
    const int G = a.G;
    int idx[rpa::kMaxOrderedSeqs];
    int len[rpa::kMaxOrderedSeqs];
    int n = 0;
    for (int b = 0; b < shape->num_seqs && n <= rpa::kMaxOrderedSeqs; ++b) {
      const int q_len = shape->h_cu_q_lens[b + 1] - shape->h_cu_q_lens[b];
      if (q_len == 0 || !decode_class(p, q_len, G)) continue;
      if (n == rpa::kMaxOrderedSeqs) {
        n = rpa::kMaxOrderedSeqs + 1;  // too many: keep the in-kernel sequence order
        break;
      }
      const int maxkv = max_kv_len_host(shape, b);
      const int ns = splits_of(p, q_len, G, maxkv);
      idx[n] = b;
      len[n] = cdiv(cdiv(maxkv, ns), 64) * 64;  // keys per item (the kernels' even split)
      ++n;
    }
    if (n <= rpa::kMaxOrderedSeqs) {
      int perm[rpa::kMaxOrderedSeqs];
      for (int i = 0; i < n; ++i) perm[i] = i;
      std::stable_sort(perm, perm + n, [&](int x, int y) { return len[x] > len[y]; });
      int first = 0;
      for (int i = 0; i < n; ++i) {
        const int b = idx[perm[i]];
        const int q_len = shape->h_cu_q_lens[b + 1] - shape->h_cu_q_lens[b];
        order.seq[i] = b;
        order.q0[i] = shape->h_cu_q_lens[b];
        order.q_len[i] = q_len;
        order.kv[i] = max_kv_len_host(shape, b);
        order.first[i] = first;
        first += shape->num_kv_heads * cdiv(q_len * G, rpa::kDecodeRows) *
                 splits_of(p, q_len, G, max_kv_len_host(shape, b));
      }
      order.first[n] = first;
      order.n = n;
    }
  }
  hipError_t e = rpa::launch_attention(a, order, shape->head_dim, kind,
                                       p.n_pf_items + p.n_dec_items, hs);
  if (e != hipSuccess) return fail(RPA_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

// ------------------------------------------------------------ static scratch ----
//
// rpa_attention_noalloc keeps the split partials and arrival counters in this file-scope
// array instead of a caller's workspace.  In host code `scratch` is only a stand-in for the
// symbol: its device address, one per GPU (each GPU holds its own copy of the array), comes
// from hipGetSymbolAddress with that device current and is the only form ever passed on.
// Nothing in it needs clearing: the counters carry each call's tag, so whatever an earlier
// call left reads as zero.
constexpr size_t kScratchBytes = RPA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

rpa_status scratch_of_current_device(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RPA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RPA_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(RPA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RPA_OK;
}

}  // namespace

extern "C" {

rpa_status rpa_attention(const rpa_shape *shape, const void *q, void *k_cache, void *v_cache,
                         const int32_t *block_tables, const int32_t *cu_q_lens,
                         const int32_t *kv_lens, float scale, const void *k_new,
                         const void *v_new, void *out, void *workspace, size_t workspace_bytes,
                         void *stream) {
  Plan p;
  rpa_status st = check_attention_call(shape, q, k_cache, v_cache, block_tables, cu_q_lens,
                                       kv_lens, scale, k_new, v_new, out, "rpa_attention", &p);
  if (st != RPA_OK) return st;
  if (shape->total_q == 0) return ok();
  const size_t need = workspace_bytes_for(shape, p);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(RPA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed",
                workspace_bytes, need);
  st = check_device();
  if (st != RPA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = refuse_capture(hs);
  if (st != RPA_OK) return st;
  return launch_planned(shape, p, q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale,
                        k_new, v_new, out, workspace, hs);
}

rpa_status rpa_attention_noalloc(const rpa_shape *shape, const void *q, void *k_cache,
                                 void *v_cache, const int32_t *block_tables,
                                 const int32_t *cu_q_lens, const int32_t *kv_lens, float scale,
                                 const void *k_new, const void *v_new, void *out, void *stream) {
  Plan p;
  rpa_status st = check_attention_call(shape, q, k_cache, v_cache, block_tables, cu_q_lens,
                                       kv_lens, scale, k_new, v_new, out,
                                       "rpa_attention_noalloc", &p);
  if (st != RPA_OK) return st;
  if (shape->total_q == 0) return ok();
  const size_t need = workspace_bytes_for(shape, p);
  if (need > kScratchBytes)
    return fail(RPA_ERR_WORKSPACE_TOO_SMALL,
                "rpa_attention_noalloc: this batch needs %zu bytes of split partials, more than "
                "the library's static scratch of %zu bytes; call rpa_attention with a workspace",
                need, kScratchBytes);
  st = check_device();
  if (st != RPA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = refuse_capture(hs);
  if (st != RPA_OK) return st;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != RPA_OK) return st;
  return launch_planned(shape, p, q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale,
                        k_new, v_new, out, need > 0 ? ws : nullptr, hs);
}

// ----------------------------------------------------------------- graph-capturable ----

}  // extern "C"

namespace {

rpa_status validate_graph(const rpa_graph_shape *s) {
  if (!s) return fail(RPA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->max_seqs < 1 || s->max_tokens < 1)
    return fail(RPA_ERR_INVALID_ARGUMENT, "max_seqs %d and max_tokens %d must be >= 1",
                s->max_seqs, s->max_tokens);
  if (s->max_splits < 1 || s->max_splits > kMaxSplits)
    return fail(RPA_ERR_INVALID_ARGUMENT, "max_splits %d must be in [1, %d]", s->max_splits,
                kMaxSplits);
  if (s->num_kv_heads < 1 || s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT,
                "num_q_heads %d must be a positive multiple of num_kv_heads %d", s->num_q_heads,
                s->num_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RPA_ERR_UNSUPPORTED, "head_dim %d is not built (64 and 128 are)", s->head_dim);
  if (s->num_q_heads / s->num_kv_heads > rpa::kPrefillRows)
    return fail(RPA_ERR_UNSUPPORTED, "group size %d exceeds %d query heads per KV head",
                s->num_q_heads / s->num_kv_heads, rpa::kPrefillRows);
  if (!is_pow2(s->page_size) || s->page_size < 16 || s->page_size > 1024)
    return fail(RPA_ERR_INVALID_ARGUMENT, "page_size %d must be a power of two in [16, 1024]",
                s->page_size);
  if (s->num_pages < 1 || s->max_pages_per_seq < 1)
    return fail(RPA_ERR_INVALID_ARGUMENT, "num_pages %d and max_pages_per_seq %d must be >= 1",
                s->num_pages, s->max_pages_per_seq);
  if (s->layout != RPA_LAYOUT_SEQ_MAJOR && s->layout != RPA_LAYOUT_HEAD_MAJOR)
    return fail(RPA_ERR_INVALID_ARGUMENT, "layout %d is not a RPA_LAYOUT_* value", s->layout);
  return validate_kv_dtype(s->kv_dtype, s->k_scale, s->v_scale);
}

// Graph workspace: [plan][split partials, (m, l) pairs, counters].
struct GraphLayout {
  size_t plan = 0, part_o = 0, part_ml = 0, counters = 0, pf_counter_base = 0, total = 0;
};

GraphLayout graph_layout(const rpa_graph_shape *s) {
  GraphLayout g;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  g.plan = take(sizeof(rpa::GraphPlan));
  const int G = s->num_q_heads / s->num_kv_heads;
  const size_t rows = s->max_splits > 1 ? (size_t)s->max_splits * s->max_tokens * s->num_q_heads : 0;
  g.part_o = take(rows * s->head_dim * sizeof(float));
  g.part_ml = take(rows * 2 * sizeof(float));
  const size_t dec_ctr = s->max_splits > 1 ? ((size_t)s->max_tokens * G + rpa::kDecodeRows) * s->num_kv_heads : 0;
  const size_t pf_ctr = s->max_splits > 1 ? (size_t)s->max_tokens * s->num_kv_heads : 0;
  g.pf_counter_base = dec_ctr;
  g.counters = take((dec_ctr + pf_ctr) * sizeof(unsigned long long));
  g.total = off;
  return g;
}

int workgroup_slots() {  // two attention workgroups per compute unit
  static int slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (slots[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    slots[dev] = 2 * cus;
  }
  return slots[dev];
}

}  // namespace

extern "C" {

size_t rpa_graph_workspace_size(const rpa_graph_shape *shape) {
  if (validate_graph(shape) != RPA_OK) return (size_t)-1;
  return graph_layout(shape).total;
}

rpa_status rpa_graph_attention(const rpa_graph_shape *shape, const void *q, void *k_cache,
                               void *v_cache, const int32_t *block_tables,
                               const int32_t *cu_q_lens, const int32_t *kv_lens, float scale,
                               const void *k_new, const void *v_new, void *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
  rpa_status st = validate_graph(shape);
  if (st != RPA_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(RPA_ERR_INVALID_ARGUMENT, "scale %g must be finite and > 0", (double)scale);
  if (!q || !k_cache || !v_cache || !block_tables || !cu_q_lens || !kv_lens || !out || !workspace)
    return fail(RPA_ERR_INVALID_ARGUMENT, "rpa_graph_attention: a device pointer is NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(RPA_ERR_INVALID_ARGUMENT, "k_new and v_new must both be given or both be NULL");
  const GraphLayout gl = graph_layout(shape);
  if (workspace_bytes < gl.total)
    return fail(RPA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < %zu needed",
                workspace_bytes, gl.total);
  st = check_device();
  if (st != RPA_OK) return st;
  // The per-call values (split sizes, item counts, tag) come from the device plan.
  rpa_shape s{};
  s.num_seqs = shape->max_seqs;
  s.total_q = shape->max_tokens;
  s.num_q_heads = shape->num_q_heads;
  s.num_kv_heads = shape->num_kv_heads;
  s.head_dim = shape->head_dim;
  s.page_size = shape->page_size;
  s.num_pages = shape->num_pages;
  s.max_pages_per_seq = shape->max_pages_per_seq;
  s.layout = shape->layout;
  char *ws = static_cast<char *>(workspace);
  const bool split = shape->max_splits > 1;
  rpa::AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k_cache = static_cast<const uint16_t *>(k_cache);
  a.v_cache = static_cast<const uint16_t *>(v_cache);
  a.out = static_cast<uint16_t *>(out);
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  a.tables = block_tables;
  a.cu_q_lens = cu_q_lens;
  a.kv_lens = kv_lens;
  a.part_o = split ? reinterpret_cast<float *>(ws + gl.part_o) : nullptr;
  a.part_ml = split ? reinterpret_cast<float *>(ws + gl.part_ml) : nullptr;
  a.counters = split ? reinterpret_cast<unsigned long long *>(ws + gl.counters) : nullptr;
  a.B = shape->max_seqs;
  a.T = shape->max_tokens;  // the partials' row layout
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.G = shape->num_q_heads / shape->num_kv_heads;
  a.page_shift = ilog2(shape->page_size);
  a.num_pages = shape->num_pages;
  fill_layout(&s, a.page_stride, a.slot_stride, a.head_stride, a.bt_seq_stride, a.bt_head_stride,
              a.kvl_seq_stride, a.kvl_head_stride);
  fill_kv_dtype(a, shape->kv_dtype, shape->k_scale, shape->v_scale);
  a.scale_log2 = scale * 1.4426950408889634f * (a.kv8 ? shape->k_scale : 1.f);
  a.out_scale = a.kv8 ? shape->v_scale : 1.f;
  a.dec_rows_max = kDecodeRowsMax;
  a.pf_tokens = std::max(1, rpa::kPrefillRows / a.G);
  a.pf_counter_base = (int32_t)gl.pf_counter_base;
  rpa::GraphPlanArgs pa{};
  pa.cu_q_lens = cu_q_lens;
  pa.kv_lens = kv_lens;
  pa.plan = reinterpret_cast<rpa::GraphPlan *>(ws + gl.plan);
  pa.B = shape->max_seqs;
  pa.T_max = shape->max_tokens;
  pa.Hkv = a.Hkv;
  pa.G = a.G;
  pa.page_size = shape->page_size;
  pa.max_pages = shape->max_pages_per_seq;
  pa.kvl_seq_stride = a.kvl_seq_stride;
  pa.kvl_head_stride = a.kvl_head_stride;
  pa.pf_tokens = a.pf_tokens;
  pa.max_splits = shape->max_splits;
  pa.decode_only_items = (int32_t)kDecodeOnlyItems;
  pa.mixed_dec_items = (int32_t)kMixedDecodeItems;
  pa.mixed_pf_items = (int32_t)kMixedPrefillItems;
  pa.prefill_only_items = (int32_t)kPrefillOnlyItems;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = rpa::launch_graph_attention(a, pa, shape->head_dim, workgroup_slots(), hs);
  if (e != hipSuccess) return fail(RPA_ERR_HIP, "graph attention launch: %s", hipGetErrorString(e));
  return ok();
}

rpa_status rpa_build_union_tables(const uint8_t *mask, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t num_q_blocks, int32_t num_kv_blocks,
                                  const int32_t *base_tables, int32_t past, int32_t kv_len,
                                  int32_t page_size, int32_t *out_tables, int32_t *out_counts,
                                  int32_t *out_kv_lens, void *stream) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(RPA_ERR_INVALID_ARGUMENT,
                "num_q_heads %d must be a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  if (num_q_blocks <= 0 || num_kv_blocks <= 0)
    return fail(RPA_ERR_INVALID_ARGUMENT, "num_q_blocks %d and num_kv_blocks %d must be > 0",
                num_q_blocks, num_kv_blocks);
  if (num_kv_blocks > rpa::kMaxUnionKvBlocks)
    return fail(RPA_ERR_UNSUPPORTED, "num_kv_blocks %d > %d", num_kv_blocks,
                rpa::kMaxUnionKvBlocks);
  if (!is_pow2(page_size) || page_size < 16)
    return fail(RPA_ERR_INVALID_ARGUMENT, "page_size %d must be a power of two >= 16", page_size);
  if (past < 0 || kv_len <= past)
    return fail(RPA_ERR_INVALID_ARGUMENT, "need 0 <= past (%d) < kv_len (%d)", past, kv_len);
  if (cdiv(kv_len, page_size) > num_kv_blocks)
    return fail(RPA_ERR_INVALID_ARGUMENT, "kv_len %d needs %d blocks > num_kv_blocks %d", kv_len,
                cdiv(kv_len, page_size), num_kv_blocks);
  if (!mask || !base_tables || !out_tables || !out_counts || !out_kv_lens)
    return fail(RPA_ERR_INVALID_ARGUMENT, "rpa_build_union_tables: a device pointer is NULL");
  rpa_status st = check_device();
  if (st != RPA_OK) return st;
  rpa::UnionArgs u{};
  u.mask = mask;
  u.base = base_tables;
  u.out_tables = out_tables;
  u.out_counts = out_counts;
  u.out_kv_lens = out_kv_lens;
  u.Hq = num_q_heads;
  u.Hkv = num_kv_heads;
  u.nQB = num_q_blocks;
  u.nKB = num_kv_blocks;
  u.past = past;
  u.kv_len = kv_len;
  u.page_size = page_size;
  hipError_t e = rpa::launch_union_tables(u, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RPA_ERR_HIP, "union tables launch: %s", hipGetErrorString(e));
  return ok();
}

const char *rpa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

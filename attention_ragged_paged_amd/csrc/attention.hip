// Ragged paged causal GQA attention for gfx950: decode, prefill and mixed kernels.
//
// Method: "Ragged Paged Attention: A High-Performance and Flexible LLM Inference Kernel for
// TPU" (summary card, "Key ideas"): attention over ragged batches whose K/V live in a paged
// cache, cache writes fused with the attention, and separate kernels for decode, prefill and
// mixed batches.  The decode / prefill split and split-K decode follow ONNX Runtime PR 31727
// ("[WebGPU] Optimized PagedAttention implementation (2/n)", "What's shipped": a split-reduce
// decode pair and a fused paged prefill with page-table-aware tile loads); causal alignment
// is that page's seqlens_q fix: token t of a sequence sits at position past + t and sees
// keys 0 .. past + t.
//
// One launch per call.  The kernels map blocks onto work items themselves, through an order
// of sequences the host builds from its length mirrors and passes in the kernel arguments
// (decode items longest first; a prefill launch's items in sequence order), or with an
// in-kernel scan over the sequences (find_item) when no order is passed, as for the prefill
// items of a mixed launch; nothing is uploaded.  A row is one
// (token, query head) pair; the G query heads of a GQA group are packed into the same item
// so every K/V byte is read once per group.
//
// Fused cache write.  When the call carries the new tokens' K/V, every reader takes keys at
// positions >= past straight from k_new / v_new, and exactly one item per (sequence, KV head)
// - the one owning the sequence's last query rows, which visits every new key - stores them
// into their page slots.  No reader ever loads a slot that this call writes.
//
// Split merges without a second launch.  Items that cover only part of a key range write
// fp32 partials (running max in log2 units, sum, unnormalised output) and then arrive on a
// per-item counter; the last to arrive merges with the log-sum-exp rule and writes bf16.
// Counters carry the call's tag in their high bits, so stale values from earlier calls
// (or uninitialised workspace) read as zero and the workspace never needs clearing.
//
// MFMA layouts (wave64).  Scores are computed transposed, S^T = K Q^T, so that a lane owns
// one query row: its softmax statistics need at most two cross-lane steps, and the S^T
// accumulator is already the B operand of the P V product computed as O^T = V^T P^T.  V^T
// comes out of LDS with the transposing read ds_read_b64_tr_b16.
#include "rpa_device.h"
#include "rpa_launch.h"

namespace rpa {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr unsigned long long kCountMask = (1ull << 24) - 1;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int64_t kv_row_offset(const AttnArgs &a, int page, int slot, int g) {
  return (int64_t)page * a.page_stride + (int64_t)slot * a.slot_stride + (int64_t)g * a.head_stride;
}

__device__ __forceinline__ int table_at(const AttnArgs &a, int b, int g, int logical) {
  return a.tables[b * a.bt_seq_stride + g * a.bt_head_stride + logical];
}

// Split partials travel between workgroups (possibly on different XCDs, each with its own
// L2) through device-coherent accesses, which are written through and read past the
// non-coherent L2 (cache policy sc1).  The writer waits for its stores to complete before it
// arrives on the counter, and the reader loads only after its arrival returned last, so no
// cache-wide writeback or invalidate is ever needed (a device-scope fence would flush the
// whole L2 of the XCD).  Output rows move 16 bytes a lane through a buffer resource over the
// item's first partial row (a wave-uniform base; lane offsets stay far below 2 GiB), so that
// a row's partial goes out in whole 16-byte pieces; the (max, sum) pairs use device-scope
// relaxed atomic stores and loads, which carry the same policy.
constexpr int kCoherent = 16;  // buffer cache-policy operand: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rows(const float *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

__device__ __forceinline__ void st_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                              const f32x4 &v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte_off, 0,
                                         kCoherent);
}

__device__ __forceinline__ f32x4 ld_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0,
                                                                         kCoherent));
}

__device__ __forceinline__ void st_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Partial output row (split s, token, head) lives at part_o + ((s T + token) Hq + head) D.
// An item's rows: tokens tok0 .., heads h0 .. of the same split; its base and a row's offset:
__device__ __forceinline__ const float *partial_base(const AttnArgs &a, int s, int tok0, int h0,
                                                     int D) {
  return a.part_o + (((int64_t)s * a.T + tok0) * a.Hq + h0) * D;
}
__device__ __forceinline__ uint32_t partial_off(const AttnArgs &a, int dtok, int dh, int d, int D) {
  return (uint32_t)(((dtok * a.Hq + dh) * D + d) * 4);
}

// Waits until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Arrive on a tagged counter; returns how many have arrived in this call (this one included).
// A value carrying another call's tag counts as zero.  Lock-free: a failed exchange means
// another arrival succeeded.
__device__ __forceinline__ unsigned arrive(unsigned long long *p, unsigned long long tag) {
  unsigned long long old = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (true) {
    const unsigned long long next = ((old & ~kCountMask) == tag) ? old + 1 : (tag | 1ull);
    if (__hip_atomic_compare_exchange_strong(p, &old, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return (unsigned)(next & kCountMask);
  }
}

// Merge the nsplit partials of one output row and write bf16: the thread's dims are the
// 16-byte chunks c + 16 q, q < D/64, so that the 16 threads of a row touch whole rows;
// out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), online over batches of 4 splits whose
// loads are all issued before any is used.
template <int D>
__device__ __forceinline__ void merge_row(const AttnArgs &a, int nsplit, int token, int h, int c,
                                          int tok0, int h0) {
  constexpr int NQ = D / 64;  // chunks per thread
  const uint32_t off = partial_off(a, token - tok0, h - h0, 4 * c, D);
  float M = kNegInf, L = 0.f;
  f32x4 o[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) o[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 4) {
    float mv[4], lv[4];
    f32x4 ov[4][NQ];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t pr = ((int64_t)min(s0 + u, nsplit - 1) * a.T + token) * a.Hq + h;
      mv[u] = ld_coherent(a.part_ml + pr * 2);
      lv[u] = ld_coherent(a.part_ml + pr * 2 + 1);
      const __amdgpu_buffer_rsrc_t rows =
          coherent_rows(partial_base(a, min(s0 + u, nsplit - 1), tok0, h0, D));
#pragma unroll
      for (int q = 0; q < NQ; ++q) ov[u][q] = ld_coherent16(rows, off + 256 * q);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < nsplit) Mn = fmaxf(Mn, mv[u]);
    const float Mu = Mn == kNegInf ? 0.f : Mn;
    const float sc = fast_exp2(M - Mu);
    L *= sc;
#pragma unroll
    for (int q = 0; q < NQ; ++q) o[q] = o[q] * sc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + u >= nsplit) continue;
      const float wv = fast_exp2(mv[u] - Mu);
      L += lv[u] * wv;
#pragma unroll
      for (int q = 0; q < NQ; ++q) o[q] += ov[u][q] * wv;
    }
    M = Mn;
  }
  const float inv = a.out_scale / L;
  uint16_t *op = a.out + ((int64_t)token * a.Hq + h) * D + 4 * c;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    *reinterpret_cast<u32x2 *>(op + 64 * q) =
        u32x2{pack_bf16x2(o[q][0] * inv, o[q][1] * inv), pack_bf16x2(o[q][2] * inv, o[q][3] * inv)};
}

// ============================================================================ decode ======
//
// A decode item is (sequence, KV head, 16-row tile, KV split): up to 16 query rows of one KV
// head (q_len * G rows taken 16 at a time) against one split of the keys.  Items are
// workgroups, so the hardware dispatcher balances them dynamically as workgroups finish
// (per-wave memory latency varies by 2x across the chip; a static split of the key stream
// leaves the slowest waves as the tail).  The 4 waves take 16-key chunks round-robin, each
// with its own online-softmax state, merged through LDS at the end.  Chunks are loaded as
// whole contiguous rows (lane l takes 16 bytes of row l/LPR: four 256-byte rows per load
// instruction, which streams ~25% faster than loading the MFMA operand layout directly)
// and staged in the wave's LDS buffers, rows XOR-swizzled in 16-byte units:
//   QK^T: v_mfma_f32_16x16x32_bf16, A = K rows (ds_read_b128), B = Q^T (in registers).
//         Lane l gets S^T[key 4(l/16) + i][row l%16], i = 0..3.
//   PV:   v_mfma_f32_16x16x16_bf16, A = V^T (transposing LDS read), B = P^T (the lane's
//         own 4 probabilities) -> O^T[dim][row].
// Each wave keeps the next chunk's loads in flight while it computes the current one
// (register double buffer); block-table entries for 64 chunks sit in one register.
template <int D>
struct DecodeSmem {
  union {
    struct {
      uint16_t k[4][16 * D];  // per-wave staged K chunk
      uint16_t v[4][16 * D];  // per-wave staged V chunk
    } stage;
    float o[4][16][D + 4];  // per-wave unnormalised outputs for the final combine
  };
  float m[4][16];
  float l[4][16];
  int last;  // split merge: this workgroup arrived last
};

__device__ __forceinline__ int dec_item_kend(int kv, int q_len, int G, int rt) {
  const int last_row = min(rt * kDecodeRows + kDecodeRows - 1, q_len * G - 1);
  return min(kv, kv - q_len + last_row / G + 1);
}

__device__ __forceinline__ int decode_count(const AttnArgs &a, int b) {
  const int q_len = a.cu_q_lens[b + 1] - a.cu_q_lens[b];
  if (q_len == 0 || !is_decode_class(a, q_len)) return 0;
  return a.Hkv * ceil_div(q_len * a.G, kDecodeRows) * num_splits_dec(a, b);
}

// Graph-capturable calls order decode items without a host: sequences fall into length
// classes of their items (longest first), items follow class by class, and within a class
// the sequence order.  dec_first[k] is the first decode item of class k.
constexpr int kDecClasses = 8;  // (4 measured 1% slower on the graph-captured decode)
struct DecodeClasses {
  int dec_first[kDecClasses + 1];
  int split;  // the call's decode split size
};

__device__ __forceinline__ int dec_class(int max_kv, int split) {
  const int ns = max(1, ceil_div(max_kv, split));
  const long long len = even_split(max_kv, ns);  // keys per item
  const long long sp = split;
  // class k holds items of (K-1-k)/K .. (K-k)/K of the split, K = kDecClasses (0: longest)
  const int q = (int)((len * kDecClasses - 1) / sp);
  return kDecClasses - 1 - min(q, kDecClasses - 1);
}

// Item id -> (rank in a host-built order, index within the sequence); rank -1 past the last
// item.
__device__ __forceinline__ ItemRef ordered_item(const SeqOrder &o, int id) {
  if (id >= o.first[o.n]) return {-1, 0};
  int lo = 0, hi = o.n;  // largest r < n with first[r] <= id
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (o.first[mid] <= id)
      lo = mid;
    else
      hi = mid;
  }
  return {lo, id - o.first[lo]};
}

template <int D, bool KV8>
__device__ void decode_item(const AttnArgs &a, int id, char *smem_raw, const SeqOrder *order,
                            const DecodeClasses *classes = nullptr) {
  constexpr int KK = D / 32;     // 16x16x32 MFMAs per chunk for QK^T; load instructions per chunk
  constexpr int MB = D / 16;     // 16x16x16 MFMAs per chunk for PV (16-dim output blocks)
  constexpr int LPR = D / 8;     // lanes per 16-key row when loading
  constexpr int RPI = 64 / LPR;  // rows per load instruction
  // FP8 cache: a lane loads 16 codes (16 bytes) of a row; new keys come as 32 bytes of bf16.
  constexpr int LPR8 = D / 16;     // lanes per row
  constexpr int RPI8 = 64 / LPR8;  // rows per load instruction
  constexpr int NI8 = 16 / RPI8;   // load instructions per 16-key chunk
  DecodeSmem<D> &sm = *reinterpret_cast<DecodeSmem<D> *>(smem_raw);
  const int tid = item_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int lrow = KV8 ? lane / LPR8 : lane / LPR;
  const int lchk = KV8 ? lane % LPR8 : lane % LPR;

  int b, q0, q_len, max_kv;
  ItemRef it;
  if (order != nullptr && order->n > 0) {  // everything from the kernel arguments
    it = ordered_item(*order, id);
    if (it.b < 0) return;
    b = order->seq[it.b];
    q0 = order->q0[it.b];
    q_len = order->q_len[it.b];
    max_kv = order->kv[it.b];
  } else if (classes != nullptr) {  // class by class, then sequence order
    if (id >= classes->dec_first[kDecClasses]) return;
    int k = 0, base = 0;  // (no indexing by k: that would put the classes in scratch memory)
#pragma unroll
    for (int kk = 1; kk < kDecClasses; ++kk)
      if (classes->dec_first[kk] <= id) {
        k = kk;
        base = classes->dec_first[kk];
      }
    it = find_item(id - base, a.B, [&](int bb) {
      const int n = decode_count(a, bb);
      return n > 0 && dec_class(max_kv_len(a, bb), classes->split) == k ? n : 0;
    });
    b = __builtin_amdgcn_readfirstlane(it.b);
    if (b < 0) return;
    q0 = a.cu_q_lens[b];
    q_len = a.cu_q_lens[b + 1] - q0;
    max_kv = max_kv_len(a, b);
  } else {
    it = find_item(id, a.B, [&](int bb) { return decode_count(a, bb); });
    b = __builtin_amdgcn_readfirstlane(it.b);
    if (b < 0) return;
    q0 = a.cu_q_lens[b];
    q_len = a.cu_q_lens[b + 1] - q0;
    max_kv = max_kv_len(a, b);
  }
  const int n_rt = ceil_div(q_len * a.G, kDecodeRows);
  const int nsplit = max(1, ceil_div(max_kv, a.split_dec));
  int rem = __builtin_amdgcn_readfirstlane(it.rem);
  const int s = rem % nsplit;
  rem /= nsplit;
  const int rt = rem % n_rt;
  const int g = rem / n_rt;
  const int kv_len = a.kvl_head_stride == 0 ? max_kv : kv_len_of(a, b, g);  // per head if head-major
  const int past = kv_len - q_len;
  const int n_rows = q_len * a.G;
  const int split = even_split(max_kv, nsplit);
  const int k_begin = s * split;
  const int k_end = min(min(kv_len, k_begin + split), dec_item_kend(kv_len, q_len, a.G, rt));
  const bool fused = a.k_new != nullptr;
  const bool writer = fused && rt == n_rt - 1;  // the last row tile visits every new key

  // This lane's query row (B operand column l%16).
  const int fr = rt * kDecodeRows + r16;
  const bool row_ok = fr < n_rows;
  const int t_row = row_ok ? fr / a.G : 0;
  const int h_row = g * a.G + (row_ok ? fr % a.G : 0);
  const int row_lim = past + t_row + 1;  // keys < row_lim are visible to this row
  bf16x8 qf[KK];
  {
    const uint16_t *qp = a.q + ((int64_t)(q0 + t_row) * a.Hq + h_row) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4 *>(qp + 32 * kk + 8 * j);
      qf[kk] = as_bf16x8(v);
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_all = k_end > k_begin ? ceil_div(k_end - k_begin, 16) : 0;
  const int n_w = n_all > w ? (n_all - w + 3) / 4 : 0;  // chunks w, w+4, ... of this wave
  uint16_t *kbuf = sm.stage.k[w];
  uint16_t *vbuf = sm.stage.v[w];
  const int page_mask = (1 << a.page_shift) - 1;
  int pg_lane = 0;  // page of this wave's chunk base + lane

  // Chunk i of this wave holds keys key0 .. key0+15 (one page: pages hold >= 16 keys); load
  // instruction t brings rows lrow + RPI*t.  Rows of new keys come from k_new / v_new.
  const uint8_t *const k8 = reinterpret_cast<const uint8_t *>(a.k_cache);
  const uint8_t *const v8 = reinterpret_cast<const uint8_t *>(a.v_cache);
  // FP8: element offset of this lane's 16 values of new key `key` in k_new / v_new (keys past
  // the sequence's end, in a chunk's tail, read its last new row instead)
  auto new_off = [&](int key) {
    return ((int64_t)(q0 + min(key, kv_len - 1) - past) * a.Hkv + g) * D + 16 * lchk;
  };
  // A chunk's cache rows: a wave-uniform base (the chunk's first row, scalar arithmetic) plus
  // a per-lane constant for load instruction t (row lrow + RPI t, the lane's 16 bytes).
  constexpr int NL = KV8 ? NI8 : KK;
  int lane_off[NL];
#pragma unroll
  for (int t = 0; t < NL; ++t)
    lane_off[t] = (lrow + (KV8 ? RPI8 : RPI) * t) * (int)a.slot_stride + (KV8 ? 16 : 8) * lchk;
  // Only a chunk whose last key reaches `past` holds new keys (wave-uniform): every other
  // chunk takes a plain path, with no per-lane choice between cache and new rows.
  auto has_new = [&](int key0) { return fused && key0 + 15 >= past; };
  auto load_chunk = [&](int base, int i, u32x4 *kr, u32x4 *vr) {
    const int key0 = k_begin + 16 * (w + 4 * (base + i));
    const int page = read_page(__builtin_amdgcn_readlane(pg_lane, i));
    if (!has_new(key0)) {
      constexpr int EB = KV8 ? 1 : 2;  // bytes per cache element
      const int64_t cb = kv_row_offset(a, page, key0 & page_mask, g) * EB;  // chunk base, bytes
      const uint8_t *const kb8 = reinterpret_cast<const uint8_t *>(a.k_cache) + cb;
      const uint8_t *const vb8 = reinterpret_cast<const uint8_t *>(a.v_cache) + cb;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        kr[t] = *reinterpret_cast<const u32x4 *>(kb8 + EB * lane_off[t]);
        vr[t] = *reinterpret_cast<const u32x4 *>(vb8 + EB * lane_off[t]);
      }
      return;
    }
    if constexpr (KV8) {
      // register t: the row's 16 codes, or for a new key the first 8 of its bf16 values (the
      // other 8 are loaded when the chunk is staged); every lane loads, so the waits before
      // each chunk's use stay exact
#pragma unroll
      for (int t = 0; t < NI8; ++t) {
        const int r = lrow + RPI8 * t;
        const int key = key0 + r;
        const uint8_t *kp = k8 + kv_row_offset(a, page, (key0 & page_mask) + r, g) + 16 * lchk;
        const uint8_t *vp = v8 + (kp - k8);
        if (fused && key >= past) {
          kp = reinterpret_cast<const uint8_t *>(a.k_new + new_off(key));
          vp = reinterpret_cast<const uint8_t *>(a.v_new + new_off(key));
        }
        kr[t] = *reinterpret_cast<const u32x4 *>(kp);
        vr[t] = *reinterpret_cast<const u32x4 *>(vp);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < KK; ++t) {
      const int r = lrow + RPI * t;
      const int key = key0 + r;
      const int64_t coff = kv_row_offset(a, page, (key0 & page_mask) + r, g) + 8 * lchk;
      const uint16_t *kp = a.k_cache + coff;
      const uint16_t *vp = a.v_cache + coff;
      if (fused && key >= past) {
        // keys past the sequence's end (the chunk's tail) read its last new row instead
        const int64_t noff = ((int64_t)(q0 + min(key, kv_len - 1) - past) * a.Hkv + g) * D + 8 * lchk;
        kp = a.k_new + noff;
        vp = a.v_new + noff;
      }
      kr[t] = *reinterpret_cast<const u32x4 *>(kp);
      vr[t] = *reinterpret_cast<const u32x4 *>(vp);
    }
  };
  auto process_chunk = [&](int base, int i, const u32x4 *kr, const u32x4 *vr) {
    const int key0 = k_begin + 16 * (w + 4 * (base + i));
    const int page = __builtin_amdgcn_readlane(pg_lane, i);  // negative: a bad entry, no store
    // Stage in LDS (V rows of keys past the item's range are zeroed: they may hold anything);
    // the writer item also stores the new keys into their page slots.
    const bool fresh = has_new(key0);
    if constexpr (KV8) {
      // New keys are quantized here exactly as the cache stores them, so every reader sees
      // the stored codes; LDS holds the codes' bf16 values in the bf16 layout.
      if (!fresh) {
#pragma unroll
        for (int t = 0; t < NI8; ++t) {
          const int r = lrow + RPI8 * t;
          u32x4 vc = vr[t];
          if (key0 + r >= k_end) vc = u32x4{0u, 0u, 0u, 0u};
          u32x4 lo, hi;
          dequant16(kr[t], lo, hi);
          *reinterpret_cast<u32x4 *>(kbuf + lds_off<D>(r, 2 * lchk)) = lo;
          *reinterpret_cast<u32x4 *>(kbuf + lds_off<D>(r, 2 * lchk + 1)) = hi;
          dequant16(vc, lo, hi);
          *reinterpret_cast<u32x4 *>(vbuf + lds_off<D>(r, 2 * lchk)) = lo;
          *reinterpret_cast<u32x4 *>(vbuf + lds_off<D>(r, 2 * lchk + 1)) = hi;
        }
      } else {
#pragma unroll
      for (int t = 0; t < NI8; ++t) {
        const int r = lrow + RPI8 * t;
        const int key = key0 + r;
        u32x4 kc = kr[t], vc = vr[t];
        if (fused && key >= past) {
          const u32x4 khi = *reinterpret_cast<const u32x4 *>(a.k_new + new_off(key) + 8);
          const u32x4 vhi = *reinterpret_cast<const u32x4 *>(a.v_new + new_off(key) + 8);
          kc = quantize16(kr[t], khi, a.k_inv);
          vc = quantize16(vr[t], vhi, a.v_inv);
          if (writer && key < k_end && page >= 0) {
            const int64_t coff = kv_row_offset(a, page, (key0 & page_mask) + r, g) + 16 * lchk;
            *reinterpret_cast<u32x4 *>(const_cast<uint8_t *>(k8) + coff) = kc;
            *reinterpret_cast<u32x4 *>(const_cast<uint8_t *>(v8) + coff) = vc;
          }
        }
        if (key >= k_end) vc = u32x4{0u, 0u, 0u, 0u};
        u32x4 lo, hi;
        dequant16(kc, lo, hi);
        *reinterpret_cast<u32x4 *>(kbuf + lds_off<D>(r, 2 * lchk)) = lo;
        *reinterpret_cast<u32x4 *>(kbuf + lds_off<D>(r, 2 * lchk + 1)) = hi;
        dequant16(vc, lo, hi);
        *reinterpret_cast<u32x4 *>(vbuf + lds_off<D>(r, 2 * lchk)) = lo;
        *reinterpret_cast<u32x4 *>(vbuf + lds_off<D>(r, 2 * lchk + 1)) = hi;
      }
      }
    } else {
#pragma unroll
    for (int t = 0; t < KK; ++t) {
      const int r = lrow + RPI * t;
      const int key = key0 + r;
      *reinterpret_cast<u32x4 *>(kbuf + lds_off<D>(r, lchk)) = kr[t];
      *reinterpret_cast<u32x4 *>(vbuf + lds_off<D>(r, lchk)) = key < k_end ? vr[t] : u32x4{0u, 0u, 0u, 0u};
    }
    if (fresh && writer) {
#pragma unroll
      for (int t = 0; t < KK; ++t) {
        const int r = lrow + RPI * t;
        const int key = key0 + r;
        if (key >= past && key < k_end && page >= 0) {
          const int64_t coff = kv_row_offset(a, page, (key0 & page_mask) + r, g) + 8 * lchk;
          *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(a.k_cache) + coff) = kr[t];
          *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(a.v_cache) + coff) = vr[t];
        }
      }
    }
    }
    // S^T = K Q^T: lane (r16, j) takes K row r16, dims 32kk + 8j .. +8 as its A operand.
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 kf = *reinterpret_cast<const u32x4 *>(kbuf + lds_off<D>(r16, 4 * kk + j));
      st = mfma16x16x32(as_bf16x8(kf), qf[kk], st);
    }
    float sv[4];
    float mloc = kNegInf;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int key = key0 + 4 * j + i4;
      const bool ok = key < k_end && key < row_lim;
      sv[i4] = ok ? st[i4] * a.scale_log2 : kNegInf;
      mloc = fmaxf(mloc, sv[i4]);
    }
    mloc = pair_max32(pair_max16(mloc));  // the row's 4 lanes: l, l ^ 16, l ^ 32, l ^ 48
    // Lazy rescale: the running max moves only when a row's max grows by more than 8 (log2
    // units), so probabilities stay below 2^8 and most chunks skip rescaling the accumulators.
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = acc[mb] * alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      p[i4] = fast_exp2(sv[i4] - m_use);
      psum += p[i4];
    }
    l_run += psum;
    const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
    // Transposing read: lane (i = l%16, j) names row 4j + i/4, dims 16mb + 4(i%4) .. +3.
    const int tr_row = 4 * j + (r16 >> 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int c = 2 * mb + ((r16 & 3) >> 1);
      const s16x4 va = lds_read_tr(vbuf + lds_off<D>(tr_row, c) + 4 * (r16 & 1));
      acc[mb] = mfma16x16x16(va, pb, acc[mb]);
    }
  };

  for (int base = 0; base < n_w; base += 64) {
    const int n = min(64, n_w - base);
    pg_lane = lane < n ? checked_page(table_at(a, b, g, (k_begin + 16 * (w + 4 * (base + lane))) >> a.page_shift),
                                      a.num_pages)
                       : 0;
    if constexpr (KV8) {
      // An FP8 chunk is half the bytes of a bf16 one: four chunks stay in flight (a register
      // ring) so that a wave keeps as many bytes in flight as the bf16 loop does.
      u32x4 k0[NI8], v0[NI8], k1[NI8], v1[NI8], k2[NI8], v2[NI8], k3[NI8], v3[NI8];
      load_chunk(base, 0, k0, v0);
      load_chunk(base, min(1, n - 1), k1, v1);
      load_chunk(base, min(2, n - 1), k2, v2);
      int i = 0;
      for (; i + 4 <= n; i += 4) {
        load_chunk(base, min(i + 3, n - 1), k3, v3);
        __builtin_amdgcn_sched_barrier(0);
        process_chunk(base, i, k0, v0);
        load_chunk(base, min(i + 4, n - 1), k0, v0);
        __builtin_amdgcn_sched_barrier(0);
        process_chunk(base, i + 1, k1, v1);
        load_chunk(base, min(i + 5, n - 1), k1, v1);
        __builtin_amdgcn_sched_barrier(0);
        process_chunk(base, i + 2, k2, v2);
        load_chunk(base, min(i + 6, n - 1), k2, v2);
        __builtin_amdgcn_sched_barrier(0);
        process_chunk(base, i + 3, k3, v3);
      }
      if (i < n) process_chunk(base, i, k0, v0);
      if (i + 1 < n) process_chunk(base, i + 1, k1, v1);
      if (i + 2 < n) process_chunk(base, i + 2, k2, v2);
      continue;
    }
    u32x4 kA[KK], vA[KK], kB[KK], vB[KK];
    load_chunk(base, 0, kA, vA);
    // Two chunks per trip, register double buffer.  Every load is unconditional (the last
    // one may repeat the final chunk, an L2 hit) so that the wait before each chunk's use
    // covers exactly that chunk's loads while the other chunk's loads stay in flight.  (A
    // third buffer measured no faster: the stream is not latency-bound here.)
    for (int i = 0; i + 1 < n; i += 2) {
      load_chunk(base, i + 1, kB, vB);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this chunk's math
      process_chunk(base, i, kA, vA);
      load_chunk(base, min(i + 2, n - 1), kA, vA);
      __builtin_amdgcn_sched_barrier(0);
      process_chunk(base, i + 1, kB, vB);
    }
    if (n & 1) process_chunk(base, n - 1, kA, vA);
  }

  // Row sum over the 4 lanes that share the row.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  __syncthreads();  // every wave is done with its staging buffers (aliased by the combine)
  if (j == 0) {
    sm.m[w][r16] = m_run;
    sm.l[w][r16] = l_run;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) sm.o[w][r16][16 * mb + 4 * j + i4] = acc[mb][i4];
  __syncthreads();

  // Combine the 4 waves: thread -> (row, 16-byte chunks c + 16 q of the row), so that the
  // 16 threads of a row read, store and merge whole rows.
  constexpr int NQ = D / 64;
  const int row = tid >> 4;
  const int c = tid & 15;
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm.m[ww][row]);
  const float M_use = M == kNegInf ? 0.f : M;
  float L = 0.f;
  f32x4 o[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) o[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const float wv = fast_exp2(sm.m[ww][row] - M_use);
    L += sm.l[ww][row] * wv;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      o[q] += *reinterpret_cast<const f32x4 *>(&sm.o[ww][row][4 * c + 64 * q]) * wv;
  }
  const int frow = rt * kDecodeRows + row;
  const bool out_ok = frow < n_rows;
  const int token = q0 + frow / a.G;
  const int h = g * a.G + frow % a.G;
  if (nsplit == 1) {
    if (!out_ok) return;
    const float inv = a.out_scale / L;
    uint16_t *op = a.out + ((int64_t)token * a.Hq + h) * D + 4 * c;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      *reinterpret_cast<u32x2 *>(op + 64 * q) =
          u32x2{pack_bf16x2(o[q][0] * inv, o[q][1] * inv), pack_bf16x2(o[q][2] * inv, o[q][3] * inv)};
    return;
  }
  // the item's rows: tokens q0 + (rt 16) / G .., heads g G .. (uniform base, per-row offsets)
  const int tok0 = q0 + rt * kDecodeRows / a.G;
  const int h0 = g * a.G;
  if (out_ok) {
    const int64_t prow = ((int64_t)s * a.T + token) * a.Hq + h;
    const __amdgpu_buffer_rsrc_t rows = coherent_rows(partial_base(a, s, tok0, h0, D));
    const uint32_t off = partial_off(a, token - tok0, h - h0, 4 * c, D);
#pragma unroll
    for (int q = 0; q < NQ; ++q) st_coherent16(rows, off + 256 * q, o[q]);
    if (c == 0) {
      st_coherent(a.part_ml + prow * 2 + 0, M);
      st_coherent(a.part_ml + prow * 2 + 1, L);
    }
  }
  // Arrive; the last of the nsplit items of this (sequence, KV head, row tile) merges.
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long *ctr = a.counters + (int64_t)(q0 * a.G + rt * kDecodeRows) * a.Hkv + g;
    sm.last = arrive(ctr, a.call_tag) == (unsigned)nsplit;
  }
  __syncthreads();
  if (!sm.last || !out_ok) return;
  merge_row<D>(a, nsplit, token, h, c, tok0, h0);
}

// =========================================================================== prefill ======
//
// A prefill item is 128 query rows of one KV head: pf_tokens = 128 / G consecutive tokens of
// each of the G query heads of the group (wave w owns rows 32w .. 32w+31), over one KV split.
// The workgroup walks 64-key tiles up to the causal limit of its last token, with two LDS
// buffers: the K/V rows of tile i+1 are loaded straight from global memory into one buffer
// (no register staging) while tile i is computed from the other, so one barrier per tile
// suffices and a tile's load latency is covered by a whole tile of compute.  Tiles below
// every row's causal limit run a body without masking.  A 64-key tile may span several
// pages (page size 16 or 32 included): each 1 KB load instruction looks its page up.
//   QK^T: v_mfma_f32_32x32x16_bf16, A = K tile rows from LDS (ds_read_b128), B = Q^T in
//         registers.  Lane l gets S^T[key 32mb + 8(v/4) + 4(l/32) + v%4][row l%32].
//   PV:   v_mfma_f32_32x32x16_bf16, A = V^T from two transposing LDS reads, B = P^T taken
//         from the lane's own S^T registers (k-slot e of lane half h maps to key
//         16kb + 8(e/4) + 4h + e%4, and the V^T reads use the same order).
// The two tile buffers live in two distinct LDS arrays, so the compiler can tell that the
// direct loads filling one buffer never alias the reads of the other and does not make
// those reads wait for the loads.  Each array holds a 64-key K tile, then the V tile.
template <int D>
constexpr int kPrefillBufBytes = 2 * kPrefillKeys * D * 2;
template <int D>
__device__ __forceinline__ int prefill_count(const AttnArgs &a, int b) {
  const int q_len = a.cu_q_lens[b + 1] - a.cu_q_lens[b];
  if (q_len == 0 || is_decode_class(a, q_len)) return 0;
  return a.Hkv * ceil_div(q_len, a.pf_tokens) * num_splits_pf(a, b);
}

template <bool B>
using bool_c = std::integral_constant<bool, B>;

template <int D, bool KV8>
__device__ void prefill_item(const AttnArgs &a, int id, char *lds0, char *lds1, int *last_flag,
                             const SeqOrder *order = nullptr) {
  constexpr int KS = D / 16;                                // QK^T MFMAs per 32-key block
  constexpr int MD = D / 32;                                // PV output blocks of 32 dims
  constexpr int kChunks = D / 8;                            // 16-byte chunks per row
  constexpr int RPI = 64 / kChunks;                         // rows per 1 KB LDS load instruction
  constexpr int LPW = kPrefillKeys / RPI / 4;               // load instructions per wave per tile
  uint16_t *const kbuf[2] = {reinterpret_cast<uint16_t *>(lds0), reinterpret_cast<uint16_t *>(lds1)};
  uint16_t *const vbuf[2] = {kbuf[0] + kPrefillKeys * D, kbuf[1] + kPrefillKeys * D};
  const int tid = item_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  ItemRef it;
  int b, q0, q_len, max_kv;
  if (order != nullptr && order->n > 0) {  // everything from the kernel arguments
    if (order->interleave) {
      // rank r of every sequence before rank r + 1 of any: id = (r n + i) Hkv nsplit + rest
      if (id >= order->first[order->n]) return;
      const int per_rank = a.Hkv * max(1, ceil_div(order->kv[0], a.split_pf));
      const int r = id / (order->n * per_rank);
      const int i = (id / per_rank) % order->n;
      it = {i, r * per_rank + id % per_rank};
    } else {
      it = ordered_item(*order, id);
      if (it.b < 0) return;
    }
    b = order->seq[it.b];
    q0 = order->q0[it.b];
    q_len = order->q_len[it.b];
    max_kv = order->kv[it.b];
  } else {
    it = find_item(id, a.B, [&](int bb) { return prefill_count<D>(a, bb); });
    b = __builtin_amdgcn_readfirstlane(it.b);
    if (b < 0) return;
    q0 = a.cu_q_lens[b];
    q_len = a.cu_q_lens[b + 1] - q0;
    max_kv = max_kv_len(a, b);
  }
  const int n_qt = ceil_div(q_len, a.pf_tokens);
  const int nsplit = max(1, ceil_div(max_kv, a.split_pf));  // as num_splits_pf
  int rem = __builtin_amdgcn_readfirstlane(it.rem);
  const int s = rem % nsplit;
  rem /= nsplit;
  const int g = rem % a.Hkv;
  const int qt = n_qt - 1 - rem / a.Hkv;  // heaviest (latest) query tiles first
  const int kv_len = a.kvl_head_stride == 0 ? max_kv : kv_len_of(a, b, g);  // per head if head-major
  const int past = kv_len - q_len;
  const int t_first = qt * a.pf_tokens;
  const int t_last = min(q_len - 1, t_first + a.pf_tokens - 1);
  const int split = even_split(max_kv, nsplit);
  const int k_begin = s * split;
  const int k_end = min(min(kv_len, k_begin + split), past + t_last + 1);
  const int n_tiles = k_end > k_begin ? ceil_div(k_end - k_begin, kPrefillKeys) : 0;
  // Tiles whose keys are all below every row's causal limit (and inside the range) need no mask.
  const int lim_all = min(k_end, past + t_first + 1);
  const int n_full = min(n_tiles, lim_all > k_begin ? (lim_all - k_begin) / kPrefillKeys : 0);
  const bool fused = a.k_new != nullptr;
  const bool writer = fused && qt == n_qt - 1;  // the last query tile visits every new key

  // This lane's query row.
  const int rr = 32 * w + r32;
  const int hg = rr / a.pf_tokens;
  const int t_row = t_first + rr % a.pf_tokens;
  const bool row_ok = hg < a.G && t_row < q_len;
  const int h_row = g * a.G + (row_ok ? hg : 0);
  const int row_lim = past + (row_ok ? t_row : 0) + 1;
  bf16x8 qf[KS];
  {
    const uint16_t *qp = a.q + ((int64_t)(q0 + (row_ok ? t_row : 0)) * a.Hq + h_row) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4 *>(qp + 16 * ks + 8 * hf);
      qf[ks] = as_bf16x8(v);
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x16 acc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[md][v] = 0.f;

  const int page_mask = (1 << a.page_shift) - 1;
  // Pages of the item's logical blocks, 64 at a time: lane l holds block pg_blk0 + l.  A tile
  // spans at most 4 blocks, so a reload happens only when a tile runs past the window.
  const int blk_begin = k_begin >> a.page_shift;
  const int blk_end = k_end > 0 ? ((k_end - 1) >> a.page_shift) + 1 : 0;
  int pg_lane = 0, pg_blk0 = 0;
  auto fetch_pages = [&](int blk0) {
    const int blk = blk0 + lane;
    pg_lane = blk < blk_end ? checked_page(table_at(a, b, g, blk), a.num_pages) : 0;
    pg_blk0 = blk0;
    // Wait here, once per window: otherwise every page lookup would wait for all loads in
    // flight, the tile loads included.
    wait_all_memory();
  };
  // Tile loads go straight from global memory into LDS: one instruction fills 1 KB, i.e.
  // RPI = 64 / (D/8) consecutive rows, lane l taking 16 bytes of row l / (D/8).  Wave w issues
  // instructions i = 4u + w.  An instruction's rows share one page (pages hold at least 16
  // rows), so its page comes from the table window with one readlane.  The lane's LDS slot is
  // fixed, so it loads the global chunk that the row's swizzle puts in that slot; the swizzle
  // depends on the instruction only through i mod 4, i.e. through w, so the chunk is a
  // per-lane constant.
  const int ld_row = lane / kChunks;                                    // row within an instruction
  const int ld_c8 = swz_chunk<D>(RPI * w + ld_row, lane % kChunks) * 8;  // global element offset
  const int grp_last = (k_end - 1) & ~(RPI - 1);  // last instruction group holding a key of the range
  // Per-item constants of the tile loads.  Cache strides fit 32 bits (elements within a page
  // and of a page); only page * page_stride needs 64.
  const uint16_t *const kc_g = a.k_cache + (int64_t)g * a.head_stride;  // KV head g's rows
  const uint16_t *const vc_g = a.v_cache + (int64_t)g * a.head_stride;
  const int new_stride = a.Hkv * D;  // elements between consecutive new tokens
  const int64_t new_row0 = ((int64_t)(q0 - past) * a.Hkv + g) * D;  // element of new key 0
  const int pstride = (int)a.page_stride;
  const int sstride = (int)a.slot_stride;
  const uint32_t lo_new = (uint32_t)(ld_row * new_stride + ld_c8) * 2u;  // lane byte offsets
  const uint32_t lo_cache = (uint32_t)(ld_row * sstride + ld_c8) * 2u;
  auto issue_group = [&](int i, int g0, bool is_new, uint32_t lo, uint16_t *kdst, uint16_t *vdst) {
    if (is_new) {
      const int64_t nb = new_row0 + (int64_t)g0 * new_stride;
      load_lds16(reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(a.k_new + nb) + lo), kdst);
      load_lds16(reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(a.v_new + nb) + lo), vdst);
    } else {
      const int page = read_page(__builtin_amdgcn_readlane(pg_lane, (g0 >> a.page_shift) - pg_blk0));
      const int64_t cb = (int64_t)page * pstride + (g0 & page_mask) * sstride;
      load_lds16(reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(kc_g + cb) + lo), kdst);
      load_lds16(reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(vc_g + cb) + lo), vdst);
    }
  };
  auto issue_tile = [&](int tile, auto par) {  // par: the tile's buffer, tile & 1
    constexpr int buf = decltype(par)::value;
    const int kt0 = k_begin + tile * kPrefillKeys;
    const int last_blk = (min(kt0 + kPrefillKeys, k_end) - 1) >> a.page_shift;
    if (last_blk - pg_blk0 >= 64) fetch_pages(kt0 >> a.page_shift);
    const bool all_new = fused && kt0 >= past;
    const bool all_cached = !fused || kt0 + kPrefillKeys <= past;
    if (kt0 + kPrefillKeys <= k_end && (all_new || all_cached)) {
      // Common case: every group of the tile is in range and of one kind.
#pragma unroll
      for (int u = 0; u < LPW; ++u) {
        const int i = 4 * u + w;
        issue_group(i, kt0 + RPI * i, all_new, all_new ? lo_new : lo_cache,
                    kbuf[buf] + i * RPI * D, vbuf[buf] + i * RPI * D);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int i = 4 * u + w;
      const int g0 = min(kt0 + RPI * i, grp_last);  // groups past the range reload the last one
      // rows past the range repeat its last key (their probabilities are zero; the slots past
      // a sequence's end may hold anything, so they are never loaded)
      const int lr = g0 + RPI > k_end ? min(ld_row, k_end - 1 - g0) : ld_row;
      uint16_t *const kdst = kbuf[buf] + i * RPI * D;
      uint16_t *const vdst = vbuf[buf] + i * RPI * D;
      if (fused && g0 < past && g0 + RPI > past) {
        // the group straddles the first new key: every row is located on its own
        const int pos = g0 + lr;
        const int64_t off = pos >= past
                                ? new_row0 + (int64_t)pos * new_stride + ld_c8
                                : (int64_t)read_page(__builtin_amdgcn_readlane(pg_lane, (g0 >> a.page_shift) - pg_blk0)) *
                                          pstride + (pos & page_mask) * sstride + ld_c8;
        load_lds16((pos >= past ? a.k_new : kc_g) + off, kdst);
        load_lds16((pos >= past ? a.v_new : vc_g) + off, vdst);
      } else {
        const bool is_new = fused && g0 >= past;
        const uint32_t lo = (uint32_t)(lr * (is_new ? new_stride : sstride) + ld_c8) * 2u;
        issue_group(i, g0, is_new, lo, kdst, vdst);
      }
    }
  };
  // The item owning the sequence's last query rows stores the tile's new keys from LDS into
  // their page slots (the page window still covers the tile).
  auto write_new_rows = [&](int tile, auto par) {
    constexpr int buf = decltype(par)::value;
    const int kt0 = k_begin + tile * kPrefillKeys;
    if (kt0 + kPrefillKeys <= past) return;
#pragma unroll
    for (int u = 0; u < kPrefillKeys * kChunks / kThreads; ++u) {
      const int cid = u * kThreads + tid;
      const int key = cid / kChunks;
      const int c = cid % kChunks;
      const int pos = kt0 + key;
      const int page = __shfl(pg_lane, (pos >> a.page_shift) - pg_blk0);  // every lane takes part
      if (pos >= past && pos < k_end && page >= 0) {
        const int64_t off = kv_row_offset(a, page, pos & page_mask, g) + c * 8;
        *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(a.k_cache) + off) =
            *reinterpret_cast<const u32x4 *>(kbuf[buf] + lds_off<D>(key, c));
        *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(a.v_cache) + off) =
            *reinterpret_cast<const u32x4 *>(vbuf[buf] + lds_off<D>(key, c));
      }
    }
  };

  // FP8 cache: tiles go through registers instead (codes, or the bf16 values of new keys),
  // and are written to LDS as the codes' bf16 values in the bf16 layout.  Wave w, round u
  // takes rows RPW8 (4u + w) .. + RPW8 - 1 of the tile (one page: RPW8 <= 16 and aligned),
  // lane l 16 values of row l / LPR8.
  constexpr int LPR8 = D / 16;                     // lanes per row
  constexpr int RPW8 = 64 / LPR8;                  // rows per wave per round
  constexpr int NR8 = kPrefillKeys / (4 * RPW8);   // rounds per tile
  const int lr8 = lane / LPR8;
  const int c16 = lane % LPR8;
  const uint8_t *const kc8 = reinterpret_cast<const uint8_t *>(a.k_cache) + (int64_t)g * a.head_stride;
  const uint8_t *const vc8 = reinterpret_cast<const uint8_t *>(a.v_cache) + (int64_t)g * a.head_stride;
  u32x4 kst[2 * NR8], vst[2 * NR8];
  auto load8 = [&](int tile) {
    const int kt0 = k_begin + tile * kPrefillKeys;
    const int last_blk = (min(kt0 + kPrefillKeys, k_end) - 1) >> a.page_shift;
    if (last_blk - pg_blk0 >= 64) fetch_pages(kt0 >> a.page_shift);
#pragma unroll
    for (int u = 0; u < NR8; ++u) {
      const int g0 = min(kt0 + RPW8 * (4 * u + w), k_end - 1);  // rows past the range repeat
      const int key = min(g0 + lr8, k_end - 1);                  // the range's last key
      // Every lane loads twice, from addresses chosen per lane (no branch): a cached row's 16
      // codes (the second load repeats the first, a cache hit), or a new row's 16 bf16 values.
      const int page = read_page(__builtin_amdgcn_readlane(pg_lane, (g0 >> a.page_shift) - pg_blk0));
      const int64_t off = (int64_t)page * pstride + (key & page_mask) * sstride + 16 * c16;
      const int64_t noff = new_row0 + (int64_t)key * new_stride + 16 * c16;
      const bool is_new = fused && key >= past;
      const uint8_t *k0 = is_new ? reinterpret_cast<const uint8_t *>(a.k_new + noff) : kc8 + off;
      const uint8_t *v0 = is_new ? reinterpret_cast<const uint8_t *>(a.v_new + noff) : vc8 + off;
      const int step = is_new ? 16 : 0;
      kst[2 * u] = *reinterpret_cast<const u32x4 *>(k0);
      kst[2 * u + 1] = *reinterpret_cast<const u32x4 *>(k0 + step);
      vst[2 * u] = *reinterpret_cast<const u32x4 *>(v0);
      vst[2 * u + 1] = *reinterpret_cast<const u32x4 *>(v0 + step);
    }
  };
  auto commit8 = [&](int tile, auto par) {
    constexpr int buf = decltype(par)::value;
    const int kt0 = k_begin + tile * kPrefillKeys;
#pragma unroll
    for (int u = 0; u < NR8; ++u) {
      const int row = RPW8 * (4 * u + w) + lr8;  // row within the tile
      const int g0 = min(kt0 + RPW8 * (4 * u + w), k_end - 1);
      const int key = min(kt0 + row, k_end - 1);
      u32x4 kc = kst[2 * u], vc = vst[2 * u];
      if (fused && key >= past) {
        kc = quantize16(kst[2 * u], kst[2 * u + 1], a.k_inv);
        vc = quantize16(vst[2 * u], vst[2 * u + 1], a.v_inv);
        const int page = __builtin_amdgcn_readlane(pg_lane, (g0 >> a.page_shift) - pg_blk0);
        if (writer && kt0 + row < k_end && page >= 0) {  // the item owning the last query rows stores them
          const int64_t off = (int64_t)page * pstride + (key & page_mask) * sstride + 16 * c16;
          *reinterpret_cast<u32x4 *>(const_cast<uint8_t *>(kc8) + off) = kc;
          *reinterpret_cast<u32x4 *>(const_cast<uint8_t *>(vc8) + off) = vc;
        }
      }
      u32x4 lo, hi;
      dequant16(kc, lo, hi);
      *reinterpret_cast<u32x4 *>(kbuf[buf] + lds_off<D>(row, 2 * c16)) = lo;
      *reinterpret_cast<u32x4 *>(kbuf[buf] + lds_off<D>(row, 2 * c16 + 1)) = hi;
      dequant16(vc, lo, hi);
      *reinterpret_cast<u32x4 *>(vbuf[buf] + lds_off<D>(row, 2 * c16)) = lo;
      *reinterpret_cast<u32x4 *>(vbuf[buf] + lds_off<D>(row, 2 * c16 + 1)) = hi;
    }
  };

  // LDS read addresses that do not change from tile to tile (bytes).
  const int k_rd_base = lds_off<D>(r32, hf) * 2;
  const int i16 = lane & 15;
  const int q4 = lane >> 4;
  const int tr_key = 4 * (q4 >> 1) + (i16 >> 2);
  const int tr_c0 = 2 * (q4 & 1) + ((i16 & 3) >> 1);
  const int v_rd_lo = (lds_off<D>(tr_key, tr_c0) + 4 * (i16 & 1)) * 2;
  const int v_rd_hi = (lds_off<D>(tr_key + 8, tr_c0) + 4 * (i16 & 1)) * 2;

  // One 64-key tile from LDS buffer tile & 1: S^T, (mask), online softmax, O^T += V^T P^T.
  // mid() runs once the score MFMAs are issued: the next tile's loads go out while those
  // MFMAs execute instead of before them, when every wave of the compute unit issues its
  // loads at once after the barrier (measured: prefill 2.5% and block-union sparse 1.5%
  // faster; interleaving the loads one by one between the MFMAs measured 2-9% slower).
  auto compute_tile = [&](int tile, auto par, auto masked, auto mid) {
    const int kt0 = k_begin + tile * kPrefillKeys;
    const uint16_t *kt = kbuf[decltype(par)::value];
    const uint16_t *vt = vbuf[decltype(par)::value];
    // K operand reads: row 32mb + r32, logical chunk 2ks + hf.  The swizzle XORs the chunk
    // index with a function of the row that is the same for both mb, so the byte address is
    // (k_rd_base ^ 32 ks) + 64 D mb: one VALU op per read.
    const char *kbytes = reinterpret_cast<const char *>(kt);
    // The score MFMAs issue at raised wave priority, so that on a SIMD shared by two waves
    // the one entering its MFMA phase goes first and the other's softmax VALU work runs
    // beside the MFMAs (measured: block-union sparse 6% faster, prefill 2%).
    __builtin_amdgcn_s_setprio(1);
    f32x16 st[2];
    u32x4 kf[2 * KS];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)
      kf[i] = *reinterpret_cast<const u32x4 *>(kbytes + ((k_rd_base ^ (32 * (i % KS))) + 64 * D * (i / KS)));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[mb][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st[mb] = mfma32x32x16(as_bf16x8(kf[mb * KS + ks]), qf[ks], st[mb]);
    }
    // Keep two operand reads in flight ahead of the MFMAs that consume them.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    mid();
    __builtin_amdgcn_s_setprio(0);
    // Row max on the raw scores: the scale is positive, so it is applied once to the max and
    // folded into the exponent below as one FMA per score.
    float mloc = kNegInf;
    const int mask_thr = min(row_lim, k_end) - kt0 - 4 * hf;  // keys kt0 + 4 hf + c, c < thr, stay
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = st[mb][v];
        if constexpr (decltype(masked)::value) {
          // element v of st[mb] is key kt0 + 4 hf + (32 mb + 8 (v / 4) + v % 4)
          x = (32 * mb + 8 * (v >> 2) + (v & 3) < mask_thr) ? x : kNegInf;
          st[mb][v] = x;
        }
        mloc = fmaxf(mloc, x);
      }
    mloc = pair_max32(mloc) * a.scale_log2;
    // Lazy rescale: the running max only moves when a row's max grows by more than 8
    // (log2 units), so probabilities stay below 2^8 and most tiles skip the rescale of the
    // accumulators entirely (the final normalisation divides by l against the same max).
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < MD; ++md) acc[md] = acc[md] * alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    bf16x8 pb[4];
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int mb = kb >> 1;
      const int v0 = 8 * (kb & 1);
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(st[mb][v0 + e], a.scale_log2, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(st[mb][v0 + e + 1], a.scale_log2, -m_use));
        w4[e >> 1] = pack_bf16x2(p0, p1);
        // the row sum takes the same bf16 probabilities the P V product uses
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w4[e >> 1]), ones,
                                                l_run, false);
      }
      pb[kb] = as_bf16x8(u32x4{w4[0], w4[1], w4[2], w4[3]});
    }

    // O^T += V^T P^T.  Lane (i = l%16, quarter q = l/16): half h = q/2 picks keys
    // 16kb + 4h + (0..3) and + 8; q%2 picks the 16-dim half of the 32-dim block.  The read
    // of block md, rows 16kb.. is at (v_rd ^ 64 md) + 4096 kb bytes for D = 128 (the row's
    // swizzle is the same for every kb and XORs the chunk 4 md + c0, c0 < 4).
    const char *vbytes = reinterpret_cast<const char *>(vt);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        int alo, ahi;
        if constexpr (D == 128) {
          alo = (v_rd_lo ^ (64 * md)) + 32 * D * kb;
          ahi = (v_rd_hi ^ (64 * md)) + 32 * D * kb;
        } else {
          alo = (lds_off<D>(16 * kb + tr_key, 4 * md + tr_c0) + 4 * (i16 & 1)) * 2;
          ahi = (lds_off<D>(16 * kb + tr_key + 8, 4 * md + tr_c0) + 4 * (i16 & 1)) * 2;
        }
        const s16x4 lo = lds_read_tr(reinterpret_cast<const uint16_t *>(vbytes + alo));
        const s16x4 hi = lds_read_tr(reinterpret_cast<const uint16_t *>(vbytes + ahi));
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
        acc[md] = mfma32x32x16(va, pb[kb], acc[md]);
      }
    }
  };
  // Tile i: (writer: store its new keys), compute tile i, issuing tile i+1 into the other
  // buffer once its score MFMAs are out, wait for tile i+1 and meet at the barrier.  The
  // buffer tile i+1 goes to was last read while computing tile i-1, which every wave
  // finished before the previous barrier.
  // Buffers are chosen at compile time (tiles are taken in pairs), which keeps the two
  // buffers' accesses apart for the compiler.
  auto step = [&](int tile, auto par, auto masked) {
    constexpr int P = decltype(par)::value;
    if constexpr (KV8) {
      // FP8: tile i+1's loads are in flight in registers while tile i is computed, then
      // they are converted into the other buffer.
      const bool more = tile + 1 < n_tiles;
      if (more) load8(tile + 1);
      compute_tile(tile, par, masked, [] {});
      if (more) commit8(tile + 1, std::integral_constant<int, 1 - P>{});
      __syncthreads();
    } else {
      if (writer) write_new_rows(tile, par);
      compute_tile(tile, par, masked, [&] {
        if (tile + 1 < n_tiles) issue_tile(tile + 1, std::integral_constant<int, 1 - P>{});
      });
      wait_all_memory();
      __syncthreads();
    }
  };
  using even = std::integral_constant<int, 0>;
  using odd = std::integral_constant<int, 1>;
  if (n_tiles > 0) {
    fetch_pages(blk_begin);
    if constexpr (KV8) {
      load8(0);
      commit8(0, even{});
    } else {
      issue_tile(0, even{});
    }
  }
  // Nothing the prologue loaded (Q, tile 0) may still be in flight inside the loop: a wait
  // there would also wait for the next tile's loads.
  wait_all_memory();
  __syncthreads();
  int tile = 0;
  for (; tile + 2 <= n_full; tile += 2) {
    step(tile, even{}, bool_c<false>{});
    step(tile + 1, odd{}, bool_c<false>{});
  }
  for (; tile + 2 <= n_tiles; tile += 2) {
    step(tile, even{}, bool_c<true>{});
    step(tile + 1, odd{}, bool_c<true>{});
  }
  if (tile < n_tiles) step(tile, even{}, bool_c<true>{});

  l_run = pair_sum32(l_run);  // the row sum over both lane halves
  const int token = q0 + t_row;
  if (nsplit == 1) {
    if (!row_ok) return;
    const float inv = a.out_scale / l_run;
    uint16_t *op = a.out + ((int64_t)token * a.Hq + h_row) * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int d = 32 * md + 8 * vq + 4 * hf;
        const uint32_t w0 = pack_bf16x2(acc[md][4 * vq + 0] * inv, acc[md][4 * vq + 1] * inv);
        const uint32_t w1 = pack_bf16x2(acc[md][4 * vq + 2] * inv, acc[md][4 * vq + 3] * inv);
        *reinterpret_cast<u32x2 *>(op + d) = u32x2{w0, w1};
      }
    return;
  }
  // The item's rows: tokens q0 + t_first .., heads g G .. (uniform base, per-row offsets).
  // The partial goes out whole rows at a time: each wave's rows are staged in LDS (free once
  // the last tile is done; rows 0..63 in the first buffer, 64..127 in the second, 16-byte
  // chunks swizzled by the row), then lane l of a group of CH = D/4 lanes stores chunk l of
  // one row, so every write-through store covers whole lines.
  const int tok0 = q0 + t_first;
  const int h0 = g * a.G;
  constexpr int CH = D / 4;             // 16-byte chunks per row
  constexpr int RPS = kThreads / CH;    // rows per workgroup-wide step
  auto stage_row = [&](int row) {
    return reinterpret_cast<float *>(row < 64 ? lds0 : lds1) + (row & 63) * D;
  };
  {
    float *st = stage_row(rr);
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int c = 8 * md + 2 * vq + hf;  // dims 4c .. 4c+3 = 32 md + 8 vq + 4 hf
        *reinterpret_cast<f32x4 *>(st + 4 * (c ^ (rr & (CH - 1)))) =
            f32x4{acc[md][4 * vq], acc[md][4 * vq + 1], acc[md][4 * vq + 2], acc[md][4 * vq + 3]};
      }
  }
  if (row_ok && hf == 0) {
    const int64_t prow = ((int64_t)s * a.T + token) * a.Hq + h_row;
    st_coherent(a.part_ml + prow * 2 + 0, m_run);
    st_coherent(a.part_ml + prow * 2 + 1, l_run);
  }
  __syncthreads();
  const int lc = tid % CH;  // this lane's chunk
  {
    const __amdgpu_buffer_rsrc_t rows = coherent_rows(partial_base(a, s, tok0, h0, D));
#pragma unroll
    for (int i = 0; i < kPrefillRows / RPS; ++i) {
      const int row = i * RPS + tid / CH;
      const int rt = row % a.pf_tokens, rhg = row / a.pf_tokens;
      if (rhg < a.G && t_first + rt < q_len)
        st_coherent16(rows, partial_off(a, rt, rhg, 4 * lc, D),
                      *reinterpret_cast<const f32x4 *>(stage_row(row) + 4 * (lc ^ (row & (CH - 1)))));
    }
  }
  // Arrive; the last of the nsplit items of this (query tile, KV head) merges all partials.
  wait_all_memory();
  __syncthreads();
  if (tid == 0) {
    unsigned long long *ctr = a.counters + a.pf_counter_base + (int64_t)(q0 + t_first) * a.Hkv + g;
    *last_flag = arrive(ctr, a.call_tag) == (unsigned)nsplit;
  }
  __syncthreads();
  if (!*last_flag) return;
  // Merge, whole rows again: kRB rows per lane group in flight, splits in batches of 4 whose
  // loads are all issued before any is used.
  constexpr int kRB = 4;
#pragma unroll 1
  for (int i0 = 0; i0 < kPrefillRows / RPS; i0 += kRB) {
    float M[kRB], L[kRB];
    f32x4 o[kRB];
    int rt[kRB], rhg[kRB];
    bool ok[kRB];
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      const int row = (i0 + j) * RPS + tid / CH;
      rt[j] = row % a.pf_tokens;
      rhg[j] = row / a.pf_tokens;
      ok[j] = rhg[j] < a.G && t_first + rt[j] < q_len;
      M[j] = kNegInf;
      L[j] = 0.f;
      o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
      float mv[kRB][4], lv[kRB][4];
      f32x4 ov[kRB][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int su = min(s0 + u, nsplit - 1);
        const __amdgpu_buffer_rsrc_t rows = coherent_rows(partial_base(a, su, tok0, h0, D));
#pragma unroll
        for (int j = 0; j < kRB; ++j) {
          // rows past the item read its first row (always valid); their results are dropped
          const int jt = ok[j] ? rt[j] : 0, jh = ok[j] ? rhg[j] : 0;
          const int64_t pr = ((int64_t)su * a.T + tok0 + jt) * a.Hq + h0 + jh;
          mv[j][u] = ld_coherent(a.part_ml + pr * 2);
          lv[j][u] = ld_coherent(a.part_ml + pr * 2 + 1);
          ov[j][u] = ld_coherent16(rows, partial_off(a, jt, jh, 4 * lc, D));
        }
      }
#pragma unroll
      for (int j = 0; j < kRB; ++j) {
        float Mn = M[j];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < nsplit) Mn = fmaxf(Mn, mv[j][u]);
        const float Mu = Mn == kNegInf ? 0.f : Mn;
        const float sc = fast_exp2(M[j] - Mu);
        L[j] *= sc;
        o[j] = o[j] * sc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (s0 + u >= nsplit) continue;
          const float wv = fast_exp2(mv[j][u] - Mu);
          L[j] += lv[j][u] * wv;
          o[j] += ov[j][u] * wv;
        }
        M[j] = Mn;
      }
    }
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      if (!ok[j]) continue;
      const float inv = a.out_scale / L[j];
      uint16_t *op = a.out + ((int64_t)(tok0 + rt[j]) * a.Hq + h0 + rhg[j]) * D + 4 * lc;
      *reinterpret_cast<u32x2 *>(op) =
          u32x2{pack_bf16x2(o[j][0] * inv, o[j][1] * inv), pack_bf16x2(o[j][2] * inv, o[j][3] * inv)};
    }
  }
}

// =========================================================================== kernels ======

#ifndef RPA_DECODE_MIN_BLOCKS
#define RPA_DECODE_MIN_BLOCKS 2
#endif
template <int D, bool KV8>
__global__ __launch_bounds__(kThreads, RPA_DECODE_MIN_BLOCKS) void decode_kernel(AttnArgs a, SeqOrder o) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(DecodeSmem<D>)];
  decode_item<D, KV8>(a, blockIdx.x, smem, &o);
}

template <int D, bool KV8>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(AttnArgs a, SeqOrder o) {
  __shared__ __attribute__((aligned(16))) char lds0[kPrefillBufBytes<D>];
  __shared__ __attribute__((aligned(16))) char lds1[kPrefillBufBytes<D>];
  __shared__ int last;
  prefill_item<D, KV8>(a, blockIdx.x, lds0, lds1, &last, &o);
}

// One launch for a batch holding both kinds: prefill items first (they are the longest),
// then the decode items, whose LDS overlays the first prefill buffer.
template <int D>
constexpr size_t kMixedLds0Bytes =
    sizeof(DecodeSmem<D>) > (size_t)kPrefillBufBytes<D> ? sizeof(DecodeSmem<D>) : kPrefillBufBytes<D>;

template <int D, bool KV8>
__global__ __launch_bounds__(kThreads, 2) void mixed_kernel(AttnArgs a, SeqOrder o) {
  __shared__ __attribute__((aligned(16))) char lds0[kMixedLds0Bytes<D>];
  __shared__ __attribute__((aligned(16))) char lds1[kPrefillBufBytes<D>];
  __shared__ int last;
  if ((int)blockIdx.x < a.n_pf_items)
    prefill_item<D, KV8>(a, blockIdx.x, lds0, lds1, &last);
  else
    decode_item<D, KV8>(a, blockIdx.x - a.n_pf_items, lds0, &o);
}

template <int D, bool KV8>
static hipError_t launch_attention_d(const AttnArgs &a, const SeqOrder &o, AttnKernel kind,
                                     int n_blocks, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_blocks), block(kThreads);
  switch (kind) {
    case AttnKernel::kDecode:
      hipLaunchKernelGGL((decode_kernel<D, KV8>), grid, block, 0, stream, a, o);
      break;
    case AttnKernel::kPrefill:
      hipLaunchKernelGGL((prefill_kernel<D, KV8>), grid, block, 0, stream, a, o);
      break;
    case AttnKernel::kMixed:
      hipLaunchKernelGGL((mixed_kernel<D, KV8>), grid, block, 0, stream, a, o);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, const SeqOrder &o, int D, AttnKernel kind,
                            int n_blocks, hipStream_t stream) {
  if (D == 128)
    return a.kv8 ? launch_attention_d<128, true>(a, o, kind, n_blocks, stream)
                 : launch_attention_d<128, false>(a, o, kind, n_blocks, stream);
  return a.kv8 ? launch_attention_d<64, true>(a, o, kind, n_blocks, stream)
               : launch_attention_d<64, false>(a, o, kind, n_blocks, stream);
}

}  // namespace rpa

// ===================================================================== graph-capturable ======
//
// One persistent launch that plans on the device.  Every workgroup reads the batch lengths
// and derives, redundantly, the same plan the host planner derives from its mirrors
// (decode-class sequences: q_len * G <= 16; KV split sizes cutting the work into about
// mixed_dec_items decode items beside prefill-class work or decode_only_items alone, and
// about mixed_pf_items prefill items beside decode work or prefill_only_items (1024-key
// minimum) alone), with at most max_splits splits per sequence.  Workgroup w runs item w first and then takes items from a queue; the last
// workgroup to leave resets the queue and advances the call tag for the next call.
namespace rpa {

__device__ __forceinline__ int g_choose_split(long long units, int longest_kv, int min_keys,
                                              long long target, int max_splits) {
  const long long per_item = max(1ll, (units + target - 1) / target);
  long long split = max(per_item * 64, (long long)min_keys);
  const long long floor_for_cap = (long long)ceil_div(ceil_div(longest_kv, 64), max_splits) * 64;
  split = max(split, floor_for_cap);
  return (int)min(split, (long long)(1 << 30));
}

struct GraphCall {
  uint32_t status;
  int split_dec, split_pf, n_pf_items, n_items;
  DecodeClasses classes;  // decode items class by class (longest items first)
};

// Workgroup-wide reduction scratch of the planning step (not shared with the items' LDS).
struct PlanScratch {
  long long units[kThreads / 64][2];  // decode, prefill 64-key units
  int longest[kThreads / 64][2];      // longest kv_len of each class
  int bad[kThreads / 64];
  long long items[kThreads / 64][kDecClasses + 1];  // decode items per class, prefill items
};

// Wave-wide reduction of non-negative 32-bit values with DPP moves (no LDS round trips):
// pairs and quads, then half rows and rows of 16 lanes (every lane then holds its row's
// result), then rows 1 and 3 take rows 0 and 2 (row broadcast of lane 15) and rows 2 and 3
// take row 1 (row broadcast of lane 31); lane 63 ends with the whole wave's result.
template <class Op>
__device__ __forceinline__ int wave_reduce_dpp(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false));  // row_mirror
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max32(int v) {
  return wave_reduce_dpp(v, [](int x, int y) { return max(x, y); });
}
__device__ __forceinline__ int wave_or32(int v) {
  return wave_reduce_dpp(v, [](int x, int y) { return x | y; });
}
// Exact for per-lane values below 2^50: the low 24 bits and the rest are summed apart
// (64 lanes of 24-bit parts stay below 2^30, of 26-bit parts below 2^32).
__device__ __forceinline__ long long wave_sum64(long long v) {
  auto add = [](int x, int y) { return (int)((unsigned)x + (unsigned)y); };
  const unsigned lo = (unsigned)wave_reduce_dpp((int)(v & 0xffffff), add);
  const unsigned hi = (unsigned)wave_reduce_dpp((int)(v >> 24), add);
  return (long long)lo + ((long long)hi << 24);
}

// The plan of a graph-capturable call, computed by every thread of the workgroup alike.
__device__ GraphCall plan_graph_call(const GraphPlanArgs &p, PlanScratch &red) {
  const int tid = threadIdx.x, wave = tid >> 6;
  // q_len and the longest kv_len of sequence b; bad when a length breaks a precondition.
  auto seq = [&](int b, int &q_len, int &kv_max) {
    q_len = p.cu_q_lens[b + 1] - p.cu_q_lens[b];
    kv_max = 0;
    bool bad = q_len < 0;
    const int heads = p.kvl_head_stride ? p.Hkv : 1;
    for (int g = 0; g < heads; ++g) {
      const int kv = p.kv_lens[b * p.kvl_seq_stride + g * p.kvl_head_stride];
      bad |= kv < q_len || ceil_div(kv, p.page_size) > p.max_pages;
      kv_max = max(kv_max, kv);
    }
    return bad;
  };
  auto is_dec = [&](int q_len) { return (long long)q_len * p.G <= kDecodeRows; };
  // The first sequence of each thread stays in registers for the second pass.
  int q0 = 0, kv0 = 0;
  int bad = tid < p.B && seq(tid, q0, kv0) ? 4 : 0;
  long long dec_units = 0, pf_units = 0;
  int dec_long = 0, pf_long = 0;
  // (selects, not branches: branches here made the compiler keep the accumulators in an
  // indexed scratch array)
  auto count_units = [&](int q_len, int kv) {
    const bool live = q_len > 0, dec = is_dec(q_len);
    const long long du = (long long)p.Hkv * ceil_div(q_len * p.G, kDecodeRows) * ceil_div(kv, 64);
    const long long pu = (long long)p.Hkv * ceil_div(q_len, p.pf_tokens) * ceil_div(kv, 64);
    dec_units += live && dec ? du : 0;
    pf_units += live && !dec ? pu : 0;
    dec_long = live && dec ? max(dec_long, kv) : dec_long;
    pf_long = live && !dec ? max(pf_long, kv) : pf_long;
  };
  if (tid < p.B) count_units(q0, kv0);
  for (int b = tid + kThreads; b < p.B; b += kThreads) {
    int q_len, kv;
    if (seq(b, q_len, kv)) bad |= 4;
    count_units(q_len, kv);
  }
  if (tid == 0) {
    if (p.cu_q_lens[0] != 0) bad |= 1;
    if (p.cu_q_lens[p.B] > p.T_max) bad |= 2;
  }
  dec_units = wave_sum64(dec_units);
  pf_units = wave_sum64(pf_units);
  dec_long = wave_max32(dec_long);
  pf_long = wave_max32(pf_long);
  bad = wave_or32(bad);
  if (lane_id() == 0) {
    red.units[wave][0] = dec_units;
    red.units[wave][1] = pf_units;
    red.longest[wave][0] = dec_long;
    red.longest[wave][1] = pf_long;
    red.bad[wave] = bad;
  }
  __syncthreads();
  dec_units = pf_units = 0;
  dec_long = pf_long = bad = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    dec_units += red.units[w][0];
    pf_units += red.units[w][1];
    dec_long = max(dec_long, red.longest[w][0]);
    pf_long = max(pf_long, red.longest[w][1]);
    bad |= red.bad[w];
  }
  GraphCall c;
  c.status = (uint32_t)bad;
  c.split_dec = dec_units > 0 ? g_choose_split(dec_units, dec_long, 256,
                                               pf_units == 0 ? p.decode_only_items : p.mixed_dec_items,
                                               p.max_splits)
                              : (1 << 30);
  c.split_pf = pf_units == 0 ? (1 << 30)
               : dec_units > 0 ? g_choose_split(pf_units, pf_long, 512, p.mixed_pf_items, p.max_splits)
                               : g_choose_split(pf_units, pf_long, 1024, p.prefill_only_items, p.max_splits);
  long long n_cls[kDecClasses], n_pf = 0;
#pragma unroll
  for (int kk = 0; kk < kDecClasses; ++kk) n_cls[kk] = 0;
  auto count_items = [&](int q_len, int kv) {
    const bool live = q_len > 0, dec = is_dec(q_len);
    const long long nd = (long long)p.Hkv * ceil_div(q_len * p.G, kDecodeRows) * max(1, ceil_div(kv, c.split_dec));
    const long long np = (long long)p.Hkv * ceil_div(q_len, p.pf_tokens) * max(1, ceil_div(kv, c.split_pf));
    const int k = dec_class(kv, c.split_dec);
#pragma unroll
    for (int kk = 0; kk < kDecClasses; ++kk) n_cls[kk] += live && dec && kk == k ? nd : 0;
    n_pf += live && !dec ? np : 0;
  };
  if (tid < p.B) count_items(q0, kv0);
  for (int b = tid + kThreads; b < p.B; b += kThreads) {
    int q_len, kv;
    seq(b, q_len, kv);
    count_items(q_len, kv);
  }
#pragma unroll
  for (int kk = 0; kk < kDecClasses; ++kk) n_cls[kk] = wave_sum64(n_cls[kk]);
  n_pf = wave_sum64(n_pf);
  if (lane_id() == 0) {
#pragma unroll
    for (int kk = 0; kk < kDecClasses; ++kk) red.items[wave][kk] = n_cls[kk];
    red.items[wave][kDecClasses] = n_pf;
  }
  __syncthreads();
  long long n_dec = 0;
  n_pf = 0;
  c.classes.dec_first[0] = 0;
#pragma unroll
  for (int kk = 0; kk < kDecClasses; ++kk) {
    long long nk = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) nk += red.items[w][kk];
    n_dec += nk;
    c.classes.dec_first[kk + 1] = __builtin_amdgcn_readfirstlane((int)n_dec);
  }
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) n_pf += red.items[w][kDecClasses];
  c.n_pf_items = bad ? 0 : (int)n_pf;
  c.n_items = bad ? 0 : (int)(n_pf + n_dec);
  // Every lane holds the same plan: keep it in scalar registers.
  c.status = __builtin_amdgcn_readfirstlane(c.status);
  c.split_dec = __builtin_amdgcn_readfirstlane(c.split_dec);
  c.classes.split = c.split_dec;
  c.split_pf = __builtin_amdgcn_readfirstlane(c.split_pf);
  c.n_pf_items = __builtin_amdgcn_readfirstlane(c.n_pf_items);
  c.n_items = __builtin_amdgcn_readfirstlane(c.n_items);
  return c;
}

// Persistent attention: items run exactly as in the mixed kernel (prefill items first).
template <int D, bool KV8>
__global__ __launch_bounds__(kThreads, 2) void graph_kernel(AttnArgs args, GraphPlanArgs p) {
  __shared__ __attribute__((aligned(16))) char lds0[kMixedLds0Bytes<D>];
  __shared__ __attribute__((aligned(16))) char lds1[kPrefillBufBytes<D>];
  __shared__ int last;
  __shared__ int s_item;
  __shared__ PlanScratch red;
  GraphPlan *plan = p.plan;
  // The tag of this call: the plan's tag is advanced only after every workgroup has left.
  const unsigned long long tag = __hip_atomic_load(&plan->tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
  const GraphCall c = plan_graph_call(p, red);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    plan->status = c.status;
    plan->split_dec = c.split_dec;
    plan->split_pf = c.split_pf;
    plan->n_pf_items = c.n_pf_items;
    plan->n_items = c.n_items;
  }
  AttnArgs a = args;
  a.split_dec = c.split_dec;
  a.split_pf = c.split_pf;
  a.n_pf_items = c.n_pf_items;
  a.call_tag = (tag & ((1ull << 40) - 1)) << 24;
  auto next_item = [&]() {
    __syncthreads();  // the item is done with the LDS and with s_item
    if (threadIdx.x == 0) s_item = (int)(gridDim.x + atomicAdd(&plan->queue, 1u));
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(s_item);
  };
  // One loop per batch kind: a loop that holds only one kind of item keeps its registers
  // to that kind (a shared loop measured ~20% slower per decode item).
  if (c.n_pf_items == 0) {
    for (int item = blockIdx.x; item < c.n_items; item = next_item())
      decode_item<D, KV8>(a, item, lds0, nullptr, &c.classes);
  } else if (c.n_pf_items == c.n_items) {
    for (int item = blockIdx.x; item < c.n_items; item = next_item())
      prefill_item<D, KV8>(a, item, lds0, lds1, &last);
  } else {
    for (int item = blockIdx.x; item < c.n_items; item = next_item()) {
      if (item < c.n_pf_items)
        prefill_item<D, KV8>(a, item, lds0, lds1, &last);
      else
        decode_item<D, KV8>(a, item - c.n_pf_items, lds0, nullptr, &c.classes);
    }
  }
  // Leaving: the queue and tag accesses of this workgroup are complete (their values were
  // used), so the last one to arrive can reset them; the next call sees the reset after the
  // kernel boundary.  Relaxed on purpose: an acquire/release here would write back and
  // invalidate the L2 of the workgroup's XCD under the workgroups still running there.
  if (threadIdx.x == 0) {
    const uint32_t left = __hip_atomic_fetch_add(&plan->exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left == gridDim.x - 1) {
      __hip_atomic_store(&plan->queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&plan->exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&plan->tag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_graph_attention(const AttnArgs &a, const GraphPlanArgs &p, int D,
                                  int n_workgroups, hipStream_t stream) {
  const dim3 grid((unsigned)n_workgroups), block(kThreads);
  if (D == 128)
    hipLaunchKernelGGL((a.kv8 ? graph_kernel<128, true> : graph_kernel<128, false>), grid, block, 0,
                       stream, a, p);
  else
    hipLaunchKernelGGL((a.kv8 ? graph_kernel<64, true> : graph_kernel<64, false>), grid, block, 0,
                       stream, a, p);
  return hipGetLastError();
}

}  // namespace rpa

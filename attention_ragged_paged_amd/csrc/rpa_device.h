// Device-side building blocks shared by the gfx950 kernels of librpa.
//
// Nothing here is used by the CPU oracle; the GPU path and the oracle share no code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define RPA_LDS __attribute__((address_space(3)))

constexpr int kThreads = 256;        // every attention workgroup: 4 wave64s
constexpr int kDecodeRows = 16;      // query rows per decode work item (one 16x16 MFMA tile)
constexpr int kPrefillRows = 128;    // query rows per prefill work item (4 waves x 32)
constexpr int kPrefillKeys = 64;     // keys per prefill KV tile

// State of a graph-capturable call at the start of its workspace.  The queue, the exit count
// and the tag persist from call to call (zero in a fresh workspace); the other fields report
// the last call's plan.
struct GraphPlan {
  uint32_t status;                 // 0: valid batch; else bit flags of broken preconditions
  int32_t split_dec, split_pf;     // keys per KV split (multiples of 64)
  int32_t n_pf_items, n_items;     // prefill items come first in the item numbering
  uint32_t queue;                  // items handed out past the first one of each workgroup
  uint32_t exits;                  // workgroups of the running call that have left
  uint32_t pad;
  unsigned long long tag;          // number of calls made so far
};

// Everything the attention kernels need, passed by value as the kernel argument.
struct AttnArgs {
  const uint16_t *q;        // [T][Hq][D] bf16
  const uint16_t *k_cache;  // paged cache, see strides
  const uint16_t *v_cache;
  uint16_t *out;            // [T][Hq][D] bf16
  const uint16_t *k_new;    // [T][Hkv][D] bf16 or null: new tokens' K/V, written in this call
  const uint16_t *v_new;
  const int32_t *tables;
  const int32_t *cu_q_lens; // [B + 1]
  const int32_t *kv_lens;
  float *part_o;            // split partials: [max_nsplit][T][Hq][D] unnormalised outputs
  float *part_ml;           // [max_nsplit][T][Hq][2]: running max (log2 units) and sum
  unsigned long long *counters;  // arrival counters: decode row groups, then prefill ones
  unsigned long long call_tag;   // this call's tag in bits 24..63 (count in bits 0..23)
  int32_t B, T, Hq, Hkv, G;
  int32_t page_shift;       // log2(page size)
  int32_t num_pages;        // pages in each cache: table entries outside [0, num_pages) are bad
  int64_t page_stride, slot_stride, head_stride;  // cache element strides
  int32_t bt_seq_stride, bt_head_stride;          // table entry (b, g, i) = tables[b*seq + g*head + i]
  int32_t kvl_seq_stride, kvl_head_stride;        // kv_len(b, g) = kv_lens[b*seq + g*head]
  float scale_log2;         // softmax scale * log2(e) (* k_scale for an FP8 cache)
  float out_scale;          // multiplies every output: 1, or v_scale for an FP8 cache
  float k_inv, v_inv;       // FP8 cache: 1 / k_scale, 1 / v_scale (fp32), for new K/V
  int32_t kv8;              // caches of FP8 E4M3 codes (selects the kernels' FP8 variants)
  int32_t dec_rows_max;     // a sequence is decode-class iff q_len * G <= dec_rows_max
  int32_t split_dec;        // keys per split of a decode-class sequence (multiple of 64)
  int32_t split_pf;         // keys per split of a prefill-class sequence (multiple of 64)
  int32_t pf_tokens;        // tokens per prefill tile: kPrefillRows / G (at least 1)
  int32_t n_pf_items;       // mixed kernel: blocks [0, n_pf_items) are prefill items
  int32_t pf_counter_base;  // first prefill counter: decode ones are (q0*G + 16*rt)*Hkv + g
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Block-table entries are preconditions, not checked on the host: an entry outside
// [0, num_pages) is kept in a page window as page 0 with the sign bit set, so that readers
// stay inside the cache (the keys they read there are unspecified) and writers, which test
// the sign bit, never store through it.
constexpr int kBadPage = (int)0x80000000u;
__device__ __forceinline__ int checked_page(int entry, int num_pages) {
  return (unsigned)entry < (unsigned)num_pages ? entry : kBadPage;
}
__device__ __forceinline__ int read_page(int checked) { return checked & 0x7fffffff; }

// The thread index, read once per work item behind an empty asm: values derived from it are
// then computed per item instead of being hoisted out of a persistent kernel's item loop,
// where they would hold registers for the whole kernel.
__device__ __forceinline__ int item_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  __builtin_assume(t >= 0 && t < kThreads);
  return t;
}

__device__ __forceinline__ int kv_len_of(const AttnArgs &a, int b, int g) {
  return a.kv_lens[b * a.kvl_seq_stride + g * a.kvl_head_stride];
}

// Longest kv_len over the KV heads of sequence b (all equal in the sequence-major layout).
__device__ __forceinline__ int max_kv_len(const AttnArgs &a, int b) {
  int m = a.kv_lens[b * a.kvl_seq_stride];
  if (a.kvl_head_stride != 0)
    for (int g = 1; g < a.Hkv; ++g) m = max(m, a.kv_lens[b * a.kvl_seq_stride + g]);
  return m;
}

__device__ __forceinline__ bool is_decode_class(const AttnArgs &a, int q_len) {
  return q_len * a.G <= a.dec_rows_max;
}

__device__ __forceinline__ int ceil_div(int x, int y) { return (x + y - 1) / y; }

// Number of KV splits of a decode-class / prefill-class sequence b (same formulas on the host).
__device__ __forceinline__ int num_splits_dec(const AttnArgs &a, int b) {
  return max(1, ceil_div(max_kv_len(a, b), a.split_dec));
}

__device__ __forceinline__ int num_splits_pf(const AttnArgs &a, int b) {
  return max(1, ceil_div(max_kv_len(a, b), a.split_pf));
}

// Keys per split of a sequence cut into nsplit splits: the range is shared out evenly (in
// multiples of 64 keys), so no split is a short leftover that would trail the others.
__device__ __forceinline__ int even_split(int max_kv, int nsplit) {
  return ceil_div(ceil_div(max_kv, nsplit), 64) * 64;
}

struct ItemRef {
  int b;    // sequence, or -1 when the id is past the last item
  int rem;  // index of the item within its sequence
};

// Maps a work-item id onto (sequence, index within the sequence), where sequence b owns
// count(b) consecutive ids.  Every lane of the wave computes the same answer: lanes take
// 64 sequences at a time, a wave-wide inclusive scan gives the running offsets.
template <class CountFn>
__device__ __forceinline__ ItemRef find_item(int id, int B, CountFn count) {
  const int lane = lane_id();
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < B ? count(b) : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (id < base + total) {
      const unsigned long long hit = __ballot(base + incl > id);
      const int l = __ffsll((long long)hit) - 1;
      const int excl = __shfl(incl - c, l);
      return {b0 + l, id - base - excl};
    }
    base += total;
  }
  return {-1, 0};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte chunk c of row r of an LDS tile stored row-major with D bf16 per row, XOR-swizzled
// by a function of the row so that, for every read the kernels issue, each 256-byte LDS
// pass touches distinct banks:
//   - the same chunk of 16 consecutive rows (a ds_read_b128 operand column), and
//   - 4 consecutive rows (4-aligned) x 4 consecutive chunks (4-aligned) (a transposing read),
// while a row stays a permutation of itself (whole-row writes are conflict-free too).
// D = 128 (16 chunks, 256-byte rows): f(r) = 4 (r mod 4) + (r / 4) mod 4.
// D = 64 (8 chunks, two rows per bank period): the same idea on q = r / 2 within a parity.
template <int D>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    const int q = r >> 1;
    return c ^ (((q & 1) << 2) | ((q >> 1) & 3));
  }
}

template <int D>
__device__ __forceinline__ int lds_off(int r, int c) {  // offset in bf16 elements
  return r * D + swz_chunk<D>(r, c) * 8;
}

// FP8 E4M3 (the OCP format: bias 7, no infinities, largest finite 448) for quantized caches.
// A new value x is stored as the code of x * inv_scale, clamped to +-448 and rounded to
// nearest even (v_cvt_pk_fp8_f32); codes are read back exactly as bf16 code values
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3 value is a bf16 value), and the
// caches' scales are applied to the scores and to the output instead.
__device__ __forceinline__ float fp8_clamp(float x) { return fminf(fmaxf(x, -448.f), 448.f); }

// 8 bf16 values (u32x4) -> 8 codes (u32x2), element i in byte i.
__device__ __forceinline__ u32x2 quantize8(const u32x4 &v, float inv) {
  u32x2 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t w0 = v[2 * i], w1 = v[2 * i + 1];
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(bf16_lo(w0) * inv), fp8_clamp(bf16_hi(w0) * inv), 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(bf16_lo(w1) * inv), fp8_clamp(bf16_hi(w1) * inv), c, true);
    r[i] = (uint32_t)c;
  }
  return r;
}

// 16 bf16 values (lo: elements 0..7, hi: 8..15) -> 16 codes.
__device__ __forceinline__ u32x4 quantize16(const u32x4 &lo, const u32x4 &hi, float inv) {
  const u32x2 a = quantize8(lo, inv), b = quantize8(hi, inv);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// 16 codes -> 16 bf16 code values (lo: elements 0..7, hi: 8..15), exact.
__device__ __forceinline__ void dequant16(const u32x4 &c, u32x4 &lo, u32x4 &hi) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[i], 1.0f, false));
    w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[i], 1.0f, true));
  }
  lo = u32x4{w[0], w[1], w[2], w[3]};
  hi = u32x4{w[4], w[5], w[6], w[7]};
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// names 8 bytes holding row i/4, columns 4*(i%4) .. 4*(i%4)+3 of a 4 x 16 block of bf16;
// it receives column i, i.e. the 4 elements (row 0..3, column i).
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((RPA_LDS s16x4 *)(p));
}

// Direct global -> LDS load (gfx950 global_load_lds_dwordx4): lane l's 16 bytes land at
// lds_base + 16 l.  lds_base must be the same in every lane of the wave.
__device__ __forceinline__ void load_lds16(const uint16_t *src, uint16_t *lds_base) {
  __builtin_amdgcn_global_load_lds((const void *)src, (RPA_LDS void *)lds_base, 16, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x16(const s16x4 &a, const s16x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask));
}

// Max / sum over the lane pair (l, l ^ 32) with the gfx950 half swap (one VALU op, no LDS
// round trip): the swap of (v, v) returns v's low half in both halves of its first result
// and v's high half in both halves of its second.
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The same over the lane pair (l, l ^ 16), with the gfx950 row swap.
__device__ __forceinline__ float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace rpa

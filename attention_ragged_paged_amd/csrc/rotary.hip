// Rotary embedding of the new tokens' Q and K, fused with the K/V scatter.
//
// "[WebGPU] Optimized PagedAttention implementation (2/n)" (ONNX Runtime PR 31727) runs, when
// rotary is on, a rotary program over Q and over K (position = past + local token; dims from
// rotary_dim on copied; V not rotated; interleaved or split pairs) and then the scatter; with
// packed QKV a split pre-pass comes first (per token: Hq*D columns of Q, then Hkv*D of K, then
// Hkv*D of V).  Here all of it is one launch: Q, K and V are read in place through row strides
// (packed QKV is three strided views of one buffer), rotated in registers, Q written out and
// K/V stored straight into their page slots (quantized for an FP8 cache).  One thread handles 8
// consecutive dims of one (token, head); a split-pair rotation also reads the partner dims
// 8-aligned rotary_dim/2 away, which rotary_dim % 16 == 0 keeps in a single chunk.
#include "rpa_device.h"
#include "rpa_launch.h"

namespace rpa {

namespace {

__device__ __forceinline__ int seq_owning(const int32_t *cu_q_lens, int B, int token) {
  int lo = 0, hi = B - 1;  // largest b with cu_q_lens[b] <= token
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q_lens[mid] <= token)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void unpack8(const u32x4 &v, float *x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(v[i]);
    x[2 * i + 1] = bf16_hi(v[i]);
  }
}

// Rotates the 8 dims d0 .. d0+7 of one row: x holds them, xp the partner dims of a split pair
// (unused when interleaved).  Pair i of position pos uses cs[i], sn[i]; each output is
// fmaf(x1, c, -(x2 * s)) for the first element of a pair and fmaf(x2, c, x1 * s) for the
// second, rounded to bf16 (nearest even).
__device__ __forceinline__ u32x4 rotate8(const float *x, const float *xp, int d0, const RotaryArgs &r,
                                         const float *cs, const float *sn) {
#pragma clang fp contract(off)
  float y[8];
  const int half = r.rotary_dim / 2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    if (d >= r.rotary_dim) {
      y[e] = x[e];
      continue;
    }
    int i;
    bool first;
    float partner;
    if (r.interleaved) {
      i = d >> 1;
      first = (d & 1) == 0;
      partner = x[e ^ 1];
    } else {
      first = d < half;
      i = first ? d : d - half;
      partner = xp[e];
    }
    const float c = cs[i], s = sn[i];
    y[e] = first ? __builtin_fmaf(x[e], c, -(partner * s)) : __builtin_fmaf(x[e], c, partner * s);
  }
  return u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
               pack_bf16x2(y[6], y[7])};
}

}  // namespace

template <int D, bool KV8>
__global__ __launch_bounds__(256) void rotary_write_kernel(RotaryArgs r) {
  constexpr int kChunks = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int heads = r.Hq + r.Hkv;
  const int64_t row = gid / kChunks;  // token * (Hq + Hkv) + head
  const int c = (int)(gid % kChunks);
  if (row >= (int64_t)r.T * heads) return;
  const int token = (int)(row / heads);
  const int hh = (int)(row % heads);  // Q heads first, then KV heads
  const int b = seq_owning(r.cu_q_lens, r.B, token);
  const int q0 = r.cu_q_lens[b];
  const int q_len = r.cu_q_lens[b + 1] - q0;
  const int pos = r.kv_lens[b * r.kvl_seq_stride] - q_len + (token - q0);  // KV head 0's past
  const int d0 = 8 * c;
  const bool rotate = d0 < r.rotary_dim;
  // Dims of the pair partners (split pairs only): rotary_dim/2 away, in one 8-dim chunk.
  const int dp = d0 < r.rotary_dim / 2 ? d0 + r.rotary_dim / 2 : d0 - r.rotary_dim / 2;
  const float *cs = r.cos_cache + (int64_t)pos * (r.rotary_dim / 2);
  const float *sn = r.sin_cache + (int64_t)pos * (r.rotary_dim / 2);

  auto rotated = [&](const uint16_t *src) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + d0);
    if (!rotate) return v;
    float x[8], xp[8];
    unpack8(v, x);
    if (!r.interleaved) unpack8(*reinterpret_cast<const u32x4 *>(src + dp), xp);
    return rotate8(x, xp, d0, r, cs, sn);
  };

  if (hh < r.Hq) {
    const u32x4 y = rotated(r.q + (int64_t)token * r.q_stride + (int64_t)hh * D);
    *reinterpret_cast<u32x4 *>(r.q_out + ((int64_t)token * r.Hq + hh) * D + d0) = y;
    return;
  }
  const int g = hh - r.Hq;
  const u32x4 kv = rotated(r.k + (int64_t)token * r.kv_stride + (int64_t)g * D);
  const u32x4 vv = *reinterpret_cast<const u32x4 *>(r.v + (int64_t)token * r.kv_stride + (int64_t)g * D + d0);
  const int page = r.tables[b * r.bt_seq_stride + g * r.bt_head_stride + (pos >> r.page_shift)];
  if ((unsigned)page >= (unsigned)r.num_pages) return;  // a bad table entry is never stored through
  const int slot = pos & ((1 << r.page_shift) - 1);
  const int64_t dst = (int64_t)page * r.page_stride + (int64_t)slot * r.slot_stride +
                      (int64_t)g * r.head_stride + d0;
  if constexpr (KV8) {
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(r.k_cache) + dst) = quantize8(kv, r.k_inv);
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(r.v_cache) + dst) = quantize8(vv, r.v_inv);
  } else {
    *reinterpret_cast<u32x4 *>(r.k_cache + dst) = kv;
    *reinterpret_cast<u32x4 *>(r.v_cache + dst) = vv;
  }
}

hipError_t launch_rotary_write(const RotaryArgs &r, int D, hipStream_t stream) {
  const int64_t threads = (int64_t)r.T * (r.Hq + r.Hkv) * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (blocks == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL((r.kv8 ? rotary_write_kernel<128, true> : rotary_write_kernel<128, false>),
                       dim3(blocks), dim3(256), 0, stream, r);
  else
    hipLaunchKernelGGL((r.kv8 ? rotary_write_kernel<64, true> : rotary_write_kernel<64, false>),
                       dim3(blocks), dim3(256), 0, stream, r);
  return hipGetLastError();
}

}  // namespace rpa

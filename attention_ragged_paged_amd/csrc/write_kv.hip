// KV scatter: copies each new token's K and V rows into its page slot.
//
// Addressing follows the scatter program of ONNX Runtime PR 31727 ("[WebGPU] Optimized
// PagedAttention implementation (2/n)", Phase 1b.1 commit note): position = past + local
// token, page = block_table[position / page_size], slot = position % page_size.  Unlike
// that program (one invocation per element, linear scan for the sequence), one thread
// here moves a 16-byte chunk, so a wave moves whole 256-byte rows (D = 128) and every
// store is a full, aligned row segment; the sequence comes from a binary search.  An FP8
// cache stores each value as the E4M3 code of x / scale (see quantize8), 8 bytes a thread.
#include "rpa_device.h"
#include "rpa_launch.h"

namespace rpa {

// Largest b in [0, B) with cu_q_lens[b] <= token: the sequence owning the token (empty
// sequences share their start with the next one, and the last of equal starts owns it).
__device__ __forceinline__ int seq_of_token(const int32_t *cu_q_lens, int B, int token) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q_lens[mid] <= token)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <int D, bool KV8>
__global__ __launch_bounds__(256) void write_kv_kernel(WriteArgs a) {
  constexpr int kChunks = D / 8;  // 16-byte chunks per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / kChunks;  // token * Hkv + g
  const int c = (int)(gid % kChunks);
  if (row >= (int64_t)a.T * a.Hkv) return;
  const int token = (int)(row / a.Hkv);
  const int g = (int)(row % a.Hkv);
  const int b = seq_of_token(a.cu_q_lens, a.B, token);
  const int q0 = a.cu_q_lens[b];
  const int q_len = a.cu_q_lens[b + 1] - q0;
  const int kv_len = a.kv_lens[b * a.kvl_seq_stride + g * a.kvl_head_stride];
  const int pos = kv_len - q_len + (token - q0);
  const int page = a.tables[b * a.bt_seq_stride + g * a.bt_head_stride + (pos >> a.page_shift)];
  if ((unsigned)page >= (unsigned)a.num_pages) return;  // a bad table entry is never stored through
  const int slot = pos & ((1 << a.page_shift) - 1);
  const int64_t dst = (int64_t)page * a.page_stride + (int64_t)slot * a.slot_stride +
                      (int64_t)g * a.head_stride + c * 8;
  const int64_t src = row * D + c * 8;
  const u32x4 kv = *reinterpret_cast<const u32x4 *>(a.k_new + src);
  const u32x4 vv = *reinterpret_cast<const u32x4 *>(a.v_new + src);
  if constexpr (KV8) {
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(a.k_cache) + dst) = quantize8(kv, a.k_inv);
    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(a.v_cache) + dst) = quantize8(vv, a.v_inv);
  } else {
    *reinterpret_cast<u32x4 *>(a.k_cache + dst) = kv;
    *reinterpret_cast<u32x4 *>(a.v_cache + dst) = vv;
  }
}

hipError_t launch_write_kv(const WriteArgs &a, int D, hipStream_t stream) {
  const int64_t threads = (int64_t)a.T * a.Hkv * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (blocks == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL((a.kv8 ? write_kv_kernel<128, true> : write_kv_kernel<128, false>), dim3(blocks),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((a.kv8 ? write_kv_kernel<64, true> : write_kv_kernel<64, false>), dim3(blocks),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rpa

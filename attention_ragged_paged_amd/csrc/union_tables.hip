// Block-union KV selection: per-KV-head block tables of one chunk from a per-head 2D mask.
//
// "CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection" ("Core
// claim" and Figure 3): the union over query blocks turns each head's 2D mask into a KV
// block set, the union over the query heads of a GQA group gives one set per KV head, and
// the set becomes a block table over KV-head-major pages (Figure 4) that the paged
// attention kernel reads in place.  Here the chunk's own blocks are always kept and the set
// is listed in ascending block order, so the compacted sequence keeps the chunk's queries
// as its last positions and the ordinary causal mask stays exact.
//
// Pass 1 (select): one workgroup per (KV head, 256 x 16 KV blocks); each thread ORs 16-byte
//   mask rows over a slice of the group's (head, query block) rows, the slices are ORed in
//   LDS, and the 0/1 flags are written into out_tables (used as scratch).
// Pass 2 (compact): one workgroup per KV head; flags -> ascending list of physical pages
//   via a workgroup prefix sum, -1 padding, count and compacted kv_len.
#include "rpa_device.h"
#include "rpa_launch.h"

namespace rpa {

constexpr int kSelBlocksPerThread = 16;   // KV blocks per thread in pass 1 (one 16-byte load)
constexpr int kSelCols = 16;              // threads along the KV-block axis
constexpr int kSelRows = 256 / kSelCols;  // threads along the (head, query block) axis

__global__ __launch_bounds__(256) void union_select_kernel(UnionArgs a) {
  __shared__ uint32_t part[kSelRows][kSelCols][kSelBlocksPerThread / 4];
  const int g = blockIdx.y;
  const int col = threadIdx.x % kSelCols;
  const int rowt = threadIdx.x / kSelCols;
  const int kb0 = (blockIdx.x * kSelCols + col) * kSelBlocksPerThread;
  const int G = a.Hq / a.Hkv;
  const int n_rows = G * a.nQB;  // (head of the group, query block) rows
  const bool aligned = (a.nKB % 16) == 0;
  uint32_t acc[4] = {0u, 0u, 0u, 0u};
  if (kb0 < a.nKB) {
    for (int r = rowt; r < n_rows; r += kSelRows) {
      const int h = g * G + r / a.nQB;
      const int qb = r % a.nQB;
      const uint8_t *row = a.mask + ((int64_t)h * a.nQB + qb) * a.nKB;
      if (aligned) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(row + kb0);
        acc[0] |= v[0];
        acc[1] |= v[1];
        acc[2] |= v[2];
        acc[3] |= v[3];
      } else {
        for (int k = 0; k < kSelBlocksPerThread && kb0 + k < a.nKB; ++k)
          acc[k >> 2] |= (uint32_t)row[kb0 + k] << (8 * (k & 3));
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) part[rowt][col][q] = acc[q];
  __syncthreads();
  if (rowt != 0 || kb0 >= a.nKB) return;
  uint32_t o[4] = {0u, 0u, 0u, 0u};
  for (int r = 0; r < kSelRows; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] |= part[r][col][q];
  const int n_valid = (a.kv_len + a.page_size - 1) / a.page_size;
  const int first_chunk = a.past / a.page_size;
  const int last_chunk = (a.kv_len - 1) / a.page_size;
  for (int k = 0; k < kSelBlocksPerThread && kb0 + k < a.nKB; ++k) {
    const int kb = kb0 + k;
    const bool byte_set = ((o[k >> 2] >> (8 * (k & 3))) & 0xffu) != 0u;
    const bool sel = kb < n_valid && (byte_set || (kb >= first_chunk && kb <= last_chunk));
    a.out_tables[(int64_t)g * a.nKB + kb] = sel ? 1 : 0;
  }
}

__global__ __launch_bounds__(1024) void union_compact_kernel(UnionArgs a) {
  __shared__ uint8_t flags[kMaxUnionKvBlocks];
  __shared__ int wave_tot[16];
  const int g = blockIdx.x;
  int32_t *row = a.out_tables + (int64_t)g * a.nKB;
  const int32_t *base = a.base + (int64_t)g * a.nKB;
  const int per = (a.nKB + 1023) / 1024;  // consecutive blocks per thread
  const int k0 = threadIdx.x * per;
  // Copy this thread's flags to LDS before anything in the row is overwritten.
  int cnt = 0;
  for (int k = k0; k < min(k0 + per, a.nKB); ++k) {
    const uint8_t f = row[k] != 0;
    flags[k] = f;
    cnt += f;
  }
  // Workgroup exclusive prefix sum of cnt.
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();  // also: every flag of the row has been read
  int wave_base = 0, total = 0;
  for (int i = 0; i < 16; ++i) {
    if (i < wv) wave_base += wave_tot[i];
    total += wave_tot[i];
  }
  int pos = wave_base + incl - cnt;
  for (int k = k0; k < min(k0 + per, a.nKB); ++k)
    if (flags[k]) row[pos++] = base[k];
  for (int i = total + threadIdx.x; i < a.nKB; i += 1024) row[i] = -1;
  if (threadIdx.x == 0) {
    const int first_chunk = a.past / a.page_size;
    const int last_chunk = (a.kv_len - 1) / a.page_size;
    a.out_counts[g] = total;
    a.out_kv_lens[g] = (total - (last_chunk - first_chunk + 1)) * a.page_size +
                       (a.kv_len - first_chunk * a.page_size);
  }
}

hipError_t launch_union_tables(const UnionArgs &a, hipStream_t stream) {
  const int per_wg = kSelCols * kSelBlocksPerThread;
  const dim3 grid1((unsigned)((a.nKB + per_wg - 1) / per_wg), (unsigned)a.Hkv);
  hipLaunchKernelGGL(union_select_kernel, grid1, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(union_compact_kernel, dim3((unsigned)a.Hkv), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rpa

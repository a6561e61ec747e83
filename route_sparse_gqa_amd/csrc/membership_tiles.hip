// Membership table and 128x128 tile classes from compacted route lists.
//
// Definition: fa4_qsa page, `_preprocess` (uint8 membership [batch, queries,
// kv_length] with padded rows) and `_block_kinds` (int32
// [batch, ceil(queries/128), ceil(keys/block_keys)] classes: 0 absent,
// 1 partial, 2 full); flex_qsa page, `_membership_flat_offset` (table
// offsets must be 64-bit once B*S_q*kv_length passes 2^31).
//
// Design: one workgroup owns one 128-row tile row of one batch and one
// segment of up to 65536 columns.  For each of its rows it scatters the
// row's list into an LDS bitmap of the segment (atomic OR, integer only),
// expands the bitmap to bytes with 16-byte stores (every byte of the row,
// padding included, is written exactly once) and adds each 128-column
// tile's popcount to a register counter owned by the thread that handles
// that tile.  Counts are integers, so the classes are deterministic.
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kTile = 128;
constexpr int kSegCols = 65536;            // columns per workgroup segment
constexpr int kSegWords = kSegCols / 32;   // bitmap words
constexpr int kSegTiles = kSegCols / kTile;  // 512 tiles per segment
constexpr int kThreads = 256;
constexpr int kTilesPerThread = kSegTiles / kThreads;  // 2

// Four bits -> four bytes holding 0 or 1 (bit k lands in byte k).
__device__ __forceinline__ uint32_t spread4(uint32_t nibble) { return (nibble * 0x00204081u) & 0x01010101u; }

__global__ void __launch_bounds__(kThreads)
    membership_tiles_kernel(const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                            int64_t S_q, int64_t K, int64_t kv_length, int64_t ldm, int64_t n_ti,
                            int64_t n_tj, int64_t n_seg, uint8_t* __restrict__ membership,
                            int32_t* __restrict__ tile_class) {
  __shared__ uint32_t bits[kSegWords];
  const int t = threadIdx.x;
  int64_t blk = blockIdx.x;
  const int64_t seg = blk % n_seg;
  blk /= n_seg;
  const int64_t ti = blk % n_ti;
  const int64_t b = blk / n_ti;

  const int64_t c0 = seg * kSegCols;
  const int seg_cols = static_cast<int>(min(static_cast<int64_t>(kSegCols), ldm - c0));  // multiple of 128
  const int n_words = seg_cols / 32;
  const int n_chunks = seg_cols / 16;
  const int n_tiles = seg_cols / kTile;
  const int64_t r0 = ti * kTile;
  const int64_t r1 = min(r0 + kTile, S_q);

  int members[kTilesPerThread] = {};
  for (int64_t i = r0; i < r1; ++i) {
    const int64_t row = b * S_q + i;
    for (int w = t; w < n_words; w += kThreads) bits[w] = 0u;
    __syncthreads();
    const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
    const int32_t* lst = route_list + row * K;
    for (int j = t; j < n; j += kThreads) {
      const int64_t c = static_cast<int64_t>(lst[j]) - c0;
      if (c >= 0 && c < seg_cols) atomicOr(&bits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    if (membership != nullptr) {
      uint8_t* dst = membership + row * ldm + c0;  // 64-bit offset
      for (int ch = t; ch < n_chunks; ch += kThreads) {
        const uint32_t h = (bits[ch >> 1] >> ((ch & 1) * 16)) & 0xFFFFu;
        uint4 o;
        o.x = spread4(h & 0xFu);
        o.y = spread4((h >> 4) & 0xFu);
        o.z = spread4((h >> 8) & 0xFu);
        o.w = spread4(h >> 12);
        *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(ch) * 16) = o;
      }
    }
    if (tile_class != nullptr) {
#pragma unroll
      for (int u = 0; u < kTilesPerThread; ++u) {
        const int tj = t + u * kThreads;
        if (tj < n_tiles) {
          const uint32_t* w = bits + tj * 4;
          members[u] += __popc(w[0]) + __popc(w[1]) + __popc(w[2]) + __popc(w[3]);
        }
      }
    }
    __syncthreads();
  }

  if (tile_class != nullptr) {
#pragma unroll
    for (int u = 0; u < kTilesPerThread; ++u) {
      const int64_t tj = seg * kSegTiles + t + u * kThreads;
      if (t + u * kThreads < n_tiles && tj < n_tj) {
        const int64_t cols = min(static_cast<int64_t>(kTile), kv_length - tj * kTile);
        const int64_t pairs = (r1 - r0) * cols;
        const int cls = members[u] == 0 ? 0 : (members[u] == pairs ? 2 : 1);
        tile_class[(b * n_ti + ti) * n_tj + tj] = cls;
      }
    }
  }
}

}  // namespace

hipError_t launch_membership_tiles(const int32_t* route_list, const int32_t* route_count, int64_t B,
                                   int64_t S_q, int64_t K, int64_t kv_length, uint8_t* membership,
                                   int32_t* tile_class, hipStream_t stream) {
  if (membership == nullptr && tile_class == nullptr) return hipSuccess;
  const int64_t ldm = (kv_length + kTile - 1) / kTile * kTile;
  const int64_t n_ti = (S_q + kTile - 1) / kTile;
  const int64_t n_tj = (kv_length + kTile - 1) / kTile;
  const int64_t n_seg = (ldm + kSegCols - 1) / kSegCols;
  const int64_t blocks = B * n_ti * n_seg;
  hipLaunchKernelGGL(membership_tiles_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream,
                     route_list, route_count, S_q, K, kv_length, ldm, n_ti, n_tj, n_seg, membership,
                     tile_class);
  return hipGetLastError();
}

}  // namespace qsa

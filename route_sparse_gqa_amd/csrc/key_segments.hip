// Key segments: the compacted route lists regrouped by 16-key tile, for the
// key-side backward kernel.
//
// The backward's dk and dv sums run over every query row that routes a key
// (fa4_qsa page: first-order autograd of the routed attention).  A segment
// is one (query row, 16-key tile) pair in which the row routes at least one
// key of the tile; it is stored as {row, mask}, bit c of the mask set iff the
// row routes key 16 * tile + c.  The segments of a (batch, tile) are
// contiguous and in ascending row order, so the key-side sums have a fixed
// order and the backward is deterministic.
//
// Construction is a stable counting sort of the segments by tile, over
// blocks of 64 query rows (one wavefront per block walks its rows in
// order):
//   1. zero the per-(batch, row block, tile) counters;
//   2. count each block's segments per tile (a segment is found at its last
//      list entry: the next entry lies in another tile or the list ends);
//   3. per (batch, tile), an exclusive scan of the counters over row blocks,
//      in place, and the tile's total;
//   4. an exclusive scan of the totals over (batch, tile): segment start of
//      each tile, plus the grand total at the end;
//   5. each block walks its rows again in order and places every segment at
//      start + an atomic increment of its (block, tile) counter; rows are
//      visited one after the other by one wavefront and a row's segments lie
//      in distinct tiles, so the order within a tile is the row order.
// Lists are read as qsa_preprocess writes them; IDs are clamped into range
// and positions checked against the capacity, so malformed lists cannot
// fault.
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kKeyTile = static_cast<int>(kSegKeyTile);
constexpr int kRowBlock = static_cast<int>(kSegRowBlock);
constexpr int kWaves = 4;
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(256) zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * 256)
    p[idx] = 0;
}

// One wavefront walks the rows of one (batch, row block) in order and, at
// each segment's last list entry, counts the segment (kFill false) or places
// it (kFill true).
template <bool kFill>
__global__ void __launch_bounds__(64 * kWaves)
    segment_walk_kernel(const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                        int64_t S_q, int64_t K, int64_t S_kv, int64_t n_rb, int64_t n_kt, int64_t n_blocks,
                        int32_t* __restrict__ counters, const int32_t* __restrict__ tile_start,
                        int2* __restrict__ segs, int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (unit >= n_blocks) return;
  const int64_t b = unit / n_rb;
  const int64_t rb = unit % n_rb;
  int32_t* cnt = counters + unit * n_kt;  // this block's counters, [n_kt]
  const int32_t id_max = static_cast<int32_t>(S_kv - 1);
  const int64_t i_end = min(rb * kRowBlock + kRowBlock, S_q);
  for (int64_t i = rb * kRowBlock; i < i_end; ++i) {
    const int64_t row = b * S_q + i;
    const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
    const int32_t* lst = route_list + row * K;
    for (int j = lane; j < n; j += 64) {
      const int32_t id = min(max(lst[j], 0), id_max);
      const int32_t tile = id / kKeyTile;
      const bool last = j + 1 >= n || min(max(lst[j + 1], 0), id_max) / kKeyTile != tile;
      if (!last) continue;
      if (!kFill) {
        atomicAdd(&cnt[tile], 1);
      } else {
        // Keys of this segment: the entries back from j that share its tile
        // (at most 16 in an ascending list).
        uint32_t mask = 0;
        for (int e = 0; e < kKeyTile && j - e >= 0; ++e) {
          const int32_t idd = min(max(lst[j - e], 0), id_max);
          if (idd / kKeyTile != tile) break;
          mask |= 1u << (idd % kKeyTile);
        }
        const int64_t pos = static_cast<int64_t>(tile_start[b * n_kt + tile]) + atomicAdd(&cnt[tile], 1);
        if (pos < capacity) segs[pos] = int2{static_cast<int32_t>(i), static_cast<int32_t>(mask)};
      }
    }
  }
}

// Per (batch, tile): exclusive scan of the block counters over row blocks,
// in place; the tile's total goes to totals.
__global__ void __launch_bounds__(256)
    column_scan_kernel(int32_t* __restrict__ counters, int64_t B, int64_t n_rb, int64_t n_kt,
                       int32_t* __restrict__ totals) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= B * n_kt) return;
  const int64_t b = idx / n_kt, t = idx % n_kt;
  int32_t run = 0;
  for (int64_t rb = 0; rb < n_rb; ++rb) {
    int32_t* p = counters + (b * n_rb + rb) * n_kt + t;
    const int32_t c = *p;
    *p = run;
    run += c;
  }
  totals[idx] = run;
}

// Exclusive scan of n totals into start[0 .. n] (start[n] = grand total);
// one workgroup walks the array in chunks of 1024.
__global__ void __launch_bounds__(kScanThreads)
    tile_scan_kernel(const int32_t* __restrict__ totals, int64_t n, int32_t* __restrict__ start) {
  __shared__ int32_t wave_sum[kScanThreads / 64];
  __shared__ int32_t carry_s;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t idx = base + threadIdx.x;
    const int32_t val = idx < n ? totals[idx] : 0;
    int32_t incl = val;  // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int32_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wave_sum[w];
    if (idx < n) start[idx] = before + incl - val;
    __syncthreads();  // every thread has read carry_s and wave_sum
    if (threadIdx.x == kScanThreads - 1) carry_s = before + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) start[n] = carry_s;
}

}  // namespace

hipError_t launch_key_segments(const int32_t* route_list, const int32_t* route_count, int64_t B, int64_t S_q,
                               int64_t K, int64_t S_kv, const SegmentBuffers& w, hipStream_t stream) {
  const int64_t n_rb = (S_q + kRowBlock - 1) / kRowBlock;
  const int64_t n_kt = (S_kv + kKeyTile - 1) / kKeyTile;
  const int64_t n_blocks = B * n_rb;
  const int64_t n_counters = n_blocks * n_kt;
  const int64_t zero_blocks = min((n_counters + 255) / 256, int64_t{65536});
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<uint32_t>(zero_blocks)), dim3(256), 0, stream, w.counters,
                     n_counters);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t walk_blocks = static_cast<uint32_t>((n_blocks + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((segment_walk_kernel<false>), dim3(walk_blocks), dim3(64 * kWaves), 0, stream, route_list,
                     route_count, S_q, K, S_kv, n_rb, n_kt, n_blocks, w.counters, nullptr, nullptr, int64_t{0});
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(column_scan_kernel, dim3(static_cast<uint32_t>((B * n_kt + 255) / 256)), dim3(256), 0, stream,
                     w.counters, B, n_rb, n_kt, w.totals);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tile_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, w.totals, B * n_kt, w.tile_start);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((segment_walk_kernel<true>), dim3(walk_blocks), dim3(64 * kWaves), 0, stream, route_list,
                     route_count, S_q, K, S_kv, n_rb, n_kt, n_blocks, w.counters, w.tile_start, w.segs, w.capacity);
  return hipGetLastError();
}

}  // namespace qsa

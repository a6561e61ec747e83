// Key segments: the compacted route lists regrouped by 64-key tile, for the
// key-side backward kernel, and the split of each tile's segments into
// bounded parts.
//
// The backward's dk and dv sums run over every query row that routes a key
// (fa4_qsa page: first-order autograd of the routed attention).  A segment
// is one (query row, 64-key tile) pair in which the row routes at least one
// key of the tile; it is stored as {row, mask lo, mask hi, 0}, bit c of the
// 64-bit mask set iff the row routes key 64 * tile + c.  The segments of a (batch, tile) are
// contiguous and in ascending row order, so the key-side sums have a fixed
// order and the backward is deterministic.
//
// Construction (every step parallel over rows or tiles, no order-dependent
// atomics):
//   1. clear a bit matrix with one bit per (query row, tile), stored as
//      words [batch][row / 32][tile] (tiles fastest, so per-tile scans read
//      consecutive words);
//   2. one wavefront per row sets the bit of every tile its list touches
//      (integer atomic OR: the result does not depend on the order);
//   3. per (batch, chunk of 256 rows, tile): popcount of the chunk's 8 words;
//   4. per (batch, tile): exclusive scan of those counts over the chunks, and
//      the tile's total;
//   5. exclusive scan of the totals over (batch, tile): each tile's first
//      segment, the grand total at the end;
//   6. one wavefront per row places each of its segments at
//      tile start + chunk prefix + popcounts of the earlier rows of its chunk,
//      i.e. at its rank among the rows that touch the tile; the key mask of a
//      run of list entries in one tile is a segmented OR-scan across the
//      wavefront's lanes, carried from one 64-entry chunk to the next;
//   7. parts: each tile's segment list is cut into parts of at most L
//      segments, L = max(64, ceil(total / max_parts)), so that no wavefront
//      of the key-side kernel carries a popular tile alone; tiles cut into
//      more than one part get consecutive partial-sum slots.
// Lists are read as qsa_preprocess writes them; IDs are clamped into range,
// so malformed lists cannot fault (a row counts each tile at most once, so
// positions stay below the grand total, which the capacity bounds).
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kKeyTile = static_cast<int>(kSegKeyTile);
constexpr int kChunkWords = static_cast<int>(kSegChunkRows / 32);
constexpr int kWaves = 4;
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(256) zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < n;
       idx += static_cast<int64_t>(gridDim.x) * 256)
    p[idx] = 0u;
}

__device__ __forceinline__ uint64_t shfl_up64(uint64_t x, int d) {
  const uint32_t lo = __shfl_up(static_cast<uint32_t>(x), d);
  const uint32_t hi = __shfl_up(static_cast<uint32_t>(x >> 32), d);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t x, int src) {
  const uint32_t lo = __shfl(static_cast<uint32_t>(x), src);
  const uint32_t hi = __shfl(static_cast<uint32_t>(x >> 32), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One wavefront per query row.  At the last list entry of each tile run it
// marks the (row, tile) bit (kFill false) or writes the segment at its rank
// (kFill true).  The list is read 64 entries at a time, the next chunk's
// entries (and the entry after it, which decides whether lane 63 ends a
// run) in flight while the current chunk is processed; the entry after each
// lane's own comes from its neighbour lane.  The rank's loads (tile start,
// chunk prefix and the words of the row's chunk) are issued together.
template <bool kFill>
__global__ void __launch_bounds__(64 * kWaves)
    row_segments_kernel(const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                        int64_t S_q, int64_t K, int64_t S_kv, int64_t n_kt, int64_t W, int64_t C, int64_t rows,
                        uint32_t* __restrict__ bits, const int32_t* __restrict__ chunk_prefix,
                        const int32_t* __restrict__ tile_start, int4* __restrict__ segs, int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t b = row / S_q;
  const int64_t i = row % S_q;
  const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
  const int32_t* lst = route_list + row * K;
  const int32_t id_max = static_cast<int32_t>(S_kv - 1);
  const int64_t w = i / 32;
  const uint32_t bit = 1u << (i % 32);
  uint32_t* words = bits + b * W * n_kt;  // word (w', t) at words[w' * n_kt + t]
  int32_t carry_tile = -1;                // tile of the run still open at the end of the previous chunk
  uint64_t carry_mask = 0;
  int32_t raw = n > 0 ? lst[min(lane, n - 1)] : 0;  // this lane's entry of the current chunk
  int32_t raw_after = n > 0 ? lst[min(64, n - 1)] : 0;  // the entry after the current chunk
  for (int base = 0; base < n; base += 64) {
    const int j = base + lane;
    const bool valid = j < n;
    const int32_t id = valid ? min(max(raw, 0), id_max) : 0;
    const int32_t tile = valid ? id / kKeyTile : -2 - lane;  // lanes past the list never join a run
    const int32_t after = min(max(raw_after, 0), id_max) / kKeyTile;
    // the next chunk's entries, in flight while this chunk is processed (read
    // unconditionally from in-range positions, values past the list unused:
    // a load under a branch would be waited for where the branch joins)
    const int nb = base + 64;
    const int32_t raw_n = lst[min(nb + lane, n - 1)];
    const int32_t raw_after_n = lst[min(nb + 64, n - 1)];
    int32_t next = __shfl_down(tile, 1);  // the tile of entry j + 1 (lane 63: the entry after the chunk)
    if (lane == 63) next = after;
    if (j + 1 >= n) next = -1;
    const bool last = valid && next != tile;
    if constexpr (!kFill) {
      if (last) atomicOr(&words[w * n_kt + tile], bit);
    } else {
      // Keys of each run: inclusive OR over the lanes of the same tile (a run
      // is contiguous in an ascending list, so equal tiles d lanes apart bound
      // a run), plus the part of the run carried from the previous chunk.
      uint64_t m = valid ? uint64_t{1} << (id % kKeyTile) : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint64_t y = shfl_up64(m, d);
        const int32_t ty = __shfl_up(tile, d);
        if (lane >= d && ty == tile) m |= y;
      }
      if (tile == carry_tile) m |= carry_mask;
      carry_tile = __shfl(tile, 63);
      carry_mask = shfl64(m, 63);
      if (last) {
        // Rank among the rows touching this tile: rows of earlier chunks, then
        // earlier words of this chunk, then earlier rows of this word.
        const int64_t c = w / kChunkWords;
        const int64_t w0 = c * kChunkWords;
        const int32_t start = tile_start[b * n_kt + tile];
        const int32_t prefix = chunk_prefix[(b * C + c) * n_kt + tile];
        uint32_t wd[kChunkWords];
#pragma unroll
        for (int k = 0; k < kChunkWords; ++k) wd[k] = w0 + k <= w ? words[(w0 + k) * n_kt + tile] : 0u;
        int64_t pos = static_cast<int64_t>(start) + prefix;
#pragma unroll
        for (int k = 0; k < kChunkWords; ++k)
          pos += __popc(w0 + k < w ? wd[k] : (w0 + k == w ? wd[k] & (bit - 1u) : 0u));
        if (pos < capacity)
          segs[pos] = int4{static_cast<int32_t>(i), static_cast<int32_t>(static_cast<uint32_t>(m)),
                           static_cast<int32_t>(static_cast<uint32_t>(m >> 32)), 0};
      }
    }
    raw = raw_n;
    raw_after = raw_after_n;
  }
}

// Per (batch, chunk, tile): number of rows of the chunk that touch the tile.
__global__ void __launch_bounds__(256)
    chunk_count_kernel(const uint32_t* __restrict__ bits, int64_t B, int64_t W, int64_t C, int64_t n_kt,
                       int32_t* __restrict__ chunk_prefix) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= B * C * n_kt) return;
  const int64_t t = idx % n_kt;
  const int64_t c = (idx / n_kt) % C;
  const int64_t b = idx / (n_kt * C);
  int32_t s = 0;
  const int64_t w_end = min((c + 1) * kChunkWords, W);
  for (int64_t w = c * kChunkWords; w < w_end; ++w) s += __popc(bits[(b * W + w) * n_kt + t]);
  chunk_prefix[idx] = s;
}

// Per (batch, tile): exclusive scan of the chunk counts over the chunks, in
// place; the tile's total goes to totals.
__global__ void __launch_bounds__(256)
    chunk_scan_kernel(int32_t* __restrict__ chunk_prefix, int64_t B, int64_t C, int64_t n_kt,
                      int32_t* __restrict__ totals) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= B * n_kt) return;
  const int64_t b = idx / n_kt, t = idx % n_kt;
  int32_t* col = chunk_prefix + b * C * n_kt + t;  // chunk c at col[c * n_kt]
  constexpr int kBatch = 16;  // counts loaded together (from clamped in-range chunks), then scanned in order
  int32_t run = 0;
  for (int64_t c0 = 0; c0 < C; c0 += kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) v[k] = col[min(c0 + k, C - 1) * n_kt];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (c0 + k < C) {
        col[(c0 + k) * n_kt] = run;
        run += v[k];
      }
    }
  }
  totals[idx] = run;
}

// Exclusive scan of one value per thread over a 1024-thread workgroup;
// returns the exclusive prefix and sets *total to the sum of all values.
__device__ int32_t block_exclusive_scan(int32_t val, int32_t* wave_sum, int32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int32_t incl = val;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int32_t before = 0, all = 0;
  for (int x = 0; x < kScanThreads / 64; ++x) {
    if (x < wave) before += wave_sum[x];
    all += wave_sum[x];
  }
  __syncthreads();  // wave_sum may be reused by the next call
  *total = all;
  return before + incl - val;
}

// Exclusive scan of the n tile totals into start[0 .. n] (start[n] = grand
// total), one workgroup walking the array in chunks of 1024.
__global__ void __launch_bounds__(kScanThreads)
    tile_scan_kernel(const int32_t* __restrict__ totals, int64_t n, int32_t* __restrict__ start) {
  __shared__ int32_t wave_sum[kScanThreads / 64];
  int32_t carry = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t idx = base + threadIdx.x;
    int32_t all;
    const int32_t ex = block_exclusive_scan(idx < n ? totals[idx] : 0, wave_sum, &all);
    if (idx < n) start[idx] = carry + ex;
    carry += all;
  }
  if (threadIdx.x == 0) start[n] = carry;
}

// Parts of at most L segments per tile (an empty tile is one part, so that
// its zero gradients are written); part_start[0 .. n] and, for tiles cut into
// more than one part, slot_start (first partial-sum slot).  plan = {L, parts}.
__global__ void __launch_bounds__(kScanThreads)
    part_plan_kernel(const int32_t* __restrict__ tile_start, int64_t n, int64_t max_parts, int32_t min_part,
                     int32_t* __restrict__ part_start, int32_t* __restrict__ slot_start, int32_t* __restrict__ plan) {
  __shared__ int32_t wave_sum[kScanThreads / 64];
  const int64_t total = tile_start[n];
  const int64_t L64 = max(static_cast<int64_t>(min_part), (total + max_parts - 1) / max_parts);
  const int32_t L = static_cast<int32_t>(L64);
  int32_t carry_p = 0, carry_s = 0;
  for (int64_t base = 0; base < n; base += kScanThreads) {
    const int64_t idx = base + threadIdx.x;
    int32_t parts = 0;
    if (idx < n) {
      const int32_t cnt = tile_start[idx + 1] - tile_start[idx];
      parts = cnt <= L ? 1 : (cnt + L - 1) / L;
    }
    int32_t all_p, all_s;
    const int32_t ex_p = block_exclusive_scan(parts, wave_sum, &all_p);
    const int32_t ex_s = block_exclusive_scan(parts > 1 ? parts : 0, wave_sum, &all_s);
    if (idx < n) {
      part_start[idx] = carry_p + ex_p;
      slot_start[idx] = carry_s + ex_s;
    }
    carry_p += all_p;
    carry_s += all_s;
  }
  if (threadIdx.x == 0) {
    part_start[n] = carry_p;
    plan[0] = L;
    plan[1] = carry_p;
  }
}

}  // namespace

hipError_t launch_key_segments(const int32_t* route_list, const int32_t* route_count, int64_t B, int64_t S_q,
                               int64_t K, int64_t S_kv, const SegmentBuffers& w, hipStream_t stream) {
  const int64_t n_kt = (S_kv + kKeyTile - 1) / kKeyTile;
  const int64_t W = (S_q + 31) / 32;
  const int64_t C = (W + kChunkWords - 1) / kChunkWords;
  const int64_t rows = B * S_q;
  const int64_t n_words = B * W * n_kt;
  const int64_t zero_blocks = min((n_words + 255) / 256, int64_t{65536});
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<uint32_t>(zero_blocks)), dim3(256), 0, stream, w.bits, n_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t row_blocks = static_cast<uint32_t>((rows + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((row_segments_kernel<false>), dim3(row_blocks), dim3(64 * kWaves), 0, stream, route_list,
                     route_count, S_q, K, S_kv, n_kt, W, C, rows, w.bits, nullptr, nullptr, nullptr, int64_t{0});
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_count_kernel, dim3(static_cast<uint32_t>((B * C * n_kt + 255) / 256)), dim3(256), 0,
                     stream, w.bits, B, W, C, n_kt, w.chunk_prefix);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_scan_kernel, dim3(static_cast<uint32_t>((B * n_kt + 255) / 256)), dim3(256), 0, stream,
                     w.chunk_prefix, B, C, n_kt, w.totals);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tile_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, w.totals, B * n_kt, w.tile_start);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((row_segments_kernel<true>), dim3(row_blocks), dim3(64 * kWaves), 0, stream, route_list,
                     route_count, S_q, K, S_kv, n_kt, W, C, rows, w.bits, w.chunk_prefix, w.tile_start, w.segs,
                     w.capacity);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(part_plan_kernel, dim3(1), dim3(kScanThreads), 0, stream, w.tile_start, B * n_kt, w.max_parts,
                     static_cast<int32_t>(kSegMinPart), w.part_start, w.slot_start, w.plan);
  return hipGetLastError();
}

}  // namespace qsa

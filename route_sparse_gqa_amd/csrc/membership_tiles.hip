// Membership table and 128x128 tile classes from compacted route lists.
//
// Definition: fa4_qsa page, `_preprocess` (uint8 membership [batch, queries,
// kv_length] with padded rows) and `_block_kinds` (int32
// [batch, ceil(queries/128), ceil(keys/block_keys)] classes: 0 absent,
// 1 partial, 2 full); flex_qsa page, `_membership_flat_offset` (table
// offsets must be 64-bit once B*S_q*kv_length passes 2^31).
//
// Design: one workgroup owns 4 rows of one 128-row tile row of one batch and
// one segment of up to 65536 columns; each of its four wavefronts owns one
// row with a private LDS bitmap of the segment (LDS sized to the segment).  Per row the wave
// scatters the row's list into the bitmap (atomic OR, integer only; the
// list passes through a small LDS buffer so that each lane takes consecutive
// entries of the sorted list and merges those in one word in registers, one
// atomic per run), expands
// it to bytes with 16-byte stores (every byte of the row, padding included,
// is written exactly once) and adds each 128-column tile's popcount to a
// register counter of the lane that owns the tile.  The workgroup sums its
// waves' counters in LDS and adds them to the tile's member count with one
// integer atomic per tile (the count buffer is the tile_class output, zeroed
// beforehand); a final pass turns counts into classes.  Integer sums make
// the classes deterministic.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kTile = 128;
constexpr int kSegCols = static_cast<int>(kMemSegCols);  // columns per workgroup segment
constexpr int kSegTiles = kSegCols / kTile;  // 512 tiles per segment
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupRows = kWaves;               // rows per workgroup: one per wavefront
constexpr int kGroups = kTile / kGroupRows;      // workgroups per tile row and segment
static_assert(kGroups == kMemGroups, "the host's grid-size check uses kMemGroups");
constexpr int kTilesPerLane = kSegTiles / 64;  // 8

constexpr int kBatch = 16;  // list entries per lane loaded together
constexpr int kStage = 4;   // entries per lane per pass through the wave's LDS staging buffer

// Four bits -> four bytes holding 0 or 1 (bit k lands in byte k).
__device__ __forceinline__ uint32_t spread4(uint32_t nibble) { return (nibble * 0x00204081u) & 0x01010101u; }

__global__ void __launch_bounds__(kThreads)
    membership_tiles_kernel(const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                            int64_t S_q, int64_t K, int64_t ldm, int64_t n_ti, int64_t n_tj, int64_t n_seg,
                            uint8_t* __restrict__ membership, int32_t* __restrict__ tile_count) {
  // Per-wave bitmaps of the segment, its tile counters, then per-wave staging buffers (sized at launch).
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  int64_t blk = blockIdx.x;
  const int grp = static_cast<int>(blk % kGroups);
  blk /= kGroups;
  const int64_t seg = blk % n_seg;
  blk /= n_seg;
  const int64_t ti = blk % n_ti;
  const int64_t b = blk / n_ti;

  const int64_t c0 = seg * kSegCols;
  const int seg_cols = static_cast<int>(min(static_cast<int64_t>(kSegCols), ldm - c0));  // multiple of 128
  const int seg_words = seg_cols / 32;
  const int n_chunks = seg_cols / 16;
  const int n_tiles = seg_cols / kTile;
  uint32_t* bits = lds + wave * seg_words;
  int* tile_sum = reinterpret_cast<int*>(lds + kWaves * seg_words);
  // 16-byte aligned: seg_words is a multiple of 4 and the counters take a multiple of 4 words
  int32_t* stage = reinterpret_cast<int32_t*>(lds + kWaves * seg_words + (n_tiles + 3) / 4 * 4) + wave * 64 * kStage;
  const int64_t r0 = ti * kTile + grp * kGroupRows;
  const int64_t r1 = min(r0 + kGroupRows, min(ti * kTile + kTile, S_q));

  if (tile_count != nullptr) {
    for (int t = threadIdx.x; t < n_tiles; t += kThreads) tile_sum[t] = 0;
  }

  int members[kTilesPerLane] = {};
  for (int64_t i = r0 + wave; i < r1; i += kWaves) {
    const int64_t row = b * S_q + i;
    const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
    for (int w = lane; w < seg_words; w += 64) bits[w] = 0u;
    wave_lds_sync();
    const int32_t* lst = route_list + row * K;
    // Batches of kBatch IDs per lane: a batch's loads are all in flight before any is used.
    for (int j0 = 0; j0 < n; j0 += 64 * kBatch) {  // wave-uniform
      int32_t id[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + 64 * u + lane;
        id[u] = j < n ? lst[j] : -1;
      }
      // In passes of 64 * kStage entries through LDS, so that each lane takes kStage consecutive
      // (ascending) entries and merges those in one bitmap word before its atomic.
#pragma unroll
      for (int r = 0; r < kBatch / kStage; ++r) {
        if (j0 + 64 * kStage * r >= n) continue;  // wave-uniform
#pragma unroll
        for (int t = 0; t < kStage; ++t) {
          const int u = kStage * r + t;
          const int64_t col = static_cast<int64_t>(id[u]) - c0;
          const bool ok = id[u] >= 0 && col >= 0 && col < seg_cols;
          stage[t * 64 + lane] = ok ? static_cast<int32_t>(col) : -1;
        }
        wave_lds_sync();
        or_slot_run<kStage>(bits, stage + lane * kStage);
        wave_lds_sync();  // the buffer is rewritten by the next pass
      }
    }
    wave_lds_sync();
    if (membership != nullptr) {
      uint8_t* dst = membership + row * ldm + c0;  // 64-bit offset
      for (int ch = lane; ch < n_chunks; ch += 64) {
        const uint32_t h = (bits[ch >> 1] >> ((ch & 1) * 16)) & 0xFFFFu;
        u32x4 o;
        o.x = spread4(h & 0xFu);
        o.y = spread4((h >> 4) & 0xFu);
        o.z = spread4((h >> 8) & 0xFu);
        o.w = spread4(h >> 12);
        *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(ch) * 16) = o;
      }
    }
    if (tile_count != nullptr) {
#pragma unroll
      for (int u = 0; u < kTilesPerLane; ++u) {
        const int tj = lane + 64 * u;
        if (tj < n_tiles) {
          const uint32_t* w = bits + 4 * tj;
          members[u] += __popc(w[0]) + __popc(w[1]) + __popc(w[2]) + __popc(w[3]);
        }
      }
    }
    wave_lds_sync();  // this row's bitmap reads are done before the next clear
  }

  if (tile_count != nullptr) {
    __syncthreads();  // counters zeroed by every thread before any wave adds
#pragma unroll
    for (int u = 0; u < kTilesPerLane; ++u) {
      const int tj = lane + 64 * u;
      if (tj < n_tiles && members[u] != 0) atomicAdd(&tile_sum[tj], members[u]);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < n_tiles; t += kThreads) {
      const int64_t tj = seg * kSegTiles + t;
      if (tj < n_tj && tile_sum[t] != 0) atomicAdd(&tile_count[(b * n_ti + ti) * n_tj + tj], tile_sum[t]);
    }
  }
}

// Member counts -> classes: 0 none, 2 every in-range pair, 1 otherwise.
__global__ void __launch_bounds__(256)
    tile_class_kernel(int32_t* __restrict__ tile, int64_t n_tiles, int64_t S_q, int64_t kv_length, int64_t n_ti,
                      int64_t n_tj) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= n_tiles) return;
  const int64_t tj = idx % n_tj;
  const int64_t ti = (idx / n_tj) % n_ti;
  const int64_t pairs = min(static_cast<int64_t>(kTile), S_q - ti * kTile) *
                        min(static_cast<int64_t>(kTile), kv_length - tj * kTile);
  const int32_t m = tile[idx];
  tile[idx] = m == 0 ? 0 : (m == pairs ? 2 : 1);
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
  const int64_t blocks = B * n_ti * n_seg * kGroups;
  // tile_class holds member counts until the final pass; the route-normalise
  // launch that precedes this one on the stream has zeroed it.
  const int64_t seg_cols = ldm < kSegCols ? ldm : kSegCols;
  const int64_t counter_words = (seg_cols / kTile + 3) / 4 * 4;  // tile counters, padded to 16 bytes
  const size_t lds_bytes =
      sizeof(uint32_t) * static_cast<size_t>(kWaves * (seg_cols / 32) + counter_words + kWaves * 64 * kStage);
  hipLaunchKernelGGL(membership_tiles_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), lds_bytes, stream,
                     route_list, route_count, S_q, K, ldm, n_ti, n_tj, n_seg, membership, tile_class);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tile_class == nullptr) return e;
  const int64_t n_tiles = B * n_ti * n_tj;
  hipLaunchKernelGGL(tile_class_kernel, dim3(static_cast<uint32_t>((n_tiles + 255) / 256)), dim3(256), 0, stream,
                     tile_class, n_tiles, S_q, kv_length, n_ti, n_tj);
  return hipGetLastError();
}

}  // namespace qsa

// Forward and reverse block lists of a tile-class table.
//
// Definition: fa4_qsa page, `_compact_blocks` (partial and full block
// columns of each block row, int32 counts [batch, 1, block_rows]) and
// `_preprocess` (forward and reverse block lists).  For each line (a block
// row for the forward lists, a block column for the reverse ones) and each
// kind (1 partial, 2 full): the count of tiles of that kind, and an index
// row holding their positions in ascending order followed by every other
// position in ascending order (the stable descending argsort of the class
// indicator, the ordering FlexAttention's BlockMask uses; only the first
// count entries are meaningful).
//
// Design: one wavefront per line.  A first pass counts the line's tiles of
// the kind with one ballot per 64 positions; a second pass places each
// position: listed ones at (listed so far + their rank within the ballot),
// the others after the count.  Forward lines read a contiguous row;
// reverse lines read a column (strided, the table is small).
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ uint32_t rank_below(uint64_t ballot, int lane) {
  return static_cast<uint32_t>(__popcll(ballot & ((uint64_t{1} << lane) - 1)));
}

__device__ void compact_line(const int32_t* __restrict__ line, int64_t n, int64_t stride, int32_t want,
                             int32_t* __restrict__ count, int32_t* __restrict__ idx, int lane) {
  int64_t total = 0;
  for (int64_t base = 0; base < n; base += 64) {
    const int64_t x = base + lane;
    const bool hit = x < n && line[x * stride] == want;
    total += __popcll(__ballot(hit));
  }
  if (count != nullptr && lane == 0) *count = static_cast<int32_t>(total);
  if (idx == nullptr) return;
  int64_t listed = 0, others = 0;
  for (int64_t base = 0; base < n; base += 64) {
    const int64_t x = base + lane;
    const bool in = x < n;
    const bool hit = in && line[x * stride] == want;
    const uint64_t bh = __ballot(hit);
    const uint64_t bo = __ballot(in && !hit);
    if (hit) idx[listed + rank_below(bh, lane)] = static_cast<int32_t>(x);
    else if (in) idx[total + others + rank_below(bo, lane)] = static_cast<int32_t>(x);
    listed += __popcll(bh);
    others += __popcll(bo);
  }
}

__global__ void __launch_bounds__(64 * kWaves)
    tile_lists_kernel(const int32_t* __restrict__ kinds, int64_t B, int64_t n_rows, int64_t n_cols,
                      int32_t* __restrict__ partial_count, int32_t* __restrict__ partial_idx,
                      int32_t* __restrict__ full_count, int32_t* __restrict__ full_idx,
                      int32_t* __restrict__ rev_partial_count, int32_t* __restrict__ rev_partial_idx,
                      int32_t* __restrict__ rev_full_count, int32_t* __restrict__ rev_full_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t line = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t n_fwd = B * n_rows;
  if (line < n_fwd) {  // block row (b, r)
    const int32_t* src = kinds + line * n_cols;
    if (partial_count != nullptr || partial_idx != nullptr)
      compact_line(src, n_cols, 1, 1, partial_count ? partial_count + line : nullptr,
                   partial_idx ? partial_idx + line * n_cols : nullptr, lane);
    if (full_count != nullptr || full_idx != nullptr)
      compact_line(src, n_cols, 1, 2, full_count ? full_count + line : nullptr,
                   full_idx ? full_idx + line * n_cols : nullptr, lane);
    return;
  }
  const int64_t o = line - n_fwd;  // block column (b, c)
  if (o >= B * n_cols) return;
  const int64_t b = o / n_cols, c = o % n_cols;
  const int32_t* src = kinds + b * n_rows * n_cols + c;
  if (rev_partial_count != nullptr || rev_partial_idx != nullptr)
    compact_line(src, n_rows, n_cols, 1, rev_partial_count ? rev_partial_count + o : nullptr,
                 rev_partial_idx ? rev_partial_idx + o * n_rows : nullptr, lane);
  if (rev_full_count != nullptr || rev_full_idx != nullptr)
    compact_line(src, n_rows, n_cols, 2, rev_full_count ? rev_full_count + o : nullptr,
                 rev_full_idx ? rev_full_idx + o * n_rows : nullptr, lane);
}

}  // namespace

hipError_t launch_tile_lists(const int32_t* kinds, int64_t B, int64_t n_rows, int64_t n_cols, int32_t* const out[8],
                             hipStream_t stream) {
  const int64_t lines = B * n_rows + B * n_cols;
  hipLaunchKernelGGL(tile_lists_kernel, dim3(static_cast<uint32_t>((lines + kWaves - 1) / kWaves)),
                     dim3(64 * kWaves), 0, stream, kinds, B, n_rows, n_cols, out[0], out[1], out[2], out[3], out[4],
                     out[5], out[6], out[7]);
  return hipGetLastError();
}

}  // namespace qsa

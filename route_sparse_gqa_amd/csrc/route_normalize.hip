// Route normalisation for gfx950: per query row, keep the valid route IDs
// (0 <= id < kv_length, int32 inputs sign-extended), sort them ascending,
// drop duplicates and compact them into an int32 list padded with -1.
//
// Definition: fa4_qsa page, `_preprocess`, routes parameter (a repeated ID
// counts once; an ID outside [0, kv_length), however large, is dropped
// before any address is formed); flex_qsa page, `_routes_to_membership`
// (negative or out-of-range entries stand for padding); qsa page,
// `QSARouteSelection` (int32 IDs, -1 marks padding).
//
// Design: one row is sorted by T = 64*W threads holding E keys each in
// registers (P = T*E >= K positions; position of register e of thread t is
// t*E + e).  Invalid slots become the key 0xFFFFFFFF, which sorts last.  The
// bitonic network exchanges partners in registers (distance < E), through
// wavefront shuffles (distance < 64*E) or through LDS (larger distances).
// Slots are loaded strided (slot e*T + t) so every load is coalesced; the
// network sorts any initial placement.  Duplicates are adjacent after the
// sort; per-thread keep counts are prefix-summed with one ballot per count
// bit, then the kept keys are compacted through LDS and written out
// coalesced.
//
// When the key range is small (kv_length <= 32 * kBitmapWords = 131072) and
// K <= kBitmapWords, a row is instead marked in an LDS bitmap of
// kv_length bits (integer atomic OR, so a repeated ID counts once by
// construction; the slots pass through LDS so that each lane takes a run of
// consecutive slots and merges the IDs that share a bitmap word in
// registers, one atomic per run).  One workgroup prefix sum over contiguous
// runs of words then gives every non-zero word its index in a compact list
// and the number of IDs before it; half-wavefronts expand one listed word
// each (lane j writes bit j's ID at its rank), so the IDs come out ascending
// with no sort and no per-bit loop: O(K + kv_length / 32) work per row
// instead of O(K log^2 K).  Rows with kv_length <= 16384 and K <= 1024 take
// one wavefront each (route_wave_kernel), the others one workgroup, whose
// LDS is sized for kv_length <= 65536 and K <= 2048 when that suffices (16
// KB, so more rows are in flight per CU) and for the limits above otherwise.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr uint32_t kAbsent = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t route_key(int64_t x, int64_t kv_length) {
  return (x >= 0 && x < kv_length) ? static_cast<uint32_t>(x) : kAbsent;
}

// Keep the smaller key at the lower position of an ascending pair, the larger
// one for a descending pair.
__device__ __forceinline__ uint32_t exchange(uint32_t mine, uint32_t other, int pos, int k, int s) {
  const bool ascending = (pos & k) == 0;
  const bool lower = (pos & s) == 0;
  return (lower == ascending) ? min(mine, other) : max(mine, other);
}

template <int W>
struct RowsPerBlock {
  static constexpr int value = W >= 4 ? 1 : 4 / W;
};

template <int E, int W, typename RouteT>
__global__ void __launch_bounds__(64 * W * RowsPerBlock<W>::value)
    route_normalize_kernel(const RouteT* __restrict__ routes, int64_t rs0, int64_t rs1, int64_t rs2,
                           int64_t S_q, int64_t K, int64_t kv_length, int64_t n_rows,
                           int32_t* __restrict__ route_list, int32_t* __restrict__ route_count,
                           int32_t* __restrict__ zero_buf, int64_t zero_count) {
  constexpr int T = 64 * W;
  constexpr int ROWS = RowsPerBlock<W>::value;
  constexpr int P = T * E;
  __shared__ uint32_t xch[ROWS][P];
  __shared__ uint32_t wave_last[ROWS][W];
  __shared__ int wave_kept[ROWS][W];

  const int tid = threadIdx.x;
  const int sub = tid / T;
  const int t = tid % T;
  const int lane = tid & 63;
  const int wave = t >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * ROWS + sub;
  const bool active = row < n_rows;  // whole rows; every thread still meets every barrier

  // ---- load (strided slots, coalesced) -----------------------------------
  uint32_t x[E];
  {
    const int64_t b = active ? row / S_q : 0;
    const int64_t i = active ? row % S_q : 0;
    const RouteT* src = routes + b * rs0 + i * rs1;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t slot = static_cast<int64_t>(e) * T + t;
      x[e] = (active && slot < K) ? route_key(static_cast<int64_t>(src[slot * rs2]), kv_length) : kAbsent;
    }
  }

  // ---- bitonic sort over positions t*E + e --------------------------------
#pragma unroll
  for (int k = 2; k <= P; k <<= 1) {
#pragma unroll
    for (int s = k >> 1; s > 0; s >>= 1) {
      if (s >= 64 * E) {  // partner in another wave of this row
#pragma unroll
        for (int e = 0; e < E; ++e) xch[sub][t * E + e] = x[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int pos = t * E + e;
          x[e] = exchange(x[e], xch[sub][pos ^ s], pos, k, s);
        }
        __syncthreads();
      } else if (s >= E) {  // partner lane in this wave, same register
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x[e]), s / E));
          x[e] = exchange(x[e], other, t * E + e, k, s);
        }
      } else {  // both positions in this thread
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & s) == 0) {
            const bool ascending = ((t * E + e) & k) == 0;
            const uint32_t a = x[e], c = x[e + s];
            x[e] = ascending ? min(a, c) : max(a, c);
            x[e + s] = ascending ? max(a, c) : min(a, c);
          }
        }
      }
    }
  }

  // ---- drop duplicates (equal keys are adjacent) --------------------------
  uint32_t prev = static_cast<uint32_t>(__shfl_up(static_cast<int>(x[E - 1]), 1));
  if (lane == 63) wave_last[sub][wave] = x[E - 1];
  __syncthreads();
  if (lane == 0) prev = wave > 0 ? wave_last[sub][wave - 1] : kAbsent;
  // position 0 has no predecessor; kAbsent never equals a valid key
  bool keep[E];
  int kept = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t before = e == 0 ? prev : x[e - 1];
    keep[e] = x[e] != kAbsent && x[e] != before;
    kept += keep[e] ? 1 : 0;
  }

  // ---- ballot prefix sum of per-thread counts (kept <= E < 32) -------------
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int offset = 0, wave_total = 0;
#pragma unroll
  for (int bit = 0; (1 << bit) <= E; ++bit) {
    const uint64_t m = __ballot((kept >> bit) & 1);
    offset += __popcll(m & below) << bit;
    wave_total += __popcll(m) << bit;
  }
  if (lane == 0) wave_kept[sub][wave] = wave_total;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int c = wave_kept[sub][w];
    offset += w < wave ? c : 0;
    total += c;
  }

  // ---- compact through LDS, then write the padded list coalesced ----------
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (keep[e]) xch[sub][offset++] = x[e];
  }
  __syncthreads();
  if (active) {
    int32_t* dst = route_list + row * K;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t slot = static_cast<int64_t>(e) * T + t;
      if (slot < K) dst[slot] = slot < total ? static_cast<int32_t>(xch[sub][slot]) : -1;
    }
    if (t == 0) route_count[row] = total;
  }
  if (zero_buf != nullptr) {  // side job: clear the tile member counters (grid-stride)
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t z = static_cast<int64_t>(blockIdx.x) * blockDim.x + tid; z < zero_count; z += stride)
      zero_buf[z] = 0;
  }
}

constexpr int kBitmapThreads = 256;
constexpr int kBitmapWords = 4096;  // largest bitmap: kv_length <= 131072, K <= 4096
constexpr int kBitmapWordsHalf = 2048;  // kv_length <= 65536, K <= 2048: half the LDS, more rows per CU

// kWords bitmap words (kv_length <= 32 kWords) and kWords route slots (K <= kWords) per row.
template <int kWords, typename RouteT>
__global__ void __launch_bounds__(kBitmapThreads)
    route_bitmap_kernel(const RouteT* __restrict__ routes, int64_t rs0, int64_t rs1, int64_t rs2, int64_t S_q,
                        int64_t K, int64_t kv_length, int32_t* __restrict__ route_list,
                        int32_t* __restrict__ route_count, int32_t* __restrict__ zero_buf, int64_t zero_count) {
  constexpr int T = kBitmapThreads;
  constexpr int kBitmapRun = kWords / T;  // bitmap words (and route slots) per thread
  __shared__ uint32_t region[kWords];   // the row's bitmap
  // The slots as IDs, then its non-zero words: index << 16 | IDs before the word.
  __shared__ __attribute__((aligned(16))) uint32_t nonzero[kWords];
  __shared__ int wave_tot[T / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nw = static_cast<int>((kv_length + 31) / 32);
  const int run = (nw + T - 1) / T;  // words per thread (<= kBitmapRun)
  const int Ki = static_cast<int>(K);

  // Every slot of the row is loaded before any is used (one memory latency per row).
  const RouteT* src = routes + (row / S_q) * rs0 + (row % S_q) * rs1;
  int64_t x[kBitmapRun];  // K <= kBitmapRun * T slots
#pragma unroll
  for (int q = 0; q < kBitmapRun; ++q) {
    const int s = q * T + tid;
    x[q] = s < Ki ? static_cast<int64_t>(src[s * rs2]) : int64_t{-1};  // int32 IDs sign-extend
  }
  for (int w = tid; w < nw; w += T) region[w] = 0u;
  // The slots as validated int32 IDs in slot order, staged in the list array (free until the scan).
#pragma unroll
  for (int q = 0; q < kBitmapRun; ++q) {
    const bool ok = x[q] >= 0 && x[q] < kv_length;
    nonzero[q * T + tid] = ok ? static_cast<uint32_t>(x[q]) : 0xFFFFFFFFu;
  }
  __syncthreads();
  if (tid * kBitmapRun < Ki)
    or_slot_run<kBitmapRun>(region, reinterpret_cast<const int32_t*>(nonzero) + tid * kBitmapRun);
  __syncthreads();

  // Thread tid owns words tid*run .. tid*run + run - 1.  One prefix sum over threads of
  // (non-zero words << 16 | set bits) places every non-zero word and every ID (both <= 4096).
  uint32_t mine[kBitmapRun];
  int packed = 0;
#pragma unroll
  for (int q = 0; q < kBitmapRun; ++q) {
    const int w = tid * run + q;
    mine[q] = (q < run && w < nw) ? region[w] : 0u;
    packed += (mine[q] != 0u ? 1 << 16 : 0) + __popc(mine[q]);
  }
  int incl = packed;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - packed, all = 0;
#pragma unroll
  for (int q = 0; q < T / 64; ++q) {
    before += q < wave ? wave_tot[q] : 0;
    all += wave_tot[q];
  }
  int slot = before >> 16, ids = before & 0xFFFF;
#pragma unroll
  for (int q = 0; q < kBitmapRun; ++q) {
    if (mine[q] != 0u) {
      nonzero[slot++] = static_cast<uint32_t>((tid * run + q) << 16 | ids);
      ids += __popc(mine[q]);
    }
  }
  __syncthreads();
  const int n_nonzero = all >> 16, total = all & 0xFFFF;

  // Each half-wavefront expands one non-zero word: lane j writes bit j's ID at its rank.
  int32_t* dst = route_list + row * K;
  const int half = lane >> 5, j = lane & 31;
  for (int e = 2 * wave + half; e < n_nonzero; e += 2 * (T / 64)) {
    const uint32_t entry = nonzero[e];
    const int w = static_cast<int>(entry >> 16);
    const uint32_t word = region[w];
    if ((word >> j) & 1u) dst[(entry & 0xFFFFu) + __popc(word & ((1u << j) - 1u))] = 32 * w + j;
  }
  for (int s = total + tid; s < Ki; s += T) dst[s] = -1;
  if (tid == 0) route_count[row] = total;
  if (zero_buf != nullptr) {  // side job: clear the tile member counters (grid-stride)
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t z = static_cast<int64_t>(blockIdx.x) * blockDim.x + tid; z < zero_count; z += stride)
      zero_buf[z] = 0;
  }
}

template <int E, int W, typename RouteT>
hipError_t launch_sorted(const RouteT* routes, const int64_t* st, int64_t B, int64_t S_q, int64_t K,
                         int64_t kv_length, int32_t* list, int32_t* count, int32_t* zb, int64_t zn,
                         hipStream_t stream) {
  constexpr int ROWS = RowsPerBlock<W>::value;
  const int64_t n_rows = B * S_q;
  const int64_t blocks = (n_rows + ROWS - 1) / ROWS;
  hipLaunchKernelGGL((route_normalize_kernel<E, W, RouteT>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * W * ROWS), 0, stream, routes, st[0], st[1], st[2], S_q, K, kv_length,
                     n_rows, list, count, zb, zn);
  return hipGetLastError();
}

// Small rows (kv_length <= 32 * kWaveWords = 16384, K <= 1024): the bitmap
// method of route_bitmap_kernel with one wavefront per row and four rows per
// workgroup, so no workgroup barrier is needed and every row of a call is in
// flight at once.  Lane l holds slots q * 64 + l and owns bitmap words
// l * wpl .. l * wpl + wpl - 1 (wpl = ceil(words / 64) <= 8) for the scan.
constexpr int kWaveRows = 4;
constexpr int kWaveWords = 512;

template <int kSlots, typename RouteT>
__global__ void __launch_bounds__(64 * kWaveRows)
    route_wave_kernel(const RouteT* __restrict__ routes, int64_t rs0, int64_t rs1, int64_t rs2, int64_t S_q,
                      int64_t n_rows, int64_t K, int64_t kv_length, int32_t* __restrict__ route_list,
                      int32_t* __restrict__ route_count, int32_t* __restrict__ zero_buf, int64_t zero_count) {
  constexpr int kWpl = kWaveWords / 64;  // bitmap words per lane at most
  __shared__ uint32_t region[kWaveRows][kWaveWords];   // each wavefront's bitmap
  // Its slots as IDs, then its non-zero words: index << 16 | IDs before the word.
  __shared__ __attribute__((aligned(16))) uint32_t nonzero[kWaveRows][64 * kSlots];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaveRows + wave;
  if (row < n_rows) {  // wavefront-uniform; the wavefronts never wait for one another
    uint32_t* bits = region[wave];
    const int nw = static_cast<int>((kv_length + 31) / 32);
    const int wpl = (nw + 63) / 64;
    const int Ki = static_cast<int>(K);
    const RouteT* src = routes + (row / S_q) * rs0 + (row % S_q) * rs1;
    int64_t x[kSlots];  // every slot is loaded before any is used
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int s = q * 64 + lane;
      x[q] = s < Ki ? static_cast<int64_t>(src[s * rs2]) : int64_t{-1};  // int32 IDs sign-extend
    }
    for (int w = lane; w < nw; w += 64) bits[w] = 0u;
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const bool ok = x[q] >= 0 && x[q] < kv_length;
      nonzero[wave][q * 64 + lane] = ok ? static_cast<uint32_t>(x[q]) : 0xFFFFFFFFu;
    }
    wave_lds_sync();
    if (lane * kSlots < Ki)
      or_slot_run<kSlots>(bits, reinterpret_cast<const int32_t*>(nonzero[wave]) + lane * kSlots);
    wave_lds_sync();

    // One wavefront prefix sum of (non-zero words << 16 | set bits) over the lanes' word runs.
    uint32_t mine[kWpl];
    int packed = 0;
#pragma unroll
    for (int q = 0; q < kWpl; ++q) {
      const int w = lane * wpl + q;
      mine[q] = (q < wpl && w < nw) ? bits[w] : 0u;
      packed += (mine[q] != 0u ? 1 << 16 : 0) + __popc(mine[q]);
    }
    int incl = packed;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int all = __shfl(incl, 63);
    const int before = incl - packed;
    int slot = before >> 16, ids = before & 0xFFFF;
#pragma unroll
    for (int q = 0; q < kWpl; ++q) {
      if (mine[q] != 0u) {
        nonzero[wave][slot++] = static_cast<uint32_t>((lane * wpl + q) << 16 | ids);
        ids += __popc(mine[q]);
      }
    }
    wave_lds_sync();
    const int n_nonzero = all >> 16, total = all & 0xFFFF;

    // Each half-wavefront expands one non-zero word: lane j writes bit j's ID at its rank.
    int32_t* dst = route_list + row * K;
    const int half = lane >> 5, j = lane & 31;
    for (int e = half; e < n_nonzero; e += 2) {
      const uint32_t entry = nonzero[wave][e];
      const int w = static_cast<int>(entry >> 16);
      const uint32_t word = bits[w];
      if ((word >> j) & 1u) dst[(entry & 0xFFFFu) + __popc(word & ((1u << j) - 1u))] = 32 * w + j;
    }
    for (int s = total + lane; s < Ki; s += 64) dst[s] = -1;
    if (lane == 0) route_count[row] = total;
  }
  if (zero_buf != nullptr) {  // side job: clear the tile member counters (grid-stride)
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t z = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; z < zero_count; z += stride)
      zero_buf[z] = 0;
  }
}

// The launch that normalises rows of K slots over kv_length keys.
enum class RoutePath { kWave8, kWave16, kBitmapHalf, kBitmap, kSorted };

RoutePath route_path(int64_t K, int64_t kv_length) {
  if (kv_length <= 32 * kWaveWords && K <= 1024) return K <= 512 ? RoutePath::kWave8 : RoutePath::kWave16;
  if (kv_length <= 32 * int64_t{kBitmapWordsHalf} && K <= kBitmapWordsHalf) return RoutePath::kBitmapHalf;
  if (kv_length <= 32 * int64_t{kBitmapWords} && K <= kBitmapWords) return RoutePath::kBitmap;
  return RoutePath::kSorted;
}

// Wavefronts per row of the sorting path (the W of launch_sorted).
int64_t sorted_waves(int64_t K) { return K <= 512 ? 1 : K <= 1024 ? 2 : K <= 2048 ? 4 : K <= 4096 ? 8 : 16; }

template <typename RouteT>
hipError_t dispatch(const RouteT* routes, const int64_t* st, int64_t B, int64_t S_q, int64_t K,
                    int64_t kv_length, int32_t* list, int32_t* count, int32_t* zb, int64_t zn,
                    hipStream_t stream) {
  const dim3 rows(static_cast<uint32_t>(B * S_q)), threads(kBitmapThreads);
  const RoutePath path = route_path(K, kv_length);
  if (path == RoutePath::kWave8 || path == RoutePath::kWave16) {  // small rows: one wavefront each
    const int64_t n_rows = B * S_q;
    const dim3 groups(static_cast<uint32_t>((n_rows + kWaveRows - 1) / kWaveRows)), wave_threads(64 * kWaveRows);
    if (path == RoutePath::kWave8)
      hipLaunchKernelGGL((route_wave_kernel<8, RouteT>), groups, wave_threads, 0, stream, routes, st[0], st[1], st[2],
                         S_q, n_rows, K, kv_length, list, count, zb, zn);
    else
      hipLaunchKernelGGL((route_wave_kernel<16, RouteT>), groups, wave_threads, 0, stream, routes, st[0], st[1],
                         st[2], S_q, n_rows, K, kv_length, list, count, zb, zn);
    return hipGetLastError();
  }
  if (path == RoutePath::kBitmapHalf) {
    hipLaunchKernelGGL((route_bitmap_kernel<kBitmapWordsHalf, RouteT>), rows, threads, 0, stream, routes, st[0],
                       st[1], st[2], S_q, K, kv_length, list, count, zb, zn);
    return hipGetLastError();
  }
  if (path == RoutePath::kBitmap) {
    hipLaunchKernelGGL((route_bitmap_kernel<kBitmapWords, RouteT>), rows, threads, 0, stream, routes, st[0], st[1],
                       st[2], S_q, K, kv_length, list, count, zb, zn);
    return hipGetLastError();
  }
  if (K <= 64) return launch_sorted<1, 1>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 128) return launch_sorted<2, 1>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 256) return launch_sorted<4, 1>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 512) return launch_sorted<8, 1>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 1024) return launch_sorted<8, 2>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 2048) return launch_sorted<8, 4>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 4096) return launch_sorted<8, 8>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  if (K <= 8192) return launch_sorted<8, 16>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
  return launch_sorted<16, 16>(routes, st, B, S_q, K, kv_length, list, count, zb, zn, stream);
}

}  // namespace

int64_t route_normalize_items_per_row(int64_t K, int64_t kv_length) {
  switch (route_path(K, kv_length)) {
    case RoutePath::kWave8:
    case RoutePath::kWave16: return 64;
    case RoutePath::kBitmapHalf:
    case RoutePath::kBitmap: return kBitmapThreads;
    default: return 64 * sorted_waves(K);  // 64 * W * ROWS threads per ROWS rows
  }
}

hipError_t launch_route_normalize(const void* routes, bool routes_int64, int64_t B, int64_t S_q,
                                  int64_t K, const int64_t route_strides[3], int64_t kv_length,
                                  int32_t* route_list, int32_t* route_count, int32_t* zero_buf,
                                  int64_t zero_count, hipStream_t stream) {
  if (routes_int64)
    return dispatch(static_cast<const int64_t*>(routes), route_strides, B, S_q, K, kv_length, route_list,
                    route_count, zero_buf, zero_count, stream);
  return dispatch(static_cast<const int32_t*>(routes), route_strides, B, S_q, K, kv_length, route_list,
                  route_count, zero_buf, zero_count, stream);
}

}  // namespace qsa

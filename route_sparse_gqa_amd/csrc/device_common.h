// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vectors stay in registers
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane
// group, slot j of lane i receives element i % 4 of the 4-element row piece
// addressed by lane 4 * j + i / 4.  With lane L addressing row L / 4,
// columns 16t + 4 * (L % 4) of a row-major bf16 tile, lane (c, g) =
// (L % 16, L / 16) receives rows 4g .. 4g+3 of column 16t + c: the A operand
// of v_mfma_f32_16x16x16_bf16 for the transposed tile.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));  // generic -> LDS address-space cast
}

// Route ID of the rows of gather load u of a chunk, for this lane: with R
// rows per load instruction, lane L loads row u * R + L / (64 / R), whose ID
// sits in lane (u * R + L / (64 / R)) of `id` (row r's ID in lane r).  The R
// IDs are read into scalar registers (v_readlane: no LDS round trip, which
// would queue behind the chunk's slab writes) and selected by the lane's row.
template <int R>
__device__ __forceinline__ int32_t chunk_row_id(int32_t id, int u, int lane) {
  const int rsel = lane / (64 / R);
  int32_t v = __builtin_amdgcn_readlane(id, u * R);
#pragma unroll
  for (int q = 1; q < R; ++q) {
    const int32_t s_id = __builtin_amdgcn_readlane(id, u * R + q);
    v = rsel == q ? s_id : v;
  }
  return v;
}

// Orders this wavefront's LDS writes before its later LDS reads (and the
// reverse); wavefront scope only, so no workgroup barrier is involved.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ORs bit (id & 31) into bits[id >> 5] for N consecutive entries of a route row staged in LDS
// (`slots`, 16-byte aligned; -1 = no ID).  Consecutive entries usually hold consecutive token IDs,
// so IDs that share a 32-bit word are merged in registers and one atomic OR is issued per run of
// such entries (lanes of one atomic instruction that hit the same address serialise); any order
// of IDs gives the same bitmap.
template <int N>
__device__ __forceinline__ void or_slot_run(uint32_t* bits, const int32_t* slots) {
  int32_t id[N];
#pragma unroll
  for (int u = 0; u < N; u += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(slots + u);
    id[u] = static_cast<int32_t>(v.x);
    id[u + 1] = static_cast<int32_t>(v.y);
    id[u + 2] = static_cast<int32_t>(v.z);
    id[u + 3] = static_cast<int32_t>(v.w);
  }
  uint32_t cur_w = 0xFFFFFFFFu, cur_b = 0u;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const uint32_t w = id[u] >= 0 ? static_cast<uint32_t>(id[u]) >> 5 : 0xFFFFFFFFu;
    const uint32_t b = id[u] >= 0 ? 1u << (id[u] & 31) : 0u;
    if (w != cur_w) {
      if (cur_b != 0u) atomicOr(&bits[cur_w], cur_b);
      cur_w = w;
      cur_b = b;
    } else {
      cur_b |= b;
    }
  }
  if (cur_b != 0u) atomicOr(&bits[cur_w], cur_b);
}

// Pairwise max / sum of each lane with the lane 16 apart (within its 32-lane
// half) and with the lane 32 apart, in registers (gfx950 permlane swaps of two
// copies leave the pair in the two results) instead of through LDS.
__device__ __forceinline__ float pair_max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Byte offset of a gathered row: 32-bit when every row of the tensor lies
// within 4 GiB of its (batch, head) base, else 64-bit.
template <bool kNarrow>
struct RowOffset {
  __device__ static __forceinline__ uint32_t of(int32_t id, int64_t stride_bytes) {
    return static_cast<uint32_t>(id) * static_cast<uint32_t>(stride_bytes);
  }
};
template <>
struct RowOffset<false> {
  __device__ static __forceinline__ int64_t of(int32_t id, int64_t stride_bytes) {
    return static_cast<int64_t>(id) * stride_bytes;
  }
};

// Range starts of one row, one per lane: lane l < P gets its range's part
// [lo, hi) of the list, clamped into [0, n], n = the row's count clamped into
// [0, K] (stored at index P); returns the mask of lanes with a non-empty part.
__device__ __forceinline__ uint64_t range_parts(const int32_t* __restrict__ offs_row, int P, int64_t K, int lane,
                                                int* lo_out, int* hi_out) {
  const int32_t o = lane <= P ? offs_row[lane] : 0;
  const int n = min(max(__shfl(o, P), 0), static_cast<int>(K));
  const int lo = min(max(o, 0), n);
  const int hi = min(max(__shfl(o, min(lane + 1, 63)), lo), n);
  *lo_out = lo;
  *hi_out = hi;
  return __ballot(lane < P && lo < hi);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace qsa

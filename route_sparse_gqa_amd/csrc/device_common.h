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

// Orders this wavefront's LDS writes before its later LDS reads (and the
// reverse); wavefront scope only, so no workgroup barrier is involved.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ORs `bits` into words[w] for every lane of the wavefront whose w is not
// 0xFFFFFFFF.  Consecutive lanes holding the same word (the runs that
// consecutive token IDs produce) are first merged by a segmented OR over
// shuffles, so each run costs one LDS atomic instead of one per lane (lanes
// of one atomic instruction that hit the same address are serialised).
// Every lane of the wavefront must call it.
__device__ __forceinline__ void wave_or_runs(uint32_t* words, uint32_t w, uint32_t bits) {
  const int lane = threadIdx.x & 63;
  const uint32_t prev = static_cast<uint32_t>(__shfl_up(static_cast<int>(w), 1));
  const bool head = lane == 0 || prev != w;
  const uint64_t heads = __ballot(head);
  const uint64_t after = heads & ~((2ull << lane) - 1ull);  // heads above this lane (lane 63: none)
  const int next = after != 0ull ? __builtin_ctzll(after) : 64;  // first lane of the next run
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t other = static_cast<uint32_t>(__shfl_down(static_cast<int>(bits), o));
    if (lane + o < next) bits |= other;  // lanes l .. min(l + 2o, next) - 1 are now merged
  }
  if (head && w != 0xFFFFFFFFu && bits != 0u) atomicOr(&words[w], bits);
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace qsa

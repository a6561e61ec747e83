// Gather-bandwidth probe behind `bench.py --calibrate-gather` (a measuring
// tool, not part of the attention library's API; built as libqsa_probe.so).
//
// Each wavefront copies chunks of 16 randomly chosen 512-byte rows of a
// strided table into its own LDS slab the way gather_attention_kernel stages
// its K and V rows (16-byte loads, two whole rows per load instruction, then
// 16-byte LDS writes), and does no arithmetic, so the time measures what the
// chip can deliver for that access pattern.  With a table that fits the L2,
// the Infinity Cache or neither, it gives the gather ceiling that bounds the
// attention kernels at each working-set size.  Unused dynamic LDS per
// workgroup (lds_pad) lowers the number of workgroups a CU holds, to measure
// the ceiling at the attention kernels' occupancy (two wavefronts per SIMD at
// D = 256).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowBytes = 512;  // one KV head's row at D = 256
constexpr int kChunk = 16;      // rows per chunk, as in the attention kernels
constexpr int kWaves = 4;

// kDirect: the rows go to LDS with global_load_lds_dwordx4 (lane L's 16 bytes land at the wave-uniform
// LDS address + 16 L) instead of through registers and LDS writes.
template <bool kDirect>
__global__ void __launch_bounds__(64 * kWaves)
    probe_gather_kernel(const uint8_t* __restrict__ table, int64_t n_rows, int64_t stride,
                        const int32_t* __restrict__ ids, int64_t n_waves, int chunks, uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t slab[kWaves][kChunk * kRowBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if (w >= n_waves) return;  // no workgroup barriers below
  const int32_t* my_ids = ids + w * chunks * kChunk;
  uint8_t* s = slab[wave];
  uint32_t acc = 0;
  for (int c = 0; c < chunks; ++c) {
    u32x4 r[kChunk / 2];
#pragma unroll
    for (int u = 0; u < kChunk / 2; ++u) {
      const int64_t row = min(max(static_cast<int64_t>(my_ids[c * kChunk + 2 * u + (lane >> 5)]), int64_t{0}),
                              n_rows - 1);
      const uint8_t* src = table + row * stride + (lane & 31) * 16;
      if constexpr (kDirect) {
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(s + u * 1024), 16, 0, 0);
#endif
      } else {
        r[u] = *reinterpret_cast<const u32x4*>(src);
      }
    }
    if constexpr (kDirect) {
      __builtin_amdgcn_s_waitcnt(0);  // the direct loads have landed in LDS
    } else {
#pragma unroll
      for (int u = 0; u < kChunk / 2; ++u) *reinterpret_cast<u32x4*>(s + u * 1024 + lane * 16) = r[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    acc += reinterpret_cast<const uint32_t*>(s)[(lane * 37 + c * 11) % (kChunk * kRowBytes / 4)];
    __builtin_amdgcn_wave_barrier();
  }
  out[w * 64 + lane] = acc;  // keeps the copies live
}

}  // namespace

// table: n_rows rows of >= 512 bytes, `stride` bytes apart (16-byte aligned); ids: n_waves * chunks * 16
// row indices (clamped into [0, n_rows)); out: n_waves * 64 words; direct: 0 through registers, 1
// straight to LDS; lds_pad: unused dynamic LDS bytes per workgroup, 0 .. 131072 (the 32 KB of slabs
// plus the pad stay within a CU's 160 KB).  Returns 0, -1 for a bad argument, -12 for a launch error.
extern "C" __attribute__((visibility("default"))) int qsa_probe_gather(const void* table, int64_t n_rows,
                                                                       int64_t stride, const int32_t* ids,
                                                                       int64_t n_waves, int chunks, int direct,
                                                                       int lds_pad, uint32_t* out, void* stream) {
  if (table == nullptr || ids == nullptr || out == nullptr || n_rows < 1 || stride < kRowBytes || stride % 16 != 0 ||
      n_waves < 1 || chunks < 1 || (direct != 0 && direct != 1) || (reinterpret_cast<uintptr_t>(table) & 15) != 0 ||
      lds_pad < 0 || lds_pad > 131072 || (n_waves + kWaves - 1) / kWaves > (int64_t{1} << 31) - 1)
    return -1;
  const dim3 grid(static_cast<uint32_t>((n_waves + kWaves - 1) / kWaves));
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* t = static_cast<const uint8_t*>(table);
  if (direct)
    hipLaunchKernelGGL(probe_gather_kernel<true>, grid, dim3(64 * kWaves), static_cast<size_t>(lds_pad), st, t, n_rows, stride, ids, n_waves,
                       chunks, out);
  else
    hipLaunchKernelGGL(probe_gather_kernel<false>, grid, dim3(64 * kWaves), static_cast<size_t>(lds_pad), st, t, n_rows, stride, ids, n_waves,
                       chunks, out);
  return hipGetLastError() == hipSuccess ? 0 : -12;
}

// Fused gather-attention for gfx950 over compacted route lists.
//
// Definition: flex_qsa page, `flex_sparse_gqa_attention` and module
// description (each query row attends exactly to its routes, empty rows give
// zero); fa4_qsa page, `fa4_sparse_gqa_attention` (no extra mask; BF16);
// qsa page, `_gathered_qsa_gqa_attention_chunk` (grouped layout
// [B, Q, Hkv, G, D]: query head h reads KV head h / G).
//
// Design (one wavefront per (b, i, hk) work unit, four per workgroup):
//  * The G query heads of the unit are the N = 16 columns of
//    v_mfma_f32_16x16x32_bf16 (padded with zero heads when G < 16).  Scores
//    are computed transposed, S^T = K Q^T, with 16 routed keys as the M rows,
//    so each lane ends up owning one head (lane % 16) and four keys per
//    16-key tile.  Row max/sum reductions are then two cross-lane xors.
//  * Routed K rows are loaded straight from global memory into the MFMA A
//    operand: lane (c, g) = (lane % 16, lane / 16) loads 16 bytes (8 dims)
//    of key c, so one load instruction gathers 16 keys x 64 contiguous bytes.
//  * PV is computed transposed too, O^T = V^T P^T, so the probabilities stay
//    in the lane that produced them (the B operand needs no shuffle) and the
//    online-softmax rescale is lane-local.  The V^T operand needs 8 keys of
//    one dim per lane, so the 32 routed V rows of a chunk are gathered with
//    coalesced 16-byte loads into this wave's LDS slab and read back
//    transposed.
//  * Online softmax in fp32 with exp2 and the scale folded into log2(e);
//    probabilities are rounded to bf16 once and the same rounded values feed
//    both the PV product and the normaliser.
#include <hip/hip_runtime.h>

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;     // work units per workgroup
constexpr int kChunk = 32;    // routes per inner iteration (PV contraction depth)

template <int D>
struct Geometry {
  static constexpr int kSteps = D / 32;                // QK^T k-steps of 32 dims
  static constexpr int kDimTiles = D / 16;             // O^T row tiles of 16 dims
  static constexpr int kLanesPerRow = D / 8;           // 16-byte pieces per V row
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kLoads = kChunk / kRowsPerLoad;  // V load instructions per chunk
  static constexpr int kStride = D + 8;                // LDS row stride in bf16 (16-byte aligned rows)
};

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ void __launch_bounds__(64 * kWaves)
    gather_attention_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                            const uint16_t* __restrict__ v, int64_t qs0, int64_t qs1, int64_t qs2,
                            int64_t ks0, int64_t ks1, int64_t ks2, int64_t vs0, int64_t vs1, int64_t vs2,
                            const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                            int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t K, int G,
                            float scale_log2e, int64_t n_units, uint16_t* __restrict__ out) {
  using Geo = Geometry<D>;
  __shared__ __attribute__((aligned(16))) uint16_t slab[kWaves][kChunk * Geo::kStride];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if (unit >= n_units) return;  // no workgroup barriers in this kernel
  const int64_t hk = unit % Hkv;
  const int64_t row = unit / Hkv;  // b * S_q + i
  const int64_t b = row / S_q;
  const int64_t i = row % S_q;
  const int c = lane & 15;  // head column of this lane; also key/dim row within a 16-tile
  const int g = lane >> 4;  // k-group of this lane
  const bool head_ok = c < G;
  uint16_t* out_row = out + (row * Hq + hk * G + c) * D;  // only dereferenced when head_ok

  const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
  if (n == 0) {  // empty route set: exactly +0.0
    if (head_ok) {
#pragma unroll
      for (int t = 0; t < Geo::kDimTiles; ++t)
        *reinterpret_cast<u32x2*>(out_row + 16 * t + 4 * g) = u32x2{0u, 0u};
    }
    return;
  }

  // Q^T as the MFMA B operand: lane (c, g) holds head c, dims 32s + 8g .. +7.
  bf16x8 qf[Geo::kSteps];
  {
    const uint16_t* qp = q + b * qs0 + i * qs1 + (hk * G + (head_ok ? c : 0)) * qs2 + 8 * g;
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s) {
      qf[s] = head_ok ? load16(qp + 32 * s) : bf16x8{};
    }
  }

  f32x4 acc[Geo::kDimTiles];
#pragma unroll
  for (int t = 0; t < Geo::kDimTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head c
  float l_run = 0.f;        // this lane's share of the running sum of head c

  const int32_t* lst = route_list + row * K;
  const uint16_t* kb = k + b * ks0 + hk * ks2 + 8 * g;
  const uint16_t* vb = v + b * vs0 + hk * vs2 + 8 * (lane % Geo::kLanesPerRow);
  uint16_t* my_slab = slab[wave];
  const int32_t id_max = static_cast<int32_t>(S_kv - 1);

  for (int base = 0; base < n; base += kChunk) {
    // Route IDs of keys base + c and base + 16 + c (tails repeat the last route).
    const int32_t id0 = min(max(lst[min(base + c, n - 1)], 0), id_max);
    const int32_t id1 = min(max(lst[min(base + 16 + c, n - 1)], 0), id_max);

    // Gather K straight into the A operand of S^T = K Q^T.
    bf16x8 kf0[Geo::kSteps], kf1[Geo::kSteps];
    {
      const uint16_t* k0 = kb + static_cast<int64_t>(id0) * ks1;
      const uint16_t* k1 = kb + static_cast<int64_t>(id1) * ks1;
#pragma unroll
      for (int s = 0; s < Geo::kSteps; ++s) {
        kf0[s] = load16(k0 + 32 * s);
        kf1[s] = load16(k1 + 32 * s);
      }
    }
    // Gather the chunk's V rows (coalesced 16-byte pieces) into registers.
    u32x4 vr[Geo::kLoads];
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int r = u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow;  // chunk row of this lane
      const int src = (u * Geo::kRowsPerLoad < 16) ? id0 : id1;       // uniform per u
      const int32_t idr = __shfl(src, r & 15);
      vr[u] = *reinterpret_cast<const u32x4*>(vb + static_cast<int64_t>(idr) * vs1);
    }

    // Scores: lane holds S^T[key 16*tau + 4g + r][head c].
    f32x4 st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s) {
      st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf0[s], qf[s], st0, 0, 0, 0);
      st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf1[s], qf[s], st1, 0, 0, 0);
    }

    // Stage V rows in LDS (row-major, padded stride).
    wave_lds_sync();  // previous chunk's transposed reads are complete
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int r = u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow;
      *reinterpret_cast<u32x4*>(my_slab + r * Geo::kStride + 8 * (lane % Geo::kLanesPerRow)) = vr[u];
    }

    // Online softmax (log2 domain).
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key0 = base + 4 * g + r, key1 = base + 16 + 4 * g + r;
      x[r] = key0 < n ? st0[r] * scale_log2e : -INFINITY;
      x[4 + r] = key1 < n ? st1[r] * scale_log2e : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: the chunk holds at least one key
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    bf16x8 pf;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 p = static_cast<__bf16>(exp2f(x[j] - m_new));
      pf[j] = p;
      psum += static_cast<float>(p);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t) acc[t] *= alpha;

    // O^T += V^T P^T; element j of lane group g is key 16*(j/4) + 4g + j%4.
    wave_lds_sync();  // V rows visible to every lane of this wave
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t) {
      bf16x8 va;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = 16 * (j >> 2) + 4 * g + (j & 3);
        va[j] = __builtin_bit_cast(__bf16, my_slab[key * Geo::kStride + 16 * t + c]);
      }
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, acc[t], 0, 0, 0);
    }
  }

  // Normalise and store: lane holds O[head c][dims 16t + 4g .. +3].
  float l_tot = l_run + __shfl_xor(l_run, 16);  // butterfly over the four lane groups of head c
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  if (head_ok) {
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t) {
      const __bf16 o0 = static_cast<__bf16>(acc[t][0] * inv), o1 = static_cast<__bf16>(acc[t][1] * inv);
      const __bf16 o2 = static_cast<__bf16>(acc[t][2] * inv), o3 = static_cast<__bf16>(acc[t][3] * inv);
      const uint32_t lo = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o0)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o1)) << 16);
      const uint32_t hi = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o2)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o3)) << 16);
      *reinterpret_cast<u32x2*>(out_row + 16 * t + 4 * g) = u32x2{lo, hi};
    }
  }
}

template <int D>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const int64_t n_units = a.B * a.S_q * a.Hkv;
  const int64_t blocks = (n_units + kWaves - 1) / kWaves;
  const float scale_log2e = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((gather_attention_kernel<D>), dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWaves), 0,
                     stream, a.q, a.k, a.v, a.qs[0], a.qs[1], a.qs[2], a.ks[0], a.ks[1], a.ks[2], a.vs[0],
                     a.vs[1], a.vs[2], a.route_list, a.route_count, a.S_q, a.S_kv, a.Hq, a.Hkv, a.K,
                     static_cast<int>(a.Hq / a.Hkv), scale_log2e, n_units, a.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_attention(const AttnArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch<64>(a, stream);
    case 128: return launch<128>(a, stream);
    case 256: return launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa

// Fused gather-attention for gfx950 over compacted route lists.
//
// Definition: flex_qsa page, `flex_sparse_gqa_attention` and module
// description (each query row attends exactly to its routes, empty rows give
// zero); fa4_qsa page, `fa4_sparse_gqa_attention` (no extra mask; BF16);
// qsa page, `_gathered_qsa_gqa_attention_chunk` (grouped layout
// [B, Q, Hkv, G, D]: query head h reads KV head h / G).
//
// Design (one wavefront per (b, i, hk) work unit, four rows of one KV head
// per workgroup, mapped so that each XCD serves one KV head, rows taken from
// the last to the first):
//  * The G query heads of the unit are the N = 16 columns of the MFMA (zero
//    padded when G < 16).  Scores are computed transposed, S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16, 16 routed keys as the M rows, so each lane
//    ends up owning one head and four keys; row max/sum reductions are two
//    cross-lane xors.  Routed K and V rows are both gathered two full rows
//    per 16-byte-per-lane load instruction (fewest cache lines per
//    instruction for the address unit) and staged in this wave's LDS slabs;
//    the K slab's 2D + 16 byte stride makes the A-operand reads (lane
//    (c, g) = (lane % 16, lane / 16) reads dims 32s + 8g .. +7 of key c)
//    conflict-free.
//  * PV is computed transposed too, O^T = V^T P^T with
//    v_mfma_f32_16x16x16_bf16: the four probabilities of a lane are exactly
//    its B operand (no shuffle) and the online-softmax rescale is
//    lane-local.  The V^T operand needs 4 keys of one dim per lane: it is
//    read from the V slab with one gfx950 transposing LDS load per 16-dim
//    tile.
//  * Software pipeline: while chunk c is computed, the K and V rows of chunk
//    c + 1 (in registers) and the route IDs of chunk c + 2 are in flight.
//    The IDs are issued before the rows and used one iteration later, so the
//    in-order load counter never makes the rows wait for them.
//  * Online softmax in fp32 with exp2 and the scale folded into log2(e).  The
//    reference max is raised only when a chunk exceeds it by more than 2^8,
//    so the accumulator rescale is skipped once the max has settled.
//    Probabilities are rounded to bf16 once; the same rounded values feed
//    both the PV product and the normaliser.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;   // work units per workgroup
constexpr int kChunk = 16;  // routes per inner iteration (M of S^T, K of PV)
constexpr float kMaxSlack = 8.0f;  // log2 headroom before the reference max is raised

template <int D>
struct Geometry {
  static constexpr int kSteps = D / 32;                 // QK^T k-steps of 32 dims
  static constexpr int kDimTiles = D / 16;              // O^T row tiles of 16 dims
  static constexpr int kLanesPerRow = D / 8;            // 16-byte pieces per V row
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kLoads = kChunk / kRowsPerLoad;  // V load instructions per chunk
  static constexpr int kStride = D + 16;                // V slab row stride in bf16 (2D + 32 bytes)
  static constexpr int kKStride = D + 8;                // K slab row stride in bf16 (2D + 16 bytes)
};

template <int D, bool kNarrow>
__global__ void __launch_bounds__(64 * kWaves)
    gather_attention_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                            const uint16_t* __restrict__ v, int64_t qs0, int64_t qs1, int64_t qs2,
                            int64_t ks0, int64_t ks1, int64_t ks2, int64_t vs0, int64_t vs1, int64_t vs2,
                            const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                            int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t K, int G,
                            float scale_log2e, int64_t n_units, uint16_t* __restrict__ out,
                            float* __restrict__ lse) {
  using Geo = Geometry<D>;
  __shared__ __attribute__((aligned(16))) uint16_t slab[kWaves][kChunk * Geo::kStride];
  __shared__ __attribute__((aligned(16))) uint16_t kslab[kWaves][kChunk * Geo::kKStride];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));  // wave-uniform
  // Workgroup x -> (KV head x % Hkv, four neighbouring rows): workgroups are
  // dealt round-robin to the 8 XCDs, so when Hkv divides 8 each XCD serves a
  // single KV head (half the K/V working set per L2 at Hkv = 2), while rows
  // still spread evenly over the XCDs.  Rows are taken from the last to the
  // first: with causal routes later rows route more keys, so the longest
  // rows start first and the short ones fill the end of the launch.
  const int64_t x = blockIdx.x;
  const int64_t hk = x % Hkv;
  const int64_t row = n_units / Hkv - 1 - ((x / Hkv) * kWaves + wave);  // b * S_q + i
  if (row < 0) return;  // the last workgroup's surplus waves; no workgroup barriers in this kernel
  const int64_t b = row / S_q;
  const int64_t i = row % S_q;
  const int c = lane & 15;  // head column of this lane; also key/dim row within a 16-tile
  const int g = lane >> 4;  // k-group of this lane
  const bool head_ok = c < G;
  uint16_t* out_row = out + (row * Hq + hk * G + c) * D;  // only dereferenced when head_ok

  const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
  if (n == 0) {  // empty route set: exactly +0.0 (and a log-sum-exp of -inf)
    if (head_ok) {
#pragma unroll
      for (int t = 0; t < Geo::kDimTiles; ++t)
        *reinterpret_cast<u32x2*>(out_row + 16 * t + 4 * g) = u32x2{0u, 0u};
      if (lse != nullptr && g == 0) lse[row * Hq + hk * G + c] = -INFINITY;
    }
    return;
  }

  // Q^T as the MFMA B operand: lane (c, g) holds head c, dims 32s + 8g .. +7.
  bf16x8 qf[Geo::kSteps];
  {
    const uint16_t* qp = q + b * qs0 + i * qs1 + (hk * G + (head_ok ? c : 0)) * qs2 + 8 * g;
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s)
      qf[s] = head_ok ? __builtin_bit_cast(bf16x8, load16(reinterpret_cast<const char*>(qp + 32 * s)))
                      : bf16x8{};
  }

  f32x4 acc[Geo::kDimTiles];
#pragma unroll
  for (int t = 0; t < Geo::kDimTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference max (log2 domain) of head c
  float l_run = 0.f;        // this lane's share of the running sum of head c

  const int32_t* lst = route_list + row * K;
  const int64_t ks1b = 2 * ks1, vs1b = 2 * vs1;  // row strides in bytes
  const char* kb = reinterpret_cast<const char*>(k + b * ks0 + hk * ks2) + 16 * (lane % Geo::kLanesPerRow);
  const char* vb = reinterpret_cast<const char*>(v + b * vs0 + hk * vs2) + 16 * (lane % Geo::kLanesPerRow);
  uint16_t* my_slab = slab[wave];
  uint16_t* my_kslab = kslab[wave];
  const int32_t id_max = static_cast<int32_t>(S_kv - 1);
  auto clamp_id = [&](int32_t x) { return min(max(x, 0), id_max); };
  // Raw route ID of key base + c (tails repeat the last route; clamped later).
  auto load_id = [&](int base) { return lst[min(base + c, n - 1)]; };
  // K rows of the chunk in 16-byte pieces, two full rows per load
  // instruction (the pattern the address unit handles best); they reach the
  // A operand of S^T = K Q^T through this wave's K slab.  Row r's ID lives in
  // lane r.
  auto load_k = [&](int32_t id, u32x4* kr) {
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int32_t idr = __shfl(id, u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow);
      kr[u] = load16(kb + RowOffset<kNarrow>::of(idr, ks1b));
    }
  };
  // V rows of the chunk in 16-byte pieces; row r's ID lives in lane r.
  auto load_v = [&](int32_t id, u32x4* vr) {
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int32_t idr = __shfl(id, u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow);
      vr[u] = load16(vb + RowOffset<kNarrow>::of(idr, vs1b));
    }
  };

  u32x4 kr[Geo::kLoads];
  u32x4 vr[Geo::kLoads];
  int32_t raw_next = load_id(kChunk);  // issued first: used after the rows below
  {
    const int32_t id0 = clamp_id(load_id(0));
    load_k(id0, kr);
    load_v(id0, vr);
  }
  int32_t id_next = clamp_id(raw_next);

  const uint16_t* tr = my_slab + (lane >> 2) * Geo::kStride + 4 * (lane & 3);
  for (int base = 0; base < n; base += kChunk) {
    const bool more = base + kChunk < n;  // wave-uniform

    // Stage this chunk's K and V rows in LDS (row-major, padded strides).
    wave_lds_sync();  // previous chunk's reads of both slabs are complete
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int r = u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow;
      const int col = 8 * (lane % Geo::kLanesPerRow);
      *reinterpret_cast<u32x4*>(my_kslab + r * Geo::kKStride + col) = kr[u];
      *reinterpret_cast<u32x4*>(my_slab + r * Geo::kStride + col) = vr[u];
    }
    wave_lds_sync();  // K and V rows visible to every lane of this wave

    // Scores: lane holds S^T[key 4g + r][head c]; the A operand is key c,
    // dims 32s + 8g .. +7 (row stride 2D + 16 bytes: conflict-free).
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* ka = my_kslab + c * Geo::kKStride + 8 * g;
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ka + 32 * s)),
                                                  qf[s], st, 0, 0, 0);

    // Prefetch: IDs two chunks ahead first, then the next chunk's K and V rows.
    if (more) {
      raw_next = load_id(base + 2 * kChunk);
      load_k(id_next, kr);
      load_v(id_next, vr);
    }

    // Online softmax (log2 domain) against a lazily raised reference max.
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = base + 4 * g + r < n ? st[r] * scale_log2e : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));      // finite: the chunk holds at least one key
    if (__ballot(mx > m_run + kMaxSlack)) {  // wave-uniform; always taken on the first chunk
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < Geo::kDimTiles; ++t) acc[t] *= alpha;
    }
    bf16x4 pf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pf[r] = static_cast<__bf16>(exp2f(x[r] - m_run));
      l_run += static_cast<float>(pf[r]);
    }
    const i16x4 pb = __builtin_bit_cast(i16x4, pf);

    // O^T += V^T P^T: one transposed LDS read gives lane (c, g) keys 4g..4g+3
    // of dim 16t + c, matching its four probabilities.
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr(tr + 16 * t), pb, acc[t], 0, 0, 0);

    if (more) id_next = clamp_id(raw_next);
  }

  // Normalise and store: lane holds O[head c][dims 16t + 4g .. +3].
  float l_tot = l_run + __shfl_xor(l_run, 16);  // butterfly over the four lane groups of head c
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  // Natural-log log-sum-exp of the scaled scores: the sum is taken against
  // the reference max m_run (log2 domain), from the same bf16-rounded
  // probabilities as the output.
  if (lse != nullptr && head_ok && g == 0) lse[row * Hq + hk * G + c] = (m_run + log2f(l_tot)) * kLn2;
  if (head_ok) {
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(acc[t][r] * inv);
      *reinterpret_cast<u32x2*>(out_row + 16 * t + 4 * g) = __builtin_bit_cast(u32x2, o);
    }
  }
}

template <int D, bool kNarrow>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const int64_t n_units = a.B * a.S_q * a.Hkv;
  const int64_t blocks = (a.B * a.S_q + kWaves - 1) / kWaves * a.Hkv;
  const float scale_log2e = a.scale * kLog2e;
  hipLaunchKernelGGL((gather_attention_kernel<D, kNarrow>), dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWaves),
                     0, stream, a.q, a.k, a.v, a.qs[0], a.qs[1], a.qs[2], a.ks[0], a.ks[1], a.ks[2], a.vs[0],
                     a.vs[1], a.vs[2], a.route_list, a.route_count, a.S_q, a.S_kv, a.Hq, a.Hkv, a.K,
                     static_cast<int>(a.Hq / a.Hkv), scale_log2e, n_units, a.out, a.lse);
  return hipGetLastError();
}

// True when (S_kv - 1) * row stride + one row fits in 32 bits for both K and V.
bool narrow_offsets(const AttnArgs& a) {
  const int64_t lim = (int64_t{1} << 32) - 1;
  if (a.ks[1] < 0 || a.vs[1] < 0) return false;
  return (a.S_kv - 1) * a.ks[1] * 2 + 2 * a.D <= lim && (a.S_kv - 1) * a.vs[1] * 2 + 2 * a.D <= lim;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  return narrow_offsets(a) ? launch<D, true>(a, stream) : launch<D, false>(a, stream);
}

}  // namespace

hipError_t launch_gather_attention(const AttnArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    case 256: return launch_d<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa

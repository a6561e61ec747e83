// Backward pass of route-sparse GQA attention for gfx950 over compacted
// route lists.
//
// Definition: fa4_qsa page (the FA4 kernel owns first-order autograd of this
// attention) and flex_qsa page, module description (rows whose routes are all
// invalid have zero output and zero gradients).  For a (b, i, h) with a
// non-empty route set R, hk = h / G and p = softmax over j in R of
// s_j = scale <q, k_j>:
//   dp_j  = <dO, v_j>,   delta = <dO, O> = sum_j p_j dp_j,
//   ds_j  = p_j (dp_j - delta),
//   dq    = scale sum_j ds_j k_j,
//   dk_j += scale ds_j q,     dv_j += p_j dO     (over every (i, h) routing j).
// p is recomputed from the forward's log-sum-exp: p_j = exp(s_j - lse).
//
// Two kernels, both deterministic (each sum is taken in a fixed order; no
// floating-point atomics), which is the part the pages leave unsupported (the
// second lives in dkdv.hip, built with its MFMA accumulators in AGPRs):
//  * dq_kernel: one wavefront per (b, i, hk) unit, mapped like the forward
//    (one KV head per XCD).  It gathers the unit's routed K and V rows in
//    16-key chunks through the wave's LDS slabs, recomputes S^T = K Q^T and
//    dP^T = V dO^T with v_mfma_f32_16x16x32_bf16 (heads on the N side, so
//    every per-head statistic is lane-local), forms dS^T, and accumulates
//    dQ^T += K^T dS^T with v_mfma_f32_16x16x16_bf16, reading K^T with the
//    transposing LDS load.  It also writes delta for the second kernel.
//  * dkdv_kernel: one workgroup per (part of a 64-key tile's segment list,
//    hk); wave w owns keys 16w .. 16w+15 of the tile, whose K and V rows
//    stay in registers as MFMA B operands.  The workgroup walks its key
//    segments (query rows that route at least one key of the tile, in
//    ascending row order, each with a 64-bit mask of the keys it routes) in
//    batches of floor(16 / G) rows whose G heads fill the 16 MFMA rows.  Per
//    batch the workgroup stages Q and dO of those rows once in LDS for all
//    four waves (double-buffered: the next batch's loads are in flight while
//    this one is computed); each wave recomputes S = Q K^T and dP = dO V^T
//    for its keys and accumulates dV^T += dO^T P and dK^T += Q^T dS, or
//    skips the batch when it routes none of them.  A tile whose list was cut
//    into several parts (popular keys) writes fp32 partial sums, which
//    dkdv_reduce_kernel adds in part order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "backward_geometry.h"
#include "device_common.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

using bwd::Geo;
using bwd::kChunk;
using bwd::kWaves;

// ---------------------------------------------------------------------------
// dq (and delta)
// ---------------------------------------------------------------------------

struct DqArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, gs0, gs1, gs2;
  const float* lse;
  const int32_t* route_list;
  const int32_t* route_count;
  int64_t S_q, S_kv, Hq, Hkv, K;
  int G;
  float scale_log2e, scale;
  int64_t n_rows;
  uint16_t* dq;
  float* delta;
  // key-range split (as the forward's): range starts, this pass's rows and fp32 partial sums
  const int32_t* offs;
  int P;
  int64_t row0, pass_rows;
  float* part;  // [pass_rows][Hkv][P][G][D]
  // the pass whose partial sums are added up (by dq_combine_kernel, or by the
  // combine workgroups interleaved into the next pass's split launch)
  int64_t comb_row0, comb_pass_rows;
  const float* comb_part;
  int64_t comb_blocks, comb_stride;  // split launch: workgroup comb_stride * k - 1 adds unit k - 1
};

// Adds the fp32 partial dq of one (row, KV head) unit's ranges in ascending
// range order and writes scale x the sum as bf16 (one wavefront): lane L
// takes the 4-element pieces L, L + 64, .. (kP of them) of the unit's G x D
// values; the ranges are read kB at a time with all their loads in flight
// together (16 16-byte loads per lane at D = 256, fewer below, which keeps
// the split dq kernel within the registers it needs anyway).  Rows with
// routes in at most one range were written by dq_kernel.
template <int D, int kP>
__device__ __forceinline__ void dq_combine_unit(const DqArgs& a, int64_t unit, int lane) {
  constexpr int kSlots = D == 256 ? 16 : D == 128 ? 8 : 4;  // 16-byte loads per lane per batch
  constexpr int kB = kSlots / kP > 0 ? kSlots / kP : 1;        // ranges per batch
  const int64_t local = unit / a.Hkv, hk = unit - local * a.Hkv;
  const int64_t row = a.comb_row0 + local;
  int lo_l, hi_l;
  uint64_t parts = range_parts(a.offs + row * (a.P + 1), a.P, a.K, lane, &lo_l, &hi_l);
  if (__builtin_popcountll(parts) < 2) return;
  const int n_pieces = a.G * D / 4;
  const float* base = a.comb_part + (local * a.Hkv + hk) * a.P * a.G * D;
  f32x4 acc[kP];
#pragma unroll
  for (int k = 0; k < kP; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  while (parts != 0) {  // wave-uniform
    int pr[kB];  // this batch's ranges, ascending; -1 past the unit's last
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      pr[j] = parts != 0 ? __builtin_ctzll(parts) : -1;
      parts &= parts - 1;
    }
    f32x4 v[kB][kP];
#pragma unroll
    for (int j = 0; j < kB; ++j)
#pragma unroll
      for (int k = 0; k < kP; ++k) {
        const int piece = lane + 64 * k;
        if (pr[j] >= 0 && piece < n_pieces) {
          const f32x4* src = reinterpret_cast<const f32x4*>(base + static_cast<int64_t>(pr[j]) * a.G * D + 4 * piece);
          v[j][k] = __builtin_nontemporal_load(src);  // read once: streamed
        }
      }
#pragma unroll
    for (int j = 0; j < kB; ++j)
#pragma unroll
      for (int k = 0; k < kP; ++k)
        if (pr[j] >= 0 && lane + 64 * k < n_pieces) acc[k] += v[j][k];
  }
  uint16_t* dst = a.dq + (row * a.Hq + hk * a.G) * D;
#pragma unroll
  for (int k = 0; k < kP; ++k) {
    const int piece = lane + 64 * k;
    if (piece < n_pieces) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = static_cast<__bf16>(acc[k][r] * a.scale);
      *reinterpret_cast<u32x2*>(dst + 4 * piece) = __builtin_bit_cast(u32x2, w);
    }
  }
}

// dq_combine_unit with kP = the pieces each lane needs, G * D / 256 rounded
// up to a power of two (at most D / 16, at G = 16).
template <int D>
__device__ __forceinline__ void dq_combine_unit(const DqArgs& a, int64_t unit, int lane) {
  if (unit >= a.comb_pass_rows * a.Hkv) return;
  const int per_lane = (a.G * D / 4 + 63) / 64;
  if constexpr (D / 16 >= 16) {
    if (per_lane > 8) return dq_combine_unit<D, 16>(a, unit, lane);
  }
  if constexpr (D / 16 >= 8) {
    if (per_lane > 4) return dq_combine_unit<D, 8>(a, unit, lane);
  }
  if (per_lane > 2) return dq_combine_unit<D, 4>(a, unit, lane);
  if (per_lane > 1) return dq_combine_unit<D, 2>(a, unit, lane);
  dq_combine_unit<D, 1>(a, unit, lane);
}

// delta = <dO, O> per (row, head), for the split dq kernel (whose units each
// see only part of a row) and the dk/dv kernel: one wavefront per (row, KV
// head), lane (c, g) summing dims 32s + 8g .. +7 of head c.
template <int D>
__global__ void __launch_bounds__(64 * kWaves) delta_kernel(const DqArgs a) {
  using Gm = Geo<D>;
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (unit >= a.n_rows * a.Hkv) return;
  const int64_t row = unit / a.Hkv, hk = unit - row * a.Hkv;
  const int64_t b = row / a.S_q, i = row - b * a.S_q;
  const int c = lane & 15, g = lane >> 4;
  const bool head_ok = c < a.G;
  const int64_t hq = hk * a.G + (head_ok ? c : 0);
  const uint16_t* gp = a.dout + b * a.gs0 + i * a.gs1 + hq * a.gs2 + 8 * g;
  const uint16_t* op = a.o + (row * a.Hq + hq) * D + 8 * g;
  float dl = 0.f;
#pragma unroll
  for (int s = 0; s < Gm::kSteps; ++s) {
    const u32x4 gw = head_ok ? load16(gp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 ow = head_ok ? load16(op + 32 * s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) dl += bf16_lo(gw[e]) * bf16_lo(ow[e]) + bf16_hi(gw[e]) * bf16_hi(ow[e]);
  }
  dl = pair_sum16(dl);
  dl = pair_sum32(dl);
  if (head_ok && g == 0) a.delta[row * a.Hq + hq] = dl;
}

// dq over a row's routes (unsplit: one unit per (row, KV head), which also
// forms delta), or over one key range of them (kSplit: units ordered range by
// range as in the forward's split, delta from delta_kernel; a unit whose row
// has routes in no other range writes dq, otherwise an fp32 partial sum that
// dq_combine_unit adds in ascending range order, in the next pass's launch or
// on its own after the last pass).
// One wavefront per workgroup, as the forward's attention kernel: a unit's
// slot and LDS are released as soon as the unit ends.
template <int D, bool kNarrow, bool kSplit>
__global__ void __launch_bounds__(64) dq_kernel(const DqArgs a) {
  using Gm = Geo<D>;
  __shared__ __attribute__((aligned(16))) uint16_t kslab[kChunk * Gm::kTrStride];
  __shared__ __attribute__((aligned(16))) uint16_t vslab[kChunk * Gm::kRowStride];

  const int64_t S_q = a.S_q, Hq = a.Hq, Hkv = a.Hkv;
  const int G = a.G;
  const int lane = threadIdx.x & 63;
  int64_t x = blockIdx.x;
  int64_t hk, row, local = 0;
  int p = 0;
  if constexpr (kSplit) {
    // Every comb_stride-th workgroup adds up one unit of the previous pass
    // instead, spread evenly over the launch; the others keep their order.
    if (a.comb_blocks > 0) {
      const int64_t k1 = (x + 1) / a.comb_stride;
      if (k1 * a.comb_stride == x + 1 && k1 <= a.comb_blocks) {
        dq_combine_unit<D>(a, k1 - 1, lane);
        return;
      }
      x -= min(x / a.comb_stride, a.comb_blocks);
    }
  }
  if constexpr (!kSplit) {
    hk = x % Hkv;  // one KV head per XCD, as in the forward
    // Rows from the last to the first, as in the forward: with causal routes the longest start first.
    row = a.n_rows - 1 - x / Hkv;
  } else {
    const int64_t phase = x / a.pass_rows;  // (range p, KV head hk), rows last to first
    p = static_cast<int>(phase / Hkv);
    hk = phase - static_cast<int64_t>(p) * Hkv;
    local = a.pass_rows - 1 - (x - phase * a.pass_rows);
    row = a.row0 + local;
  }
  const int64_t b = row / S_q;
  const int64_t i = row % S_q;
  const int c = lane & 15;  // head column (N side); key / dim row within a 16-tile
  const int g = lane >> 4;
  const bool head_ok = c < G;
  const int64_t hq = hk * G + (head_ok ? c : 0);
  uint16_t* dq_row = a.dq + (row * Hq + hk * G + c) * D;  // only dereferenced when head_ok

  int first = 0, n;
  bool direct = true;
  if constexpr (!kSplit) {
    n = static_cast<int>(min(max(static_cast<int64_t>(a.route_count[row]), int64_t{0}), a.K));
  } else {
    int lo_l, hi_l;
    const uint64_t parts = range_parts(a.offs + row * (a.P + 1), a.P, a.K, lane, &lo_l, &hi_l);
    if (((parts >> p) & 1u) == 0) {
      if (!(parts == 0 && p == 0)) return;  // nothing in this range; an empty row is written once, below
      n = 0;
    } else {
      first = __shfl(lo_l, p);
      n = __shfl(hi_l, p) - first;
      direct = __builtin_popcountll(parts) == 1;
    }
  }
  if (n == 0) {  // empty route set: zero gradient, nothing reaches dk / dv
    if (head_ok) {
#pragma unroll
      for (int t = 0; t < Gm::kDimTiles; ++t)
        *reinterpret_cast<u32x2*>(dq_row + 16 * t + 4 * g) = u32x2{0u, 0u};
      if (!kSplit && g == 0) a.delta[row * Hq + hk * G + c] = 0.f;
    }
    return;
  }

  // Q^T and dO^T as MFMA B operands: lane (c, g) holds head c, dims 32s + 8g .. +7.
  bf16x8 qf[Gm::kSteps], gf[Gm::kSteps];
  float dl = 0.f;  // delta = <dO, O> for head c
  {
    const uint16_t* qp = a.q + b * a.qs0 + i * a.qs1 + hq * a.qs2 + 8 * g;
    const uint16_t* gp = a.dout + b * a.gs0 + i * a.gs1 + hq * a.gs2 + 8 * g;
    const uint16_t* op = a.o + (row * Hq + hq) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < Gm::kSteps; ++s) {
      const u32x4 qw = head_ok ? load16(qp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 gw = head_ok ? load16(gp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, qw);
      gf[s] = __builtin_bit_cast(bf16x8, gw);
      if constexpr (!kSplit) {
        const u32x4 ow = head_ok ? load16(op + 32 * s) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) dl += bf16_lo(gw[e]) * bf16_lo(ow[e]) + bf16_hi(gw[e]) * bf16_hi(ow[e]);
      }
    }
  }
  if constexpr (!kSplit) {
    dl = pair_sum16(dl);
    dl = pair_sum32(dl);
    if (head_ok && g == 0) a.delta[row * Hq + hq] = dl;
  } else {
    dl = head_ok ? a.delta[row * Hq + hq] : 0.f;
  }
  const float lse2 = head_ok ? a.lse[row * Hq + hq] * kLog2e : 0.f;

  f32x4 acc[Gm::kDimTiles];
#pragma unroll
  for (int t = 0; t < Gm::kDimTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* lst = a.route_list + row * a.K + first;
  const int64_t ks1b = 2 * a.ks1, vs1b = 2 * a.vs1;
  const char* kb = reinterpret_cast<const char*>(a.k + b * a.ks0 + hk * a.ks2) + 16 * (lane % Gm::kLanesPerRow);
  const char* vb = reinterpret_cast<const char*>(a.v + b * a.vs0 + hk * a.vs2) + 16 * (lane % Gm::kLanesPerRow);
  uint16_t* my_k = kslab;
  uint16_t* my_v = vslab;
  const int32_t id_max = static_cast<int32_t>(a.S_kv - 1);
  auto clamp_id = [&](int32_t xid) { return min(max(xid, 0), id_max); };
  auto load_id = [&](int base) { return lst[min(base + c, n - 1)]; };
  // K and V rows of a chunk; on the 32-bit path K and V share their row
  // stride, so one offset serves both.
  auto load_kv = [&](int32_t id, u32x4* kr, u32x4* vr) {
    int32_t idr[Gm::kLoads];
#pragma unroll
    for (int u = 0; u < Gm::kLoads; ++u) {
      idr[u] = chunk_row_id<Gm::kRowsPerLoad>(id, u, lane);
      kr[u] = load16(kb + RowOffset<kNarrow>::of(idr[u], ks1b));
    }
#pragma unroll
    for (int u = 0; u < Gm::kLoads; ++u) {
      if constexpr (kNarrow)
        vr[u] = load16(vb + RowOffset<true>::of(idr[u], ks1b));
      else
        vr[u] = load16(vb + RowOffset<false>::of(idr[u], vs1b));
    }
  };

  u32x4 kr[Gm::kLoads], vr[Gm::kLoads];
  int32_t raw_next = load_id(kChunk);
  {
    const int32_t id0 = clamp_id(load_id(0));
    load_kv(id0, kr, vr);
  }
  int32_t id_next = clamp_id(raw_next);

  const uint16_t* ktr = my_k + (lane >> 2) * Gm::kTrStride + 4 * (lane & 3);
  for (int base = 0; base < n; base += kChunk) {
    const bool more = base + kChunk < n;

    wave_lds_sync();  // the previous chunk's slab reads are complete
#pragma unroll
    for (int u = 0; u < Gm::kLoads; ++u) {
      const int r = u * Gm::kRowsPerLoad + lane / Gm::kLanesPerRow;
      const int col = 8 * (lane % Gm::kLanesPerRow);
      *reinterpret_cast<u32x4*>(my_k + r * Gm::kTrStride + col) = kr[u];
      *reinterpret_cast<u32x4*>(my_v + r * Gm::kRowStride + col) = vr[u];
    }
    // Prefetch as soon as the rows are staged: IDs two chunks ahead, then the next chunk's rows.
    if (more) {
      raw_next = load_id(base + 2 * kChunk);
      load_kv(id_next, kr, vr);
    }
    wave_lds_sync();

    // S^T[key 4g + r][head c] and dP^T[key 4g + r][head c]; A operands are
    // rows of the slabs (key c, dims 32s + 8g .. +7).
    f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* ka = my_k + c * Gm::kTrStride + 8 * g;
    const uint16_t* va = my_v + c * Gm::kRowStride + 8 * g;
#pragma unroll
    for (int s = 0; s < Gm::kSteps; ++s) {
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, load16(ka + 32 * s)), qf[s], st, 0, 0, 0);
      dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, load16(va + 32 * s)), gf[s], dpt, 0, 0,
                                                    0);
    }

    // dS^T = P^T (dP^T - delta), P^T = exp2(S^T scale log2e - lse2); keys past n
    // (the repeated tail) and padded heads contribute nothing.
    bf16x4 dsb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool on = head_ok && base + 4 * g + r < n;
      const float pr = on ? __builtin_amdgcn_exp2f(st[r] * a.scale_log2e - lse2) : 0.f;  // hardware exp2
      dsb[r] = static_cast<__bf16>(pr * (dpt[r] - dl));
    }
    const i16x4 db = __builtin_bit_cast(i16x4, dsb);

    // dQ^T += K^T dS^T: the transposed read gives lane (c, g) keys 4g .. 4g+3 of dim 16t + c.
#pragma unroll
    for (int t = 0; t < Gm::kDimTiles; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr(ktr + 16 * t), db, acc[t], 0, 0, 0);

    if (more) id_next = clamp_id(raw_next);
  }

  if (head_ok) {
    if (direct) {
#pragma unroll
      for (int t = 0; t < Gm::kDimTiles; ++t) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = static_cast<__bf16>(acc[t][r] * a.scale);
        *reinterpret_cast<u32x2*>(dq_row + 16 * t + 4 * g) = __builtin_bit_cast(u32x2, w);
      }
    } else {  // fp32 partial sum [G][D] of this range, unscaled
      float* dst = a.part + (((local * Hkv + hk) * a.P + p) * G + c) * D;
#pragma unroll
      for (int t = 0; t < Gm::kDimTiles; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * g) = acc[t];
    }
  }
}

// The combine of one pass on its own: one wavefront per (row, KV head) unit.
template <int D>
__global__ void __launch_bounds__(64 * kWaves) dq_combine_kernel(const DqArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  dq_combine_unit<D>(a, static_cast<int64_t>(blockIdx.x) * kWaves + wave, threadIdx.x & 63);
}

// True when K and V share a non-negative row stride and every row fits 32-bit
// byte offsets from its (batch, head) base.
bool narrow_offsets(const BwdArgs& a) {
  const int64_t lim = (int64_t{1} << 32) - 1;
  if (a.ks[1] < 0 || a.vs[1] != a.ks[1]) return false;  // one offset serves K and V
  return (a.S_kv - 1) * a.ks[1] * 2 + 2 * a.D <= lim && (a.S_kv - 1) * a.vs[1] * 2 + 2 * a.D <= lim;
}

template <int D, bool kNarrow>
hipError_t launch_dq_d(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = a.B * a.S_q;
  DqArgs k{};
  k.q = a.q; k.k = a.k; k.v = a.v; k.o = a.out; k.dout = a.dout;
  k.qs0 = a.qs[0]; k.qs1 = a.qs[1]; k.qs2 = a.qs[2];
  k.ks0 = a.ks[0]; k.ks1 = a.ks[1]; k.ks2 = a.ks[2];
  k.vs0 = a.vs[0]; k.vs1 = a.vs[1]; k.vs2 = a.vs[2];
  k.gs0 = a.gs[0]; k.gs1 = a.gs[1]; k.gs2 = a.gs[2];
  k.lse = a.lse;
  k.route_list = a.route_list;
  k.route_count = a.route_count;
  k.S_q = a.S_q; k.S_kv = a.S_kv; k.Hq = a.Hq; k.Hkv = a.Hkv; k.K = a.K;
  k.G = static_cast<int>(a.Hq / a.Hkv);
  k.scale_log2e = a.scale * kLog2e;
  k.scale = a.scale;
  k.n_rows = rows;
  k.dq = a.dq;
  k.delta = a.delta;
  if (!a.split.use) {
    hipLaunchKernelGGL((dq_kernel<D, kNarrow, false>), dim3(static_cast<uint32_t>(rows * a.Hkv)), dim3(64), 0,
                       stream, k);
    return hipGetLastError();
  }
  hipError_t e = launch_range_offsets(a.route_list, a.route_count, rows, a.K, a.S_kv, a.split, a.offs, stream);
  if (e != hipSuccess) return e;
  const uint32_t unit_blocks = static_cast<uint32_t>((rows * a.Hkv + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((delta_kernel<D>), dim3(unit_blocks), dim3(64 * kWaves), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k.offs = a.offs;
  k.P = a.split.P;
  // Passes from the last rows to the first; each pass's split launch also
  // adds up the previous pass's partial sums, from the other of the two
  // partial buffers, and the last pass is added up on its own.
  const int64_t n_pass = (rows + a.dq_pass_rows - 1) / a.dq_pass_rows;
  for (int64_t i = 0; i <= n_pass; ++i) {
    if (i > 0) {  // the previous pass, to be added up
      k.comb_row0 = k.row0;
      k.comb_pass_rows = k.pass_rows;
      k.comb_part = k.part;
    }
    const int64_t comb_units = i > 0 ? k.comb_pass_rows * a.Hkv : 0;
    if (i == n_pass) {
      hipLaunchKernelGGL((dq_combine_kernel<D>), dim3(static_cast<uint32_t>((comb_units + kWaves - 1) / kWaves)),
                         dim3(64 * kWaves), 0, stream, k);
      return hipGetLastError();
    }
    const int64_t r_end = rows - i * a.dq_pass_rows;
    k.row0 = std::max<int64_t>(r_end - a.dq_pass_rows, 0);
    k.pass_rows = r_end - k.row0;
    k.part = a.dq_part[i & 1];
    const int64_t split_blocks = k.pass_rows * a.split.P * a.Hkv;
    k.comb_blocks = comb_units;
    k.comb_stride = comb_units > 0 ? (split_blocks + comb_units) / comb_units : 0;
    hipLaunchKernelGGL((dq_kernel<D, kNarrow, true>), dim3(static_cast<uint32_t>(split_blocks + comb_units)),
                       dim3(64), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_dq_any(const BwdArgs& a, hipStream_t stream) {
  return narrow_offsets(a) ? launch_dq_d<D, true>(a, stream) : launch_dq_d<D, false>(a, stream);
}

}  // namespace

hipError_t launch_attention_dq(const BwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_dq_any<64>(a, stream);
    case 128: return launch_dq_any<128>(a, stream);
    case 256: return launch_dq_any<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa

// Fused gather-attention for gfx950 over compacted route lists.
//
// Definition: flex_qsa page, `flex_sparse_gqa_attention` and module
// description (each query row attends exactly to its routes, empty rows give
// zero); fa4_qsa page, `fa4_sparse_gqa_attention` (no extra mask; BF16);
// qsa page, `_gathered_qsa_gqa_attention_chunk` (grouped layout
// [B, Q, Hkv, G, D]: query head h reads KV head h / G).
//
// Design (one wavefront per (b, i, hk) work unit and per workgroup, mapped
// so that each XCD serves one KV head, rows taken from the last to the
// first):
//  * The G query heads of the unit are the N = 16 columns of the MFMA (zero
//    padded when G < 16).  Scores are computed transposed, S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16, 16 routed keys as the M rows, so each lane
//    ends up owning one head and four keys; a head's max and sum over its
//    four lane groups are two gfx950 lane swaps (permlane16 and permlane32).
//    Routed K and V rows are both gathered two full rows
//    per 16-byte-per-lane load instruction (fewest cache lines per
//    instruction for the address unit) and staged in this wave's LDS slabs;
//    both slabs have a 2D + 32 byte row stride, with which the bank-conflict
//    counter reads zero for the row stores, the A-operand reads (lane
//    (c, g) = (lane % 16, lane / 16) reads dims 32s + 8g .. +7 of key c) and
//    the transposing V reads.
//  * PV is computed transposed too, O^T = V^T P^T with
//    v_mfma_f32_16x16x16_bf16: the four probabilities of a lane are exactly
//    its B operand (no shuffle) and the online-softmax rescale is
//    lane-local.  The V^T operand needs 4 keys of one dim per lane: it is
//    read from the V slab with one gfx950 transposing LDS load per 16-dim
//    tile.
//  * Software pipeline: while chunk c is computed, the K and V rows of chunk
//    c + 1 (in registers) and the route IDs of chunk c + 2 are in flight.
//    The IDs are issued before the rows and used one iteration later, so the
//    in-order load counter never makes the rows wait for them.  Within a
//    chunk the LDS sees, in order: the K rows' writes, the score operands'
//    reads, the V rows' writes (LDS operations of a wave run in order, so
//    the operand reads wait only for the K writes), and the next chunk's
//    loads are issued right after, with their row IDs taken by lane reads
//    rather than LDS permutes.
//  * Online softmax in fp32 with exp2 and the scale folded into log2(e).  The
//    reference max is raised only when a chunk exceeds it by more than 2^8,
//    so the accumulator rescale is skipped once the max has settled.
//    Probabilities are rounded to bf16 once; the same rounded values feed
//    both the PV product and the normaliser.
//
// Key-range split (kSplit), for key ranges larger than an XCD's L2: a work
// unit is (row, KV head, key range [pW, (p+1)W)); the unit's part of the
// row's ascending list is [offs[p], offs[p+1]) of the range-start table.
// Workgroups are ordered range-major, so at any time every XCD gathers from
// one W-key range of one KV head (4 MiB of K and V).  A unit whose row has
// routes in no other range writes the output itself; otherwise it writes
// its normalised partial output (bf16) and the log2 of its softmax sum
// against its own maximum, and `combine_unit` merges the partials of the row
// in ascending range order:
//   out = sum_p 2^(s_p - M) o_p / sum_p 2^(s_p - M),  M = max_p s_p,
// which is the softmax over the union of the ranges (the ranges partition
// the row's route set).  The rows go in passes (partials of one pass in
// workspace), last rows first; the workgroups merging a pass are spread
// through the next pass's split launch, which writes the other of two
// partial buffers, and `range_combine_kernel` merges the last pass.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kWaves = 4;   // wavefronts per workgroup of the range-start and combine kernels
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
  static constexpr int kKStride = D + 16;               // K slab row stride in bf16 (2D + 32 bytes)
};

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2;
  const int32_t* route_list;
  const int32_t* route_count;
  int64_t S_q, S_kv, Hq, Hkv, K;
  int G;
  float scale_log2e;
  int64_t n_units;  // unsplit: B * S_q * Hkv
  uint16_t* out;
  float* lse;
  // key-range split
  const int32_t* offs;  // [B * S_q][P + 1] range starts within each row's list
  int P;
  int64_t row0, pass_rows;             // rows [row0, row0 + pass_rows) of this pass
  uint16_t* part_o;                    // [pass_rows][Hkv][P][G][D] bf16
  float* part_lse;                     // [pass_rows][Hkv][P][G] fp32, log2 domain
  // the pass whose partials are merged (by the combine kernel, or by the
  // combine workgroups interleaved into the next pass's split launch)
  int64_t comb_row0, comb_pass_rows;
  const uint16_t* comb_part_o;
  const float* comb_part_lse;
  int64_t comb_blocks, comb_stride;  // split launch: workgroup comb_stride * k - 1 merges unit k - 1
};

// Merges the partial results of one (row, KV head) unit of a split pass
// (one wavefront): lane L takes the 8-element pieces L, L + 64, .. (kP of
// them) of the unit's G x D outputs.  The unit's ranges are taken in
// ascending order, kB at a time with all their loads in flight together (16
// 16-byte loads per lane at D = 256, 4 below: the split kernel then needs no
// more registers than its gather), and folded into a running sum against
// the largest log2-sum-exp seen so far:
//   out = sum_p 2^(s_p - M) o_p / sum_p 2^(s_p - M),  M = max_p s_p.
// Rows with routes in at most one range were written by the split kernel and
// are skipped.
template <int D, int kP>
__device__ __forceinline__ void combine_unit(const KernelArgs& a, int64_t unit, int lane) {
  constexpr int kB = (D == 256 ? 16 : 4) / kP;  // ranges per batch
  const int64_t local = unit / a.Hkv;
  const int64_t hk = unit - local * a.Hkv;
  const int64_t row = a.comb_row0 + local;
  const int G = a.G;
  int lo_l, hi_l;
  uint64_t parts = range_parts(a.offs + row * (a.P + 1), a.P, a.K, lane, &lo_l, &hi_l);
  if (__builtin_popcountll(parts) < 2) return;

  const int n_pieces = G * D / 8;
  const int64_t u0 = (local * a.Hkv + hk) * a.P;  // partial index of range 0 of this unit
  float mx[kP], wsum[kP];
  float acc[kP][8];
#pragma unroll
  for (int k = 0; k < kP; ++k) {
    mx[k] = -INFINITY;
    wsum[k] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  }
  while (parts != 0) {  // wave-uniform
    int pr[kB];  // this batch's ranges, ascending; -1 past the unit's last
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      pr[j] = parts != 0 ? __builtin_ctzll(parts) : -1;
      parts &= parts - 1;
    }
    float ls[kB][kP];
    u32x4 v[kB][kP];
#pragma unroll
    for (int j = 0; j < kB; ++j)
#pragma unroll
      for (int k = 0; k < kP; ++k) {
        const int piece = lane + 64 * k;
        if (pr[j] >= 0 && piece < n_pieces) {
          const int64_t u = u0 + pr[j];
          ls[j][k] = a.comb_part_lse[u * G + piece * 8 / D];
          const u32x4* src = reinterpret_cast<const u32x4*>(a.comb_part_o + (u * G * D + piece * 8));
          v[j][k] = __builtin_nontemporal_load(src);  // read once: streamed
        }
      }
#pragma unroll
    for (int k = 0; k < kP; ++k) {
      if (lane + 64 * k >= n_pieces) continue;
      float bm = ls[0][k];  // pr[0] >= 0: the batch holds at least one range
#pragma unroll
      for (int j = 1; j < kB; ++j)
        if (pr[j] >= 0) bm = fmaxf(bm, ls[j][k]);
      const float m_new = fmaxf(mx[k], bm);
      const float alpha = exp2f(mx[k] - m_new);  // 0 on the first batch
      mx[k] = m_new;
      wsum[k] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][e] *= alpha;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (pr[j] < 0) continue;
        const float w = exp2f(ls[j][k] - m_new);
        wsum[k] += w;
        const uint32_t words[4] = {v[j][k].x, v[j][k].y, v[j][k].z, v[j][k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[k][2 * e] += w * bf16_lo(words[e]);
          acc[k][2 * e + 1] += w * bf16_hi(words[e]);
        }
      }
    }
  }
  uint16_t* out_unit = a.out + (row * a.Hq + hk * G) * D;
#pragma unroll
  for (int k = 0; k < kP; ++k) {
    const int piece = lane + 64 * k;
    if (piece < n_pieces) {
      const float inv = 1.0f / wsum[k];
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(acc[k][e] * inv);
      *reinterpret_cast<u32x4*>(out_unit + piece * 8) = __builtin_bit_cast(u32x4, o);
      if (a.lse != nullptr && (piece * 8) % D == 0)
        a.lse[row * a.Hq + hk * G + piece * 8 / D] = (mx[k] + log2f(wsum[k])) * kLn2;
    }
  }
}

// combine_unit with kP = the pieces each lane needs, G * D / 512 rounded up
// to a power of two (at most D / 32, at G = 16).
template <int D>
__device__ __forceinline__ void combine_unit(const KernelArgs& a, int64_t unit, int lane) {
  if (unit >= a.comb_pass_rows * a.Hkv) return;
  const int per_lane = (a.G * D / 8 + 63) / 64;
  if constexpr (D / 32 >= 8) {
    if (per_lane > 4) return combine_unit<D, 8>(a, unit, lane);
  }
  if constexpr (D / 32 >= 4) {
    if (per_lane > 2) return combine_unit<D, 4>(a, unit, lane);
  }
  if (per_lane > 1) return combine_unit<D, 2>(a, unit, lane);
  combine_unit<D, 1>(a, unit, lane);
}

// One wavefront per workgroup: a unit's workgroup slot and LDS are released
// as soon as its unit ends, and the CU starts the next unit at once.  (Four
// units per workgroup held the slots of all four until the longest ended;
// within one key range the units of neighbouring rows differ widely in
// length.)
template <int D, bool kNarrow, bool kSplit>
__global__ void __launch_bounds__(64) gather_attention_kernel(const KernelArgs a) {
  using Geo = Geometry<D>;
  __shared__ __attribute__((aligned(16))) uint16_t slab[kChunk * Geo::kStride];
  __shared__ __attribute__((aligned(16))) uint16_t kslab[kChunk * Geo::kKStride];

  const int64_t S_q = a.S_q, Hq = a.Hq, Hkv = a.Hkv;
  const int G = a.G;
  const int lane = threadIdx.x & 63;
  int64_t x = blockIdx.x;
  int64_t hk, row, local = 0;
  int p = 0;
  if constexpr (kSplit) {
    // Every comb_stride-th workgroup merges one unit of the previous pass
    // instead, spread evenly over the launch; the others keep their order.
    if (a.comb_blocks > 0) {
      const int64_t k1 = (x + 1) / a.comb_stride;
      if (k1 * a.comb_stride == x + 1 && k1 <= a.comb_blocks) {
        combine_unit<D>(a, k1 - 1, lane);
        return;
      }
      x -= min(x / a.comb_stride, a.comb_blocks);
    }
  }
  if constexpr (!kSplit) {
    // Workgroup x -> (KV head x % Hkv, row): workgroups are dealt round-robin
    // to the 8 XCDs, so when Hkv divides 8 each XCD serves a single KV head
    // (half the K/V working set per L2 at Hkv = 2), while rows still spread
    // evenly over the XCDs.  Rows are taken from the last to the first: with
    // causal routes later rows route more keys, so the longest rows start
    // first and the short ones fill the end of the launch.
    hk = x % Hkv;
    row = a.n_units / Hkv - 1 - x / Hkv;  // b * S_q + i
  } else {
    // Workgroup x -> phase x / pass_rows = (range p, KV head hk), then a row
    // of the pass, last rows first.  Consecutive workgroups go to all XCDs in
    // turn, so the XCDs sweep the phases together.
    const int64_t phase = x / a.pass_rows;
    p = static_cast<int>(phase / Hkv);
    hk = phase - static_cast<int64_t>(p) * Hkv;
    local = a.pass_rows - 1 - (x - phase * a.pass_rows);
    row = a.row0 + local;
  }
  const int64_t b = row / S_q;
  const int64_t i = row % S_q;
  const int c = lane & 15;  // head column of this lane; also key/dim row within a 16-tile
  const int g = lane >> 4;  // k-group of this lane
  const bool head_ok = c < G;
  uint16_t* out_row = a.out + (row * Hq + hk * G + c) * D;  // only dereferenced when head_ok

  int first = 0, n;  // this unit's part of the row's list: [first, first + n)
  bool direct = true;  // the unit writes the output (not a partial)
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
  if (n == 0) {  // empty route set: exactly +0.0 (and a log-sum-exp of -inf)
    if (head_ok) {
#pragma unroll
      for (int t = 0; t < Geo::kDimTiles; ++t)
        *reinterpret_cast<u32x2*>(out_row + 16 * t + 4 * g) = u32x2{0u, 0u};
      if (a.lse != nullptr && g == 0) a.lse[row * Hq + hk * G + c] = -INFINITY;
    }
    return;
  }

  // Q^T as the MFMA B operand: lane (c, g) holds head c, dims 32s + 8g .. +7.
  bf16x8 qf[Geo::kSteps];
  {
    const uint16_t* qp = a.q + b * a.qs0 + i * a.qs1 + (hk * G + (head_ok ? c : 0)) * a.qs2 + 8 * g;
    // Unsplit, each query row is read once: streamed past the caches, which
    // keeps them for K and V (the split rereads a row once per range, and the
    // Infinity Cache serves those rereads).
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s) {
      const u32x4* src = reinterpret_cast<const u32x4*>(qp + 32 * s);
      if (!head_ok)
        qf[s] = bf16x8{};
      else if constexpr (kSplit)
        qf[s] = __builtin_bit_cast(bf16x8, load16(src));
      else
        qf[s] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(src));
    }
  }

  f32x4 acc[Geo::kDimTiles];
#pragma unroll
  for (int t = 0; t < Geo::kDimTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference max (log2 domain) of head c
  float l_run = 0.f;        // this lane's share of the running sum of head c

  const int32_t* lst = a.route_list + row * a.K + first;
  const int64_t ks1b = 2 * a.ks1, vs1b = 2 * a.vs1;  // row strides in bytes
  const char* kb = reinterpret_cast<const char*>(a.k + b * a.ks0 + hk * a.ks2) + 16 * (lane % Geo::kLanesPerRow);
  const char* vb = reinterpret_cast<const char*>(a.v + b * a.vs0 + hk * a.vs2) + 16 * (lane % Geo::kLanesPerRow);
  uint16_t* my_slab = slab;
  uint16_t* my_kslab = kslab;
  const int32_t id_max = static_cast<int32_t>(a.S_kv - 1);
  auto clamp_id = [&](int32_t x) { return min(max(x, 0), id_max); };
  // Raw route ID of key base + c (tails repeat the last route; clamped later).
  auto load_id = [&](int base) { return lst[min(base + c, n - 1)]; };
  // K and V rows of the chunk in 16-byte pieces, two full rows per load
  // instruction (the pattern the address unit handles best); K reaches the A
  // operand of S^T = K Q^T through this wave's K slab, V the PV product
  // through the V slab.  Row r's ID lives in lane r.  The 32-bit path is
  // taken only when K and V share their row stride, so one offset serves both.
  auto load_kv = [&](int32_t id, u32x4* kr, u32x4* vr) {
    int32_t idr[Geo::kLoads];
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      idr[u] = chunk_row_id<Geo::kRowsPerLoad>(id, u, lane);
      kr[u] = load16(kb + RowOffset<kNarrow>::of(idr[u], ks1b));
    }
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      if constexpr (kNarrow)
        vr[u] = load16(vb + RowOffset<true>::of(idr[u], ks1b));
      else
        vr[u] = load16(vb + RowOffset<false>::of(idr[u], vs1b));
    }
  };

  u32x4 kr[Geo::kLoads];
  u32x4 vr[Geo::kLoads];
  int32_t raw_next = load_id(kChunk);  // issued first: used after the rows below
  {
    const int32_t id0 = clamp_id(load_id(0));
    load_kv(id0, kr, vr);
  }
  int32_t id_next = clamp_id(raw_next);

  const uint16_t* tr = my_slab + (lane >> 2) * Geo::kStride + 4 * (lane & 3);
  for (int base = 0; base < n; base += kChunk) {
    const bool more = base + kChunk < n;  // wave-uniform

    // Stage this chunk's K rows in LDS, read the score operands right behind
    // them, then stage the V rows (row-major, padded strides): the operand
    // reads do not queue behind the V writes.
    wave_lds_sync();  // previous chunk's reads of both slabs are complete
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int r = u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow;
      const int col = 8 * (lane % Geo::kLanesPerRow);
      *reinterpret_cast<u32x4*>(my_kslab + r * Geo::kKStride + col) = kr[u];
    }
    wave_lds_sync();  // K rows visible to every lane of this wave
    // Scores: lane holds S^T[key 4g + r][head c]; the A operand is key c,
    // dims 32s + 8g .. +7.
    const uint16_t* ka = my_kslab + c * Geo::kKStride + 8 * g;
    bf16x8 kf[Geo::kSteps];
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s) kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ka + 32 * s));
    __builtin_amdgcn_sched_barrier(0);  // the operand reads stay ahead of the V writes
#pragma unroll
    for (int u = 0; u < Geo::kLoads; ++u) {
      const int r = u * Geo::kRowsPerLoad + lane / Geo::kLanesPerRow;
      const int col = 8 * (lane % Geo::kLanesPerRow);
      *reinterpret_cast<u32x4*>(my_slab + r * Geo::kStride + col) = vr[u];
    }
    // Prefetch, as soon as the rows are staged (the registers are free again):
    // IDs two chunks ahead first, then the next chunk's K and V rows.
    if (more) {
      raw_next = load_id(base + 2 * kChunk);
      load_kv(id_next, kr, vr);
    }
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Geo::kSteps; ++s) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], st, 0, 0, 0);

    // Online softmax (log2 domain) against a lazily raised reference max.
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = base + 4 * g + r < n ? st[r] * a.scale_log2e : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = pair_max16(mx);
    mx = pair_max32(mx);                     // finite: the chunk holds at least one key
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
      pf[r] = static_cast<__bf16>(__builtin_amdgcn_exp2f(x[r] - m_run));  // hardware exp2, rounded to bf16
      l_run += static_cast<float>(pf[r]);
    }
    const i16x4 pb = __builtin_bit_cast(i16x4, pf);
    wave_lds_sync();  // V rows visible to every lane of this wave

    // O^T += V^T P^T: one transposed LDS read gives lane (c, g) keys 4g..4g+3
    // of dim 16t + c, matching its four probabilities.
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr(tr + 16 * t), pb, acc[t], 0, 0, 0);

    if (more) id_next = clamp_id(raw_next);
  }

  // Normalise and store: lane holds O[head c][dims 16t + 4g .. +3].
  float l_tot = pair_sum16(l_run);  // butterfly over the four lane groups of head c
  l_tot = pair_sum32(l_tot);
  const float inv = 1.0f / l_tot;
  // Natural-log log-sum-exp of the scaled scores: the sum is taken against
  // the reference max m_run (log2 domain), from the same bf16-rounded
  // probabilities as the output.  A partial keeps it in the log2 domain.
  if (direct) {
    if (a.lse != nullptr && head_ok && g == 0) a.lse[row * Hq + hk * G + c] = (m_run + log2f(l_tot)) * kLn2;
  } else if (head_ok && g == 0) {
    a.part_lse[((local * Hkv + hk) * a.P + p) * G + c] = m_run + log2f(l_tot);
  }
  uint16_t* dst = direct ? out_row : a.part_o + (((local * Hkv + hk) * a.P + p) * G + c) * D;
  if (head_ok) {
#pragma unroll
    for (int t = 0; t < Geo::kDimTiles; ++t) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(acc[t][r] * inv);
      if (direct)
        *reinterpret_cast<u32x2*>(dst + 16 * t + 4 * g) = __builtin_bit_cast(u32x2, o);
      else  // read once, by the combine: streamed past the caches (keeps the L2 for K and V)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x2, o), reinterpret_cast<u32x2*>(dst + 16 * t + 4 * g));
    }
  }
}

// The combine of one pass on its own: one wavefront per (row, KV head) unit.
template <int D>
__global__ void __launch_bounds__(64 * kWaves) range_combine_kernel(const KernelArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  combine_unit<D>(a, static_cast<int64_t>(blockIdx.x) * kWaves + wave, threadIdx.x & 63);
}

// Range starts of each row's list: offs[row][p] = the first position whose
// ID (clamped into [0, S_kv)) lies in range p or a later one, offs[row][P] =
// the row's count clamped into [0, K].  One wavefront per row; for an
// ascending list every entry is written exactly once: by the position where
// the range changes, or by the end for ranges past the last ID.
__global__ void __launch_bounds__(64 * kWaves)
    range_offsets_kernel(const int32_t* __restrict__ route_list, const int32_t* __restrict__ route_count,
                         int64_t rows, int64_t K, int64_t S_kv, int w_shift, int P, int32_t* __restrict__ offs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int n = static_cast<int>(min(max(static_cast<int64_t>(route_count[row]), int64_t{0}), K));
  const int32_t* lst = route_list + row * K;
  int32_t* o = offs + row * (P + 1);
  const int32_t id_max = static_cast<int32_t>(S_kv - 1);
  auto range_of = [&](int32_t id) { return min(max(id, 0), id_max) >> w_shift; };
  int r_carry = -1;  // range of the entry before this block (-1 before the first)
  if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(route_list) & 15) == 0) {
    // Every row 16-byte aligned: lane L takes entries 4L .. 4L+3 of each 256-entry block with one load
    // (in bounds: an entry below n <= K starts a group of four that ends at K - 1 at most).
    for (int j0 = 0; j0 < n; j0 += 256) {
      const int j = j0 + 4 * lane;
      int r[4] = {P, P, P, P};  // past the end: the end sentinel, written below
      if (j < n) {
        const u32x4 w = load16(lst + j);
        const int32_t ids[4] = {static_cast<int32_t>(w.x), static_cast<int32_t>(w.y), static_cast<int32_t>(w.z),
                                static_cast<int32_t>(w.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < n) r[e] = range_of(ids[e]);
      }
      const int r_up = __shfl(r[3], (lane + 63) & 63);
      int r_prev = lane == 0 ? r_carry : r_up;  // the previous entry's range, from the lane before
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (j + e < n)
          for (int q = r_prev + 1; q <= r[e]; ++q) o[q] = j + e;
        r_prev = r[e];
      }
      r_carry = __shfl(r[3], 63);
    }
  } else {
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const int r = j < n ? range_of(lst[j]) : P;  // past the end: the end sentinel, written below
      const int r_up = __shfl(r, (lane + 63) & 63);
      const int r_prev = lane == 0 ? r_carry : r_up;  // the previous entry's range, from the lane before
      if (j < n)
        for (int q = r_prev + 1; q <= r; ++q) o[q] = j;
      r_carry = __shfl(r, 63);
    }
  }
  if (lane == 0) {  // ranges past the last entry start at the end
    const int r_last = n > 0 ? range_of(lst[n - 1]) : -1;
    for (int q = r_last + 1; q <= P; ++q) o[q] = n;
  }
}

KernelArgs kernel_args(const AttnArgs& a) {
  KernelArgs k{};
  k.q = a.q; k.k = a.k; k.v = a.v;
  k.qs0 = a.qs[0]; k.qs1 = a.qs[1]; k.qs2 = a.qs[2];
  k.ks0 = a.ks[0]; k.ks1 = a.ks[1]; k.ks2 = a.ks[2];
  k.vs0 = a.vs[0]; k.vs1 = a.vs[1]; k.vs2 = a.vs[2];
  k.route_list = a.route_list;
  k.route_count = a.route_count;
  k.S_q = a.S_q; k.S_kv = a.S_kv; k.Hq = a.Hq; k.Hkv = a.Hkv; k.K = a.K;
  k.G = static_cast<int>(a.Hq / a.Hkv);
  k.scale_log2e = a.scale * kLog2e;
  k.n_units = a.B * a.S_q * a.Hkv;
  k.out = a.out;
  k.lse = a.lse;
  return k;
}

template <int D, bool kNarrow>
hipError_t launch(const AttnArgs& a, const SplitPlan& plan, const SplitBuffers& w, hipStream_t stream) {
  KernelArgs k = kernel_args(a);
  const int64_t rows = a.B * a.S_q;
  if (!plan.use) {
    hipLaunchKernelGGL((gather_attention_kernel<D, kNarrow, false>), dim3(static_cast<uint32_t>(rows * a.Hkv)),
                       dim3(64), 0, stream, k);
    return hipGetLastError();
  }
  if (hipError_t e = launch_range_offsets(a.route_list, a.route_count, rows, a.K, a.S_kv, plan, w.offs, stream);
      e != hipSuccess)
    return e;
  k.offs = w.offs;
  k.P = plan.P;
  // Passes from the last rows to the first (with causal routes the later
  // rows reach more ranges, so the combine left for the end is the smallest).
  // Each pass's split launch also merges the previous pass's partials, from
  // the other of the two partial buffers; the last pass is merged on its own.
  const int64_t n_pass = (rows + w.pass_rows - 1) / w.pass_rows;
  for (int64_t i = 0; i <= n_pass; ++i) {
    if (i > 0) {  // the previous pass, to be merged
      k.comb_row0 = k.row0;
      k.comb_pass_rows = k.pass_rows;
      k.comb_part_o = k.part_o;
      k.comb_part_lse = k.part_lse;
    }
    const int64_t comb_units = i > 0 ? k.comb_pass_rows * a.Hkv : 0;
    if (i == n_pass) {
      hipLaunchKernelGGL((range_combine_kernel<D>), dim3(static_cast<uint32_t>((comb_units + kWaves - 1) / kWaves)),
                         dim3(64 * kWaves), 0, stream, k);
      return hipGetLastError();
    }
    const int64_t r_end = rows - i * w.pass_rows;
    k.row0 = std::max<int64_t>(r_end - w.pass_rows, 0);
    k.pass_rows = r_end - k.row0;
    k.part_o = w.part_o[i & 1];
    k.part_lse = w.part_lse[i & 1];
    const int64_t gather_blocks = k.pass_rows * plan.P * a.Hkv;
    k.comb_blocks = comb_units;
    k.comb_stride = comb_units > 0 ? (gather_blocks + comb_units) / comb_units : 0;
    hipLaunchKernelGGL((gather_attention_kernel<D, kNarrow, true>),
                       dim3(static_cast<uint32_t>(gather_blocks + comb_units)), dim3(64), 0, stream, k);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

// True when K and V share a non-negative row stride and (S_kv - 1) * stride +
// one row fits in 32 bits (then one 32-bit offset addresses both rows).
bool narrow_offsets(const AttnArgs& a) {
  const int64_t lim = (int64_t{1} << 32) - 1;
  if (a.ks[1] < 0 || a.vs[1] != a.ks[1]) return false;  // one offset serves K and V
  return (a.S_kv - 1) * a.ks[1] * 2 + 2 * a.D <= lim && (a.S_kv - 1) * a.vs[1] * 2 + 2 * a.D <= lim;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const SplitPlan& plan, const SplitBuffers& w, hipStream_t stream) {
  return narrow_offsets(a) ? launch<D, true>(a, plan, w, stream) : launch<D, false>(a, plan, w, stream);
}

}  // namespace

hipError_t launch_range_offsets(const int32_t* route_list, const int32_t* route_count, int64_t rows, int64_t K,
                                int64_t S_kv, const SplitPlan& plan, int32_t* offs, hipStream_t stream) {
  hipLaunchKernelGGL(range_offsets_kernel, dim3(static_cast<uint32_t>((rows + kWaves - 1) / kWaves)),
                     dim3(64 * kWaves), 0, stream, route_list, route_count, rows, K, S_kv, plan.w_shift, plan.P,
                     offs);
  return hipGetLastError();
}

SplitPlan split_plan(int64_t rows, int64_t S_kv, int64_t Hq, int64_t D) {
  SplitPlan plan;
  int w_shift = 0;
  while ((int64_t{2} << w_shift) * 4 * D <= kRangeBytes) ++w_shift;  // largest W with W * 4D <= kRangeBytes
  while ((S_kv + (int64_t{1} << w_shift) - 1) >> w_shift > kMaxRanges) ++w_shift;
  plan.w_shift = w_shift;
  plan.P = static_cast<int>((S_kv + (int64_t{1} << w_shift) - 1) >> w_shift);
  // Up to 4 ranges (16 MiB of K and V per KV head) the unsplit kernel, which gives each XCD one KV head,
  // keeps routes that stay within a document or window in the L2 well enough that the split's extra
  // work units and partial results cost more than they save (measured on packed THD rows).
  plan.use = plan.P >= kMinRanges;
  if (plan.use) {
    plan.offs_bytes = (rows * (plan.P + 1) * 4 + 255) / 256 * 256;
    plan.part_o_row_bytes = Hq * plan.P * 2 * D;
    plan.part_lse_row_bytes = Hq * plan.P * 4;
  }
  return plan;
}

int64_t split_workspace_bytes(const SplitPlan& plan, int64_t pass_rows, int64_t rows) {
  auto r256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t buffers = pass_rows < rows ? 2 : 1;
  return plan.offs_bytes +
         buffers * (r256(pass_rows * plan.part_o_row_bytes) + r256(pass_rows * plan.part_lse_row_bytes));
}

hipError_t launch_gather_attention(const AttnArgs& a, const SplitPlan& plan, const SplitBuffers& w,
                                   hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_d<64>(a, plan, w, stream);
    case 128: return launch_d<128>(a, plan, w, stream);
    case 256: return launch_d<256>(a, plan, w, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa

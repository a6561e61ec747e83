// dk and dv of route-sparse GQA attention for gfx950: the key side of the
// backward (dq and delta: attention_backward.hip).
//
// Definition: fa4_qsa page (the FA4 kernel owns first-order autograd of this
// attention) and flex_qsa page, module description (keys no valid route
// names get zero gradients).  For every (b, i, h) routing key j, with
// p_j = exp(s_j - lse), dp_j = <dO, v_j> and delta = <dO, O>:
//   dk_j += scale p_j (dp_j - delta) q,   dv_j += p_j dO.
//
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
//
// This file is built without the VGPR form of the MFMA accumulators that the
// other kernels use: dK and dV only ever accumulate (no rescale), so their
// 2 x 16 x D fp32 sums sit in AGPRs and leave the VGPRs to the staged
// operands, which the compiler then reads ahead of the matrix instructions.
#include <hip/hip_runtime.h>

#include "backward_geometry.h"
#include "device_common.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

using bwd::Geo;
using bwd::kChunk;
using bwd::kWaves;
constexpr int kRecChunk = 1024;  // segment records staged in LDS at a time

template <int D, bool kNarrow>
__global__ void __launch_bounds__(64 * kWaves)
    dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                const uint16_t* __restrict__ dout, int64_t qs0, int64_t qs1, int64_t qs2, int64_t ks0, int64_t ks1,
                int64_t ks2, int64_t vs0, int64_t vs1, int64_t vs2, int64_t gs0, int64_t gs1, int64_t gs2,
                const float* __restrict__ lse, const float* __restrict__ delta, const int32_t* __restrict__ seg_start,
                const int4* __restrict__ segs, const int32_t* __restrict__ part_start,
                const int32_t* __restrict__ slot_start, const int32_t* __restrict__ plan, int64_t S_q, int64_t S_kv,
                int64_t Hq, int64_t Hkv, int G, int rows_per_batch, int64_t n_kt, int64_t n_tiles, float scale_log2e,
                float scale, float* __restrict__ partial, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using Gm = Geo<D>;
  constexpr int kThreads = 64 * kWaves;
  constexpr int kPieces = 2 * kChunk * Gm::kLanesPerRow;  // 16-byte pieces of Q and dO per batch
  constexpr int kPer = kPieces / kThreads;                  // per thread
  static_assert(kPer * kThreads == kPieces, "staging must split evenly over the workgroup");
  // Double-buffered staging of one batch: Q and dO of its 16 (row, head)
  // columns, and per column (lse2, delta) and the 64-bit key mask.
  __shared__ __attribute__((aligned(16))) uint16_t slab[2][2][kChunk * Gm::kTrStride];
  __shared__ float2 stat[2][kChunk];
  __shared__ uint2 cmask[2][kChunk];
  __shared__ int4 recs[kRecChunk];  // segment records of the part (a chunk at a time)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t x = blockIdx.x;
  const int64_t hk = x % Hkv;  // one KV head per XCD
  // Work item of this workgroup: part f of the split (parts numbered tile by tile).
  const int32_t f = static_cast<int32_t>(x / Hkv);
  if (f >= plan[1]) return;  // uniform over the workgroup
  int64_t lo = 0, hi = n_tiles;  // the tile u with part_start[u] <= f < part_start[u + 1]
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (part_start[mid] <= f) lo = mid; else hi = mid;
  }
  const int64_t unit = lo;  // b * n_kt + 64-key tile
  const int32_t part = f - part_start[unit];
  const int32_t n_parts = part_start[unit + 1] - part_start[unit];
  const int32_t part_len = plan[0];
  const int64_t b = unit / n_kt;
  const int kbit = 16 * wave + (lane & 15);         // this lane's key within the 64-key tile
  const int64_t key0 = (unit % n_kt) * 64 + 16 * wave;  // this wave's first key
  const int c = lane & 15;  // key (N side); col / dim row within a 16-tile
  const int g = lane >> 4;

  // K and V of the wave's 16 keys as B operands: lane (c, g) holds key c, dims 32s + 8g .. +7.
  bf16x8 kf[Gm::kSteps], vf[Gm::kSteps];
  {
    const int64_t key = min(key0 + c, S_kv - 1);
    const uint16_t* kp = k + b * ks0 + key * ks1 + hk * ks2 + 8 * g;
    const uint16_t* vp = v + b * vs0 + key * vs1 + hk * vs2 + 8 * g;
#pragma unroll
    for (int s = 0; s < Gm::kSteps; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, load16(kp + 32 * s));
      vf[s] = __builtin_bit_cast(bf16x8, load16(vp + 32 * s));
    }
  }
  f32x4 acc_k[Gm::kDimTiles], acc_v[Gm::kDimTiles];
#pragma unroll
  for (int t = 0; t < Gm::kDimTiles; ++t) acc_k[t] = acc_v[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int cols = rows_per_batch * G;  // MFMA rows in use: (row slot, head) = (col / G, col % G)
  const int32_t s_begin = seg_start[unit] + part * part_len;
  const int32_t s_end = min(seg_start[unit + 1], s_begin + part_len);
  const int64_t q_head0 = hk * G;
  const int32_t row_max = static_cast<int32_t>(S_q - 1);

  // The part's segment records are staged in LDS (kRecChunk at a time), so a
  // batch's loads take their addresses from LDS and never wait on another
  // global load.  Batches then flow through two register stages (loads of
  // batches i + 1 and i + 2 in flight while batch i is computed) into a
  // double-buffered LDS slab.
  // Every load is issued unconditionally from an in-range address (a load
  // under a divergent branch would make the compiler wait for it at the
  // branch's join, i.e. at once).  A column past the batch stages the
  // chunk's last record's row (finite data) with a cleared key mask, so its
  // P and dS are exactly zero and it adds nothing.
  struct Stage {
    u32x4 pre[kPer];
    float2 stat;
    uint2 mask;
    uint32_t ok;  // stat and mask belong to a batch column
  };
  // Batch-invariant bases of this thread's staged pieces: Q or dO of head
  // q_head0 + col % G at the piece's dims; each batch adds its row's offset.
  const char* src_base[kPer];
  int64_t src_stride[kPer];  // row stride in bytes
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int pc = tid + kThreads * u;
    const int m = pc / (kChunk * Gm::kLanesPerRow);  // 0: Q, 1: dO
    const int col = (pc / Gm::kLanesPerRow) % kChunk;
    const int piece = 8 * (pc % Gm::kLanesPerRow);
    const int64_t h = q_head0 + col % G;
    src_base[u] = reinterpret_cast<const char*>(m == 0 ? q + b * qs0 + h * qs2 : dout + b * gs0 + h * gs2) + 2 * piece;
    src_stride[u] = 2 * (m == 0 ? qs1 : gs1);
  }
  int32_t n_rec = 0;  // records staged for the current chunk (>= 1 while batches run)
  // A fetch in two halves: `plan` reads the batch's records from LDS and forms
  // the addresses, `issue` starts the global loads.  The step plans the fetch
  // before its compute and stash, so those LDS reads do not queue behind the
  // stash's slab writes ahead of the loads.
  struct Plan {
    const char* src[kPer];
    int64_t idx;
    uint2 mask;
    uint32_t ok;
  };
  auto plan_fetch = [&](int32_t sb) {  // sb: first record of the batch, within the chunk
    Plan P;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int col = ((tid + kThreads * u) / Gm::kLanesPerRow) % kChunk;
      const int32_t ir = min(max(recs[min(sb + col / G, n_rec - 1)].x, 0), row_max);
      P.src[u] = src_base[u] + RowOffset<kNarrow>::of(ir, src_stride[u]);
    }
    const int col = tid % kChunk;  // only threads below kChunk stash it
    const int slot = col / G;
    const int4 e = recs[min(sb + slot, n_rec - 1)];
    P.idx = (b * S_q + min(max(e.x, 0), row_max)) * Hq + q_head0 + col % G;
    P.mask = uint2{static_cast<uint32_t>(e.y), static_cast<uint32_t>(e.z)};
    P.ok = tid < kChunk && col < cols && sb + slot < n_rec ? 1u : 0u;
    return P;
  };
  auto issue = [&](Stage& S, const Plan& P) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) S.pre[u] = load16(P.src[u]);
    S.stat = float2{lse[P.idx], delta[P.idx]};  // raw: any arithmetic here would wait for the loads
    S.mask = P.mask;
    S.ok = P.ok;
  };
  auto fetch = [&](Stage& S, int32_t sb) { issue(S, plan_fetch(sb)); };
  auto stash = [&](const Stage& S, int buf) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = tid + kThreads * u;
      const int m = pc / (kChunk * Gm::kLanesPerRow);
      const int col = (pc / Gm::kLanesPerRow) % kChunk;
      const int piece = 8 * (pc % Gm::kLanesPerRow);
      *reinterpret_cast<u32x4*>(&slab[buf][m][col * Gm::kTrStride + piece]) = S.pre[u];
    }
    if (tid < kChunk) {
      const bool ok = S.ok != 0u;
      stat[buf][tid] = ok ? S.stat : float2{0.f, 0.f};
      cmask[buf][tid] = ok ? S.mask : uint2{0u, 0u};
    }
  };
  auto compute = [&](int cur) {
    // Per-column statistics for this lane's columns 4g .. 4g+3 and key c.
    float lse2[4], dl[4];
    bool on[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float2 st2 = stat[cur][4 * g + r];
      const uint2 mk = cmask[cur][4 * g + r];
      lse2[r] = st2.x * kLog2e;
      dl[r] = st2.y;
      on[r] = ((kbit < 32 ? mk.x >> kbit : mk.y >> (kbit - 32)) & 1u) != 0;
    }
    // Waves whose 16 keys no row of the batch routes skip the products.
    if (__ballot(on[0] || on[1] || on[2] || on[3])) {
      const uint16_t* my_q = slab[cur][0];
      const uint16_t* my_g = slab[cur][1];
      // S[col 4g + r][key c] = Q K^T and dP = dO V^T; A operands are slab rows
      // (col c, dims 32s + 8g .. +7).
      f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* qa = my_q + c * Gm::kTrStride + 8 * g;
      const uint16_t* ga = my_g + c * Gm::kTrStride + 8 * g;
#pragma unroll
      for (int s = 0; s < Gm::kSteps; ++s) {
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, load16(qa + 32 * s)), kf[s], st, 0, 0,
                                                     0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, load16(ga + 32 * s)), vf[s], dp, 0, 0,
                                                     0);
      }
      bf16x4 pb, dsb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // hardware exp2 (v_exp_f32): p is rounded to bf16 right after
        const float p = on[r] ? __builtin_amdgcn_exp2f(st[r] * scale_log2e - lse2[r]) : 0.f;
        pb[r] = static_cast<__bf16>(p);
        dsb[r] = static_cast<__bf16>(p * (dp[r] - dl[r]));
      }
      const i16x4 pi = __builtin_bit_cast(i16x4, pb);
      const i16x4 di = __builtin_bit_cast(i16x4, dsb);
      // dV^T += dO^T P and dK^T += Q^T dS: the transposed reads give lane (c, g)
      // columns 4g .. 4g+3 of dim 16t + c, matching its four P / dS values.
      const uint16_t* qtr = my_q + (lane >> 2) * Gm::kTrStride + 4 * (lane & 3);
      const uint16_t* gtr = my_g + (lane >> 2) * Gm::kTrStride + 4 * (lane & 3);
#pragma unroll
      for (int t = 0; t < Gm::kDimTiles; ++t) {
        acc_v[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr(gtr + 16 * t), pi, acc_v[t], 0, 0, 0);
        acc_k[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr(qtr + 16 * t), di, acc_k[t], 0, 0, 0);
      }
    }
  };

  Stage A, B;
  for (int32_t c0 = s_begin; c0 < s_end; c0 += kRecChunk) {
    n_rec = min(s_end - c0, static_cast<int32_t>(kRecChunk));
    __syncthreads();  // the previous chunk's records and slabs are no longer read
    for (int e = tid; e < n_rec; e += kThreads) recs[e] = segs[c0 + e];
    __syncthreads();
    const int32_t n_batches = (n_rec + rows_per_batch - 1) / rows_per_batch;
    // Fetches run unconditionally (past the last batch they read in-range
    // rows that are never stashed): with the same loads in flight on every
    // path, the wait before a stash covers that stage's loads only, not the
    // other stage's, which stay in flight across the batch.
    fetch(A, 0);
    stash(A, 0);
    fetch(A, rows_per_batch);
    fetch(B, 2 * rows_per_batch);
    __syncthreads();
    // X holds batch bi + 1 (the other stage holds bi + 2); the two stages swap roles every batch.
    auto step = [&](int32_t bi, Stage& X) {
      const Plan next = plan_fetch((bi + 3) * rows_per_batch);
      const int cur = bi & 1;
      compute(cur);
      if (bi + 1 < n_batches) stash(X, cur ^ 1);  // the other buffer was last read before the previous barrier
      issue(X, next);
      __syncthreads();
    };
    // Pairs of batches, then the odd last one: every path back to the loop
    // head then has A's loads issued before B's, which lets the compiler's
    // wait before a stash cover that stage's loads only.  (A loop that could
    // also come round after step A alone made it assume either order and
    // wait for the other stage's first load too.)
    int32_t bi = 0;
    for (; bi + 1 < n_batches; bi += 2) {  // workgroup-uniform
      step(bi, A);
      step(bi + 1, B);
    }
    if (bi < n_batches) step(bi, A);
    __builtin_amdgcn_s_waitcnt(0);  // the fetches past the last batch land before the next chunk reuses the stages
  }

  if (n_parts > 1) {
    // One part of a split tile: fp32 partial sums in the lane-native layout
    // [slot][hk][wave][dk tiles, dv tiles][lane][4], reduced in part order later.
    float* dst = partial + (((static_cast<int64_t>(slot_start[unit]) + part) * Hkv + hk) * kWaves + wave) *
                               (2 * Gm::kDimTiles * 256);
#pragma unroll
    for (int t = 0; t < Gm::kDimTiles; ++t) {
      *reinterpret_cast<f32x4*>(dst + (t * 64 + lane) * 4) = acc_k[t];
      *reinterpret_cast<f32x4*>(dst + ((Gm::kDimTiles + t) * 64 + lane) * 4) = acc_v[t];
    }
    return;
  }
  // Lane (c, g) holds dims 16t + 4g .. +3 of key key0 + c.
  if (key0 + c < S_kv) {
    const int64_t off = ((b * S_kv + key0 + c) * Hkv + hk) * D + 4 * g;
#pragma unroll
    for (int t = 0; t < Gm::kDimTiles; ++t) {
      bf16x4 wk, wv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wk[r] = static_cast<__bf16>(acc_k[t][r] * scale);
        wv[r] = static_cast<__bf16>(acc_v[t][r]);
      }
      *reinterpret_cast<u32x2*>(dk + off + 16 * t) = __builtin_bit_cast(u32x2, wk);
      *reinterpret_cast<u32x2*>(dv + off + 16 * t) = __builtin_bit_cast(u32x2, wv);
    }
  }
}

// Split tiles: sum the parts' partial sums in part order (a fixed order, so
// the result is deterministic) and write dk and dv.  One workgroup per
// (b, 64-key tile, hk, key group w of dkdv_kernel's wave w); its four waves
// each sum a quarter of the group's dk and dv slices, two parts' loads in
// flight at a time.  Tiles that were not split were written by dkdv_kernel.
template <int D>
__global__ void __launch_bounds__(64 * kWaves)
    dkdv_reduce_kernel(const int32_t* __restrict__ part_start, const int32_t* __restrict__ slot_start,
                       const float* __restrict__ partial, int64_t S_kv, int64_t Hkv, int64_t n_kt, int64_t n_tiles,
                       float scale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using Gm = Geo<D>;
  constexpr int kSlices = 2 * Gm::kDimTiles;  // dk tiles, then dv tiles, per key group
  constexpr int kMine = kSlices / kWaves;     // slices per wave: this wave sums slices wave + kWaves * j
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  int64_t x = blockIdx.x;
  const int64_t hk = x % Hkv;
  x /= Hkv;
  const int w = static_cast<int>(x % kWaves);  // key group: keys 16w .. 16w+15 of the tile
  const int64_t unit = x / kWaves;
  if (unit >= n_tiles) return;
  const int32_t n_parts = part_start[unit + 1] - part_start[unit];
  if (n_parts <= 1) return;
  const int64_t b = unit / n_kt;
  const int64_t key0 = (unit % n_kt) * 64 + 16 * w;
  const int c = lane & 15;
  const int g = lane >> 4;
  auto part_ptr = [&](int32_t p) {
    return partial + (((static_cast<int64_t>(slot_start[unit]) + p) * Hkv + hk) * kWaves + w) * (kSlices * 256) +
           lane * 4;
  };
  f32x4 acc[kMine];
#pragma unroll
  for (int j = 0; j < kMine; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int32_t p = 0;
  for (; p + 1 < n_parts; p += 2) {  // parts p and p + 1 loaded together, added in order
    const float* s0 = part_ptr(p);
    const float* s1 = part_ptr(p + 1);
    f32x4 a0[kMine], a1[kMine];
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      a0[j] = *reinterpret_cast<const f32x4*>(s0 + (wave + kWaves * j) * 256);
      a1[j] = *reinterpret_cast<const f32x4*>(s1 + (wave + kWaves * j) * 256);
    }
#pragma unroll
    for (int j = 0; j < kMine; ++j) acc[j] = (acc[j] + a0[j]) + a1[j];
  }
  if (p < n_parts) {
    const float* s0 = part_ptr(p);
#pragma unroll
    for (int j = 0; j < kMine; ++j) acc[j] += *reinterpret_cast<const f32x4*>(s0 + (wave + kWaves * j) * 256);
  }
  if (key0 + c < S_kv) {
    const int64_t off = ((b * S_kv + key0 + c) * Hkv + hk) * D + 4 * g;
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int slice = wave + kWaves * j;
      const bool is_k = slice < Gm::kDimTiles;
      const int t = is_k ? slice : slice - Gm::kDimTiles;
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(is_k ? acc[j][r] * scale : acc[j][r]);
      *reinterpret_cast<u32x2*>((is_k ? dk : dv) + off + 16 * t) = __builtin_bit_cast(u32x2, o);
    }
  }
}

// True when every Q and dO row lies within 4 GiB of its (batch, head) base,
// so the staged rows' offsets can be formed in 32 bits.
bool narrow_rows(const BwdArgs& a) {
  const int64_t lim = (int64_t{1} << 32) - 1;
  if (a.qs[1] < 0 || a.gs[1] < 0) return false;
  return (a.S_q - 1) * a.qs[1] * 2 <= lim && (a.S_q - 1) * a.gs[1] * 2 <= lim;
}

template <int D>
hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t stream) {
  const int64_t n_kt = (a.S_kv + 63) / 64;
  const int64_t n_tiles = a.B * n_kt;
  // Parts never exceed n_tiles + max_parts; workgroups past the planned count exit.
  const int64_t blocks = (n_tiles + a.max_parts) * a.Hkv;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  auto kernel = narrow_rows(a) ? dkdv_kernel<D, true> : dkdv_kernel<D, false>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWaves), 0, stream, a.q, a.k, a.v,
                     a.dout, a.qs[0], a.qs[1], a.qs[2], a.ks[0], a.ks[1], a.ks[2], a.vs[0], a.vs[1], a.vs[2],
                     a.gs[0], a.gs[1], a.gs[2], a.lse, a.delta, a.seg_start, a.segs, a.part_start, a.slot_start,
                     a.plan, a.S_q, a.S_kv, a.Hq, a.Hkv, G, kChunk / G, n_kt, n_tiles, a.scale * kLog2e, a.scale,
                     a.partial, a.dk, a.dv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_reduce_kernel<D>), dim3(static_cast<uint32_t>(n_tiles * kWaves * a.Hkv)), dim3(64 * kWaves), 0,
                     stream, a.part_start, a.slot_start, a.partial, a.S_kv, a.Hkv, n_kt, n_tiles, a.scale, a.dk, a.dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_dkdv(const BwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_dkdv_d<64>(a, stream);
    case 128: return launch_dkdv_d<128>(a, stream);
    case 256: return launch_dkdv_d<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa

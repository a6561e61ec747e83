// Route selection for gfx950: compressed-block scores on the matrix cores,
// then a per-row top-k by radix select, expanded to token IDs with the
// incomplete causal tail appended.
//
// Definition: qsa page, `select_qsa_token_ids`.  Query row i stands at
// global position t = q_offset + i and sees nv = floor((t + 1) / c) complete
// blocks; block j scores sum_h relu(<q[t,h], k[j]>) / sqrt(D) (the positive
// 1/sqrt(D) factor orders nothing, so the kernels rank the unscaled sums);
// the best kb = token_budget / c blocks are kept (equal scores: the smaller
// block index), written in ascending block order as c token IDs each, then
// the tokens nv*c .. t of the incomplete tail go to the last c - 1 slots.
// Rows at or past their batch's logical length are all -1.
//
// Design:
//  * select_scores_kernel -- a workgroup owns 16/HG query rows of one batch
//    (HG = head groups of 16) and a segment of up to 4096 blocks, walked in
//    LDS chunks of 32 KB of block keys (row stride 2D + 32 bytes, with which
//    the bank-conflict counter reads zero for the operand reads and row
//    stores).  The next chunk is prefetched into registers
//    while the current one is used; the rows' queries are loaded once and
//    stay in registers as the A operand.  Per 16 blocks a wave runs
//    v_mfma_f32_16x16x32_bf16 with the 16 index heads of a row on M and the
//    16 blocks on N; lane (n, g) then holds heads 4g .. 4g+3 of block n, so
//    the relu and three adds give a partial sum, and three gfx950 lane swaps
//    (two across the wave's halves, one across 16-lane rows; registers only)
//    complete the sums of four rows and leave row g's sum in lane group g,
//    which holds a chunk's sums in registers and stores them once the next
//    chunk is staged (vector loads and stores share one wait counter, so a
//    store issued before the staging would be waited for there).  The
//    segments of one row tile run on one XCD; the tiles that see the most
//    blocks are dispatched first.  fp32 scores go to a [rows, ld] workspace,
//    only for rows that see more than kb blocks, only for visible blocks.
//  * select_topk_kernel -- one workgroup per query row.  Scores sit in
//    registers (E per thread, coalesced loads; each launch covers rows whose
//    length fits its E, slots past the row hold 0); three LDS-histogram
//    passes over the nonzero float bit patterns (non-negative floats order
//    like their bits; 11, 11 and 10 bits) find the kb-th largest value tau
//    and how many of the values equal to tau to keep; when a pass needs its
//    boundary bin whole, the search stops there and every key at or above
//    the bin's lower bound is kept (no tie to split).  Ballots build bitmaps
//    of the values above tau and of those equal to it; a block prefix over
//    the words keeps the lowest-index ties and places every kept block at its
//    rank, in ascending block order.  The row is then written coalesced.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "qsa.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kSegmentBlocks = 4096;  // blocks per score workgroup at most
constexpr int kBins = 2048;           // histogram bins of one radix pass (11 bits)

template <int D, int kChunkKB>
struct SelGeo {
  static constexpr int kSteps = D / 32;                  // K-slices of one 16x16x32 product
  static constexpr int kStride = D + 16;                 // LDS row stride (bf16): 2D + 32 bytes
  static constexpr int kPieces = D / 8;                  // 16-byte pieces of one key row
  static constexpr int kChunk = kChunkKB * 512 / D;      // blocks per LDS chunk (kChunkKB KB of keys)
  static constexpr int kPerThread = kChunk * kPieces / kScoreThreads;  // 16-byte pieces per thread: 8 or 4
};

// relu on the bit pattern: negative values and -0.0 (sign bit set, negative as int32) become +0.0.
__device__ __forceinline__ float relu(float v) { return __int_as_float(max(__float_as_int(v), 0)); }

__device__ __forceinline__ int64_t clamp_len(int64_t L, int64_t q_end) { return L < 0 ? 0 : (L > q_end ? q_end : L); }

// kChunkKB = 32: half the barriers; 16 (D = 128, rows that see more than one segment): the smaller
// prefetch leaves room for four wavefronts per SIMD instead of three, which the compiler is held to.
template <int D, int HG, int kChunkKB>
__global__ void __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(kChunkKB == 16 ? 4 : 1)))
    select_scores_kernel(const uint16_t* __restrict__ iq, int64_t qs0, int64_t qs1, int64_t qs2,
                         const uint16_t* __restrict__ ck, int64_t cs0, int64_t cs1,
                         const int64_t* __restrict__ seq_lens, int64_t S_q, int64_t H, int64_t q_offset,
                         int64_t c, int64_t kb, int64_t tile0, int64_t n_tiles, int64_t tiles_per_batch,
                         int64_t n_segments, int64_t row_base, int64_t ld, float* __restrict__ scores) {
  using Geo = SelGeo<D, kChunkKB>;
  constexpr int RW = 4 / HG;   // query rows per wave
  constexpr int RPW = 4 * RW;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t kslab[Geo::kChunk * Geo::kStride];

  // Workgroup w -> (tile, segment): tiles in groups of 8, the segments of
  // tile 8q + x on workgroups congruent to x mod 8 (one XCD); tiles are taken
  // from the last (which see the most blocks) to the first.
  const int64_t w = blockIdx.x;
  const int64_t x = w % 8, rest = w / 8;
  const int64_t seg = rest % n_segments;
  const int64_t rank = (rest / n_segments) * 8 + x;
  if (rank >= n_tiles) return;  // every exit precedes the first barrier
  const int64_t tile = tile0 + (n_tiles - 1 - rank);
  const int64_t b = tile / tiles_per_batch;
  const int64_t i0 = (tile % tiles_per_batch) * RPW;
  const int64_t L = clamp_len(seq_lens[b], q_offset + S_q);
  // Non-padding rows are a prefix of the tile; the last one sees the most blocks.
  const int64_t i_last = min(min(i0 + RPW - 1, S_q - 1), L - 1 - q_offset);
  if (i_last < i0) return;
  const int64_t nv_max = (q_offset + i_last + 1) / c;
  const int64_t seg0 = seg * kSegmentBlocks;
  if (nv_max <= kb || seg0 >= nv_max) return;
  const int64_t seg_end = min(nv_max, seg0 + kSegmentBlocks);
  const int n_chunks = static_cast<int>((seg_end - seg0 + Geo::kChunk - 1) / Geo::kChunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;  // head row of the A operand; block column of B and of the result
  const int g = lane >> 4;  // k-group of the operands; head quad of the result

  // Key pieces of one chunk: thread tid holds piece tid % kPieces of blocks tid / kPieces + u kRows
  // (zeros past seg_end).  One address per chunk and a constant stride per piece; only the last,
  // partial chunk of a segment tests its blocks against seg_end.
  constexpr int kRows = kScoreThreads / Geo::kPieces;  // blocks covered by one piece per thread
  const int prow = tid / Geo::kPieces, pcol = 8 * (tid % Geo::kPieces);
  const uint16_t* kbase = ck + b * cs0 + prow * cs1 + pcol;
  const int64_t kstep = kRows * cs1;
  u32x4 pre[Geo::kPerThread];
  auto fetch = [&](int64_t j0) {
    const uint16_t* src = kbase + j0 * cs1;
    if (j0 + Geo::kChunk <= seg_end) {  // workgroup-uniform
#pragma unroll
      for (int u = 0; u < Geo::kPerThread; ++u) pre[u] = load16(src + u * kstep);
    } else {
      const int64_t left = seg_end - j0 - prow;  // this thread's blocks in range: kRows u < left
#pragma unroll
      for (int u = 0; u < Geo::kPerThread; ++u)
        pre[u] = kRows * u < left ? load16(src + u * kstep) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  uint16_t* sdst = kslab + prow * Geo::kStride + pcol;
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < Geo::kPerThread; ++u) *reinterpret_cast<u32x4*>(sdst + u * kRows * Geo::kStride) = pre[u];
  };
  fetch(seg0);

  // Queries as the A operand: lane (m, g) holds head 16 hg + m, dims 32s + 8g .. +7.
  bf16x8 qf[RW][HG][Geo::kSteps];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t i = i0 + wave * RW + r;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const int head = 16 * hg + m;
      const bool ok = i <= i_last && head < H;
      const uint16_t* qp = iq + b * qs0 + (ok ? i : 0) * qs1 + (ok ? head : 0) * qs2 + 8 * g;
#pragma unroll
      for (int s = 0; s < Geo::kSteps; ++s)
        qf[r][hg][s] = ok ? __builtin_bit_cast(bf16x8, load16(qp + 32 * s)) : bf16x8{};
    }
  }

  // Row stored by this lane (lane group g owns row g of the wave) and its visible blocks.
  const int64_t my_i = i0 + wave * RW + g;
  const bool my_row = g < RW && my_i <= i_last;
  const int64_t my_nv = my_row ? (q_offset + my_i + 1) / c : 0;
  const bool my_store = my_row && my_nv > kb;
  float* my_out = scores + (my_store ? (b * S_q + my_i - row_base) * ld : 0);

  stage();
  __syncthreads();

  for (int ch = 0; ch < n_chunks; ++ch) {
    const int64_t j0 = seg0 + static_cast<int64_t>(ch) * Geo::kChunk;
    fetch(j0 + Geo::kChunk);  // in flight while this chunk is scored (past the segment: zeros, no loads)
    const int n_sub = static_cast<int>((min(static_cast<int64_t>(Geo::kChunk), seg_end - j0) + 15) / 16);
    constexpr int kSub = Geo::kChunk / 16;
    float held[kSub];
#pragma unroll
    for (int sc = 0; sc < kSub; ++sc) {
      held[sc] = 0.f;
      if (sc >= n_sub) continue;
      bf16x8 kf[Geo::kSteps];
      const uint16_t* kp = kslab + (16 * sc + m) * Geo::kStride + 8 * g;
#pragma unroll
      for (int s = 0; s < Geo::kSteps; ++s)
        kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + 32 * s));

      float part[4] = {0.f, 0.f, 0.f, 0.f};  // rows past RW stay 0
#pragma unroll
      for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < Geo::kSteps; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[r][hg][s], kf[s], acc, 0, 0, 0);
          const float sum = relu(acc[0]) + relu(acc[1]) + relu(acc[2]) + relu(acc[3]);
          part[r] = hg == 0 ? sum : part[r] + sum;
        }
      }
      // Lane groups 0+2 and 1+3 combine rows 0 and 2 (p02) and rows 1 and 3 (p13); then groups
      // 0+1 and 2+3 finish them, leaving row g's sum in lane group g.
      const u32x2 p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const u32x2 p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float xs = __uint_as_float(p02[0]) + __uint_as_float(p02[1]);
      const float ys = __uint_as_float(p13[0]) + __uint_as_float(p13[1]);
      const u32x2 z = __builtin_amdgcn_permlane16_swap(__float_as_uint(xs), __float_as_uint(ys), false, false);
      const float total = __uint_as_float(z[0]) + __uint_as_float(z[1]);  // >= +0.0: sums of relu terms
      held[sc] = total;
    }
    __syncthreads();  // every wave is done with this chunk's keys
    stage();
    __syncthreads();
    // The chunk's scores are stored only now, so that the wait before the staging above covers
    // the next chunk's loads and none of these stores.
#pragma unroll
    for (int sc = 0; sc < kSub; ++sc) {
      const int64_t j = j0 + 16 * sc + m;
      if (my_store && j < my_nv) my_out[j] = held[sc];
    }
  }
}

// Exclusive prefix sum of x over the workgroup's threads (in thread order),
// and the total.  Every thread must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int q = 0; q < NT / 64; ++q) {
    const int v = wave_tot[q];
    before += q < wave ? v : 0;
    sum += v;
  }
  __syncthreads();  // wave_tot is reused by the next call
  *total = sum;
  return before + incl - x;
}

template <int NT, int E>
__global__ void __launch_bounds__(NT)
    select_topk_kernel(const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ seq_lens,
                       int64_t S_q, int64_t q_offset, int64_t c, int64_t kb, int64_t budget, int64_t W,
                       int64_t row_base, int64_t row0, int32_t* __restrict__ out) {
  constexpr int kWaves = NT / 64;
  constexpr int kWords = NT * E / 64;  // <= NT: one bitmap word per thread at most
  constexpr int kBinsPerThread = kBins / NT;
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t gt_words[kWords];
  __shared__ uint64_t eq_words[kWords];
  __shared__ int32_t kept[QSA_MAX_SELECT_BLOCKS];
  __shared__ int wave_tot[kWaves];
  __shared__ int found[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row = row0 + blockIdx.x;  // b * S_q + i; the workspace starts at row row_base
  const int64_t b = row / S_q, i = row % S_q;
  const int64_t t = q_offset + i;
  int32_t* orow = out + row * W;
  if (t >= clamp_len(seq_lens[b], q_offset + S_q)) {  // padding query
    for (int64_t s = tid; s < W; s += NT) orow[s] = -1;
    return;
  }
  const int64_t nv = (t + 1) / c;
  const int64_t tail0 = nv * c, tail_n = t + 1 - tail0;
  const bool sparse = kb > 0 && nv > kb;
  const int64_t mc = (kb < nv ? kb : nv) * c;  // slots holding kept-block tokens

  if (sparse) {  // workgroup-uniform
    const float* srow = scores + (row - row_base) * ld;
    const int n = static_cast<int>(nv);  // <= NT * E (the launch picks E for the row's length)
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = e * NT + tid;
      key[e] = idx < n ? __float_as_uint(srow[idx]) : 0u;
    }
    // Slots past the row hold key 0.  Zero keys (+0.0 scores and those slots) are the smallest
    // values and are left out of the histograms: while at least `remaining` nonzero keys carry
    // the prefix, the kb-th largest value is the same with or without them; when fewer do (only
    // possible with prefix 0), tau is 0 and the rest are zeros, which the lowest-index rule below
    // takes from the row's own (lower indices, and the row has more than kb values).
    uint32_t prefix = 0, hi_mask = 0;
    int remaining = static_cast<int>(kb);
    bool settled = false;  // workgroup-uniform: tau found to be 0, or the boundary bin is kept whole
    bool whole = false;    // workgroup-uniform: every key >= tau is kept and no tie is split
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      if (settled) continue;
      const int sh = p == 0 ? 21 : (p == 1 ? 10 : 0);
      const uint32_t dmask = p == 2 ? 0x3FFu : 0x7FFu;
      for (int q = tid; q < kBins; q += NT) hist[q] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (key[e] != 0u && (key[e] & hi_mask) == prefix) atomicAdd(&hist[(key[e] >> sh) & dmask], 1u);
      }
      __syncthreads();
      int local = 0;
#pragma unroll
      for (int q = 0; q < kBinsPerThread; ++q) local += static_cast<int>(hist[tid * kBinsPerThread + q]);
      int total = 0;
      const int before = block_exclusive_scan<NT>(local, wave_tot, &total);
      if (total < remaining) {  // workgroup-uniform
        prefix = 0u;
        remaining -= total;
        settled = true;
        continue;
      }
      const int above = total - before - local;  // candidates in higher bins than this thread's
      if (above < remaining && above + local >= remaining) {
        int acc = above;
        for (int q = kBinsPerThread - 1; q >= 0; --q) {
          const int h = static_cast<int>(hist[tid * kBinsPerThread + q]);
          if (acc + h >= remaining) {
            found[0] = tid * kBinsPerThread + q;
            found[1] = remaining - acc;
            break;
          }
          acc += h;
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(found[0]) << sh;
      hi_mask |= dmask << sh;
      remaining = found[1];
      // The boundary bin is needed whole: every key >= prefix (its lower bits zero) is kept, exactly
      // kb of them, and the lower digits need no pass.  prefix 0 is left to the general path (zero
      // keys are not in the histograms).
      if (p < 2 && prefix != 0u && static_cast<int>(hist[found[0]]) == remaining) {
        whole = true;
        settled = true;
      }
      __syncthreads();  // found and hist are rewritten by the next pass
    }
    const uint32_t tau = prefix;  // the kb-th largest value; keep `remaining` of the values equal to it

    // A zero past the row is never above tau; it equals tau only when tau is 0, and then the
    // lowest-index rule below takes the row's own zeros (all at lower indices, and at least
    // `remaining` of them) first.
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t bg = __ballot(whole ? key[e] >= tau : key[e] > tau);
      const uint64_t be = __ballot(!whole && key[e] == tau);
      if (lane == 0) {
        gt_words[e * kWaves + wave] = bg;  // word e * kWaves + wave covers blocks 64 * word .. +63
        eq_words[e * kWaves + wave] = be;
      }
    }
    __syncthreads();
    const uint64_t eqw = tid < kWords ? eq_words[tid] : 0ull;
    const uint64_t gtw = tid < kWords ? gt_words[tid] : 0ull;
    int total = 0;
    const int eq_before = block_exclusive_scan<NT>(__popcll(eqw), wave_tot, &total);
    const int take = min(max(remaining - eq_before, 0), __popcll(eqw));  // lowest-index ties first
    uint64_t keep = gtw, rest = eqw;
    for (int q = 0; q < take; ++q) {
      const uint64_t low = rest & (~rest + 1ull);
      keep |= low;
      rest ^= low;
    }
    int rank = block_exclusive_scan<NT>(__popcll(keep), wave_tot, &total);
    while (keep != 0ull) {
      if (rank < kb) kept[rank] = 64 * tid + __builtin_ctzll(keep);  // rank < kb always; guards LDS
      ++rank;
      keep &= keep - 1ull;
    }
    __syncthreads();
  }

  // Kept blocks as c token IDs each, then -1 up to the budget, then the tail (no division).
  const int ci = static_cast<int>(c), mi = static_cast<int>(mc / c), Wi = static_cast<int>(W);
  const int budget_i = static_cast<int>(budget), tail0_i = static_cast<int>(tail0), tail_ni = static_cast<int>(tail_n);
  for (int r = tid; r < mi; r += NT) {
    const int blk = sparse ? kept[r] : r;
    for (int u = 0; u < ci; ++u) orow[r * ci + u] = blk * ci + u;
  }
  for (int s = mi * ci + tid; s < budget_i; s += NT) orow[s] = -1;
  for (int s = budget_i + tid; s < Wi; s += NT) orow[s] = s - budget_i < tail_ni ? tail0_i + (s - budget_i) : -1;
}

template <int D>
hipError_t launch_scores_d(const SelectArgs& a, int hg, int64_t tile0, int64_t n_tiles, int64_t tiles_per_batch,
                           int64_t n_segments, int64_t row_base, int64_t ld, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((n_tiles + 7) / 8 * 8 * n_segments));
  const int64_t kb = a.token_budget / a.compress_ratio;
#define QSA_SCORES(HG, KB)                                                                                      \
  hipLaunchKernelGGL((select_scores_kernel<D, HG, KB>), grid, dim3(kScoreThreads), 0, stream, a.iq, a.qs[0],   \
                     a.qs[1], a.qs[2], a.ck, a.cs[0], a.cs[1], a.seq_lens, a.S_q, a.H, a.q_offset,              \
                     a.compress_ratio, kb, tile0, n_tiles, tiles_per_batch, n_segments, row_base, ld, a.scores)
  if constexpr (D == 128) {
    if (n_segments > 1) {  // long rows: many workgroups per tile, occupancy pays
      switch (hg) {
        case 1: QSA_SCORES(1, 16); break;
        case 2: QSA_SCORES(2, 16); break;
        default: QSA_SCORES(4, 16); break;
      }
      return hipGetLastError();
    }
  }
  {
    switch (hg) {
      case 1: QSA_SCORES(1, 32); break;
      case 2: QSA_SCORES(2, 32); break;
      default: QSA_SCORES(4, 32); break;
    }
  }
#undef QSA_SCORES
  return hipGetLastError();
}

// Register width of the top-k for rows that see up to nv blocks: 256 threads x E slots, E a power
// of two from 4 to 64, then 1024 x 64.
int topk_class(int64_t nv) {
  int cls = 0;
  while (cls < 4 && nv > (int64_t{256} << (cls + 2))) ++cls;
  return nv > 256 * 64 ? 5 : cls;
}

hipError_t launch_topk_rows(const SelectArgs& a, int cls, int64_t row_base, int64_t row0, int64_t rows, int64_t ld,
                            hipStream_t stream) {
  const int64_t c = a.compress_ratio, kb = a.token_budget / c, W = a.token_budget + c - 1;
  const dim3 grid(static_cast<uint32_t>(rows));
#define QSA_TOPK(NT, E)                                                                                          \
  hipLaunchKernelGGL((select_topk_kernel<NT, E>), grid, dim3(NT), 0, stream, a.scores, ld, a.seq_lens, a.S_q, \
                     a.q_offset, c, kb, a.token_budget, W, row_base, row0, a.out)
  switch (cls) {
    case 0: QSA_TOPK(256, 4); break;
    case 1: QSA_TOPK(256, 8); break;
    case 2: QSA_TOPK(256, 16); break;
    case 3: QSA_TOPK(256, 32); break;
    case 4: QSA_TOPK(256, 64); break;
    default: QSA_TOPK(1024, 64); break;
  }
#undef QSA_TOPK
  return hipGetLastError();
}

// Rows [row_base, row_base + rows) of the pass, split into runs of rows of one register class
// (the visible blocks grow with the query position), one launch per run.  With more runs than
// kMaxTopkLaunches (many batch rows that each span several classes) one launch at the class of
// the longest row does all.
hipError_t launch_topk(const SelectArgs& a, int64_t nv_all, int64_t row_base, int64_t rows, int64_t ld,
                       hipStream_t stream) {
  constexpr int64_t kMaxTopkLaunches = 64;
  const int64_t c = a.compress_ratio, row_end = row_base + rows;
  auto class_of_row = [&](int64_t r) { return topk_class((a.q_offset + r % a.S_q + 1) / c); };
  // Next row after r (same batch row) whose class differs, or the batch row's end.
  auto run_end = [&](int64_t r) {
    const int cls = class_of_row(r);
    const int64_t batch_end = (r / a.S_q + 1) * a.S_q;
    if (cls == 5) return min(batch_end, row_end);
    // last position t with (t + 1) / c <= 256 << (cls + 2): t + 1 < ((256 << (cls + 2)) + 1) * c
    const int64_t t_lim = ((int64_t{256} << (cls + 2)) + 1) * c - 1;  // first t past the class
    const int64_t r_lim = r - r % a.S_q + (t_lim - a.q_offset);
    return min(min(batch_end, row_end), max(r_lim, r + 1));
  };
  // Adjacent runs of one class (the next batch row starting where the last one ended) merge.
  auto merged_end = [&](int64_t r) {
    const int cls = class_of_row(r);
    int64_t e = run_end(r);
    while (e < row_end && class_of_row(e) == cls) e = run_end(e);
    return e;
  };
  int64_t n_runs = 0;
  for (int64_t r = row_base; r < row_end && n_runs <= kMaxTopkLaunches; r = merged_end(r)) ++n_runs;
  if (n_runs > kMaxTopkLaunches) return launch_topk_rows(a, topk_class(nv_all), row_base, row_base, rows, ld, stream);
  for (int64_t r = row_base; r < row_end;) {
    const int64_t e = merged_end(r);
    const hipError_t err = launch_topk_rows(a, class_of_row(r), row_base, r, e - r, ld, stream);
    if (err != hipSuccess) return err;
    r = e;
  }
  return hipSuccess;
}

}  // namespace

int64_t select_rows_per_tile(int64_t H) { return H <= 16 ? 16 : (H <= 32 ? 8 : 4); }

int64_t select_score_ld(int64_t S_q, int64_t q_offset, int64_t c) {
  const int64_t nv_all = (q_offset + S_q) / c;
  return (nv_all < 1 ? 1 : nv_all + 63) / 64 * 64;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  const int64_t c = a.compress_ratio, kb = a.token_budget / c;
  const int64_t nv_all = (a.q_offset + a.S_q) / c;  // blocks the last query row sees
  const int64_t rpt = select_rows_per_tile(a.H);
  const int hg = static_cast<int>(16 / rpt);
  const int64_t tiles_per_batch = (a.S_q + rpt - 1) / rpt;
  const int64_t n_tiles = a.B * tiles_per_batch;
  const int64_t ld = select_score_ld(a.S_q, a.q_offset, c);
  const bool scoring = kb > 0 && nv_all > kb;
  const int64_t tiles_per_pass =
      scoring ? static_cast<int64_t>(a.workspace_bytes / (static_cast<size_t>(rpt * ld) * sizeof(float))) : n_tiles;
  if (tiles_per_pass < 1) return hipErrorInvalidValue;  // the entry point checks the size first
  const int64_t n_segments = (nv_all + kSegmentBlocks - 1) / kSegmentBlocks;
  for (int64_t t0 = 0; t0 < n_tiles; t0 += tiles_per_pass) {
    const int64_t t1 = std::min(n_tiles, t0 + tiles_per_pass);
    const int64_t row_base = (t0 / tiles_per_batch) * a.S_q + (t0 % tiles_per_batch) * rpt;
    const int64_t last = t1 - 1;
    const int64_t row_end = (last / tiles_per_batch) * a.S_q + std::min((last % tiles_per_batch) * rpt + rpt, a.S_q);
    if (scoring) {
      hipError_t e;
      switch (a.D) {
        case 64: e = launch_scores_d<64>(a, hg, t0, t1 - t0, tiles_per_batch, n_segments, row_base, ld, stream); break;
        case 128: e = launch_scores_d<128>(a, hg, t0, t1 - t0, tiles_per_batch, n_segments, row_base, ld, stream); break;
        default: e = launch_scores_d<256>(a, hg, t0, t1 - t0, tiles_per_batch, n_segments, row_base, ld, stream); break;
      }
      if (e != hipSuccess) return e;
    }
    const hipError_t e = launch_topk(a, nv_all, row_base, row_end - row_base, ld, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qsa

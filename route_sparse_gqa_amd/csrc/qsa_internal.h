// Internal launchers shared by the C-ABI entry points (not exported).
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stdint.h>

namespace qsa {

// One launch holds fewer than 2^32 work-items per grid dimension
// (gridDim.x * blockDim.x); kMaxBlocks is that limit in 256-thread
// workgroups, the size of most launches here, kMaxWaveBlocks in
// one-wavefront workgroups (the attention kernel's).
constexpr int64_t kMaxLaunchItems = (int64_t{1} << 32) - 1;
constexpr int64_t kMaxBlocks = kMaxLaunchItems / 256;
constexpr int64_t kMaxWaveBlocks = kMaxLaunchItems / 64;

// Work-items per query row of the route normalisation launch that K and
// kv_length select (the host checks B * S_q times it against kMaxLaunchItems).
int64_t route_normalize_items_per_row(int64_t K, int64_t kv_length);

// Route normalisation: [B*S_q rows, K slots] -> ascending distinct valid IDs.
// When zero_buf is non-null the same launch also sets its zero_count int32
// entries to 0 (the tile member counters of the membership pass).
hipError_t launch_route_normalize(const void* routes, bool routes_int64, int64_t B, int64_t S_q,
                                  int64_t K, const int64_t route_strides[3], int64_t kv_length,
                                  int32_t* route_list, int32_t* route_count, int32_t* zero_buf,
                                  int64_t zero_count, hipStream_t stream);

// Membership table and/or 128x128 tile classes from compacted lists: one
// workgroup per (batch, 128-row tile row, segment of kMemSegCols columns,
// group of 128 / kMemGroups rows), i.e. B * ceil(S_q/128) * ceil(ldm/kMemSegCols)
// * kMemGroups workgroups.
constexpr int64_t kMemSegCols = 65536;
constexpr int64_t kMemGroups = 32;
hipError_t launch_membership_tiles(const int32_t* route_list, const int32_t* route_count, int64_t B,
                                   int64_t S_q, int64_t K, int64_t kv_length, uint8_t* membership,
                                   int32_t* tile_class, hipStream_t stream);

// Forward and reverse partial/full block lists of a tile-class table; out =
// {partial_count, partial_idx, full_count, full_idx, rev_partial_count,
// rev_partial_idx, rev_full_count, rev_full_idx}, each nullable.
hipError_t launch_tile_lists(const int32_t* kinds, int64_t B, int64_t n_rows, int64_t n_cols, int32_t* const out[8],
                             hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qs[4], ks[4], vs[4];
  const int32_t* route_list;
  const int32_t* route_count;
  int64_t B, S_q, S_kv, Hq, Hkv, D, K;
  float scale;
  uint16_t* out;
  float* lse;  // nullable: [B*S_q*Hq] natural-log log-sum-exp
};

// Key-range split of the attention (used when one KV head's K and V rows
// exceed what one XCD's L2 holds): each row's sorted list is cut at
// multiples of W = 2^w_shift key IDs into P ranges; the workgroups take the
// ranges one after another for all rows of a pass, so every XCD's L2 holds
// one range at a time; rows with routes in several ranges get one partial
// result per range, merged by a combine pass.
constexpr int64_t kRangeBytes = int64_t{4} << 20;  // K + V bytes of one KV head's range
constexpr int kMinRanges = 5;                       // fewer ranges (<= 16 MiB per KV head): no split
constexpr int kMaxRanges = 63;                      // ranges per row (one wavefront lane each, plus the end)
constexpr int64_t kMinPassRows = 256;               // smallest pass the workspace must hold

struct SplitPlan {
  bool use = false;
  int w_shift = 0;   // range width W = 2^w_shift key IDs
  int P = 1;         // ranges: ceil(S_kv / W) <= kMaxRanges
  int64_t offs_bytes = 0;          // [rows][P + 1] int32 range starts (256-B aligned size)
  int64_t part_o_row_bytes = 0;    // partial outputs of one query row: Hq * P * D bf16
  int64_t part_lse_row_bytes = 0;  // their log2-sum-exps: Hq * P fp32
};

SplitPlan split_plan(int64_t rows, int64_t S_kv, int64_t Hq, int64_t D);

// Workspace of a split attention: range starts, then for each pass row the
// partial outputs [Hkv][P][G][D] bf16 and their log2-sum-exps [Hkv][P][G]
// fp32, twice when there is more than one pass (a pass's partials are merged
// while the next pass gathers into the other buffer).
struct SplitBuffers {
  int32_t* offs;
  uint16_t* part_o[2];
  float* part_lse[2];
  int64_t pass_rows;  // rows per pass (a multiple of 4, or every row)
};

// Bytes of split workspace for passes of pass_rows of the call's rows (plan.use must hold).
int64_t split_workspace_bytes(const SplitPlan& plan, int64_t pass_rows, int64_t rows);

// qsa_forward's checks and launches.  When `scratch` is non-null it is
// called after the argument checks with the smallest workspace the call can
// run in (lists plus the split's smallest pass) and the stream, and supplies
// the workspace pointer and size in place of the arguments (or an error).
typedef int (*ScratchFn)(size_t need, void* stream, void** workspace, size_t* workspace_bytes);
int forward_entry(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
                  const void* v, const int64_t v_strides[4], const void* routes, int routes_dtype,
                  const int64_t route_strides[3], int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                  int64_t D, int64_t K, float scale, void* out, void* workspace, size_t workspace_bytes,
                  ScratchFn scratch, void* stream);

// Range starts of each row's list for a split plan: offs [rows][P + 1].
hipError_t launch_range_offsets(const int32_t* route_list, const int32_t* route_count, int64_t rows, int64_t K,
                                int64_t S_kv, const SplitPlan& plan, int32_t* offs, hipStream_t stream);

// Fused gather-attention over compacted lists; with plan.use, the range
// starts, then per pass the split attention and the combine.
hipError_t launch_gather_attention(const AttnArgs& a, const SplitPlan& plan, const SplitBuffers& w,
                                   hipStream_t stream);

// Key segments (route lists regrouped by 64-key tile, rows ascending) and
// their split into parts for the key-side backward kernel.
constexpr int64_t kSegKeyTile = 64;     // keys per tile of the key-side backward (one workgroup)
constexpr int64_t kSegChunkRows = 256;  // query rows per popcount-prefix chunk
constexpr int64_t kSegMinPart = 64;     // smallest part length (segments)
constexpr int64_t kSegPartsTotal = 4096;  // target parts (workgroups) over all KV heads

struct SegmentBuffers {
  uint32_t* bits;         // [B][ceil(S_q/32)][n_kt] one bit per (query row, tile)
  int32_t* chunk_prefix;  // [B][ceil(S_q/256)][n_kt]
  int32_t* totals;        // [B * n_kt]
  int32_t* tile_start;    // [B * n_kt + 1]: segments of (b, t) are [start[b*n_kt+t], start[b*n_kt+t+1])
  int4* segs;             // [capacity] {query row within the batch, key mask lo, key mask hi, 0}
  int64_t capacity;
  int32_t* part_start;    // [B * n_kt + 1]
  int32_t* slot_start;    // [B * n_kt]
  int32_t* plan;          // [2]: part length, number of parts
  int64_t max_parts;      // parts per KV head the split aims at
};

hipError_t launch_key_segments(const int32_t* route_list, const int32_t* route_count, int64_t B, int64_t S_q,
                               int64_t K, int64_t S_kv, const SegmentBuffers& w, hipStream_t stream);

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;   // forward output [B, S_q, Hq, D], contiguous
  const uint16_t* dout;  // upstream gradient, strided like q
  int64_t qs[4], ks[4], vs[4], gs[4];
  const float* lse;      // [B * S_q * Hq] natural-log log-sum-exp of the forward
  float* delta;          // [B * S_q * Hq] <dout, out>, written by the dq pass
  const int32_t* route_list;
  const int32_t* route_count;
  const int32_t* seg_start;   // tile_start of the key segments
  const int4* segs;
  const int32_t* part_start;
  const int32_t* slot_start;
  const int32_t* plan;
  float* partial;             // [slots][Hkv][4 waves][2][D/16][64][4] fp32 partial sums of split tiles
  int64_t max_parts;
  int64_t B, S_q, S_kv, Hq, Hkv, D, K;
  float scale;
  uint16_t* dq;  // [B, S_q, Hq, D] contiguous
  uint16_t* dk;  // [B, S_kv, Hkv, D] contiguous
  uint16_t* dv;  // [B, S_kv, Hkv, D] contiguous
  // key-range split of dq (the forward's plan): range starts and fp32 partial sums of a pass, in two
  // buffers when there is more than one pass (the same buffer twice otherwise)
  SplitPlan split;
  int32_t* offs;         // [B * S_q][P + 1]
  float* dq_part[2];     // [dq_pass_rows][Hkv][P][G][D] each
  int64_t dq_pass_rows;
};

constexpr int64_t kDqPassRows = 4096;  // rows per pass of the split dq (two partial buffers of them)

// dq and delta (one wavefront per (b, i, hk)); then dk and dv (one wavefront
// workgroup per (part of a 64-key tile, hk)) over the key segments.
hipError_t launch_attention_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attention_dkdv(const BwdArgs& a, hipStream_t stream);

// Route selection by compressed-block scores (scores into `scores`, then a
// per-row top-k), in passes of whole row tiles that fit workspace_bytes.
struct SelectArgs {
  const uint16_t* iq;  // [B, S_q, H, D] bf16
  const uint16_t* ck;  // [B, n_blocks, 1, D] bf16
  int64_t qs[4], cs[4];
  const int64_t* seq_lens;  // [B]
  int64_t B, S_q, H, D, q_offset, token_budget, compress_ratio;
  int32_t* out;    // [B, S_q, token_budget + compress_ratio - 1]
  float* scores;   // workspace
  size_t workspace_bytes;
};

int64_t select_rows_per_tile(int64_t H);  // query rows per score workgroup (16, 8 or 4)
int64_t select_score_ld(int64_t S_q, int64_t q_offset, int64_t c);  // floats per score row
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

// Upper bound of the partial-sum slots the split can use, per KV head.
inline int64_t seg_max_slots(int64_t max_parts, int64_t capacity) {
  const int64_t by_capacity = (capacity + kSegMinPart - 1) / kSegMinPart;
  return 2 * (max_parts < by_capacity ? max_parts : by_capacity);
}

}  // namespace qsa

// Internal launchers shared by the C-ABI entry points (not exported).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qsa {

// Route normalisation: [B*S_q rows, K slots] -> ascending distinct valid IDs.
// When zero_buf is non-null the same launch also sets its zero_count int32
// entries to 0 (the tile member counters of the membership pass).
hipError_t launch_route_normalize(const void* routes, bool routes_int64, int64_t B, int64_t S_q,
                                  int64_t K, const int64_t route_strides[3], int64_t kv_length,
                                  int32_t* route_list, int32_t* route_count, int32_t* zero_buf,
                                  int64_t zero_count, hipStream_t stream);

// Membership table and/or 128x128 tile classes from compacted lists.
hipError_t launch_membership_tiles(const int32_t* route_list, const int32_t* route_count, int64_t B,
                                   int64_t S_q, int64_t K, int64_t kv_length, uint8_t* membership,
                                   int32_t* tile_class, hipStream_t stream);

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
};

// Fused gather-attention over compacted lists.
hipError_t launch_gather_attention(const AttnArgs& a, hipStream_t stream);

}  // namespace qsa

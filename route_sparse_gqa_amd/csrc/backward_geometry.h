// Tile geometry shared by the backward kernels: dq (attention_backward.hip)
// and dk/dv (dkdv.hip), which are built with different MFMA register forms.
#pragma once

namespace qsa {
namespace bwd {

constexpr int kWaves = 4;   // work units per workgroup
constexpr int kChunk = 16;  // keys per dq iteration; keys per dkdv tile; MFMA rows per dkdv batch

template <int D>
struct Geo {
  static constexpr int kSteps = D / 32;                 // 32-dim k-steps of the score products
  static constexpr int kDimTiles = D / 16;              // 16-dim output tiles
  static constexpr int kLanesPerRow = D / 8;            // 16-byte pieces per row
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kLoads = kChunk / kRowsPerLoad;  // load instructions per 16 rows
  static constexpr int kTrStride = D + 16;              // slabs read transposed: 2D + 32 bytes per row
  static constexpr int kRowStride = D + 8;              // slabs read by rows only: 2D + 16 bytes per row
};

}  // namespace bwd
}  // namespace qsa

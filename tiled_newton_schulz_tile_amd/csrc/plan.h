// Host-side planning of a HiMuon step: validation, the tile partition of every
// layer, the split of tiles between the fused kernel and the large-tile GEMM path,
// chunking of the GEMM path under the workspace budget, and the step's counters.
// Pure host code: nothing here touches a device.
#pragma once

#include <string>
#include <vector>

#include "himuon.h"
#include "himuon_internal.h"

namespace himuon {

// Kernel tile edge of the fused path for a tile whose longer side is e (0 if the
// tile needs the GEMM path).
int fused_edge_for(int64_t e);

struct FusedGroup {
  int ts;             // kernel tile edge
  bool dense;         // tiles fill ts x ts exactly, rows 16-byte aligned
  int64_t first, n;   // range in Plan::ftiles
};

struct Range {
  int64_t first = 0, n = 0;
};

struct GemmChunk {
  int64_t first, n;   // range in Plan::gtiles
  size_t ws_bytes;    // workspace the chunk uses
  Range mom, stg, sym, upd, app;  // ranges in the work lists
  bool long_k;        // every GEMM K of its tiles >= kGemmLongK: K slices of 64
  bool t256;          // every tile 256 x 256 and bf16 planes: one workgroup per tile product
  bool b256;          // otherwise every side a multiple of 256, bf16 planes: 256-blocks
};

struct Plan {
  std::vector<himuon_layer> layers;
  std::vector<LayerDesc> ldesc;
  himuon_config cfg{};
  F8Exps f8{};                 // fp8 plane exponents (HIMUON_PREC_BF16F8)
  int32_t tile = 0;
  std::vector<FusedTile> ftiles;    // grouped by kernel edge, each group in table order
  std::vector<FusedGroup> fgroups;
  std::vector<GemmTile> gtiles;
  std::vector<GemmChunk> chunks;
  // work lists of the GEMM path, concatenated over chunks
  std::vector<GemmWork> wmom, wstg, wsym, wupd, wapp;
  std::vector<himuon_tile> order;   // every tile in table order (layer, row-major)
  himuon_stats stats{};
  size_t workspace_bytes = 0;
};

// Validates and fills everything but the partition.  Returns HIMUON_OK or an error
// with a message in err.
himuon_status plan_init(Plan &p, const himuon_layer *layers, int32_t n, const himuon_config *cfg,
                        std::string &err);

// (Re)builds the partition for tile size T (0 = FULL).
himuon_status plan_partition(Plan &p, int32_t tile, std::string &err);

}  // namespace himuon

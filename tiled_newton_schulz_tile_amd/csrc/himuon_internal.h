// Internal descriptors shared by the host planner (plan.cpp, api.cpp) and the HIP
// kernels.  Plain structs with fixed layout: they are copied byte for byte into
// device memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace himuon {

// Per-layer device descriptor.
struct LayerDesc {
  float *w;           // fp32 weights
  void *m;            // momentum (state dtype)
  const void *g;      // gradient (state dtype)
  float *u;           // optional fp32 update output
  int64_t ld_w, ld_m, ld_g, ld_u;
  int32_t rows, cols;
  int32_t vec_ok;     // 1 when M, G rows allow 16-byte vector access at 8-element steps
  int32_t vec_w;      // 1 when W (and U) rows allow 16-byte vector access at 4-float steps
};
static_assert(sizeof(LayerDesc) == 80, "LayerDesc layout");

// One tile of the fused path (tile edge <= kernel tile edge).
struct FusedTile {
  int32_t layer;
  int32_t row0, col0;
  int16_t h, w;
};
static_assert(sizeof(FusedTile) == 16, "FusedTile layout");

// One tile (or whole matrix) of the large-tile GEMM path.
struct GemmTile {
  int32_t layer;
  int32_t row0, col0;
  int32_t h, w;       // global orientation
  int32_t r, s;       // oriented: r = min(h, w) rows, s = max(h, w) columns
  int32_t tall;       // h > w: the tile is iterated transposed
  int64_t ws_x0, ws_x1, ws_a, ws_b;  // byte offsets into the workspace (per chunk)
  int64_t ws_scale;   // byte offset of the tile's fp32 scale / norm accumulator
};

enum Prec : int { PREC_F32 = 0, PREC_BF16 = 1, PREC_BF16X3 = 2 };

struct NSParams {
  float a, b, c;
  float beta, eps, lr;
  int32_t steps;
  int32_t write_update;
};

// ---- launchers (ns_fused.hip) --------------------------------------------------
// Runs momentum, K NS steps and the weight update for every tile of `tiles`
// (device array of n FusedTile) with kernel tile edge ts in {32, 64, 128}.  dense:
// every tile is exactly ts x ts with 16-byte aligned rows (no edge handling).
hipError_t launch_fused(int ts, int prec, int state_bf16, bool dense, const LayerDesc *layers,
                        const FusedTile *tiles, int64_t n, const NSParams &p,
                        hipStream_t stream);

// LDS bytes one workgroup of the fused kernel uses (for the planner's stats).
size_t fused_lds_bytes(int ts, int prec);

}  // namespace himuon

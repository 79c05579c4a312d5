// Internal descriptors shared by the host planner (plan.cpp, api.cpp) and the HIP
// kernels.  Plain structs with fixed layout: they are copied byte for byte into
// device memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "himuon.h"

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

// One tile (or whole matrix) of the large-tile GEMM path.  Its workspace holds the
// oriented tile X (r x s, two buffers), A and B (r x r) as row-major planes with
// leading dimensions ldx = roundup(s, 64) and lda = roundup(r, 64) (zero padded):
// fp32 planes for PREC_F32, else a bf16 "hi" plane followed by a bf16 "lo" plane.
// 256 x 256 tiles run in place: one X buffer (ws_x1 = ws_x0) and B over A (ws_b = ws_a).
struct GemmTile {
  int32_t layer;
  int32_t row0, col0;
  int32_t h, w;       // global orientation
  int32_t r, s;       // oriented: r = min(h, w) rows, s = max(h, w) columns
  int32_t tall;       // h > w: the tile is iterated transposed
  int32_t ldx, lda;   // padded leading dimensions of the X and A/B planes (elements)
  int32_t nred;       // momentum blocks (partial sums of squares)
  int32_t pad_;
  int64_t ws_x0, ws_x1, ws_a, ws_b;  // byte offsets into the workspace
  int64_t ws_red;     // nred fp32 partial sums, then the tile's 1 / (||Y||_F + eps)
};
static_assert(sizeof(GemmTile) == 88, "GemmTile layout");

// One work item of a grouped launch of the GEMM path: tile index (into the plan's
// GemmTile table) and block coordinates.
struct GemmWork {
  int32_t tile, bi, bj;
};

// Elements per momentum block of the GEMM path.
constexpr int kGemmMomentumBlock = 8192;
// GEMM products whose K (the padded short and long side of every tile in a chunk) is at
// least this long stream K slices of 64 elements (whole 128-byte lines of bf16 rows)
// through one LDS stage; shorter ones use slices of 32 through two stages, which hides
// more latency when a block has only a few slices.
constexpr int64_t kGemmLongK = 1024;
// Block rows per group in the work order of long-K products.
constexpr int kGemmGroupRows = 8;

enum Prec : int { PREC_F32 = 0, PREC_BF16 = 1, PREC_BF16X3 = 2, PREC_BF16F8 = 3 };

// Power-of-two scales of the fp8 planes (PREC_BF16F8), per NS step k (the last entry
// serves every later step): the e4m3 hi plane of a matrix holds x * 2^e, its lo plane
// (x - bf16(x)) * 2^(e + 8).  e is chosen from a bound on the matrix's entries so that
// no scaled value reaches the e4m3 range limit.
constexpr int kF8Steps = 16;
struct F8Exps {
  int8_t x[kF8Steps];   // X_k (input of step k); x[k + 1] for the X stored by step k
  int8_t a[kF8Steps];   // A_k = X_k X_k^T, stored as the operand of A^2 (c != 0)
  int8_t b[kF8Steps];   // B_k = b A_k + c A_k^2, the update's operand (a X_k is added in fp32)
};

// PREC_BF16F8 on full e x e tiles of the fused kernel: the Gram product of the first
// kF8PlainGramSteps NS steps, and the square product of the first
// f8_plain_square_steps(e, dense) steps (with A stored as its bf16 plane alone), take the
// bf16 operands only.  (128-tiles outside the dense group, whose kernel instance has no
// registers to spare for the plain square, keep the split square.)  On dense 128-tiles
// the update product B X of the first f8_plain_update_steps(e, dense) steps takes them
// too, except in the last step (B stored as its bf16 plane alone; the a X term stays in
// fp32), and X_0, which then no product reads in split form, is stored without its e4m3
// planes.  (Other 128-tiles lack the registers; on 64-tiles the plain update raised the
// error of quintic runs with K = 8 on ragged stacks above 5e-3 max-abs.)  Dense 128-tiles
// run the Gram product of the first f8_plain_gram_steps(e, dense) steps plain, and an X
// whose next Gram and update are both plain is stored as bf16 hi + lo alone.
constexpr int kF8PlainGramSteps = 1;
constexpr int f8_plain_square_steps(int edge, bool dense) { return edge == 128 && !dense ? 0 : 2; }
constexpr int f8_plain_gram_steps(int edge, bool dense) { return edge == 128 && dense ? 2 : kF8PlainGramSteps; }
constexpr int f8_plain_update_steps(int edge, bool dense) { return edge == 128 && dense ? 2 : 0; }

struct NSParams {
  float a, b, c;
  float beta, eps, lr;
  int32_t steps;
  int32_t write_update;
  int32_t identity;  // gather -> scatter only: no normalisation (steps is 0 then)
  F8Exps f8;
  // PREC_BF16F8 requests on 256-tiles (run with the bf16x3 products): the Gram product of
  // the first plain_gram NS steps and the square product of the first plain_square take
  // the bf16 hi operands only, as on full fused tiles; 0 for every other request
  int32_t plain_gram, plain_square;
};

// Fills e with the fp8 plane exponents for coefficients (a, b, c) over `steps` steps;
// returns false if some bound is not finite (the coefficients blow up).
bool f8_exponents(double a, double b, double c, int steps, F8Exps &e);

// Sets the calling thread's himuon_last_error() message and returns s (api.cpp).
himuon_status set_error(himuon_status s, const std::string &msg);

// ---- launchers (ns_fused.hip) --------------------------------------------------
// Runs momentum, K NS steps and the weight update for every tile of `tiles`
// (device array of n FusedTile) with kernel tile edge ts in {32, 64, 128}.  dense:
// every tile is exactly ts x ts with 16-byte aligned rows (no edge handling).
hipError_t launch_fused(int ts, int prec, int state_bf16, bool dense, const LayerDesc *layers,
                        const FusedTile *tiles, int64_t n, const NSParams &p,
                        hipStream_t stream);

// LDS bytes one workgroup of the fused kernel uses (for the planner's stats).
size_t fused_lds_bytes(int ts, int prec);

// ---- launchers (ns_gemm.hip) ---------------------------------------------------
// Work lists of one chunk of the GEMM path (device arrays).
struct GemmChunkLaunch {
  int64_t tile_first, tile_n;          // tiles [first, first + n) of the table
  const GemmWork *mom;  int64_t n_mom; // (tile, block, 0): momentum blocks
  const GemmWork *stg;  int64_t n_stg; // (tile, bi, bj): 64-blocks of the oriented X
  const GemmWork *sym;  int64_t n_sym; // (tile, bi <= bj): 128-blocks of r x r
  const GemmWork *upd;  int64_t n_upd; // (tile, bi, bj): 128-blocks of r x s
  const GemmWork *app;  int64_t n_app; // (tile, bi, bj): 64-blocks of the h x w tile
  int32_t long_k;                       // K slices of 64 (one LDS stage) instead of 32 (two)
  int32_t t256;                         // every tile 256 x 256 (bf16 planes): one workgroup
                                        // per tile and product; sym / upd lists unused
  int32_t b256;                         // every side a multiple of 256 (bf16 planes): sym /
                                        // upd lists hold 256-blocks
};
// Runs one full step for the tiles of a chunk: momentum and partial norms, norm
// reduction, staging of X0, K Newton-Schulz steps as grouped MFMA GEMMs, update.
hipError_t launch_gemm_chunk(int prec, int state_bf16, const LayerDesc *layers, const GemmTile *tiles,
                             const GemmChunkLaunch &c, char *workspace, const NSParams &p,
                             hipStream_t stream);

// ---- flat memory-pass reference (stream.hip) -------------------------------------
// M <- beta M + G (stored in the state dtype), W <- W - lr M over n contiguous elements.
hipError_t launch_stream_step(void *m, const void *g, float *w, int64_t n, bool state_bf16, float beta, float lr,
                              hipStream_t stream);

// ---- Sign-Muon local kernels (sign.hip) -----------------------------------------
// Sign of a rows x cols fp32 matrix (leading dimension ld) packed to one bit per entry
// (row-major entry k at byte k / 8, bit k % 8; 1 = non-negative).  bits: 8-byte aligned,
// ceil(rows * cols / 8) bytes.
hipError_t launch_sign_pack(const float *o, int64_t rows, int64_t cols, int64_t ld, unsigned char *bits,
                            hipStream_t stream);
// Majority vote over `workers` packed buffers (worker m at bits + m * stride; bits and
// stride 4-byte aligned): out[k] = +-scale, ties +scale; out fp32 or bf16.
hipError_t launch_sign_vote(const unsigned char *bits, int workers, int64_t stride, int64_t n, bool out_bf16,
                            void *out, float scale, hipStream_t stream);

}  // namespace himuon

/*
 * himuon.h -- C ABI of libhimuon, the HiMuon (Hierarchical Muon) optimizer step on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described in "Hierarchical Muon: Tiled Newton-Schulz
 * Updates for Efficient Muon Optimization" (Abstract): every momentum-gradient
 * matrix is cut into T x T tiles, the same finite Newton-Schulz (NS) map runs on
 * each tile independently, and the tile results are put back in place and applied
 * to the weights.  The page names tile-size-dependent GPU kernels, cross-layer
 * batching, memory-bounded chunking and runtime tile-size schedules as what this
 * structure allows; this library provides each of them.
 *
 * One step, for every layer (W fp32 H x W weights, M momentum, G gradient):
 *   M <- beta * M + G                       (formed as one fp32 fused multiply-add,
 *                                            stored in the momentum dtype, RNE)
 *   for every tile Y of M (row-major grid anchored at (0,0), ragged edge tiles
 *   kept at their own h x w size; T = HIMUON_TILE_FULL or T >= max(H, W) is one
 *   tile per matrix):
 *     X = Y / (||Y||_F + eps), transposed when h > w so that X is r x s, r <= s
 *     K times:  A = X X^T;  X <- a X + (b A + c A^2) X
 *     O_tile = X (transposed back when h > w)
 *   W <- W - lr * O
 * The coefficients (a, b, c) are a parameter: cubic (1.5, -0.5, 0) and quintic
 * (3.4445, -4.7750, 2.0315) are the two shipped settings.
 *
 * Conventions for every entry point:
 *  - returns himuon_status; never throws; never blocks on the GPU except where
 *    stated; a failure leaves a message in himuon_last_error() (per thread).
 *  - matrices are row-major; ld_* are leading dimensions in elements (>= cols).
 *  - all device pointers are owned by the caller and must stay valid while a
 *    step that uses them is in flight.  Layers must not alias one another.
 */
#ifndef HIMUON_H
#define HIMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define HIMUON_API __attribute__((visibility("default")))
#else
#define HIMUON_API
#endif

typedef enum {
  HIMUON_OK = 0,
  HIMUON_EINVAL = -1,       /* bad argument, shape, leading dimension or config   */
  HIMUON_EBUDGET = -2,      /* workspace budget below what one tile needs          */
  HIMUON_ENOMEM = -3,       /* host or device allocation failed                    */
  HIMUON_EDEVICE = -4,      /* HIP runtime error (launch, copy, no device)         */
  HIMUON_EUNSUPPORTED = -5  /* valid request the library does not implement        */
} himuon_status;

/* storage dtype of momentum and gradient */
typedef enum { HIMUON_F32 = 0, HIMUON_BF16 = 1 } himuon_dtype;

/* arithmetic of the NS matrix products (all accumulate in fp32) */
typedef enum {
  HIMUON_PREC_F32 = 0,    /* fp32 operands (fp32 MFMA)                                  */
  HIMUON_PREC_BF16 = 1,   /* operands rounded once to bf16, one bf16 MFMA per product   */
  HIMUON_PREC_BF16X3 = 2, /* operands split x = hi + lo (both bf16), three bf16 products
                             hi*hi + hi*lo + lo*hi per product: fp32-class accuracy at
                             3x the bf16 MFMA work                                       */
  HIMUON_PREC_BF16F8 = 3  /* the same split, with the two correction products hi*lo and
                             lo*hi on e4m3 (fp8) MFMA at twice the bf16 rate: 2x the bf16
                             MFMA time; each fp8 operand carries a power-of-two scale
                             chosen at plan time from bounds on the iterates.  Fused tiles
                             of edge 64 and 128 run it; smaller tiles and the large-tile
                             path run HIMUON_PREC_BF16X3 (256-tiles and 256-blocks with
                             the plain early Gram and square below).  On tiles that fill
                             64 x 64 or 128 x 128, the Gram product of NS step 0 and the
                             square product of steps 0 and 1 use the bf16 hi operands
                             alone, and on dense 128-tiles (full, 16-byte aligned rows)
                             so do the Gram and B X products of step 1 and the B X
                             product of step 0 (never the last step's B X); other
                             128-tiles keep the split square and update.
                             The a X term of each step is added in fp32 from X
                             held to about 2^-17 (bf16 hi + lo, or fp32), not through the
                             e4m3 operands, so rounding noise does not build up in the
                             empty directions of low-rank tiles.  himuon_plan returns
                             HIMUON_EINVAL if the coefficients' iterates are unbounded.   */
} himuon_precision;

#define HIMUON_TILE_FULL 0            /* one tile per matrix: full-matrix Muon        */
#define HIMUON_FLAG_WRITE_UPDATE 1u   /* also store O (fp32) to layer.update          */
/* Test mode: the step runs the momentum update, the gather of every tile (oriented on its
   short side) and the scatter back, with no normalisation and no Newton-Schulz step, so
   O = M as stored.  O, W <- W - lr O and, with HIMUON_FLAG_WRITE_UPDATE, U = O are
   bit-exact copies of the stored momentum whenever the path holds X in fp32
   (HIMUON_PREC_F32) or the state is bf16; it checks tile indexing and reassembly.  The
   plan's steps and coefficients are ignored while it is set.                          */
#define HIMUON_FLAG_IDENTITY_MAP 2u

typedef struct { double a, b, c; } himuon_coeffs;

typedef struct {
  int64_t rows, cols;            /* H, W                                               */
  int64_t ld_w, ld_m, ld_g, ld_u;/* leading dimensions in elements, >= cols            */
  float *weight;                 /* device, fp32 master weights, updated in place      */
  void *momentum;                /* device, state dtype, updated in place              */
  const void *grad;              /* device, state dtype, read only                     */
  float *update;                 /* device fp32 H x W or NULL; written when the plan has
                                    HIMUON_FLAG_WRITE_UPDATE                           */
} himuon_layer;

typedef struct {
  int32_t tile;                  /* T >= 1, or HIMUON_TILE_FULL                        */
  int32_t steps;                 /* K >= 0                                             */
  himuon_coeffs coeffs;          /* (a, b, c)                                          */
  float beta;                    /* momentum factor, e.g. 0.95                         */
  float eps;                     /* normaliser guard, e.g. 1e-7 (>= 0); a zero tile maps
                                    to zero for every eps, 0 included.  ||Y||_F is
                                    formed in fp32; where the sum of squares leaves
                                    [2^-100, 2^100] it is recomputed from the tile
                                    scaled by a power of two, so very large and very
                                    small tiles normalise as in exact arithmetic (on
                                    the large-tile path while ||Y||_F < 2^126)         */
  size_t workspace_budget;       /* bytes of caller workspace the plan may use         */
  himuon_dtype state_dtype;      /* dtype of momentum and grad, same for all layers    */
  himuon_precision precision;    /* arithmetic of the NS products                      */
  uint32_t flags;                /* HIMUON_FLAG_*                                      */
} himuon_config;

typedef struct {
  int32_t tile;                  /* current T (0 = FULL)                               */
  int32_t kernel_tile;           /* LDS tile edge of the fused kernel (32/64/128), or 0
                                    when the large-tile GEMM path runs                 */
  int64_t layers, tiles;         /* tiles of the current partition                     */
  int64_t fused_tiles;           /* tiles run by the fused kernel                      */
  int64_t gemm_tiles;            /* tiles run by the large-tile GEMM path              */
  int64_t chunks;                /* launches groups of the GEMM path (>= 1 if any)     */
  size_t workspace_bytes;        /* workspace one step needs (<= budget)               */
  size_t table_bytes;            /* device bytes of the descriptor tables              */
  double ns_flops;               /* algorithmic NS flops per step:
                                    sum over tiles K (4 r^2 s + 2 r^3 [c != 0])        */
  double issued_flops;           /* MFMA flops issued per step (padding, symmetric
                                    blocks and the BF16X3 split included)              */
  double step_bytes;             /* algorithmic HBM bytes per step: G, M read, M
                                    written (state dtype), W read and written (fp32)   */
} himuon_stats;

typedef struct {
  int32_t layer;                 /* index into the plan's layer list                   */
  int32_t transposed;            /* 1 when h > w (iterated on the transpose)           */
  int64_t row0, col0, rows, cols;/* tile origin and size inside its matrix             */
} himuon_tile;

/* Runtime calls a plan has made so far (for callers that must know which calls allocate
   or wait): device allocations, pinned host allocations, and host waits on the GPU
   (blocking copies, event waits).  himuon_step adds to none of them. */
typedef struct {
  int64_t device_allocs;
  int64_t host_allocs;
  int64_t host_waits;
} himuon_runtime_counts;

typedef struct himuon_plan_s himuon_plan_t;

/* Validate the layers and config and build the tile-descriptor table over all layers
 * (row-major tiles, layers in order), the chunk list of the large-tile path and the
 * workspace layout.  The plan binds to the current HIP device: it allocates the device
 * copy of the tables there and uploads it with a blocking copy.  When no GPU is
 * visible the plan is host-only (stats and tiles work; himuon_step returns EDEVICE).
 * The layer array is copied; the layers' device pointers are not touched.  EINVAL: bad
 * shape/ld/pointer/config, including coefficients that are not finite in fp32, a
 * nonzero c that rounds to zero in fp32, or |b / c| > 2^100 (the kernels accumulate
 * c A^2 + b A as c ((b / c) A + A^2) in fp32); EBUDGET: the budget cannot hold the
 * workspace of the largest single tile; ENOMEM / EDEVICE: the device tables could not be
 * allocated or copied.  */
HIMUON_API himuon_status himuon_plan(const himuon_layer *layers, int32_t n_layers,
                          const himuon_config *cfg, himuon_plan_t **out);

/* Workspace bytes one step of this plan needs (<= cfg.workspace_budget; 0 when every
 * tile runs in the fused kernel). */
HIMUON_API himuon_status himuon_workspace_size(const himuon_plan_t *p, size_t *bytes);

/* Enqueue one full step (momentum, tiled NS, weight update) for every layer on
 * hip_stream (a hipStream_t; NULL = the default stream).  workspace is a device
 * buffer of at least himuon_workspace_size bytes (may be NULL when that is 0).
 * Enqueue only: it allocates nothing and never waits for the GPU, so it may be
 * captured into a HIP graph.  Steps and tile-size changes of one plan go on one
 * stream (or the caller orders them).  EINVAL: workspace too small, non-finite lr,
 * another current device than the plan's; EDEVICE: a launch failed, or the plan is
 * host-only. */
HIMUON_API himuon_status himuon_step(himuon_plan_t *p, void *workspace, size_t ws_bytes,
                          float lr, void *hip_stream);

/* Change T between steps (runtime tile-size schedule).  Rebuilds the tables on the
 * host and enqueues their upload on hip_stream into the plan's second device buffer
 * (the one the steps before the last change read), so steps enqueued later on that
 * stream use the new T and steps already queued keep theirs.  It allocates only when
 * the new tables outgrow that buffer or its pinned staging (outgrown buffers are kept
 * until himuon_plan_destroy), and waits only when the staging is still being read by
 * the upload of the change before the previous one.  A new T whose workspace exceeds
 * the budget gives more chunks, not an error, unless a single tile does not fit
 * (EBUDGET); on any error the plan keeps its current T. */
HIMUON_API himuon_status himuon_set_tile_schedule(himuon_plan_t *p, int32_t tile, void *hip_stream);

/* Runtime calls (allocations, host waits) the plan has made since himuon_plan. */
HIMUON_API himuon_status himuon_plan_runtime_counts(const himuon_plan_t *p, himuon_runtime_counts *out);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): himuon_step with the large-tile
 * path's workspace taken from a static per-device array of
 * HIMUON_STATIC_WORKSPACE_BYTES (each GPU the library runs on holds its own copy until
 * the process ends) instead of a caller buffer.  It allocates nothing and never waits
 * for the GPU.  Plans that need no workspace (every tile in the fused kernel) run as
 * with himuon_step.  Calls on one GPU share the array, so steps that overlap on one
 * device (on different streams, or from different threads) race on it; the array
 * needs no clearing (each step writes every workspace byte it reads).  EBUDGET: the
 * plan's workspace exceeds HIMUON_STATIC_WORKSPACE_BYTES (plan with a workspace_budget
 * at most that large: the large-tile path then runs in more chunks); other errors as
 * for himuon_step. */
#define HIMUON_STATIC_WORKSPACE_BYTES (64u << 20)
HIMUON_API himuon_status himuon_step_static(himuon_plan_t *p, float lr, void *hip_stream);

/* Counters of the current partition. */
HIMUON_API himuon_status himuon_plan_stats(const himuon_plan_t *p, himuon_stats *out);

/* Copy up to cap tile descriptors (in table order) into out; *n receives the total
 * number of tiles.  out may be NULL with cap 0 to query the count. */
HIMUON_API himuon_status himuon_plan_tiles(const himuon_plan_t *p, himuon_tile *out, int64_t cap,
                                int64_t *n);

/* Release the plan and its device tables.  The caller synchronises the stream of
 * the last step first. */
HIMUON_API void himuon_plan_destroy(himuon_plan_t *p);

/* Message of the last failure on this thread ("" if none). */
HIMUON_API const char *himuon_last_error(void);

/* The momentum and weight update of the step with the map O = M, over one flat run of n
   elements and no tiling: M <- beta M + G (one fp32 fused multiply-add, stored in
   state_dtype with round-to-nearest-even), W <- W - lr M (M as stored).  It moves the
   bytes of a step's memory pass (the momentum and weight lines of the step described at
   the top of this file) and nothing else, so its rate is the HBM rate that read/write mix
   reaches on the device: the reference against which the tiled step's memory pass is
   measured.  For the same values its M and W are bit-exact to himuon_step's with
   HIMUON_FLAG_IDENTITY_MAP (bf16 state, or fp32 state with HIMUON_PREC_F32).  m, g: device arrays of n elements of
   state_dtype (HIMUON_F32 or HIMUON_BF16); w: device fp32, n elements; when all three
   are 16-byte aligned the kernel moves 8 elements per thread and turn.  Enqueued on
   hip_stream.  EINVAL: NULL pointers with n > 0, n < 0, a bad dtype, non-finite beta or
   lr.  EDEVICE: launch failure.                                                       */
HIMUON_API himuon_status himuon_stream_step(void *m, const void *g, float *w, int64_t n,
                                            himuon_dtype state_dtype, float beta, float lr,
                                            void *hip_stream);

/* ---- Sign-Muon, local pieces ----------------------------------------------------
   "Sign-Muon: Communication-Efficient Distributed Muon Optimization" (Figures 1 and 6):
   a worker forms the entrywise sign S in {-1, +1} of its Newton-Schulz direction, packs
   it to one bit per entry for an all-gather, and takes the majority vote of the gathered
   buffers locally.  The collective itself is not part of this library.                */

/* Packs sign(o) of a rows x cols fp32 device matrix (row-major, leading dimension
   ld >= cols) into `bits` (device, 8-byte aligned, ceil(rows * cols / 8) bytes, written
   in full): entry k = i * cols + j is bit k % 8 (least significant first) of byte k / 8,
   1 for o >= 0 (so sign(0) = +1), 0 otherwise (NaN included).  Enqueued on hip_stream.
   EINVAL: NULL pointers with rows * cols > 0, negative sizes, ld < cols, misaligned bits.
   EDEVICE: launch failure.                                                            */
HIMUON_API himuon_status himuon_sign_pack(const float *o, int64_t rows, int64_t cols, int64_t ld,
                                          uint8_t *bits, void *hip_stream);

/* Majority vote over the packed sign buffers of `workers` workers (1..255), worker m's
   buffer at bits + m * stride (device; bits and stride 4-byte aligned, stride >=
   ceil(n / 8)): out[k] = +scale if at least half of the workers have bit k set, else
   -scale, for k < n (a tie counts as +1).  out: device array of n elements of out_dtype
   (HIMUON_F32 or HIMUON_BF16).  Enqueued on hip_stream.  EINVAL on bad arguments,
   EDEVICE on launch failure.                                                          */
HIMUON_API himuon_status himuon_sign_vote(const uint8_t *bits, int32_t workers, int64_t stride, int64_t n,
                                          himuon_dtype out_dtype, void *out, float scale, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HIMUON_H */

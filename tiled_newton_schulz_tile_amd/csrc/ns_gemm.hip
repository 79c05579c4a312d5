// Large-tile path of the HiMuon step on gfx950: tiles longer than 128 (T > 128) and
// full matrices (T = FULL, full-matrix Muon).  The same finite Newton-Schulz map as the
// fused kernel ("Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
// Optimization", Abstract), run as grouped GEMMs over every tile of a workspace chunk,
// with X, A and B resident in HBM between launches (memory-bounded chunking: the host
// cuts the tile list into chunks whose workspace fits the caller's budget).
//
// Per chunk and step:
//   momentum     M <- beta M + G; per-block partial sums of squares (fixed order)
//   norm         per tile, the partials summed in a fixed order: 1 / (||Y||_F + eps)
//   stage        X0 = Y / (||Y|| + eps), oriented on the short side (LDS transpose for
//                tall tiles), written as planes (fp32, or bf16 hi + lo), zero padded
//   K times      A = X X^T           (symmetric: upper 128-blocks only, mirrored)
//                B = b A + c A A^T   (symmetric, epilogue adds b A; skipped when c = 0)
//                X <- (a I + B) X    (a on B's diagonal; plain bf16 adds a X in fp32)
//   apply        W <- W - lr O, O reoriented (LDS transpose for tall tiles)
// GEMM blocks are 128 x 128; K slices of 32 (two LDS stages) or, when every K of a chunk
// is long, of 64 (one stage) are staged through LDS from registers loaded one slice
// ahead; four waves each own a 64 x 64 block (2 x 2 MFMA 32x32 tiles).  Chunks whose
// sides are multiples of 256 use 256 x 256 blocks of eight waves (gemm_b256_kernel), and
// chunks of 256 x 256 tiles one workgroup per tile for all K steps, in place
// (gemm_t256_ns_kernel).
// Operands are read with plain (not non-temporal) loads: a K slice of 32 bf16 is half
// of a 128-byte line, and the other half is read by the next slice, from L2.
#include <type_traits>

#include "device_common.h"
#include "himuon_internal.h"

namespace himuon {
namespace {

using namespace dev;

constexpr int BM = 128;
constexpr int THREADS = 256;

enum Mode : int { MODE_GRAM = 0, MODE_SQUARE = 1, MODE_UPDATE = 2 };

struct GemmParams {
  float a, b, c;
  int xsel;      // X buffer read this step (0: ws_x0, 1: ws_x1); the other is written
  int fold;      // a added to B's diagonal (fp32, bf16x3); plain bf16 adds a X in fp32
  int plain_gram, plain_square;   // 256-tiles: early steps whose Gram / square take hi only
};

// Scalar copies of one GemmTile (read word by word so nothing lands in private memory).
struct TileG {
  int layer, row0, col0, h, w, r, s, tall, ldx, lda, nred;
  int64_t x0, x1, a, b, red;
};
__device__ __forceinline__ TileG tile_of(const GemmTile *tiles, int i) {
  const GemmTile *t = tiles + i;
  return TileG{t->layer, t->row0, t->col0, t->h,   t->w,    t->r,   t->s, t->tall,
               t->ldx,   t->lda,  t->nred, t->ws_x0, t->ws_x1, t->ws_a, t->ws_b, t->ws_red};
}

// Eight fp32 values as bf16 hi = RNE(v) and lo = RNE(v - hi), two elements per
// conversion; v - hi is exact in fp32, and hi is read back from the packed pair (low
// half: shift up, high half: mask) rather than converted again.
__device__ __forceinline__ void split8(const float (&v)[8], u32x4 &hb, u32x4 &lb) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hb[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    lb[q] = pack_bf16x2(v[2 * q] - __builtin_bit_cast(float, hb[q] << 16),
                        v[2 * q + 1] - __builtin_bit_cast(float, hb[q] & 0xffff0000u));
  }
}

// A matrix of `rows` rows and leading dimension ld in the workspace, in the
// precision's plane format.
template <int PREC>
struct Planes {
  char *base;
  int rows, ld;
  __device__ __bf16 *hi() const { return reinterpret_cast<__bf16 *>(base); }
  __device__ __bf16 *lo() const { return reinterpret_cast<__bf16 *>(base + (int64_t)rows * ld * 2); }
  __device__ float *f() const { return reinterpret_cast<float *>(base); }
  // fp32 value of element (i, j)
  __device__ __forceinline__ float get(int i, int j) const {
    const int64_t o = (int64_t)i * ld + j;
    if constexpr (PREC == PREC_F32) {
      return gmem(f())[o];
    } else {
      const unsigned short h = gmem(reinterpret_cast<const unsigned short *>(hi()))[o];
      const unsigned short l = gmem(reinterpret_cast<const unsigned short *>(lo()))[o];
      return bf16_bits_to_f32(h) + bf16_bits_to_f32(l);
    }
  }
  // fp32 values of 16 consecutive elements of row i from column j (j multiple of 16,
  // j + 16 <= ld): two 16-byte loads per plane
  __device__ __forceinline__ void get16(int i, int j, float (&v)[16]) const {
    const int64_t o = (int64_t)i * ld + j;
    if constexpr (PREC == PREC_F32) {
      const GLOBAL_AS f32x4 *s = reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(f() + o));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = s[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
      }
    } else {
      const GLOBAL_AS u32x4 *sh = reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(hi() + o));
      const GLOBAL_AS u32x4 *sl = reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(lo() + o));
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 h = sh[q], l = sl[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * q + 2 * e] = __builtin_bit_cast(float, h[e] << 16) + __builtin_bit_cast(float, l[e] << 16);
          v[8 * q + 2 * e + 1] = __builtin_bit_cast(float, h[e] & 0xffff0000u) +
                                 __builtin_bit_cast(float, l[e] & 0xffff0000u);
        }
      }
    }
  }
  // fp32 values of 8 consecutive elements of row i from column j (j multiple of 8,
  // j + 8 <= ld): one 16-byte load per bf16 plane
  __device__ __forceinline__ void get8(int i, int j, float (&v)[8]) const {
    const int64_t o = (int64_t)i * ld + j;
    if constexpr (PREC == PREC_F32) {
      const GLOBAL_AS f32x4 *s = reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(f() + o));
      const f32x4 x0 = s[0], x1 = s[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = x0[e];
        v[e + 4] = x1[e];
      }
    } else {
      const u32x4 h = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(hi() + o));
      const u32x4 l = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(lo() + o));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __builtin_bit_cast(float, h[e] << 16) + __builtin_bit_cast(float, l[e] << 16);
        v[2 * e + 1] = __builtin_bit_cast(float, h[e] & 0xffff0000u) + __builtin_bit_cast(float, l[e] & 0xffff0000u);
      }
    }
  }
  // store 8 consecutive values of row i starting at column j (j multiple of 8, j + 8 <= ld)
  __device__ __forceinline__ void put8(int i, int j, const float (&v)[8]) const {
    const int64_t o = (int64_t)i * ld + j;
    if constexpr (PREC == PREC_F32) {
      GLOBAL_AS f32x4 *d = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(f() + o));
      d[0] = f32x4{v[0], v[1], v[2], v[3]};
      d[1] = f32x4{v[4], v[5], v[6], v[7]};
    } else {
      u32x4 hb, lb;
      split8(v, hb, lb);
      *reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(hi() + o)) = hb;
      if constexpr (PREC == PREC_BF16X3 || PREC == PREC_BF16) *reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(lo() + o)) = lb;
    }
  }
  // store 16 consecutive values of row i starting at column j (j multiple of 16,
  // j + 16 <= ld)
  __device__ __forceinline__ void put16(int i, int j, const float (&v)[16]) const {
    const int64_t o = (int64_t)i * ld + j;
    if constexpr (PREC == PREC_F32) {
      GLOBAL_AS f32x4 *d = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(f() + o));
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else {
      GLOBAL_AS u32x4 *dh = reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(hi() + o));
      GLOBAL_AS u32x4 *dl = reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(lo() + o));
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float(&w)[8] = *reinterpret_cast<const float(*)[8]>(&v[8 * q]);
        u32x4 hb, lb;
        split8(w, hb, lb);
        dh[q] = hb;
        if constexpr (PREC == PREC_BF16X3 || PREC == PREC_BF16) dl[q] = lb;
      }
    }
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Fixed-order workgroup sum (4 waves); every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float *red4) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
  __syncthreads();
  const float s = (red4[0] + red4[1]) + (red4[2] + red4[3]);
  __syncthreads();
  return s;
}

// ------------------------------------------------------------------ momentum
// Work item (tile, block, -): elements [block * 8192, +8192) of the tile, row-major in
// its own orientation.  Stores the new momentum and the block's sum of squares of the
// stored values.
template <typename S>
__global__ __launch_bounds__(THREADS) void gemm_momentum_kernel(const LayerDesc *__restrict__ layers,
                                                                const GemmTile *__restrict__ tiles,
                                                                const GemmWork *__restrict__ work, char *ws,
                                                                float beta) {
  __shared__ float red4[4];
  const GemmWork wk = work[blockIdx.x];
  const TileG t = tile_of(tiles, wk.tile);
  const LayerDesc *L = layers + t.layer;
  S *mb = reinterpret_cast<S *>(L->m);
  const S *gb = reinterpret_cast<const S *>(L->g);
  const int64_t ldm = L->ld_m, ldg = L->ld_g;
  const bool vec = L->vec_ok;
  const int64_t total = (int64_t)t.h * t.w;
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kGemmMomentumBlock / (8 * THREADS); ++c) {
    const int64_t e0 = ((int64_t)wk.bi * (kGemmMomentumBlock / 8) + c * THREADS + threadIdx.x) * 8;
    if (e0 >= total) continue;
    const int i0 = (int)(e0 / t.w), j0 = (int)(e0 % t.w);
    if (vec && j0 + 8 <= t.w && ((t.col0 + j0) & 7) == 0) {
      const int64_t om = (int64_t)(t.row0 + i0) * ldm + t.col0 + j0;
      const int64_t og = (int64_t)(t.row0 + i0) * ldg + t.col0 + j0;
      if constexpr (sizeof(S) == 2) {
        const u32x4 m = __builtin_nontemporal_load(reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(mb + om)));
        const u32x4 g = __builtin_nontemporal_load(reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(gb + og)));
        unsigned short code[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const unsigned mw = m[q >> 1], gw = g[q >> 1];
          const float mv = __builtin_bit_cast(float, (q & 1) ? (mw & 0xffff0000u) : (mw << 16));
          const float gv = __builtin_bit_cast(float, (q & 1) ? (gw & 0xffff0000u) : (gw << 16));
          code[q] = to_bf16_bits(__builtin_fmaf(beta, mv, gv));
          const float v = bf16_bits_to_f32(code[q]);
          ss = __builtin_fmaf(v, v, ss);
        }
        *reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(mb + om)) =
            u32x4{code[0] | (unsigned)code[1] << 16, code[2] | (unsigned)code[3] << 16,
                  code[4] | (unsigned)code[5] << 16, code[6] | (unsigned)code[7] << 16};
      } else {
        const GLOBAL_AS f32x4 *pm = reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(mb + om));
        const GLOBAL_AS f32x4 *pg = reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(gb + og));
        f32x4 m0 = pm[0], m1 = pm[1];
        const f32x4 g0 = pg[0], g1 = pg[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          m0[q] = __builtin_fmaf(beta, m0[q], g0[q]);
          ss = __builtin_fmaf(m0[q], m0[q], ss);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          m1[q] = __builtin_fmaf(beta, m1[q], g1[q]);
          ss = __builtin_fmaf(m1[q], m1[q], ss);
        }
        GLOBAL_AS f32x4 *dm = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(mb + om));
        dm[0] = m0;
        dm[1] = m1;
      }
    } else {
      for (int q = 0; q < 8; ++q) {
        const int64_t e = e0 + q;
        if (e >= total) break;
        const int i = (int)(e / t.w), j = (int)(e % t.w);
        const int64_t om = (int64_t)(t.row0 + i) * ldm + t.col0 + j;
        const int64_t og = (int64_t)(t.row0 + i) * ldg + t.col0 + j;
        float v;
        if constexpr (sizeof(S) == 2) {
          const float mv = bf16_bits_to_f32(gmem(reinterpret_cast<const unsigned short *>(mb))[om]);
          const float gv = bf16_bits_to_f32(gmem(reinterpret_cast<const unsigned short *>(gb))[og]);
          const unsigned short code = to_bf16_bits(__builtin_fmaf(beta, mv, gv));
          gmem(reinterpret_cast<unsigned short *>(mb))[om] = code;
          v = bf16_bits_to_f32(code);
        } else {
          v = __builtin_fmaf(beta, gmem(mb)[om], gmem(gb)[og]);
          gmem(mb)[om] = v;
        }
        ss = __builtin_fmaf(v, v, ss);
      }
    }
  }
  ss = block_sum(ss, red4);
  if (threadIdx.x == 0) gmem(reinterpret_cast<float *>(ws + t.red))[wk.bi] = ss;
}

// ------------------------------------------------------------------ norm
// Fixed-order workgroup maximum (4 waves); every thread gets the result.
__device__ __forceinline__ float block_max(float v, float *red4) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
  __syncthreads();
  const float m = __builtin_fmaxf(__builtin_fmaxf(red4[0], red4[1]), __builtin_fmaxf(red4[2], red4[3]));
  __syncthreads();
  return m;
}

// One workgroup per tile: the partial sums in a fixed order; stores 1 / (sqrt(ss) + eps)
// (1 in the identity test mode).  Outside [2^-100, 2^100] (a zero tile, entries beyond
// about 1e15 or very small ones, an overflow) the fp32 sum of squares is recomputed from
// the stored momentum scaled by the power of two s = s1 s2 that brings its largest
// magnitude into [1/2, 1), and 1 / (|Y| + eps) = s / (s |Y| + s eps).  (That factor
// leaves the fp32 normal range only for |Y| beyond about 2^126.)
template <typename S>
__global__ __launch_bounds__(THREADS) void gemm_norm_kernel(const LayerDesc *__restrict__ layers,
                                                            const GemmTile *__restrict__ tiles, int first,
                                                            char *ws, float eps, int identity) {
  __shared__ float red4[4];
  const TileG t = tile_of(tiles, first + (int)blockIdx.x);
  GLOBAL_AS float *p = gmem(reinterpret_cast<float *>(ws + t.red));
  float ss = 0.f;
  for (int q = threadIdx.x; q < t.nred; q += THREADS) ss += p[q];
  ss = block_sum(ss, red4);
  float inv;
  if (!identity && !(ss >= 0x1p-100f && ss <= 0x1p100f)) {   // uniform over the workgroup
    const LayerDesc *L = layers + t.layer;
    const S *mb = reinterpret_cast<const S *>(L->m);
    const int64_t total = (int64_t)t.h * t.w, ldm = L->ld_m;
    auto at = [&](int64_t e) -> float {
      const int64_t o = (int64_t)(t.row0 + e / t.w) * ldm + t.col0 + e % t.w;
      if constexpr (sizeof(S) == 2) {
        return bf16_bits_to_f32(gmem(reinterpret_cast<const unsigned short *>(mb))[o]);
      } else {
        return gmem(mb)[o];
      }
    };
    float mx = 0.f;
    for (int64_t e = threadIdx.x; e < total; e += THREADS) mx = __builtin_fmaxf(mx, __builtin_fabsf(at(e)));
    mx = block_max(mx, red4);
    float s1 = 1.f, s2 = 1.f;
    if (mx > 0.f && mx <= 0x1.fffffep127f) {   // nonzero and finite
      int ex;
      (void)__builtin_frexpf(mx, &ex);
      s1 = __builtin_ldexpf(1.f, (-ex) / 2);
      s2 = __builtin_ldexpf(1.f, -ex - (-ex) / 2);
      float s2s = 0.f;
      for (int64_t e = threadIdx.x; e < total; e += THREADS) {
        const float v = at(e) * s1 * s2;
        s2s = __builtin_fmaf(v, v, s2s);
      }
      ss = block_sum(s2s, red4);
    }
    // a zero tile stays zero, also with eps = 0 (divisor 0)
    const float den = __builtin_sqrtf(ss) + (eps * s1) * s2;
    inv = den > 0.f ? (s1 / den) * s2 : (den == 0.f ? 0.f : den);   // a NaN (from NaN entries) passes on
  } else {
    // a zero tile stays zero, also with eps = 0 (divisor 0)
    const float den = __builtin_sqrtf(ss) + eps;
    inv = den > 0.f ? 1.0f / den : (den == 0.f ? 0.f : den);   // a NaN (from NaN entries) passes on
  }
  if (threadIdx.x == 0) p[t.nred] = identity ? 1.0f : inv;
}

// ------------------------------------------------------------------ stage / apply
// Tall tiles (transposed on their short side): 64 x 64 blocks through an LDS tile (pitch
// 65); thread t covers row t / 4, columns 16 (t % 4) .. +15 of the block.  Wide and square
// tiles need no transpose: strips of 16 rows x 256 columns, thread t covering row t / 16,
// columns 8 (t % 16) .. +7 and 128 + 8 (t % 16) .. +7, so that every load and store
// instruction of a wave covers contiguous runs of a row (512 B of fp32 weights, 256 B of
// each bf16 plane).
constexpr int SB = 64, SBP = 65;
constexpr int STRIP_R = 16, STRIP_C = 256;

// 16 consecutive state values of tile row gi from tile column gj, zero outside the tile.
template <typename S>
__device__ __forceinline__ void load_state16(const LayerDesc *L, const S *mb, int64_t ldm, const TileG &t, int gi,
                                             int gj, float (&v)[16]) {
  if (gi < t.h && gj + 16 <= t.w && L->vec_ok && ((t.col0 + gj) & 7) == 0) {
    const int64_t o = (int64_t)(t.row0 + gi) * ldm + t.col0 + gj;
    if constexpr (sizeof(S) == 2) {
      const GLOBAL_AS u32x4 *p = reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(mb + o));
      const u32x4 a = p[0], b = p[1];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const unsigned wa = a[q >> 1], wb = b[q >> 1];
        v[q] = __builtin_bit_cast(float, (q & 1) ? (wa & 0xffff0000u) : (wa << 16));
        v[q + 8] = __builtin_bit_cast(float, (q & 1) ? (wb & 0xffff0000u) : (wb << 16));
      }
    } else {
      const GLOBAL_AS f32x4 *p = reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(mb + o));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = p[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float x = 0.f;
      if (gi < t.h && gj + q < t.w) {
        const int64_t o = (int64_t)(t.row0 + gi) * ldm + t.col0 + gj + q;
        if constexpr (sizeof(S) == 2)
          x = bf16_bits_to_f32(gmem(reinterpret_cast<const unsigned short *>(mb))[o]);
        else
          x = gmem(mb)[o];
      }
      v[q] = x;
    }
  }
}

// 8 consecutive state values of tile row gi from tile column gj, zero outside the tile.
template <typename S>
__device__ __forceinline__ void load_state8(const LayerDesc *L, const S *mb, int64_t ldm, const TileG &t, int gi,
                                            int gj, float (&v)[8]) {
  if (gi < t.h && gj + 8 <= t.w && L->vec_ok && ((t.col0 + gj) & 7) == 0) {
    const int64_t o = (int64_t)(t.row0 + gi) * ldm + t.col0 + gj;
    if constexpr (sizeof(S) == 2) {
      const u32x4 a = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(mb + o));
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = __builtin_bit_cast(float, (q & 1) ? (a[q >> 1] & 0xffff0000u) : (a[q >> 1] << 16));
    } else {
      const GLOBAL_AS f32x4 *p = reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(mb + o));
      const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = x0[e];
        v[e + 4] = x1[e];
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float x = 0.f;
      if (gi < t.h && gj + q < t.w) {
        const int64_t o = (int64_t)(t.row0 + gi) * ldm + t.col0 + gj + q;
        if constexpr (sizeof(S) == 2)
          x = bf16_bits_to_f32(gmem(reinterpret_cast<const unsigned short *>(mb))[o]);
        else
          x = gmem(mb)[o];
      }
      v[q] = x;
    }
  }
}

// W <- W - lr o (and U <- o) for the n <= 16 weights of tile row gi from column gj.
__device__ __forceinline__ void apply16(const LayerDesc *L, const TileG &t, int gi, int gj, const float (&o)[16],
                                        float lr_, int write_u) {
  const int n = t.w - gj < 16 ? t.w - gj : 16;
  float *wrow = L->w + (int64_t)(t.row0 + gi) * L->ld_w + t.col0 + gj;
  const float nlr = -lr_;
  if (n == 16 && L->vec_w && ((t.col0 + gj) & 3) == 0) {
    GLOBAL_AS f32x4 *p = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(wrow));
    f32x4 x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = p[q];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[q][e] = __builtin_fmaf(nlr, o[4 * q + e], x[q][e]);
      p[q] = x[q];
    }
    if (write_u) {
      GLOBAL_AS f32x4 *u = reinterpret_cast<GLOBAL_AS f32x4 *>(
          gmem(L->u + (int64_t)(t.row0 + gi) * L->ld_u + t.col0 + gj));
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    }
  } else {
    GLOBAL_AS float *p = gmem(wrow);
    for (int q = 0; q < n; ++q) p[q] = __builtin_fmaf(nlr, o[q], p[q]);
    if (write_u) {
      GLOBAL_AS float *u = gmem(L->u + (int64_t)(t.row0 + gi) * L->ld_u + t.col0 + gj);
      for (int q = 0; q < n; ++q) u[q] = o[q];
    }
  }
}

// Work item (tile, bi, bj): tall tiles, oriented block rows [64 bi, +64), columns
// [64 bj, +64) of X0 (r x ldx); other tiles, rows [16 bi, +16), columns [256 bj, +256).
// Zeros outside the r x s tile.
template <typename S, int PREC>
__global__ __launch_bounds__(THREADS) void gemm_stage_kernel(const LayerDesc *__restrict__ layers,
                                                             const GemmTile *__restrict__ tiles,
                                                             const GemmWork *__restrict__ work, char *ws) {
  __shared__ float blk[SB * SBP];
  const GemmWork wk = work[blockIdx.x];
  const TileG t = tile_of(tiles, wk.tile);
  const LayerDesc *L = layers + t.layer;
  const float inv = gmem(reinterpret_cast<const float *>(ws + t.red))[t.nred];
  const S *mb = reinterpret_cast<const S *>(L->m);
  const int64_t ldm = L->ld_m;
  const Planes<PREC> X{ws + t.x0, t.r, t.ldx};
  if (!t.tall) {   // uniform over the workgroup: no transpose, straight from registers
    // two pieces of 8 columns, 128 apart: each load and store instruction of a wave then
    // covers contiguous 256-byte runs of a row
    const int gi = wk.bi * STRIP_R + (int)(threadIdx.x >> 4);
    const int gj = wk.bj * STRIP_C + (int)(threadIdx.x & 15) * 8;
    if (gi >= t.r) return;
    float v[2][8];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      if (gj + 128 * p < t.ldx) load_state8<S>(L, mb, ldm, t, gi, gj + 128 * p, v[p]);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (gj + 128 * p >= t.ldx) break;
#pragma unroll
      for (int q = 0; q < 8; ++q) v[p][q] *= inv;
      X.put8(gi, gj + 128 * p, v[p]);   // ldx is a multiple of 64 and gj of 8
    }
    return;
  }
  const int lr = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 16;
  // the global block this oriented block comes from
  {
    const int gi = wk.bj * SB + lr;
    const int gj = wk.bi * SB + lc;
    float v[16];
    load_state16<S>(L, mb, ldm, t, gi, gj, v);
#pragma unroll
    for (int q = 0; q < 16; ++q) blk[lr * SBP + lc + q] = v[q] * inv;
  }
  __syncthreads();
  const int orow = wk.bi * SB + lr, ocol = wk.bj * SB + lc;
  if (orow < t.r && ocol < t.ldx) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = blk[(lc + q) * SBP + lr];
    X.put16(orow, ocol, v);
  }
}

// Work item (tile, bi, bj): tall tiles, global block rows [64 bi, +64), columns
// [64 bj, +64) of the h x w tile; other tiles, rows [16 bi, +16), columns [256 bj, +256).
// O comes from the X buffer the last step wrote.
template <int PREC>
__global__ __launch_bounds__(THREADS) void gemm_apply_kernel(const LayerDesc *__restrict__ layers,
                                                             const GemmTile *__restrict__ tiles,
                                                             const GemmWork *__restrict__ work, char *ws,
                                                             int xsel, float lr_, int write_u) {
  __shared__ float blk[SB * SBP];
  const GemmWork wk = work[blockIdx.x];
  const TileG t = tile_of(tiles, wk.tile);
  const LayerDesc *L = layers + t.layer;
  const Planes<PREC> X{ws + (xsel ? t.x1 : t.x0), t.r, t.ldx};
  if (!t.tall) {   // uniform over the workgroup: O row gi is X row gi
    // two pieces of 8 columns, 128 apart (contiguous 512-byte runs of W per instruction)
    const int gi = wk.bi * STRIP_R + (int)(threadIdx.x >> 4);
    const int gj = wk.bj * STRIP_C + (int)(threadIdx.x & 15) * 8;
    if (gi >= t.h) return;
    float o[2][8];
    f32x4 w[2][2];
    bool vec[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int j = gj + 128 * p;
      vec[p] = j < t.w && t.w - j >= 8 && L->vec_w && ((t.col0 + j) & 3) == 0;
      if (j < t.w) X.get8(gi, j, o[p]);   // j + 8 <= ldx: ldx is a multiple of 64 and j of 8
      if (vec[p]) {
        const GLOBAL_AS f32x4 *pw = reinterpret_cast<const GLOBAL_AS f32x4 *>(
            gmem(L->w + (int64_t)(t.row0 + gi) * L->ld_w + t.col0 + j));
        w[p][0] = pw[0];
        w[p][1] = pw[1];
      }
    }
    const float nlr = -lr_;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int j = gj + 128 * p;
      if (j >= t.w) break;
      float *wrow = L->w + (int64_t)(t.row0 + gi) * L->ld_w + t.col0 + j;
      float *urow = write_u ? L->u + (int64_t)(t.row0 + gi) * L->ld_u + t.col0 + j : nullptr;
      if (vec[p]) {
        GLOBAL_AS f32x4 *pw = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(wrow));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[p][h][e] = __builtin_fmaf(nlr, o[p][4 * h + e], w[p][h][e]);
          pw[h] = w[p][h];
        }
        if (write_u) {
          GLOBAL_AS f32x4 *pu = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(urow));
          pu[0] = f32x4{o[p][0], o[p][1], o[p][2], o[p][3]};
          pu[1] = f32x4{o[p][4], o[p][5], o[p][6], o[p][7]};
        }
      } else {
        const int nn = t.w - j < 8 ? t.w - j : 8;
        GLOBAL_AS float *pw = gmem(wrow);
        for (int q = 0; q < nn; ++q) pw[q] = __builtin_fmaf(nlr, o[p][q], pw[q]);
        if (write_u) {
          GLOBAL_AS float *pu = gmem(urow);
          for (int q = 0; q < nn; ++q) pu[q] = o[p][q];
        }
      }
    }
    return;
  }
  const int lr = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 16;
  const int or0 = wk.bj * SB;   // oriented block holding this block
  const int oc0 = wk.bi * SB;
  {
    const int oi = or0 + lr, oj = oc0 + lc;
    float v[16];
    if (oi < t.r && oj < t.s) {
      X.get16(oi, oj, v);   // oj + 16 <= ldx: ldx is a multiple of 64 and oj of 16
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) blk[lr * SBP + lc + q] = oj + q < t.s ? v[q] : 0.f;
  }
  __syncthreads();
  const int gi = wk.bi * SB + lr, gj = wk.bj * SB + lc;
  if (gi >= t.h || gj >= t.w) return;
  float o[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) o[q] = blk[(lc + q) * SBP + lr];
  apply16(L, t, gi, gj, o, lr_, write_u);
}

// ------------------------------------------------------------------ grouped GEMMs
// Workgroups are dispatched to the eight XCDs round robin (block b on XCD b % 8).  The
// work list holds the blocks of one tile next to each other, so each XCD takes one
// contiguous run of it: the blocks that read the same tile's operands then share that
// XCD's L2.
__device__ __forceinline__ int xcd_work_index() {
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  const int per = nb / 8, rem = nb % 8, x = b % 8;
  return x * per + (x < rem ? x : rem) + b / 8;
}

// LDS tile of one operand for one K step, per plane: [rows][BK + pad] (row operand) or
// [BK][BM + pad] (column operand of the update, read with ds_read_tr).
// BK: the K slice (32: two LDS stages; 64: one stage).
template <int PREC, int BK>
struct GemmLds {
  static constexpr bool F32 = PREC == PREC_F32;
  static constexpr int NPL = PREC == PREC_BF16X3 ? 2 : 1;     // planes staged
  static constexpr int RP = F32 ? BK + 4 : BK + 8;            // row-operand pitch (elements)
  static constexpr int CP = F32 ? BM + 4 : BM + 8;            // column-operand pitch
  static constexpr int ES = F32 ? 4 : 2;                      // element bytes
  static constexpr int ROWT = BM * RP * ES;                   // one plane of a row tile
  static constexpr int COLT = BK * CP * ES;                   // one plane of a column tile
  static constexpr int STAGE = NPL * (ROWT + (ROWT > COLT ? ROWT : COLT));
  static constexpr int SP = BM + 4;                           // fp32 staging pitch
  static constexpr int NSTAGE = BK == 32 ? 2 : 1;
  static constexpr int BYTES = NSTAGE * STAGE > BM * SP * 4 ? NSTAGE * STAGE : BM * SP * 4;
  static constexpr int CPR = BK * ES / 16;       // 16-byte chunks per row of a row tile
  static constexpr int CPC = BM * ES / 16;       //                per k row of a column tile
  static constexpr int NQ = BM * CPR / THREADS;  // chunks per thread, per plane and operand
  static_assert(BM * CPR % THREADS == 0 && BK * CPC == BM * CPR, "whole chunks per thread");
};

// Per-thread registers of one K step's global loads (both operands, all planes).
template <int PREC, int BK>
struct KRegs {
  static constexpr int N = GemmLds<PREC, BK>::NPL * GemmLds<PREC, BK>::NQ;
  u32x4 l[N], r[N];
};

template <int PREC, int MODE, int BK>
__device__ __forceinline__ void gemm_load(KRegs<PREC, BK> &kr, const Planes<PREC> &Lp, int i0,
                                          const Planes<PREC> &Rp, int j0, int kb) {
  using LD = GemmLds<PREC, BK>;
  const int tid = threadIdx.x;
  constexpr int EPC = 16 / LD::ES;   // elements per 16-byte chunk
#pragma unroll
  for (int pl = 0; pl < LD::NPL; ++pl) {
    const char *lb = PREC == PREC_F32 ? reinterpret_cast<const char *>(Lp.f())
                                      : reinterpret_cast<const char *>(pl ? Lp.lo() : Lp.hi());
    const char *rb = PREC == PREC_F32 ? reinterpret_cast<const char *>(Rp.f())
                                      : reinterpret_cast<const char *>(pl ? Rp.lo() : Rp.hi());
#pragma unroll
    for (int q = 0; q < LD::NQ; ++q) {
      const int idx = tid + q * THREADS;
      const int row = idx / LD::CPR, ch = idx % LD::CPR;   // BM rows x CPR chunks
      const int gi = i0 + row;
      kr.l[pl * LD::NQ + q] =
          gi < Lp.rows ? *(reinterpret_cast<const GLOBAL_AS u32x4 *>(
                             gmem(lb + ((int64_t)gi * Lp.ld + kb + ch * EPC) * LD::ES)))
                       : u32x4{0, 0, 0, 0};
      if constexpr (MODE == MODE_UPDATE) {
        const int kr_ = idx / LD::CPC, cc = idx % LD::CPC;   // BK k rows x CPC chunks
        const int gk = kb + kr_, gj = j0 + cc * EPC;
        kr.r[pl * LD::NQ + q] =
            (gk < Rp.rows && gj < Rp.ld) ? *(reinterpret_cast<const GLOBAL_AS u32x4 *>(
                                               gmem(rb + ((int64_t)gk * Rp.ld + gj) * LD::ES)))
                                         : u32x4{0, 0, 0, 0};
      } else {
        const int gj = j0 + row;
        kr.r[pl * LD::NQ + q] =
            gj < Rp.rows ? *(reinterpret_cast<const GLOBAL_AS u32x4 *>(
                               gmem(rb + ((int64_t)gj * Rp.ld + kb + ch * EPC) * LD::ES)))
                         : u32x4{0, 0, 0, 0};
      }
    }
  }
}

template <int PREC, int MODE, int BK>
__device__ __forceinline__ void gemm_store_lds(const KRegs<PREC, BK> &kr, char *stage) {
  using LD = GemmLds<PREC, BK>;
  const int tid = threadIdx.x;
  constexpr int EPC = 16 / LD::ES;
  char *lt = stage;                         // row tiles of L: NPL planes
  char *rt = stage + LD::NPL * LD::ROWT;    // then the R tiles
#pragma unroll
  for (int pl = 0; pl < LD::NPL; ++pl) {
#pragma unroll
    for (int q = 0; q < LD::NQ; ++q) {
      const int idx = tid + q * THREADS;
      const int row = idx / LD::CPR, ch = idx % LD::CPR;
      *reinterpret_cast<u32x4 *>(lt + pl * LD::ROWT + (row * LD::RP + ch * EPC) * LD::ES) = kr.l[pl * LD::NQ + q];
      if constexpr (MODE == MODE_UPDATE) {
        const int kr_ = idx / LD::CPC, cc = idx % LD::CPC;
        *reinterpret_cast<u32x4 *>(rt + pl * LD::COLT + (kr_ * LD::CP + cc * EPC) * LD::ES) = kr.r[pl * LD::NQ + q];
      } else {
        *reinterpret_cast<u32x4 *>(rt + pl * LD::ROWT + (row * LD::RP + ch * EPC) * LD::ES) = kr.r[pl * LD::NQ + q];
      }
    }
  }
}

// MFMAs of one K step from an LDS stage; wave block rows wm*64.., columns wn*64...
template <int PREC, int MODE, int BK>
__device__ __forceinline__ void gemm_compute(f32x16 (&acc)[2][2], const char *stage, int wm, int wn, int lane) {
  using LD = GemmLds<PREC, BK>;
  const int li = lane & 31, half = lane >> 5;
  const char *lt = stage;
  const char *rt = stage + LD::NPL * LD::ROWT;
  if constexpr (PREC == PREC_F32) {
    const float *L = reinterpret_cast<const float *>(lt);
    const float *R = reinterpret_cast<const float *>(rt);
#pragma unroll
    for (int kc = 0; kc < BK; kc += 8) {
      const int k = kc + 4 * half;
      f32x4 lf[2], rf[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        lf[b] = *reinterpret_cast<const f32x4 *>(L + (wm * 64 + b * 32 + li) * LD::RP + k);
        if constexpr (MODE == MODE_UPDATE) {
#pragma unroll
          for (int e = 0; e < 4; ++e) rf[b][e] = R[(k + e) * LD::CP + wn * 64 + b * 32 + li];
        } else {
          rf[b] = *reinterpret_cast<const f32x4 *>(R + (wn * 64 + b * 32 + li) * LD::RP + k);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mma_f32(lf[bi][e], rf[bj][e], acc[bi][bj]);
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < BK; kc += 16) {
      const int k = kc + 8 * half;
      bf16x8 lh[2], ll[2], rh[2], rl[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const __bf16 *L0 = reinterpret_cast<const __bf16 *>(lt);
        lh[b] = *reinterpret_cast<const bf16x8 *>(L0 + (wm * 64 + b * 32 + li) * LD::RP + k);
        if constexpr (MODE == MODE_UPDATE) {
          rh[b] = tr_frag(reinterpret_cast<const __bf16 *>(rt), LD::CP, k, wn * 64 + b * 32, lane);
        } else {
          rh[b] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const __bf16 *>(rt) +
                                                    (wn * 64 + b * 32 + li) * LD::RP + k);
        }
        if constexpr (PREC == PREC_BF16X3) {
          const __bf16 *L1 = reinterpret_cast<const __bf16 *>(lt + LD::ROWT);
          ll[b] = *reinterpret_cast<const bf16x8 *>(L1 + (wm * 64 + b * 32 + li) * LD::RP + k);
          if constexpr (MODE == MODE_UPDATE) {
            rl[b] = tr_frag(reinterpret_cast<const __bf16 *>(rt + LD::COLT), LD::CP, k, wn * 64 + b * 32, lane);
          } else {
            rl[b] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const __bf16 *>(rt + LD::ROWT) +
                                                      (wn * 64 + b * 32 + li) * LD::RP + k);
          }
        }
      }
      if constexpr (PREC == PREC_BF16X3) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mma_bf16(ll[bi], rh[bj], acc[bi][bj]);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mma_bf16(lh[bi], rl[bj], acc[bi][bj]);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mma_bf16(lh[bi], rh[bj], acc[bi][bj]);
    }
  }
}

// One 128 x 128 output block of a NS product for one work item.
//   GRAM    D = X X^T over the tile's X (upper blocks); writes A, or B = b A (+ a I) if c = 0
//   SQUARE  D = A A^T; writes B = b A + c D (+ a I)
//   UPDATE  D = B X;   writes X_next = D (+ a X for plain bf16)
template <int PREC, int MODE, int BK>
__global__ __launch_bounds__(THREADS) void gemm_ns_kernel(const GemmTile *__restrict__ tiles,
                                                          const GemmWork *__restrict__ work, char *ws,
                                                          GemmParams gp) {
  using LD = GemmLds<PREC, BK>;
  __shared__ __attribute__((aligned(16))) char lds[LD::BYTES];
  const GemmWork wk = work[xcd_work_index()];
  const TileG t = tile_of(tiles, wk.tile);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i0 = wk.bi * BM, j0 = wk.bj * BM;

  const Planes<PREC> Xc{ws + (gp.xsel ? t.x1 : t.x0), t.r, t.ldx};
  const Planes<PREC> Xn{ws + (gp.xsel ? t.x0 : t.x1), t.r, t.ldx};
  const Planes<PREC> A{ws + t.a, t.r, t.lda};
  const Planes<PREC> B{ws + t.b, t.r, t.lda};
  const Planes<PREC> Lp = MODE == MODE_GRAM ? Xc : (MODE == MODE_SQUARE ? A : B);
  const Planes<PREC> Rp = MODE == MODE_GRAM ? Xc : (MODE == MODE_SQUARE ? A : Xc);
  const int kdim = MODE == MODE_GRAM ? t.ldx : t.lda;

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = f32x16{};

  // The next K slice's global loads are in flight in registers while the MFMAs read the
  // current one from LDS.  Slices of 32 alternate between two LDS stages (one barrier
  // per slice); slices of 64 (whole 128-byte lines of bf16 rows, for long K) use one
  // stage, and two workgroups share a CU, so one's LDS stores overlap the other's
  // products.
  KRegs<PREC, BK> kr;
  gemm_load<PREC, MODE, BK>(kr, Lp, i0, Rp, j0, 0);
  gemm_store_lds<PREC, MODE, BK>(kr, lds);
  __syncthreads();
  int cur = 0;
  for (int kb = 0; kb < kdim; kb += BK) {
    const bool more = kb + BK < kdim;
    if (more) gemm_load<PREC, MODE, BK>(kr, Lp, i0, Rp, j0, kb + BK);
    gemm_compute<PREC, MODE, BK>(acc, lds + cur * LD::STAGE, wm, wn, lane);
    if constexpr (LD::NSTAGE == 2) {
      if (more) gemm_store_lds<PREC, MODE, BK>(kr, lds + (cur ^ 1) * LD::STAGE);
      __syncthreads();
      cur ^= 1;
    } else {
      __syncthreads();   // the stage fully read
      if (more) {
        gemm_store_lds<PREC, MODE, BK>(kr, lds);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: stage D^T in LDS (fp32), then write rows with 16-element stores
  float *st = reinterpret_cast<float *>(lds);
  {
    const int li = lane & 31, half = lane >> 5;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int il = wm * 64 + bi * 32 + 8 * g + 4 * half;
          const int jl = wn * 64 + bj * 32 + li;
          *reinterpret_cast<f32x4 *>(st + jl * LD::SP + il) =
              f32x4{acc[bi][bj][4 * g], acc[bi][bj][4 * g + 1], acc[bi][bj][4 * g + 2], acc[bi][bj][4 * g + 3]};
        }
  }
  __syncthreads();
  const float a = gp.a, b = gp.b, c = gp.c;
  const bool fold = gp.fold != 0;
  // value of the product element (i, j) as stored; e is element (i, j) of the matrix the
  // epilogue adds (A for the square, X for an update without a folded into B)
  auto finish = [&](float d, float e, int i, int j) -> float {
    if constexpr (MODE == MODE_GRAM) {
      if (c != 0.f) return d;
      return b * d + ((fold && i == j) ? a : 0.f);
    } else if constexpr (MODE == MODE_SQUARE) {
      return __builtin_fmaf(c, d, b * e) + ((fold && i == j) ? a : 0.f);
    } else {
      return fold ? d : __builtin_fmaf(a, e, d);
    }
  };
  // the 16 elements of that matrix at row i from column j (coalesced loads)
  auto addend16 = [&](int i, int j, float (&e)[16]) {
    if constexpr (MODE == MODE_SQUARE) {
      A.get16(i, j, e);
    } else if constexpr (MODE == MODE_UPDATE) {
      if (!fold) {
        Xc.get16(i, j, e);
        return;
      }
    }
    if constexpr (MODE != MODE_SQUARE) {
#pragma unroll
      for (int q = 0; q < 16; ++q) e[q] = 0.f;
    }
  };
  const Planes<PREC> O = MODE == MODE_GRAM ? (c != 0.f ? A : B) : (MODE == MODE_SQUARE ? B : Xn);
  const int valid = MODE == MODE_UPDATE ? t.s : t.r;   // valid columns; the rest up to ld is 0
  const int ldo = O.ld;
  // (1) D rows: row i = i0 + il, columns j0 + jl .. +15 (staging columns)
  for (int u = threadIdx.x; u < BM * (BM / 16); u += THREADS) {
    const int il = u >> 3, jl = (u & 7) * 16;
    const int i = i0 + il, j = j0 + jl;
    if (i >= t.r || j >= ldo) continue;
    float v[16], e[16];
    addend16(i, j, e);
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = j + q < valid ? finish(st[(jl + q) * LD::SP + il], e[q], i, j + q) : 0.f;
    O.put16(i, j, v);
  }
  // (2) symmetric products: the mirrored block D^T at rows j0 + jl, columns i0 + il
  if constexpr (MODE != MODE_UPDATE) {
    if (wk.bi != wk.bj) {
      for (int u = threadIdx.x; u < BM * (BM / 16); u += THREADS) {
        const int jl = u >> 3, il = (u & 7) * 16;
        const int j = j0 + jl, i = i0 + il;
        if (j >= t.r || i >= ldo) continue;
        // element (i + q, j) of the symmetric A equals (j, i + q): a contiguous row
        float v[16], e[16];
        addend16(j, i, e);
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = i + q < valid ? finish(st[jl * LD::SP + il + q], e[q], i + q, j) : 0.f;
        O.put16(j, i, v);
      }
    }
  }
}

// ------------------------------------------------------------------ 256-tiles
// Chunks whose tiles are all 256 x 256 (T = 256 on sides that are multiples of 256) run
// each product of a tile in one workgroup: eight waves of 64 x 128 cover the whole
// 256 x 256 output, so the tile's operands are streamed once per product instead of
// once per 128-block (three or four times).  The symmetric products compute every block
// (no mirror); K = 256 through two LDS stages, in slices of 64 (whole 128-byte lines,
// twice the bytes in flight) for the symmetric products and of 32 for the update, whose
// two operand panels leave no registers for more.  bf16 and bf16x3 planes.  With c != 0
// the Gram writes only columns 128.. of A to the workspace and hands rows 0..127 (by
// symmetry the square's first two K slices) to the square through LDS.
constexpr int T2 = 256, T2_THREADS = 512;


template <int PREC, int MODE>
struct T2Lds {
  static constexpr int BK = MODE == MODE_UPDATE ? 32 : 64;  // K slice
  static constexpr int NPL = PREC == PREC_BF16X3 ? 2 : 1;   // planes staged
  static constexpr int RP = BK + 8;                         // row panel pitch (elements)
  static constexpr int CP = T2 + 8;                         // column panel pitch (update)
  static constexpr int ROWT = T2 * RP * 2;                  // one plane of the row panel
  static constexpr int COLT = BK * CP * 2;                  // one plane of the column panel
  static constexpr int STAGE = NPL * (ROWT + (MODE == MODE_UPDATE ? COLT : 0));
  // fp32 staging of one column half of D, row-major, pitch 4 mod 32 words: eight
  // consecutive rows written at one column (16-byte pieces) and two rows of 8-column
  // pieces read by eight lanes each fall on distinct banks
  static constexpr int SP = T2 / 2 + 4;
  static constexpr int STG = T2 * SP * 4;
  static constexpr int BYTES = 2 * STAGE > STG ? 2 * STAGE : STG;
  static constexpr int NQ = T2 * (BK / 8) / T2_THREADS;     // 16-byte chunks per thread, plane, operand
  static_assert(T2 * (BK / 8) % T2_THREADS == 0 && BK * (T2 / 8) == T2 * (BK / 8), "whole chunks");
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// One product of a 256 x 256 tile by the whole workgroup, in place: X is read from and
// written back to the x0 planes, and B to the planes of A.  That is safe because the K
// loop has read every operand before the epilogue writes, and each output element is
// written by the thread that reads its addend (X for the update without a folded a)
// just before.  The accumulators belong to the caller: with c != 0 the Gram product
// leaves (b / c) A in them (fp32, as accumulated) after storing A, and the square
// product accumulates A A^T onto that, so B = c ((b / c) A + A^2) needs no second read
// of A; the Gram and update products start from zero.
// The step's ends for a 256-tile, fused into the tile's workgroup: the momentum, the
// norm and X0 before the first product, and the W update in the epilogue of the last
// update product (the step's O is X_K in fp32 as that epilogue forms it; 256-tiles are
// square, so never transposed): W <- W - lr O by one fused multiply-add, and O itself to
// U when asked.
struct T256Apply {
  const LayerDesc *layers;
  float lr;
  int write_u;
  float beta, eps;
};

// Fixed-order sum and maximum over the 8 waves of a 256-tile workgroup; every thread
// gets the result.
__device__ __forceinline__ float t256_sum(float v, float *red8) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = ((red8[0] + red8[1]) + (red8[2] + red8[3])) + ((red8[4] + red8[5]) + (red8[6] + red8[7]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float t256_max(float v, float *red8) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red8[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) r = __builtin_fmaxf(r, red8[k]);
  __syncthreads();
  return r;
}

// M <- beta M + G for the 256-tile (stored in the state dtype), 1 / (|M|_F + eps) of the
// stored values, and X0 = M inv into the x0 planes.  Thread t takes 8 columns of rows
// t / 32 + 16 k, k < 16, in every pass, so each thread re-reads only what it stored.  The
// norm is rescaled by a power of two where its sum of squares leaves [2^-100, 2^100], as
// in the norm kernel.
template <typename S, int PREC>
__device__ __forceinline__ void t256_front(const TileG &t, char *ws, const T256Apply &io, float *red8) {
  const LayerDesc *L = io.layers + t.layer;
  S *mb = reinterpret_cast<S *>(L->m);
  const S *gb = reinterpret_cast<const S *>(L->g);
  const int64_t ldm = L->ld_m, ldg = L->ld_g;
  const int cc = (threadIdx.x & 31) * 8, rr = threadIdx.x >> 5;
  const bool vec = L->vec_ok;   // rows 16-byte aligned (the tile's columns start at a multiple of 256)
  const float beta = io.beta;
  constexpr int NK = T2 / 16;   // row pieces per thread
  if constexpr (sizeof(S) == 2) {
    if (vec) {   // (uniform)
      // bf16 state in aligned rows: every load is issued before the first store (M is
      // updated in place, so a store to M would otherwise hold back the next piece's
      // loads), and the stored codes stay in registers for the norm and X0.  Same
      // arithmetic, in the same order, as the general path below.
      auto f32_of = [](const u32x4 &w, int q) {
        return __builtin_bit_cast(float, (q & 1) ? (w[q >> 1] & 0xffff0000u) : (w[q >> 1] << 16));
      };
      u32x4 mc[NK], gc[NK];
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int64_t i = t.row0 + rr + 16 * k;
        mc[k] = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(mb + i * ldm + t.col0 + cc));
        gc[k] = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(gb + i * ldg + t.col0 + cc));
      }
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        unsigned short code[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) code[q] = to_bf16_bits(__builtin_fmaf(beta, f32_of(mc[k], q), f32_of(gc[k], q)));
        mc[k] = u32x4{code[0] | (unsigned)code[1] << 16, code[2] | (unsigned)code[3] << 16,
                      code[4] | (unsigned)code[5] << 16, code[6] | (unsigned)code[7] << 16};
        *reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(mb + (int64_t)(t.row0 + rr + 16 * k) * ldm + t.col0 + cc)) = mc[k];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float v = f32_of(mc[k], q);
          ss = __builtin_fmaf(v, v, ss);
        }
      }
      ss = t256_sum(ss, red8);
      float s1 = 1.f, s2 = 1.f;
      if (!(ss >= 0x1p-100f && ss <= 0x1p100f)) {   // uniform over the workgroup
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < NK; ++k)
#pragma unroll
          for (int q = 0; q < 8; ++q) mx = __builtin_fmaxf(mx, __builtin_fabsf(f32_of(mc[k], q)));
        mx = t256_max(mx, red8);
        if (mx > 0.f && mx <= 0x1.fffffep127f) {   // nonzero and finite
          int ex;
          (void)__builtin_frexpf(mx, &ex);
          s1 = __builtin_ldexpf(1.f, (-ex) / 2);
          s2 = __builtin_ldexpf(1.f, -ex - (-ex) / 2);
          float s2s = 0.f;
#pragma unroll
          for (int k = 0; k < NK; ++k)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float x = f32_of(mc[k], q) * s1 * s2;
              s2s = __builtin_fmaf(x, x, s2s);
            }
          ss = t256_sum(s2s, red8);
        }
      }
      const float den = __builtin_sqrtf(ss) + (io.eps * s1) * s2;
      const float inv = den > 0.f ? (s1 / den) * s2 : (den == 0.f ? 0.f : den);
      const Planes<PREC> X{ws + t.x0, t.r, t.ldx};
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = f32_of(mc[k], q) * inv;
        X.put8(rr + 16 * k, cc, v);
      }
      __syncthreads();   // X0 complete before the first product reads it
      return;
    }
  }
  float ss = 0.f;
  for (int k = 0; k < T2 / 16; ++k) {
    const int i = rr + 16 * k;
    S *mp = mb + (int64_t)(t.row0 + i) * ldm + t.col0 + cc;
    const S *gp = gb + (int64_t)(t.row0 + i) * ldg + t.col0 + cc;
    float v[8];
    if constexpr (sizeof(S) == 2) {
      unsigned short code[8];
      if (vec) {
        const u32x4 m = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(mp));
        const u32x4 g = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(gp));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const unsigned mw = m[q >> 1], gw = g[q >> 1];
          code[q] = to_bf16_bits(__builtin_fmaf(beta, __builtin_bit_cast(float, (q & 1) ? (mw & 0xffff0000u) : (mw << 16)),
                                                __builtin_bit_cast(float, (q & 1) ? (gw & 0xffff0000u) : (gw << 16))));
        }
        *reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(mp)) =
            u32x4{code[0] | (unsigned)code[1] << 16, code[2] | (unsigned)code[3] << 16,
                  code[4] | (unsigned)code[5] << 16, code[6] | (unsigned)code[7] << 16};
      } else {
        GLOBAL_AS unsigned short *m16 = gmem(reinterpret_cast<unsigned short *>(mp));
        const GLOBAL_AS unsigned short *g16 = gmem(reinterpret_cast<const unsigned short *>(gp));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          code[q] = to_bf16_bits(__builtin_fmaf(beta, bf16_bits_to_f32(m16[q]), bf16_bits_to_f32(g16[q])));
          m16[q] = code[q];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = bf16_bits_to_f32(code[q]);
    } else {
      GLOBAL_AS float *m32 = gmem(mp);
      const GLOBAL_AS float *g32 = gmem(gp);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[q] = __builtin_fmaf(beta, m32[q], g32[q]);
        m32[q] = v[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) ss = __builtin_fmaf(v[q], v[q], ss);
  }
  ss = t256_sum(ss, red8);
  float s1 = 1.f, s2 = 1.f;
  if (!(ss >= 0x1p-100f && ss <= 0x1p100f)) {   // uniform over the workgroup
    float mx = 0.f;
    for (int k = 0; k < T2 / 16; ++k) {
      float v[8];
      load_state8<S>(L, mb, ldm, t, rr + 16 * k, cc, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[q]));
    }
    mx = t256_max(mx, red8);
    if (mx > 0.f && mx <= 0x1.fffffep127f) {   // nonzero and finite
      int ex;
      (void)__builtin_frexpf(mx, &ex);
      s1 = __builtin_ldexpf(1.f, (-ex) / 2);
      s2 = __builtin_ldexpf(1.f, -ex - (-ex) / 2);
      float s2s = 0.f;
      for (int k = 0; k < T2 / 16; ++k) {
        float v[8];
        load_state8<S>(L, mb, ldm, t, rr + 16 * k, cc, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float x = v[q] * s1 * s2;
          s2s = __builtin_fmaf(x, x, s2s);
        }
      }
      ss = t256_sum(s2s, red8);
    }
  }
  // a zero tile stays zero, also with eps = 0 (divisor 0); a NaN passes on
  const float den = __builtin_sqrtf(ss) + (io.eps * s1) * s2;
  const float inv = den > 0.f ? (s1 / den) * s2 : (den == 0.f ? 0.f : den);
  const Planes<PREC> X{ws + t.x0, t.r, t.ldx};
  for (int k = 0; k < T2 / 16; ++k) {
    float v[8];
    load_state8<S>(L, mb, ldm, t, rr + 16 * k, cc, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] *= inv;
    X.put8(rr + 16 * k, cc, v);
  }
  __syncthreads();   // X0 complete before the first product reads it
}

// Hand the rows k < 64 NW of a symmetric product's result (held in the accumulators
// of the waves with wm < NW) to the next product as the first K slices of its row
// panel: element (i, k) of that panel is R(k, i), so each lane's four consecutive rows
// k of one column i are one 8-byte piece of panel row i, in the consumer's stage layout
// LS (slice k / BK in stage k / BK) and split into hi and lo as the workspace planes
// would hold them.  val(d, k, i) forms the result from the accumulated d, as the
// producer's epilogue does.  (The accumulated R(k, i) and R(i, k) can differ in the
// last fp32 bits: the bf16x3 correction terms reach them in opposite orders.)
template <class LS, int NW, class F>
__device__ __forceinline__ void t256_hand_over(const f32x16 (&acc)[2][4], char *lds, int wm, int wn, int li, int half,
                                               F &&val) {
  static_assert(64 * NW <= 2 * LS::BK, "the handed-over slices fit the two stages");
  if (wm < NW) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int k0 = wm * 64 + bi * 32;   // a multiple of 32: one slice per bi
      char *stage = lds + (k0 / LS::BK) * LS::STAGE;
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int k = k0 + 8 * g + 4 * half;
          const int i = wn * 128 + bj * 32 + li;
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = val(acc[bi][bj][4 * g + e], k + e, i);
          const u32x2 hi = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          const int o = (i * LS::RP + k % LS::BK) * 2;
          *reinterpret_cast<u32x2 *>(stage + o) = hi;
          if constexpr (LS::NPL == 2)
            *reinterpret_cast<u32x2 *>(stage + LS::ROWT + o) =
                u32x2{pack_bf16x2(x[0] - __builtin_bit_cast(float, hi[0] << 16),
                                  x[1] - __builtin_bit_cast(float, hi[0] & 0xffff0000u)),
                      pack_bf16x2(x[2] - __builtin_bit_cast(float, hi[1] << 16),
                                  x[3] - __builtin_bit_cast(float, hi[1] & 0xffff0000u))};
        }
    }
  }
  __syncthreads();   // the stages are complete before the next product reads them
}

// plain (bf16x3 planes, the symmetric products of early steps; uniform): the product of
// the hi operands alone, one bf16 product instead of three, with only the hi planes
// loaded.
template <int PREC, int MODE, bool APPLY = false>
__device__ __forceinline__ void t256_product(const TileG &t, char *ws, const GemmParams &gp, char *lds,
                                             f32x16 (&acc)[2][4], const T256Apply &ap = T256Apply{},
                                             bool plain = false) {
  static_assert(PREC == PREC_BF16 || PREC == PREC_BF16X3, "bf16 planes");
  using LD = T2Lds<PREC, MODE>;
  constexpr bool SPLIT = PREC == PREC_BF16X3;
  const bool lo_in = SPLIT && !(MODE != MODE_UPDATE && plain);   // (uniform) lo planes loaded and multiplied
  // (the thread index is made opaque so that the addresses derived from it are formed
  // inside each product rather than hoisted out of the NS loop for all three at once)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // rows 64 wm.., columns 128 wn..
  const int li = lane & 31, half = lane >> 5;

  const Planes<PREC> Xc{ws + t.x0, T2, T2};
  const Planes<PREC> Xn = Xc;
  const Planes<PREC> A{ws + t.a, T2, T2};
  const Planes<PREC> B = A;
  // row operand: X (Gram), A (square), B (update); the symmetric products' column
  // operand is the same panel, the update's is X read along its columns
  const Planes<PREC> Lp = MODE == MODE_GRAM ? Xc : (MODE == MODE_SQUARE ? A : B);

  u32x4 rl_[LD::NPL * LD::NQ], rr_[LD::NPL * LD::NQ];
  auto load = [&](int kb) {
#pragma unroll
    for (int pl = 0; pl < LD::NPL; ++pl) {
      if (pl == 1 && !lo_in) break;
      const __bf16 *lb = pl ? Lp.lo() : Lp.hi();
      const __bf16 *xb = pl ? Xc.lo() : Xc.hi();
#pragma unroll
      for (int q = 0; q < LD::NQ; ++q) {
        const int idx = tid + q * T2_THREADS;
        const int row = idx / (LD::BK / 8), ch = idx % (LD::BK / 8);
        rl_[pl * LD::NQ + q] = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(lb + (int64_t)row * T2 + kb + ch * 8));
        if constexpr (MODE == MODE_UPDATE) {
          const int kr = idx / (T2 / 8), cc = idx % (T2 / 8);
          rr_[pl * LD::NQ + q] = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(xb + (int64_t)(kb + kr) * T2 + cc * 8));
        }
      }
    }
  };
  auto store = [&](char *stage) {
#pragma unroll
    for (int pl = 0; pl < LD::NPL; ++pl) {
      if (pl == 1 && !lo_in) break;
#pragma unroll
      for (int q = 0; q < LD::NQ; ++q) {
        const int idx = tid + q * T2_THREADS;
        const int row = idx / (LD::BK / 8), ch = idx % (LD::BK / 8);
        *reinterpret_cast<u32x4 *>(stage + pl * LD::ROWT + (row * LD::RP + ch * 8) * 2) = rl_[pl * LD::NQ + q];
        if constexpr (MODE == MODE_UPDATE) {
          const int kr = idx / (T2 / 8), cc = idx % (T2 / 8);
          *reinterpret_cast<u32x4 *>(stage + LD::NPL * LD::ROWT + pl * LD::COLT + (kr * LD::CP + cc * 8) * 2) =
              rr_[pl * LD::NQ + q];
        }
      }
    }
  };

  if constexpr (MODE != MODE_SQUARE) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x16{};
  }
  auto compute = [&](const char *stage) {
    const __bf16 *L0 = reinterpret_cast<const __bf16 *>(stage);
    const __bf16 *L1 = reinterpret_cast<const __bf16 *>(stage + LD::ROWT);
    const __bf16 *C0 = reinterpret_cast<const __bf16 *>(stage + LD::NPL * LD::ROWT);
    const __bf16 *C1 = reinterpret_cast<const __bf16 *>(stage + LD::NPL * LD::ROWT + LD::COLT);
#pragma unroll
    for (int kc = 0; kc < LD::BK; kc += 16) {
      const int k = kc + 8 * half;
      bf16x8 lh[2], ll[2], rh[4], rl[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        lh[b] = *reinterpret_cast<const bf16x8 *>(L0 + (wm * 64 + b * 32 + li) * LD::RP + k);
        if (SPLIT && lo_in)
          ll[b] = *reinterpret_cast<const bf16x8 *>(L1 + (wm * 64 + b * 32 + li) * LD::RP + k);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if constexpr (MODE == MODE_UPDATE) {
          rh[b] = tr_frag(C0, LD::CP, k, wn * 128 + b * 32, lane);
          if constexpr (SPLIT) rl[b] = tr_frag(C1, LD::CP, k, wn * 128 + b * 32, lane);
        } else {
          rh[b] = *reinterpret_cast<const bf16x8 *>(L0 + (wn * 128 + b * 32 + li) * LD::RP + k);
          if (SPLIT && lo_in)
            rl[b] = *reinterpret_cast<const bf16x8 *>(L1 + (wn * 128 + b * 32 + li) * LD::RP + k);
        }
      }
      if (SPLIT && lo_in) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mma_bf16(ll[bi], rh[bj], acc[bi][bj]);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mma_bf16(lh[bi], rl[bj], acc[bi][bj]);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mma_bf16(lh[bi], rh[bj], acc[bi][bj]);
    }
  };

  if constexpr (MODE == MODE_SQUARE) {
    // Slices 0 and 1 (k < 128) are already in stages 0 and 1, written there from the
    // Gram's accumulators; slice n + 2 is loaded while slice n is multiplied and takes
    // its stage after it.
    constexpr int NSL = T2 / LD::BK;
    static_assert(NSL == 4, "two slices handed over, two loaded");
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
      const bool more = n + 2 < NSL;
      if (more) load((n + 2) * LD::BK);
      compute(lds + (n & 1) * LD::STAGE);
      __syncthreads();
      if (more) store(lds + (n & 1) * LD::STAGE);
    }
  } else if constexpr (MODE == MODE_UPDATE) {
    // The B row panels of slices 0 and 1 (k < 64) are already in stages 0 and 1, written
    // there by the product that formed B; their X column panels are loaded first (slice
    // 1's into the row registers, which these slices do not need).  Then slice n + 2 is
    // loaded while slice n is multiplied and takes its stage after it.
    constexpr int NSL = T2 / LD::BK;
#pragma unroll
    for (int pl = 0; pl < LD::NPL; ++pl) {
      const __bf16 *xb = pl ? Xc.lo() : Xc.hi();
#pragma unroll
      for (int q = 0; q < LD::NQ; ++q) {
        const int idx = tid + q * T2_THREADS;
        const int kr = idx / (T2 / 8), cc = idx % (T2 / 8);
        rr_[pl * LD::NQ + q] = *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(xb + (int64_t)kr * T2 + cc * 8));
        rl_[pl * LD::NQ + q] =
            *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(xb + (int64_t)(LD::BK + kr) * T2 + cc * 8));
      }
    }
#pragma unroll
    for (int pl = 0; pl < LD::NPL; ++pl) {
#pragma unroll
      for (int q = 0; q < LD::NQ; ++q) {
        const int idx = tid + q * T2_THREADS;
        const int kr = idx / (T2 / 8), cc = idx % (T2 / 8);
        const int o = LD::NPL * LD::ROWT + pl * LD::COLT + (kr * LD::CP + cc * 8) * 2;
        *reinterpret_cast<u32x4 *>(lds + o) = rr_[pl * LD::NQ + q];
        *reinterpret_cast<u32x4 *>(lds + LD::STAGE + o) = rl_[pl * LD::NQ + q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
      const bool more = n + 2 < NSL;
      if (more) load((n + 2) * LD::BK);
      compute(lds + (n & 1) * LD::STAGE);
      __syncthreads();
      if (more) store(lds + (n & 1) * LD::STAGE);
    }
  } else {
    // the next slice's loads are in flight while the MFMAs read the current stage
    load(0);
    store(lds);
    __syncthreads();
    int cur = 0;
    for (int kb = 0; kb < T2; kb += LD::BK) {
      const bool more = kb + LD::BK < T2;
      if (more) load(kb + LD::BK);
      compute(lds + cur * LD::STAGE);
      if (more) store(lds + (cur ^ 1) * LD::STAGE);
      __syncthreads();
      cur ^= 1;
    }
  }

  // ---- epilogue, one column half at a time: the half staged in LDS (fp32), then rows
  // written as 8-element pieces, eight lanes to 128 contiguous bytes of a row
  float *st = reinterpret_cast<float *>(lds);
  const float a = gp.a, b = gp.b, c = gp.c;
  const bool fold = gp.fold != 0;
  const Planes<PREC> O = MODE == MODE_GRAM ? (c != 0.f ? A : B) : (MODE == MODE_SQUARE ? B : Xn);
  // With c != 0 the Gram's A goes to the square product alone: its columns 128.. (the
  // square's last two K slices) through the workspace, its rows 0..127 (by symmetry the
  // first two slices) straight into the square's LDS stages below.  B (from the square,
  // or from the Gram when c = 0) goes to the update the same way: columns 64.. through
  // the workspace, rows 0..63 into the update's first two stages.
  const bool hand_a = MODE == MODE_GRAM && c != 0.f;
  const bool hand_b = MODE == MODE_SQUARE || (MODE == MODE_GRAM && c == 0.f);
  // The Gram and square results are symmetric, so column half h of D is row half h
  // transposed: the waves holding rows 128 h.. stage their blocks at the transposed
  // positions, a lane's four consecutive rows of one column as one 16-byte piece.  (The
  // value staged for (i, j) is then the one accumulated at (j, i); the two differ only
  // in the order the correction terms reached them.)  The update's result is staged
  // at its own positions, by the waves holding columns 128 h.., one element at a time.
  constexpr bool SYM = MODE != MODE_UPDATE;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (hand_a && h == 0) continue;   // (uniform)
    if constexpr (SYM) {
      if ((wm >> 1) == h) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int jl = (wm & 1) * 64 + bi * 32 + 8 * g + 4 * half;   // row of D, less 128 h
              const int i = wn * 128 + bj * 32 + li;                        // column of D
              *reinterpret_cast<f32x4 *>(st + i * LD::SP + jl) =
                  f32x4{acc[bi][bj][4 * g], acc[bi][bj][4 * g + 1], acc[bi][bj][4 * g + 2], acc[bi][bj][4 * g + 3]};
            }
      }
    } else if (wn == h) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int il = wm * 64 + bi * 32 + 8 * g + 4 * half;
            const int jl = bj * 32 + li;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(il + e) * LD::SP + jl] = acc[bi][bj][4 * g + e];
          }
    }
    __syncthreads();
    // thread u takes row u / 8 and, in that row, the 8-element pieces at columns
    // 8 (u % 8) and 8 (u % 8) + 64 of the half
#pragma unroll
    for (int q4 = 0; q4 < T2 * (T2 / 2 / 16) / T2_THREADS; ++q4) {
      const int u = tid + q4 * T2_THREADS;
      const int i = u >> 3;
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        const int jl = (u & 7) * 8 + 64 * pc;
        const int j = h * (T2 / 2) + jl;
        float e[8];
        if constexpr (MODE == MODE_UPDATE) {
          if (!fold) Xc.get8(i, j, e);
        }
        float dv[8];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const f32x4 x = *reinterpret_cast<const f32x4 *>(st + i * LD::SP + jl + 4 * m);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) dv[4 * m + e2] = x[e2];
        }
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float d = dv[q];
          const bool dg = fold && i == j + q;
          if constexpr (MODE == MODE_GRAM) {
            v[q] = c != 0.f ? d : b * d + (dg ? a : 0.f);
          } else if constexpr (MODE == MODE_SQUARE) {
            v[q] = c * d + (dg ? a : 0.f);   // d = (b / c) A + A^2
          } else {
            v[q] = fold ? d : __builtin_fmaf(a, e[q], d);
          }
        }
        if constexpr (APPLY) {
          const LayerDesc *L = ap.layers + t.layer;
          float *wrow = L->w + (int64_t)(t.row0 + i) * L->ld_w + t.col0 + j;
          const float nlr = -ap.lr;
          if (L->vec_w) {   // 16-byte aligned rows (the tile's columns start at a multiple of 256)
            GLOBAL_AS f32x4 *pw = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(wrow));
            f32x4 w4[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) w4[m] = pw[m];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) w4[m][e2] = __builtin_fmaf(nlr, v[4 * m + e2], w4[m][e2]);
              pw[m] = w4[m];
            }
          } else {
            GLOBAL_AS float *pw = gmem(wrow);
#pragma unroll
            for (int q = 0; q < 8; ++q) pw[q] = __builtin_fmaf(nlr, v[q], pw[q]);
          }
          if (ap.write_u) {
            GLOBAL_AS float *pu = gmem(L->u + (int64_t)(t.row0 + i) * L->ld_u + t.col0 + j);
#pragma unroll
            for (int q = 0; q < 8; ++q) pu[q] = v[q];
          }
        } else {
          if (!(hand_b && j < 64)) O.put8(i, j, v);
        }
      }
    }
    __syncthreads();   // the staging read before the next half lands
  }
  if constexpr (MODE == MODE_GRAM) {
    if (hand_a) {
      t256_hand_over<T2Lds<PREC, MODE_SQUARE>, 2>(acc, lds, wm, wn, li, half, [](float d, int, int) { return d; });
    } else {
      t256_hand_over<T2Lds<PREC, MODE_UPDATE>, 1>(acc, lds, wm, wn, li, half, [&](float d, int r, int q) {
        return b * d + ((fold && r == q) ? a : 0.f);
      });
    }
    if (c != 0.f) {   // (uniform) seed the square product with (b / c) A
      const float bc = b / c;
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[bi][bj][e] *= bc;
    }
  }
  if constexpr (MODE == MODE_SQUARE) {
    t256_hand_over<T2Lds<PREC, MODE_UPDATE>, 1>(acc, lds, wm, wn, li, half, [&](float d, int r, int q) {
      return c * d + ((fold && r == q) ? a : 0.f);   // d = (b / c) A + A^2
    });
  }
}

// All K Newton-Schulz steps of one 256 x 256 tile per workgroup (every tile of the chunk
// is 256 x 256 with ldx = lda = 256, the planner's chunk kind): Gram, square and update
// in turn, in place (X in its x0 planes, A then B in the planes of A).  The tile's
// 512 KB of planes are written and read back by one CU between the products, so they
// come back from the L2 and the Infinity Cache rather than HBM.
template <int PREC>
constexpr int t256_ns_lds() {
  constexpr int g = T2Lds<PREC, MODE_GRAM>::BYTES, s = T2Lds<PREC, MODE_SQUARE>::BYTES,
                u = T2Lds<PREC, MODE_UPDATE>::BYTES;
  return g > s ? (g > u ? g : u) : (s > u ? s : u);
}
template <typename S, int PREC>
__global__ __launch_bounds__(T2_THREADS) void gemm_t256_ns_kernel(const GemmTile *__restrict__ tiles, int first,
                                                                  char *ws, GemmParams gp, int steps,
                                                                  T256Apply ap) {
  __shared__ __attribute__((aligned(16))) char lds[t256_ns_lds<PREC>()];
  __shared__ float red8[8];
  const TileG t = tile_of(tiles, first + (int)blockIdx.x);
  t256_front<S, PREC>(t, ws, ap, red8);
  f32x16 acc[2][4];
  for (int it = 0; it < steps; ++it) {
    // (each product ends at a barrier after its last global stores, so the next one's
    // loads see them: one workgroup, one CU, one L1)
    t256_product<PREC, MODE_GRAM>(t, ws, gp, lds, acc, T256Apply{}, it < gp.plain_gram);
    if (gp.c != 0.f) t256_product<PREC, MODE_SQUARE>(t, ws, gp, lds, acc, T256Apply{}, it < gp.plain_square);
    if (it + 1 < steps) {
      t256_product<PREC, MODE_UPDATE>(t, ws, gp, lds, acc);
    } else {   // the last update applies O to W instead of storing X_K
      t256_product<PREC, MODE_UPDATE, true>(t, ws, gp, lds, acc, ap);
    }
  }
}

// ------------------------------------------------------------------ 256-blocks
// Chunks of matrices (or tiles) whose two sides are multiples of 256, other than single
// 256 x 256 tiles, run each product in 256 x 256 output blocks: eight waves of 64 x 128,
// K in slices of 32 through two LDS stages, half the operand-panel traffic per output
// element of the 128-blocks.  The symmetric products compute the blocks with bi <= bj
// and write the off-diagonal ones to both positions; a diagonal block's two operand
// panels are the same rows, loaded and staged once (SAME).
template <int PREC, int MODE>
struct B2Lds {
  static constexpr int BK = 32;
  static constexpr int NPL = PREC == PREC_BF16X3 ? 2 : 1;
  static constexpr int RP = BK + 8, CP = T2 + 8;
  static constexpr int ROWT = T2 * RP * 2;                      // one plane of a row panel
  static constexpr int COLT = BK * CP * 2;                      // one plane of the column panel
  static constexpr int RT = MODE == MODE_UPDATE ? COLT : ROWT;  // one plane of the column operand
  static constexpr int STAGE = NPL * (ROWT + RT);
  static constexpr int SP = T2 / 2 + 8;                         // D of a column half, row-major
  static constexpr int SPT = T2 + 4;                            // its transpose (mirror pass)
  static constexpr int STG = T2 * SP * 4 > (T2 / 2) * SPT * 4 ? T2 * SP * 4 : (T2 / 2) * SPT * 4;
  static constexpr int BYTES = 2 * STAGE > STG ? 2 * STAGE : STG;
  static constexpr int NQ = T2 * (BK / 8) / T2_THREADS;
  static_assert(T2 * (BK / 8) % T2_THREADS == 0 && BK * (T2 / 8) == T2 * (BK / 8), "whole chunks");
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// PLAIN (bf16x3 symmetric products only): the product of the hi planes alone, the lo
// operand planes neither loaded nor read; the result is still stored as both planes.
template <int PREC, int MODE, bool SAME, bool PLAIN>
__device__ __forceinline__ void b256_block(const TileG &t, int i0, int j0, char *ws, const GemmParams &gp,
                                           char *lds) {
  using LD = B2Lds<PREC, MODE>;
  constexpr int BK = LD::BK;
  static_assert(!PLAIN || (PREC == PREC_BF16X3 && MODE != MODE_UPDATE), "plain symmetric bf16x3 products");
  constexpr int NLD = PLAIN ? 1 : LD::NPL;     // operand planes loaded and staged
  constexpr bool SPLIT = PREC == PREC_BF16X3 && !PLAIN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // rows 64 wm.., columns 128 wn.. of the block
  const int li = lane & 31, half = lane >> 5;

  const Planes<PREC> Xc{ws + (gp.xsel ? t.x1 : t.x0), t.r, t.ldx};
  const Planes<PREC> Xn{ws + (gp.xsel ? t.x0 : t.x1), t.r, t.ldx};
  const Planes<PREC> A{ws + t.a, t.r, t.lda};
  const Planes<PREC> B{ws + t.b, t.r, t.lda};
  const Planes<PREC> Lp = MODE == MODE_GRAM ? Xc : (MODE == MODE_SQUARE ? A : B);
  const int kdim = MODE == MODE_GRAM ? t.ldx : t.lda;

  u32x4 rl_[LD::NPL * LD::NQ], rr_[LD::NPL * LD::NQ];
  auto load = [&](int kb) {
#pragma unroll
    for (int pl = 0; pl < NLD; ++pl) {
      const __bf16 *lb = pl ? Lp.lo() : Lp.hi();
      const __bf16 *xb = pl ? Xc.lo() : Xc.hi();
#pragma unroll
      for (int q = 0; q < LD::NQ; ++q) {
        const int idx = tid + q * T2_THREADS;
        const int row = idx / (BK / 8), ch = idx % (BK / 8);
        rl_[pl * LD::NQ + q] =
            *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(lb + (int64_t)(i0 + row) * Lp.ld + kb + ch * 8));
        if constexpr (MODE == MODE_UPDATE) {
          const int kr = idx / (T2 / 8), cc = idx % (T2 / 8);
          rr_[pl * LD::NQ + q] =
              *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(xb + (int64_t)(kb + kr) * Xc.ld + j0 + cc * 8));
        } else if constexpr (!SAME) {
          rr_[pl * LD::NQ + q] =
              *reinterpret_cast<const GLOBAL_AS u32x4 *>(gmem(lb + (int64_t)(j0 + row) * Lp.ld + kb + ch * 8));
        }
      }
    }
  };
  auto store = [&](char *stage) {
#pragma unroll
    for (int pl = 0; pl < NLD; ++pl) {
#pragma unroll
      for (int q = 0; q < LD::NQ; ++q) {
        const int idx = tid + q * T2_THREADS;
        const int row = idx / (BK / 8), ch = idx % (BK / 8);
        *reinterpret_cast<u32x4 *>(stage + pl * LD::ROWT + (row * LD::RP + ch * 8) * 2) = rl_[pl * LD::NQ + q];
        char *rt = stage + LD::NPL * LD::ROWT + pl * LD::RT;
        if constexpr (MODE == MODE_UPDATE) {
          const int kr = idx / (T2 / 8), cc = idx % (T2 / 8);
          *reinterpret_cast<u32x4 *>(rt + (kr * LD::CP + cc * 8) * 2) = rr_[pl * LD::NQ + q];
        } else if constexpr (!SAME) {
          *reinterpret_cast<u32x4 *>(rt + (row * LD::RP + ch * 8) * 2) = rr_[pl * LD::NQ + q];
        }
      }
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x16{};
  auto compute = [&](const char *stage) {
    const __bf16 *L0 = reinterpret_cast<const __bf16 *>(stage);
    const __bf16 *L1 = reinterpret_cast<const __bf16 *>(stage + LD::ROWT);
    const char *rs = SAME ? stage : stage + LD::NPL * LD::ROWT;
    const __bf16 *R0 = reinterpret_cast<const __bf16 *>(rs);
    const __bf16 *R1 = reinterpret_cast<const __bf16 *>(rs + (SAME ? LD::ROWT : LD::RT));
#pragma unroll
    for (int kc = 0; kc < BK; kc += 16) {
      const int k = kc + 8 * half;
      bf16x8 lh[2], ll[2], rh[4], rl[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        lh[b] = *reinterpret_cast<const bf16x8 *>(L0 + (wm * 64 + b * 32 + li) * LD::RP + k);
        if constexpr (SPLIT)
          ll[b] = *reinterpret_cast<const bf16x8 *>(L1 + (wm * 64 + b * 32 + li) * LD::RP + k);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if constexpr (MODE == MODE_UPDATE) {
          rh[b] = tr_frag(R0, LD::CP, k, wn * 128 + b * 32, lane);
          if constexpr (SPLIT) rl[b] = tr_frag(R1, LD::CP, k, wn * 128 + b * 32, lane);
        } else {
          rh[b] = *reinterpret_cast<const bf16x8 *>(R0 + (wn * 128 + b * 32 + li) * LD::RP + k);
          if constexpr (SPLIT)
            rl[b] = *reinterpret_cast<const bf16x8 *>(R1 + (wn * 128 + b * 32 + li) * LD::RP + k);
        }
      }
      if constexpr (SPLIT) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mma_bf16(ll[bi], rh[bj], acc[bi][bj]);
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mma_bf16(lh[bi], rl[bj], acc[bi][bj]);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mma_bf16(lh[bi], rh[bj], acc[bi][bj]);
    }
  };

  load(0);
  store(lds);
  __syncthreads();
  int cur = 0;
  for (int kb = 0; kb < kdim; kb += BK) {
    const bool more = kb + BK < kdim;
    if (more) load(kb + BK);
    compute(lds + cur * LD::STAGE);
    if (more) store(lds + (cur ^ 1) * LD::STAGE);
    __syncthreads();
    cur ^= 1;
  }

  // ---- epilogue, one column half at a time: the half staged row-major for the block's
  // own rows, then (off-diagonal symmetric blocks) transposed for the mirrored rows
  float *st = reinterpret_cast<float *>(lds);
  const float a = gp.a, b = gp.b, c = gp.c;
  const bool fold = gp.fold != 0;
  const Planes<PREC> O = MODE == MODE_GRAM ? (c != 0.f ? A : B) : (MODE == MODE_SQUARE ? B : Xn);
  // value stored at output (i, j) from the product d; e: element (i, j) of the addend
  auto finish = [&](float d, float e, int i, int j) -> float {
    const bool dg = fold && i == j;
    if constexpr (MODE == MODE_GRAM) {
      return c != 0.f ? d : b * d + (dg ? a : 0.f);
    } else if constexpr (MODE == MODE_SQUARE) {
      return __builtin_fmaf(c, d, b * e) + (dg ? a : 0.f);
    } else {
      return fold ? d : __builtin_fmaf(a, e, d);
    }
  };
  auto addend16 = [&](int i, int j, float (&e)[16]) {
    if constexpr (MODE == MODE_SQUARE) {
      A.get16(i, j, e);
    } else if constexpr (MODE == MODE_UPDATE) {
      if (!fold) Xc.get16(i, j, e);
    }
  };
  constexpr bool MIRROR = MODE != MODE_UPDATE && !SAME;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    if (wn == h) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int il = wm * 64 + bi * 32 + 8 * g + 4 * half, jl = bj * 32 + li;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(il + e) * LD::SP + jl] = acc[bi][bj][4 * g + e];
          }
    }
    __syncthreads();
#pragma unroll
    for (int q4 = 0; q4 < T2 * (T2 / 2 / 16) / T2_THREADS; ++q4) {
      const int u = tid + q4 * T2_THREADS;
      const int il = u >> 3, jl = (u & 7) * 16;   // block row il, columns 128 h + jl .. +15
      const int gi = i0 + il, gj = j0 + h * (T2 / 2) + jl;
      float e[16], dv[16], v[16];
      addend16(gi, gj, e);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(st + il * LD::SP + jl + 4 * m);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) dv[4 * m + e2] = x[e2];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = finish(dv[q], e[q], gi, gj + q);
      O.put16(gi, gj, v);
    }
    __syncthreads();
    if constexpr (MIRROR) {
      // D^T of the half: row jl (column 128 h + jl of the block) holds the mirrored row
      if (wn == h) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int il = wm * 64 + bi * 32 + 8 * g + 4 * half, jl = bj * 32 + li;
              *reinterpret_cast<f32x4 *>(st + jl * LD::SPT + il) =
                  f32x4{acc[bi][bj][4 * g], acc[bi][bj][4 * g + 1], acc[bi][bj][4 * g + 2], acc[bi][bj][4 * g + 3]};
            }
      }
      __syncthreads();
#pragma unroll
      for (int q4 = 0; q4 < (T2 / 2) * (T2 / 16) / T2_THREADS; ++q4) {
        const int u = tid + q4 * T2_THREADS;
        const int jl = u >> 4, il = (u & 15) * 16;   // mirrored row 128 h + jl, columns il .. +15
        const int gi = j0 + h * (T2 / 2) + jl, gj = i0 + il;
        float e[16], dv[16], v[16];
        addend16(gi, gj, e);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 x = *reinterpret_cast<const f32x4 *>(st + jl * LD::SPT + il + 4 * m);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) dv[4 * m + e2] = x[e2];
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = finish(dv[q], e[q], gi, gj + q);
        O.put16(gi, gj, v);
      }
      __syncthreads();
    }
  }
}

template <int PREC, int MODE, bool PLAIN = false>
__global__ __launch_bounds__(T2_THREADS) void gemm_b256_kernel(const GemmTile *__restrict__ tiles,
                                                               const GemmWork *__restrict__ work, char *ws,
                                                               GemmParams gp) {
  static_assert(PREC == PREC_BF16 || PREC == PREC_BF16X3, "bf16 planes");
  __shared__ __attribute__((aligned(16))) char lds[B2Lds<PREC, MODE>::BYTES];
  const GemmWork wk = work[xcd_work_index()];
  const TileG t = tile_of(tiles, wk.tile);
  // sides of every tile of the chunk are multiples of 256 (the planner's chunk kind), so
  // ldx = s, lda = r and no block reaches past them
  if (MODE != MODE_UPDATE && wk.bi == wk.bj) {   // uniform over the workgroup
    b256_block<PREC, MODE, true, PLAIN>(t, wk.bi * T2, wk.bj * T2, ws, gp, lds);
  } else {
    b256_block<PREC, MODE, false, PLAIN>(t, wk.bi * T2, wk.bj * T2, ws, gp, lds);
  }
}

template <typename S, int PREC>
hipError_t run_chunk(const LayerDesc *layers, const GemmTile *tiles, const GemmChunkLaunch &c, char *ws,
                     const NSParams &p, hipStream_t stream) {
  auto grid = [](int64_t n) { return dim3((unsigned)n); };
  if (c.n_mom > 0x7fffffff || c.n_stg > 0x7fffffff || c.n_sym > 0x7fffffff || c.n_upd > 0x7fffffff ||
      c.n_app > 0x7fffffff || c.tile_first + c.tile_n > 0x7fffffff)
    return hipErrorInvalidValue;
  if ((c.t256 || c.b256) && PREC != PREC_BF16 && PREC != PREC_BF16X3) return hipErrorInvalidValue;
  // 256-tile chunks with NS steps run the momentum, the norm and X0 inside their NS
  // kernel (the identity mode has no NS steps)
  const bool front = c.t256 && p.steps > 0;
  if (c.n_mom && !front) hipLaunchKernelGGL(gemm_momentum_kernel<S>, grid(c.n_mom), dim3(THREADS), 0, stream, layers, tiles, c.mom, ws, p.beta);
  if (c.tile_n && !front) hipLaunchKernelGGL(gemm_norm_kernel<S>, grid(c.tile_n), dim3(THREADS), 0, stream, layers, tiles, (int)c.tile_first, ws, p.eps, p.identity);
  if (c.n_stg && !front) hipLaunchKernelGGL((gemm_stage_kernel<S, PREC>), grid(c.n_stg), dim3(THREADS), 0, stream, layers, tiles, c.stg, ws);
  GemmParams gp{p.a, p.b, p.c, 0, PREC != PREC_BF16, p.plain_gram, p.plain_square};
  auto products = [&](auto bkc) {
    constexpr int BK = decltype(bkc)::value;
    for (int it = 0; it < p.steps; ++it) {
      gp.xsel = it & 1;
      hipLaunchKernelGGL((gemm_ns_kernel<PREC, MODE_GRAM, BK>), grid(c.n_sym), dim3(THREADS), 0, stream, tiles, c.sym, ws, gp);
      if (p.c != 0.f)
        hipLaunchKernelGGL((gemm_ns_kernel<PREC, MODE_SQUARE, BK>), grid(c.n_sym), dim3(THREADS), 0, stream, tiles, c.sym, ws, gp);
      hipLaunchKernelGGL((gemm_ns_kernel<PREC, MODE_UPDATE, BK>), grid(c.n_upd), dim3(THREADS), 0, stream, tiles, c.upd, ws, gp);
    }
  };
  if constexpr (PREC == PREC_BF16 || PREC == PREC_BF16X3) {
    if (c.t256 && p.steps > 0) {
      hipLaunchKernelGGL((gemm_t256_ns_kernel<S, PREC>), dim3((unsigned)c.tile_n), dim3(T2_THREADS), 0, stream, tiles,
                         (int)c.tile_first, ws, gp, p.steps, T256Apply{layers, p.lr, p.write_update, p.beta, p.eps});
    }
  }
  if constexpr (PREC == PREC_BF16 || PREC == PREC_BF16X3) {
    if (c.b256) {
      for (int it = 0; it < p.steps; ++it) {
        gp.xsel = it & 1;
        const dim3 bl(T2_THREADS);
        // bf16f8 requests (run with the bf16x3 products): the early symmetric products on
        // the hi planes alone, as on 256-tiles
        const bool plain_g = PREC == PREC_BF16X3 && it < p.plain_gram;
        const bool plain_s = PREC == PREC_BF16X3 && it < p.plain_square;
        if (plain_g)
          hipLaunchKernelGGL((gemm_b256_kernel<PREC, MODE_GRAM, PREC == PREC_BF16X3>), grid(c.n_sym), bl, 0, stream,
                             tiles, c.sym, ws, gp);
        else
          hipLaunchKernelGGL((gemm_b256_kernel<PREC, MODE_GRAM>), grid(c.n_sym), bl, 0, stream, tiles, c.sym, ws, gp);
        if (p.c != 0.f && plain_s)
          hipLaunchKernelGGL((gemm_b256_kernel<PREC, MODE_SQUARE, PREC == PREC_BF16X3>), grid(c.n_sym), bl, 0, stream,
                             tiles, c.sym, ws, gp);
        else if (p.c != 0.f)
          hipLaunchKernelGGL((gemm_b256_kernel<PREC, MODE_SQUARE>), grid(c.n_sym), bl, 0, stream, tiles, c.sym, ws, gp);
        hipLaunchKernelGGL((gemm_b256_kernel<PREC, MODE_UPDATE>), grid(c.n_upd), bl, 0, stream, tiles, c.upd, ws, gp);
      }
    }
  }
  if (c.t256 || c.b256) {
    // products launched above (bf16 planes only: the planner marks no fp32 chunk)
  } else if (c.long_k) {
    products(std::integral_constant<int, 64>{});
  } else {
    products(std::integral_constant<int, 32>{});
  }
  // the 256-tile kernel applies W itself after its last step (with no steps, X0 is
  // applied from the x0 planes); the per-product launches alternate the X buffers
  if (c.t256 && p.steps > 0) return hipGetLastError();
  const int xfinal = c.t256 ? 0 : (p.steps & 1);
  if (c.n_app)
    hipLaunchKernelGGL((gemm_apply_kernel<PREC>), grid(c.n_app), dim3(THREADS), 0, stream, layers, tiles, c.app, ws,
                       xfinal, p.lr, p.write_update);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_chunk(int prec, int state_bf16, const LayerDesc *layers, const GemmTile *tiles,
                             const GemmChunkLaunch &c, char *ws, const NSParams &p, hipStream_t stream) {
  if (c.tile_n <= 0) return hipSuccess;
  switch (prec) {
    case PREC_F32:
      return state_bf16 ? run_chunk<__bf16, PREC_F32>(layers, tiles, c, ws, p, stream)
                        : run_chunk<float, PREC_F32>(layers, tiles, c, ws, p, stream);
    case PREC_BF16:
      return state_bf16 ? run_chunk<__bf16, PREC_BF16>(layers, tiles, c, ws, p, stream)
                        : run_chunk<float, PREC_BF16>(layers, tiles, c, ws, p, stream);
    case PREC_BF16X3:
      return state_bf16 ? run_chunk<__bf16, PREC_BF16X3>(layers, tiles, c, ws, p, stream)
                        : run_chunk<float, PREC_BF16X3>(layers, tiles, c, ws, p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace himuon

// Fused HiMuon tile kernel for tiles up to 128 x 128 on gfx950.
//
// One workgroup owns one or more tiles and takes each of them through the whole
// step without leaving the CU:
//   momentum  M <- beta M + G  (HBM read of G and M, write of M),
//   per-tile Frobenius norm (fixed-order reduction, wavefront shuffles),
//   K Newton-Schulz steps with X, A = X X^T and B = b A + c A^2 resident in LDS
//   and registers (MFMA 32x32 tiles, fp32 accumulation),
//   W <- W - lr O  (HBM read and write of W).
// HBM therefore sees exactly one read and one write of every element; no
// workspace.  The same finite NS map runs on every tile independently, which is
// what "Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
// Optimization" (Abstract) defines; cross-layer batching comes from the tile
// table, which spans all layers of the plan.
//
// Data layout in LDS, per tile (edge TS in {32, 64, 128}, zero padded):
//   X  : the oriented tile (short side r = rows), row-major, TS x TS
//   AB : A = X X^T, then B = b A + c A^2 (both symmetric), row-major, TS x TS
// Element formats: PREC_F32 one fp32 array; PREC_BF16 one bf16 array;
// PREC_BF16X3 two bf16 arrays (hi = bf16(x), lo = bf16(x - hi)); PREC_BF16F8 the bf16
// hi array and two e4m3 arrays, h8 = e4m3(x 2^e) and l8 = e4m3((x - hi) 2^(e+8)), with
// a power-of-two exponent e per matrix and step.
// Each wave owns a 64 x 32 block (32 x 32 when TS = 32) of every product, so a 128 tile
// has 8 waves and two waves share each SIMD: one wave's LDS and VALU work overlaps the
// other's MFMAs.
//
// Products (all as D[m][n] = sum_k P[m][k] Q[n][k] with contiguous k):
//   Gram    A[p][q]   = sum_k X[p][k] X[q][k]
//   square  S[p][q]   = sum_k A[p][k] A[q][k]            (A symmetric)
//   update  D[j][i]   = sum_k X[k][j] B[i][k] = (B X)^T  (B symmetric)
// With fp32 or bf16x3 (hi + lo) operands, a is added to B's diagonal and the update is
// one product X^T (a I + B).  With plain bf16 operands, and with bf16 + e4m3 operands
// (whose X carries only about 2^-13 of precision), the update accumulates X^T B on top
// of a X^T formed in fp32 (from X in registers, or from bf16 hi + lo planes), so the
// a X term does not see the operands' rounding.
#include <type_traits>

#include "device_common.h"
#include "himuon_internal.h"

namespace himuon {
namespace {

using namespace dev;

// A wave's accumulators: NI x NJ MFMA 32x32 output blocks.
template <int NI, int NJ>
struct Acc {
  f32x16 b[NI][NJ];
};

// ------------------------------------------------------------------ geometry
#ifndef HIMUON_SCHED_GEMM
#define HIMUON_SCHED_GEMM 1
#endif
// order the GEMM loops' LDS reads and MFMAs explicitly (reads one chunk ahead)
constexpr bool SCHED_GEMM = HIMUON_SCHED_GEMM != 0;

template <int TS, int PREC>
struct Geo {
  // each wave owns a WBM x WBN block of every product; two waves share a SIMD
  static constexpr int WBM = TS >= 64 ? 64 : 32;      // wave block rows
  static constexpr int WBN = 32;                      // wave block columns
  static constexpr int NI = WBM / 32, NJ = WBN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int WPT = (TS / WBM) * (TS / WBN); // waves per tile: 8, 2, 1
  static constexpr int TPB = WPT == 1 ? 4 : 1;        // tiles per workgroup
  static constexpr int NT = 64 * WPT;                 // threads per tile
  static constexpr int THREADS = NT * TPB;
  // bf16 rows of 128-tiles are 256 bytes, unpadded, with their 16-byte chunks permuted
  // (chunk c of row r is stored at c ^ swz(r)): sixteen consecutive rows reading one
  // chunk, and four rows reading four adjacent chunks (transposing reads), then touch
  // sixteen distinct chunks.  Other tiles use a padded pitch.
  static constexpr bool SWZ = TS == 128;
  static constexpr int PB = SWZ ? TS : TS + 8;        // bf16 row pitch (elements)
  static constexpr int PF = TS + 4;                   // fp32 row pitch (elements)
  // e4m3 rows (PREC_BF16F8): 128 bytes for 128-tiles, their 16-byte chunks permuted
  // (chunk c of row r at c ^ swz8(r)), else padded to a multiple of 16 bytes
  static constexpr int P8 = SWZ ? TS : TS + 16;
  static constexpr int REGION = PREC == PREC_F32 ? TS * PF * 4
                              : PREC == PREC_BF16 ? TS * PB * 2
                              : PREC == PREC_BF16X3 ? TS * PB * 4 : TS * PB * 2 + 2 * TS * P8;
  // Tile area: [X] [AB] [X lo].  PREC_BF16F8 128-tiles keep a bf16 lo plane of X
  // (x - hi, pitch PB, 32 KB) after AB, which fills the 160 KB of LDS; 64-tiles keep
  // that precision in registers instead.
  static constexpr int XLO = PREC == PREC_BF16F8 && TS == 128 ? TS * PB * 2 : 0;
  // the fp32 staging copy (pitch PF) overlays the area from its start
  static constexpr int ST_BYTES = TS * PF * 4;
  static constexpr int BASE = 2 * REGION + XLO > ST_BYTES ? 2 * REGION + XLO : ST_BYTES;
  // the norm's per-wave partial sums: the last words of AB where the staging copy does
  // not reach them (AB is free from a tile's last barrier until its first A is stored),
  // else a slot of their own after the tile's planes
  static constexpr bool RED_IN_AB = 2 * REGION - 64 >= ST_BYTES;
  static constexpr int RED_OFF = RED_IN_AB ? 2 * REGION - 4 * WPT : BASE;
  static constexpr int TILE_LDS = BASE + (RED_IN_AB ? 0 : 64);
  // the instance without NS steps holds only the fp32 staging copy and the partial sums
  static constexpr int K0_RED_OFF = ST_BYTES, K0_LDS = ST_BYTES + 64;
  // the chunk permutation of row r: the two 2-bit halves of r % 16 swapped
  static __device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
  // column c of a row congruent to r16 modulo 16, as stored
  static __device__ __forceinline__ int bcol(int r16, int c) {
    if constexpr (SWZ) {
      return c ^ (swz(r16) << 3);
    } else {
      return c;
    }
  }
  // element offset of (r, c) in a bf16 matrix
  static __device__ __forceinline__ int bidx(int r, int c) { return r * PB + bcol(r & 15, c); }
  // The e4m3 rows' chunk permutation, a function of r % 16: sixteen consecutive rows
  // reading one chunk, and the eight rows of a transposing read (two adjacent chunks
  // each), then fall on distinct 16-byte bank groups of two 128-byte rows.
  static __device__ __forceinline__ int swz8(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
  // byte column c of a row congruent to r16 modulo 16, as stored
  static __device__ __forceinline__ int b8col(int r16, int c) {
    if constexpr (SWZ) {
      return c ^ (swz8(r16) << 4);
    } else {
      return c;
    }
  }
  static __device__ __forceinline__ int b8idx(int r, int c) { return r * P8 + b8col(r & 15, c); }
  // workgroup barriers synchronise one tile: several tiles per workgroup only with
  // one wave per tile
  static_assert(WPT == 1 || TPB == 1, "tile groups must not share s_barrier");
};

// A matrix in LDS in the precision's element format.
template <int PREC>
struct Mat;
template <>
struct Mat<PREC_F32> {
  float *f;
};
template <>
struct Mat<PREC_BF16> {
  __bf16 *hi;
};
template <>
struct Mat<PREC_BF16X3> {
  __bf16 *hi, *lo;
};
template <>
struct Mat<PREC_BF16F8> {
  __bf16 *hi;
  unsigned char *h8, *l8;
};

template <int TS, int PREC>
__device__ __forceinline__ Mat<PREC> make_mat(char *base) {
  Mat<PREC> m;
  if constexpr (PREC == PREC_F32) {
    m.f = reinterpret_cast<float *>(base);
  } else if constexpr (PREC == PREC_BF16) {
    m.hi = reinterpret_cast<__bf16 *>(base);
  } else if constexpr (PREC == PREC_BF16F8) {
    using G = Geo<TS, PREC>;
    m.hi = reinterpret_cast<__bf16 *>(base);
    m.h8 = reinterpret_cast<unsigned char *>(base + TS * G::PB * 2);
    m.l8 = reinterpret_cast<unsigned char *>(base + TS * G::PB * 2 + TS * G::P8);
  } else {
    m.hi = reinterpret_cast<__bf16 *>(base);
    m.lo = reinterpret_cast<__bf16 *>(base + TS * Geo<TS, PREC>::PB * 2);
  }
  return m;
}

// Synchronise the threads that share one tile.
template <int WPT>
__device__ __forceinline__ void tile_sync() {
  if constexpr (WPT > 1) {
    // this wave's LDS traffic is complete, then meet the other waves of the tile;
    // global loads in flight (the next tile's prefetch) are deliberately not waited for
    lds_barrier();
  } else {
    // one wave per tile: LDS traffic of a wave is processed in order; only the
    // compiler has to be kept from moving LDS accesses across this point
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Sum (resp. maximum) of one float per thread over the WPT waves of a tile, in a fixed
// order; every thread gets the result.  red holds WPT floats; the caller separates two
// uses of it by a tile_sync.
template <int WPT>
__device__ __forceinline__ float tile_sum(float v, float *red, int lane, int wv) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if constexpr (WPT > 1) {
    if (lane == 0) red[wv] = v;
    tile_sync<WPT>();
    v = red[0];
#pragma unroll
    for (int i = 1; i < WPT; ++i) v += red[i];
  }
  return v;
}
template <int WPT>
__device__ __forceinline__ float tile_max(float v, float *red, int lane, int wv) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  if constexpr (WPT > 1) {
    if (lane == 0) red[wv] = v;
    tile_sync<WPT>();
    v = red[0];
#pragma unroll
    for (int i = 1; i < WPT; ++i) v = __builtin_fmaxf(v, red[i]);
  }
  return v;
}

// Transposing operand read (see dev::tr_frag) in the tile's bf16 layout G::bidx.  The
// 8-byte pieces stay inside one 16-byte chunk, so the chunk permutation moves them whole.
template <class G>
__device__ __forceinline__ bf16x8 tr_frag_g(const __bf16 *buf, int k, int m, int lane) {
  // k = (multiple of 16) + 8 * (lane / 32): the rows' residues modulo 16 depend on the
  // lane only
  const int L = lane & 15, g = (lane >> 4) & 1, h8 = (lane >> 5) * 8;
  const int col = m + 16 * g + 4 * (L & 3);
  const __bf16 *p0 = buf + (k + (L >> 2)) * G::PB + G::bcol(h8 + (L >> 2), col);
  const __bf16 *p1 = buf + (k + 4 + (L >> 2)) * G::PB + G::bcol(h8 + 4 + (L >> 2), col);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(p1));
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Transposing e4m3 operand read: lane l receives buf[kb + 32 (l / 32) + i][m + l % 32] as
// byte i, i = 0..31.  ds_read_tr8_b64 works on groups of 16 lanes: lane i of a group
// receives byte i % 8 of the 8-byte pieces read by lanes i / 8 + 2 j, j = 0..7.  So lane
// t reads 8 consecutive columns (from 8 (t % 2)) of row t / 2 and receives column t of
// eight consecutive rows; four such reads cover the 32 rows of the lane's k run.
template <class G>
__device__ __forceinline__ i32x8 tr8_frag_g(const unsigned char *buf, int kb, int m, int lane) {
  const int t = lane & 15, g = lane >> 4;
  const int col = m + 16 * (g & 1) + 8 * (t & 1);
  const int r0 = kb + 32 * (g >> 1) + (t >> 1);
  i32x8 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2 *)(buf + G::b8idx(r0 + 8 * q, col)));
    out[2 * q] = v[0];
    out[2 * q + 1] = v[1];
  }
  return out;
}

// ------------------------------------------------------------------ wave GEMM
// acc.b[bi][bj] (+)= sum_k L(m, k) R(n, k) for m in the wave's L block, n in its R block.
// L(m, k) = Lmat[m][k] (TRANS_L false) or Lmat[k][m] (TRANS_L true); R(n, k) = Rmat[n][k].
// MFMA lane layout (32x32): operand lane l holds row (l % 32) of its 32-block and a
// run of contiguous k selected by l / 32; both operands use the same k runs.
// NB <= NI: only the first NB 32-row blocks of the L block take part.  RALIAS: the R
// block is L's first block (same matrix, same rows), so its fragments are not read again.

// One k-chunk of operand fragments (16 k for bf16 operands, 8 for fp32).
template <int TS, int PREC>
struct Frags {
  static constexpr int NI = Geo<TS, PREC>::NI, NJ = Geo<TS, PREC>::NJ;
  f32x4 lf[NI], rf[NJ];     // fp32
  bf16x8 lh[NI], rh[NJ];    // bf16 (hi parts)
  bf16x8 ll[NI], rl[NJ];    // bf16x3 lo parts
};

template <int TS, int PREC, bool TRANS_L, int NB, bool RALIAS>
__device__ __forceinline__ void load_frags(Frags<TS, PREC> &f, const Mat<PREC> &Lm, int l0, const Mat<PREC> &Rm,
                                           int r0, int lane, int kb) {
  using G = Geo<TS, PREC>;
  constexpr int NJ = G::NJ;
  static_assert(!RALIAS || (NJ == 1 && !TRANS_L), "aliased operands are one plain block");
  const int li = lane & 31, half = lane >> 5;
  if constexpr (PREC == PREC_F32) {
    constexpr int PF = G::PF;
    const int k = kb + 4 * half;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int m = l0 + b * 32 + li;
      if constexpr (TRANS_L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f.lf[b][e] = Lm.f[(k + e) * PF + m];
      } else {
        f.lf[b] = *reinterpret_cast<const f32x4 *>(Lm.f + m * PF + k);
      }
    }
    if constexpr (RALIAS) {
      f.rf[0] = f.lf[0];
    } else {
#pragma unroll
      for (int b = 0; b < NJ; ++b) f.rf[b] = *reinterpret_cast<const f32x4 *>(Rm.f + (r0 + b * 32 + li) * PF + k);
    }
  } else {
    const int k = kb + 8 * half;
    // the operands' rows are all congruent to lane % 16 modulo 16, so one column offset
    // serves every plain read of this chunk; kept opaque so that it is formed here,
    // once per chunk, rather than hoisted for every chunk of the loop
    int ko = G::bcol(li & 15, k);
    if constexpr (G::SWZ) asm("" : "+v"(ko));
    // issued in the order the MFMAs consume them (see mma_frags)
    auto lread = [&](const __bf16 *plane, int b) -> bf16x8 {
      if constexpr (TRANS_L) {
        return tr_frag_g<G>(plane, k, l0 + b * 32, lane);
      } else {
        return *reinterpret_cast<const bf16x8 *>(plane + (l0 + b * 32 + li) * G::PB + ko);
      }
    };
    auto rread = [&](const __bf16 *plane, int b) -> bf16x8 {
      return *reinterpret_cast<const bf16x8 *>(plane + (r0 + b * 32 + li) * G::PB + ko);
    };
    if constexpr (RALIAS) {
      f.lh[0] = lread(Lm.hi, 0);
      if constexpr (PREC == PREC_BF16X3) f.ll[0] = lread(Lm.lo, 0);
#pragma unroll
      for (int b = 1; b < NB; ++b) {
        if constexpr (PREC == PREC_BF16X3) f.ll[b] = lread(Lm.lo, b);
        f.lh[b] = lread(Lm.hi, b);
      }
      f.rh[0] = f.lh[0];
      if constexpr (PREC == PREC_BF16X3) f.rl[0] = f.ll[0];
    } else {
#pragma unroll
      for (int b = 0; b < NJ; ++b) f.rh[b] = rread(Rm.hi, b);
      if constexpr (PREC == PREC_BF16X3) {
#pragma unroll
        for (int b = 0; b < NB; ++b) f.ll[b] = lread(Lm.lo, b);
#pragma unroll
        for (int b = 0; b < NJ; ++b) f.rl[b] = rread(Rm.lo, b);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) f.lh[b] = lread(Lm.hi, b);
    }
  }
}

// The MFMAs of one chunk; zero: this chunk starts the sum (the accumulators are not read).
template <int TS, int PREC, int NB>
__device__ __forceinline__ void mma_frags(Acc<Geo<TS, PREC>::NI, Geo<TS, PREC>::NJ> &acc, const Frags<TS, PREC> &f,
                                          bool zero) {
  constexpr int NJ = Geo<TS, PREC>::NJ;
  if constexpr (PREC == PREC_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NJ; ++bj)
          acc.b[bi][bj] = mma_f32(f.lf[bi][e], f.rf[bj][e], (zero && e == 0) ? f32x16{} : acc.b[bi][bj]);
  } else if constexpr (PREC == PREC_BF16X3) {
    // small cross terms first: lo * hi + hi * lo + hi * hi
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj) acc.b[bi][bj] = mma_bf16(f.ll[bi], f.rh[bj], zero ? f32x16{} : acc.b[bi][bj]);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj) acc.b[bi][bj] = mma_bf16(f.lh[bi], f.rl[bj], acc.b[bi][bj]);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj) acc.b[bi][bj] = mma_bf16(f.lh[bi], f.rh[bj], acc.b[bi][bj]);
  } else {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj) acc.b[bi][bj] = mma_bf16(f.lh[bi], f.rh[bj], zero ? f32x16{} : acc.b[bi][bj]);
  }
}

// reads of the next chunk go out during the first half of a chunk's MFMAs
template <int NM, int NR>
constexpr int reads_per_mfma() {
  return (NR + (NM + 1) / 2 - 1) / ((NM + 1) / 2);
}

// Instruction-scheduler directives: NM MFMAs, each followed by up to RPM LDS reads,
// until NR reads are placed.
template <int NM, int NR, int RPM>
__device__ __forceinline__ void sched_mfma_reads() {
  if constexpr (NM > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR < RPM ? NR : RPM, 0);
    sched_mfma_reads<NM - 1, (NR > RPM ? NR - RPM : 0), RPM>();
  }
}
template <int NC, int NM, int NR>
__device__ __forceinline__ void sched_chunks() {
  if constexpr (NC > 1) {
    sched_mfma_reads<NM, NR, reads_per_mfma<NM, NR>()>();
    sched_chunks<NC - 1, NM, NR>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
}

// ---- PREC_BF16F8 products.  Per 64-k chunk, four stages of MFMAs: the correction
// products h8_L l8_R and l8_L h8_R (one e4m3 MFMA, K = 64, per output block each), then
// the main product hi_L hi_R in two 32-k halves (two bf16 MFMAs per block each), so that
// every stage takes the same MFMA time.  The operands of stage i + 1 are read from LDS
// while the MFMAs of stage i run, so a wave holds the operands of at most two stages.
template <int TS>
struct F8Half {   // one e4m3 plane of each side, one 64-k chunk
  static constexpr int NI = Geo<TS, PREC_BF16F8>::NI, NJ = Geo<TS, PREC_BF16F8>::NJ;
  i32x8 l[NI], r[NJ];
};
template <int TS>
struct HiPiece {  // bf16 hi of each side, one 32-k half chunk (two 16-k pieces)
  static constexpr int NI = Geo<TS, PREC_BF16F8>::NI, NJ = Geo<TS, PREC_BF16F8>::NJ;
  bf16x8 l[2][NI], r[2][NJ];
};

// The e4m3 operands of one correction product: L from plane lp (rows, or columns when
// TRANS_L), R from plane rp, k in [kb, kb + 64).  READ_R false: R is not read; B0 = 1: the
// first L block is not read (the caller supplies both, from the other correction stage,
// when R is L's first block).
template <int TS, bool TRANS_L, int NB, bool READ_R = true, int B0 = 0>
__device__ __forceinline__ void load_f8(F8Half<TS> &f, const unsigned char *lp, int l0, const unsigned char *rp,
                                        int r0, int lane, int kb) {
  using G = Geo<TS, PREC_BF16F8>;
  const int li = lane & 31, half = lane >> 5;
  // plain reads: 32 bytes of row r from byte kb + 32 (lane / 32); the rows are all
  // congruent to lane % 16 modulo 16, so two column offsets serve every plain read
  int ko0 = G::b8col(li & 15, kb + 32 * half), ko1 = G::b8col(li & 15, kb + 32 * half + 16);
  if constexpr (G::SWZ) {
    asm("" : "+v"(ko0));
    asm("" : "+v"(ko1));
  }
  auto prow = [&](const unsigned char *plane, int r) -> i32x8 {
    const i32x4 a = *reinterpret_cast<const i32x4 *>(plane + r * G::P8 + ko0);
    const i32x4 b = *reinterpret_cast<const i32x4 *>(plane + r * G::P8 + ko1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  if constexpr (READ_R) {
#pragma unroll
    for (int b = 0; b < G::NJ; ++b) f.r[b] = prow(rp, r0 + b * 32 + li);
  }
#pragma unroll
  for (int b = B0; b < NB; ++b) {
    if constexpr (TRANS_L) {
      f.l[b] = tr8_frag_g<G>(lp, kb, l0 + b * 32, lane);
    } else {
      f.l[b] = prow(lp, l0 + b * 32 + li);
    }
  }
}

// bf16 hi operands of the 32-k half chunk at k0 (two 16-k pieces)
template <int TS, bool TRANS_L, int NB, bool RALIAS>
__device__ __forceinline__ void load_hi(HiPiece<TS> &h, const Mat<PREC_BF16F8> &Lm, int l0, const Mat<PREC_BF16F8> &Rm,
                                        int r0, int lane, int k0) {
  using G = Geo<TS, PREC_BF16F8>;
  const int li = lane & 31, half = lane >> 5;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int k = k0 + 16 * p + 8 * half;
    int ko = G::bcol(li & 15, k);
    if constexpr (G::SWZ) asm("" : "+v"(ko));
    if constexpr (!RALIAS) {
#pragma unroll
      for (int b = 0; b < G::NJ; ++b)
        h.r[p][b] = *reinterpret_cast<const bf16x8 *>(Rm.hi + (r0 + b * 32 + li) * G::PB + ko);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if constexpr (TRANS_L) {
        h.l[p][b] = tr_frag_g<G>(Lm.hi, k, l0 + b * 32, lane);
      } else {
        h.l[p][b] = *reinterpret_cast<const bf16x8 *>(Lm.hi + (l0 + b * 32 + li) * G::PB + ko);
      }
    }
    if constexpr (RALIAS) h.r[p][0] = h.l[p][0];
  }
}

// Scheduler directives for the stage sequence: stage i's MFMAs, each followed by some
// of stage i + 1's reads.  Stage kinds: 0, 1 the correction products, 2, 3 the halves.
// NRF / NRB: reads of the first / second correction stage, NRH: of a half.
template <int ST, int NST, int NMF, int NRF, int NRB, int NMH, int NRH>
__device__ __forceinline__ void sched_f8() {
  constexpr int kind = ST % 4, next = (ST + 1) % 4;
  constexpr int NM = kind < 2 ? NMF : NMH;
  if constexpr (ST + 1 < NST) {
    constexpr int NR = next == 0 ? NRF : next == 1 ? NRB : NRH;
    if constexpr (NR > 0) {
      sched_mfma_reads<NM, NR, (NR + NM - 1) / NM>();
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    }
    sched_f8<ST + 1, NST, NMF, NRF, NRB, NMH, NRH>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
}

// sc: the E8M0 scale byte of both correction products, 127 - (eL + eR + 8), which undoes
// the operands' exponents
template <int TS, bool TRANS_L, bool ZERO, int NB, bool RALIAS>
__device__ __forceinline__ void wave_gemm_f8(Acc<Geo<TS, PREC_BF16F8>::NI, Geo<TS, PREC_BF16F8>::NJ> &acc,
                                             const Mat<PREC_BF16F8> &Lm, int l0, const Mat<PREC_BF16F8> &Rm, int r0,
                                             int lane, int sc) {
  using G = Geo<TS, PREC_BF16F8>;
  constexpr int NJ = G::NJ;
  static_assert(TS % 64 == 0, "e4m3 products run on 64-k chunks");
  constexpr int NC = TS / 64;
  // RALIAS: the R block is L's first block, so the second correction stage's operands
  // l8_L[0] and h8_R are the first stage's l8_R and h8_L[0], kept in registers
  static_assert(!RALIAS || !TRANS_L, "aliased operands are plain rows");
  constexpr int NRF = NB * (TRANS_L ? 4 : 2) + 2 * NJ;            // reads of one correction stage
  constexpr int NRB = RALIAS ? 2 * (NB - 1) : NRF;                 // of the second one
  constexpr int NRH = 2 * (NB * (TRANS_L ? 2 : 1) + (RALIAS ? 0 : NJ));  // reads of one half
  constexpr int NMF = NB * NJ, NMH = 2 * NB * NJ;
  F8Half<TS> fa, fb;
  HiPiece<TS> h[2];
  load_f8<TS, TRANS_L, NB>(fa, Lm.h8, l0, Rm.l8, r0, lane, 0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int kb = 64 * c;
    // h8_L l8_R (small terms first)
    if constexpr (RALIAS) {
      load_f8<TS, TRANS_L, NB, false, 1>(fb, Lm.l8, l0, Rm.h8, r0, lane, kb);
      fb.l[0] = fa.r[0];
      fb.r[0] = fa.l[0];
    } else {
      load_f8<TS, TRANS_L, NB>(fb, Lm.l8, l0, Rm.h8, r0, lane, kb);
    }
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj)
        acc.b[bi][bj] = mma_f8s(fa.l[bi], fa.r[bj], (ZERO && c == 0) ? f32x16{} : acc.b[bi][bj], sc, 127);
    // l8_L h8_R
    load_hi<TS, TRANS_L, NB, RALIAS>(h[0], Lm, l0, Rm, r0, lane, kb);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj) acc.b[bi][bj] = mma_f8s(fb.l[bi], fb.r[bj], acc.b[bi][bj], sc, 127);
    // hi_L hi_R in two halves
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (s2 == 0) {
        load_hi<TS, TRANS_L, NB, RALIAS>(h[1], Lm, l0, Rm, r0, lane, kb + 32);
      } else if (c + 1 < NC) {
        load_f8<TS, TRANS_L, NB>(fa, Lm.h8, l0, Rm.l8, r0, lane, kb + 64);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
          for (int bj = 0; bj < NJ; ++bj) acc.b[bi][bj] = mma_bf16(h[s2].l[p][bi], h[s2].r[p][bj], acc.b[bi][bj]);
    }
  }
  if constexpr (SCHED_GEMM) {
    __builtin_amdgcn_sched_group_barrier(0x100, NRF, 0);
    sched_f8<0, 4 * NC, NMF, NRF, NRB, NMH, NRH>();
  }
}

// Full K = TS contraction in the fp32, bf16 and bf16x3 formats; ZERO: start from zero,
// else accumulate onto acc.  The fragments of chunk c + 1 are read from LDS while the
// MFMAs of chunk c run.
template <int TS, int PREC, bool TRANS_L, bool ZERO, int NB, bool RALIAS>
__device__ __forceinline__ void wave_gemm_std(Acc<Geo<TS, PREC>::NI, Geo<TS, PREC>::NJ> &acc, const Mat<PREC> &Lm,
                                              int l0, const Mat<PREC> &Rm, int r0, int lane) {
  using G = Geo<TS, PREC>;
  static_assert(NB >= 1 && NB <= G::NI, "row blocks");
  constexpr int KC = PREC == PREC_F32 ? 8 : 16;
  constexpr int NC = TS / KC;
  // LDS read and MFMA instructions per chunk
  constexpr int PLANES = PREC == PREC_BF16X3 ? 2 : 1;
  constexpr int LREADS = PREC == PREC_F32 ? (TRANS_L ? 4 : 1) : (TRANS_L ? 2 : 1);
  constexpr int NR = PLANES * (NB * LREADS + (RALIAS ? 0 : G::NJ));
  constexpr int NM = (PREC == PREC_F32 ? 4 : PREC == PREC_BF16X3 ? 3 : 1) * NB * G::NJ;
  Frags<TS, PREC> f[2];
  load_frags<TS, PREC, TRANS_L, NB, RALIAS>(f[0], Lm, l0, Rm, r0, lane, 0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + 1 < NC) load_frags<TS, PREC, TRANS_L, NB, RALIAS>(f[(c + 1) & 1], Lm, l0, Rm, r0, lane, (c + 1) * KC);
    mma_frags<TS, PREC, NB>(acc, f[c & 1], ZERO && c == 0);
  }
  if constexpr (SCHED_GEMM) {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    sched_chunks<NC, NM, NR>();
  }
}

// Full K = TS contraction; ZERO: start from zero, else accumulate onto acc.
// f8sc: the correction products' scale byte (PREC_BF16F8 only).
template <int TS, int PREC, bool TRANS_L, bool ZERO, int NB = Geo<TS, PREC>::NI, bool RALIAS = false>
__device__ __forceinline__ void wave_gemm(Acc<Geo<TS, PREC>::NI, Geo<TS, PREC>::NJ> &acc, const Mat<PREC> &Lm, int l0,
                                          const Mat<PREC> &Rm, int r0, int lane, int f8sc = 127) {
  if constexpr (PREC == PREC_BF16F8) {
    wave_gemm_f8<TS, TRANS_L, ZERO, NB, RALIAS>(acc, Lm, l0, Rm, r0, lane, f8sc);
  } else {
    wave_gemm_std<TS, PREC, TRANS_L, ZERO, NB, RALIAS>(acc, Lm, l0, Rm, r0, lane);
  }
}

// ------------------------------------------------------------------ symmetric products
// A = X X^T and A^2 are symmetric: of the (TS/32)^2 32x32 blocks only those on and
// above the diagonal are computed, each off-diagonal block written to both of its
// positions.  A job is the part one wave computes: NB row blocks from row p0 against
// the column block q0.  For 128-tiles the ten blocks fall on the four SIMDs (waves w and
// w + 4 share one) as 3 + 3 + 2 + 2 instead of 4 + 4 + 4 + 4, and each of the two busier
// SIMDs holds one off-diagonal block (the one that needs the second, untransposed copy).
struct SymJob {
  int p0, q0, nb;
  bool alias;  // q0 == p0: the column block is the first row block
};

template <int TS>
__device__ __forceinline__ SymJob sym_job(int wv) {
  if constexpr (TS == 128) {
    // w0: (0,0) (1,0)   w1: (2,2) (3,2)   w2: (0,2)   w3: (0,3)
    // w4: (1,1)         w5: (3,3)         w6: (1,2)   w7: (1,3)
    switch (wv) {
      case 0: return {0, 0, 2, true};
      case 1: return {64, 64, 2, true};
      case 2: return {0, 64, 1, false};
      case 3: return {0, 96, 1, false};
      case 4: return {32, 32, 1, true};
      case 5: return {96, 96, 1, true};
      case 6: return {32, 64, 1, false};
      default: return {32, 96, 1, false};
    }
  } else if constexpr (TS == 64) {
    // w0: (0,0) (1,0)   w1: (1,1)
    return wv == 0 ? SymJob{0, 0, 2, true} : SymJob{32, 32, 1, true};
  } else {
    return {0, 0, 1, true};
  }
}

// Runs f(NB, RALIAS) (as integral constants) for the wave's job.
template <int TS, class F>
__device__ __forceinline__ void with_job(const SymJob &jb, F &&f) {
  if constexpr (TS == 128) {
    if (jb.nb == 2) {
      f(std::integral_constant<int, 2>{}, std::true_type{});
    } else if (jb.alias) {
      f(std::integral_constant<int, 1>{}, std::true_type{});
    } else {
      f(std::integral_constant<int, 1>{}, std::false_type{});
    }
  } else if constexpr (TS == 64) {
    if (jb.nb == 2) {
      f(std::integral_constant<int, 2>{}, std::true_type{});
    } else {
      f(std::integral_constant<int, 1>{}, std::true_type{});
    }
  } else {
    f(std::integral_constant<int, 1>{}, std::true_type{});
  }
}

// Element (bi, bj, r) of a wave's accumulators sits at
//   row = p0 + bi*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = q0 + bj*32 + lane%32.
// These helpers move 4 consecutive rows (r%4 = 0..3) of one column at a time to or
// from position [col][row..row+3] of a row-major LDS matrix, i.e. they store the
// transpose of the accumulator block.

// The exponents of one kind of matrix over the NS steps, as packed bytes in scalar
// registers: entry k of the table is the current one at step k, and the last entry
// serves every later step.  (Indexing the kernel argument by the step would move it to
// scratch memory.)
struct ExpStream {
  uint64_t lo = 0, hi = 0;
  int n = 0;
  __device__ __forceinline__ void init(const int8_t (&e)[kF8Steps]) {
    static_assert(kF8Steps == 16, "two 64-bit words");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo |= (uint64_t)(uint8_t)e[i] << (8 * i);
      hi |= (uint64_t)(uint8_t)e[8 + i] << (8 * i);
    }
  }
  __device__ __forceinline__ int cur() const { return (int)(int8_t)(lo & 0xff); }
  __device__ __forceinline__ int next() const { return n + 1 < kF8Steps ? (int)(int8_t)((lo >> 8) & 0xff) : cur(); }
  __device__ __forceinline__ void advance() {
    if (n + 1 < kF8Steps) {
      lo = (lo >> 8) | (hi << 56);
      hi >>= 8;
      ++n;
    }
  }
};

// The three exponent streams of PREC_BF16F8 (X, A, B); empty for the other formats.
template <bool ON>
struct F8Steps {
  __device__ __forceinline__ void init(const F8Exps &) {}
  __device__ __forceinline__ int x() const { return 0; }
  __device__ __forceinline__ int xn() const { return 0; }
  __device__ __forceinline__ int a() const { return 0; }
  __device__ __forceinline__ int b() const { return 0; }
  __device__ __forceinline__ void advance() {}
};
template <>
struct F8Steps<true> {
  ExpStream sx, sa, sb;
  __device__ __forceinline__ void init(const F8Exps &e) {
    sx.init(e.x);
    sa.init(e.a);
    sb.init(e.b);
  }
  __device__ __forceinline__ int x() const { return sx.cur(); }
  __device__ __forceinline__ int xn() const { return sx.next(); }
  __device__ __forceinline__ int a() const { return sa.cur(); }
  __device__ __forceinline__ int b() const { return sb.cur(); }
  __device__ __forceinline__ void advance() {
    sx.advance();
    sa.advance();
    sb.advance();
  }
};

// Divisors of the e4m3 planes (PREC_BF16F8): the hi plane holds x / h = x 2^e, the lo
// plane r / l = r 2^(e + 8).
struct F8S {
  float h = 1.f, l = 1.f / 256.f;
};
__device__ __forceinline__ F8S f8s_of(int e) { return F8S{pow2i(-e), pow2i(-e - 8)}; }

// Store the transpose of the accumulators' first NB row blocks into a matrix in the
// precision's format.  SCALE: the stored value is s_store * acc; BACK: afterwards acc <-
// s_back * acc (one pass over the accumulators serves both).  MIRROR (symmetric
// results): blocks off the diagonal are also stored untransposed, at [row][col].
// f8: the e4m3 planes' multipliers.  LO (PREC_BF16F8): the residual x - hi is also
// stored as bf16 in the plane lo (same layout as hi), which with hi gives the value to
// about 2^-17; only the storing wave reads it back.
template <int TS, int PREC, bool SCALE = false, bool BACK = false, int NB = Geo<TS, PREC>::NI, bool MIRROR = false,
          bool LO = false>
__device__ __forceinline__ void store_acc_t(Acc<Geo<TS, PREC>::NI, Geo<TS, PREC>::NJ> &acc, const Mat<PREC> &m, int p0, int q0,
                                            int lane, float s_store = 1.f, float s_back = 1.f, F8S f8 = F8S{},
                                            __bf16 *lo = nullptr) {
  using G = Geo<TS, PREC>;
  static_assert(!LO || PREC == PREC_BF16F8, "a separate lo plane only beside the e4m3 planes");
  const int li = lane & 31, half = lane >> 5;
#pragma unroll
  for (int bi = 0; bi < NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < G::NJ; ++bj) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = p0 + bi * 32 + 8 * g + 4 * half;
        const int col = q0 + bj * 32 + li;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc.b[bi][bj][4 * g + e];
          v[e] = SCALE ? x * s_store : x;
          if constexpr (BACK) acc.b[bi][bj][4 * g + e] = x * s_back;
        }
        if constexpr (PREC == PREC_BF16F8) {
          // hi (bf16) as below; h8 and l8 (e4m3) at [col][row .. row+3]: one 4-byte write each
          const int o = col * G::PB + G::bcol(li & 15, row);
          const u32x2 hi = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2 *>(m.hi + o) = hi;
          const float r0 = v[0] - __builtin_bit_cast(float, hi[0] << 16);
          const float r1 = v[1] - __builtin_bit_cast(float, hi[0] & 0xffff0000u);
          const float r2 = v[2] - __builtin_bit_cast(float, hi[1] << 16);
          const float r3 = v[3] - __builtin_bit_cast(float, hi[1] & 0xffff0000u);
          const int o8 = col * G::P8 + G::b8col(li & 15, row);
          *reinterpret_cast<unsigned *>(m.h8 + o8) = pack_fp8x4(v[0], v[1], v[2], v[3], f8.h);
          *reinterpret_cast<unsigned *>(m.l8 + o8) = pack_fp8x4(r0, r1, r2, r3, f8.l);
          if constexpr (LO) *reinterpret_cast<u32x2 *>(lo + o) = u32x2{pack_bf16x2(r0, r1), pack_bf16x2(r2, r3)};
        } else if constexpr (PREC == PREC_F32) {
          *reinterpret_cast<f32x4 *>(m.f + col * G::PF + row) = v;
          if (MIRROR && p0 + bi * 32 != q0 + bj * 32) {   // off the diagonal (wave-uniform)
#pragma unroll
            for (int e = 0; e < 4; ++e) m.f[(row + e) * G::PF + col] = v[e];
          }
        } else {
          // col = (multiple of 32) + lane % 32
          const int o = col * G::PB + G::bcol(li & 15, row);
          const u32x2 hi = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2 *>(m.hi + o) = hi;
          if constexpr (PREC == PREC_BF16X3) {
            // the residuals v - hi are exact in fp32; hi is read back from the packed
            // pair (low half: shift up, high half: mask), not converted again
            const u32x2 lo = u32x2{pack_bf16x2(v[0] - __builtin_bit_cast(float, hi[0] << 16),
                                   v[1] - __builtin_bit_cast(float, hi[0] & 0xffff0000u)),
                       pack_bf16x2(v[2] - __builtin_bit_cast(float, hi[1] << 16),
                                   v[3] - __builtin_bit_cast(float, hi[1] & 0xffff0000u))};
            *reinterpret_cast<u32x2 *>(m.lo + o) = lo;
          }
        }
      }
    }
  if constexpr (MIRROR && PREC != PREC_F32) {
    // Off-diagonal blocks: read the block just stored (this wave's own LDS writes,
    // processed in order) back with transposing reads, which hand each lane eight
    // consecutive columns of one row of the untransposed block, and store those as one
    // 16-byte chunk at [row][col].
    // (the lane index is made opaque here so that the lane-dependent addresses are
    // formed at this point instead of being kept live across the whole iteration)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 31, lh = ln >> 5;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      if (p0 + bi * 32 == q0) continue;   // wave-uniform
      const int r = p0 + bi * 32 + lr;
#pragma unroll
      for (int ks = 0; ks < 32; ks += 16) {
        const int k = q0 + ks + 8 * lh;
        const int od = G::bidx(r, k);
        const bf16x8 vh = tr_frag_g<G>(m.hi, k, p0 + bi * 32, ln);
        if constexpr (PREC == PREC_BF16X3) {
          const bf16x8 vl = tr_frag_g<G>(m.lo, k, p0 + bi * 32, ln);
          *reinterpret_cast<bf16x8 *>(m.lo + od) = vl;
        }
        *reinterpret_cast<bf16x8 *>(m.hi + od) = vh;
      }
      if constexpr (PREC == PREC_BF16F8) {
        // e4m3 planes: lane t of a 16-lane group g reads 8 bytes of row q0 + 16 u + 8 (g / 2)
        // + t / 2 of the transposed copy, and the transposing read hands lane t 8
        // consecutive columns (q0 + 16 u + 8 (g / 2) ..) of row pb + 16 (g % 2) + t of the
        // untransposed block, stored as one 8-byte piece.
        const int pb = p0 + bi * 32, t = ln & 15, gg = ln >> 4;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int so = G::b8idx(q0 + 16 * u + 8 * (gg >> 1) + (t >> 1), pb + 16 * (gg & 1) + 8 * (t & 1));
          const int dof = G::b8idx(pb + 16 * (gg & 1) + t, q0 + 16 * u + 8 * (gg >> 1));
          const i32x2 a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2 *)(m.h8 + so));
          const i32x2 b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2 *)(m.l8 + so));
          *reinterpret_cast<i32x2 *>(m.h8 + dof) = a;
          *reinterpret_cast<i32x2 *>(m.l8 + dof) = b;
        }
      }
    }
  }
}

// m[i][i] += d for the diagonal elements inside the first NB row blocks of the block
// at (p0, q0).  Each of them was written by this same wave (the block is stored
// transposed, and (i, i) is its own transpose), and LDS accesses of one wave complete
// in order.
template <int TS, int PREC, int NB = Geo<TS, PREC>::NI>
__device__ __forceinline__ void add_diag(const Mat<PREC> &m, int p0, int q0, int lane, float d) {
  using G = Geo<TS, PREC>;
  if (q0 < p0 || q0 >= p0 + NB * 32 || lane >= G::WBN) return;
  const int i = q0 + lane;
  if constexpr (PREC == PREC_F32) {
    m.f[i * G::PF + i] += d;
  } else {
    const int o = G::bidx(i, i);
    const float v = (float)m.hi[o] + (float)m.lo[o] + d;
    const __bf16 hi = (__bf16)v;
    m.hi[o] = hi;
    m.lo[o] = (__bf16)(v - (float)hi);
  }
}

// The a X term of the update (PREC_BF16F8): this wave's block of X read back from its hi
// and lo planes (the positions store_acc_t<..., LO> writes), where hi + lo is exact in fp32
// and holds X to about 2^-17.  The reads are issued before the barrier that ends the
// update (X is unchanged until after it) and added to the accumulators after it, so the
// wave does not wait for its MFMA results before the barrier.
template <int TS>
struct XPiece {
  static constexpr int NI = Geo<TS, PREC_BF16F8>::NI, NJ = Geo<TS, PREC_BF16F8>::NJ;
  u32x2 h[NI][NJ][4], l[NI][NJ][4];
  __device__ __forceinline__ void load(const __bf16 *hi, const __bf16 *lo, int p0, int q0, int lane) {
    using G = Geo<TS, PREC_BF16F8>;
    // (the lane index is made opaque so that these addresses are formed here rather than
    // hoisted out of the tile loop, where they would hold registers across every product)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int li = ln & 31, half = ln >> 5;
#pragma unroll
    for (int bi = 0; bi < NI; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int o = (q0 + bj * 32 + li) * G::PB + G::bcol(li & 15, p0 + bi * 32 + 8 * g + 4 * half);
          h[bi][bj][g] = *reinterpret_cast<const u32x2 *>(hi + o);
          l[bi][bj][g] = *reinterpret_cast<const u32x2 *>(lo + o);
        }
  }
  // acc += a (hi + lo)
  __device__ __forceinline__ void add_to(Acc<NI, NJ> &acc, float a) const {
#pragma unroll
    for (int bi = 0; bi < NI; ++bi)
#pragma unroll
      for (int bj = 0; bj < NJ; ++bj)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned hw = h[bi][bj][g][e >> 1], lw = l[bi][bj][g][e >> 1];
            const float hv = __builtin_bit_cast(float, (e & 1) ? (hw & 0xffff0000u) : (hw << 16));
            const float lv = __builtin_bit_cast(float, (e & 1) ? (lw & 0xffff0000u) : (lw << 16));
            acc.b[bi][bj][4 * g + e] = __builtin_fmaf(a, hv + lv, acc.b[bi][bj][4 * g + e]);
          }
  }
};

// fp32 staging (pitch PF) <-> accumulators, transposed as above; load scales by s.
template <int TS, int PREC>
__device__ __forceinline__ void load_acc_t(Acc<Geo<TS, PREC>::NI, Geo<TS, PREC>::NJ> &acc, const float *st, int p0, int q0, int lane, float s) {
  using G = Geo<TS, PREC>;
  const int li = lane & 31, half = lane >> 5;
#pragma unroll
  for (int bi = 0; bi < G::NI; ++bi)
#pragma unroll
    for (int bj = 0; bj < G::NJ; ++bj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = p0 + bi * 32 + 8 * g + 4 * half;
        const int col = q0 + bj * 32 + li;
        f32x4 v = *reinterpret_cast<const f32x4 *>(st + col * G::PF + row);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc.b[bi][bj][4 * g + e] = v[e] * s;
      }
}

template <int TS, int PREC>
__device__ __forceinline__ void store_acc_t_f32(const Acc<Geo<TS, PREC>::NI, Geo<TS, PREC>::NJ> &acc, float *st, int p0, int q0, int lane) {
  using G = Geo<TS, PREC>;
  const int li = lane & 31, half = lane >> 5;
#pragma unroll
  for (int bi = 0; bi < G::NI; ++bi)
#pragma unroll
    for (int bj = 0; bj < G::NJ; ++bj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = p0 + bi * 32 + 8 * g + 4 * half;
        const int col = q0 + bj * 32 + li;
        f32x4 v = {acc.b[bi][bj][4 * g + 0], acc.b[bi][bj][4 * g + 1], acc.b[bi][bj][4 * g + 2],
                   acc.b[bi][bj][4 * g + 3]};
        *reinterpret_cast<f32x4 *>(st + col * G::PF + row) = v;
      }
}

// ------------------------------------------------------------------ global access
// 8 consecutive state elements of one row.
template <typename S>
struct Chunk8;
template <>
struct Chunk8<__bf16> {
  u32x4 v;
  __device__ __forceinline__ float get(int e) const {
    const unsigned int w = v[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Chunk8<float> {
  f32x4 a, b;
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// n (0..8) valid elements at p; the rest read as zero
template <typename S>
__device__ __forceinline__ Chunk8<S> load_chunk(const S *p, int n, bool vec) {
  Chunk8<S> c;
  if constexpr (sizeof(S) == 2) {
    if (vec && n == 8) {
      c.v = __builtin_nontemporal_load(gmem(reinterpret_cast<const u32x4 *>(p)));
    } else {
      const GLOBAL_AS unsigned short *q = gmem(reinterpret_cast<const unsigned short *>(p));
      unsigned short t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = e < n ? q[e] : 0;
      c.v = u32x4{t[0] | (unsigned)t[1] << 16, t[2] | (unsigned)t[3] << 16,
                  t[4] | (unsigned)t[5] << 16, t[6] | (unsigned)t[7] << 16};
    }
  } else {
    if (vec && n == 8) {
      c.a = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4 *>(p)));
      c.b = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4 *>(p) + 1));
    } else {
      const GLOBAL_AS float *q = gmem(p);
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = e < n ? q[e] : 0.f;
      c.a = f32x4{t[0], t[1], t[2], t[3]};
      c.b = f32x4{t[4], t[5], t[6], t[7]};
    }
  }
  return c;
}

template <typename S>
__device__ __forceinline__ Chunk8<S> load_chunk_vec(const S *p) {
  Chunk8<S> c;
  if constexpr (sizeof(S) == 2) {
    c.v = __builtin_nontemporal_load(gmem(reinterpret_cast<const u32x4 *>(p)));
  } else {
    c.a = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4 *>(p)));
    c.b = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4 *>(p) + 1));
  }
  return c;
}


__device__ __forceinline__ int clamp_n(int n, int hi) { return n < 0 ? 0 : (n > hi ? hi : n); }

// A tile descriptor unpacked into 32-bit scalars (kept in registers, passed by value).
struct TileView {
  int layer, row0, col0, h, w;
};
__device__ __forceinline__ TileView view_of(const FusedTile *tiles, int64_t i) {
  // read as four words (h and w share the last one, both non-negative)
  const int *q = reinterpret_cast<const int *>(tiles + i);
  const int hw = q[3];
  return TileView{q[0], q[1], q[2], hw & 0xffff, (int)((unsigned)hw >> 16)};
}

// A layer descriptor read field by field into scalars.
struct LayerView {
  float *w;
  void *m;
  const void *g;
  float *u;
  int64_t ld_w, ld_m, ld_g, ld_u;
  int vec_ok, vec_w;
};
__device__ __forceinline__ LayerView layer_of(const LayerDesc *layers, int i) {
  const LayerDesc *d = layers + i;
  return LayerView{d->w, d->m, d->g, d->u, d->ld_w, d->ld_m, d->ld_g, d->ld_u, d->vec_ok, d->vec_w};
}

// Per-thread share of one tile's HBM traffic: GM_IT chunks of 8 state elements of G and
// of M (momentum prologue), W_IT chunks of 4 weights (update epilogue).  Chunk q of a
// thread covers tile row q / (TS/8), columns 8 (q % (TS/8)) .. +7 (resp. 4-wide for W).
template <int TS, int NT, typename S>
struct TileRegs {
  static constexpr int CPR = TS / 8, GM_IT = TS * CPR / NT;
  static constexpr int WPR = TS / 4, W_IT = TS * WPR / NT;
  // a thread's chunks lie NT / CPR (resp. NT / WPR) rows apart in one column position,
  // so dense tiles address them from one row pointer and a uniform row stride
  static_assert(NT % CPR == 0 && NT % WPR == 0, "whole rows per pass");
  static constexpr int GM_ROWS = NT / CPR, W_ROWS = NT / WPR;
  Chunk8<S> g[GM_IT], m[GM_IT];
  f32x4 w[W_IT];

  // DENSE: the tile fills TS x TS and its rows are 16-byte aligned, so every chunk is a
  // full vector access and the code has no data-dependent branches (a branch merge
  // would make the compiler wait for the loads in flight).
  template <bool DENSE>
  __device__ __forceinline__ void load_gm(TileView t, const LayerView &L, int gt) {
    const S *mb = reinterpret_cast<const S *>(L.m);
    const S *gb = reinterpret_cast<const S *>(L.g);
    if constexpr (DENSE) {
      asm volatile("" : "+v"(gt));   // (formed per tile, as in the X0 stores)
      const int64_t r0 = t.row0 + gt / CPR;
      const int c = (gt % CPR) * 8;
      const S *gp = gb + r0 * L.ld_g + t.col0 + c;
      const S *mp = mb + r0 * L.ld_m + t.col0 + c;
      const int64_t sg = (int64_t)GM_ROWS * L.ld_g, sm = (int64_t)GM_ROWS * L.ld_m;
#pragma unroll
      for (int i = 0; i < GM_IT; ++i) {
        g[i] = load_chunk_vec<S>(gp + i * sg);
        m[i] = load_chunk_vec<S>(mp + i * sm);
      }
      return;
    }
    const bool vec = L.vec_ok && (t.col0 % 8 == 0);
#pragma unroll
    for (int i = 0; i < GM_IT; ++i) {
      const int q = gt + i * NT;
      const int r = q / CPR, c = (q % CPR) * 8;
      const int n = r < t.h ? clamp_n(t.w - c, 8) : 0;
      const int64_t gr = (int64_t)(t.row0 + r);
      g[i] = load_chunk<S>(gb + gr * L.ld_g + t.col0 + c, n, vec);
      m[i] = load_chunk<S>(mb + gr * L.ld_m + t.col0 + c, n, vec);
    }
  }

  template <bool DENSE>
  __device__ __forceinline__ void load_w(TileView t, const LayerView &L, int gt) {
    if constexpr (DENSE) {
      const float *wp = L.w + (int64_t)(t.row0 + gt / WPR) * L.ld_w + t.col0 + (gt % WPR) * 4;
      const int64_t sw = (int64_t)W_ROWS * L.ld_w;
#pragma unroll
      for (int i = 0; i < W_IT; ++i)
        w[i] = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4 *>(wp + i * sw)));
      return;
    }
    const bool vec = L.vec_w && (t.col0 % 4 == 0);
#pragma unroll
    for (int i = 0; i < W_IT; ++i) {
      const int q = gt + i * NT;
      const int r = q / WPR, c = (q % WPR) * 4;
      const int n = r < t.h ? clamp_n(t.w - c, 4) : 0;
      const float *src = L.w + (int64_t)(t.row0 + r) * L.ld_w + t.col0 + c;
      if (vec && n == 4) {
        w[i] = __builtin_nontemporal_load(gmem(reinterpret_cast<const f32x4 *>(src)));
      } else {
        const GLOBAL_AS float *q4 = gmem(src);
        float tmp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) tmp[e] = e < n ? q4[e] : 0.f;
        w[i] = f32x4{tmp[0], tmp[1], tmp[2], tmp[3]};
      }
    }
  }

  // Dense tiles: M <- beta M + G, stored, with the new values (as stored) left in v and
  // the sum of their squares (this thread's share, fixed order) returned.
  __device__ __forceinline__ float momentum_dense(TileView t, const LayerView &L, int gt, float beta,
                                                  float (&v)[GM_IT][8]) const {
    S *mb = reinterpret_cast<S *>(L.m);
    asm volatile("" : "+v"(gt));   // (formed per tile, as in the X0 stores)
    S *mp = mb + (int64_t)(t.row0 + gt / CPR) * L.ld_m + t.col0 + (gt % CPR) * 8;
    const int64_t sm = (int64_t)GM_ROWS * L.ld_m;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < GM_IT; ++i) {
      S *dst = mp + i * sm;
      if constexpr (sizeof(S) == 2) {
        unsigned code[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          code[e / 2] = pack_bf16x2(__builtin_fmaf(beta, m[i].get(e), g[i].get(e)),
                                    __builtin_fmaf(beta, m[i].get(e + 1), g[i].get(e + 1)));
          v[i][e] = __builtin_bit_cast(float, code[e / 2] << 16);
          v[i][e + 1] = __builtin_bit_cast(float, code[e / 2] & 0xffff0000u);
        }
        *gmem(reinterpret_cast<u32x4 *>(dst)) = u32x4{code[0], code[1], code[2], code[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = __builtin_fmaf(beta, m[i].get(e), g[i].get(e));
        gmem(reinterpret_cast<f32x4 *>(dst))[0] = f32x4{v[i][0], v[i][1], v[i][2], v[i][3]};
        gmem(reinterpret_cast<f32x4 *>(dst))[1] = f32x4{v[i][4], v[i][5], v[i][6], v[i][7]};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[i][e], v[i][e], ss);
    }
    return ss;
  }

  // M <- beta M + G: store the new momentum and stage its values, oriented on the
  // short side and zero padded, as fp32 TS x TS (pitch PF) in LDS.
  template <int PF, bool DENSE>
  __device__ __forceinline__ void momentum(TileView t, const LayerView &L, int gt, float beta, float *st) const {
    S *mb = reinterpret_cast<S *>(L.m);
    const bool vec = DENSE || (L.vec_ok && (t.col0 % 8 == 0));
    const bool tall = !DENSE && t.h > t.w;
#pragma unroll
    for (int i = 0; i < GM_IT; ++i) {
      const int q = gt + i * NT;
      const int r = q / CPR, c = (q % CPR) * 8;
      const int n = DENSE ? 8 : (r < t.h ? clamp_n(t.w - c, 8) : 0);
      S *dst = mb + (int64_t)(t.row0 + r) * L.ld_m + t.col0 + c;
      float v[8];
      if constexpr (sizeof(S) == 2) {
        unsigned short code[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          code[e] = to_bf16_bits(__builtin_fmaf(beta, m[i].get(e), g[i].get(e)));
          v[e] = __builtin_bit_cast(float, (unsigned)code[e] << 16);
        }
        if (vec && n == 8) {
          *gmem(reinterpret_cast<u32x4 *>(dst)) =
              u32x4{code[0] | (unsigned)code[1] << 16, code[2] | (unsigned)code[3] << 16,
                    code[4] | (unsigned)code[5] << 16, code[6] | (unsigned)code[7] << 16};
        } else {
          GLOBAL_AS unsigned short *d16 = gmem(reinterpret_cast<unsigned short *>(dst));
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < n) d16[e] = code[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(beta, m[i].get(e), g[i].get(e));
        if (vec && n == 8) {
          gmem(reinterpret_cast<f32x4 *>(dst))[0] = f32x4{v[0], v[1], v[2], v[3]};
          gmem(reinterpret_cast<f32x4 *>(dst))[1] = f32x4{v[4], v[5], v[6], v[7]};
        } else {
          GLOBAL_AS float *d32 = gmem(dst);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < n) d32[e] = v[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e >= n) v[e] = 0.f;  // zero padding
      if (!tall) {
        *reinterpret_cast<f32x4 *>(st + r * PF + c) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(st + r * PF + c + 4) = f32x4{v[4], v[5], v[6], v[7]};
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) st[(c + e) * PF + r] = v[e];
      }
    }
  }

  // W <- W - lr O (and U <- O) from the staged fp32 output tile, O = oscale * staged.
  template <int PF, bool DENSE>
  __device__ __forceinline__ void update(TileView t, const LayerView &L, int gt, float lr, bool write_u,
                         const float *st, float oscale = 1.f) const {
    const bool vec = DENSE || (L.vec_w && (t.col0 % 4 == 0));
    const bool tall = !DENSE && t.h > t.w;
    const float nlr = -lr;
#pragma unroll
    for (int i = 0; i < W_IT; ++i) {
      const int q = gt + i * NT;
      const int r = q / WPR, c = (q % WPR) * 4;
      const int n = DENSE ? 4 : (r < t.h ? clamp_n(t.w - c, 4) : 0);
      if (n == 0) continue;
      float o[4];
      if (!tall) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(st + r * PF + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[e] * oscale;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st[(c + e) * PF + r] * oscale;
      }
      float nw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) nw[e] = __builtin_fmaf(nlr, o[e], w[i][e]);
      // (dense tiles: one row pointer and a uniform stride, as in load_w)
      GLOBAL_AS float *dst =
          DENSE ? gmem(L.w + (int64_t)(t.row0 + gt / WPR) * L.ld_w + t.col0 + (gt % WPR) * 4 +
                       i * ((int64_t)W_ROWS * L.ld_w))
                : gmem(L.w + (int64_t)(t.row0 + r) * L.ld_w + t.col0 + c);
      if (vec && n == 4) {
        *reinterpret_cast<GLOBAL_AS f32x4 *>(dst) = f32x4{nw[0], nw[1], nw[2], nw[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < n) dst[e] = nw[e];
      }
      if (write_u) {
        GLOBAL_AS float *ud =
            DENSE ? gmem(L.u + (int64_t)(t.row0 + gt / WPR) * L.ld_u + t.col0 + (gt % WPR) * 4 +
                         i * ((int64_t)W_ROWS * L.ld_u))
                  : gmem(L.u + (int64_t)(t.row0 + r) * L.ld_u + t.col0 + c);
        if (vec && n == 4) {
          *reinterpret_cast<GLOBAL_AS f32x4 *>(ud) = f32x4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < n) ud[e] = o[e];
        }
      }
    }
  }
};

// ------------------------------------------------------------------ the kernel
// Persistent: each tile group of a workgroup walks tiles tix, tix + stride, ...  While
// tile i iterates, the loads of tile i+1's G and M are in flight (bf16 state), so their
// HBM latency hides behind the MFMA work.  NS false: the instance for K = 0 (and the
// identity test mode), with no Newton-Schulz code: W's loads go out early without their
// registers being held across an iteration, and with a quarter of the LDS and at most
// 128 registers (dense tiles) twice as many tile groups stay resident per CU.
template <int TS, int PREC, typename S, bool DENSE, bool NS>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Geo<TS, PREC>::THREADS)))
__attribute__((amdgpu_waves_per_eu(NS || !DENSE ? 2 : 4, NS || !DENSE ? 2 : 4)))
void fused_step_kernel(const LayerDesc *__restrict__ layers, const FusedTile *__restrict__ tiles,
                       int64_t ntiles, NSParams prm) {
  using G = Geo<TS, PREC>;
  constexpr int NT = G::NT, NI = G::NI, NJ = G::NJ, PF = G::PF;
  constexpr bool PREFETCH = sizeof(S) == 2;
  constexpr int AREA = NS ? G::TILE_LDS : G::K0_LDS;   // LDS bytes per tile group
  __shared__ __attribute__((aligned(16))) char lds[G::TPB * AREA];

  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / NT);  // tile slot in the workgroup
  const int gt = threadIdx.x % NT;                                     // thread within the tile group
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(gt >> 6);             // wave within the tile group
  const int64_t stride = (int64_t)gridDim.x * G::TPB;
  int64_t tix = (int64_t)blockIdx.x * G::TPB + grp;
  if (tix >= ntiles) return;                                           // uniform per tile group

  char *area = lds + grp * AREA;
  float *st = reinterpret_cast<float *>(area);          // fp32 staging, TS x PF
  const Mat<PREC> X = make_mat<TS, PREC>(area);
  const Mat<PREC> AB = make_mat<TS, PREC>(area + G::REGION);
  __bf16 *const xlo = reinterpret_cast<__bf16 *>(area + 2 * G::REGION);   // G::XLO bytes
  float *const red = reinterpret_cast<float *>(area + (NS ? G::RED_OFF : G::K0_RED_OFF));   // G::WPT floats
  const int p0 = (wv / (TS / G::WBN)) * G::WBM;          // wave block origin (rows)
  const int q0 = (wv % (TS / G::WBN)) * G::WBN;          //                   (columns)
  const float ca = prm.a, cb = prm.b, cc = prm.c;
  const int fx0 = PREC == PREC_BF16F8 ? (int)prm.f8.x[0] : 0;   // exponent of X_0's e4m3 planes

  TileRegs<TS, NT, S> io;
  TileView t = view_of(tiles, tix);
  LayerView L = layer_of(layers, t.layer);
  io.template load_gm<DENSE>(t, L, gt);

  while (true) {
    // ---- momentum, Frobenius norm, X0 -------------------------------------------
    // DIRECT (dense tiles, a folded into B): each thread keeps its new momentum values in
    // registers, the norm comes from their squares, and X0 = M / (|M| + eps) is written
    // to the LDS copy of X straight from them.  Otherwise the tile is staged in fp32,
    // oriented on its short side and zero padded, and X0 formed from the staging copy.
    // (The summation order is fixed either way.)
    // (PREC_BF16F8 64-tiles keep X in fp32 registers from X0 on, so they stage it)
    // (the instance without NS steps always stages: the staged momentum is its output, O =
    // inv * M, scaled in the weight update)
    constexpr bool DIRECT = NS && DENSE && PREC != PREC_BF16 && !(PREC == PREC_BF16F8 && G::XLO == 0);
    float vd[DIRECT ? TileRegs<TS, NT, S>::GM_IT : 1][8];
    float ss = 0.f;
    if constexpr (DIRECT) {
      ss = io.momentum_dense(t, L, gt, prm.beta, vd);
    } else {
      io.template momentum<PF, DENSE>(t, L, gt, prm.beta, st);
    }
    // Without NS steps (K = 0, and the identity test mode) W's loads go out now, ahead of
    // the next tile's prefetch, so their latency passes during the staging below; with
    // NS steps they go out at the end (their registers are busy meanwhile).
    if constexpr (!NS) io.template load_w<DENSE>(t, L, gt);
    const int64_t nxt = tix + stride;
    TileView tn = t;
    LayerView Ln = L;
    if constexpr (PREFETCH) {
      if (nxt < ntiles) {
        tn = view_of(tiles, nxt);
        Ln = layer_of(layers, tn.layer);
        io.template load_gm<DENSE>(tn, Ln, gt);
      }
    }
    if constexpr (!DIRECT) tile_sync<G::WPT>();   // the staging copy is complete
    float inv = 1.0f;
    if (!prm.identity) {   // (uniform) the identity test mode takes no norm
      if constexpr (!DIRECT) {
        constexpr int C4 = TS * TS / 4;
#pragma unroll 4
        for (int q = gt; q < C4; q += NT) {
          const int r = q / (TS / 4), c = (q % (TS / 4)) * 4;
          const f32x4 v = *reinterpret_cast<const f32x4 *>(st + r * PF + c);
          ss = __builtin_fmaf(v[0], v[0], ss);
          ss = __builtin_fmaf(v[1], v[1], ss);
          ss = __builtin_fmaf(v[2], v[2], ss);
          ss = __builtin_fmaf(v[3], v[3], ss);
        }
      }
      ss = tile_sum<G::WPT>(ss, red, lane, wv);
      // Outside [2^-100, 2^100] (a zero tile, entries beyond about 1e15 or below 1e-17 on
      // a full tile, an overflow) the fp32 sum of squares is recomputed from the values
      // scaled by the power of two s = s1 s2 that brings the largest magnitude into
      // [1/2, 1): X0 = (s Y) / (s |Y| + s eps) is the same map, and no square overflows
      // or falls below the normal range.  The scaled values replace the unscaled ones
      // (in registers, or in the staging copy), so X0 below takes them as they are.
      float es1 = 1.f, es2 = 1.f;   // s = es1 es2 for the eps term
      if (!(ss >= 0x1p-100f && ss <= 0x1p100f)) {   // (uniform over the tile)
        float mx = 0.f;
        if constexpr (DIRECT) {
#pragma unroll
          for (int i = 0; i < TileRegs<TS, NT, S>::GM_IT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(vd[i][e]));
        } else {
#pragma unroll 1
          for (int q = gt; q < TS * TS / 4; q += NT) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(st + (q / (TS / 4)) * PF + (q % (TS / 4)) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[e]));
          }
        }
        tile_sync<G::WPT>();   // every wave has read the partial sums
        mx = tile_max<G::WPT>(mx, red, lane, wv);
        if (mx > 0.f && mx <= 0x1.fffffep127f) {   // (uniform) nonzero and finite
          int ex;
          (void)__builtin_frexpf(mx, &ex);
          const float s1 = __builtin_ldexpf(1.f, (-ex) / 2), s2 = __builtin_ldexpf(1.f, -ex - (-ex) / 2);
          float s2s = 0.f;
          if constexpr (DIRECT) {
#pragma unroll
            for (int i = 0; i < TileRegs<TS, NT, S>::GM_IT; ++i)
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                vd[i][e] = vd[i][e] * s1 * s2;
                s2s = __builtin_fmaf(vd[i][e], vd[i][e], s2s);
              }
          } else {
#pragma unroll 1
            for (int q = gt; q < TS * TS / 4; q += NT) {
              f32x4 *pv = reinterpret_cast<f32x4 *>(st + (q / (TS / 4)) * PF + (q % (TS / 4)) * 4);
              f32x4 v = *pv;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v[e] = v[e] * s1 * s2;
                s2s = __builtin_fmaf(v[e], v[e], s2s);
              }
              *pv = v;
            }
          }
          tile_sync<G::WPT>();   // every wave has read the maximum (and the staging copy is rescaled)
          ss = tile_sum<G::WPT>(s2s, red, lane, wv);
          es1 = s1;
          es2 = s2;
        }
      }
      // a zero tile stays zero, also with eps = 0 (divisor 0); (eps s1) s2 may round to
      // infinity for a tile far below eps, whose X0 is then 0 (its true size is below
      // the fp32 range)
      const float den = __builtin_sqrtf(ss) + (prm.eps * es1) * es2;
      inv = den > 0.f ? 1.0f / den : (den == 0.f ? 0.f : den);   // a NaN (from NaN entries) passes on
    }

    // X in registers (fp32, MFMA output layout of the update product: block holds X^T)
    Acc<NI, NJ> xr;
    if constexpr (DIRECT) {
      constexpr int CPR = TS / 8;
      // (the thread index is made opaque so that these LDS offsets are formed here for
      // each tile rather than once per launch and held, or spilled, across the tile loop)
      int gq = gt;
      asm volatile("" : "+v"(gq));
#pragma unroll
      for (int i = 0; i < TileRegs<TS, NT, S>::GM_IT; ++i) {
        const int q = gq + i * NT;
        const int r = q / CPR, c = (q % CPR) * 8;
        if constexpr (!NS) {
          // no iteration: the output is X0 itself, staged for the update in fp32
#pragma unroll
          for (int e = 0; e < 8; ++e) st[r * PF + c + e] = vd[i][e] * inv;
        } else if constexpr (PREC == PREC_F32) {
          f32x4 a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = vd[i][e] * inv;
            b[e] = vd[i][e + 4] * inv;
          }
          *reinterpret_cast<f32x4 *>(X.f + r * PF + c) = a;
          *reinterpret_cast<f32x4 *>(X.f + r * PF + c + 4) = b;
        } else if constexpr (PREC == PREC_BF16F8) {
          const F8S f8 = f8s_of(fx0);
          u32x4 hi;
          float xv[8], rv[8];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            xv[e] = vd[i][e] * inv;
            xv[e + 1] = vd[i][e + 1] * inv;
            hi[e / 2] = pack_bf16x2(xv[e], xv[e + 1]);
            rv[e] = __builtin_fmaf(vd[i][e], inv, -__builtin_bit_cast(float, hi[e / 2] << 16));
            rv[e + 1] = __builtin_fmaf(vd[i][e + 1], inv, -__builtin_bit_cast(float, hi[e / 2] & 0xffff0000u));
          }
          *reinterpret_cast<u32x4 *>(X.hi + G::bidx(r, c)) = hi;
          // (dense tiles are full: with the Gram and the update of step 0 plain, nothing
          // reads X_0's e4m3 planes)
          if constexpr (kF8PlainGramSteps < 1 || f8_plain_update_steps(TS, DENSE) < 1) {
            const int o8 = G::b8idx(r, c);
            *reinterpret_cast<u32x2 *>(X.h8 + o8) = u32x2{pack_fp8x4(xv[0], xv[1], xv[2], xv[3], f8.h),
                                                          pack_fp8x4(xv[4], xv[5], xv[6], xv[7], f8.h)};
            *reinterpret_cast<u32x2 *>(X.l8 + o8) = u32x2{pack_fp8x4(rv[0], rv[1], rv[2], rv[3], f8.l),
                                                          pack_fp8x4(rv[4], rv[5], rv[6], rv[7], f8.l)};
          }
          if constexpr (G::XLO > 0)
            *reinterpret_cast<u32x4 *>(xlo + G::bidx(r, c)) =
                u32x4{pack_bf16x2(rv[0], rv[1]), pack_bf16x2(rv[2], rv[3]), pack_bf16x2(rv[4], rv[5]),
                      pack_bf16x2(rv[6], rv[7])};
        } else {
          u32x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float x0 = vd[i][e] * inv, x1 = vd[i][e + 1] * inv;
            hi[e / 2] = pack_bf16x2(x0, x1);
            lo[e / 2] = pack_bf16x2(__builtin_fmaf(vd[i][e], inv, -__builtin_bit_cast(float, hi[e / 2] << 16)),
                                    __builtin_fmaf(vd[i][e + 1], inv, -__builtin_bit_cast(float, hi[e / 2] & 0xffff0000u)));
          }
          const int o = G::bidx(r, c);
          *reinterpret_cast<u32x4 *>(X.hi + o) = hi;
          *reinterpret_cast<u32x4 *>(X.lo + o) = lo;
        }
      }
      tile_sync<G::WPT>();
    } else {
      if constexpr (NS) {
        load_acc_t<TS, PREC>(xr, st, p0, q0, lane, inv);
        tile_sync<G::WPT>();
        constexpr bool PLAIN_X0 = PREC == PREC_BF16F8 && G::XLO == 0 && kF8PlainGramSteps >= 1 &&
                                  f8_plain_update_steps(TS, DENSE) >= 1;
        bool plain_x0 = false;
        if constexpr (PLAIN_X0) {
          plain_x0 = DENSE || (t.h == TS && t.w == TS);   // (wave-uniform) step 0 reads hi alone
          if (plain_x0) store_acc_t<TS, PREC_BF16>(xr, Mat<PREC_BF16>{X.hi}, p0, q0, lane);
        }
        if (!plain_x0)
          store_acc_t<TS, PREC, false, false, NI, false, (G::XLO > 0)>(xr, X, p0, q0, lane, 1.f, 1.f,
                                                                        f8s_of(fx0), xlo);
        tile_sync<G::WPT>();
      }
    }

    // ---- K Newton-Schulz steps ------------------------------------------------
    // FOLD_A (fp32 and bf16x3): X <- (a I + B) X with a folded into B's diagonal; the
    // LDS copy of X (fp32, or hi + lo bf16) carries X between steps.  Plain bf16 keeps
    // X in fp32 registers and forms a X there, since its LDS copy is bf16-rounded;
    // bf16f8 (its own loop below) forms a X in fp32 as well.
    constexpr bool FOLD_A = PREC != PREC_BF16;
    // Dense tiles issue the loads of W before the last update product, so that their
    // HBM latency passes while it runs (the other variants, and PREC_BF16F8 with its
    // larger operand fragments, lack the registers).
    constexpr bool EARLY_W = DENSE && (PREC != PREC_BF16F8 || TS < 128);
    const SymJob jb = sym_job<TS>(wv);
    // e4m3 plane exponents of the current step (PREC_BF16F8); a product's scale byte
    // 127 - (eL + eR + 8) undoes its operands' exponents
    constexpr bool F8 = PREC == PREC_BF16F8;
    F8Steps<F8> fs;
    if constexpr (F8) fs.init(prm.f8);
    // The symmetric part of a step, on the wave's job: B (with a on its diagonal when
    // folded) ends up in AB.
    // On full TS x TS tiles PREC_BF16F8 runs the first steps partly in plain bf16 (hi
    // operands only): the Gram product of step 0, and the square product of steps 0 and 1
    // with A stored as its hi plane alone.  While the singular values of X are still
    // small the A^2 term is small against a I + b A, and the rounding error of an r x r
    // Gram matrix is spread over r directions, so these roundings cost no accuracy at
    // r = 64 or 128; once the singular values saturate (from step 2 on), and on thin
    // ragged tiles (few large singular values), every product takes the correction terms.
    // (128-tiles outside the dense group keep the square product split: their instance
    // has no registers to spare for the plain variant, and a spill there slows the
    // whole tile loop)
    constexpr int PLAIN_GRAM_STEPS = f8_plain_gram_steps(TS, DENSE), PLAIN_SQUARE_STEPS = f8_plain_square_steps(TS, DENSE);
    constexpr int PLAIN_UPDATE_STEPS = f8_plain_update_steps(TS, DENSE);
    const bool full = DENSE || (t.h == TS && t.w == TS);         // wave-uniform
    auto sym_part = [&](int it) {
      const int ex = fs.x(), ea = fs.a(), eb = fs.b();
      const bool pg = F8 && full && it < PLAIN_GRAM_STEPS;      // wave-uniform
      const bool pa = F8 && full && it < PLAIN_SQUARE_STEPS && cc != 0.f;
      // B stored as its hi plane alone (the last step keeps the split update)
      const bool pu = F8 && full && it < PLAIN_UPDATE_STEPS && it + 1 < prm.steps;
      Acc<NI, NJ> acc;
      with_job<TS>(jb, [&](auto NBC, auto ALC) {
        constexpr int NB = decltype(NBC)::value;
        constexpr bool AL = decltype(ALC)::value;
        if constexpr (F8) {
          const Mat<PREC_BF16> Xh{X.hi}, ABh{AB.hi};
          if (pg) {
            wave_gemm_std<TS, PREC_BF16, false, true, NB, AL>(acc, Xh, jb.p0, Xh, jb.q0, lane);   // A = X X^T
          } else {
            wave_gemm<TS, PREC, false, true, NB, AL>(acc, X, jb.p0, X, jb.q0, lane, 127 - (2 * ex + 8));
          }
          if (cc == 0.f && pu) {
            store_acc_t<TS, PREC_BF16, true, false, NB, true>(acc, ABh, jb.p0, jb.q0, lane, cb);   // B = b A
          } else if (cc == 0.f) {
            store_acc_t<TS, PREC, true, false, NB, true>(acc, AB, jb.p0, jb.q0, lane, cb, 1.f, f8s_of(eb));   // B = b A
          } else if (pa) {
            store_acc_t<TS, PREC_BF16, false, true, NB, true>(acc, ABh, jb.p0, jb.q0, lane, 1.f, cb / cc);
          } else {
            store_acc_t<TS, PREC, false, true, NB, true>(acc, AB, jb.p0, jb.q0, lane, 1.f, cb / cc, f8s_of(ea));
          }
        } else {
          wave_gemm<TS, PREC, false, true, NB, AL>(acc, X, jb.p0, X, jb.q0, lane);   // A = X X^T
          if (cc != 0.f) {
            // B = b A + c A^2 = c ((b/c) A + A A^T): accumulate A A^T onto (b/c) A
            store_acc_t<TS, PREC, false, true, NB, true>(acc, AB, jb.p0, jb.q0, lane, 1.f, cb / cc);
          } else {
            store_acc_t<TS, PREC, true, false, NB, true>(acc, AB, jb.p0, jb.q0, lane, cb);   // B = b A
            if constexpr (FOLD_A) add_diag<TS, PREC, NB>(AB, jb.p0, jb.q0, lane, ca);       // B + a I
          }
        }
      });
      if (cc != 0.f) {
        tile_sync<G::WPT>();
        with_job<TS>(jb, [&](auto NBC, auto ALC) {
          constexpr int NB = decltype(NBC)::value;
          constexpr bool AL = decltype(ALC)::value;
          if constexpr (F8) {
            const Mat<PREC_BF16> ABh{AB.hi};
            if (pa) {
              wave_gemm_std<TS, PREC_BF16, false, false, NB, AL>(acc, ABh, jb.p0, ABh, jb.q0, lane);
            } else {
              wave_gemm<TS, PREC, false, false, NB, AL>(acc, AB, jb.p0, AB, jb.q0, lane, 127 - (2 * ea + 8));
            }
          } else {
            wave_gemm<TS, PREC, false, false, NB, AL>(acc, AB, jb.p0, AB, jb.q0, lane);
          }
        });
        tile_sync<G::WPT>();                                             // A fully read
        with_job<TS>(jb, [&](auto NBC, auto) {
          constexpr int NB = decltype(NBC)::value;
          if constexpr (F8) {
            if (pu) {
              store_acc_t<TS, PREC_BF16, true, false, NB, true>(acc, Mat<PREC_BF16>{AB.hi}, jb.p0, jb.q0, lane, cc);
            } else {
              store_acc_t<TS, PREC, true, false, NB, true>(acc, AB, jb.p0, jb.q0, lane, cc, 1.f, f8s_of(eb));   // B
            }
          } else {
            store_acc_t<TS, PREC, true, false, NB, true>(acc, AB, jb.p0, jb.q0, lane, cc);   // B
            if constexpr (FOLD_A) add_diag<TS, PREC, NB>(AB, jb.p0, jb.q0, lane, ca);       // B + a I
          }
        });
      }
    };
    if constexpr (!NS) {
      // no Newton-Schulz steps
    } else if constexpr (F8) {
      for (int it = 0; it < prm.steps; ++it) {
        sym_part(it);
        const int sxb = 127 - (fs.x() + fs.b() + 8);
        // The a X term in fp32, from X accurate to about 2^-17: X itself, in registers since
        // the last update (64-tiles), or the hi and lo planes of this wave's own block,
        // added after the product (128-tiles).  Rounding noise in the a X term would grow
        // by a factor of about a per step in the empty directions of a low-rank tile; in
        // B X it does not.
        constexpr bool XREG = G::XLO == 0;
        if constexpr (XREG) {
#pragma unroll
          for (int bi = 0; bi < NI; ++bi)
#pragma unroll
            for (int bj = 0; bj < NJ; ++bj)
#pragma unroll
              for (int e = 0; e < 16; ++e) xr.b[bi][bj][e] *= ca;
        }
        tile_sync<G::WPT>();
        if (it + 1 == prm.steps) {
          if constexpr (EARLY_W) io.template load_w<DENSE>(t, L, gt);
          wave_gemm<TS, PREC, true, !XREG>(xr, X, p0, AB, q0, lane, sxb);   // X^T <- a X^T + X^T B
          if constexpr (!XREG) {
            XPiece<TS> xp;
            xp.load(X.hi, xlo, p0, q0, lane);
            tile_sync<G::WPT>();
            xp.add_to(xr, ca);
          } else {
            tile_sync<G::WPT>();
          }
          break;
        }
        // X^T <- a X^T + X^T B; in the first steps of a full tile on the hi planes alone
        if (PLAIN_UPDATE_STEPS > 0 && full && it < PLAIN_UPDATE_STEPS) {
          // (an opaque lane index, so that this product's LDS addresses are formed here
          // rather than hoisted out of the loop and held across it)
          int ln = lane;
          asm volatile("" : "+v"(ln));
          wave_gemm_std<TS, PREC_BF16, true, !XREG, NI, false>(xr, Mat<PREC_BF16>{X.hi}, p0,
                                                               Mat<PREC_BF16>{AB.hi}, q0, ln);
        } else {
          wave_gemm<TS, PREC, true, !XREG>(xr, X, p0, AB, q0, lane, sxb);
        }
        if constexpr (!XREG) {
          XPiece<TS> xp;
          xp.load(X.hi, xlo, p0, q0, lane);
          tile_sync<G::WPT>();
          xp.add_to(xr, ca);
        } else {
          tile_sync<G::WPT>();
        }
        // X_{it+1}: without its e4m3 planes when the next step's Gram and update both read
        // hi alone (hi + lo is the bf16x3 layout, lo where the a X term reads it)
        bool plain_x = false;
        if constexpr (G::XLO > 0 && PLAIN_GRAM_STEPS > 1 && PLAIN_UPDATE_STEPS > 1) {
          plain_x = full && it + 1 < PLAIN_GRAM_STEPS && it + 1 < PLAIN_UPDATE_STEPS && it + 2 < prm.steps;
          if (plain_x) store_acc_t<TS, PREC_BF16X3>(xr, Mat<PREC_BF16X3>{X.hi, xlo}, p0, q0, lane);
        }
        if (!plain_x)
          store_acc_t<TS, PREC, false, false, NI, false, (G::XLO > 0)>(xr, X, p0, q0, lane, 1.f, 1.f,
                                                                        f8s_of(fs.xn()), xlo);
        tile_sync<G::WPT>();
        fs.advance();
      }
    } else if (prm.steps > 0) {
      for (int it = 0;; ++it) {
        sym_part(it);
        if constexpr (!FOLD_A) {
#pragma unroll
          for (int bi = 0; bi < NI; ++bi)
#pragma unroll
            for (int bj = 0; bj < NJ; ++bj)
#pragma unroll
              for (int e = 0; e < 16; ++e) xr.b[bi][bj][e] *= ca;
        }
        tile_sync<G::WPT>();
        if (it + 1 == prm.steps) {
          if constexpr (EARLY_W) io.template load_w<DENSE>(t, L, gt);
          wave_gemm<TS, PREC, true, FOLD_A>(xr, X, p0, AB, q0, lane);   // X^T <- X^T (aI + B)
          tile_sync<G::WPT>();
          break;
        }
        wave_gemm<TS, PREC, true, FOLD_A>(xr, X, p0, AB, q0, lane);     // X^T <- X^T (aI + B)
        tile_sync<G::WPT>();
        store_acc_t<TS, PREC>(xr, X, p0, q0, lane);
        tile_sync<G::WPT>();
      }
    }
    if constexpr (NS && !EARLY_W) io.template load_w<DENSE>(t, L, gt);

    // ---- reassembly and weight update ------------------------------------------
    if constexpr (NS) {
      tile_sync<G::WPT>();
      store_acc_t_f32<TS, PREC>(xr, st, p0, q0, lane);
    }
    tile_sync<G::WPT>();
    io.template update<PF, DENSE>(t, L, gt, prm.lr, prm.write_update != 0, st, NS ? 1.f : inv);
    if (nxt >= ntiles) break;
    tile_sync<G::WPT>();                 // staging fully read before the next tile lands
    tix = nxt;
    if constexpr (PREFETCH) {
      t = tn;
      L = Ln;
    } else {
      t = view_of(tiles, tix);
      L = layer_of(layers, t.layer);
      io.template load_gm<DENSE>(t, L, gt);
    }
  }
}

// Workgroups per CU the fused kernel can keep resident, and CUs of the current device.
template <class F>
int resident_groups(F kernel, int threads) {
  static thread_local int cached_dev = -1;
  static thread_local int cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached_dev = dev;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

template <int TS, int PREC, typename S, bool DENSE, bool NS = true>
hipError_t launch_one(const LayerDesc *layers, const FusedTile *tiles, int64_t n,
                      const NSParams &p, hipStream_t stream) {
  using G = Geo<TS, PREC>;
  auto kern = fused_step_kernel<TS, PREC, S, DENSE, NS>;
  int64_t blocks = (n + G::TPB - 1) / G::TPB;
  const int resident = resident_groups(kern, G::THREADS);
  if (resident <= 0) return hipErrorInvalidDevice;
  if (blocks > resident) blocks = resident;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(G::THREADS), 0, stream, layers, tiles, n, p);
  return hipGetLastError();
}

template <int TS, int PREC, bool NS = true>
hipError_t launch_state(int state_bf16, bool dense, const LayerDesc *layers, const FusedTile *tiles,
                        int64_t n, const NSParams &p, hipStream_t stream) {
  if (state_bf16)
    return dense ? launch_one<TS, PREC, __bf16, true, NS>(layers, tiles, n, p, stream)
                 : launch_one<TS, PREC, __bf16, false, NS>(layers, tiles, n, p, stream);
  return dense ? launch_one<TS, PREC, float, true, NS>(layers, tiles, n, p, stream)
               : launch_one<TS, PREC, float, false, NS>(layers, tiles, n, p, stream);
}

template <int TS>
hipError_t launch_prec(int prec, int state_bf16, bool dense, const LayerDesc *layers,
                       const FusedTile *tiles, int64_t n, const NSParams &p, hipStream_t stream) {
  // without NS steps no product runs, so the arithmetic scheme does not matter: one
  // instance (fp32 staging) serves them all
  if (p.steps == 0) return launch_state<TS, PREC_F32, false>(state_bf16, dense, layers, tiles, n, p, stream);
  switch (prec) {
    case PREC_F32: return launch_state<TS, PREC_F32>(state_bf16, dense, layers, tiles, n, p, stream);
    case PREC_BF16: return launch_state<TS, PREC_BF16>(state_bf16, dense, layers, tiles, n, p, stream);
    case PREC_BF16X3: return launch_state<TS, PREC_BF16X3>(state_bf16, dense, layers, tiles, n, p, stream);
    case PREC_BF16F8:
      if constexpr (TS >= 64) {
        return launch_state<TS, PREC_BF16F8>(state_bf16, dense, layers, tiles, n, p, stream);
      } else {
        return hipErrorInvalidValue;   // the caller runs these tiles with PREC_BF16X3
      }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fused(int ts, int prec, int state_bf16, bool dense, const LayerDesc *layers,
                        const FusedTile *tiles, int64_t n, const NSParams &p, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  switch (ts) {
    case 32: return launch_prec<32>(prec, state_bf16, dense, layers, tiles, n, p, stream);
    case 64: return launch_prec<64>(prec, state_bf16, dense, layers, tiles, n, p, stream);
    case 128: return launch_prec<128>(prec, state_bf16, dense, layers, tiles, n, p, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t fused_lds_bytes(int ts, int prec) {
  auto f = [&](auto tsc) -> size_t {
    constexpr int TS = decltype(tsc)::value;
    switch (prec) {
      case PREC_F32: return Geo<TS, PREC_F32>::TPB * Geo<TS, PREC_F32>::TILE_LDS;
      case PREC_BF16: return Geo<TS, PREC_BF16>::TPB * Geo<TS, PREC_BF16>::TILE_LDS;
      case PREC_BF16F8:
        if constexpr (TS >= 64) return Geo<TS, PREC_BF16F8>::TPB * Geo<TS, PREC_BF16F8>::TILE_LDS;
        [[fallthrough]];
      default: return Geo<TS, PREC_BF16X3>::TPB * Geo<TS, PREC_BF16X3>::TILE_LDS;
    }
  };
  switch (ts) {
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    default: return 0;
  }
}

}  // namespace himuon

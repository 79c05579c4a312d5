// Host planner of the HiMuon step (see plan.h).
//
// The partition follows "Hierarchical Muon: Tiled Newton-Schulz Updates for
// Efficient Muon Optimization" (Abstract): each matrix is cut into T x T tiles;
// here the grid is anchored at (0, 0), tiles are listed row-major, layer after
// layer, and the last tile row / column keeps its ragged size.  T = 0 (FULL) or
// T >= max(H, W) gives one tile per matrix.  Tiles whose longer side is at most
// 128 run in the fused kernel (edge 32, 64 or 128, zero padded); larger tiles
// take the GEMM path, whose workspace is cut into chunks under the budget
// (memory-bounded chunking, same page).
#include "plan.h"

#include <cmath>
#include <cstdint>
#include <sstream>

namespace himuon {

namespace {
constexpr int64_t kMaxDim = (int64_t)1 << 30;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool finite(double v) { return std::isfinite(v); }
}  // namespace

int fused_edge_for(int64_t e) {
  if (e <= 0) return 0;
  if (e <= 32) return 32;
  if (e <= 64) return 64;
  if (e <= 128) return 128;
  return 0;
}

namespace {
int64_t roundup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

// byte sizes of the planes of one GEMM tile (4 bytes per element in every precision:
// one fp32 plane, or bf16 hi and lo planes)
struct GemmSizes {
  int64_t r, s, ldx, lda, nred;
  size_t x, ab, red;
};
GemmSizes gemm_sizes(int64_t h, int64_t w) {
  GemmSizes z;
  z.r = std::min(h, w);
  z.s = std::max(h, w);
  z.ldx = roundup(z.s, 64);   // whole K slices of the GEMM kernels
  z.lda = roundup(z.r, 64);
  z.nred = cdiv(h * w, kGemmMomentumBlock);
  z.x = align256((size_t)z.r * z.ldx * 4);
  z.ab = align256((size_t)z.r * z.lda * 4);
  z.red = align256((size_t)(z.nred + 1) * 4);
  return z;
}

// Product kernel of a large-path tile (bf16 planes, every precision except fp32):
// 1: exactly 256 x 256, one workgroup per tile and product; 2: both sides multiples of
// 256 (so ldx = s and lda = r), 256-blocks; 0: 128-blocks.  Chunks hold one kind.
int gemm_kind(const GemmTile &g, int prec) {
  if (prec == HIMUON_PREC_F32) return 0;
  if (g.r == 256 && g.s == 256) return 1;
  return g.r % 256 == 0 && g.s % 256 == 0 ? 2 : 0;
}

// Workspace of one tile of the given kind: 256 x 256 tiles run their NS steps in place
// (one X and one A/B buffer), the others alternate two X buffers and keep A and B apart.
size_t tile_workspace(const GemmTile &g, int prec) {
  const GemmSizes z = gemm_sizes(g.h, g.w);
  return gemm_kind(g, prec) == 1 ? z.x + z.ab + z.red : 2 * z.x + 2 * z.ab + z.red;
}
}  // namespace


himuon_status plan_init(Plan &p, const himuon_layer *layers, int32_t n, const himuon_config *cfg,
                        std::string &err) {
  std::ostringstream m;
  if (!cfg) {
    err = "config is NULL";
    return HIMUON_EINVAL;
  }
  if (n < 0 || (n > 0 && !layers)) {
    err = "layer list is NULL or n_layers < 0";
    return HIMUON_EINVAL;
  }
  const himuon_config &c = *cfg;
  if (c.tile < 0) {
    err = "tile must be >= 1 or HIMUON_TILE_FULL (0)";
    return HIMUON_EINVAL;
  }
  if (c.steps < 0 || c.steps > 10000) {
    err = "steps must be in [0, 10000]";
    return HIMUON_EINVAL;
  }
  if (!finite(c.coeffs.a) || !finite(c.coeffs.b) || !finite(c.coeffs.c) || !std::isfinite(c.beta) ||
      !std::isfinite(c.eps) || c.eps < 0) {
    err = "coefficients, beta and eps must be finite (eps >= 0)";
    return HIMUON_EINVAL;
  }
  {
    // The kernels take the coefficients in fp32, and with c != 0 form B = c ((b / c) A +
    // A^2) (the square accumulated onto (b / c) A, whose entries are at most 1 in
    // magnitude): the fp32 values must be finite, a nonzero c must stay nonzero, and
    // b / c must stay far from the fp32 range so that the accumulators cannot overflow.
    const float fa = (float)c.coeffs.a, fb = (float)c.coeffs.b, fc = (float)c.coeffs.c;
    if (!std::isfinite(fa) || !std::isfinite(fb) || !std::isfinite(fc) || (c.coeffs.c != 0.0 && fc == 0.f) ||
        (fc != 0.f && !(std::fabs(fb / fc) <= 0x1p100f))) {
      err = "coefficients must be finite in fp32, a nonzero c must be representable, and |b / c| <= 2^100";
      return HIMUON_EINVAL;
    }
  }
  if (c.state_dtype != HIMUON_F32 && c.state_dtype != HIMUON_BF16) {
    err = "state_dtype must be HIMUON_F32 or HIMUON_BF16";
    return HIMUON_EINVAL;
  }
  if (c.precision != HIMUON_PREC_F32 && c.precision != HIMUON_PREC_BF16 &&
      c.precision != HIMUON_PREC_BF16X3 && c.precision != HIMUON_PREC_BF16F8) {
    err = "precision must be HIMUON_PREC_F32, HIMUON_PREC_BF16, HIMUON_PREC_BF16X3 or HIMUON_PREC_BF16F8";
    return HIMUON_EINVAL;
  }
  if (c.precision == HIMUON_PREC_BF16F8 && !f8_exponents(c.coeffs.a, c.coeffs.b, c.coeffs.c, c.steps, p.f8)) {
    err = "HIMUON_PREC_BF16F8: the coefficients' iterates are unbounded; use HIMUON_PREC_BF16X3";
    return HIMUON_EINVAL;
  }
  if (c.flags & ~(HIMUON_FLAG_WRITE_UPDATE | HIMUON_FLAG_IDENTITY_MAP)) {
    err = "unknown flag bits";
    return HIMUON_EINVAL;
  }
  const bool want_u = c.flags & HIMUON_FLAG_WRITE_UPDATE;
  const size_t esz = c.state_dtype == HIMUON_BF16 ? 2 : 4;
  p.layers.assign(layers, layers + n);
  p.ldesc.clear();
  for (int32_t i = 0; i < n; ++i) {
    const himuon_layer &L = layers[i];
    if (L.rows < 0 || L.cols < 0 || L.rows >= kMaxDim || L.cols >= kMaxDim) {
      m << "layer " << i << ": rows/cols out of range";
      err = m.str();
      return HIMUON_EINVAL;
    }
    const bool empty = L.rows == 0 || L.cols == 0;
    if (!empty) {
      if (L.ld_w < L.cols || L.ld_m < L.cols || L.ld_g < L.cols || (want_u && L.ld_u < L.cols)) {
        m << "layer " << i << ": leading dimension smaller than cols";
        err = m.str();
        return HIMUON_EINVAL;
      }
      if (!L.weight || !L.momentum || !L.grad || (want_u && !L.update)) {
        m << "layer " << i << ": NULL device pointer";
        err = m.str();
        return HIMUON_EINVAL;
      }
      if (((uintptr_t)L.weight & 3) || ((uintptr_t)L.momentum & (esz - 1)) ||
          ((uintptr_t)L.grad & (esz - 1)) || (want_u && ((uintptr_t)L.update & 3))) {
        m << "layer " << i << ": pointer not aligned to its element size";
        err = m.str();
        return HIMUON_EINVAL;
      }
    }
    LayerDesc d{};
    d.w = L.weight;
    d.m = L.momentum;
    d.g = L.grad;
    d.u = want_u ? L.update : nullptr;
    d.ld_w = L.ld_w;
    d.ld_m = L.ld_m;
    d.ld_g = L.ld_g;
    d.ld_u = want_u ? L.ld_u : 0;
    d.rows = (int32_t)L.rows;
    d.cols = (int32_t)L.cols;
    d.vec_ok = (L.ld_m % 8 == 0) && (L.ld_g % 8 == 0) && ((uintptr_t)L.momentum % 16 == 0) &&
               ((uintptr_t)L.grad % 16 == 0);
    d.vec_w = (L.ld_w % 4 == 0) && ((uintptr_t)L.weight % 16 == 0) &&
              (!want_u || ((L.ld_u % 4 == 0) && ((uintptr_t)L.update % 16 == 0)));
    p.ldesc.push_back(d);
  }
  p.cfg = c;
  return HIMUON_OK;
}

// Bounds on the entries of the matrices of each NS step, from bounds on singular values
// (an entry never exceeds the largest singular value): X_0 = Y / (|Y|_F + eps) has
// sigma_max < 1; A = X X^T has sigma_max(X)^2; B = b A + c A^2 has the largest |b l +
// c l^2| over eigenvalues l in [0, sigma_max(X)^2]; and X' = p(X) has the largest
// |a s + b s^3 + c s^5| over s in [0, sigma_max(X)].  The maxima of these polynomials on
// an interval are taken at its ends or at a real critical point inside it.
namespace {
double max_abs_quad(double a, double b, double c, double L) {   // max |a + b l + c l^2|, l in [0, L]
  auto f = [&](double l) { return std::fabs(a + b * l + c * l * l); };
  double m = std::max(f(0.0), f(L));
  if (c != 0.0) {
    const double v = -b / (2.0 * c);
    if (v > 0.0 && v < L) m = std::max(m, f(v));
  }
  return m;
}
double max_abs_odd5(double a, double b, double c, double S) {   // max |a s + b s^3 + c s^5|, s in [0, S]
  auto g = [&](double x) { return std::fabs(x * (a + b * x * x + c * x * x * x * x)); };
  double m = std::max(g(0.0), g(S));
  // g'(s) = a + 3 b u + 5 c u^2 with u = s^2
  double us[2];
  int nu = 0;
  if (c != 0.0) {
    const double disc = 9.0 * b * b - 20.0 * a * c;
    if (disc >= 0.0) {
      const double r = std::sqrt(disc);
      us[nu++] = (-3.0 * b + r) / (10.0 * c);
      us[nu++] = (-3.0 * b - r) / (10.0 * c);
    }
  } else if (b != 0.0) {
    us[nu++] = -a / (3.0 * b);
  }
  for (int i = 0; i < nu; ++i)
    if (us[i] > 0.0 && us[i] < S * S) m = std::max(m, g(std::sqrt(us[i])));
  return m;
}
// the largest e with bound * 2^e <= 224 (half the e4m3 limit), clamped to [-60, 59]
int f8_exp_for(double bound) {
  if (!(bound > 1e-30)) return 59;
  const double e = std::floor(std::log2(224.0 / bound));
  return (int)std::max(-60.0, std::min(59.0, e));
}
}  // namespace

bool f8_exponents(double a, double b, double c, int steps, F8Exps &e) {
  double xs = 1.0;   // bound on sigma_max(X_k)
  for (int i = 0; i < kF8Steps; ++i) e.x[i] = e.a[i] = e.b[i] = 59;
  const int n = std::max(steps, 1);
  for (int k = 0; k <= n; ++k) {
    if (!std::isfinite(xs) || xs > 1e30) return false;
    const int i = std::min(k, kF8Steps - 1);
    // the last slot serves every later step: keep the smallest exponent
    e.x[i] = (int8_t)std::min<int>(e.x[i], f8_exp_for(xs));
    if (k == n) break;
    const double as = xs * xs;
    e.a[i] = (int8_t)std::min<int>(e.a[i], f8_exp_for(as));
    // the update's e4m3 operand is B = b A + c A^2 alone (its a X term is formed in fp32)
    e.b[i] = (int8_t)std::min<int>(e.b[i], f8_exp_for(max_abs_quad(0.0, b, c, as)));
    xs = max_abs_odd5(a, b, c, xs);
  }
  return true;
}

himuon_status plan_partition(Plan &p, int32_t tile, std::string &err) {
  if (tile < 0) {
    err = "tile must be >= 1 or HIMUON_TILE_FULL (0)";
    return HIMUON_EINVAL;
  }
  const himuon_config &c = p.cfg;
  const int prec = (int)c.precision;
  const int64_t K = c.steps;
  const bool quintic = c.coeffs.c != 0.0;
  // MFMA work per product in units of one bf16 product: the split scheme issues three;
  // BF16F8 one bf16 product and two e4m3 products at twice the rate (fused tiles of edge
  // 64 and 128; smaller and larger tiles run the BF16X3 products)
  const double split = prec == HIMUON_PREC_BF16X3 || prec == HIMUON_PREC_BF16F8 ? 3.0 : 1.0;
  const size_t esz = c.state_dtype == HIMUON_BF16 ? 2 : 4;

  std::vector<FusedTile> by_edge[3][2];   // [edge][dense]
  std::vector<GemmTile> gt;
  std::vector<himuon_tile> order;
  double ns_flops = 0, issued = 0, bytes = 0;
  size_t max_ws = 0;
  for (size_t li = 0; li < p.layers.size(); ++li) {
    const int64_t H = p.layers[li].rows, W = p.layers[li].cols;
    if (H == 0 || W == 0) continue;
    bytes += (double)H * W * (3.0 * esz + 8.0);
    const int64_t T = tile == 0 ? std::max(H, W) : tile;
    for (int64_t r0 = 0; r0 < H; r0 += T) {
      for (int64_t c0 = 0; c0 < W; c0 += T) {
        const int64_t h = std::min(T, H - r0), w = std::min(T, W - c0);
        const int64_t r = std::min(h, w), s = std::max(h, w);
        ns_flops += (double)K * (4.0 * r * r * s + (quintic ? 2.0 * r * r * r : 0.0));
        order.push_back(himuon_tile{(int32_t)li, h > w ? 1 : 0, r0, c0, h, w});
        const int e = fused_edge_for(s);
        if (e) {
          const LayerDesc &d = p.ldesc[li];
          const bool dense = h == e && w == e && d.vec_ok && d.vec_w && c0 % 8 == 0;
          by_edge[e == 32 ? 0 : (e == 64 ? 1 : 2)][dense ? 1 : 0].push_back(
              FusedTile{(int32_t)li, (int32_t)r0, (int32_t)c0, (int16_t)h, (int16_t)w});
          {
            // the symmetric products (X X^T, A^2) run on the (nb + 1) / (2 nb) share of
            // 32x32 blocks on and above the diagonal; the update on all blocks.  bf16f8
            // issues two bf16-product units per product, one for the plain products of
            // the first steps on full tiles (Gram, square and update).
            const double nb = e / 32.0, f = (nb + 1.0) / (2.0 * nb);
            if (prec == HIMUON_PREC_BF16F8 && e >= 64) {
              const bool full = h == e && w == e;
              const int pg = full ? f8_plain_gram_steps(e, dense) : 0, ps = full ? f8_plain_square_steps(e, dense) : 0;
              const int pu = full ? f8_plain_update_steps(e, dense) : 0;   // never the last step
              for (int k = 0; k < K; ++k) {
                const double units = f * (k < pg ? 1.0 : 2.0) + (quintic ? f * (k < ps ? 1.0 : 2.0) : 0.0) +
                                     (k < pu && k + 1 < K ? 1.0 : 2.0);
                issued += 2.0 * e * e * e * units;
              }
            } else {
              issued += (double)K * split * 2.0 * e * e * e * (1.0 + f * (quintic ? 2.0 : 1.0));
            }
          }
        } else {
          const GemmSizes z = gemm_sizes(h, w);
          GemmTile g{};
          g.layer = (int32_t)li;
          g.row0 = (int32_t)r0;
          g.col0 = (int32_t)c0;
          g.h = (int32_t)h;
          g.w = (int32_t)w;
          g.r = (int32_t)r;
          g.s = (int32_t)s;
          g.tall = h > w;
          g.ldx = (int32_t)z.ldx;
          g.lda = (int32_t)z.lda;
          g.nred = (int32_t)z.nred;
          gt.push_back(g);
          max_ws = std::max(max_ws, tile_workspace(g, prec));
          const int kind = gemm_kind(g, prec);
          if (kind == 1) {
            // one workgroup per tile and product, every 256 x 256 block computed; bf16f8
            // requests run the bf16x3 products with the plain early symmetric products
            const double e3 = 2.0 * 256.0 * 256.0 * 256.0;
            const bool f8 = prec == HIMUON_PREC_BF16F8;
            const int pg = f8 ? kF8PlainGramSteps : 0, ps = f8 ? f8_plain_square_steps(256, true) : 0;
            for (int k = 0; k < K; ++k)
              issued += e3 * ((k < pg ? 1.0 : split) + (quintic ? (k < ps ? 1.0 : split) : 0.0) + split);
          } else if (kind == 2) {
            // 256-blocks: symmetric products on the upper blocks only; the update over all;
            // bf16f8 requests: the same plain early symmetric products as 256-tiles
            const double nb = (double)(r / 256), nbs = (double)(s / 256);
            const double sym = nb * (nb + 1) / 2 * 2.0 * 256 * 256;
            const bool f8 = prec == HIMUON_PREC_BF16F8;
            const int pg = f8 ? kF8PlainGramSteps : 0, ps = f8 ? f8_plain_square_steps(256, true) : 0;
            for (int k = 0; k < K; ++k)
              issued += (k < pg ? 1.0 : split) * sym * z.ldx + (quintic ? (k < ps ? 1.0 : split) * sym * z.lda : 0.0) +
                        split * 2.0 * 256 * 256 * nb * nbs * z.lda;
          } else {
            // 128-blocks as launched: symmetric products on the upper blocks only, K
            // padded to 64; the update over all blocks
            const double nb = (double)cdiv(r, 128), nbs = (double)cdiv(z.ldx, 128);
            const double sym = nb * (nb + 1) / 2 * 2.0 * 128 * 128;
            issued += (double)K * split * (sym * z.ldx + (quintic ? sym * z.lda : 0.0) +
                                           2.0 * 128 * 128 * nb * nbs * z.lda);
          }
        }
      }
    }
  }
  if (!gt.empty() && max_ws > c.workspace_budget) {
    std::ostringstream m;
    m << "workspace budget " << c.workspace_budget << " B is below the " << max_ws
      << " B one tile of the large-tile path needs";
    err = m.str();
    return HIMUON_EBUDGET;
  }
  // chunks: consecutive GEMM tiles whose workspaces fit the budget together; each chunk
  // gets the work lists of its grouped launches
  std::vector<GemmChunk> chunks;
  std::vector<GemmWork> wmom, wstg, wsym, wupd, wapp;
  size_t ws_max = 0;
  {
    size_t cur = 0;
    int64_t first = 0;
    auto close_chunk = [&](int64_t end) {
      GemmChunk ch{};
      ch.first = first;
      ch.n = end - first;
      ch.ws_bytes = cur;
      ch.mom.first = (int64_t)wmom.size();
      ch.stg.first = (int64_t)wstg.size();
      ch.sym.first = (int64_t)wsym.size();
      ch.upd.first = (int64_t)wupd.size();
      ch.app.first = (int64_t)wapp.size();
      ch.long_k = true;
      for (int64_t i = first; i < end; ++i)
        ch.long_k = ch.long_k && gt[(size_t)i].lda >= kGemmLongK && gt[(size_t)i].ldx >= kGemmLongK;
      // chunks are cut where the kind changes, so the first tile's kind is the chunk's
      const int kind = end > first ? gemm_kind(gt[(size_t)first], prec) : 0;
      ch.t256 = kind == 1;
      ch.b256 = kind == 2;
      // Products of long-K chunks list their blocks in groups of block rows (kGemmGroupRows
      // of 128, half as many of 256), column by column inside a group, so that the
      // workgroups in flight on one XCD (a contiguous run of the list) share the K slices
      // of a few row and column panels in that XCD's L2.  Short-K chunks keep the
      // row-major order.
      for (int64_t i = first; i < end; ++i) {
        const GemmTile &g = gt[(size_t)i];
        const int32_t ti = (int32_t)i;
        for (int32_t b = 0; b < g.nred; ++b) wmom.push_back(GemmWork{ti, b, 0});
        // stage / apply: 64 x 64 blocks for tall tiles (LDS transpose), else strips of
        // 16 rows x 256 columns (straight from registers)
        const int64_t sr = g.tall ? 64 : 16, sc = g.tall ? 64 : 256;
        for (int32_t bi = 0; bi < (int32_t)cdiv(g.r, sr); ++bi)
          for (int32_t bj = 0; bj < (int32_t)cdiv(g.ldx, sc); ++bj) wstg.push_back(GemmWork{ti, bi, bj});
        // product blocks: 256 x 256 in 256-block chunks, else 128 x 128
        const int64_t pb = ch.b256 ? 256 : 128;
        const int32_t nb = (int32_t)cdiv(g.r, pb), nbj = (int32_t)cdiv(g.ldx, pb);
        const int32_t grp = ch.long_k ? (ch.b256 ? kGemmGroupRows / 2 : kGemmGroupRows) : 0;
        if (ch.t256) {
          // products address their tiles directly: no block lists
        } else if (grp > 0) {
          for (int32_t b0 = 0; b0 < nb; b0 += grp) {
            const int32_t b1 = std::min(nb, b0 + grp);
            for (int32_t bj = b0; bj < nb; ++bj)
              for (int32_t bi = b0; bi < b1 && bi <= bj; ++bi) wsym.push_back(GemmWork{ti, bi, bj});
            for (int32_t bj = 0; bj < nbj; ++bj)
              for (int32_t bi = b0; bi < b1; ++bi) wupd.push_back(GemmWork{ti, bi, bj});
          }
        } else {
          for (int32_t bi = 0; bi < nb; ++bi)
            for (int32_t bj = bi; bj < nb; ++bj) wsym.push_back(GemmWork{ti, bi, bj});
          for (int32_t bi = 0; bi < nb; ++bi)
            for (int32_t bj = 0; bj < nbj; ++bj) wupd.push_back(GemmWork{ti, bi, bj});
        }
        for (int32_t bi = 0; bi < (int32_t)cdiv(g.h, sr); ++bi)
          for (int32_t bj = 0; bj < (int32_t)cdiv(g.w, sc); ++bj) wapp.push_back(GemmWork{ti, bi, bj});
      }
      ch.mom.n = (int64_t)wmom.size() - ch.mom.first;
      ch.stg.n = (int64_t)wstg.size() - ch.stg.first;
      ch.sym.n = (int64_t)wsym.size() - ch.sym.first;
      ch.upd.n = (int64_t)wupd.size() - ch.upd.first;
      ch.app.n = (int64_t)wapp.size() - ch.app.first;
      chunks.push_back(ch);
      ws_max = std::max(ws_max, cur);
    };
    for (size_t i = 0; i < gt.size(); ++i) {
      const size_t need = tile_workspace(gt[i], prec);
      const bool kind_change = i > (size_t)first && gemm_kind(gt[i], prec) != gemm_kind(gt[(size_t)first], prec);
      if ((cur + need > c.workspace_budget || kind_change) && i > (size_t)first) {
        close_chunk((int64_t)i);
        first = (int64_t)i;
        cur = 0;
      }
      const GemmSizes z = gemm_sizes(gt[i].h, gt[i].w);
      if (gemm_kind(gt[i], prec) == 1) {   // in place: x1 and b alias x0 and a
        gt[i].ws_x0 = gt[i].ws_x1 = (int64_t)cur;
        gt[i].ws_a = gt[i].ws_b = (int64_t)(cur + z.x);
        gt[i].ws_red = (int64_t)(cur + z.x + z.ab);
      } else {
        gt[i].ws_x0 = (int64_t)cur;
        gt[i].ws_x1 = (int64_t)(cur + z.x);
        gt[i].ws_a = (int64_t)(cur + 2 * z.x);
        gt[i].ws_b = (int64_t)(cur + 2 * z.x + z.ab);
        gt[i].ws_red = (int64_t)(cur + 2 * z.x + 2 * z.ab);
      }
      cur += need;
    }
    if (!gt.empty()) close_chunk((int64_t)gt.size());
  }

  p.tile = tile;
  p.ftiles.clear();
  p.fgroups.clear();
  const int edges[3] = {32, 64, 128};
  for (int k = 0; k < 3; ++k) {
    for (int dn = 1; dn >= 0; --dn) {
      const auto &v = by_edge[k][dn];
      if (v.empty()) continue;
      p.fgroups.push_back(FusedGroup{edges[k], dn == 1, (int64_t)p.ftiles.size(), (int64_t)v.size()});
      p.ftiles.insert(p.ftiles.end(), v.begin(), v.end());
    }
  }
  p.gtiles = std::move(gt);
  p.chunks = std::move(chunks);
  p.wmom = std::move(wmom);
  p.wstg = std::move(wstg);
  p.wsym = std::move(wsym);
  p.wupd = std::move(wupd);
  p.wapp = std::move(wapp);
  p.order = std::move(order);
  p.workspace_bytes = ws_max;

  himuon_stats &st = p.stats;
  st = himuon_stats{};
  st.tile = tile;
  st.kernel_tile = 0;
  if (p.gtiles.empty() && !p.fgroups.empty()) {
    st.kernel_tile = p.fgroups[0].ts;
    for (const FusedGroup &g : p.fgroups)
      if (g.ts != st.kernel_tile) st.kernel_tile = 0;
  }
  st.layers = (int64_t)p.layers.size();
  st.tiles = (int64_t)p.order.size();
  st.fused_tiles = (int64_t)p.ftiles.size();
  st.gemm_tiles = (int64_t)p.gtiles.size();
  st.chunks = (int64_t)p.chunks.size();
  st.workspace_bytes = ws_max;
  st.table_bytes = p.ldesc.size() * sizeof(LayerDesc) + p.ftiles.size() * sizeof(FusedTile) +
                   p.gtiles.size() * sizeof(GemmTile) +
                   (p.wmom.size() + p.wstg.size() + p.wsym.size() + p.wupd.size() + p.wapp.size()) *
                       sizeof(GemmWork);
  st.ns_flops = ns_flops;
  st.issued_flops = issued;
  st.step_bytes = bytes;
  return HIMUON_OK;
}

}  // namespace himuon

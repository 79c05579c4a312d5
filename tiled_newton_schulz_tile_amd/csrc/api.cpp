// C ABI of libhimuon (include/himuon.h): plan lifetime, device upload of the
// descriptor tables, and the launches of one step.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>
#include <new>
#include <string>

#include "himuon.h"
#include "himuon_internal.h"
#include "plan.h"

struct himuon_plan_s {
  himuon::Plan plan;
  // device copy of [LayerDesc... | FusedTile... | GemmTile...]
  int device = -1;
  char *d_buf = nullptr;
  size_t d_cap = 0;
  char *h_stage = nullptr;  // pinned staging for the upload
  size_t h_cap = 0;
  hipEvent_t ev = nullptr;  // completion of the last upload from h_stage
  bool ev_pending = false;
  bool dirty = true;
  size_t off_ftiles = 0, off_gtiles = 0;
  size_t off_w[5] = {0, 0, 0, 0, 0};  // work lists: momentum, stage, sym, update, apply
};

namespace {

thread_local std::string g_err;

himuon_status fail(himuon_status s, const std::string &msg) {
  g_err = msg;
  return s;
}

himuon_status hip_fail(hipError_t e, const char *what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return HIMUON_EDEVICE;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Upload the tables if the partition changed since the last upload.
himuon_status ensure_tables(himuon_plan_t *p, hipStream_t stream) {
  hipError_t e;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->device >= 0 && dev != p->device)
    return fail(HIMUON_EINVAL, "plan is bound to another device than the current one");
  if (!p->dirty) return HIMUON_OK;
  p->device = dev;
  const himuon::Plan &pl = p->plan;
  const size_t lb = align256(pl.ldesc.size() * sizeof(himuon::LayerDesc));
  const size_t fb = align256(pl.ftiles.size() * sizeof(himuon::FusedTile));
  const size_t gb = align256(pl.gtiles.size() * sizeof(himuon::GemmTile));
  const std::vector<himuon::GemmWork> *wl[5] = {&pl.wmom, &pl.wstg, &pl.wsym, &pl.wupd, &pl.wapp};
  size_t wb[5], wtot = 0;
  for (int k = 0; k < 5; ++k) {
    wb[k] = align256(wl[k]->size() * sizeof(himuon::GemmWork));
    wtot += wb[k];
  }
  const size_t total = std::max<size_t>(lb + fb + gb + wtot, 256);
  if (!p->ev) {
    if ((e = hipEventCreateWithFlags(&p->ev, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "hipEventCreate");
  }
  if (total > p->d_cap) {
    // the old table may still be read by queued steps on this stream
    if (p->d_buf) {
      if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      (void)hipFree(p->d_buf);
      p->d_buf = nullptr;
      p->d_cap = 0;
    }
    if ((e = hipMalloc(&p->d_buf, total)) != hipSuccess) {
      p->d_buf = nullptr;
      return e == hipErrorOutOfMemory ? fail(HIMUON_ENOMEM, "hipMalloc of the tile table failed")
                                      : hip_fail(e, "hipMalloc");
    }
    p->d_cap = total;
  }
  if (p->ev_pending) {
    if ((e = hipEventSynchronize(p->ev)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    p->ev_pending = false;
  }
  if (total > p->h_cap) {
    if (p->h_stage) (void)hipHostFree(p->h_stage);
    p->h_stage = nullptr;
    p->h_cap = 0;
    if ((e = hipHostMalloc((void **)&p->h_stage, total, hipHostMallocDefault)) != hipSuccess) {
      p->h_stage = nullptr;
      return fail(HIMUON_ENOMEM, "hipHostMalloc of the upload staging failed");
    }
    p->h_cap = total;
  }
  std::memset(p->h_stage, 0, total);
  std::memcpy(p->h_stage, pl.ldesc.data(), pl.ldesc.size() * sizeof(himuon::LayerDesc));
  std::memcpy(p->h_stage + lb, pl.ftiles.data(), pl.ftiles.size() * sizeof(himuon::FusedTile));
  std::memcpy(p->h_stage + lb + fb, pl.gtiles.data(), pl.gtiles.size() * sizeof(himuon::GemmTile));
  size_t off = lb + fb + gb;
  for (int k = 0; k < 5; ++k) {
    std::memcpy(p->h_stage + off, wl[k]->data(), wl[k]->size() * sizeof(himuon::GemmWork));
    p->off_w[k] = off;
    off += wb[k];
  }
  if ((e = hipMemcpyAsync(p->d_buf, p->h_stage, total, hipMemcpyHostToDevice, stream)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync of the tile table");
  if ((e = hipEventRecord(p->ev, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  p->ev_pending = true;
  p->off_ftiles = lb;
  p->off_gtiles = lb + fb;
  p->dirty = false;
  return HIMUON_OK;
}

}  // namespace

extern "C" {

himuon_status himuon_plan(const himuon_layer *layers, int32_t n_layers, const himuon_config *cfg,
                          himuon_plan_t **out) {
  if (!out) return fail(HIMUON_EINVAL, "out is NULL");
  *out = nullptr;
  himuon_plan_t *p = new (std::nothrow) himuon_plan_s();
  if (!p) return fail(HIMUON_ENOMEM, "host allocation failed");
  std::string err;
  himuon_status s = himuon::plan_init(p->plan, layers, n_layers, cfg, err);
  if (s == HIMUON_OK) s = himuon::plan_partition(p->plan, cfg->tile, err);
  if (s != HIMUON_OK) {
    delete p;
    return fail(s, err);
  }
  *out = p;
  g_err.clear();
  return HIMUON_OK;
}

himuon_status himuon_workspace_size(const himuon_plan_t *p, size_t *bytes) {
  if (!p || !bytes) return fail(HIMUON_EINVAL, "NULL argument");
  *bytes = p->plan.workspace_bytes;
  return HIMUON_OK;
}

himuon_status himuon_step(himuon_plan_t *p, void *workspace, size_t ws_bytes, float lr,
                          void *hip_stream) {
  if (!p) return fail(HIMUON_EINVAL, "plan is NULL");
  if (!std::isfinite(lr)) return fail(HIMUON_EINVAL, "lr must be finite");
  const himuon::Plan &pl = p->plan;
  if (pl.workspace_bytes && (!workspace || ws_bytes < pl.workspace_bytes))
    return fail(HIMUON_EINVAL, "workspace smaller than himuon_workspace_size");
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  himuon_status s = ensure_tables(p, stream);
  if (s != HIMUON_OK) return s;
  const himuon_config &c = pl.cfg;
  himuon::NSParams prm{};
  prm.a = (float)c.coeffs.a;
  prm.b = (float)c.coeffs.b;
  prm.c = (float)c.coeffs.c;
  prm.beta = c.beta;
  prm.eps = c.eps;
  prm.lr = lr;
  prm.identity = (c.flags & HIMUON_FLAG_IDENTITY_MAP) ? 1 : 0;
  prm.steps = prm.identity ? 0 : c.steps;
  prm.write_update = (c.flags & HIMUON_FLAG_WRITE_UPDATE) ? 1 : 0;
  prm.f8 = pl.f8;
  // the e4m3 correction products exist for fused tiles of edge 64 and 128 only
  const int gemm_prec = c.precision == HIMUON_PREC_BF16F8 ? (int)HIMUON_PREC_BF16X3 : (int)c.precision;
  const auto *dl = reinterpret_cast<const himuon::LayerDesc *>(p->d_buf);
  const auto *dft = reinterpret_cast<const himuon::FusedTile *>(p->d_buf + p->off_ftiles);
  for (const himuon::FusedGroup &g : pl.fgroups) {
    const int fprec = c.precision == HIMUON_PREC_BF16F8 && g.ts < 64 ? (int)HIMUON_PREC_BF16X3 : (int)c.precision;
    hipError_t e = himuon::launch_fused(g.ts, fprec, c.state_dtype == HIMUON_BF16,
                                        g.dense, dl, dft + g.first, g.n, prm, stream);
    if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
  }
  if (!pl.chunks.empty()) {
    const auto *dgt = reinterpret_cast<const himuon::GemmTile *>(p->d_buf + p->off_gtiles);
    const himuon::GemmWork *dw[5];
    for (int k = 0; k < 5; ++k) dw[k] = reinterpret_cast<const himuon::GemmWork *>(p->d_buf + p->off_w[k]);
    for (const himuon::GemmChunk &ch : pl.chunks) {
      himuon::GemmChunkLaunch cl{};
      cl.tile_first = ch.first;
      cl.tile_n = ch.n;
      cl.mom = dw[0] + ch.mom.first;
      cl.n_mom = ch.mom.n;
      cl.stg = dw[1] + ch.stg.first;
      cl.n_stg = ch.stg.n;
      cl.sym = dw[2] + ch.sym.first;
      cl.n_sym = ch.sym.n;
      cl.upd = dw[3] + ch.upd.first;
      cl.n_upd = ch.upd.n;
      cl.app = dw[4] + ch.app.first;
      cl.n_app = ch.app.n;
      cl.long_k = ch.long_k ? 1 : 0;
      cl.t256 = ch.t256 ? 1 : 0;
      cl.b256 = ch.b256 ? 1 : 0;
      hipError_t e = himuon::launch_gemm_chunk(gemm_prec, c.state_dtype == HIMUON_BF16, dl, dgt, cl,
                                               reinterpret_cast<char *>(workspace), prm, stream);
      if (e != hipSuccess) return hip_fail(e, "large-tile kernel launch");
    }
  }
  return HIMUON_OK;
}

himuon_status himuon_set_tile_schedule(himuon_plan_t *p, int32_t tile) {
  if (!p) return fail(HIMUON_EINVAL, "plan is NULL");
  if (tile == p->plan.tile) return HIMUON_OK;
  himuon::Plan trial = p->plan;
  std::string err;
  himuon_status s = himuon::plan_partition(trial, tile, err);
  if (s != HIMUON_OK) return fail(s, err);
  p->plan = std::move(trial);
  p->dirty = true;
  return HIMUON_OK;
}

himuon_status himuon_plan_stats(const himuon_plan_t *p, himuon_stats *out) {
  if (!p || !out) return fail(HIMUON_EINVAL, "NULL argument");
  *out = p->plan.stats;
  return HIMUON_OK;
}

himuon_status himuon_plan_tiles(const himuon_plan_t *p, himuon_tile *out, int64_t cap, int64_t *n) {
  if (!p || !n || cap < 0 || (cap > 0 && !out)) return fail(HIMUON_EINVAL, "bad argument");
  const auto &o = p->plan.order;
  *n = (int64_t)o.size();
  const int64_t k = std::min<int64_t>(cap, (int64_t)o.size());
  if (k > 0) std::memcpy(out, o.data(), (size_t)k * sizeof(himuon_tile));
  return HIMUON_OK;
}

void himuon_plan_destroy(himuon_plan_t *p) {
  if (!p) return;
  if (p->ev) {
    if (p->ev_pending) (void)hipEventSynchronize(p->ev);
    (void)hipEventDestroy(p->ev);
  }
  if (p->d_buf) (void)hipFree(p->d_buf);
  if (p->h_stage) (void)hipHostFree(p->h_stage);
  delete p;
}

const char *himuon_last_error(void) { return g_err.c_str(); }

}  // extern "C"

extern "C" HIMUON_API himuon_status himuon_sign_pack(const float *o, int64_t rows, int64_t cols, int64_t ld,
                                                     uint8_t *bits, void *hip_stream) {
  if (rows < 0 || cols < 0 || ld < cols) return fail(HIMUON_EINVAL, "sizes must be >= 0 and ld >= cols");
  if (rows == 0 || cols == 0) return HIMUON_OK;
  if (rows > (INT64_MAX / 2) / cols) return fail(HIMUON_EINVAL, "rows * cols too large");
  if (!o || !bits) return fail(HIMUON_EINVAL, "NULL pointer");
  if (reinterpret_cast<uintptr_t>(bits) % 8) return fail(HIMUON_EINVAL, "bits must be 8-byte aligned");
  hipError_t e = himuon::launch_sign_pack(o, rows, cols, ld, bits, reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? HIMUON_OK : hip_fail(e, "sign pack launch");
}

extern "C" HIMUON_API himuon_status himuon_sign_vote(const uint8_t *bits, int32_t workers, int64_t stride, int64_t n,
                                                     himuon_dtype out_dtype, void *out, float scale,
                                                     void *hip_stream) {
  if (n < 0) return fail(HIMUON_EINVAL, "n must be >= 0");
  if (workers < 1 || workers > 255) return fail(HIMUON_EINVAL, "workers must be in [1, 255]");
  if (out_dtype != HIMUON_F32 && out_dtype != HIMUON_BF16) return fail(HIMUON_EINVAL, "out_dtype");
  if (!std::isfinite(scale)) return fail(HIMUON_EINVAL, "scale must be finite");
  if (n == 0) return HIMUON_OK;
  if (!bits || !out) return fail(HIMUON_EINVAL, "NULL pointer");
  if (stride < (n + 7) / 8 || stride % 4 || reinterpret_cast<uintptr_t>(bits) % 4)
    return fail(HIMUON_EINVAL, "stride must be >= ceil(n / 8), and bits and stride 4-byte aligned");
  hipError_t e = himuon::launch_sign_vote(bits, workers, stride, n, out_dtype == HIMUON_BF16, out, scale,
                                          reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? HIMUON_OK : hip_fail(e, "sign vote launch");
}

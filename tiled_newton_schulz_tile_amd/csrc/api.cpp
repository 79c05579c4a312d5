// C ABI of libhimuon (include/himuon.h): plan lifetime, the double-buffered device copy
// of the descriptor tables, and the launches of one step (which allocate nothing and
// never wait for the GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>
#include <new>
#include <string>

#include "himuon.h"
#include "himuon_internal.h"
#include "plan.h"

namespace {

// Byte layout of the device copy of the tables: [LayerDesc... | FusedTile... | GemmTile... |
// five GemmWork lists], each part 256-byte aligned.
struct TableLayout {
  size_t total = 0, off_ftiles = 0, off_gtiles = 0;
  size_t off_w[5] = {0, 0, 0, 0, 0};  // work lists: momentum, stage, sym, update, apply
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

const std::vector<himuon::GemmWork> *work_list(const himuon::Plan &pl, int k) {
  const std::vector<himuon::GemmWork> *wl[5] = {&pl.wmom, &pl.wstg, &pl.wsym, &pl.wupd, &pl.wapp};
  return wl[k];
}

TableLayout layout_of(const himuon::Plan &pl) {
  TableLayout t;
  size_t off = align256(pl.ldesc.size() * sizeof(himuon::LayerDesc));
  t.off_ftiles = off;
  off += align256(pl.ftiles.size() * sizeof(himuon::FusedTile));
  t.off_gtiles = off;
  off += align256(pl.gtiles.size() * sizeof(himuon::GemmTile));
  for (int k = 0; k < 5; ++k) {
    t.off_w[k] = off;
    off += align256(work_list(pl, k)->size() * sizeof(himuon::GemmWork));
  }
  t.total = std::max<size_t>(off, 256);
  return t;
}

void fill_tables(char *dst, const himuon::Plan &pl, const TableLayout &t) {
  std::memset(dst, 0, t.total);
  std::memcpy(dst, pl.ldesc.data(), pl.ldesc.size() * sizeof(himuon::LayerDesc));
  std::memcpy(dst + t.off_ftiles, pl.ftiles.data(), pl.ftiles.size() * sizeof(himuon::FusedTile));
  std::memcpy(dst + t.off_gtiles, pl.gtiles.data(), pl.gtiles.size() * sizeof(himuon::GemmTile));
  for (int k = 0; k < 5; ++k)
    std::memcpy(dst + t.off_w[k], work_list(pl, k)->data(), work_list(pl, k)->size() * sizeof(himuon::GemmWork));
}

// One device copy of the tables and the pinned staging its last upload came from.
struct TableBuf {
  char *d = nullptr;
  size_t cap = 0;
  char *h = nullptr;
  size_t hcap = 0;
  hipEvent_t ev = nullptr;  // recorded after the last upload from h
  bool pending = false;     // ev recorded and not yet seen complete
  TableLayout lay;
};

}  // namespace

struct himuon_plan_s {
  himuon::Plan plan;
  int device = -1;                 // device holding the tables; -1: no GPU at plan time
  TableBuf buf[2];                 // double-buffered device tables
  int active = 0;                  // the buffer the next step reads
  std::vector<void *> retired_d;   // outgrown device buffers (possibly still read by queued
  std::vector<void *> retired_h;   // steps) and pinned staging, released by destroy
  himuon_runtime_counts counts{};
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

himuon_status check_device(const himuon_plan_t *p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) return fail(HIMUON_EINVAL, "plan is bound to another device than the current one");
  return HIMUON_OK;
}

// Device tables of a new plan: allocated and uploaded with a blocking copy.  A process
// without a GPU gets a host-only plan (device -1).
himuon_status bind_device(himuon_plan_t *p) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();   // leave no stale error for the next launch check
    p->device = -1;
    return HIMUON_OK;
  }
  hipError_t e;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
  TableBuf &b = p->buf[0];
  b.lay = layout_of(p->plan);
  if ((e = hipMalloc(&b.d, b.lay.total)) != hipSuccess) {
    b.d = nullptr;
    return e == hipErrorOutOfMemory ? fail(HIMUON_ENOMEM, "hipMalloc of the tile table failed")
                                    : hip_fail(e, "hipMalloc");
  }
  b.cap = b.lay.total;
  ++p->counts.device_allocs;
  std::vector<char> host(b.lay.total);
  fill_tables(host.data(), p->plan, b.lay);
  if ((e = hipMemcpy(b.d, host.data(), b.lay.total, hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(e, "hipMemcpy of the tile table");
  ++p->counts.host_waits;
  p->device = dev;
  p->active = 0;
  return HIMUON_OK;
}

// Puts the tables of `pl` into the spare buffer, stream-ordered on `stream`, and makes it
// the active one.  Allocates only when the spare is too small; waits only when the
// spare's staging is still being read by the upload of two schedule changes ago.
himuon_status upload_spare(himuon_plan_t *p, const himuon::Plan &pl, hipStream_t stream) {
  hipError_t e;
  const int s = 1 - p->active;
  TableBuf &b = p->buf[s];
  const TableLayout lay = layout_of(pl);
  if (!b.ev) {
    if ((e = hipEventCreateWithFlags(&b.ev, hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "hipEventCreate");
  }
  if (lay.total > b.cap) {
    const size_t cap = std::max(lay.total, b.cap + b.cap / 2);
    char *d = nullptr;
    if ((e = hipMalloc(&d, cap)) != hipSuccess)
      return e == hipErrorOutOfMemory ? fail(HIMUON_ENOMEM, "hipMalloc of the tile table failed")
                                      : hip_fail(e, "hipMalloc");
    ++p->counts.device_allocs;
    if (b.d) p->retired_d.push_back(b.d);   // queued steps may still read it
    b.d = d;
    b.cap = cap;
  }
  if (lay.total > b.hcap) {
    const size_t cap = std::max(lay.total, b.hcap + b.hcap / 2);
    char *h = nullptr;
    if ((e = hipHostMalloc((void **)&h, cap, hipHostMallocDefault)) != hipSuccess)
      return fail(HIMUON_ENOMEM, "hipHostMalloc of the upload staging failed");
    ++p->counts.host_allocs;
    if (b.h) p->retired_h.push_back(b.h);   // a pending upload may still read it
    b.h = h;
    b.hcap = cap;
    b.pending = false;
  } else if (b.pending) {
    e = hipEventQuery(b.ev);
    if (e == hipErrorNotReady) {
      if ((e = hipEventSynchronize(b.ev)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      ++p->counts.host_waits;
    } else if (e != hipSuccess) {
      return hip_fail(e, "hipEventQuery");
    }
    b.pending = false;
  }
  fill_tables(b.h, pl, lay);
  if ((e = hipMemcpyAsync(b.d, b.h, lay.total, hipMemcpyHostToDevice, stream)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync of the tile table");
  if ((e = hipEventRecord(b.ev, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  b.pending = true;
  b.lay = lay;
  p->active = s;
  return HIMUON_OK;
}

}  // namespace

himuon_status himuon::set_error(himuon_status s, const std::string &msg) { return fail(s, msg); }

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
  if ((s = bind_device(p)) != HIMUON_OK) {
    const std::string msg = g_err;
    himuon_plan_destroy(p);
    return fail(s, msg);
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
  if (p->device < 0) return fail(HIMUON_EDEVICE, "the plan has no device tables (no GPU was visible to himuon_plan)");
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  himuon_status s = check_device(p);
  if (s != HIMUON_OK) return s;
  const TableBuf &tb = p->buf[p->active];
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
  if (c.precision == HIMUON_PREC_BF16F8) {
    prm.plain_gram = himuon::kF8PlainGramSteps;
    prm.plain_square = himuon::f8_plain_square_steps(256, true);
  }
  // the e4m3 correction products exist for fused tiles of edge 64 and 128 only
  const int gemm_prec = c.precision == HIMUON_PREC_BF16F8 ? (int)HIMUON_PREC_BF16X3 : (int)c.precision;
  const auto *dl = reinterpret_cast<const himuon::LayerDesc *>(tb.d);
  const auto *dft = reinterpret_cast<const himuon::FusedTile *>(tb.d + tb.lay.off_ftiles);
  for (const himuon::FusedGroup &g : pl.fgroups) {
    const int fprec = c.precision == HIMUON_PREC_BF16F8 && g.ts < 64 ? (int)HIMUON_PREC_BF16X3 : (int)c.precision;
    hipError_t e = himuon::launch_fused(g.ts, fprec, c.state_dtype == HIMUON_BF16,
                                        g.dense, dl, dft + g.first, g.n, prm, stream);
    if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
  }
  if (!pl.chunks.empty()) {
    const auto *dgt = reinterpret_cast<const himuon::GemmTile *>(tb.d + tb.lay.off_gtiles);
    const himuon::GemmWork *dw[5];
    for (int k = 0; k < 5; ++k) dw[k] = reinterpret_cast<const himuon::GemmWork *>(tb.d + tb.lay.off_w[k]);
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

himuon_status himuon_set_tile_schedule(himuon_plan_t *p, int32_t tile, void *hip_stream) {
  if (!p) return fail(HIMUON_EINVAL, "plan is NULL");
  if (tile == p->plan.tile) return HIMUON_OK;
  himuon::Plan trial = p->plan;
  std::string err;
  himuon_status s = himuon::plan_partition(trial, tile, err);
  if (s != HIMUON_OK) return fail(s, err);
  if (p->device >= 0) {
    if ((s = check_device(p)) != HIMUON_OK) return s;
    if ((s = upload_spare(p, trial, reinterpret_cast<hipStream_t>(hip_stream))) != HIMUON_OK) return s;
  }
  p->plan = std::move(trial);
  return HIMUON_OK;
}

himuon_status himuon_plan_runtime_counts(const himuon_plan_t *p, himuon_runtime_counts *out) {
  if (!p || !out) return fail(HIMUON_EINVAL, "NULL argument");
  *out = p->counts;
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
  for (TableBuf &b : p->buf) {
    if (b.ev) {
      if (b.pending) (void)hipEventSynchronize(b.ev);
      (void)hipEventDestroy(b.ev);
    }
    if (b.d) (void)hipFree(b.d);
    if (b.h) (void)hipHostFree(b.h);
  }
  for (void *d : p->retired_d) (void)hipFree(d);
  for (void *h : p->retired_h) (void)hipHostFree(h);
  delete p;
}

const char *himuon_last_error(void) { return g_err.c_str(); }

}  // extern "C"

extern "C" HIMUON_API himuon_status himuon_stream_step(void *m, const void *g, float *w, int64_t n,
                                                       himuon_dtype state_dtype, float beta, float lr,
                                                       void *hip_stream) {
  if (n < 0) return fail(HIMUON_EINVAL, "n must be >= 0");
  if (state_dtype != HIMUON_F32 && state_dtype != HIMUON_BF16) return fail(HIMUON_EINVAL, "state_dtype");
  if (!std::isfinite(beta) || !std::isfinite(lr)) return fail(HIMUON_EINVAL, "beta and lr must be finite");
  if (n == 0) return HIMUON_OK;
  if (!m || !g || !w) return fail(HIMUON_EINVAL, "NULL pointer");
  hipError_t e = himuon::launch_stream_step(m, g, w, n, state_dtype == HIMUON_BF16, beta, lr,
                                            reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? HIMUON_OK : hip_fail(e, "stream step launch");
}

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

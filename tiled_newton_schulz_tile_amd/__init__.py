"""Python binding of libhimuon, the HiMuon optimizer step on MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
libhimuon.so (see include/himuon.h).  PyTorch provides device memory and streams.
The module refuses to import when the library has not been built; there is no
fallback implementation.

Low-level functions carry the C names (himuon_plan, himuon_step, ...).  The class
HiMuon wraps them for lists of torch tensors.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "HiMuonError", "himuon_layer", "himuon_config", "himuon_stats", "himuon_tile",
    "himuon_plan", "himuon_workspace_size", "himuon_step", "himuon_set_tile_schedule",
    "himuon_plan_stats", "himuon_plan_tiles", "himuon_plan_destroy", "himuon_last_error",
    "himuon_plan_runtime_counts", "himuon_runtime_counts", "himuon_step_static", "STATIC_WORKSPACE_BYTES",
    "himuon_stream_step",
    "HiMuon", "CUBIC", "QUINTIC", "TILE_FULL", "F32", "BF16", "PREC_F32", "PREC_BF16",
    "PREC_BF16X3", "PREC_BF16F8", "FLAG_WRITE_UPDATE", "FLAG_IDENTITY_MAP", "library_path", "EXPORTED",
]

CUBIC = (1.5, -0.5, 0.0)
QUINTIC = (3.4445, -4.7750, 2.0315)
TILE_FULL = 0
F32, BF16 = 0, 1
PREC_F32, PREC_BF16, PREC_BF16X3, PREC_BF16F8 = 0, 1, 2, 3
FLAG_WRITE_UPDATE = 1
FLAG_IDENTITY_MAP = 2
STATIC_WORKSPACE_BYTES = 64 << 20   # HIMUON_STATIC_WORKSPACE_BYTES

STATUS = {0: "HIMUON_OK", -1: "HIMUON_EINVAL", -2: "HIMUON_EBUDGET", -3: "HIMUON_ENOMEM",
          -4: "HIMUON_EDEVICE", -5: "HIMUON_EUNSUPPORTED"}

# every entry point include/himuon.h declares
EXPORTED = ("himuon_plan", "himuon_workspace_size", "himuon_step", "himuon_set_tile_schedule",
            "himuon_plan_stats", "himuon_plan_tiles", "himuon_plan_destroy", "himuon_last_error",
            "himuon_plan_runtime_counts", "himuon_step_static", "himuon_stream_step", "himuon_sign_pack",
            "himuon_sign_vote")


class HiMuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class himuon_coeffs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_double), ("b", ctypes.c_double), ("c", ctypes.c_double)]


class himuon_layer(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_w", ctypes.c_int64), ("ld_m", ctypes.c_int64),
                ("ld_g", ctypes.c_int64), ("ld_u", ctypes.c_int64),
                ("weight", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("grad", ctypes.c_void_p), ("update", ctypes.c_void_p)]


class himuon_config(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("steps", ctypes.c_int32), ("coeffs", himuon_coeffs),
                ("beta", ctypes.c_float), ("eps", ctypes.c_float),
                ("workspace_budget", ctypes.c_size_t), ("state_dtype", ctypes.c_int),
                ("precision", ctypes.c_int), ("flags", ctypes.c_uint32)]


class himuon_stats(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("kernel_tile", ctypes.c_int32),
                ("layers", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("fused_tiles", ctypes.c_int64), ("gemm_tiles", ctypes.c_int64),
                ("chunks", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("table_bytes", ctypes.c_size_t), ("ns_flops", ctypes.c_double),
                ("issued_flops", ctypes.c_double), ("step_bytes", ctypes.c_double)]


class himuon_runtime_counts(ctypes.Structure):
    _fields_ = [("device_allocs", ctypes.c_int64), ("host_allocs", ctypes.c_int64),
                ("host_waits", ctypes.c_int64)]


class himuon_tile(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("transposed", ctypes.c_int32),
                ("row0", ctypes.c_int64), ("col0", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhimuon.so")


def _load() -> ctypes.CDLL:
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python tiled_newton_schulz_tile_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    missing = [n for n in EXPORTED if not hasattr(lib, n)]
    if missing:
        raise ImportError(f"{path} is stale (no {', '.join(missing)}): rebuild it with "
                          "`python tiled_newton_schulz_tile_amd/build.py`")
    P = ctypes.c_void_p
    lib.himuon_plan.argtypes = [ctypes.POINTER(himuon_layer), ctypes.c_int32,
                                ctypes.POINTER(himuon_config), ctypes.POINTER(P)]
    lib.himuon_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.himuon_step.argtypes = [P, P, ctypes.c_size_t, ctypes.c_float, P]
    lib.himuon_step_static.argtypes = [P, ctypes.c_float, P]
    lib.himuon_set_tile_schedule.argtypes = [P, ctypes.c_int32, P]
    lib.himuon_plan_runtime_counts.argtypes = [P, ctypes.POINTER(himuon_runtime_counts)]
    lib.himuon_plan_stats.argtypes = [P, ctypes.POINTER(himuon_stats)]
    lib.himuon_plan_tiles.argtypes = [P, ctypes.POINTER(himuon_tile), ctypes.c_int64,
                                      ctypes.POINTER(ctypes.c_int64)]
    lib.himuon_plan_destroy.argtypes = [P]
    lib.himuon_plan_destroy.restype = None
    lib.himuon_stream_step.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_float, P]
    lib.himuon_sign_pack.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P]
    lib.himuon_sign_vote.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                     P, ctypes.c_float, P]
    lib.himuon_last_error.argtypes = []
    lib.himuon_last_error.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("himuon_plan_destroy", "himuon_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise HiMuonError(status, himuon_last_error())


# ------------------------------------------------------------------ C names
def himuon_last_error() -> str:
    return _lib.himuon_last_error().decode()


def himuon_plan(layers, cfg: himuon_config) -> ctypes.c_void_p:
    """layers: sequence of himuon_layer.  Returns an opaque plan handle."""
    arr = (himuon_layer * max(1, len(layers)))(*layers)
    out = ctypes.c_void_p()
    _check(_lib.himuon_plan(arr, len(layers), ctypes.byref(cfg), ctypes.byref(out)))
    return out


def himuon_workspace_size(plan) -> int:
    n = ctypes.c_size_t()
    _check(_lib.himuon_workspace_size(plan, ctypes.byref(n)))
    return n.value


def himuon_step(plan, workspace_ptr: int, ws_bytes: int, lr: float, stream_ptr: int) -> None:
    _check(_lib.himuon_step(plan, workspace_ptr or None, ws_bytes, lr, stream_ptr or None))


def himuon_step_static(plan, lr: float, stream_ptr: int) -> None:
    _check(_lib.himuon_step_static(plan, lr, stream_ptr or None))


def himuon_set_tile_schedule(plan, tile: int, stream_ptr: int) -> None:
    _check(_lib.himuon_set_tile_schedule(plan, tile, stream_ptr or None))


def himuon_plan_runtime_counts(plan) -> dict:
    c = himuon_runtime_counts()
    _check(_lib.himuon_plan_runtime_counts(plan, ctypes.byref(c)))
    return {name: getattr(c, name) for name, _ in himuon_runtime_counts._fields_}


def himuon_plan_stats(plan) -> dict:
    s = himuon_stats()
    _check(_lib.himuon_plan_stats(plan, ctypes.byref(s)))
    return {name: getattr(s, name) for name, _ in himuon_stats._fields_}


def himuon_plan_tiles(plan) -> list:
    n = ctypes.c_int64()
    _check(_lib.himuon_plan_tiles(plan, None, 0, ctypes.byref(n)))
    arr = (himuon_tile * max(1, n.value))()
    _check(_lib.himuon_plan_tiles(plan, arr, n.value, ctypes.byref(n)))
    return [(t.layer, t.transposed, t.row0, t.col0, t.rows, t.cols) for t in arr[:n.value]]


def himuon_plan_destroy(plan) -> None:
    _lib.himuon_plan_destroy(plan)


def himuon_stream_step(m_ptr: int, g_ptr: int, w_ptr: int, n: int, state_dtype: int, beta: float, lr: float,
                       stream_ptr: int) -> None:
    _check(_lib.himuon_stream_step(m_ptr or None, g_ptr or None, w_ptr or None, n, state_dtype, beta, lr,
                                   stream_ptr or None))


def himuon_sign_pack(o_ptr: int, rows: int, cols: int, ld: int, bits_ptr: int, stream_ptr: int) -> None:
    _check(_lib.himuon_sign_pack(o_ptr or None, rows, cols, ld, bits_ptr or None, stream_ptr or None))


def himuon_sign_vote(bits_ptr: int, workers: int, stride: int, n: int, out_dtype: int, out_ptr: int,
                     scale: float, stream_ptr: int) -> None:
    _check(_lib.himuon_sign_vote(bits_ptr or None, workers, stride, n, out_dtype, out_ptr or None, scale,
                                 stream_ptr or None))


# ------------------------------------------------------------------ torch wrapper
def make_config(tile: int, steps: int = 5, coeffs=QUINTIC, beta: float = 0.95, eps: float = 1e-7,
                workspace_budget: int = 4 * 10 ** 9, state_dtype: int = BF16,
                precision: int = PREC_BF16X3,
                flags: int = 0) -> himuon_config:
    return himuon_config(tile, steps, himuon_coeffs(*coeffs), beta, eps, workspace_budget,
                         state_dtype, precision, flags)


def layer_from_tensors(W, M, G, U=None) -> himuon_layer:
    """himuon_layer for row-major 2-D tensors (unit column stride)."""
    for t in (W, M, G) + ((U,) if U is not None else ()):
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError("tensors must be 2-D with unit column stride")
        if t.shape != W.shape:
            raise ValueError("W, M, G (and U) must have the same shape")
    H, Wd = W.shape
    ld = lambda t: max(t.stride(0), Wd, 1)  # noqa: E731
    return himuon_layer(H, Wd, ld(W), ld(M), ld(G), ld(U) if U is not None else 0,
                        W.data_ptr(), M.data_ptr(), G.data_ptr(),
                        U.data_ptr() if U is not None else None)


class HiMuon:
    """HiMuon step over a list of layers given as torch tensors.

    layers: list of (W fp32, M, G) or (W, M, G, U) device tensors; M and G share
    one dtype (torch.float32 or torch.bfloat16).  U (fp32) receives the NS output O
    when given (HIMUON_FLAG_WRITE_UPDATE).  The workspace of the large-tile path is
    a torch byte tensor on the layers' device.  identity=True sets
    HIMUON_FLAG_IDENTITY_MAP (gather -> scatter only, O = M; a test mode).
    """

    def __init__(self, layers, tile: int, steps: int = 5, coeffs=QUINTIC, beta: float = 0.95,
                 eps: float = 1e-7, workspace_budget: int = 4 * 10 ** 9, precision=None,
                 identity: bool = False):
        import torch
        self._torch = torch
        if not layers:
            raise ValueError("no layers")
        sd = layers[0][1].dtype
        if sd not in (torch.float32, torch.bfloat16):
            raise ValueError("momentum/grad dtype must be float32 or bfloat16")
        for l in layers:
            if l[0].dtype != torch.float32 or l[1].dtype != sd or l[2].dtype != sd:
                raise ValueError("W must be float32; M and G share one dtype across layers")
        if precision is None:
            precision = PREC_F32 if sd == torch.float32 else PREC_BF16X3
        write_u = all(len(l) > 3 and l[3] is not None for l in layers)
        self.layers = list(layers)
        self.cfg = make_config(tile, steps, coeffs, beta, eps, workspace_budget,
                               F32 if sd == torch.float32 else BF16, precision,
                               (FLAG_WRITE_UPDATE if write_u else 0) |
                               (FLAG_IDENTITY_MAP if identity else 0))
        self._c_layers = [layer_from_tensors(*l[:3], l[3] if write_u else None) for l in layers]
        self.plan = himuon_plan(self._c_layers, self.cfg)
        self.device = layers[0][0].device
        self.workspace = None
        self._alloc_workspace()

    def _alloc_workspace(self):
        n = himuon_workspace_size(self.plan)
        if n and (self.workspace is None or self.workspace.numel() < n):
            self.workspace = self._torch.empty(n, dtype=self._torch.uint8, device=self.device)

    def step(self, lr: float = 0.02, stream=None) -> None:
        torch = self._torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        ws = self.workspace
        himuon_step(self.plan, ws.data_ptr() if ws is not None else 0,
                    ws.numel() if ws is not None else 0, lr, s.cuda_stream)

    def set_tile_schedule(self, tile: int, stream=None) -> None:
        """Change T from the next step on; the table upload is enqueued on `stream` (the
        current stream by default), the stream the following steps should use."""
        torch = self._torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        himuon_set_tile_schedule(self.plan, tile, s.cuda_stream)
        self._alloc_workspace()

    def runtime_counts(self) -> dict:
        return himuon_plan_runtime_counts(self.plan)

    def stats(self) -> dict:
        return himuon_plan_stats(self.plan)

    def tiles(self) -> list:
        return himuon_plan_tiles(self.plan)

    def close(self) -> None:
        if self.plan:
            himuon_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

"""Sign-Muon's local path on top of HiMuon.

"Sign-Muon: Communication-Efficient Distributed Muon Optimization" (Figures 1 and 6, and
its remark on practical orthogonalization with 1-bit communication): each worker takes
its Newton-Schulz direction (here the tiled map O_T = HiMuon_T(M) of its momentum),
forms the entrywise sign, packs it to one bit per entry for an all-gather, takes the
majority vote of the gathered buffers, and steps with the voted sign matrix, or with its
polar map computed locally.  The all-gather is not part of this library: `step` takes
the other workers' packed buffers as an argument (none on a single worker) and returns
this worker's.

Every stage runs in the library's kernels: the direction (a HiMuon step with lr = 0 that
writes O), himuon_sign_pack, himuon_sign_vote, and the update W <- W - lr D through a
second plan over (W, S_bar): with HIMUON_FLAG_IDENTITY_MAP D = S_bar exactly, else
D = HiMuon_T'(S_bar).
"""
from __future__ import annotations

from . import BF16, F32, HiMuon, PREC_BF16X3, QUINTIC, himuon_sign_pack, himuon_sign_vote


def packed_bytes(n: int) -> int:
    """Bytes of one worker's packed buffer for n entries, rounded up to 8 (the kernels'
    alignment); the first ceil(n / 8) hold the signs."""
    return ((n + 7) // 8 + 7) // 8 * 8


def sign_pack(O, out=None, stream=None):
    """Packed sign of the 2-D float32 CUDA tensor O (unit column stride): a uint8 tensor of
    packed_bytes(O.numel()) bytes, entry k = i * cols + j at byte k // 8, bit k % 8."""
    import torch
    if O.dim() != 2 or O.dtype != torch.float32 or not O.is_cuda or (O.shape[1] > 1 and O.stride(1) != 1):
        raise ValueError("O must be a 2-D float32 CUDA tensor with unit column stride")
    rows, cols = O.shape
    nb = packed_bytes(rows * cols)
    if out is None:
        out = torch.zeros(nb, dtype=torch.uint8, device=O.device)
    elif out.numel() < nb or out.dtype != torch.uint8:
        raise ValueError("out too small")
    s = stream if stream is not None else torch.cuda.current_stream(O.device)
    himuon_sign_pack(O.data_ptr(), rows, cols, max(O.stride(0), cols, 1), out.data_ptr(), s.cuda_stream)
    return out


def sign_vote(gathered, n: int, dtype=None, scale: float = 1.0, out=None, stream=None):
    """Majority vote over a (workers, stride) uint8 CUDA tensor of packed buffers (stride a
    multiple of 4): a length-n tensor of +-scale (ties +scale) in dtype (default bf16)."""
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be float32 or bfloat16")
    if gathered.dim() != 2 or gathered.dtype != torch.uint8 or not gathered.is_contiguous():
        raise ValueError("gathered must be a contiguous (workers, stride) uint8 tensor")
    if out is None:
        out = torch.empty(n, dtype=dtype, device=gathered.device)
    s = stream if stream is not None else torch.cuda.current_stream(gathered.device)
    himuon_sign_vote(gathered.data_ptr(), gathered.shape[0], gathered.shape[1], n,
                     F32 if dtype == torch.float32 else BF16, out.data_ptr(), scale, s.cuda_stream)
    return out


class SignMuonLocal:
    """One worker's Sign-Muon step over layers (W fp32, M, G) with HiMuon directions.

    tile, steps, coeffs, beta, precision: the direction's HiMuon map and momentum.
    polar_tile: None steps with the voted sign matrix itself; an int (0 = FULL) steps with
    HiMuon_{polar_tile}(S_bar) (polar_steps, polar_coeffs)."""

    def __init__(self, layers, tile: int, steps: int = 5, coeffs=QUINTIC, beta: float = 0.95,
                 precision=PREC_BF16X3, polar_tile=None, polar_steps: int = 5, polar_coeffs=QUINTIC,
                 eps: float = 1e-7, workspace_budget: int = 4 * 10 ** 9):
        import torch
        self.layers = list(layers)
        dev = self.layers[0][0].device
        self.U = [torch.empty(W.shape, dtype=torch.float32, device=dev) for W, _, _ in self.layers]
        self.direction = HiMuon([(W, M, G, U) for (W, M, G), U in zip(self.layers, self.U)], tile, steps,
                                coeffs, beta, eps, workspace_budget, precision=precision)
        self.n = [W.numel() for W, _, _ in self.layers]
        self.bits = [torch.zeros(packed_bytes(n), dtype=torch.uint8, device=dev) for n in self.n]
        self.sbar = [torch.empty(W.shape, dtype=torch.bfloat16, device=dev) for W, _, _ in self.layers]
        self._mz = [torch.zeros(W.shape, dtype=torch.bfloat16, device=dev) for W, _, _ in self.layers]
        apply_layers = [(W, mz, sb) for (W, _, _), mz, sb in zip(self.layers, self._mz, self.sbar)]
        if polar_tile is None:
            self.apply = HiMuon(apply_layers, 128, 0, coeffs, 0.0, eps, workspace_budget,
                                precision=precision, identity=True)
        else:
            self.apply = HiMuon(apply_layers, polar_tile, polar_steps, polar_coeffs, 0.0, eps,
                                workspace_budget, precision=precision)

    def step(self, lr: float, gathered=None):
        """gathered: None, or per layer a (workers - 1, packed_bytes) uint8 CUDA tensor of
        the other workers' packed signs.  Returns this worker's packed signs per layer."""
        import torch
        self.direction.step(0.0)
        for U, b in zip(self.U, self.bits):
            sign_pack(U, out=b)
        for i, (b, sb) in enumerate(zip(self.bits, self.sbar)):
            allb = b.view(1, -1) if gathered is None else torch.cat([b.view(1, -1), gathered[i]], 0)
            sign_vote(allb, self.n[i], torch.bfloat16, 1.0, out=sb.view(-1))
        self.apply.step(lr)
        return self.bits

    def close(self):
        self.direction.close()
        self.apply.close()

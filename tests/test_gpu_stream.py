"""himuon_stream_step, the flat memory-pass reference (MI355X only): the momentum update
M <- beta M + G (one fp32 fused multiply-add, stored in the state dtype) and the weight
update W <- W - lr M over one contiguous run.  M is checked bit for bit against the
oracle's stored-momentum model, W to one ulp against W0 - lr M in fp64, both on the
vector path (16-byte aligned, with a ragged tail of n % 8 elements) and on the element
path (misaligned starts); and both bit for bit against himuon_step in the identity test
mode on the same values, whose memory pass it stands for."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
DEV = "cuda"
BETA, LR = 0.95, 0.02


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(n, dtype, seed, offset):
    """M, G (state dtype) and W (fp32) on the device, each starting `offset` elements into
    its own allocation (offset 0: 16-byte aligned)."""
    gen = torch.Generator().manual_seed(seed)
    G = synth.power_law_matrix(1, n, seed, dtype=torch.float32).reshape(-1) if n else torch.zeros(0)
    M = 0.5 * torch.randn(n, generator=gen)
    W = torch.randn(n, generator=gen)

    def place(x, dt):
        buf = torch.zeros(n + offset, dtype=dt, device=DEV)
        v = buf[offset:]
        v.copy_(x.to(dt))
        return v

    return place(M, dtype), place(G, dtype), place(W, torch.float32)


def _ulp_diff(a, b):
    return (a.view(torch.int32).long() - b.view(torch.int32).long()).abs().max().item() if a.numel() else 0


@pytest.mark.parametrize("n", [1, 7, 8, 9, 4096 + 5, 1_000_003])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("offset", [0, 1])
def test_stream_step_matches_oracle(n, dtype, offset):
    _need_gpu()
    m, g, w = _inputs(n, dtype, 70 + n % 97, offset)
    m0, g0, w0 = m.cpu().float().numpy(), g.cpu().float().numpy(), w.cpu().double()
    stream = torch.cuda.current_stream().cuda_stream
    hm.himuon_stream_step(m.data_ptr(), g.data_ptr(), w.data_ptr(), n,
                          hm.BF16 if dtype == torch.bfloat16 else hm.F32, BETA, LR, stream)
    torch.cuda.synchronize()
    want_m = oracle.momentum_stored(m0, g0, BETA, "bf16" if dtype == torch.bfloat16 else "f32")
    got_m = m.cpu().float().numpy()
    assert np.array_equal(got_m, want_m)
    want_w = (w0 - float(np.float32(LR)) * torch.from_numpy(want_m).double()).float()
    assert _ulp_diff(w.cpu(), want_w) <= 1


@pytest.mark.parametrize("shape", [(1000, 1537), (4096, 1024)])
@pytest.mark.parametrize("state,prec", [(torch.bfloat16, hm.PREC_BF16F8), (torch.float32, hm.PREC_F32)])
@pytest.mark.parametrize("T", [64, 128])
def test_stream_step_equals_identity_step(shape, state, prec, T):
    _need_gpu()
    H, W = shape
    G = synth.power_law_matrix(H, W, 31, dtype=torch.float32).to(state).to(DEV)
    M0 = (0.5 * synth.power_law_matrix(H, W, 32, dtype=torch.float32)).to(state).to(DEV)
    W0 = torch.randn(H, W, generator=torch.Generator().manual_seed(33)).to(DEV)
    Ma, Wa = M0.clone(), W0.clone()
    opt = hm.HiMuon([(Wa, Ma, G)], T, 5, hm.QUINTIC, BETA, 1e-7, precision=prec, identity=True)
    opt.step(LR)
    Mb, Wb = M0.clone(), W0.clone()
    hm.himuon_stream_step(Mb.data_ptr(), G.data_ptr(), Wb.data_ptr(), H * W,
                          hm.BF16 if state == torch.bfloat16 else hm.F32, BETA, LR,
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    opt.close()
    assert torch.equal(Ma.view(torch.int16 if state == torch.bfloat16 else torch.int32),
                       Mb.view(torch.int16 if state == torch.bfloat16 else torch.int32))
    assert torch.equal(Wa.view(torch.int32), Wb.view(torch.int32))


def test_stream_step_rejects_bad_arguments():
    _need_gpu()
    x = torch.zeros(16, device=DEV)
    p = x.data_ptr()
    for args in [(p, p, p, -1, hm.F32, BETA, LR), (0, p, p, 4, hm.F32, BETA, LR), (p, p, p, 4, 7, BETA, LR),
                 (p, p, p, 4, hm.F32, float("nan"), LR), (p, p, p, 4, hm.F32, BETA, float("inf"))]:
        with pytest.raises(hm.HiMuonError):
            hm.himuon_stream_step(*args, 0)
    hm.himuon_stream_step(0, 0, 0, 0, hm.F32, BETA, LR, 0)   # n = 0: nothing to do

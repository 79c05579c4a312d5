"""himuon_step enqueues only (no allocation, no wait), so a step can be captured into a
HIP graph and replayed (MI355X only).  Each replay is checked bit for bit against the
same step run eagerly from the same state, with unrelated eager work and host
synchronisations between the replays; and a step on a side stream against the oracle.
The graph holds only the library's kernel launches (no memset nodes)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
SHAPES = [(768, 2304), (3072, 768), (512, 512)]
LR = 0.02


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _state(seed):
    out = []
    for i, (h, w) in enumerate(SHAPES):
        W = synth.weights(h, w, seed + i, "cuda")
        M = (0.5 * synth.power_law_matrix(h, w, seed + 10 + i, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
        G = synth.power_law_matrix(h, w, seed + 20 + i, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        out.append((W, M, G))
    return out


def _copy_into(dst, src):
    for (Wd, Md, Gd), (Ws, Ms, Gs) in zip(dst, src):
        Wd.copy_(Ws)
        Md.copy_(Ms)
        Gd.copy_(Gs)


@pytest.mark.parametrize("T,prec", [(128, hm.PREC_BF16F8), (64, hm.PREC_BF16X3), (256, hm.PREC_BF16X3),
                                    (0, hm.PREC_BF16X3)])
def test_captured_step_replays_like_eager_steps(T, prec):
    _need_gpu()
    init = _state(900)
    steps = 4
    # eager reference: `steps` steps from the initial state, state after each
    ref_layers = [tuple(x.clone() for x in l) for l in init]
    opt = hm.HiMuon(ref_layers, T, 5, hm.QUINTIC, precision=prec)
    want = []
    for _ in range(steps):
        opt.step(LR)
        torch.cuda.synchronize()
        want.append([(W.clone(), M.clone()) for W, M, _ in ref_layers])
    opt.close()

    layers = [tuple(x.clone() for x in l) for l in init]
    g_opt = hm.HiMuon(layers, T, 5, hm.QUINTIC, precision=prec)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g_opt.step(LR)                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _copy_into(layers, init)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_opt.step(LR)
    assert g_opt.runtime_counts()["device_allocs"] == 1   # the plan's tables, nothing since
    scratch = torch.zeros(1 << 20, device="cuda")
    for k in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        for (W, M, _), (Wr, Mr) in zip(layers, want[k]):
            assert torch.equal(W.view(torch.int32), Wr.view(torch.int32)), k
            assert torch.equal(M.view(torch.int16), Mr.view(torch.int16)), k
        scratch.add_(1.0)                                 # unrelated eager work between replays
        torch.cuda.synchronize()
    del graph
    g_opt.close()


def test_step_on_a_side_stream_follows_the_oracle():
    _need_gpu()
    layers = _state(950)
    U = [torch.full(W.shape, float("nan"), device="cuda") for W, _, _ in layers]
    M0 = [M.float().cpu().numpy() for _, M, _ in layers]
    G0 = [G.float().cpu().numpy() for _, _, G in layers]
    opt = hm.HiMuon([l + (u,) for l, u in zip(layers, U)], 128, 5, hm.QUINTIC, precision=hm.PREC_BF16F8)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        opt.step(LR)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    opt.close()
    for (W, M, G), u, m0, g0 in zip(layers, U, M0, G0):
        want_m = oracle.momentum_stored(m0, g0, 0.95, "bf16")
        assert np.array_equal(M.float().cpu().numpy(), want_m)
        O = oracle.tiled_ns(want_m.astype(np.float64), 128, 5, oracle.COEFFS_QUINTIC)
        d = u.double().cpu().numpy() - O
        assert np.abs(d).max() <= 2e-2 and np.linalg.norm(d) / np.linalg.norm(O) <= 1e-2

"""himuon_step_static (the step with its workspace in the library's static per-device
array, for callers that cannot allocate) against himuon_step with a caller workspace, on
the same inputs, through the C ABI: two calls in a row, the second on a smaller input,
each bit-identical to the existing entry point and inside the oracle's bf16 bar
(MI355X only)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
Q = oracle.COEFFS_QUINTIC


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make(shapes, seed):
    Gs = [synth.power_law_matrix(h, w, seed + i, dtype=torch.float32).to(torch.bfloat16).cuda()
          for i, (h, w) in enumerate(shapes)]
    Ws = [synth.weights(h, w, seed + 50 + i, "cuda") for i, (h, w) in enumerate(shapes)]
    Ms = [0.5 * g.clone() for g in Gs]
    Us = [torch.full(g.shape, float("nan"), device="cuda") for g in Gs]
    return Ws, Ms, Gs, Us


def copies(state):
    return [[t.clone() for t in ts] for ts in state]


def plan_of(state, T, budget):
    Ws, Ms, Gs, Us = state
    layers = [hm.layer_from_tensors(w, m, g, u) for w, m, g, u in zip(Ws, Ms, Gs, Us)]
    cfg = hm.make_config(T, 5, Q, 0.95, 1e-7, budget, hm.BF16, hm.PREC_BF16X3, hm.FLAG_WRITE_UPDATE)
    return hm.himuon_plan(layers, cfg), layers


def run_pair(shapes, T, seed, budget):
    """One step through himuon_step (caller workspace) and one through himuon_step_static
    on identical copies of the inputs; returns both states after the step."""
    a = make(shapes, seed)
    b = copies(a)
    M0 = [m.float().cpu().numpy() for m in a[1]]
    pa, la = plan_of(a, T, budget)
    pb, lb = plan_of(b, T, budget)
    try:
        need = hm.himuon_workspace_size(pa)
        assert 0 < need <= hm.STATIC_WORKSPACE_BYTES, need
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        hm.himuon_step(pa, ws.data_ptr(), need, 0.02, stream)
        before = hm.himuon_plan_runtime_counts(pb)
        hm.himuon_step_static(pb, 0.02, stream)
        torch.cuda.synchronize()
        assert hm.himuon_plan_runtime_counts(pb) == before      # no allocation, no wait
    finally:
        hm.himuon_plan_destroy(pa)
        hm.himuon_plan_destroy(pb)
    for x, y in zip(a, b):
        for s, t in zip(x, y):
            assert torch.equal(s, t)                              # bit for bit, W, M, G and O
    for m0, g, m, u in zip(M0, a[2], a[1], a[3]):
        assert np.array_equal(m.float().cpu().numpy(),
                              oracle.momentum_stored(m0, g.float().cpu().numpy(), 0.95, "bf16"))
        O = oracle.tiled_ns(m.double().cpu().numpy(), T, 5, Q)
        d = u.double().cpu().numpy() - O
        assert np.abs(d).max() <= 2e-2 and np.linalg.norm(d) / np.linalg.norm(O) <= 1e-2
    return need


def test_static_step_matches_step_on_two_calls_smaller_second():
    _need_gpu()
    # first call: 256-tiles and ragged large tiles, in several chunks under a 16 MiB budget
    n1 = run_pair([(520, 610), (300, 170), (700, 900)], 256, 800, 16 << 20)
    # second call, smaller: one 300 x 400 matrix at FULL
    n2 = run_pair([(300, 400)], 0, 900, 16 << 20)
    assert n2 < n1


def test_static_step_refuses_a_workspace_beyond_its_size():
    _need_gpu()
    state = make([(4096, 4096)], 950)
    p, _ = plan_of(state, 0, 1 << 30)
    try:
        assert hm.himuon_workspace_size(p) > hm.STATIC_WORKSPACE_BYTES
        st = hm._lib.himuon_step_static(p, ctypes.c_float(0.02), None)
        assert st == -2 and "static workspace" in hm.himuon_last_error()
    finally:
        hm.himuon_plan_destroy(p)


def test_static_step_without_workspace_is_the_plain_step():
    _need_gpu()
    a = make([(300, 170), (128, 512)], 960)
    b = copies(a)
    pa, _ = plan_of(a, 128, 1 << 30)
    pb, _ = plan_of(b, 128, 1 << 30)
    try:
        assert hm.himuon_workspace_size(pa) == 0
        stream = torch.cuda.current_stream().cuda_stream
        hm.himuon_step(pa, 0, 0, 0.02, stream)
        hm.himuon_step_static(pb, 0.02, stream)
        torch.cuda.synchronize()
    finally:
        hm.himuon_plan_destroy(pa)
        hm.himuon_plan_destroy(pb)
    for x, y in zip(a, b):
        for s, t in zip(x, y):
            assert torch.equal(s, t)

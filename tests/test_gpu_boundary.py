"""The C-ABI step contract on the GPU: himuon_step enqueues work only (no allocation,
no host wait), a tile-size change uploads its tables stream-ordered into the plan's
second buffer, and every step computes what the oracle computes for the T it was
enqueued with (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
Q = oracle.COEFFS_QUINTIC
SHAPES = [(300, 170), (520, 610), (130, 700)]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make_layers(seed):
    Gs = [synth.power_law_matrix(h, w, seed + i, dtype=torch.float32).to(torch.bfloat16).cuda()
          for i, (h, w) in enumerate(SHAPES)]
    Ms = [torch.zeros_like(g) for g in Gs]
    Ws = [torch.zeros(g.shape, dtype=torch.float32, device="cuda") for g in Gs]
    Us = [torch.zeros(g.shape, dtype=torch.float32, device="cuda") for g in Gs]
    return Gs, Ms, Ws, Us


def check_step(opt, Gs, Ms, Us, T, prec):
    pre = [m.cpu().clone() for m in Ms]
    opt.step(0.02)
    torch.cuda.synchronize()
    for g, m0, m, u in zip(Gs, pre, Ms, Us):
        want_m = oracle.momentum_stored(m0.float().numpy(), g.cpu().float().numpy(), 0.95, "bf16")
        assert np.array_equal(m.cpu().float().numpy(), want_m)
        O = oracle.tiled_ns(m.cpu().double().numpy(), T, 5, Q)
        d = u.cpu().double().numpy() - O
        assert np.abs(d).max() <= 2e-2 and np.linalg.norm(d) / np.linalg.norm(O) <= 1e-2, T


@pytest.mark.parametrize("prec", [hm.PREC_BF16X3, hm.PREC_BF16F8])
def test_steps_allocate_nothing_across_a_tile_schedule(prec):
    _need_gpu()
    Gs, Ms, Ws, Us = make_layers(900)
    opt = hm.HiMuon(list(zip(Ws, Ms, Gs, Us)), 64, 5, Q, precision=prec, workspace_budget=1 << 30)
    try:
        c0 = opt.runtime_counts()
        # himuon_plan made the device tables and uploaded them with one blocking copy
        assert c0 == {"device_allocs": 1, "host_allocs": 0, "host_waits": 1}
        schedule = [64, 128, 256, 0, 64, 128, 256, 0, 64]
        seen = []
        for i, T in enumerate(schedule):
            if i:
                opt.set_tile_schedule(T)
            before = opt.runtime_counts()
            for _ in range(2):
                check_step(opt, Gs, Ms, Us, T, prec)
            # steps make no runtime calls of their own
            assert opt.runtime_counts() == before, T
            seen.append(before)
        # the second pass over the schedule finds both buffers large enough: no allocation
        assert seen[-1]["device_allocs"] == seen[4]["device_allocs"]
        assert seen[-1]["host_allocs"] == seen[4]["host_allocs"]
    finally:
        opt.close()


def test_back_to_back_schedule_changes_take_the_last_tile_size():
    # two changes without a step between them: the step after them runs the last T, the
    # steps queued before them keep theirs (stream order on one stream)
    _need_gpu()
    Gs, Ms, Ws, Us = make_layers(950)
    opt = hm.HiMuon(list(zip(Ws, Ms, Gs, Us)), 128, 5, Q, precision=hm.PREC_BF16X3)
    try:
        check_step(opt, Gs, Ms, Us, 128, hm.PREC_BF16X3)
        opt.set_tile_schedule(64)
        opt.set_tile_schedule(256)
        check_step(opt, Gs, Ms, Us, 256, hm.PREC_BF16X3)
        # enqueue a step at 256, a change to 64 and a step at 64 with no host sync between
        s = torch.cuda.current_stream()
        U256 = None
        opt.step(0.02, s)
        U256 = [u.clone() for u in Us]            # stream-ordered copy of the 256 result
        M256 = [m.clone() for m in Ms]
        opt.set_tile_schedule(64, s)
        opt.step(0.02, s)
        torch.cuda.synchronize()
        for m, u in zip(M256, U256):
            O = oracle.tiled_ns(m.cpu().double().numpy(), 256, 5, Q)
            assert np.abs(u.cpu().double().numpy() - O).max() <= 2e-2
        for m, u in zip(Ms, Us):
            O = oracle.tiled_ns(m.cpu().double().numpy(), 64, 5, Q)
            assert np.abs(u.cpu().double().numpy() - O).max() <= 2e-2
    finally:
        opt.close()

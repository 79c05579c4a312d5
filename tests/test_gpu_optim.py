"""torch.optim integration on the GPU (MI355X only): the optimizer's HiMuon update is
the library step itself and follows the fp64 oracle step by step over a tile-size
schedule, per-group learning rates and a state_dict round trip keep their meaning, and a
small synthetic regression trains."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
from tiled_newton_schulz_tile_amd.optim import HiMuonOptimizer, TileSchedule  # noqa: E402


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("prec", [hm.PREC_BF16X3, hm.PREC_BF16F8])
def test_optimizer_step_equals_library_step(prec):
    _need_gpu()
    shapes = [(300, 170), (128, 512), (64, 64)]
    P = [torch.nn.Parameter(synth.weights(h, w, 10 + i, "cuda")) for i, (h, w) in enumerate(shapes)]
    W_ref = [p.detach().clone() for p in P]
    grads = [synth.power_law_matrix(h, w, 20 + i, device="cuda", dtype=torch.float32)
             for i, (h, w) in enumerate(shapes)]
    opt = HiMuonOptimizer(P, lr=0.02, tile=64, precision=prec)
    M_ref = [torch.zeros(h, w, dtype=torch.bfloat16, device="cuda") for h, w in shapes]
    G_ref = [torch.zeros_like(m) for m in M_ref]
    ref = hm.HiMuon(list(zip(W_ref, M_ref, G_ref)), 64, 5, hm.QUINTIC, precision=prec)
    for step in range(3):
        for p, g, gr in zip(P, grads, G_ref):
            p.grad = (1.0 + step) * g
            gr.copy_(p.grad)
        opt.step()
        ref.step(0.02)
    torch.cuda.synchronize()
    for p, w, m in zip(P, W_ref, M_ref):
        assert torch.equal(p.detach(), w)
        assert torch.equal(opt.momentum(p), m)
    opt.close()
    ref.close()


@pytest.mark.parametrize("prec", [hm.PREC_BF16X3, hm.PREC_BF16F8])
def test_optimizer_follows_oracle_over_a_tile_schedule(prec):
    """HiMuonOptimizer over TileSchedule.every([64, 128, 256, FULL], 2): every step is
    compared with oracle.step from the GPU's pre-step state (W, M, and the gradient as the
    optimizer stores it, bf16): momentum bit-exact, W within lr times the bf16 bar."""
    _need_gpu()
    shapes = [(300, 170), (520, 610), (64, 64), (130, 700)]
    P = [torch.nn.Parameter(synth.weights(h, w, 30 + i, "cuda")) for i, (h, w) in enumerate(shapes)]
    sched = TileSchedule.every([64, 128, 256, 0], 2)
    opt = HiMuonOptimizer(P, lr=0.02, tile=sched, precision=prec, workspace_budget=1 << 30)
    lr = 0.02
    for step in range(8):
        T = sched(step)
        grads = [synth.power_law_matrix(h, w, 100 * step + i, device="cuda", dtype=torch.float32)
                 for i, (h, w) in enumerate(shapes)]
        for p, g in zip(P, grads):
            p.grad = g
        W0 = [p.detach().double().cpu().numpy() for p in P]
        M0 = [opt.momentum(p).float().cpu().numpy() if step else np.zeros(p.shape, np.float32) for p in P]
        Gb = [g.to(torch.bfloat16).float().cpu().numpy() for g in grads]
        opt.step()
        torch.cuda.synchronize()
        assert opt._engines[0].stats()["tile"] == T
        for p, w0, m0, gb in zip(P, W0, M0, Gb):
            m = opt.momentum(p).float().cpu().numpy()
            assert np.array_equal(m, oracle.momentum_stored(m0, gb, 0.95, "bf16")), (step, T)
            (w_ref, _, o_ref), = oracle.step([(w0, np.zeros_like(w0), m.astype(np.float64))], T, 5, hm.QUINTIC,
                                             beta=0.0, lr=lr)
            w = p.detach().double().cpu().numpy()
            o = (w0 - w) / lr
            d = o - o_ref
            assert np.abs(d).max() <= 2e-2 and np.linalg.norm(d) / np.linalg.norm(o_ref) <= 1e-2, (step, T)
            assert np.abs(w - w_ref).max() <= lr * 2e-2 + 1e-6
    opt.close()


def test_state_dict_round_trip_resumes_momentum_and_schedule():
    """Three steps, a state_dict, a fresh optimizer over copies of the weights restored
    from it: the next steps match the original optimizer bit for bit (momentum, weights,
    and the tile schedule position)."""
    _need_gpu()
    shapes = [(300, 170), (128, 512)]
    sched = TileSchedule([(0, 64), (4, 128)])
    P = [torch.nn.Parameter(synth.weights(h, w, 50 + i, "cuda")) for i, (h, w) in enumerate(shapes)]
    opt = HiMuonOptimizer(P, lr=0.02, tile=sched)
    grads = [[synth.power_law_matrix(h, w, 60 + 10 * s + i, device="cuda", dtype=torch.float32)
              for i, (h, w) in enumerate(shapes)] for s in range(6)]
    for s in range(3):
        for p, g in zip(P, grads[s]):
            p.grad = g
        opt.step()
    sd = opt.state_dict()
    Q2 = [torch.nn.Parameter(p.detach().clone()) for p in P]
    opt2 = HiMuonOptimizer(Q2, lr=0.02, tile=sched)
    opt2.load_state_dict(sd)
    assert opt2.step_count == 3
    for s in range(3, 6):
        for p, q, g in zip(P, Q2, grads[s]):
            p.grad = g
            q.grad = g.clone()
        opt.step()
        opt2.step()
        torch.cuda.synchronize()
        assert opt2._engines[0].stats()["tile"] == sched(s)
        for p, q in zip(P, Q2):
            assert torch.equal(p.detach(), q.detach())
            assert torch.equal(opt.momentum(p), opt2.momentum(q))
    opt.close()
    opt2.close()


def test_per_group_learning_rates():
    """Two parameter groups with their own lr (and an lr change between steps, as a
    scheduler makes): each weight moves by exactly its group's lr times the HiMuon
    direction of the same momentum."""
    _need_gpu()
    a = torch.nn.Parameter(torch.zeros(256, 384, device="cuda"))
    b = torch.nn.Parameter(torch.zeros(256, 384, device="cuda"))
    opt = HiMuonOptimizer([{"params": [a]}, {"params": [b], "lr": 0.005}], lr=0.02, tile=128)
    g = synth.power_law_matrix(256, 384, 77, device="cuda", dtype=torch.float32)
    for lr_a in (0.02, 0.01):
        opt.param_groups[0]["lr"] = lr_a
        a.grad, b.grad = g, g.clone()
        a0, b0 = a.detach().clone(), b.detach().clone()
        opt.step()
        torch.cuda.synchronize()
        assert torch.equal(opt.momentum(a), opt.momentum(b))
        da, db = (a0 - a.detach()) / lr_a, (b0 - b.detach()) / 0.005
        assert torch.allclose(da, db, atol=1e-4, rtol=0)
    assert len(opt._engines) == 2
    opt.close()


def test_tile_schedule_reaches_the_plan():
    _need_gpu()
    P = [torch.nn.Parameter(torch.zeros(512, 512, device="cuda"))]
    opt = HiMuonOptimizer(P, tile=TileSchedule([(0, 64), (2, 128), (4, 0)]))
    seen = []
    for _ in range(6):
        P[0].grad = torch.randn(512, 512, device="cuda")
        opt.step()
        seen.append(opt._engines[0].stats()["tile"])
    assert seen == [64, 64, 128, 128, 0, 0]
    opt.close()


def test_synthetic_regression_trains():
    """A 3-layer MLP fits a fixed random teacher: HiMuon on the three weight matrices,
    AdamW on the biases; the loss falls below a tenth of its start within 150 steps."""
    _need_gpu()
    torch.manual_seed(0)
    gen = torch.Generator(device="cuda").manual_seed(1)
    teacher = torch.nn.Sequential(torch.nn.Linear(64, 128), torch.nn.Tanh(), torch.nn.Linear(128, 16)).cuda()
    model = torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(), torch.nn.Linear(256, 256),
                                torch.nn.GELU(), torch.nn.Linear(256, 16)).cuda()
    opt = HiMuonOptimizer(model.parameters(), lr=0.02, tile=TileSchedule.every([64, 128], 75),
                          fallback_lr=3e-3)
    losses = []
    for _ in range(150):
        x = torch.randn(512, 64, device="cuda", generator=gen)
        with torch.no_grad():
            y = teacher(x)
        loss = torch.nn.functional.mse_loss(model(x), y)
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(loss.item())
    opt.close()
    start, end = sum(losses[:5]) / 5, sum(losses[-5:]) / 5
    print(f"\nsynthetic regression: loss {start:.4f} -> {end:.4f}")
    assert all(map(lambda v: v == v, losses))
    assert end < 0.1 * start


def test_wrapper_overhead_on_gpt2_stack():
    """Optimizer step (gradient copies + HiMuon + AdamW on nothing) against the bare
    library step on the GPT-2-shaped stack; printed, and bounded loosely."""
    _need_gpu()
    shapes = synth.STACKS["gpt2-small-12L"]
    P = [torch.nn.Parameter(synth.weights(h, w, i, "cuda")) for i, (h, w) in enumerate(shapes)]
    for p in P:
        p.grad = 0.01 * torch.randn(p.shape, device="cuda")
    opt = HiMuonOptimizer(P, tile=128)

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e3

    t_opt = timed(opt.step)
    t_lib = timed(lambda: opt._engines[0].step(0.02))
    print(f"\nGPT-2 stack: optimizer step {t_opt:.3f} ms, library step {t_lib:.3f} ms")
    opt.close()
    assert t_opt < 3 * t_lib + 5.0

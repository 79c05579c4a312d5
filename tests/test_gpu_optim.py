"""torch.optim integration on the GPU (MI355X only): the optimizer's HiMuon update is
the library step itself, the tile-size schedule reaches the plan, and a small synthetic
regression trains."""
import time

import pytest
import torch

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


def test_tile_schedule_reaches_the_plan():
    _need_gpu()
    P = [torch.nn.Parameter(torch.zeros(512, 512, device="cuda"))]
    opt = HiMuonOptimizer(P, tile=TileSchedule([(0, 64), (2, 128), (4, 0)]))
    seen = []
    for _ in range(6):
        P[0].grad = torch.randn(512, 512, device="cuda")
        opt.step()
        seen.append(opt._engine.stats()["tile"])
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
    t_lib = timed(lambda: opt._engine.step(0.02))
    print(f"\nGPT-2 stack: optimizer step {t_opt:.3f} ms, library step {t_lib:.3f} ms")
    opt.close()
    assert t_opt < 3 * t_lib + 5.0

"""Host logic of the torch.optim integration: the tile-size schedule and which
parameters go through HiMuon (no GPU needed)."""
import pytest
import torch

hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
from tiled_newton_schulz_tile_amd.optim import HiMuonOptimizer, TileSchedule, split_params  # noqa: E402


def test_schedule_piecewise_constant():
    s = TileSchedule([(0, 64), (10, 128), (20, 256), (30, 0)])
    assert [s(i) for i in (0, 9, 10, 19, 20, 29, 30, 10 ** 6)] == [64, 64, 128, 128, 256, 256, 0, 0]
    assert TileSchedule(128)(12345) == 128
    e = TileSchedule.every([64, 128, 256, 0], 10)
    assert [e(i) for i in (0, 10, 25, 39, 40, 400)] == [64, 128, 256, 0, 0, 0]


@pytest.mark.parametrize("spec", [[], [(1, 64)], [(0, 64), (0, 128)], [(0, 64), (5, -1)]])
def test_schedule_rejects_bad_specs(spec):
    with pytest.raises(ValueError):
        TileSchedule(spec)


def test_split_params_convention():
    w1 = torch.nn.Parameter(torch.zeros(8, 4))
    b1 = torch.nn.Parameter(torch.zeros(8))
    emb = torch.nn.Parameter(torch.zeros(16, 4))
    frozen = torch.nn.Parameter(torch.zeros(4, 4), requires_grad=False)
    conv = torch.nn.Parameter(torch.zeros(2, 2, 3, 3))
    groups, other = split_params([{"params": [w1, b1, frozen, conv]}, {"params": [emb], "use_himuon": False}],
                                 0.02)
    assert [(lr, [id(p) for p in ps]) for lr, ps in groups] == [(0.02, [id(w1)])]
    assert {id(p) for p in other} == {id(b1), id(conv), id(emb)}
    groups, other = split_params([w1, b1], 0.02)
    assert groups == [(0.02, [w1])] and other == [b1]


def test_split_params_groups_by_learning_rate():
    # a group with its own lr gets its own HiMuon group (and plan); equal lrs share one
    a, b, c = (torch.nn.Parameter(torch.zeros(8, 4)) for _ in range(3))
    groups, other = split_params([{"params": [a]}, {"params": [b], "lr": 0.01}, {"params": [c], "lr": 0.02}],
                                 0.02)
    assert [(lr, [id(p) for p in ps]) for lr, ps in groups] == [(0.02, [id(a), id(c)]), (0.01, [id(b)])]
    assert other == []


def test_optimizer_refuses_host_parameters():
    with pytest.raises(ValueError):
        HiMuonOptimizer([torch.nn.Parameter(torch.zeros(8, 8))])
    with pytest.raises(ValueError):
        HiMuonOptimizer([torch.nn.Parameter(torch.zeros(8))])

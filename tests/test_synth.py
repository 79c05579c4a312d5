"""The seeded input recipe: power-law spectrum plus Gaussian noise, Haar factors."""
import torch

import synth


def test_haar_columns_orthonormal_and_seeded():
    g = torch.Generator().manual_seed(3)
    U = synth.haar_columns(50, 20, g, "cpu", torch.float64)
    assert torch.allclose(U.T @ U, torch.eye(20, dtype=torch.float64), atol=1e-12)
    g2 = torch.Generator().manual_seed(3)
    assert torch.equal(U, synth.haar_columns(50, 20, g2, "cpu", torch.float64))


def test_power_law_spectrum_without_noise():
    G = synth.power_law_matrix(40, 60, 0, noise=0.0)
    s = torch.linalg.svdvals(G)
    want = 1.0 / torch.arange(1, 41, dtype=torch.float64)
    assert torch.allclose(s, want, atol=1e-12)


def test_noise_level_and_dtype():
    G = synth.power_law_matrix(256, 512, 0, dtype=torch.float32)
    assert G.dtype == torch.float32 and G.shape == (256, 512)
    Gn = synth.power_law_matrix(256, 512, 0, noise=0.0)
    resid = G.double() - Gn
    assert abs(resid.std().item() - 0.01) < 5e-4


def test_stack_shapes_and_ragged_draw():
    assert len(synth.STACKS["llama3-8b-32L"]) == 224
    assert sum(h * w for h, w in synth.STACKS["llama3-8b-32L"]) == 6979321856
    assert sum(h * w for h, w in synth.STACKS["gpt2-small-12L"]) == 84934656
    assert sum(h * w for h, w in synth.STACKS["decoder-1b-16L"]) == 1073741824
    rs = synth.ragged_shapes()
    assert len(rs) == 24 and rs == synth.ragged_shapes()
    assert all(100 <= h <= 6000 and 100 <= w <= 6000 and h % 32 and w % 32 for h, w in rs)


def test_stack_inputs_shared_factors():
    ins = synth.stack_inputs([(30, 50), (50, 30), (30, 50)], 10, share_factors=True,
                             state_dtype=torch.float32)
    assert [t[2].shape for t in ins] == [(30, 50), (50, 30), (30, 50)]
    assert all((t[1] == 0).all() for t in ins)
    assert not torch.equal(ins[0][2], ins[2][2])  # noise differs per matrix

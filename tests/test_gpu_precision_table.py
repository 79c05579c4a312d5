"""Accuracy of each arithmetic scheme of the HIP path against the fp64 oracle, per
(T, K, coefficients) cell, on a GPT-2-shaped layer of power-law matrices.  The table is
printed (run with -s); the assertions pin which cells meet the bars:
fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and relative Frobenius <= 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
Q, C = oracle.COEFFS_QUINTIC, oracle.COEFFS_CUBIC
SHAPES = [(768, 2304), (3072, 768)]
_cache = {}


def run(T, K, coeffs, prec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    state = torch.float32 if prec == hm.PREC_F32 else torch.bfloat16
    mats = [synth.power_law_matrix(h, w, 2000 + i, dtype=torch.float32) for i, (h, w) in enumerate(SHAPES)]
    layers = []
    for g in mats:
        G = g.to(state).cuda()
        layers.append((torch.zeros(g.shape, device="cuda"), torch.zeros_like(G), G,
                       torch.zeros(g.shape, device="cuda")))
    opt = hm.HiMuon(layers, T, K, coeffs, precision=prec)
    opt.step(0.02)
    torch.cuda.synchronize()
    opt.close()
    worst = [0.0, 0.0]
    for (_, M, _, U) in layers:
        key = (T, K, coeffs, state)
        Mn = M.double().cpu().numpy()
        O = oracle.tiled_ns(Mn, T, K, coeffs)
        d = U.double().cpu().numpy() - O
        worst[0] = max(worst[0], float(np.abs(d).max()))
        worst[1] = max(worst[1], float(np.linalg.norm(d) / np.linalg.norm(O)))
        del key
    return worst


CELLS = [(T, K, co) for T in (32, 64, 128, 256) for K in (5, 8) for co in ("quintic", "cubic")]


@pytest.mark.parametrize("T,K,co", CELLS)
def test_precision_cell(T, K, co):
    coeffs = Q if co == "quintic" else C
    row = {}
    for name, prec in (("f32", hm.PREC_F32), ("bf16x3", hm.PREC_BF16X3), ("bf16f8", hm.PREC_BF16F8),
                       ("bf16", hm.PREC_BF16)):
        row[name] = run(T, K, coeffs, prec)
    print(f"\nPRECISION T={T} K={K} {co}: " +
          "  ".join(f"{n}: max-abs {v[0]:.2e} rel-F {v[1]:.2e}" for n, v in row.items()), flush=True)
    assert row["f32"][0] <= 1e-4
    assert row["bf16x3"][0] <= 2e-2 and row["bf16x3"][1] <= 1e-2
    assert row["bf16f8"][0] <= 2e-2 and row["bf16f8"][1] <= 1e-2
    if co == "cubic":
        assert row["bf16"][0] <= 2e-2 and row["bf16"][1] <= 1e-2

"""Matrix-function diagnostics from the HIP path against the oracle's (MI355X only).

The same definitions (deviation from the FULL map, singular values, alignment with the
polar factor) evaluated on O_T from the kernels and on the fp64 oracle's O_T, for the
same stored momentum.  Bars follow the arithmetic of the path: fp32 within 1e-4,
bf16x3 within 2e-3 (values of order one)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import diagnostics as odg

pytestmark = pytest.mark.gpu
hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
dg = pytest.importorskip("tiled_newton_schulz_tile_amd.diagnostics")
Q, C = oracle.COEFFS_QUINTIC, oracle.COEFFS_CUBIC


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # (H, W, state dtype, precision, tiles, coefficients, bar)
    (256, 512, torch.float32, hm.PREC_F32, [32, 64, 128, 0], Q, 1e-4),
    (512, 512, torch.bfloat16, hm.PREC_BF16X3, [32, 64, 128, 256, 0], Q, 2e-3),
    (1024, 256, torch.bfloat16, hm.PREC_BF16X3, [64, 128, 200, 0], C, 2e-3),
]


@pytest.mark.parametrize("H,W,state,prec,tiles,coeffs,bar", CASES)
def test_diagnostics_match_oracle(H, W, state, prec, tiles, coeffs, bar):
    _need_gpu()
    M = synth.power_law_matrix(H, W, 61, dtype=torch.float32).to(state)
    got = dg.report(M.cuda(), tiles, 5, coeffs, precision=prec)
    want = odg.report(M.double().numpy(), tiles, 5, coeffs)
    for T in tiles:
        g, w = got[T], want[T]
        assert abs(g["deviation"] - w["deviation"]) <= bar, (T, g["deviation"], w["deviation"])
        assert abs(g["alignment"] - w["alignment"]) <= bar, (T, g["alignment"], w["alignment"])
        assert abs(g["cosine"] - w["cosine"]) <= bar, (T, g["cosine"], w["cosine"])
        assert abs(g["dual_alignment"] - w["dual_alignment"]) <= bar, T
        assert np.abs(g["spectrum"] - w["spectrum"]).max() <= bar, T
    assert got[0]["deviation"] == 0.0


def test_ns_output_rejects_host_tensor():
    with pytest.raises(ValueError):
        dg.ns_output(torch.zeros(4, 4), 2)

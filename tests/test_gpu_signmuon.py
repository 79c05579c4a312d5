"""Sign-Muon local kernels against the oracle (MI355X only): packing and voting bit for
bit, and the whole local step (direction, sign, vote, update) end to end."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import signmuon as osm

pytestmark = pytest.mark.gpu
hm = pytest.importorskip("tiled_newton_schulz_tile_amd")
sm = pytest.importorskip("tiled_newton_schulz_tile_amd.signmuon")
Q = oracle.COEFFS_QUINTIC


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("rows,cols,ld", [(1, 1, 1), (3, 7, 7), (8, 8, 8), (65, 33, 40), (300, 170, 170),
                                          (1, 1000, 1000), (513, 129, 256)])
def test_pack_bit_exact(rows, cols, ld):
    _need_gpu()
    g = torch.Generator().manual_seed(rows * 1000 + cols)
    base = torch.randn(rows, ld, generator=g)
    base[torch.rand(rows, ld, generator=g) < 0.05] = 0.0
    base[torch.rand(rows, ld, generator=g) < 0.05] = -0.0
    O = base.cuda()[:, :cols]
    bits = sm.sign_pack(O)
    torch.cuda.synchronize()
    want = osm.pack(osm.sign(base[:, :cols].numpy()))
    got = bits.cpu().numpy()
    assert np.array_equal(got[:want.size], want)
    assert not got[want.size:].any()          # padding bytes untouched (zero)


@pytest.mark.parametrize("workers", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n", [1, 31, 32, 33, 1000, 100003])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_vote_bit_exact(workers, n, dtype):
    _need_gpu()
    rng = np.random.default_rng(workers * 7 + n)
    nb = sm.packed_bytes(n)
    bufs = np.zeros((workers, nb), dtype=np.uint8)
    for m in range(workers):
        bufs[m, :(n + 7) // 8] = osm.pack(np.where(rng.random(n) < 0.5, -1, 1))
    out = sm.sign_vote(torch.from_numpy(bufs).cuda(), n, dtype, scale=0.5)
    torch.cuda.synchronize()
    want = 0.5 * osm.vote(list(bufs[:, :(n + 7) // 8]), n).astype(np.float32)
    assert np.array_equal(out.float().cpu().numpy(), want)


def test_local_step_identity_update_single_and_many_workers():
    _need_gpu()
    shapes = [(300, 170), (128, 256)]
    Gs = [synth.power_law_matrix(h, w, 70 + i, device="cuda", dtype=torch.float32).to(torch.bfloat16)
          for i, (h, w) in enumerate(shapes)]
    Ms = [torch.zeros_like(g) for g in Gs]
    Ws = [synth.weights(h, w, 80 + i, "cuda") for i, (h, w) in enumerate(shapes)]
    W0 = [w.clone() for w in Ws]
    opt = sm.SignMuonLocal(list(zip(Ws, Ms, Gs)), 64)
    lr = 0.01
    lr32 = float(np.float32(lr))     # the kernels take lr as float32
    # one worker: S_bar = sign(O)
    bits = opt.step(lr)
    torch.cuda.synchronize()
    for i, (w0, w, U, M) in enumerate(zip(W0, Ws, opt.U, Ms)):
        S = osm.sign(U.cpu().numpy())
        assert np.array_equal(bits[i].cpu().numpy()[:(U.numel() + 7) // 8], osm.pack(S))
        want = (w0.double() - lr32 * torch.from_numpy(S).double().cuda()).float()
        assert (w.view(torch.int32) - want.view(torch.int32)).abs().max().item() <= 1
        # the direction is the tiled map of the stored momentum: signs agree with the
        # oracle wherever the oracle's entry is not within the bf16x3 error of zero
        O = oracle.tiled_ns(M.double().cpu().numpy(), 64, 5, Q)
        sure = np.abs(O) > 1e-3
        assert np.array_equal(S[sure], osm.sign(O)[sure])
    # two more workers with random signs: S_bar is the vote of the three
    W1 = [w.clone() for w in Ws]
    rng = np.random.default_rng(3)
    others = []
    for n in opt.n:
        o = np.zeros((2, sm.packed_bytes(n)), dtype=np.uint8)
        for m in range(2):
            o[m, :(n + 7) // 8] = osm.pack(np.where(rng.random(n) < 0.5, -1, 1))
        others.append(o)
    bits = opt.step(lr, [torch.from_numpy(o).cuda() for o in others])
    torch.cuda.synchronize()
    for i, (w1, w) in enumerate(zip(W1, Ws)):
        n = opt.n[i]
        own = bits[i].cpu().numpy()[:(n + 7) // 8]
        Sbar = osm.vote([own] + list(others[i][:, :(n + 7) // 8]), n).reshape(w.shape)
        want = (w1.double() - lr32 * torch.from_numpy(Sbar).double().cuda()).float()
        assert (w.view(torch.int32) - want.view(torch.int32)).abs().max().item() <= 1
    opt.close()


def test_local_step_with_local_polar():
    _need_gpu()
    shapes = [(256, 384)]
    Gs = [synth.power_law_matrix(h, w, 90, device="cuda", dtype=torch.float32).to(torch.bfloat16)
          for h, w in shapes]
    Ms = [torch.zeros_like(g) for g in Gs]
    Ws = [synth.weights(h, w, 91, "cuda") for h, w in shapes]
    W0 = [w.clone() for w in Ws]
    opt = sm.SignMuonLocal(list(zip(Ws, Ms, Gs)), 128, polar_tile=128)
    lr = 0.02
    opt.step(lr)
    torch.cuda.synchronize()
    Sbar = opt.sbar[0].double().cpu().numpy()
    O = oracle.tiled_ns(Sbar, 128, 5, Q)
    got = (W0[0].double() - Ws[0].double()).cpu().numpy() / lr
    assert np.abs(got - O).max() <= 2e-2
    assert np.linalg.norm(got - O) / np.linalg.norm(O) <= 1e-2
    opt.close()


def test_pack_and_vote_reject_bad_arguments():
    _need_gpu()
    with pytest.raises(hm.HiMuonError):
        hm.himuon_sign_pack(0, 4, 4, 4, 0, 0)
    b = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(hm.HiMuonError):
        hm.himuon_sign_vote(b.data_ptr(), 0, 16, 8, hm.F32, b.data_ptr(), 1.0, 0)
    with pytest.raises(hm.HiMuonError):
        hm.himuon_sign_vote(b.data_ptr(), 1, 6, 8, hm.F32, b.data_ptr(), 1.0, 0)

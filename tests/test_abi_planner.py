"""C-ABI library on the CPU: it loads, exports every entry point of include/himuon.h,
and its planner (host code only, no device calls) builds the same tile table as the
oracle, bit for bit, with the oracle's flop and byte counts."""
import os
import re
import subprocess

import pytest

import oracle
import synth
import tiled_newton_schulz_tile_amd as hm

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "himuon.h")
FAKE = 1 << 32  # device addresses are not touched by the planner


def declared_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"HIMUON_API\s+[\w\s\*]*?\b(himuon_\w+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = declared_entry_points()
    assert names == sorted(hm.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", hm.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
    # the library's own C++ internals stay hidden
    assert all(not e.startswith("_ZN6himuon") for e in exported)


def fake_layers(shapes, write_update=False):
    out = []
    for i, (H, W) in enumerate(shapes):
        base = FAKE * (i + 1)
        out.append(hm.himuon_layer(H, W, W, W, W, W if write_update else 0,
                                   base, base + (1 << 30), base + (2 << 30),
                                   base + (3 << 30) if write_update else None))
    return out


def plan_for(shapes, T, **kw):
    cfg = hm.make_config(T, **kw)
    return hm.himuon_plan(fake_layers(shapes, kw.get("flags", 0) & 1), cfg)


@pytest.mark.parametrize("shapes,T", [
    ([(256, 512)], 64), ([(256, 512)], 128), ([(256, 512)], 512), ([(256, 512)], 0),
    ([(250, 500), (37, 53), (130, 70)], 64), ([(97, 131)], 32), ([(300, 170)], 100),
    ([(5, 3), (1, 1), (0, 7)], 2), ([(768, 2304), (3072, 768)], 128),
])
def test_tile_table_equals_oracle(shapes, T):
    p = plan_for(shapes, T)
    try:
        got = hm.himuon_plan_tiles(p)
        want = [(li, int(h > w), r0, c0, h, w) for li, (H, W) in enumerate(shapes)
                for r0, c0, h, w in oracle.tiles(H, W, T)]
        assert got == want
    finally:
        hm.himuon_plan_destroy(p)


@pytest.mark.parametrize("name,T", [("single-256x512", 64), ("gpt2-small-12L", 128),
                                    ("decoder-1b-16L", 32), ("llama3-8b-32L", 128)])
@pytest.mark.parametrize("coeffs", [hm.QUINTIC, hm.CUBIC])
def test_stats_match_oracle_counts(name, T, coeffs):
    shapes = synth.STACKS[name]
    p = plan_for(shapes, T, coeffs=coeffs, steps=5)
    try:
        st = hm.himuon_plan_stats(p)
        assert st["tiles"] == sum(len(oracle.tiles(H, W, T)) for H, W in shapes)
        assert st["ns_flops"] == oracle.ns_flops(shapes, T, 5, coeffs)
        assert st["step_bytes"] == oracle.step_bytes(shapes, 2)
        assert st["fused_tiles"] == st["tiles"] and st["gemm_tiles"] == 0
        assert st["workspace_bytes"] == 0 and hm.himuon_workspace_size(p) == 0
        assert st["kernel_tile"] == (32 if T <= 32 else 64 if T <= 64 else 128)
    finally:
        hm.himuon_plan_destroy(p)


def test_identity_flag_accepted_with_and_without_update():
    for flags in (hm.FLAG_IDENTITY_MAP, hm.FLAG_IDENTITY_MAP | hm.FLAG_WRITE_UPDATE):
        p = plan_for([(300, 170), (64, 64)], 128, flags=flags)
        hm.himuon_plan_destroy(p)


def test_llama_stack_tile_count_and_work():
    p = plan_for(synth.STACKS["llama3-8b-32L"], 128)
    st = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st["tiles"] == 425984
    assert st["ns_flops"] == 6 * 6979321856 * 128 * 5
    # BF16X3 issues three bf16 products per product; the two symmetric products run on
    # 10 of the 16 32x32 blocks of a 128-tile: 3 * (2 * 10/16 + 1) / 3 = 2.25x the work
    assert st["issued_flops"] == 2.25 * st["ns_flops"]


def test_bf16f8_issues_one_bf16_and_two_half_rate_products():
    p = plan_for(synth.STACKS["llama3-8b-32L"], 128, precision=hm.PREC_BF16F8)
    st = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st["ns_flops"] == 6 * 6979321856 * 128 * 5
    # hi*hi in bf16 plus two e4m3 products at twice the rate: 2 bf16-product units per
    # product (units of 2 T^3 flops), on 10 of 16 blocks for the symmetric ones; on full
    # 128-tiles the Gram and update products of step 0 and the square product of steps 0
    # and 1 are plain bf16 (1 unit):
    #   steps 0, 1: 10/16 * 1 + 10/16 * 1 + 1 = 2.25, steps 2..4: 10/16 * 2 * 2 + 2 = 4.5
    assert st["issued_flops"] == (2 * 2.25 + 3 * 4.5) * 2 * 128 ** 3 * 425984
    # full 64-tiles: plain Gram in step 0 and plain square in steps 0 and 1 (3 of 4 blocks)
    p = plan_for(synth.STACKS["llama3-8b-32L"], 64, precision=hm.PREC_BF16F8)
    st64 = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st64["issued_flops"] == (3.5 + 4.25 + 3 * 5.0) * 2 * 64 ** 3 * (6979321856 // 64 ** 2)
    # ragged tiles take every correction product: 2 units per product in every step
    p = plan_for([(100, 200)], 128, precision=hm.PREC_BF16F8)
    str_ = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert str_["issued_flops"] == 2 * 5 * (2 * 10 / 16 * 2 + 2) * 2 * 128 ** 3
    # edge-32 tiles run the bf16x3 products
    p = plan_for([(256, 512)], 32, precision=hm.PREC_BF16F8)
    st32 = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    p = plan_for([(256, 512)], 32, precision=hm.PREC_BF16X3)
    assert st32["issued_flops"] == hm.himuon_plan_stats(p)["issued_flops"]
    hm.himuon_plan_destroy(p)


def test_256_tile_chunks_and_work():
    # Tiles of exactly 256 x 256 with bf16 planes run each product as one workgroup per
    # tile over the whole 256 x 256 output, so the symmetric products issue all four
    # 128-blocks: three bf16 products (bf16x3) of 2 * 256^3 per product, Gram + square +
    # update = 3x the algorithmic work of the quintic step
    p = plan_for(synth.STACKS["llama3-8b-32L"], 256, precision=hm.PREC_BF16X3)
    st = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st["tiles"] == st["gemm_tiles"] == 6979321856 // 256 ** 2
    assert st["ns_flops"] == 6 * 6979321856 * 256 * 5
    assert st["issued_flops"] == 3 * st["ns_flops"]
    # bf16f8 requests run the same products, with the Gram of step 0 and the square of
    # steps 0 and 1 on the hi operands alone (one bf16 product instead of three):
    # (1 + 1 + 3) + (3 + 1 + 3) + 3 * (3 + 3 + 3) = 39 units of 2 * 256^3 per tile, not 45
    p = plan_for(synth.STACKS["llama3-8b-32L"], 256, precision=hm.PREC_BF16F8)
    st8 = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st8["issued_flops"] == 39 * 2 * 256 ** 3 * (6979321856 // 256 ** 2)
    # fp32 keeps the 128-block kernel: upper blocks of the symmetric products (3 of 4)
    p = plan_for(synth.STACKS["llama3-8b-32L"], 256, precision=hm.PREC_F32)
    st = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st["issued_flops"] == 5 * (0.75 * 2 + 0.75 * 2 + 2) * 256 ** 3 * (6979321856 // 256 ** 2)
    # chunks are cut where the kind changes: 512x512 and the two full tiles of 300x600
    # (6 tiles of 256), then its three ragged tiles of the large-tile path (256x88 and
    # two 44x256; its 44x88 tile goes to the fused kernel), then 256x256 again
    shapes = [(512, 512), (300, 600), (256, 256)]
    for prec, chunks in ((hm.PREC_BF16X3, 3), (hm.PREC_BF16, 3), (hm.PREC_BF16F8, 3), (hm.PREC_F32, 1)):
        p = plan_for(shapes, 256, precision=prec)
        st = hm.himuon_plan_stats(p)
        hm.himuon_plan_destroy(p)
        assert (st["tiles"], st["gemm_tiles"], st["chunks"]) == (11, 10, chunks), prec


def test_256_block_issued_work_at_full():
    # every side of the 8B stack is a multiple of 256: the products run in 256-blocks,
    # the symmetric ones (Gram over K = s, square over K = r) on the nb (nb + 1) / 2 upper
    # blocks, the update (K = r) on all nb x (s / 256) blocks; bf16x3 issues 3 products
    shapes = synth.STACKS["llama3-8b-32L"]
    want = 0.0
    for H, W in shapes:
        r, s_ = min(H, W), max(H, W)
        nb, nbs = r // 256, s_ // 256
        sym = nb * (nb + 1) / 2 * 2.0 * 256 * 256
        want += 5 * 3 * (sym * s_ + sym * r + 2.0 * 256 * 256 * nb * nbs * r)
    p = plan_for(shapes, 0, precision=hm.PREC_BF16X3)
    st = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st["gemm_tiles"] == len(shapes)
    assert st["issued_flops"] == pytest.approx(want, rel=1e-12)
    # bf16f8 requests run the same products with the Gram of step 0 and the square of
    # steps 0 and 1 on the hi planes alone (one product each instead of three)
    want8 = 0.0
    for H, W in shapes:
        r, s_ = min(H, W), max(H, W)
        nb, nbs = r // 256, s_ // 256
        sym = nb * (nb + 1) / 2 * 2.0 * 256 * 256
        want8 += (1 + 4 * 3) * sym * s_ + (2 * 1 + 3 * 3) * sym * r + 5 * 3 * 2.0 * 256 * 256 * nb * nbs * r
    p = plan_for(shapes, 0, precision=hm.PREC_BF16F8)
    st8 = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    assert st8["issued_flops"] == pytest.approx(want8, rel=1e-12)
    # a side that is not a multiple of 256 keeps the 128-blocks
    p = plan_for([(4096, 4000)], 0, precision=hm.PREC_BF16X3)
    st = hm.himuon_plan_stats(p)
    hm.himuon_plan_destroy(p)
    # short side r = 4000: 32 block rows, K of the square and the update padded to 4032;
    # long side 4096: 32 block columns, K of the Gram 4096
    nb, nbs = -(-4000 // 128), 4096 // 128
    sym = nb * (nb + 1) / 2 * 2.0 * 128 * 128
    assert st["issued_flops"] == pytest.approx(5 * 3 * (sym * 4096 + sym * 4032 + 2.0 * 128 * 128 * nb * nbs * 4032),
                                               rel=1e-12)


@pytest.mark.parametrize("coeffs,K,ok", [
    (hm.QUINTIC, 5, True), (hm.QUINTIC, 100, True), (hm.CUBIC, 8, True),
    ((2.0, -1.5, 0.5), 6, True), ((10.0, 10.0, 10.0), 5, False), ((3.0, 0.0, 0.0), 200, False),
])
def test_bf16f8_needs_bounded_iterates(coeffs, K, ok):
    # the e4m3 scales come from bounds on the iterates: 10 s + 10 s^3 + 10 s^5 and 3 s
    # grow without bound, so the plan is refused; the shipped presets are bounded
    if ok:
        hm.himuon_plan_destroy(plan_for([(300, 170)], 128, steps=K, coeffs=coeffs, precision=hm.PREC_BF16F8))
    else:
        with pytest.raises(hm.HiMuonError) as e:
            plan_for([(300, 170)], 128, steps=K, coeffs=coeffs, precision=hm.PREC_BF16F8)
        assert e.value.status == -1 and "unbounded" in str(e.value)
        # the other precisions do not depend on the bounds
        hm.himuon_plan_destroy(plan_for([(300, 170)], 128, steps=K, coeffs=coeffs, precision=hm.PREC_BF16X3))


def test_full_and_large_tiles_use_gemm_path_and_chunks():
    shapes = [(4096, 14336), (14336, 4096), (4096, 1024)]
    p = plan_for(shapes, 0, workspace_budget=10 ** 9)
    try:
        st = hm.himuon_plan_stats(p)
        assert st["gemm_tiles"] == 3 and st["fused_tiles"] == 0
        assert st["chunks"] >= 2 and 0 < st["workspace_bytes"] <= 10 ** 9
        assert st["ns_flops"] == oracle.ns_flops(shapes, 0, 5, hm.QUINTIC)
    finally:
        hm.himuon_plan_destroy(p)


def test_budget_too_small_for_one_tile_is_ebudget():
    with pytest.raises(hm.HiMuonError) as e:
        plan_for([(4096, 4096)], 0, workspace_budget=1000)
    assert e.value.status == -2 and "budget" in str(e.value)


def test_set_tile_schedule_rebuilds_table():
    shapes = [(300, 170), (100, 260)]
    p = plan_for(shapes, 64, workspace_budget=10 ** 9)
    try:
        for T in (128, 32, 256, 0, 64):
            hm.himuon_set_tile_schedule(p, T, 0)
            want = [(li, int(h > w), r0, c0, h, w) for li, (H, W) in enumerate(shapes)
                    for r0, c0, h, w in oracle.tiles(H, W, T)]
            assert hm.himuon_plan_tiles(p) == want
            assert hm.himuon_plan_stats(p)["tile"] == T
        with pytest.raises(hm.HiMuonError):
            hm.himuon_set_tile_schedule(p, -3, 0)
        assert hm.himuon_plan_stats(p)["tile"] == 64  # unchanged after a failed change
    finally:
        hm.himuon_plan_destroy(p)


@pytest.mark.parametrize("mutate,msg", [
    (lambda L, c: setattr(L[0], "ld_m", 100), "leading dimension"),
    (lambda L, c: setattr(L[0], "weight", None), "NULL"),
    (lambda L, c: setattr(L[0], "grad", FAKE + 1), "aligned"),
    (lambda L, c: setattr(L[0], "rows", -1), "rows/cols"),
    (lambda L, c: setattr(c, "tile", -1), "tile"),
    (lambda L, c: setattr(c, "steps", -1), "steps"),
    (lambda L, c: setattr(c, "precision", 7), "precision"),
    (lambda L, c: setattr(c, "state_dtype", 5), "state_dtype"),
    (lambda L, c: setattr(c, "flags", 8), "flag"),
    (lambda L, c: setattr(c, "eps", float("nan")), "finite"),
    # the kernels take B = c ((b / c) A + A^2) in fp32: b / c must stay far from overflow,
    # a nonzero c must not round to zero, and every coefficient must be finite in fp32
    (lambda L, c: setattr(c, "coeffs", hm.himuon_coeffs(3.4445, -4.775, 1e-37)), "b / c"),
    (lambda L, c: setattr(c, "coeffs", hm.himuon_coeffs(3.4445, -4.775, 1e-50)), "b / c"),
    (lambda L, c: setattr(c, "coeffs", hm.himuon_coeffs(1e39, -0.5, 0.0)), "fp32"),
    (lambda L, c: setattr(L[0], "update", None) or setattr(c, "flags", 1), "NULL"),
])
def test_invalid_arguments_are_einval(mutate, msg):
    L = fake_layers([(200, 300)], write_update=True)
    cfg = hm.make_config(64)
    mutate(L, cfg)
    with pytest.raises(hm.HiMuonError) as e:
        hm.himuon_plan(L, cfg)
    assert e.value.status == -1 and msg in str(e.value)


def test_empty_plan_and_empty_matrices():
    p = hm.himuon_plan([], hm.make_config(64))
    assert hm.himuon_plan_stats(p)["tiles"] == 0
    hm.himuon_plan_destroy(p)
    p = plan_for([(0, 10), (10, 0)], 64)
    assert hm.himuon_plan_tiles(p) == []
    hm.himuon_plan_destroy(p)


def test_null_arguments_rejected():
    assert hm._lib.himuon_plan(None, 0, None, None) == -1
    assert hm._lib.himuon_step(None, None, 0, 0.02, None) == -1
    assert hm._lib.himuon_plan_stats(None, None) == -1
    hm._lib.himuon_plan_destroy(None)  # no-op


def test_stream_step_validates_before_touching_a_device():
    # argument checks return before any HIP call, so they run without a GPU
    P = 256   # a non-null address that is never dereferenced
    lib = hm._lib
    assert lib.himuon_stream_step(P, P, P, -1, hm.BF16, 0.95, 0.02, None) == -1
    assert lib.himuon_stream_step(None, P, P, 8, hm.BF16, 0.95, 0.02, None) == -1
    assert lib.himuon_stream_step(P, None, P, 8, hm.F32, 0.95, 0.02, None) == -1
    assert lib.himuon_stream_step(P, P, None, 8, hm.F32, 0.95, 0.02, None) == -1
    assert lib.himuon_stream_step(P, P, P, 8, 9, 0.95, 0.02, None) == -1
    assert lib.himuon_stream_step(P, P, P, 8, hm.BF16, float("nan"), 0.02, None) == -1
    assert lib.himuon_stream_step(P, P, P, 8, hm.BF16, 0.95, float("inf"), None) == -1
    assert "finite" in hm.himuon_last_error()
    assert lib.himuon_stream_step(None, None, None, 0, hm.BF16, 0.95, 0.02, None) == 0   # nothing to do


def test_host_only_plan_counts_no_runtime_calls_and_refuses_to_step():
    # without a GPU the plan is host-only: it made no allocation or wait, a tile-size
    # change makes none either, and a step is refused with EDEVICE
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the plan binds to it (covered by the GPU tests)")
    p = plan_for([(300, 170)], 64)
    try:
        assert hm.himuon_plan_runtime_counts(p) == {"device_allocs": 0, "host_allocs": 0, "host_waits": 0}
        hm.himuon_set_tile_schedule(p, 128, 0)
        assert hm.himuon_plan_runtime_counts(p) == {"device_allocs": 0, "host_allocs": 0, "host_waits": 0}
        assert hm._lib.himuon_step(p, None, 0, 0.02, None) == -4
        assert "no device tables" in hm.himuon_last_error()
    finally:
        hm.himuon_plan_destroy(p)


def test_256_tiles_run_in_place():
    # 256 x 256 tiles iterate in place: one X buffer and one A/B buffer (4 B per element
    # each), half the workspace of the other large tiles, which alternate two X buffers
    p = plan_for([(512, 512)], 256, workspace_budget=10 ** 9)
    # ragged: in table order two 256 x 256 tiles, then a 256 x 8 edge tile (two X buffers),
    # per tile row; chunks are cut where the kind changes, so four chunks
    q = plan_for([(512, 520)], 256, workspace_budget=10 ** 9)
    try:
        per_tile = 2 * 256 * 256 * 4 + 256                       # X, A/B, partial sums (8 + 1 floats)
        assert hm.himuon_workspace_size(p) == 4 * per_tile
        st = hm.himuon_plan_stats(q)
        edge = 2 * 8 * 256 * 4 + 2 * 8 * 64 * 4 + 256            # r = 8, ldx = 256, lda = 64
        assert st["gemm_tiles"] == 6 and st["chunks"] == 4
        assert hm.himuon_workspace_size(q) == max(2 * per_tile, edge)
    finally:
        hm.himuon_plan_destroy(p)
        hm.himuon_plan_destroy(q)

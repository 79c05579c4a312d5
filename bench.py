"""Benchmark of one HiMuon optimizer step on one MI355X.

Workload: the Llama-3-8B-shaped stack (32 layers of q/o 4096x4096, k/v 4096x1024,
gate/up 4096x14336, down 14336x4096: 224 matrices, 6,979,321,856 parameters),
bf16 momentum and gradient, fp32 master weights, T = 128, K = 5, quintic
coefficients, workspace budget 4e9 bytes.  A step is momentum update, tiled
Newton-Schulz and weight update over every matrix, inputs resident in HBM.

Prints one JSON line.  `value` is the whole-step throughput in algorithmic NS
TFLOP/s (sum over tiles of K (4 r^2 s + 2 r^3) per step / step time);
`ms_per_step` is the step time.  `roofline` prices the step's one fused-kernel
launch against both of its bounds, MFMA (algorithmic flops at the bf16 dense peak)
and HBM (14 algorithmic bytes per element at 8 TB/s), and names the larger as the
bound.  `sweep` gives the same figures per T (including FULL, the full-matrix Muon
baseline), `memory_pass` the identity-map step (momentum, gather, scatter and weight
update of every tile with no Newton-Schulz step: the fused path's HBM stream alone),
and `schemes` the step in each arithmetic scheme that holds the bf16 bar.

    python bench.py [--steps K] [--warmup W] [--tile T] [--sweep 32,64,256,full] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
METRIC = "HiMuon step ms & NS TFLOP/s (% MFMA peak) vs T, 8B-shaped stack"

# HBM bytes of one launch of the T=128 fused kernel (bf16f8) on this workload, from two
# rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), scaled by the
# readings of a 1 GiB elementwise copy (x2.0 read, x1.0 write).  Valid only for the
# kernel source it was measured on (sha256 prefix of ns_fused.hip followed by the two
# headers it includes); null otherwise.
TRAFFIC_T128 = {"source_sha256_16": "c052f9a1f7329e72", "precision": "bf16f8", "fetch_kib": 27291272.4375,
                "write_kib": 40894464.0, "fetch_scale": 2.0, "write_scale": 1.0}


KERNEL_SOURCES = ("ns_fused.hip", "himuon_internal.h", "device_common.h")


def measured_traffic():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tiled_newton_schulz_tile_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()[:16]
    t = TRAFFIC_T128
    if not t["source_sha256_16"] or sha != t["source_sha256_16"]:
        return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])


STACK_TEXT = {"llama3-8b-32L": "Llama-3-8B-shaped stack", "decoder-1b-16L": "1B-class decoder stack",
              "gpt2-small-12L": "GPT-2-small-shaped stack", "single-256x512": "single 256x512 matrix"}

# name -> (library constant, dtype field, description)
PRECISIONS = {
    "bf16f8": ("PREC_BF16F8", "bf16+e4m3",
               "bf16f8: operands split x = hi + lo; hi*hi on bf16 MFMA, hi*lo and lo*hi on "
               "e4m3 MFMA with power-of-two block scales; fp32 accumulate"),
    "bf16x3": ("PREC_BF16X3", "bf16",
               "bf16x3: operands split hi+lo bf16, 3 MFMA products, fp32 accumulate"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_inputs(shapes, device, seed0=3000, kind="power-law"):
    """Seeded inputs.  power-law: the recipe of the synth module (Haar factors shared per
    shape).  randn: G = 0.01 N(0, 1), used for counter runs, where the QR of the recipe
    cannot run under the profiler; the kernels' traffic does not depend on the values."""
    import synth
    import torch
    t0 = time.time()
    if kind == "randn":
        g = torch.Generator(device=device).manual_seed(seed0)
        layers = []
        for h, w in shapes:
            G = (0.01 * torch.randn(h, w, device=device, generator=g)).to(torch.bfloat16)
            layers.append((synth.weights(h, w, seed0, device), torch.zeros_like(G), G))
    else:
        layers = synth.stack_inputs(shapes, seed0, device=device, state_dtype=torch.bfloat16,
                                    share_factors=True)
    torch.cuda.synchronize()
    log(f"[bench] generated {len(layers)} matrices ({kind}) in {time.time() - t0:.1f}s")
    return layers


def copy_calibration(device, nbytes=1 << 30):
    """A plain elementwise copy of known size (nbytes read, nbytes written) whose
    FETCH_SIZE / WRITE_SIZE readings scale the counters of the HiMuon kernels."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {nbytes} B read, {nbytes} B written")


def time_steps(opt, steps, warmup, lr=0.02):
    """Times `steps` steps after `warmup` untimed ones with HIP events on the stream
    the kernels are launched on; returns per-step milliseconds."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        opt.step(lr, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        opt.step(lr, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def stream_reference(dev, step_bytes, n, steps, warmup, lr=0.02):
    """The memory pass's bytes as one flat stream: himuon_stream_step (M <- beta M + G
    stored in bf16, W <- W - lr M) over n contiguous elements in buffers of its own,
    timed with HIP events like a step; the HBM rate this read/write mix reaches."""
    import torch
    import tiled_newton_schulz_tile_amd as hm
    g = torch.randn(n, dtype=torch.bfloat16, device=dev, generator=torch.Generator(device=dev).manual_seed(91))
    m = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    w = torch.randn(n, dtype=torch.float32, device=dev, generator=torch.Generator(device=dev).manual_seed(92))
    stream = torch.cuda.current_stream()

    def launch():
        hm.himuon_stream_step(m.data_ptr(), g.data_ptr(), w.data_ptr(), n, hm.BF16, 0.95, lr, stream.cuda_stream)

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        launch()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) / steps
    del g, m, w
    torch.cuda.empty_cache()
    gbps = step_bytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "hbm_gbps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "what": "himuon_stream_step over one flat run of the stack's element count: the same 14 B "
                    "per element (G, M read; M written; W read and written) with no tiling"}


def rates(st, ms):
    """Both bounds of a step of `ms` milliseconds: algorithmic NS flops at the bf16 MFMA
    peak and algorithmic HBM bytes at the HBM peak; the larger lower bound names it."""
    tflops = st["ns_flops"] / (ms * 1e-3) / 1e12
    gbps = st["step_bytes"] / (ms * 1e-3) / 1e9
    t_mfma = st["ns_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    t_hbm = st["step_bytes"] / (HBM_PEAK_GBPS * 1e9) * 1e3
    return {"ms": round(ms, 4), "ns_tflops": round(tflops, 3),
            "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
            "hbm_gbps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "floor_ms": {"mfma": round(t_mfma, 4), "hbm": round(t_hbm, 4)},
            "bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "frac_of_roofline": round(max(t_mfma, t_hbm) / ms, 4)}


def cpu_baseline(K, coeffs, tile, shapes):
    """The fp64 oracle on the host, on a bounded sample of the workload: the seven
    matrices of one decoder layer of the stack (momentum + tiled NS + update; about
    10-15 s of CPU work).  Throughput in algorithmic NS TFLOP/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads") or 0) for i in threadpool_info()) or os.cpu_count()
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    layer = list(shapes[:7])
    rng = np.random.default_rng(0)
    mats = []
    for H, W in layer:
        G = rng.standard_normal((H, W), dtype=np.float32) * 0.01
        mats.append((np.zeros((H, W), dtype=np.float32), np.zeros((H, W), dtype=np.float32), G))
    t0 = time.time()
    oracle.step(mats, tile, K, coeffs)
    dt = time.time() - t0
    fl = oracle.ns_flops(layer, tile, K, coeffs)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one decoder layer of the stack ({len(layer)} matrices, "
                      f"{sum(h * w for h, w in layer)} params; T={tile}, K={K}, quintic, fp64 numpy "
                      f"{np.__version__}), {dt:.1f} s for {fl:.3e} NS flops; whole-step time at this "
                      f"rate scales by the flop ratio",
            "seconds": dt, "host_cpus": os.cpu_count()}


def run_diagnostics(args):
    """Matrix-function diagnostics sweep (not the step benchmark): the three distinct
    matrix shapes of the 1B-shaped stack, power-law inputs, bf16 state, bf16x3, K=5
    quintic; per T the deviation from the FULL map, the alignment with the polar factor,
    the extreme singular values of O_T and the device time of the NS step.  The fp64
    oracle computes the same diagnostics of one 512 x 512 matrix beside it."""
    import torch
    import synth
    import tiled_newton_schulz_tile_amd as hm
    from tiled_newton_schulz_tile_amd import diagnostics as dg
    tiles = [32, 64, 128, 256, 0]
    shapes = sorted(set(synth.STACKS["decoder-1b-16L"]))
    res = {}
    for i, (H, W) in enumerate(shapes):
        M = synth.power_law_matrix(H, W, 7000 + i, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        rep = dg.report(M, tiles, 5, hm.QUINTIC, precision=hm.PREC_BF16X3, spectrum=False)
        res[f"{H}x{W}"] = {("full" if T == 0 else str(T)): {k: round(v, 6) for k, v in rep[T].items()}
                           for T in tiles}
        log(f"[diag] {H}x{W}: " + "  ".join(
            f"T={'full' if T == 0 else T}: dev {rep[T]['deviation']:.4f} cos {rep[T]['cosine']:.4f} "
            f"align {rep[T]['alignment']:.4f} dual {rep[T]['dual_alignment']:.4f} "
            f"sv [{rep[T]['sv_min']:.3f}, {rep[T]['sv_max']:.3f}] {rep[T]['ms']:.2f} ms" for T in tiles))
    cpu = None
    if not args.no_cpu:
        import oracle.diagnostics as odg
        M = synth.power_law_matrix(512, 512, 7100, dtype=torch.float32).to(torch.bfloat16)
        t0 = time.time()
        odg.report(M.double().numpy(), tiles, 5, hm.QUINTIC)
        cpu = {"sample": "512x512 power-law matrix, the same five T", "seconds": round(time.time() - t0, 3),
               "kind": "oracle"}
        t0 = time.time()
        dg.report(M.cuda(), tiles, 5, hm.QUINTIC, precision=hm.PREC_BF16X3)
        cpu["gpu_seconds_same_sample"] = round(time.time() - t0, 3)
    print(json.dumps({"metric": "matrix-function diagnostics vs T (deviation and cosine against FULL, "
                                "alignment and dual alignment with the polar factor, singular values of O_T)",
                      "data": "synthetic: G = U diag(1/i) V^T + 0.01 N(0,1), Haar U, V; seeded",
                      "config": {"workload": "decoder-1b-16L distinct shapes", "ns_steps": 5,
                                 "coeffs": "quintic", "state_dtype": "bf16", "precision": "bf16x3"},
                      "results": res, "cpu_baseline": cpu}), flush=True)


def run_sign(args):
    """Sign-Muon local kernels on 2^28 entries (a 16384 x 16384 fp32 direction): sign +
    1-bit pack, and the majority vote of 8 workers' packed buffers into bf16.  Both are
    HBM streams; algorithmic bytes: pack 4 B read + 1/8 B written per entry, vote 1/8 B read
    per worker + 2 B written per entry.  The numpy oracle does the same on 2^22 entries."""
    import numpy as np
    import torch
    from tiled_newton_schulz_tile_amd import signmuon as sm
    rows = cols = 16384
    n, workers = rows * cols, 8
    g = torch.Generator(device="cuda").manual_seed(0)
    O = torch.randn(rows, cols, device="cuda", generator=g)
    bits = torch.zeros(sm.packed_bytes(n), dtype=torch.uint8, device="cuda")
    gathered = torch.randint(0, 256, (workers, sm.packed_bytes(n)), dtype=torch.uint8, device="cuda", generator=g)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_pack = timed(lambda: sm.sign_pack(O, out=bits), args.steps)
    ms_vote = timed(lambda: sm.sign_vote(gathered, n, torch.bfloat16, out=out), args.steps)
    b_pack = n * 4 + (n + 7) // 8
    b_vote = workers * ((n + 7) // 8) + 2 * n
    res = {}
    for name, ms, b in (("sign_pack_kernel", ms_pack, b_pack), ("sign_vote_kernel<bf16>, 8 workers", ms_vote, b_vote)):
        gbs = b / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bytes": b, "GB/s": round(gbs, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBPS, 4)}}
        log(f"[sign] {name}: {ms:.3f} ms, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBPS:.1f} % of HBM peak)")
    cpu = None
    if not args.no_cpu:
        import oracle.signmuon as osm
        m = 1 << 22
        x = np.random.default_rng(0).standard_normal(m).astype(np.float32)
        t0 = time.time()
        packed = osm.pack(osm.sign(x))
        t_pack = time.time() - t0
        bufs = [packed] * workers
        t0 = time.time()
        osm.vote(bufs, m)
        t_vote = time.time() - t0
        cpu = {"kind": "oracle", "sample": f"{m} entries, 8 workers", "pack_seconds": round(t_pack, 4),
               "vote_seconds": round(t_vote, 4),
               "pack_GB/s": round((4 * m + m / 8) / t_pack / 1e9, 3),
               "vote_GB/s": round((workers * m / 8 + 2 * m) / t_vote / 1e9, 3)}
    print(json.dumps({"metric": "Sign-Muon local kernels: HBM GB/s", "data": "synthetic: N(0,1) direction, "
                      "uniform random packed buffers; seeded", "config": {"workload": "16384x16384 direction, "
                      "8 workers", "entries": n}, "results": res, "cpu_baseline": cpu}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tile", type=int, default=128)
    ap.add_argument("--sweep", type=str, default="32,64,256,full")
    ap.add_argument("--sweep-steps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-memory-pass", action="store_true", help="skip the identity-map (HBM-only) leg")
    ap.add_argument("--no-schemes", action="store_true", help="skip timing the other arithmetic scheme")
    ap.add_argument("--workload", type=str, default="llama3-8b-32L")
    ap.add_argument("--inputs", choices=["power-law", "randn"], default="power-law")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--precision", choices=sorted(PRECISIONS), default="bf16f8",
                    help="arithmetic of the NS products (bf16f8: bf16 main product, e4m3 "
                         "correction products; bf16x3: three bf16 products)")
    ap.add_argument("--diagnostics", action="store_true",
                    help="run the matrix-function diagnostics sweep instead of the step benchmark")
    ap.add_argument("--sign", action="store_true",
                    help="time the Sign-Muon sign-pack and vote kernels instead of the step benchmark")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the HiMuon step is tile-local and the library runs "
              "it on one MI355X; sharding its tiles across GPUs is designed, not built. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import tiled_newton_schulz_tile_amd as hm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.diagnostics:
        run_diagnostics(args)
        return
    if args.sign:
        run_sign(args)
        return
    dev = torch.device("cuda:0")
    shapes = synth.STACKS[args.workload]
    K, coeffs = 5, hm.QUINTIC
    layers = build_inputs(shapes, dev, kind=args.inputs)
    prec_const, prec_dtype, prec_text = PRECISIONS[args.precision]

    def plan(tile, prec_name, identity=False):
        return hm.HiMuon(layers, tile, K, coeffs, beta=0.95, eps=1e-7, workspace_budget=4 * 10 ** 9,
                         precision=getattr(hm, PRECISIONS[prec_name][0]), identity=identity)

    opt = plan(args.tile, args.precision)
    st = opt.stats()
    log(f"[bench] plan: {st['tiles']} tiles, kernel tile {st['kernel_tile']}, "
        f"{st['ns_flops']:.4e} NS flops/step, workspace {st['workspace_bytes']} B")
    ms = time_steps(opt, args.steps, args.warmup)
    ms_mean = sum(ms) / len(ms)
    log(f"[bench] T={args.tile}: {ms_mean:.3f} ms/step (min {min(ms):.3f}, max {max(ms):.3f})")
    tflops = st["ns_flops"] / (ms_mean * 1e-3) / 1e12
    issued = st["issued_flops"] / (ms_mean * 1e-3) / 1e12
    gbps = st["step_bytes"] / (ms_mean * 1e-3) / 1e9
    head = rates(st, ms_mean)

    sweep = [dict({"tile": args.tile}, **head)]
    for tok in [t for t in args.sweep.split(",") if t.strip()]:
        T = 0 if tok.strip().lower() == "full" else int(tok)
        if T == args.tile:
            continue
        try:
            opt.set_tile_schedule(T)
            s2 = opt.stats()
            m2 = time_steps(opt, args.sweep_steps, 1)
            m2 = sum(m2) / len(m2)
            r2 = rates(s2, m2)
            sweep.append(dict({"tile": "full" if T == 0 else T,
                               "path": "fused" if s2["gemm_tiles"] == 0 else "large-tile"}, **r2))
            log(f"[bench] sweep T={tok}: {m2:.3f} ms/step, {r2['ns_tflops']:.1f} NS TFLOP/s "
                f"({r2['pct_mfma_peak']:.1f} % MFMA), {r2['hbm_gbps']:.0f} GB/s ({r2['pct_hbm_peak']:.1f} % HBM), "
                f"{r2['bound']}-bound, {100 * r2['frac_of_roofline']:.1f} % of its roofline")
        except hm.HiMuonError as e:
            sweep.append({"tile": tok, "error": str(e)})
            log(f"[bench] sweep T={tok}: {e}")
    opt.close()

    # the fused path's HBM stream alone: the identity-map step at the headline T
    mem = None
    if not args.no_memory_pass:
        idp = plan(args.tile, args.precision, identity=True)
        mi = time_steps(idp, args.steps, args.warmup)
        mi = sum(mi) / len(mi)
        ist = idp.stats()
        idp.close()
        mgbps = ist["step_bytes"] / (mi * 1e-3) / 1e9
        mem = {"ms": round(mi, 4), "bytes_per_step": ist["step_bytes"], "hbm_gbps": round(mgbps, 1),
               "pct_hbm_peak": round(100 * mgbps / HBM_PEAK_GBPS, 2),
               "what": "HIMUON_FLAG_IDENTITY_MAP: momentum, gather, scatter and W update of every tile, "
                       "no NS step; 14 B per element"}
        log(f"[bench] memory pass (identity map) T={args.tile}: {mi:.3f} ms, {mgbps:.0f} GB/s "
            f"({100 * mgbps / HBM_PEAK_GBPS:.1f} % of HBM peak)")
        ref = stream_reference(dev, ist["step_bytes"], sum(h * w for h, w in shapes), args.steps, args.warmup)
        mem["stream_reference"] = ref
        mem["frac_of_stream_reference"] = round(ref["ms"] / mi, 4)
        log(f"[bench] flat stream of the same bytes: {ref['ms']:.3f} ms, {ref['hbm_gbps']:.0f} GB/s; "
            f"memory pass at {100 * ref['ms'] / mi:.1f} % of it")

    # the other scheme that holds the bf16 bar, same T
    schemes = {args.precision: {"ms": round(ms_mean, 4), "ns_tflops": round(tflops, 3)}}
    if not args.no_schemes:
        for other in sorted(PRECISIONS):
            if other == args.precision:
                continue
            op2 = plan(args.tile, other)
            m3 = time_steps(op2, args.steps, args.warmup)
            op2.close()
            m3 = sum(m3) / len(m3)
            schemes[other] = {"ms": round(m3, 4), "ns_tflops": round(st["ns_flops"] / (m3 * 1e-3) / 1e12, 3)}
            log(f"[bench] scheme {other} T={args.tile}: {m3:.3f} ms/step")

    if args.copy_calibration:
        copy_calibration(dev)

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the oracle on the host (bounded sample)")
        cpu = cpu_baseline(K, coeffs, args.tile, shapes)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads "
            f"({cpu['seconds']:.1f}s)")
        cpu.pop("seconds", None)

    n_params = sum(h * w for h, w in shapes)
    kt = st["kernel_tile"]
    terms = {"mfma": {"achieved": head["ns_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(head["pct_mfma_peak"] / 100, 4), "floor_ms": head["floor_ms"]["mfma"]},
             "hbm": {"achieved": head["hbm_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(head["pct_hbm_peak"] / 100, 4), "floor_ms": head["floor_ms"]["hbm"]}}
    bound = head["bound"]
    if kt > 0 and st["gemm_tiles"] == 0:
        # one launch of the fused kernel per step: the step time is its duration
        kprec = args.precision if (args.precision != "bf16f8" or kt >= 64) else "bf16x3"
        roofline = dict(terms[bound], bound=bound, terms=terms,
                        traffic=measured_traffic() if (kt == 128 and args.tile == 128
                                                       and args.workload == "llama3-8b-32L"
                                                       and args.precision == TRAFFIC_T128["precision"])
                        else None,
                        kernel=f"fused_step_kernel<{kt}, {kprec}, bf16 state>", launches_per_step=1,
                        algorithmic_flops_per_launch=st["ns_flops"], issued_flops_per_launch=st["issued_flops"],
                        algorithmic_bytes_per_launch=st["step_bytes"])
    else:
        # the large-tile path: per chunk, momentum, norm, stage and apply launches plus the
        # NS products (bf16x3 arithmetic); rates are over the whole step, not one kernel
        roofline = dict(terms[bound], bound=bound, terms=terms, traffic=None,
                        kernel="large-tile path (GEMM products in bf16x3: gemm_t256_ns_kernel runs all K "
                               "steps of a 256x256 tile in one workgroup, one launch per chunk; "
                               "gemm_b256_kernel (sides multiples of 256) or gemm_ns_kernel run one launch "
                               "per product and NS step; whole step)",
                        chunks_per_step=int(st["chunks"]),
                        algorithmic_flops_per_step=st["ns_flops"], issued_flops_per_step=st["issued_flops"],
                        algorithmic_bytes_per_step=st["step_bytes"])

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec_dtype,
        "precision": prec_text,
        "data": ("synthetic: G = U diag(1/i) V^T + 0.01 N(0,1) per matrix (Haar U, V shared per "
                 "shape), M0 = 0, W0 = 0.02 N(0,1); seeded") if args.inputs == "power-law" else
                "synthetic: G = 0.01 N(0,1), M0 = 0, W0 = 0.02 N(0,1); seeded (counter run)",
        "config": {"workload": f"{args.workload} HiMuon step ({STACK_TEXT.get(args.workload, args.workload)}, "
                               f"{len(shapes)} matrices, {n_params:.3g} params), T={args.tile}, K={K}, quintic",
                   "tile": args.tile, "ns_steps": K, "coeffs": "quintic", "state_dtype": "bf16",
                   "weight_dtype": "f32", "workspace_budget": 4 * 10 ** 9,
                   "tiles": st["tiles"], "params": n_params},
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "issued_mfma_tflops": round(issued, 2),
        "hbm_gbps": round(gbps, 1),
        "roofline": roofline,
        "sweep": sweep,
        "memory_pass": mem,
        "schemes": schemes,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

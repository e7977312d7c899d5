"""Throughput of the ROCS shared forward stack on one MI355X.

One step = one rocs_stack_forward over one batch of the GLM MLP stack workload
(B = 256 requests, N_b ~ U{64..512} candidates, d_R = d_C = 512, three GLM
MLP blocks of hidden 1024 per group with residual and group-local RMSNorm,
scalar head; bf16 storage, fp32 accumulation), inputs resident in HBM.

Prints one JSON line: candidates/s, MFMA utilisation, the same-GPU
dense-broadcast comparator and its speedup, the roofline of the dominant
kernel (the IKBO candidate GEMM, timed with HIP events on its launch
stream) and the CPU oracle's rate on a bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15  # dense MFMA bf16, FLOP/s
PEAK_HBM = 8.0e12   # bytes/s
METRIC = "candidates/sec through ROCS layer stack, MFMA util %, speedup vs dense broadcast"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def glm_mlp_work(cfg, B_r, B_c):
    """Algorithmic FLOPs and bytes of one shared-execution step (request side once, candidate side per candidate)."""
    d, H = cfg.d_r, cfg.hidden
    F = 0.0
    Bts = 0.0
    for _ in range(cfg.n_blocks):
        # up: [B_r x 2H] = x_r [W_RR; W_CR]^T ; candidates: [B_c x H] from d
        F += 2.0 * B_r * (2 * H) * d + 2.0 * B_c * H * d
        # down: [B_r x 2d] from H ; candidates [B_c x d] from H
        F += 2.0 * B_r * (2 * d) * H + 2.0 * B_c * d * H
        # bytes: activations read/written once, weights once, Z once (fp32 write + read)
        Bts += 2 * (B_r + B_c) * d + 2 * (B_r + B_c) * H          # up: read x, write h
        Bts += 2 * (2 * H * d + H * d)                              # up weights W_RR, W_CR, W_CC
        Bts += 2 * 4 * B_r * H                                      # Z write + read
        Bts += 2 * (B_r + B_c) * H + 2 * 2 * (B_r + B_c) * d        # down: read h, read residual, write o
        Bts += 2 * (2 * d * H + d * H) + 2 * 4 * B_r * d
        Bts += 2 * 2 * (B_r + B_c) * d                              # RMSNorm read + write
        Bts += 4 * B_c                                              # cand2req reads
    F += 2.0 * B_r * d + 2.0 * B_c * d                              # head
    Bts += 2 * (B_r + B_c) * d + 4 * B_c
    return F, Bts


def step_latencies(fn, n=100):
    """Per-step latency distribution: each step bracketed by its own events
    on the launch stream (steps back to back, as a serving loop runs them)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = np.sort(np.array([e0.elapsed_time(e1) for e0, e1 in ev]))
    return {"steps": n, "p50_ms": float(np.percentile(t, 50)), "p99_ms": float(np.percentile(t, 99)),
            "max_ms": float(t[-1])}


def time_steps(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


ROOFLINE_KERNEL = "gemm_bf16_mixed_kernel<256, 128>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_candidate_gemm_glm_mlp.json")
# sources the candidate GEMM is compiled from (the counters are void once any of them changes)
GEMM_SRCS = [os.path.join(ROOT, "request_candidate_sharing_amd", "csrc", f)
             for f in ("rocs_gemm.hip", "rocs_mfma.h", "rocs_device.h")]


def gemm_source_sha():
    import hashlib

    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(alg_bytes):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    only while the kernel source is the one the counters were taken on."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != gemm_source_sha():
        return None
    return t.get("bytes_per_launch")


def candidate_gemm_roofline(st, reps=10, sets=3):
    """Times the dominant kernel alone: the IKBO candidate GEMM of the GLM MLP up
    projection (x_c [B_c, 512] -> [B_c, 1024], ReLU, Z[m_i] gathered in the
    epilogue), launched through rocs_lcb_candidate on torch's current stream and
    bracketed by events on that stream.  Launches rotate over `sets` buffer
    sets (> 256 MB in total) so the Infinity Cache cannot hold the operands
    between launches, as in the stack."""
    import torch
    from request_candidate_sharing_amd import rocs as R

    cfg = st.cfg
    B_r, B_c = st.B_r, st.B_c
    K, N = cfg.d_r, cfg.hidden
    g = torch.Generator(device="cuda").manual_seed(0)
    bf = torch.bfloat16
    w = (torch.randn(N, K, generator=g, device="cuda") * K ** -0.5).to(bf)
    z = torch.randn(B_r, N, generator=g, device="cuda")
    bufs = [(torch.randn(B_c, K, generator=g, device="cuda").to(bf), torch.empty(B_c, N, device="cuda", dtype=bf))
            for _ in range(sets)]
    s = R.cur_stream()

    def launch(b):
        R.rocs_lcb_candidate(st.batch, R.ROCS_BF16, b[0], K, K, w, None, N, R.ROCS_ACT_RELU, z, N, None, 0, b[1],
                             N, s)

    for b in bufs:
        launch(b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for b in bufs:
            launch(b)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / (reps * sets)
    flops = 2.0 * B_c * N * K
    # algorithmic bytes: x_c read once, y_c written once, W_CC once, Z (fp32, B_r rows) once, cand2req once
    byts = 2.0 * B_c * K + 2.0 * B_c * N + 2.0 * N * K + 4.0 * B_r * N + 4.0 * B_c
    t_mfma, t_hbm = flops / PEAK_BF16, byts / PEAK_HBM
    if t_hbm >= t_mfma:
        rf = {"bound": "hbm", "achieved": byts / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        rf = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s"}
    rf["frac"] = rf["achieved"] / rf["peak"]
    rf["traffic"] = measured_traffic(byts)
    rf["kernel"] = ROOFLINE_KERNEL + " via rocs_lcb_candidate (GLM up projection, B_c x 512 -> B_c x 1024, Z[m_i] epilogue)"
    rf["avg_launch_us"] = t * 1e6
    rf["alg_flops_per_launch"] = flops
    rf["alg_bytes_per_launch"] = byts
    rf["mfma_frac"] = flops / t / PEAK_BF16
    rf["hbm_frac"] = byts / t / PEAK_HBM
    return rf


def copy_calibration(mib=1024, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {mib} MiB")


def oracle_threads() -> int:
    """Threads of the BLAS pool the numpy oracle runs on."""
    try:
        from threadpoolctl import threadpool_info

        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(inp, seconds):
    import oracle

    threads = oracle_threads()
    counts = inp["counts"]
    done, n_req, t_total = 0, 0, 0.0
    for b in range(len(counts)):
        if counts[b] == 0:
            continue
        t0 = time.perf_counter()
        oracle.oracle_forward(inp, requests=[b])
        t_total += time.perf_counter() - t0
        done += int(counts[b])
        n_req += 1
        if t_total >= seconds:
            break
    return {"value": done / t_total, "unit": "candidates/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 numpy oracle (dense masked model, materialized broadcast) on requests 0..{n_req - 1} "
                      f"of the same batch: {done} candidates in {t_total:.1f} s"}


def other_workload(args):
    """Shared (and dense-broadcast) step time of another workload's stack, for profiling."""
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    cfg = S.config(args.workload)
    inp = S.make_inputs(cfg)
    if args.shuffle:
        inp = S.shuffle_candidates(inp)
    B_r, B_c = cfg.B, int(len(inp["cand2req"]))
    log(f"bench: workload {args.workload} ({cfg.name()}) B_r={B_r} B_c={B_c}" + (" shuffled" if args.shuffle else ""))
    st = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
    t_sh, _ = time_steps(st.run, args.steps, args.warmup)
    del st
    out = {"workload": args.workload, "name": cfg.name(), "B_r": B_r, "B_c": B_c,
           "ms_per_step": t_sh / args.steps * 1e3, "candidates_per_s": B_c * args.steps / t_sh}
    if not args.no_dense:
        de = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
        t_de, _ = time_steps(de.run, args.steps, args.warmup)
        out["dense_broadcast_ms_per_step"] = t_de / args.steps * 1e3
        out["speedup_vs_dense_broadcast"] = t_de / t_sh
    print(json.dumps(out), flush=True)


def regime_study(args):
    """Shared vs dense-broadcast step time on the GLM MLP stack shapes with a
    fixed number of candidates per request, N in {1, 10, 100, 500, 1000}
    (256 requests): the regime in which request sharing pays, and the
    N = 500 ratio check."""
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    cfg = S.config(2)
    for n in (1, 10, 100, 500, 1000):
        inp = S.make_inputs(cfg, counts=[n] * cfg.B)
        B_r, B_c = cfg.B, int(len(inp["cand2req"]))
        st = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
        t_sh, _ = time_steps(st.run, args.steps, args.warmup)
        del st
        de = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
        t_de, _ = time_steps(de.run, args.steps, args.warmup)
        del de
        F, _ = glm_mlp_work(cfg, B_r, B_c)
        sh = t_sh / args.steps
        st = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
        lat = step_latencies(st.run, 50)
        del st
        print(json.dumps({"study": "regime", "workload": 2, "n_per_request": n, "B_r": B_r, "B_c": B_c,
                          "shared_ms": sh * 1e3, "dense_broadcast_ms": t_de / args.steps * 1e3,
                          "speedup_vs_dense_broadcast": t_de / t_sh, "candidates_per_s": B_c / sh,
                          "mfma_util_pct": 100.0 * F / sh / PEAK_BF16, "step_latency": lat}), flush=True)


def order_study(args):
    """Shared step time with candidates contiguous per request (offsets given)
    and in a random global order (offsets NULL: the kernels resolve
    cand2req row by row and the attention plan sorts candidates on the
    device)."""
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    for k in (2, 3, 4, 5):
        cfg = S.config(k)
        inp = S.make_inputs(cfg)
        res = {}
        for name, data in (("contiguous", inp), ("shuffled", S.shuffle_candidates(inp))):
            st = DeviceStack(data, mode=R.ROCS_EXEC_SHARED)
            t, _ = time_steps(st.run, args.steps, args.warmup)
            del st
            res[name] = t / args.steps * 1e3
        print(json.dumps({"study": "candidate_order", "workload": k, "B_r": cfg.B, "B_c": int(len(inp["cand2req"])),
                          "contiguous_ms": res["contiguous"], "shuffled_ms": res["shuffled"],
                          "shuffled_over_contiguous": res["shuffled"] / res["contiguous"]}), flush=True)


def ugsep_work(cfg, B_r, B_c, dense=False):
    """Algorithmic FLOPs of one UG-Sep TokenMixer step: per layer and token, the
    two FFN GEMMs (2 * rows * dim * hidden each); the U side runs on B_r rows
    when shared and on B_c rows in the dense comparator."""
    R_u = B_c if dense else B_r
    per = 2 * 2.0 * cfg.dim * cfg.hidden
    comp = 2.0 * R_u * cfg.n_g * cfg.n_u * cfg.dim if cfg.comp else 0.0
    return cfg.n_layers * (per * (cfg.n_u * R_u + cfg.n_g * B_c) + comp)


def ugsep_study(args):
    """The UG-Separation TokenMixer workload: U tokens once per request vs
    the dense comparator that copies them to every candidate, with the CPU
    oracle's rate on a bounded sample."""
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceUgsep

    cfg = S.ugsep_config("tokenmixer")
    inp = S.make_ugsep_inputs(cfg)
    B_r, B_c = cfg.B, int(len(inp["cand2req"]))
    log(f"bench: UG-Sep TokenMixer B_r={B_r} B_c={B_c}")
    st = DeviceUgsep(inp, mode=R.ROCS_UGSEP_SHARED)
    t_sh, _ = time_steps(st.run, args.steps, args.warmup)
    del st
    sh = t_sh / args.steps
    F = ugsep_work(cfg, B_r, B_c)
    out = {"study": "ugsep", "workload": S.UGSEP_NAMES["tokenmixer"], "B_r": B_r, "B_c": B_c,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": sh * 1e3, "candidates_per_s": B_c / sh,
           "alg_flops_per_step": F, "mfma_util_pct": 100.0 * F / sh / PEAK_BF16}
    if not args.no_dense:
        de = DeviceUgsep(inp, mode=R.ROCS_UGSEP_DENSE)
        t_de, _ = time_steps(de.run, args.steps, args.warmup)
        del de
        Fd = ugsep_work(cfg, B_r, B_c, dense=True)
        out.update(dense_ms_per_step=t_de / args.steps * 1e3, speedup_vs_dense=t_de / t_sh,
                   saved_fraction=1.0 - t_sh / t_de, flop_saved_fraction=1.0 - F / Fd,
                   dense_mfma_util_pct=100.0 * Fd / (t_de / args.steps) / PEAK_BF16)
    if not args.no_cpu:
        from oracle import ugsep as U

        done, t0 = 0, time.perf_counter()
        cores = oracle_threads()
        while time.perf_counter() - t0 < args.cpu_seconds:
            cand = np.arange(done, min(done + 16, B_c))
            U.ugsep_forward(inp, candidates=cand, requests=[])
            done += len(cand)
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": done / el, "unit": "candidates/s", "cores": cores, "kind": "oracle",
                               "sample": f"oracle (fp64 numpy, per candidate) on the first {done} candidates "
                                         f"of the same batch in {el:.1f} s"}
    print(json.dumps(out), flush=True)


def w8a16_study(args):
    """Latency of the W8A16 linear layer against the bf16 GEMM of the same
    shape, at the layer shapes of the UG-Separation page's W8A16 table.
    Weights rotate over buffer sets larger than the 256 MB MALL, so each
    launch streams its weights from HBM as a layer of a deep model would."""
    import torch
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R

    page = {(16, 1280, 2560): -50.2, (16, 1280, 640): -40.0, (8, 1280, 2560): -46.8, (8, 1280, 640): -55.0}
    st = R.cur_stream()
    # the page's shapes, then two larger ones where the weight stream dominates
    for (M, K, N) in S.W8A16_SHAPES + [(16, 4096, 4096), (16, 8192, 8192)]:
        d = S.make_w8a16_inputs(M, K, N)
        x = torch.as_tensor(d["x"], device="cuda").to(torch.bfloat16)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        b = torch.as_tensor(d["bias"], device="cuda").to(torch.bfloat16)
        sc = torch.as_tensor(d["scale"], device="cuda")
        sets8 = max(2, (320 << 20) // (N * K))
        sets16 = max(2, (320 << 20) // (2 * N * K))
        wq = torch.as_tensor(d["codes"], device="cuda").unsqueeze(0).repeat(sets8, 1, 1)
        wb = torch.randn(sets16, N, K, device="cuda").to(torch.bfloat16)

        def t8(i):
            R.rocs_w8a16_linear(M, N, K, x, K, wq[i % sets8], K, sc, b, 0, y, N, st)

        def t16(i):
            R.rocs_lcb_request(R.ROCS_BF16, M, x, K, K, wb[i % sets16], None, b, N, 0, 0, None, 0, y, N, None, 0, st)

        res = {}
        for name, fn in (("w8a16", t8), ("bf16", t16)):
            for i in range(args.warmup * 10):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(args.steps * 20, 200)
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / reps
        print(json.dumps({"study": "w8a16", "M": M, "K": K, "N": N, "w8a16_us": res["w8a16"], "bf16_us": res["bf16"],
                          "latency_change_pct": 100.0 * (res["w8a16"] / res["bf16"] - 1.0),
                          "page_latency_change_pct": page.get((M, K, N)),
                          "w8a16_weight_GBps": N * K / res["w8a16"] / 1e3,
                          "bf16_weight_GBps": 2 * N * K / res["bf16"] / 1e3}), flush=True)
        del wq, wb


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-broadcast comparator")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--roofline-reps", type=int, default=10)
    ap.add_argument("--copy-calib", action="store_true", help="only run the copy kernel used to scale HBM counters")
    ap.add_argument("--workload", type=int, default=2,
                    help="profiling aid: time another workload's stack (1-5); the benchmark line is workload 2")
    ap.add_argument("--regime", action="store_true",
                    help="study: shared vs dense broadcast at N = 1..1000 candidates per request (workload 2 shapes)")
    ap.add_argument("--ugsep", action="store_true",
                    help="the UG-Separation TokenMixer workload (shared vs dense comparator), one JSON line")
    ap.add_argument("--w8a16", action="store_true",
                    help="W8A16 linear vs the bf16 GEMM at the UG-Separation page's W8A16 shapes, one JSON line each")
    ap.add_argument("--order", action="store_true",
                    help="study: contiguous vs shuffled candidate order on workloads 2-5")
    ap.add_argument("--shuffle", action="store_true",
                    help="with --workload k (k != 2): candidates in one random global order (offsets NULL)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the ROCS stack runs on a single MI355X "
              "(requests would shard across GPUs with no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calib:
        torch.cuda.set_device(0)
        copy_calibration()
        return

    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    torch.cuda.set_device(0)
    if args.regime:
        return regime_study(args)
    if args.order:
        return order_study(args)
    if args.ugsep:
        return ugsep_study(args)
    if args.w8a16:
        return w8a16_study(args)
    if args.workload != 2:
        return other_workload(args)
    cfg = S.config(2)
    inp = S.make_inputs(cfg)
    B_r, B_c = cfg.B, int(len(inp["cand2req"]))
    log(f"bench: {cfg.name()} B_r={B_r} B_c={B_c}")

    shared = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
    t_sh, wall_sh = time_steps(shared.run, args.steps, args.warmup)
    ms = t_sh / args.steps * 1e3
    value = B_c * args.steps / t_sh
    log(f"bench: shared {ms:.3f} ms/step, {value:.4g} candidates/s (wall {wall_sh:.3f} s)")
    F, Bts = glm_mlp_work(cfg, B_r, B_c)
    step_s = t_sh / args.steps

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) features, N(0,1/fan_in) weights)",
        "config": {
            "workload": "GLM MLP stack: B_r=256 requests, candidates/request ~U{64..512} (B_c=%d), d_R=d_C=512, "
                        "3 GLM MLP blocks (hidden 1024 per group, ReLU) + residual + group-local RMSNorm, "
                        "scalar GLM head; bf16 storage, fp32 accumulate" % B_c,
            "B_r": B_r, "B_c": B_c, "global_batch": B_c, "seq_len": 0, "parallelism": "single GPU",
        },
        "mfma_util_pct": 100.0 * F / step_s / PEAK_BF16,
        "hbm_util_pct": 100.0 * Bts / step_s / PEAK_HBM,
        "alg_flops_per_step": F,
        "alg_bytes_per_step": Bts,
    }
    out["step_latency"] = step_latencies(shared.run)
    log(f"bench: step latency p50 {out['step_latency']['p50_ms']:.3f} ms, p99 {out['step_latency']['p99_ms']:.3f} ms")
    if not args.no_dense:
        dense = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
        t_de, _ = time_steps(dense.run, args.steps, args.warmup)
        out["dense_broadcast"] = {"value": B_c * args.steps / t_de, "ms_per_step": t_de / args.steps * 1e3}
        out["speedup_vs_dense_broadcast"] = t_de / t_sh
        log(f"bench: dense broadcast {t_de / args.steps * 1e3:.3f} ms/step, speedup {t_de / t_sh:.3f}x")
        del dense
    out["roofline"] = candidate_gemm_roofline(shared, args.roofline_reps)
    log(f"bench: candidate GEMM {out['roofline']['avg_launch_us']:.1f} us/launch, "
        f"{out['roofline']['achieved']:.1f} {out['roofline']['unit']} ({out['roofline']['frac']:.3f} of peak)")
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        log(f"bench: cpu oracle {out['cpu_baseline']['value']:.4g} candidates/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

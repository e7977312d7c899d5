"""Throughput of the ROCS shared forward stack on one MI355X.

One step = one rocs_stack_forward over one batch of the ranking-scale stack
(B = 32 requests, ~1000 candidates each, a user sequence of 1024 events x 512
with a two-layer request-only encoder, four interaction layers each a GLM MLP
of hidden 2048 followed by DCA cross-attention to that depth's shared K/V,
a per-candidate logit head; bf16 storage, fp32 accumulation), inputs resident
in HBM.

Prints one JSON line: candidates/s, MFMA utilisation, the same-GPU
dense-broadcast comparator and its speedup, the roofline of the dominant
kernel (the IKBO candidate GEMM, timed with HIP events on its launch
stream), the GLM MLP stack's numbers as extra keys, and the CPU oracle's
rate on a bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import itertools
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


def glm_mlp_costs(cfg):
    """Per-request and per-candidate FLOPs of the GLM MLP stack ([R] §2.3:
    C_R is paid once per request, C_C once per candidate).

    Request side: each GLM linear's request GEMM [Y_R || Z] = X_R [W_RR; W_CR]^T
    and the head's request dot.  Candidate side: X_C W_CC^T per layer and the
    head's candidate dot."""
    dr, dc, Hr, Hc = cfg.d_r, cfg.d_c, cfg.hid_r, cfg.hidden
    C_R = cfg.n_blocks * (2.0 * dr * (Hr + Hc) + 2.0 * Hr * (dr + dc)) + 2.0 * dr
    C_C = cfg.n_blocks * (2.0 * dc * Hc + 2.0 * Hc * dc) + 2.0 * dc
    return C_R, C_C


def glm_mlp_work(cfg, B_r, B_c):
    """Algorithmic FLOPs and bytes of one shared-execution step (request side
    once, candidate side per candidate); bytes count each kernel's operands
    read once and outputs written once, weights once, Z (fp32) once each way."""
    C_R, C_C = glm_mlp_costs(cfg)
    F = B_r * C_R + B_c * C_C
    dr, dc, Hr, Hc = cfg.d_r, cfg.d_c, cfg.hid_r, cfg.hidden
    Bts = 0.0
    for _ in range(cfg.n_blocks):
        Bts += 2 * (B_r * dr + B_c * dc) + 2 * (B_r * Hr + B_c * Hc)   # up: read x, write h
        Bts += 2 * (dr * (Hr + Hc) + dc * Hc)                           # up weights W_RR, W_CR, W_CC
        Bts += 2 * 4 * B_r * Hc                                         # Z write + read
        Bts += 2 * (B_r * Hr + B_c * Hc) + 2 * 2 * (B_r * dr + B_c * dc)  # down: read h, read residual, write o
        Bts += 2 * (Hr * (dr + dc) + Hc * dc) + 2 * 4 * B_r * dc
        Bts += 2 * 2 * (B_r * dr + B_c * dc)                            # RMSNorm read + write
        Bts += 2 * 4 * B_c                                              # cand2req reads
    Bts += 2 * (B_r * dr + B_c * dc) + 4 * B_c + 4 * B_c                # head: rows, map, logits
    return F, Bts


def dca_costs(cfg):
    """Per-request and per-candidate FLOPs of a DCA stack.  Request side
    ([R] §2.2, request-only encoder; K/V projected once per request and
    depth): encoder layers, K/V projections, each GLM linear's request GEMM,
    the request queries' attention and the head's request dot.  Candidate
    side: each GLM linear's X_C W_CC^T, the candidate query's attention over
    L keys, the head's candidate dot."""
    d, L, ffn, H = cfg.d_seq, cfg.L, cfg.ffn, cfg.hidden
    enc = cfg.n_enc * (2.0 * L * d * 3 * d + 4.0 * L * L * d + 2.0 * L * d * d + 4.0 * L * d * ffn)
    kv = cfg.n_int * 2.0 * L * d * 4 * d
    C_R, C_C = enc + kv, 0.0
    din_r, din_c = cfg.d_r, cfg.d_c
    for _ in range(cfg.n_int):
        if cfg.qgen_lcb:
            C_R += 2.0 * din_r * (din_r + din_c)
            C_C += 2.0 * din_c * din_c
        C_R += 2.0 * din_r * (2 * H) + 2.0 * H * (2 * d) + 4.0 * L * d
        C_C += 2.0 * din_c * H + 2.0 * H * d + 4.0 * L * d
        din_r, din_c = 2 * d, 2 * d
    if cfg.head:
        C_R += 2.0 * din_r
        C_C += 2.0 * din_c
    return C_R, C_C


def dca_work(cfg, B_r, B_c):
    """Algorithmic FLOPs and bytes of one shared DCA stack step.  Bytes count
    each kernel's operands read once and outputs written once (weights once,
    Z and K/V at request size, bf16 activations, fp32 Z)."""
    C_R, C_C = dca_costs(cfg)
    F = B_r * C_R + B_c * C_C
    d, L, ffn, H = cfg.d_seq, cfg.L, cfg.ffn, cfg.hidden
    BL = B_r * L
    enc = (2 * BL * d + 6 * d * d + 6 * BL * d        # QKV projection
           + 6 * BL * d + 2 * BL * d                  # self-attention
           + 6 * BL * d + 2 * d * d                   # out projection + residual
           + 4 * BL * d                               # LayerNorm
           + 2 * BL * d + 2 * ffn * d + 2 * BL * ffn  # FFN1
           + 2 * BL * ffn + 2 * d * ffn + 4 * BL * d  # FFN2 + residual
           + 4 * BL * d)                              # LayerNorm
    Bts = cfg.n_enc * enc + cfg.n_int * (2 * BL * d + 8 * d * d + 8 * BL * d)

    def linear(din_r, din_c, dout_r, dout_c):
        req = 2 * B_r * din_r + 2 * din_r * (dout_r + dout_c) + 2 * B_r * dout_r + 4 * B_r * dout_c
        cand = 2 * B_c * din_c + 2 * dout_c * din_c + 2 * B_c * dout_c + 4 * B_r * dout_c + 4 * B_c
        return req + cand

    din_r, din_c = cfg.d_r, cfg.d_c
    for _ in range(cfg.n_int):
        if cfg.qgen_lcb:
            Bts += linear(din_r, din_c, din_r, din_c)
        Bts += linear(din_r, din_c, H, H) + linear(H, H, d, d)
        Bts += 2 * B_r * d + 4 * BL * d + 2 * B_r * d                 # request-query attention
        Bts += 2 * B_c * d + 4 * BL * d + 2 * B_c * d + 4 * B_c       # candidate-query attention
        din_r, din_c = 2 * d, 2 * d
    if cfg.head:
        Bts += 2 * (B_r * din_r + B_c * din_c) + 8 * B_c
    return F, Bts


def step_series(fn, n=100):
    """Per-step GPU times (ms) of n back-to-back steps, each bracketed by its
    own events on the launch stream (as a serving loop runs them)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in ev])


def latency_summary(t):
    """p50 / p99 / max of a per-step series, plus what shapes its tail: the
    share of steps more than 10 % above the median, the median of the first
    and last quarter of the series (drift), and the lag-1 autocorrelation
    (slow steps in runs point at a slowly varying cause such as clocks;
    isolated ones at interference)."""
    t = np.asarray(t, dtype=np.float64)
    p50 = float(np.percentile(t, 50))
    q = max(1, len(t) // 4)
    d = t - t.mean()
    ac = float(np.dot(d[:-1], d[1:]) / max(np.dot(d, d), 1e-30)) if len(t) > 2 else 0.0
    return {"steps": int(len(t)), "p50_ms": p50, "p99_ms": float(np.percentile(t, 99)), "max_ms": float(t.max()),
            "mean_ms": float(t.mean()), "frac_above_1.1x_p50": float(np.mean(t > 1.1 * p50)),
            "first_quarter_p50_ms": float(np.median(t[:q])), "last_quarter_p50_ms": float(np.median(t[-q:])),
            "lag1_autocorr": ac}


def step_latencies(fn, n=100):
    return latency_summary(step_series(fn, n))


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


ROOFLINE_KERNEL = ("gemm_bf16_big_kernel<256, 256, 2, 4, 2> via rocs_lcb_candidate (interaction-layer MLP1 of the "
                   "ranking stack, layers 2-4: B_c x 1024 -> B_c x 2048, ReLU, Z[m_i] epilogue)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_candidate_gemm_ranking_stack.json")
# sources the candidate GEMM is compiled from (the counters are void once any of them changes)
GEMM_SRCS = [os.path.join(ROOT, "request_candidate_sharing_amd", "csrc", f)
             for f in ("rocs_gemm.hip", "rocs_gemm_tile.inc", "rocs_mfma.h", "rocs_device.h")]


def gemm_source_sha():
    import hashlib

    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    only while the kernel source is the one the counters were taken on."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != gemm_source_sha():
        return None
    return t.get("bytes_per_launch")


def candidate_gemm_roofline(batch, B_r, B_c, K, N, what, reps=10, min_set_bytes=300 << 20):
    """Times the dominant kernel alone: one IKBO candidate GEMM
    (x_c [B_c, K] -> [B_c, N], ReLU, Z[m_i] gathered in the epilogue) launched
    through rocs_lcb_candidate on torch's current stream and bracketed by
    HIP events recorded on that same stream.  Launches rotate over buffer
    sets larger than the 256 MB Infinity Cache in total, so operands come
    from HBM, as in the stack."""
    import torch
    from request_candidate_sharing_amd import rocs as R

    g = torch.Generator(device="cuda").manual_seed(0)
    bf = torch.bfloat16
    w = (torch.randn(N, K, generator=g, device="cuda") * K ** -0.5).to(bf)
    z = torch.randn(B_r, N, generator=g, device="cuda")
    per_set = 2 * B_c * (K + N)
    sets = max(2, -(-min_set_bytes // per_set))
    bufs = [(torch.randn(B_c, K, generator=g, device="cuda").to(bf), torch.empty(B_c, N, device="cuda", dtype=bf))
            for _ in range(sets)]
    s = R.cur_stream()

    def launch(b):
        R.rocs_lcb_candidate(batch, R.ROCS_BF16, b[0], K, K, w, None, N, R.ROCS_ACT_RELU, z, N, None, 0, b[1],
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
    rf["traffic"] = measured_traffic()
    rf["kernel"] = what
    rf["avg_launch_us"] = t * 1e6
    rf["launches_timed"] = reps * sets
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


def copy_bandwidth():
    """The practical HBM ceiling: a plain device copy (torch's copy kernel) at
    stack-like sizes, two buffer pairs in alternation, bytes read + written."""
    import torch

    for mb in (64, 150, 512, 2048):
        n = mb * (1 << 20) // 2
        xs = [torch.ones(n, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        ys = [torch.empty_like(xs[0]) for _ in range(2)]
        for i in range(4):
            ys[i % 2].copy_(xs[i % 2])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 40
        e0.record()
        for i in range(reps):
            ys[i % 2].copy_(xs[i % 2])
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps / 1e3
        print(json.dumps({"study": "copy_bw", "copy_MB": mb, "us": t * 1e6,
                          "TBps_read_plus_write": 2 * n * 2 / t / 1e12}), flush=True)
        del xs, ys


def oracle_threads() -> int:
    """Threads of the BLAS pool the numpy oracle runs on."""
    try:
        from threadpoolctl import threadpool_info

        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(inp, seconds, max_cands=None):
    """The oracle on whole requests of the same batch until about ``seconds``
    of CPU time.  ``max_cands`` caps the sample at the first candidates of
    the first request instead (a request of the ranking-scale stack alone
    takes longer than the bound); the oracle's cost is per candidate, so
    candidates/s is unchanged by the cap."""
    import oracle
    import rocs_synth as S

    threads = oracle_threads()
    counts = inp["counts"]
    if max_cands is not None:
        b = int(np.nonzero(counts)[0][0])
        n = min(int(counts[b]), max_cands)
        sub = dict(inp)
        keep = np.zeros(len(counts), dtype=np.int64)
        keep[b] = n
        sub.update(S.make_batch(keep))
        o = int(inp["offsets"][b])
        sub["x_c"] = inp["x_c"][o:o + n]
        t0 = time.perf_counter()
        oracle.oracle_forward(sub, requests=[b])
        el = time.perf_counter() - t0
        return {"value": n / el, "unit": "candidates/s", "cores": threads, "kind": "oracle",
                "sample": f"float64 numpy oracle (dense masked model, materialized broadcast) on request {b} "
                          f"of the same batch, its first {n} of {int(counts[b])} candidates (the request's "
                          f"sequence encoder included): {n} candidates in {el:.1f} s"}
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
    ser = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED_SERIAL)
    t_se, _ = time_steps(ser.run, args.steps, args.warmup)
    del ser
    out["serial_schedule_ms_per_step"] = t_se / args.steps * 1e3
    fu = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED_FUSED)
    t_fu, _ = time_steps(fu.run, args.steps, args.warmup)
    del fu
    out["fused_glm_ms_per_step"] = t_fu / args.steps * 1e3
    if not args.no_dense:
        de = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
        t_de, _ = time_steps(de.run, args.steps, args.warmup)
        out["dense_broadcast_ms_per_step"] = t_de / args.steps * 1e3
        out["speedup_vs_dense_broadcast"] = t_de / t_sh
    print(json.dumps(out), flush=True)


def rrr_study(args):
    """Request-oriented resource reallocation ([R] §2.3): the GLM MLP stack
    with its request-side path r times as wide (d_R = r 512, hidden_R =
    r 1024; candidate side fixed) at N fixed candidates per request.  For
    each (r, N): the FLOP accounting of the page (C_R once per request, C_C
    per candidate, FLOPs@1 = C_R + C_C, FLOPs@100 = C_C + C_R/100, C_amort(N)
    = C_C + C_R/N), the measured shared and dense-broadcast step times, the
    measured time per candidate, and the step-latency distribution."""
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    rs = [int(x) for x in args.rrr_r.split(",")]
    ns = [int(x) for x in args.rrr_n.split(",")]
    for r in rs:
        for n in ns:
            cfg = S.rrr_config(r, n)
            inp = S.make_inputs(cfg)
            B_r, B_c = cfg.B, int(len(inp["cand2req"]))
            C_R, C_C = glm_mlp_costs(cfg)
            out = {"study": "rrr", "r": r, "n_per_request": n, "B_r": B_r, "B_c": B_c, "d_R": cfg.d_r,
                   "hidden_R": cfg.hid_r, "d_C": cfg.d_c, "hidden_C": cfg.hidden,
                   "C_R_flops": C_R, "C_C_flops": C_C, "C_R_over_C_C": C_R / C_C,
                   "flops_at_1": C_R + C_C, "flops_at_100": C_C + C_R / 100.0, "C_amort_N": C_C + C_R / n}
            st = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
            t_sh, _ = time_steps(st.run, args.steps, args.warmup)
            sh = t_sh / args.steps
            out.update(shared_ms=sh * 1e3, us_per_candidate=sh * 1e6 / B_c, candidates_per_s=B_c / sh)
            out["step_latency"] = latency_summary(step_series(st.run, args.latency_steps))
            del st
            if not args.no_dense:
                de = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
                t_de, _ = time_steps(de.run, args.steps, args.warmup)
                del de
                out.update(dense_broadcast_ms=t_de / args.steps * 1e3, speedup_vs_dense_broadcast=t_de / t_sh)
            print(json.dumps(out), flush=True)


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
    # the U side's FFN on 8-bit weights (ROCS_UGSEP_SHARED_W8A16): whole
    # step, and the U side alone (a batch with no candidates), bf16 vs W8A16
    quant = S.make_ugsep_w8a16(inp)
    w8 = DeviceUgsep(inp, mode=R.ROCS_UGSEP_SHARED_W8A16, quant=quant)
    t_w8, _ = time_steps(w8.run, args.steps, args.warmup)
    del w8
    out.update(w8a16_ms_per_step=t_w8 / args.steps * 1e3, w8a16_candidates_per_s=B_c * args.steps / t_w8)
    # (three copies of the weights in rotation, 315 MB or more of U weights,
    # so the 256 MB MALL cannot serve them from one call to the next)
    inp0 = S.make_ugsep_inputs(cfg, counts=[0] * cfg.B)
    reps = 21 * args.steps
    for mode, key, q in ((R.ROCS_UGSEP_SHARED, "u_side_bf16_us", None),
                         (R.ROCS_UGSEP_SHARED_W8A16, "u_side_w8a16_us", quant)):
        us = [DeviceUgsep(inp0, mode=mode, quant=q) for _ in range(3)]
        it = iter(range(1 << 30))
        t_u, _ = time_steps(lambda: us[next(it) % 3].run(), reps, args.warmup)
        del us
        out[key] = t_u / reps * 1e6
    out["u_side_change_pct"] = 100.0 * (out["u_side_w8a16_us"] / out["u_side_bf16_us"] - 1.0)
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


def fused_glm_study(args):
    """One GLM linear as one launch (request and candidate tiles in one grid,
    completion counters) against the request and candidate launches, on the
    GLM MLP stack's two linears at full size (256 requests, 73,704
    candidates): 512 -> [1024 | 1024] with ReLU, and 1024 -> [512 | 512] with
    a residual.  Both calls write the same bits (checked here)."""
    import torch
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R

    cfg = S.config(2)
    inp = S.make_inputs(cfg)
    B_r = cfg.B
    g = torch.Generator(device="cuda").manual_seed(7)
    bf = torch.bfloat16
    rn = lambda *sh, sc=1.0: (torch.randn(*sh, device="cuda", generator=g) * sc).to(bf)
    st = R.cur_stream()
    ws = torch.empty(R.rocs_lcb_fused_workspace_size(B_r), dtype=torch.uint8, device="cuda")
    # the stack's batch, then 100 and 10 candidates per request (grids of about
    # four rounds of CUs, then less than one)
    batches = [("U{64..512} per request", inp["cand2req"])]
    for n in (100, 10):
        batches.append(("%d per request" % n, np.repeat(np.arange(B_r, dtype=np.int32), n)))
    for (bname, c2r_np), (name, K, N, act, res) in itertools.product(
            batches, (("up 512 -> 1024, ReLU", 512, 1024, R.ROCS_ACT_RELU, False),
                      ("down 1024 -> 512, residual", 1024, 512, R.ROCS_ACT_NONE, True))):
        B_c = int(len(c2r_np))
        counts = np.bincount(c2r_np, minlength=B_r)
        off = torch.as_tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
        c2r = torch.as_tensor(np.ascontiguousarray(c2r_np, dtype=np.int32), device="cuda")
        batch = R.batch(B_r, B_c, off, c2r)
        x_r, x_c = rn(B_r, K), rn(B_c, K)
        w_rr, w_cr, w_cc = rn(N, K, sc=K ** -0.5), rn(N, K, sc=K ** -0.5), rn(N, K, sc=K ** -0.5)
        b_r, b_c = rn(N, sc=0.5), rn(N, sc=0.5)
        r_r, r_c = (rn(B_r, N), rn(B_c, N)) if res else (None, None)
        outs = {}
        for mode in ("two", "one"):
            y_r, y_c = torch.empty(B_r, N, dtype=bf, device="cuda"), torch.empty(B_c, N, dtype=bf, device="cuda")
            z = torch.empty(B_r, N, dtype=torch.float32, device="cuda")
            a = (batch, R.ROCS_BF16, x_r, K, K, x_c, K, K, w_rr, w_cr, w_cc, b_r, b_c, N, N, act, r_r,
                 N if res else 0, r_c, N if res else 0, y_r, N, y_c, N, z, N)
            if mode == "two":
                fn = lambda: R.rocs_lcb_forward(*a, st)
            else:
                fn = lambda: R.rocs_lcb_forward_fused(*a, ws, ws.numel(), st)
            for _ in range(args.warmup * 4):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(args.steps * 5, 100)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            outs[mode] = (e0.elapsed_time(e1) * 1e3 / reps, y_r.clone(), y_c.clone(), z.clone())
        same = all(torch.equal(outs["two"][i], outs["one"][i]) for i in (1, 2, 3))
        print(json.dumps({"study": "fused_glm", "layer": name, "candidates": bname, "B_r": B_r, "B_c": B_c,
                          "two_launches_us": outs["two"][0], "one_launch_us": outs["one"][0],
                          "same_bits": bool(same)}), flush=True)


def blas_reference_study(args):
    """Context only, not the product path: the vendor GEMM (torch.mm, which
    dispatches to hipBLASLt) on the candidate GEMM shapes of the stacks,
    without the fused request-contribution epilogue, and a large square GEMM
    for the practical bf16 rate of the part.  Operands stay resident (the
    same buffers every launch)."""
    import torch

    shapes = [("ranking stack MLP1", 32486, 1024, 2048), ("ranking stack layer-1 MLP1", 32486, 512, 2048),
              ("ranking stack MLP2", 32486, 2048, 512), ("GLM MLP stack up", 73704, 512, 1024),
              ("GLM MLP stack down", 73704, 1024, 512), ("Wukong-style MLP1", 30231, 8960, 1024),
              ("square", 8192, 8192, 8192)]
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, M, K, N in shapes:
        x = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        wt = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(args.warmup):
            torch.mm(x, wt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(args.steps, 30)
        e0.record()
        for _ in range(reps):
            torch.mm(x, wt)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        print(json.dumps({"study": "blas_reference", "shape": name, "M": M, "K": K, "N": N, "us": us,
                          "tflops": 2.0 * M * N * K / us / 1e6, "frac": 2.0 * M * N * K / us / 1e6 / 2500.0}),
              flush=True)
        del x, wt


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
    # the page's shapes, then larger ones where the weight stream dominates, and
    # more activation rows
    for (M, K, N) in S.W8A16_SHAPES + [(16, 4096, 4096), (16, 8192, 8192), (32, 1280, 2560), (64, 1280, 2560),
                                       (32, 4096, 4096)]:
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


def glm_stack_line(args):
    """The GLM MLP stack (B_r = 256, U{64..512} candidates per request, d 512,
    three blocks of hidden 1024) in the shared and dense-broadcast modes:
    extra keys of the headline line."""
    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    cfg = S.config(2)
    inp = S.make_inputs(cfg)
    B_r, B_c = cfg.B, int(len(inp["cand2req"]))
    st = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
    t_sh, _ = time_steps(st.run, args.steps, args.warmup)
    sh = t_sh / args.steps
    F, Bts = glm_mlp_work(cfg, B_r, B_c)
    out = {"workload": "GLM MLP stack: B_r=256, candidates/request ~U{64..512} (B_c=%d), d_R=d_C=512, 3 GLM MLP "
                       "blocks (hidden 1024 per group) + residual + group RMSNorm, scalar head" % B_c,
           "B_r": B_r, "B_c": B_c, "ms_per_step": sh * 1e3, "candidates_per_s": B_c / sh,
           "mfma_util_pct": 100.0 * F / sh / PEAK_BF16, "hbm_util_pct": 100.0 * Bts / sh / PEAK_HBM}
    del st
    ser = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED_SERIAL)
    t_se, _ = time_steps(ser.run, args.steps, args.warmup)
    del ser
    out["serial_schedule_ms_per_step"] = t_se / args.steps * 1e3
    # each GLM linear's request and candidate tiles in one launch
    fu = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED_FUSED)
    t_fu, _ = time_steps(fu.run, args.steps, args.warmup)
    del fu
    out["fused_glm_ms_per_step"] = t_fu / args.steps * 1e3
    if not args.no_dense:
        de = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
        t_de, _ = time_steps(de.run, args.steps, args.warmup)
        del de
        out["dense_broadcast_ms_per_step"] = t_de / args.steps * 1e3
        out["speedup_vs_dense_broadcast"] = t_de / t_sh
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-broadcast comparator")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-glm", action="store_true", help="skip the GLM MLP stack extra keys")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-cands", type=int, default=256,
                    help="candidates of one request the CPU oracle evaluates for the ranking-scale stack")
    ap.add_argument("--roofline-reps", type=int, default=10)
    ap.add_argument("--steady-steps", type=int, default=100,
                    help="steps of the steady-state window timed after the contract's timed steps")
    ap.add_argument("--latency-steps", type=int, default=100)
    ap.add_argument("--copy-calib", action="store_true", help="only run the copy kernel used to scale HBM counters")
    ap.add_argument("--copy-bw", action="store_true", help="study: plain device copy bandwidth (the practical HBM ceiling)")
    ap.add_argument("--workload", type=int, default=5,
                    help="5 (default) is the benchmark line; 1-4 time another workload's stack (profiling aid)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant kernel's timing (the ranking stack's MLP1 candidate GEMM), for counters")
    ap.add_argument("--rrr", action="store_true",
                    help="study: request-side scaling r x candidates per request N on the GLM MLP stack shapes")
    ap.add_argument("--rrr-r", default="1,2,4")
    ap.add_argument("--rrr-n", default="1,10,100,500,1000")
    ap.add_argument("--ugsep", action="store_true",
                    help="the UG-Separation TokenMixer workload (shared vs dense comparator), one JSON line")
    ap.add_argument("--w8a16", action="store_true",
                    help="W8A16 linear vs the bf16 GEMM at the UG-Separation page's W8A16 shapes, one JSON line each")
    ap.add_argument("--blas-ref", action="store_true",
                    help="context: the vendor GEMM (torch.mm) on the stacks' candidate GEMM shapes, no epilogue")
    ap.add_argument("--fused-glm", action="store_true",
                    help="study: a GLM linear as one launch vs two launches (GLM MLP stack shapes)")
    ap.add_argument("--order", action="store_true",
                    help="study: contiguous vs shuffled candidate order on workloads 2-5")
    ap.add_argument("--shuffle", action="store_true",
                    help="with --workload k (k != 5): candidates in one random global order (offsets NULL)")
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
    if args.copy_bw:
        torch.cuda.set_device(0)
        copy_bandwidth()
        return

    import rocs_synth as S
    from request_candidate_sharing_amd import rocs as R
    from request_candidate_sharing_amd.stacks import DeviceStack

    torch.cuda.set_device(0)
    if args.rrr:
        return rrr_study(args)
    if args.order:
        return order_study(args)
    if args.ugsep:
        return ugsep_study(args)
    if args.w8a16:
        return w8a16_study(args)
    if args.fused_glm:
        return fused_glm_study(args)
    if args.blas_ref:
        return blas_reference_study(args)
    if args.workload != 5:
        return other_workload(args)

    cfg = S.config(5)
    if args.roofline_only:
        b = S.make_batch(S.make_inputs(cfg.with_(L=1, n_enc=0, n_int=0, head=False))["counts"])
        c2r = torch.as_tensor(b["cand2req"], device="cuda")
        offs = torch.as_tensor(b["offsets"], device="cuda")
        B_r, B_c = cfg.B, int(b["offsets"][-1])
        rf = candidate_gemm_roofline(R.batch(B_r, B_c, offs, c2r), B_r, B_c, 2 * cfg.d_seq, cfg.hidden,
                                     ROOFLINE_KERNEL, args.roofline_reps)
        print(json.dumps({"roofline_only": rf}), flush=True)
        return
    inp = S.make_inputs(cfg)
    B_r, B_c = cfg.B, int(len(inp["cand2req"]))
    log(f"bench: {cfg.name()} B_r={B_r} B_c={B_c}")
    F, Bts = dca_work(cfg, B_r, B_c)
    shared = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED)
    dense_out = None
    if not args.no_dense:
        # the comparator runs first, so the shared steps below start on a busy, clocked-up GPU
        dense = DeviceStack(inp, mode=R.ROCS_EXEC_DENSE_BROADCAST)
        t_de, _ = time_steps(dense.run, args.steps, args.warmup)
        dense_out = {"value": B_c * args.steps / t_de, "ms_per_step": t_de / args.steps * 1e3}
        log(f"bench: dense broadcast {t_de / args.steps * 1e3:.3f} ms/step")
        del dense

    t_sh, wall_sh = time_steps(shared.run, args.steps, args.warmup)
    ms = t_sh / args.steps * 1e3
    value = B_c * args.steps / t_sh
    step_s = t_sh / args.steps
    log(f"bench: shared {ms:.3f} ms/step, {value:.4g} candidates/s (wall {wall_sh:.3f} s)")

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
        "data": "synthetic (seeded N(0,1) features and sequences, N(0,1/fan_in) weights)",
        "config": {
            "workload": "ranking-scale full stack: B_r=32 requests, ~1000 candidates/request (log-normal +-30%%, "
                        "B_c=%d), user sequence L=1024 x d=512 with a 2-layer request-only encoder (8 heads), "
                        "4 interaction layers each a GLM MLP of hidden 2048 (d_R=d_C=512) + DCA cross-attention "
                        "to that depth's shared K/V, per-candidate logit head; bf16 storage, fp32 accumulate" % B_c,
            "B_r": B_r, "B_c": B_c, "global_batch": B_c, "seq_len": cfg.L, "parallelism": "single GPU",
        },
        "mfma_util_pct": 100.0 * F / step_s / PEAK_BF16,
        "hbm_util_pct": 100.0 * Bts / step_s / PEAK_HBM,
        "alg_flops_per_step": F,
        "alg_bytes_per_step": Bts,
    }
    # the same launches with every one on the caller's stream (no request lane)
    ser = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED_SERIAL)
    t_se, _ = time_steps(ser.run, args.steps, args.warmup)
    del ser
    out["serial_schedule"] = {"ms_per_step": t_se / args.steps * 1e3, "two_lane_saving_ms": t_se / args.steps * 1e3 - ms}
    log(f"bench: serial schedule {t_se / args.steps * 1e3:.3f} ms/step")
    # serial, with each GLM linear's request and candidate tiles in one launch
    fu = DeviceStack(inp, mode=R.ROCS_EXEC_SHARED_FUSED)
    t_fu, _ = time_steps(fu.run, args.steps, args.warmup)
    del fu
    out["fused_glm_schedule"] = {"ms_per_step": t_fu / args.steps * 1e3}
    log(f"bench: fused GLM schedule {t_fu / args.steps * 1e3:.3f} ms/step")
    if dense_out is not None:
        out["dense_broadcast"] = dense_out
        out["speedup_vs_dense_broadcast"] = dense_out["ms_per_step"] / ms
        log(f"bench: speedup vs dense broadcast {out['speedup_vs_dense_broadcast']:.2f}x")
    if args.steady_steps > 0:
        t_st, _ = time_steps(shared.run, args.steady_steps, 0)
        out["steady_state"] = {"steps": args.steady_steps, "ms_per_step": t_st / args.steady_steps * 1e3,
                               "candidates_per_s": B_c * args.steady_steps / t_st}
        log(f"bench: steady state {t_st / args.steady_steps * 1e3:.3f} ms/step over {args.steady_steps} steps")
    if args.latency_steps > 0:
        out["step_latency"] = step_latencies(shared.run, args.latency_steps)
        log(f"bench: step latency p50 {out['step_latency']['p50_ms']:.3f} ms, "
            f"p99 {out['step_latency']['p99_ms']:.3f} ms")
    K, N = 2 * cfg.d_seq, cfg.hidden
    out["roofline"] = candidate_gemm_roofline(shared.batch, B_r, B_c, K, N, ROOFLINE_KERNEL, args.roofline_reps)
    log(f"bench: candidate GEMM {out['roofline']['avg_launch_us']:.1f} us/launch, "
        f"{out['roofline']['achieved']:.1f} {out['roofline']['unit']} ({out['roofline']['frac']:.3f} of peak)")
    del shared
    if not args.no_glm:
        out["glm_mlp_stack"] = glm_stack_line(args)
        log(f"bench: GLM MLP stack {out['glm_mlp_stack']['ms_per_step']:.3f} ms/step")
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, max_cands=args.cpu_cands)
        log(f"bench: cpu oracle {out['cpu_baseline']['value']:.4g} candidates/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

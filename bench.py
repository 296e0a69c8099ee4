"""Benchmark of batched draft verification on one MI355X.

One step = spec_verify_sample on the B=64, gamma=7, V=128256 bf16 workload
(T = 0.7): the row sweep over all 960 target/draft rows, the accept scan and
the residual / bonus draw.  Inputs sit in HBM before timing starts; the step
rotates over R >= 4 input replicas (>= 1 GB) so the 256 MB Infinity Cache
cannot serve them.  Prints ONE JSON line.

Besides the headline: the per-step time distribution (median, p10, p90 from
events around every step), the row sweep alone (the roofline line) and a
plain stream read of the same bytes (the HBM rate reachable on this device),
the same workload under the Zipf recipe (reading B), and the oracle itself on
the host's cores as the CPU baseline (the sampling workload; greedy,
greedy-tree and stochastic-tree verification; the EAGLE-style LM head plus
verification with BLAS on every core).  The CPU-baseline leg, the only one
that runs the oracle, also reports the parity counts of this run's GPU
outputs (headline and Zipf batches) against it.

Secondary legs (same JSON line, "modes"): greedy verification of the same
tensors; early-exit sampling; greedy and stochastic tree verification (B=32,
63-node binary tree); KV-cache compaction to the accepted paths; one EAGLE-2
tree expansion and the re-ranking into a tree; the EAGLE-style LM-head
projection + verification (B=64, gamma=5, d=4096).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
COUNTERS = os.path.join(ROOT, "profiles", "row_stats_b64g7v128k_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-modes", action="store_true", help="skip the greedy / tree / LM-head legs")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle parity counts (they also need the CPU-baseline leg)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work of each oracle baseline leg")
    ap.add_argument("--settle", type=float, default=0.2,
                    help="seconds of each leg's own call before its warm-up steps (GPU clocks leave idle)")
    return ap.parse_args()


def kernel_source_hash():
    """Hash of what the row sweep kernel is built from: its sources and the
    parameter struct it takes (other structs in the shared header do not
    change its code)."""
    import re
    csrc = os.path.join(ROOT, "lossless_draft_verification_03_amd", "csrc")
    h = hashlib.sha1()
    for f in ("rowstats.hip", "sweep_segment.hpp", "sv_common.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "sv_kernels.hpp")) as fh:
        m = re.search(r"struct RowStatsParams \{.*?\n\};", fh.read(), re.S)
    h.update(m.group(0).encode() if m else b"")
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the row sweep from the committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_hash") != kernel_source_hash():
        return None
    return c.get("sweep_hbm_bytes_per_launch")


def time_events(fn, n, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n          # ms per call


def settle(fn, seconds):
    """Run fn(0), fn(1), ... back to back for about `seconds`, then wait for
    the GPU.  An idle MI355X takes some milliseconds of load to bring its
    clocks to their working level (about 10 ms here: the first hundred-odd
    calls of a verification step run 10-15% slower), so every leg first
    loads the GPU with its own call; the warm-up steps and the timed steps
    follow.  The queue is drained every 16 calls so that it never runs far
    ahead of the GPU."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def step_distribution(fn, n, stream):
    """Per-call times (ms) from an event pair around every call, in a pass
    of its own (the headline's timed region has no events inside it)."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    ev[-1][1].synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": round(float(np.median(t)), 5), "p10_ms": round(float(np.percentile(t, 10)), 5),
            "p90_ms": round(float(np.percentile(t, 90)), 5), "calls": n}


# ------------------------------------------------------ oracle worker pool
# The oracle runs in forked worker processes: each inherits the batch below
# (set before the fork, never copied) and takes a slice of its sequences.
_BATCH = {}


def _cpu_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _spans(B, n):
    step = (B + n - 1) // n
    return [(b0, min(B, b0 + step)) for b0 in range(0, B, step)]


def _oracle_slice(span):
    """The oracle on sequences [b0, b1) of the batch; _BATCH["kind"] names the
    verification ("sample" when absent)."""
    import oracle
    b0, b1 = span
    f = _BATCH
    kind = f.get("kind", "sample")
    if kind == "greedy":
        return oracle.verify_greedy(f["target"][b0:b1], f["dtype"], f["tokens"][b0:b1])
    if kind == "tree":
        return oracle.verify_tree(f["target"][b0:b1], f["dtype"], f["tokens"][b0:b1], f["parent"])
    if kind == "tree_sample":
        return oracle.verify_tree_sample(f["target"][b0:b1], f["draft"][b0:b1], f["dtype"], f["tokens"][b0:b1],
                                         f["parent"], f["uniforms"][b0:b1], f["T"], siblings=f["siblings"])
    return oracle.verify_sample(f["target"][b0:b1], f["draft"][b0:b1], f["dtype"], f["tokens"][b0:b1],
                                f["uniforms"][b0:b1], f["T"])


def _classify_slice(span):
    from parity import classify_sample
    acc, out, infos = _oracle_slice(span)
    b0, b1 = span
    res = classify_sample(_BATCH["gacc"][b0:b1], _BATCH["gout"][b0:b1], acc, out, infos)
    return res["exact"], res["explained"], len(res["unexplained"]), [d[3] for d in res["details"]]


def _time_slice(span):
    _oracle_slice(span)
    return span[1] - span[0]


def _with_batch(batch, fn, spans, repeat_until=None):
    """Run fn over the spans in a fork pool with `batch` visible to the
    workers; with repeat_until (seconds), repeat whole passes until at least
    that much wall time has gone.  Returns (results of the last pass,
    passes, seconds)."""
    import multiprocessing
    _BATCH.clear()
    _BATCH.update(batch)
    try:
        with multiprocessing.get_context("fork").Pool(len(spans)) as pool:
            t0 = time.perf_counter()
            passes = 0
            while True:
                res = pool.map(fn, spans)
                passes += 1
                el = time.perf_counter() - t0
                if repeat_until is None or el >= repeat_until:
                    return res, passes, el
    finally:
        _BATCH.clear()


def parity_counts(w, gacc, gout):
    """Sequences whose GPU outputs equal the oracle's, disagreements that an
    oracle margin below 1e-6 explains (with those margins), and unexplained
    ones, over the whole batch."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    B = len(gacc)
    batch = dict(target=w["target"], draft=w["draft"], dtype=w["dtype"], tokens=w["draft_tokens"],
                 uniforms=w["uniforms"], T=float(w["temperature"]), gacc=gacc, gout=gout)
    res, _, _ = _with_batch(batch, _classify_slice, _spans(B, _cpu_workers()))
    return {"sequences": B, "exact": sum(r[0] for r in res), "explained": sum(r[1] for r in res),
            "unexplained": sum(r[2] for r in res), "explained_margins": [m for r in res for m in r[3]],
            "rule": "outputs equal, or the first differing decision at an oracle margin below 1e-6"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); verification shards over the "
              "batch with no exchange, so N GPUs run N independent copies of this benchmark.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import lossless_draft_verification_03_amd as L
    from gen import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    # ------------------------------------------------------------ headline
    w = make_workload("b64g7v128k", cache=True)
    B, g, V, T = w["B"], w["gamma"], w["V"], float(w["temperature"])
    rows_t, rows_d = B * (g + 1), B * g
    R = max(4, args.replicas)
    reps = []
    base = torch.cat([d(w["target"]).view(rows_t, V), d(w["draft"]).view(rows_d, V)], 0)
    for _ in range(R):
        buf = base.clone()                      # target rows then draft rows, contiguous
        reps.append((buf, buf[:rows_t].view(B, g + 1, V), buf[rows_t:].view(B, g, V)))
    del base
    x, u = d(w["draft_tokens"]), d(w["uniforms"])
    ws = L.new_workspace(L.MODE_SAMPLE, B, g, V, device=dev)
    out = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, g + 1), dtype=torch.int32, device=dev))

    def step(i):
        _, t, dr = reps[i % R]
        L.verify_sample(t, dr, x, u, T, ws=ws, out=out)

    settle(step, args.settle)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = B * g / (ms * 1e-3)
    accepted = out[0].float().mean().item()

    # dominant kernel alone: the row sweep over the same 960 rows, launched
    # through spec_row_partials (the same kernel instance spec_verify_sample
    # launches first, with the same segments, writing the same partials)
    rs_out = torch.empty((rows_t + rows_d, L.lib.spec_row_segments(V, L.SPEC_BF16), 24), dtype=torch.uint8,
                         device=dev)

    def sweep(i):
        L.row_partials(reps[i % R][0], T, 1, out=rs_out)

    settle(sweep, args.settle)
    for i in range(args.warmup):
        sweep(i)
    k1_ms = time_events(sweep, args.steps, stream)
    k1_bytes = (rows_t + rows_d) * V * 2
    k1_gbs = k1_bytes / (k1_ms * 1e-3) / 1e9
    step_gbs = k1_bytes / (ms * 1e-3) / 1e9

    result = {
        "metric": "verified positions/s + HBM GB/s (% of peak), B=64 gamma=7 V=128256 bf16",
        "value": round(value, 1),
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: target ~ N(0,2) bf16, draft = target + N(0,0.8), drafts drawn from q)",
        "config": {"workload": "spec_verify_sample B=64 gamma=7 V=128256 bf16 T=0.7", "B": B, "gamma": g,
                   "V": V, "temperature": T, "replicas": R, "parallelism": "single GPU"},
        "hbm_gbs_step": round(step_gbs, 1),
        "hbm_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "mean_accept_len": round(accepted, 3),
        "roofline": {"bound": "hbm", "kernel": "k_row_sweep<bf16,sum> over the 960 rows (spec_row_partials)",
                     "achieved": round(k1_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "bytes_per_launch": k1_bytes,
                     "avg_launch_us": round(k1_ms * 1e3, 2)},
        "wall_s_timed_region": round(wall, 4),
    }
    settle(step, args.settle)
    result["step_distribution"] = step_distribution(step, args.steps, stream)

    # the HBM read rate reachable here: a plain read of the same 246 MB
    # replicas with the sweep's load pattern and no arithmetic
    sink = torch.empty(max(1, L.lib.spec_stream_read_sink_words(k1_bytes)), dtype=torch.int32, device=dev)

    def sread(i):
        L.stream_read(reps[i % R][0], sink=sink)

    settle(sread, args.settle)
    for i in range(args.warmup):
        sread(i)
    sr_ms = time_events(sread, args.steps, stream)
    sr_gbs = k1_bytes / (sr_ms * 1e-3) / 1e9
    result["stream_read"] = {"GBs": round(sr_gbs, 1), "frac_of_peak": round(sr_gbs / HBM_PEAK_GBS, 4),
                             "bytes": k1_bytes, "avg_launch_us": round(sr_ms * 1e3, 2),
                             "sweep_frac_of_stream_read": round(k1_gbs / sr_gbs, 4),
                             "step_frac_of_stream_read": round(step_gbs / sr_gbs, 4)}

    # this run's outputs for the parity counts (one fresh call, outputs
    # filled with -7 first so nothing stale can pass), and greedy mode's; the
    # oracle compares them in the CPU-baseline leg below
    parity_outs = {}
    if not args.no_parity:
        pout = (torch.full((B,), -7, dtype=torch.int32, device=dev),
                torch.full((B, g + 1), -7, dtype=torch.int32, device=dev))
        L.verify_sample(reps[0][1], reps[0][2], x, u, T, ws=ws, out=pout)
        gout_ = (torch.full((B,), -7, dtype=torch.int32, device=dev),
                 torch.full((B, g + 1), -7, dtype=torch.int32, device=dev))
        L.verify_greedy(reps[0][1], x, out=gout_)
        parity_outs["sample"] = (pout[0].cpu().numpy(), pout[1].cpu().numpy())
        parity_outs["greedy"] = (gout_[0].cpu().numpy(), gout_[1].cpu().numpy())

    # the same shapes under the Zipf recipe (target N(0, 3) - 1.1 ln pi(v)
    # over one seeded permutation, draft noise N(0, 0.8))
    wb = make_workload("b64g7v128k", logits="zipf", target_std=3.0, zipf_slope=1.1, cache=True)
    base_b = torch.cat([d(wb["target"]).view(rows_t, V), d(wb["draft"]).view(rows_d, V)], 0)
    reps_b = []
    for _ in range(4):
        buf = base_b.clone()
        reps_b.append((buf[:rows_t].view(B, g + 1, V), buf[rows_t:].view(B, g, V)))
    del base_b
    xb, ub = d(wb["draft_tokens"]), d(wb["uniforms"])
    bout = (torch.full((B,), -7, dtype=torch.int32, device=dev), torch.full((B, g + 1), -7, dtype=torch.int32,
                                                                           device=dev))

    def bstep_(i):
        L.verify_sample(reps_b[i % 4][0], reps_b[i % 4][1], xb, ub, T, ws=ws, out=bout)

    settle(bstep_, args.settle)
    for i in range(args.warmup):
        bstep_(i)
    bms = time_events(bstep_, args.steps, stream)
    result["reading_b_zipf"] = {"ms": round(bms, 5), "positions_per_s": round(B * g / (bms * 1e-3), 1),
                                "hbm_frac_step": round(k1_bytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "mean_accept_len": round(bout[0].float().mean().item(), 3)}
    if not args.no_parity:
        parity_outs["zipf"] = (bout[0].cpu().numpy(), bout[1].cpu().numpy())
    del reps_b
    torch.cuda.empty_cache()

    # ------------------------------------------------------- other modes
    if not args.no_modes:
        modes = {}
        # the small stochastic case: B = 8, gamma = 5, V = 32000, fp32 Zipf
        # logits (11.3 MB a call, latency-bound); 24 replicas (270 MB) rotate
        # so the Infinity Cache cannot serve them
        wz = make_workload("zipf32k", cache=True)
        zB, zg, zV, zT = wz["B"], wz["gamma"], wz["V"], float(wz["temperature"])
        zbase = torch.cat([d(wz["target"]).reshape(-1), d(wz["draft"]).reshape(-1)])
        zn_t = zB * (zg + 1) * zV
        zreps = []
        for _ in range(24):
            zbuf = zbase.clone()
            zreps.append((zbuf[:zn_t].view(zB, zg + 1, zV), zbuf[zn_t:].view(zB, zg, zV)))
        del zbase
        zx, zu = d(wz["draft_tokens"]), d(wz["uniforms"])
        zws = L.new_workspace(L.MODE_SAMPLE, zB, zg, zV, device=dev)
        zout = (torch.empty(zB, dtype=torch.int32, device=dev), torch.empty((zB, zg + 1), dtype=torch.int32, device=dev))

        def zstep(i):
            L.verify_sample(zreps[i % 24][0], zreps[i % 24][1], zx, zu, zT, ws=zws, out=zout)

        settle(zstep, args.settle)
        for i in range(args.warmup):
            zstep(i)
        zms = time_events(zstep, args.steps, stream)
        zbytes = zB * (2 * zg + 1) * zV * 4
        modes["sample_b8g5v32k_f32_zipf"] = {
            "ms": round(zms, 5), "positions_per_s": round(zB * zg / (zms * 1e-3), 1), "bytes": zbytes,
            "GBs": round(zbytes / (zms * 1e-3) / 1e9, 1), "mean_accept_len": round(zout[0].float().mean().item(), 3)}
        del zreps
        # greedy on the same replicas (target rows only)
        gws = L.new_workspace(L.MODE_GREEDY, B, g, V, device=dev)
        gout = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, g + 1), dtype=torch.int32, device=dev))

        def gstep(i):
            L.verify_greedy(reps[i % R][1], x, ws=gws, out=gout)

        settle(gstep, args.settle)
        for i in range(args.warmup):
            gstep(i)
        gms = time_events(gstep, args.steps, stream)
        gbytes = rows_t * V * 2
        modes["greedy_b64g7v128k"] = {"ms": round(gms, 5), "positions_per_s": round(B * g / (gms * 1e-3), 1),
                                      "GBs": round(gbytes / (gms * 1e-3) / 1e9, 1),
                                      "frac": round(gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # early-exit verification on the same replicas, then on a batch with
        # low acceptance (draft noise 3.0) against the full sweep
        def ee_blocks(K):
            # the library's blocks: K positions each; K = 0: position 0, then
            # the rest; K = -1: 1, 2, 4, ... positions
            out, i0, n = [], 0, (K if K > 0 else 1)
            while i0 <= g:
                out.append((i0, min(i0 + n, g + 1)))
                i0, n = min(i0 + n, g + 1), (K if K > 0 else (g if K == 0 else 2 * n))
            return out

        def ee_bytes(acc_h, K):
            # a sequence reads a block iff it accepted every position before the
            # block; a position has a target row and, below gamma, a draft row
            j = np.clip(acc_h, 0, g)
            rows = 0
            for i0, i1 in ee_blocks(K):
                live = j >= i0
                rows += int(live.sum()) * ((i1 - i0) + (min(i1, g) - min(i0, g)))
            return rows * V * 2
        K_auto = 0

        eout = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty((B, g + 1), dtype=torch.int32, device=dev))

        def estep(i, K=0):
            _, t, dr = reps[i % R]
            L.verify_sample(t, dr, x, u, T, ws=ws, out=eout, early_exit=True, positions_per_launch=K)

        settle(estep, args.settle)
        for i in range(args.warmup):
            estep(i)
            estep(i, 1)
            estep(i, -1)
        ems1 = time_events(lambda i: estep(i, 1), args.steps, stream)
        emsd = time_events(lambda i: estep(i, -1), args.steps, stream)
        ems = time_events(estep, args.steps, stream)
        ee = {"ms": round(ems, 5), "blocks": ee_blocks(K_auto),
              "positions_per_s": round(B * g / (ems * 1e-3), 1),
              "rows_bytes_read": ee_bytes(eout[0].cpu().numpy(), K_auto), "full_sweep_ms": round(ms, 5),
              "ms_one_position_per_launch": round(ems1, 5),
              "ms_doubling_blocks": round(emsd, 5)}
        del reps
        torch.cuda.empty_cache()
        wl = make_workload("b64g7v128k", draft_noise=3.0, seed=5)
        lo_base = torch.cat([d(wl["target"]).view(rows_t, V), d(wl["draft"]).view(rows_d, V)], 0)
        lo = []
        for _ in range(4):
            buf = lo_base.clone()
            lo.append((buf[:rows_t].view(B, g + 1, V), buf[rows_t:].view(B, g, V)))
        del lo_base
        lx, lu = d(wl["draft_tokens"]), d(wl["uniforms"])

        def lstep(i, early, K=0):
            L.verify_sample(lo[i % 4][0], lo[i % 4][1], lx, lu, T, ws=ws, out=eout, early_exit=early,
                            positions_per_launch=K)

        settle(lambda i: lstep(i, False), args.settle)
        for i in range(args.warmup):
            lstep(i, False)
            lstep(i, True)
            lstep(i, True, 1)
            lstep(i, True, -1)
        lfull = time_events(lambda i: lstep(i, False), args.steps, stream)
        lee1 = time_events(lambda i: lstep(i, True, 1), args.steps, stream)
        leed = time_events(lambda i: lstep(i, True, -1), args.steps, stream)
        lee = time_events(lambda i: lstep(i, True), args.steps, stream)
        ee["low_acceptance"] = {"draft_noise": 3.0, "mean_accept_len": round(eout[0].float().mean().item(), 3),
                                "full_sweep_ms": round(lfull, 5), "early_exit_ms": round(lee, 5),
                                "early_exit_ms_one_position_per_launch": round(lee1, 5),
                                "early_exit_ms_doubling_blocks": round(leed, 5),
                                "rows_bytes_read": ee_bytes(eout[0].cpu().numpy(), K_auto)}
        del lo
        torch.cuda.empty_cache()
        # the same low-acceptance sequences tiled to 256 (4x the bytes per position)
        B4 = 4 * B
        t4 = np.concatenate([wl["target"]] * 4, 0)
        d4 = np.concatenate([wl["draft"]] * 4, 0)
        lo4 = [(d(t4), d(d4)) for _ in range(2)]
        del t4, d4
        x4, u4 = d(np.concatenate([wl["draft_tokens"]] * 4, 0)), d(np.concatenate([wl["uniforms"]] * 4, 0))
        ws4 = L.new_workspace(L.MODE_SAMPLE, B4, g, V, device=dev)
        out4 = (torch.empty(B4, dtype=torch.int32, device=dev), torch.empty((B4, g + 1), dtype=torch.int32, device=dev))

        def l4(i, early, K=0):
            L.verify_sample(lo4[i % 2][0], lo4[i % 2][1], x4, u4, T, ws=ws4, out=out4, early_exit=early,
                            positions_per_launch=K)

        settle(lambda i: l4(i, False), args.settle)
        for i in range(2):
            l4(i, False)
            l4(i, True)
            l4(i, True, 1)
            l4(i, True, -1)
        ee["low_acceptance_b256"] = {
            "full_sweep_ms": round(time_events(lambda i: l4(i, False), 10, stream), 5),
            "early_exit_ms": round(time_events(lambda i: l4(i, True), 10, stream), 5),
            "early_exit_ms_one_position_per_launch": round(time_events(lambda i: l4(i, True, 1), 10, stream), 5),
            "early_exit_ms_doubling_blocks": round(time_events(lambda i: l4(i, True, -1), 10, stream), 5)}
        modes["early_exit_b64g7v128k"] = ee
        del lo4, ws4
        torch.cuda.empty_cache()
        # tree
        tw = make_workload("tree63", cache=True)
        tt = d(tw["target"])
        tt2 = tt.clone()
        tn, tp = d(tw["node_tokens"]), d(tw["parent"])
        tws = L.new_workspace(L.MODE_TREE, tw["B"], tw["N"], tw["V"], device=dev)
        tout = (torch.empty(tw["B"], dtype=torch.int32, device=dev),
                torch.empty((tw["B"], tw["N"]), dtype=torch.int32, device=dev),
                torch.empty((tw["B"], tw["N"]), dtype=torch.int32, device=dev))

        def tstep(i):
            L.verify_tree(tt if i % 2 == 0 else tt2, tn, tp, ws=tws, out=tout)

        settle(tstep, args.settle)
        for i in range(args.warmup):
            tstep(i)
        tms = time_events(tstep, args.steps, stream)
        tbytes = tw["B"] * tw["N"] * tw["V"] * 2
        modes["tree_b32n63v128k"] = {"ms": round(tms, 5),
                                     "nodes_per_s": round(tw["B"] * (tw["N"] - 1) / (tms * 1e-3), 1),
                                     "GBs": round(tbytes / (tms * 1e-3) / 1e9, 1),
                                     "frac": round(tbytes / (tms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "mean_accept_len": round(tout[0].float().mean().item(), 3)}
        del tt, tt2
        torch.cuda.empty_cache()
        # stochastic tree verification: 32 sequences, 63-node binary tree,
        # target and draft rows bf16, children drawn from their parent's q
        sw = make_workload("tree_sample63", cache=True)
        st_, sd_ = d(sw["target"]), d(sw["draft"])
        sn, sp, su = d(sw["node_tokens"]), d(sw["parent"]), d(sw["uniforms"])
        sws = L.new_workspace(L.MODE_TREE_SAMPLE, sw["B"], sw["N"], sw["V"], -1, device=dev)   # n_sweep -1
        sout = (torch.empty(sw["B"], dtype=torch.int32, device=dev),
                torch.empty((sw["B"], sw["N"]), dtype=torch.int32, device=dev),
                torch.empty((sw["B"], sw["N"]), dtype=torch.int32, device=dev))
        sT = float(sw["temperature"])

        def sstep(i):
            L.verify_tree_sample(st_, sd_, sn, sp, su, sT, ws=sws, out=sout)

        settle(sstep, args.settle)
        for i in range(args.warmup):
            sstep(i)
        sms = time_events(sstep, args.steps, stream)
        # the verifier reads a swept prefix of nodes plus the nodes its walks
        # visit; full_sweep_equiv_GBs is the rate a sweep of every node's two
        # rows would need to finish in the same time
        sbytes = 2 * sw["B"] * sw["N"] * sw["V"] * 2
        modes["tree_sample_b32n63v128k"] = {
            "ms": round(sms, 5), "sequences_per_s": round(sw["B"] / (sms * 1e-3), 1),
            "full_sweep_equiv_GBs": round(sbytes / (sms * 1e-3) / 1e9, 1),
            "mean_accept_len": round(sout[0].float().mean().item(), 3),
            "max_accept_len": int(sout[0].max().item())}
        del st_, sd_
        # the same shapes with each node's two children drawn from q without
        # replacement (distinct tokens, the top-k style of tree)
        rw = make_workload("tree_sample63", siblings="without_replacement", seed=3, cache=True)
        rt_, rd_ = d(rw["target"]), d(rw["draft"])
        rn, rp, ru = d(rw["node_tokens"]), d(rw["parent"]), d(rw["uniforms"])

        def rstep(i):
            L.verify_tree_sample(rt_, rd_, rn, rp, ru, sT, ws=sws, out=sout, siblings="without_replacement")

        settle(rstep, args.settle)
        for i in range(args.warmup):
            rstep(i)
        rms = time_events(rstep, args.steps, stream)
        modes["tree_sample_distinct_b32n63v128k"] = {
            "ms": round(rms, 5), "sequences_per_s": round(rw["B"] / (rms * 1e-3), 1),
            "mean_accept_len": round(sout[0].float().mean().item(), 3),
            "max_accept_len": int(sout[0].max().item())}
        del rt_, rd_, sws
        torch.cuda.empty_cache()
        # KV compaction to the paths the tree verifier accepted: a cache of
        # 32 layers x (K, V) planes of 8 heads x 128 bf16 per entry
        kB, kP, kE = tw["B"], 64, 8 * 128 * 2
        kS = 512 + tw["N"]
        kv = torch.zeros((kB, kP, kS, kE), dtype=torch.uint8, device=dev)
        kpre = torch.from_numpy(np.random.default_rng(0).integers(0, 513, kB).astype(np.int32)).to(dev)
        kacc, kpath = tout[0].clone(), tout[1].clone()
        knew = torch.empty(kB, dtype=torch.int32, device=dev)

        def kstep(i):
            L.kv_compact(kv, kpre, kacc, kpath, new_len=knew)

        settle(kstep, args.settle)
        for i in range(args.warmup):
            kstep(i)
        kms = time_events(kstep, args.steps, stream)
        acc_h, path_h = kacc.cpu().numpy(), kpath.cpu().numpy()
        moved = sum(int(np.sum(path_h[b, :acc_h[b]] != np.arange(1, acc_h[b] + 1))) for b in range(kB))
        kbytes = 2 * moved * kP * kE
        modes["kv_compact_b32n63_l32h8d128"] = {
            "ms": round(kms, 5), "entries_moved": moved * kP, "bytes_moved": kbytes,
            "GBs": round(kbytes / (kms * 1e-3) / 1e9, 1), "frac": round(kbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del kv
        torch.cuda.empty_cache()
        # EAGLE-2 tree: one expansion depth (32 sequences x 8 frontier rows,
        # top-8 children each, next frontier 8) over bf16 draft rows, then
        # re-ranking a 6-depth table to 63 drafted nodes
        xB, xK, xk = 32, 8, 8
        gen_t = torch.Generator(device=dev).manual_seed(0)
        xrep = [(torch.randn((xB, xK, V), device=dev, generator=gen_t) * 2.0).to(torch.bfloat16) for _ in range(4)]
        xcap = 1 + xk + 5 * xK * xk
        xtable = L.new_tree_table(xB, xcap, torch.zeros(xB, dtype=torch.int32), device=dev)
        # a depth-1 frontier of 8 nodes under the root
        xtable[0][:, 1:1 + xK] = 0
        xtable[1][:, 1:1 + xK] = torch.arange(xK, dtype=torch.int32, device=dev)
        xtable[2][:, 1:1 + xK] = -0.25 * torch.arange(1, xK + 1, dtype=torch.float64, device=dev)
        xtable[3][:, 1:1 + xK] = 1
        xfront = torch.arange(1, xK + 1, dtype=torch.int32, device=dev).repeat(xB, 1)
        xws = L.new_workspace(L.MODE_TREE_EXPAND, xB, xK, V, device=dev)
        xnext = torch.empty((xB, xK), dtype=torch.int32, device=dev)

        def xstep(i):
            L.tree_expand(xrep[i % 4], xfront, xtable, 1 + xK, 1.0, xk, xK, ws=xws, next_frontier=xnext)

        settle(xstep, args.settle)
        for i in range(args.warmup):
            xstep(i)
        xms = time_events(xstep, args.steps, stream)
        xbytes = xB * xK * V * 2
        # fill the remaining depths so the build has a full table
        off = 1 + xK + xK * xk
        fr = xnext.clone()
        for dpt in range(4):
            L.tree_expand(xrep[dpt % 4], fr, xtable, off, 1.0, xk, xK, ws=xws, next_frontier=xnext)
            off += xK * xk
            fr = xnext.clone()
        bout = L.tree_build(xtable, off, 63)

        def bstep(i):
            L.tree_build(xtable, off, 63, out=bout)

        settle(bstep, args.settle)
        for i in range(args.warmup):
            bstep(i)
        bms = time_events(bstep, args.steps, stream)
        modes["tree_expand_b32k8v128k"] = {
            "ms": round(xms, 5), "rows_per_s": round(xB * xK / (xms * 1e-3), 1),
            "GBs": round(xbytes / (xms * 1e-3) / 1e9, 1), "frac": round(xbytes / (xms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "build_ms_63_of_%d" % off: round(bms, 5)}
        del xrep
        torch.cuda.empty_cache()
        # EAGLE-style LM head
        ew = make_workload("eagle_lmhead", cache=True)
        eB, eg, ed, eV = ew["B"], ew["gamma"], ew["d"], ew["V"]
        ft, fd, W = d(ew["feat_t"]), d(ew["feat_d"]), d(ew["W"])
        ex, eu = d(ew["draft_tokens"]), d(ew["uniforms"])
        ews = L.new_workspace(L.MODE_LMHEAD, eB, eg, eV, ed, device=dev)
        eout = (torch.empty(eB, dtype=torch.int32, device=dev), torch.empty((eB, eg + 1), dtype=torch.int32, device=dev))
        M = eB * (2 * eg + 1)
        flops = 2.0 * M * ed * eV
        proj_out = torch.empty((M, eV), dtype=torch.float32, device=dev)
        fcat = torch.cat([ft, fd], 0)
        # the same head in the [V, d] layout a linear layer's weight is stored in
        Wvd = W.t().contiguous()
        # the projection as lmhead_verify runs it: feature rows staged in a
        # workspace first (lmhead_project_staged)
        pws = torch.empty(L.lib.lmhead_project_workspace_bytes(M, ed), dtype=torch.uint8, device=dev)
        for name, layout, Wl in (("w_vd", L.W_VD, Wvd), ("w_dv", L.W_DV, W)):
            def pstep(i, Wl=Wl, layout=layout):
                L.lmhead_project(fcat, Wl, out=proj_out, layout=layout, ws=pws)

            def estep(i, Wl=Wl, layout=layout):
                L.lmhead_verify(ft, fd, Wl, ex, eu, float(ew["temperature"]), ws=ews, out=eout, layout=layout)

            # the engine clock settles after tens of ms of MFMA work: time the
            # GEMM at its steady state
            settle(pstep, args.settle)
            for i in range(60):
                pstep(i)
            pms = time_events(pstep, 20, stream)
            settle(estep, args.settle)
            for i in range(3):
                estep(i)
            ems = time_events(estep, 20, stream)
            modes[f"eagle_lmhead_b64g5d4096_{name}"] = {
                "ms": round(ems, 4), "positions_per_s": round(eB * eg / (ems * 1e-3), 1),
                "gemm_ms": round(pms, 4), "gemm_tflops": round(flops / (pms * 1e-3) / 1e12, 1),
                "gemm_frac": round(flops / (pms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del Wvd
        result["modes"] = modes

    # --------------------------------------------------------- CPU baseline
    # (the only leg that runs the oracle: the baseline timings, and the parity
    # counts of the GPU outputs captured above)
    if not args.no_cpu_baseline and parity_outs:
        result["parity"] = parity_counts(w, *parity_outs["sample"])
        import oracle
        oacc, oout = oracle.verify_greedy(w["target"], "bf16", w["draft_tokens"])
        gacc_, gout_np = parity_outs["greedy"]
        result["parity"]["greedy_bit_exact_sequences"] = int(np.sum(
            (gacc_ == oacc) & np.all(gout_np == oout, axis=1)))
        result["reading_b_zipf"]["parity"] = parity_counts(wb, *parity_outs["zipf"])
    if not args.no_cpu_baseline:
        # the oracle as it stands, float64 NumPy, on the headline batch: the
        # 64 sequences split over one forked worker process per core, whole
        # passes repeated for about args.cpu_seconds
        nw = _cpu_workers()
        batch = dict(target=w["target"], draft=w["draft"], dtype="bf16", tokens=w["draft_tokens"],
                     uniforms=w["uniforms"], T=T)
        _, passes, el = _with_batch(batch, _time_slice, _spans(B, nw), repeat_until=args.cpu_seconds)
        result["cpu_baseline"] = {"value": round(passes * B * g / el, 2), "unit": "verified positions/s",
                                  "cores": nw, "kind": "oracle",
                                  "sample": f"{passes} passes over the same {B}-sequence batch (B=64 gamma=7 "
                                            f"V=128256 bf16), sequences split over {nw} forked worker "
                                            f"processes (float64 NumPy, one thread each), {el:.1f} s",
                                  "gpu_over_cpu": round(value / (passes * B * g / el), 1)}
        if not args.no_modes:
            # the other verifications, the same way (forked workers over the
            # sequences, whole passes for about half of args.cpu_seconds)
            def mode_leg(key, batch, B_, units, unit, what, gpu):
                _, passes, el = _with_batch(batch, _time_slice, _spans(B_, nw), repeat_until=args.cpu_seconds / 2)
                cv = passes * units / el
                result["cpu_baseline"][key] = {
                    "value": round(cv, 2), "unit": unit, "cores": nw, "kind": "oracle",
                    "sample": f"{passes} passes over {what}, sequences split over {nw} forked worker processes "
                              f"(float64 NumPy), {el:.1f} s",
                    "gpu_over_cpu": round(gpu / cv, 1) if gpu else None}

            md = result.get("modes", {})
            mode_leg("greedy_b64g7v128k", dict(kind="greedy", target=w["target"], dtype="bf16",
                                                tokens=w["draft_tokens"]),
                     B, B * g, "verified positions/s", f"the same {B}-sequence batch (greedy, target rows only)",
                     md.get("greedy_b64g7v128k", {}).get("positions_per_s"))
            tw = make_workload("tree63", cache=True)
            mode_leg("tree_b32n63v128k", dict(kind="tree", target=tw["target"], dtype="bf16",
                                               tokens=tw["node_tokens"], parent=tw["parent"]),
                     tw["B"], tw["B"] * (tw["N"] - 1), "verified nodes/s",
                     f"{tw['B']} greedy trees of {tw['N']} nodes (V={tw['V']} bf16)",
                     md.get("tree_b32n63v128k", {}).get("nodes_per_s"))
            sw = make_workload("tree_sample63", cache=True)
            mode_leg("tree_sample_b32n63v128k", dict(kind="tree_sample", target=sw["target"], draft=sw["draft"],
                                                      dtype="bf16", tokens=sw["node_tokens"], parent=sw["parent"],
                                                      uniforms=sw["uniforms"], T=float(sw["temperature"]),
                                                      siblings="iid"),
                     sw["B"], sw["B"], "sequences/s",
                     f"{sw['B']} sampled trees of {sw['N']} nodes (V={sw['V']} bf16, i.i.d. siblings)",
                     md.get("tree_sample_b32n63v128k", {}).get("sequences_per_s"))
            del tw, sw
            # the EAGLE-style path: float64 LM head (BLAS on every core) and
            # verification of the resulting logits, 16 sequences per pass
            import oracle
            from threadpoolctl import threadpool_limits
            ew = make_workload("eagle_lmhead", cache=True)
            eB, eg = ew["B"], ew["gamma"]
            nseq = 16
            rt = np.concatenate([np.arange(b * (eg + 1), (b + 1) * (eg + 1)) for b in range(nseq)])
            rd = np.concatenate([np.arange(b * eg, (b + 1) * eg) for b in range(nseq)])
            with threadpool_limits(limits=nw):
                t0, passes = time.perf_counter(), 0
                while True:
                    oracle.lmhead_verify(ew["feat_t"][rt], ew["feat_d"][rd], ew["W"], ew["draft_tokens"][:nseq],
                                         ew["uniforms"][:nseq], float(ew["temperature"]))
                    passes += 1
                    el = time.perf_counter() - t0
                    if el >= args.cpu_seconds:
                        break
            cv = passes * nseq * eg / el
            e_gpu = result.get("modes", {}).get("eagle_lmhead_b64g5d4096_w_dv", {}).get("positions_per_s")
            result["cpu_baseline"]["eagle_lmhead_b64g5d4096"] = {
                "value": round(cv, 2), "unit": "verified positions/s", "cores": nw, "kind": "oracle",
                "sample": f"{passes} passes over {nseq} of the 64 sequences ({nseq * (2 * eg + 1)} feature rows, "
                          f"float64 GEMM with BLAS on {nw} threads, then verification), {el:.1f} s",
                "gpu_over_cpu": round(e_gpu / cv, 1) if e_gpu else None}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of one DSpark draft/verify step on one MI355X.

One step = dspark_draft_markov_conf (gamma sequential Markov-head positions,
then the confidence head) -> [dspark_schedule] -> dspark_verify, on seeded synthetic
inputs already resident in HBM.  The headline workload is B=128 requests,
gamma=7, V=151936, r=256, temperature 1 with the confidence head (d=4096);
every request verifies all gamma positions, so one step verifies B*gamma
draft positions.

Prints one JSON line (see the fields below).  Usage:
    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--workload sample]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

METRIC = "verified draft positions/sec at B=128,γ=7,V=152k; % of HBM roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the part needs a few dozen steps to reach its steady clocks and caches:
    # 5 warm-up steps read ~4% slow, 50 are within noise of 100
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="sample", choices=["tiny", "greedy", "sample", "sched", "rnn"])
    ap.add_argument("--seed", type=int, default=0x5EED)
    ap.add_argument("--cpu-sample", type=int, default=128,
                    help="requests of the same batch the CPU oracle runs for cpu_baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle step (new seed each pass) until this much time has passed")
    ap.add_argument("--cpu-max-passes", type=int, default=8)
    ap.add_argument("--cpu-single-sample", type=int, default=32,
                    help="requests of the batch the single-thread oracle run covers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-diag", action="store_true",
                    help="skip timing the acceptance-probability diagnostic pass")
    ap.add_argument("--diag-calls", type=int, default=10)
    ap.add_argument("--no-timing-pass", action="store_true",
                    help="skip the per-kernel event pass (used under a profiler)")
    ap.add_argument("--draft-crossover", action="store_true",
                    help="time draft calls of the whole-draft kernel against the per-position sweeps over batch "
                         "sizes (instead of the step benchmark)")
    ap.add_argument("--sts-fit", action="store_true",
                    help="time the per-position temperature fit on a held-out set of 2^20 drafts "
                         "(gamma 7, 64 candidates, 15 bins) instead of the step benchmark; one JSON line")
    ap.add_argument("--verify-layout", action="store_true",
                    help="time one verify call with the target padded to gamma + 1 rows per request against "
                         "the same call with the target rows packed end to end (scheduled workload, K_b from "
                         "the GPU scheduler) instead of the step benchmark; one JSON line")
    ap.add_argument("--schedule", action="store_true",
                    help="time the synchronous and asynchronous prefix schedulers over batch sizes (gamma 7, "
                         "4096-entry SPS table), each checked against the oracle, instead of the step "
                         "benchmark; one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer a few times: the reference kernel of known "
                         "traffic used to scale the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration(n_iter: int = 3):
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n_iter):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                      "iterations": n_iter}))


def draft_crossover(seed: int):
    """Draft call time (gamma = 7, V = 151936, r = 256) of the whole-draft
    kernel against the per-position sweeps over batch sizes, sampling and
    greedy: the measurement behind the library's default batch bound for the
    whole-draft kernel.  Prints one JSON line per (T, B)."""
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    import semi_ar_draft_amd as dk

    def ctx_with(v):
        old = os.environ.get("DSPARK_PERSIST")
        os.environ["DSPARK_PERSIST"] = v
        try:
            return dk.Context(0)
        finally:
            if old is None:
                del os.environ["DSPARK_PERSIST"]
            else:
                os.environ["DSPARK_PERSIST"] = old

    wl = synth.WORKLOADS["sample"].with_(conf=False)
    inp = synth.make_inputs(wl, seed=seed)
    U, W1, W2 = inp["U"].cuda(), inp["W1"].cuda(), inp["W2"].cuda()
    anc, req = inp["anchor"].cuda(), inp["req_ids"].cuda()
    G = wl.gamma
    whole, sweeps = ctx_with("2"), ctx_with("0")
    for T in (1.0, 0.0):
        for B in (16, 32, 48, 64, 96, 128):
            us = []
            for ctx in (whole, sweeps):
                out = (torch.empty((B, G), dtype=torch.int32, device="cuda"),
                       torch.empty((B, G), dtype=torch.float32, device="cuda"),
                       torch.empty((B, G), dtype=torch.float32, device="cuda"))
                for i in range(3):
                    ctx.draft_markov(U[:B], W1, W2, anc[:B], req[:B], T, 11 + i, G, out=out)
                ctx.check()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                for i in range(30):
                    ctx.draft_markov(U[:B], W1, W2, anc[:B], req[:B], T, 100 + i, G, out=out)
                b.record()
                torch.cuda.synchronize()
                ctx.check()
                us.append(1e3 * a.elapsed_time(b) / 30)
            print(json.dumps({"temperature": T, "B": B, "gamma": G, "V": wl.V, "whole_draft_us": round(us[0], 1),
                              "per_position_sweeps_us": round(us[1], 1), "speedup": round(us[1] / us[0], 3)}),
                  flush=True)
    whole.close()
    sweeps.close()


# ALU roofline of the temperature fit's scoring pass.  An evaluation (one
# draft, one candidate) needs at least: 5 fp32 operations (scale the logit,
# 1 + e, times the prefix, times M for the bin, label - score), 2
# transcendental ones (exponential, reciprocal) and 1 float-to-int conversion
# (the bin); the accumulation goes to LDS, a separate pipe.  Issue rates per
# CU per clock: 128 fp32 lanes (the published 157.3 TFLOP/s = 256 CUs x
# 2.4 GHz x 128 lanes x 2 for an FMA), a quarter of that for the
# transcendental instructions and half for conversions (both measured on this
# part with independent instruction chains: 31 and ~64 lanes per CU per
# clock).  Peak = 256 x 2.4 GHz / (5/128 + 2/32 + 1/64) evaluations per second.
STS_CU_CYCLES_PER_EVAL = 5 / 128 + 2 / 32 + 1 / 64
STS_PEAK_GEVALS = 256 * 2.4e9 / STS_CU_CYCLES_PER_EVAL / 1e9


def sts_fit_bench(args):
    """Fit of the per-position confidence temperatures on a synthetic held-out
    set: N = 2^20 drafts of gamma = 7 positions, 64 candidate temperatures,
    15 bins.  value = candidate evaluations (N x candidates x positions) per
    second of whole fits."""
    import torch
    import synth
    import semi_ar_draft_amd as dk

    N, G, n_grid, M = 1 << 20, 7, 64, 15
    d = synth.sts_calibration_set(N, G, seed=2024)
    grid = synth.sts_grid(n_grid)
    l, a, gd = d["logit"].cuda(), d["accept_len"].cuda(), grid.cuda()
    ctx = dk.Context(0)
    out = (torch.empty((G,), dtype=torch.float32, device="cuda"), torch.empty((G,), dtype=torch.int32, device="cuda"),
           torch.empty((G, n_grid), dtype=torch.float64, device="cuda"))
    steps, warmup = max(args.steps, 1), max(args.warmup, 0)
    for _ in range(warmup):
        ctx.sts_fit(l, a, gd, M, out=out)
    ctx.check()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx.sts_fit(l, a, gd, M, out=out)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    ctx.check()
    evals = N * n_grid * G
    # per-kernel durations: events attached to each dispatch
    ctx.timing(True)
    ctx.read_timing()
    for _ in range(steps):
        ctx.sts_fit(l, a, gd, M, out=out)
    tm = ctx.read_timing()
    ctx.timing(False)
    ctx.check()
    h_ms, h_n = tm["sts_fit"]
    hist_us = 1e3 * h_ms / h_n
    achieved = N * n_grid / (hist_us * 1e-6) / 1e9          # Geval/s of one scoring pass
    line = {
        "metric": "STS temperature fit: candidate evaluations/sec (drafts x candidates x positions)",
        "value": evals / (ms * 1e-3), "unit": "evaluations/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sts_fit", "N": N, "gamma": G, "candidates": n_grid, "bins": M},
        "roofline": {"bound": "alu", "kernel": "sts_hist", "achieved": achieved, "peak": STS_PEAK_GEVALS,
                     "unit": "Geval/s", "frac": achieved / STS_PEAK_GEVALS,
                     "traffic": profile_traffic(STS_TRAFFIC_PROFILE, {"name": "sts_fit", "N": N, "gamma": G,
                                                                      "candidates": n_grid, "bins": M})},
        "kernels_us": {"sts_hist_per_position": hist_us},
    }
    if not args.no_cpu_baseline:
        import oracle
        ns = 1 << 17
        ll, aa, gg = d["logit"][:ns].numpy(), d["accept_len"][:ns].numpy(), grid.numpy()
        t0 = time.perf_counter()
        oracle.sts_fit(ll, aa, gg, M)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": ns * n_grid * G / dt, "unit": "evaluations/s", "cores": 1,
                                "kind": "oracle", "sample": f"the first {ns} drafts of the same set, one fit"}
    ctx.close()
    print(json.dumps(line), flush=True)


def verify_layout_bench(args):
    """Verification of the scheduled workload (B = 512, gamma = 7, V = 129280)
    with the target padded to gamma + 1 rows per request (dspark_verify)
    against the same call on the target rows 1 .. K_b + 1 packed end to end
    (dspark_verify_packed).  One draft + confidence + schedule gives the
    tokens and K_b; the packed copy is made outside the timed region; the
    two layouts are timed in alternating blocks of calls on the same inputs
    and seed, and their outputs must agree exactly.  value = the packed
    call's time."""
    import torch
    import synth
    import semi_ar_draft_amd as dk

    wl = synth.WORKLOADS["sched"]
    inp = synth.make_inputs(wl)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, G, V = wl.B, wl.gamma, wl.V
    dev = torch.device("cuda", 0)
    ctx = dk.Context(0)
    tok = torch.empty((B, G), dtype=torch.int32, device=dev)
    lse = torch.empty((B, G), dtype=torch.float32, device=dev)
    ytok = torch.empty((B, G), dtype=torch.float32, device=dev)
    conf = torch.empty((B, G), dtype=torch.float32, device=dev)
    surv = torch.empty((B, G), dtype=torch.float32, device=dev)
    K = torch.empty((B,), dtype=torch.int32, device=dev)
    nsel = torch.empty((1,), dtype=torch.int32, device=dev)
    theta = torch.empty((1,), dtype=torch.float64, device=dev)
    T, seed = d["temperature"], args.seed
    ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, seed, G, d["h"], d["E"],
                          d["wc"], d["bc"], d.get("sts_T"), out=(tok, lse, ytok, conf, surv))
    ctx.schedule(surv, d["sps"], out=(K, nsel, theta))
    ctx.check()
    # rows 1 .. K_b + 1 of every request, in request order
    Kc = K.cpu().to(torch.int64)
    offs = torch.zeros(B, dtype=torch.int64)
    offs[1:] = torch.cumsum(Kc + 1, 0)[:-1]
    n_rows = int((Kc + 1).sum().item())
    flat = torch.cat([b * (G + 1) + torch.arange(int(Kc[b]) + 1) for b in range(B)]).to(dev)
    packed = d["target"].reshape(B * (G + 1), V).index_select(0, flat).contiguous()
    toffs = offs.to(torch.int32).to(dev)
    torch.cuda.synchronize()
    outs = {m: (torch.empty((B,), dtype=torch.int32, device=dev),
                torch.empty((B, G + 1), dtype=torch.int32, device=dev)) for m in ("padded", "packed")}

    def call(m):
        if m == "padded":
            ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, K, d["req_ids"], T,
                       seed, out=outs[m])
        else:
            ctx.verify_packed(packed, toffs, d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, K,
                              d["req_ids"], T, seed, out=outs[m])

    n, rounds = max(args.steps, 1), 3
    for m in ("padded", "packed"):
        for _ in range(max(args.warmup, 1)):
            call(m)
    ctx.check()
    torch.cuda.synchronize()
    us = {"padded": [], "packed": []}
    for _ in range(rounds):
        for m in ("padded", "packed"):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                call(m)
            e1.record()
            torch.cuda.synchronize()
            us[m].append(1e3 * e0.elapsed_time(e1) / n)
    ctx.check()
    same = all(torch.equal(a, b) for a, b in zip(outs["padded"], outs["packed"]))
    A = outs["packed"][0].cpu().to(torch.int64)
    needed = int(torch.where(A < Kc, A + 1, Kc + 1).sum().item())
    line = {
        "metric": "verify call time, target rows packed end to end (padded layout beside it)",
        "value": min(us["packed"]), "unit": "us per verify call", "n_gpus": 1, "steps": n * rounds,
        "warmup": max(args.warmup, 1), "ms_per_step": min(us["packed"]) / 1e3, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "sched: B=512 gamma=7 V=129280 r=256 T=1, K_b from the GPU scheduler",
                   "B": B, "gamma": G, "V": V},
        "padded_us": [round(x, 2) for x in us["padded"]], "packed_us": [round(x, 2) for x in us["packed"]],
        "K_sum": int(Kc.sum().item()), "packed_rows": n_rows, "padded_rows": B * (G + 1),
        "needed_rows": needed, "packed_target_bytes": 4 * n_rows * V, "padded_target_bytes": 4 * B * (G + 1) * V,
        "outputs_identical": same,
    }
    ctx.close()
    print(json.dumps(line), flush=True)
    if not same:
        sys.exit(1)


def schedule_bench(args):
    """The prefix schedulers alone: dspark_schedule (synchronous, early stop)
    and dspark_schedule_async (capacity from survivals of an earlier step,
    global search) on synthetic survival rows (each row gamma = 7 sorted
    uniforms) and the 4096-entry SPS table of the scheduled workload, over
    batch sizes up to the library's B * gamma <= 4096, each timed over a
    block of calls between events.  The cpu_baseline leg (unless
    --no-cpu-baseline) times the oracle on the same inputs and compares its
    K, n and theta with the library's (exact, theta to 1e-12).  value = the
    synchronous call at B = 512 (the scheduled workload)."""
    import numpy as np
    import torch
    import synth
    import semi_ar_draft_amd as dk

    G = 7
    sps = synth.sps_table(4096)
    sps_d = sps.cuda()
    ctx = dk.Context(0)
    n = max(args.steps, 1)
    rows, ok = [], True
    for B in (128, 512, 585):
        surv = synth.survival_rows(B, G, seed=900 + B)
        hist = synth.survival_rows(B, G, seed=1900 + B)
        sd, hd = surv.cuda(), hist.cuda()
        out = (torch.empty((B,), dtype=torch.int32, device="cuda"), torch.empty((1,), dtype=torch.int32, device="cuda"),
               torch.empty((1,), dtype=torch.float64, device="cuda"))
        rec = {"B": B, "gamma": G}
        for mode in ("sync", "async"):
            def call():
                if mode == "sync":
                    ctx.schedule(sd, sps_d, out=out)
                else:
                    ctx.schedule_async(sd, hd, sps_d, out=out)
            for _ in range(max(args.warmup, 1)):
                call()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                call()
            e1.record()
            torch.cuda.synchronize()
            ctx.check()
            rec[mode] = {"us_per_call": round(1e3 * e0.elapsed_time(e1) / n, 2),
                         "n_selected": int(out[1].item())}
            if not args.no_cpu_baseline:
                import oracle
                cpu_s = float("inf")
                for _ in range(3):                             # the fastest of three oracle calls
                    t0 = time.perf_counter()
                    ref = oracle.schedule(surv.numpy(), sps.numpy()) if mode == "sync" else \
                        oracle.schedule_async(surv.numpy(), hist.numpy(), sps.numpy())
                    cpu_s = min(cpu_s, time.perf_counter() - t0)
                same = (np.array_equal(out[0].cpu().numpy().astype(np.int64), ref.K)
                        and int(out[1].item()) == ref.n_selected
                        and abs(float(out[2].item()) - ref.theta) <= 1e-12 * abs(ref.theta))
                ok = ok and same
                rec[mode].update({"matches_oracle": same, "oracle_ms_per_call": round(1e3 * cpu_s, 2)})
        rows.append(rec)
        print(f"[bench] schedule B={B}: sync {rec['sync']['us_per_call']} us, async {rec['async']['us_per_call']} us",
              file=sys.stderr, flush=True)
    ctx.close()
    at512 = next(r for r in rows if r["B"] == 512)["sync"]
    v = at512["us_per_call"]
    line = {
        "metric": "prefix scheduler call time (B x gamma candidates, 4096-entry SPS table)",
        "value": v, "unit": "us per call", "n_gpus": 1, "steps": n, "warmup": max(args.warmup, 1),
        "ms_per_step": v / 1e3, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 survivals, f64 scan", "data": "synthetic",
        "config": {"workload": "schedule: gamma=7, SPS 4096 entries, B in {128, 512, 585}", "gamma": G},
        "sizes": rows,
        "cpu_baseline": None if args.no_cpu_baseline else
        {"value": at512["oracle_ms_per_call"] * 1e3, "unit": "us per call", "cores": 1, "kind": "oracle",
         "sample": "one synchronous call at B = 512 on the same input, fastest of three"},
        "parity_ok": None if args.no_cpu_baseline else ok,
    }
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(1)


def stream_read_peak(ctx, n_bytes: int = 1 << 30, reps: int = 10) -> float:
    """Read bandwidth (GB/s) of the library's streaming-read calibration over
    a buffer four times the 256 MB last-level cache, so that every pass
    reads from HBM; each call also runs its one-workgroup sum of the
    partials (~1% of the call)."""
    import torch
    n = n_bytes // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    out = torch.empty((1,), dtype=torch.float32, device="cuda")
    for _ in range(3):
        ctx.stream_read(x, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ctx.stream_read(x, out=out)
    e1.record()
    torch.cuda.synchronize()
    ctx.check()
    if float(out.item()) != float(n):
        raise RuntimeError(f"stream read calibration summed {out.item()} for {n} ones")
    return n_bytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "draft_chain_traffic_B128_V151936_r256_T1.json")


STS_TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                   "sts_fit_traffic_N1048576_g7_c64_b15.json")


def measured_traffic(wl_name, B, V, r, T):
    """HBM bytes per launch of the dominant draft kernel from the committed
    counter profile."""
    return profile_traffic(TRAFFIC_PROFILE, {"name": wl_name, "B": B, "V": V, "r": r, "temperature": T})


def profile_traffic(path, workload):
    """HBM bytes per launch of a kernel from a committed counter profile
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the counter
    reads for a copy kernel of known size).  None when the workload differs
    or the kernel sources have changed since the counters were taken."""
    try:
        with open(path) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    w = prof.get("workload", {})
    if any(w.get(k) != v for k, v in workload.items()):
        return None
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in prof.get("source_files", []):
        try:
            with open(os.path.join(root, rel), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    if h.hexdigest() != prof.get("source_sha256"):
        return None
    return float(prof["traffic_bytes_per_launch"])


def sweep_bytes(B, V, r, wbytes, hbytes=None):
    """Algorithmic HBM bytes of one vocabulary sweep with the head's bias:
    U rows (4 B per logit), the whole W2, the rank-r vectors the bias is
    projected from (gathered W1 rows, or the GRU head's fp32 states)."""
    return 4 * B * V + wbytes * r * V + (wbytes if hbytes is None else hbytes) * B * r


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.draft_crossover:
        draft_crossover(args.seed)
        return
    if args.schedule:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        schedule_bench(args)
        return
    if args.verify_layout:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        verify_layout_bench(args)
        return
    if args.sts_fit:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        sts_fit_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request; each GPU would run its share of the batch)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import semi_ar_draft_amd as dk

    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    inp = synth.make_inputs(wl)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    gru = inp.get("gru")
    if gru is not None:
        d["gru"] = {k: v.cuda() for k, v in gru.items()}
    print(f"[bench] inputs {wl.name} B={wl.B} gamma={wl.gamma} V={wl.V} r={wl.r} "
          f"generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    B, G, V, r = wl.B, wl.gamma, wl.V, wl.r
    dev = torch.device("cuda", 0)
    ctx = dk.Context(0)
    # outputs allocated once, outside the timed region
    tok = torch.empty((B, G), dtype=torch.int32, device=dev)
    lse = torch.empty((B, G), dtype=torch.float32, device=dev)
    ytok = torch.empty((B, G), dtype=torch.float32, device=dev)
    conf = torch.empty((B, G), dtype=torch.float32, device=dev)
    surv = torch.empty((B, G), dtype=torch.float32, device=dev)
    Ksch = torch.empty((B,), dtype=torch.int32, device=dev)
    nsel = torch.empty((1,), dtype=torch.int32, device=dev)
    theta = torch.empty((1,), dtype=torch.float64, device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    states = torch.empty((G, B, r), dtype=torch.float32, device=dev) if gru is not None else None
    n_steps_max = max(args.steps, 1)
    K_log = torch.zeros((n_steps_max, B), dtype=torch.int32, device=dev)
    A_log = torch.zeros((n_steps_max, B), dtype=torch.int32, device=dev)
    T = d["temperature"]
    has_conf = d.get("h") is not None
    sched = d.get("sps") is not None

    def step(i, log=None):
        seed = args.seed ^ i
        if gru is None and has_conf:
            # draft and confidence head; the draft's merge runs in the confidence launch
            ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, seed, G,
                                  d["h"], d["E"], d["wc"], d["bc"], d.get("sts_T"),
                                  out=(tok, lse, ytok, conf, surv))
        elif gru is None:
            ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, seed, G,
                             out=(tok, lse, ytok))
        else:
            ctx.draft_rnn(d["U"], d["W1"], d["W2"], d["gru"], d["req_ids"], T, seed, G,
                          out=(tok, lse, ytok, states))
        if has_conf and gru is not None:
            ctx.confidence(d["h"], d["E"], d["anchor"], tok, d["wc"], d["bc"], d.get("sts_T"),
                           out=(conf, surv))
        K = None
        if sched:
            K = Ksch if log is None else K_log[log]
            ctx.schedule(surv, d["sps"], out=(K, nsel, theta))
        # the timed steps write their accept lengths straight into the log rows
        ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, K,
                   d["req_ids"], T, seed, out=(acc if log is None else A_log[log], out), states=states)

    for i in range(args.warmup):
        step(1000 + i)
    ctx.check()
    torch.cuda.synchronize()

    # ---- timed region: production launch path (graph for the draft loop) ----
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i, log=i)
    e1.record()
    torch.cuda.synchronize()
    ctx.check()
    elapsed_ms = e0.elapsed_time(e1)
    ms_per_step = elapsed_ms / args.steps
    if sched:
        positions = int(K_log[:args.steps].sum().item())
        Ks = K_log[:args.steps].cpu()
    else:
        positions = B * G * args.steps
        Ks = torch.full((args.steps, B), G, dtype=torch.int32)
    A = A_log[:args.steps].cpu()
    value = positions / (elapsed_ms / 1e3)
    needed_rows = float(torch.where(A < Ks, A + 1, Ks + 1).sum().item()) / args.steps
    # rows the verify windows read: the library's windows (rows 1-2, 3-4, then
    # the rest, or DSPARK_VERIFY_WINDOWS) -- a window reads rows lo..min(hi,
    # K_b + 1) of the requests that kept every row before it
    ends = [int(x) for x in os.environ.get("DSPARK_VERIFY_WINDOWS", "2,4").split(",") if x]
    ends = [e for e in ends if e < G + 1] + [G + 1]
    read = torch.zeros_like(Ks)
    lo = 1
    for hi in ends:
        pend = (A >= lo - 1) & (Ks >= lo - 1)
        n = torch.clamp(torch.minimum(torch.full_like(Ks, hi), Ks + 1) - lo + 1, min=0)
        read += torch.where(pend, n, torch.zeros_like(n))
        lo = hi + 1
    read_rows = float(read.sum().item()) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, "
          f"{value / 1e6:.3f} M positions/s", file=sys.stderr, flush=True)

    # ---- per-kernel event pass: same steps, every kernel bracketed by events ----
    per_kernel = {}
    roofline = None
    ms_per_step_timed_pass = None
    if not args.no_timing_pass:
        ctx.timing(True)
        ctx.read_timing()
        torch.cuda.synchronize()
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record()
        for i in range(args.steps):
            step(i)
        f1.record()
        torch.cuda.synchronize()
        ms_per_step_timed_pass = f0.elapsed_time(f1) / args.steps
        tk = ctx.read_timing()
        ctx.timing(False)
        for name, (ms, n) in tk.items():
            if n:
                per_kernel[name] = {"launches_per_step": n / args.steps, "avg_us": 1e3 * ms / n,
                                    "us_per_step": 1e3 * ms / args.steps}
        wbytes = 2 if d["W1"].dtype == torch.bfloat16 else 4
        # dominant kernel: the draft sweep -- one launch per position, or the
        # whole-draft kernel (Markov head, bf16, r = 256, B <= 128): one
        # launch for all gamma positions, W2 read once and held in registers
        # the chained draft (every position in one launch, W2 streamed per
        # position), else the per-position sweeps or the whole-draft kernel
        chained = "draft_chain" in per_kernel
        sw = per_kernel["draft_chain"] if chained else per_kernel["draft_sweep"]
        whole = not chained and gru is None and G > 1 and round(sw["launches_per_step"]) == 1
        pos_per_launch = G if (whole or chained) else 1
        # the library's timing events, attached to each dispatch
        # (hipExtLaunchKernel), bracket the kernel's execution alone
        sweep_timing = "library timing events attached to each sweep dispatch, averaged over the timed steps"
        if whole:
            b_sweep = G * (4 * B * V + wbytes * B * r) + wbytes * r * V
            if os.environ.get("DSPARK_PERSIST_COOP") != "0":
                # no dispatch-attached events for a cooperative launch: stream
                # events around it, which include the ordering gap before it
                sweep_timing = ("library timing events recorded on the stream around each cooperative launch, "
                                "averaged over the timed steps")
        elif chained:
            b_sweep = G * sweep_bytes(B, V, r, wbytes, None)
        else:
            b_sweep = sweep_bytes(B, V, r, wbytes, 4 if gru is not None else None)
        if gru is None and G >= 3:
            # Cross-check, and the cost per launch inside the chain: draft
            # calls of gamma and of gamma' < gamma positions back to back, one
            # event pair per batch; the difference over gamma - gamma' is one
            # sweep plus the dispatch gap before it (the combine cancels).
            # gamma' >= 3 keeps the calls GPU-bound.
            g2 = max(3, G // 2)
            o2 = (torch.empty((B, g2), dtype=torch.int32, device=dev),
                  torch.empty((B, g2), dtype=torch.float32, device=dev),
                  torch.empty((B, g2), dtype=torch.float32, device=dev))

            def draft_batch(g, out, n=50):
                for i in range(3):
                    ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, 7000 + i, g, out=out)
                torch.cuda.synchronize()
                a0 = torch.cuda.Event(enable_timing=True)
                a1 = torch.cuda.Event(enable_timing=True)
                a0.record()
                for i in range(n):
                    ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, 8000 + i, g, out=out)
                a1.record()
                torch.cuda.synchronize()
                return 1e3 * a0.elapsed_time(a1) / n

            if g2 < G:
                t_full = draft_batch(G, (tok, lse, ytok))
                t_part = draft_batch(g2, o2)
                sw["in_chain_us"] = (t_full - t_part) / (G - g2)
                sw["in_chain_timing"] = (f"draft calls of {G} and {g2} positions back to back, one event pair per "
                                         f"50 calls: ({t_full:.1f} - {t_part:.1f}) us / {G - g2}")
        sw["alg_bytes"] = b_sweep
        sw["positions_per_launch"] = pos_per_launch
        sw["alg_GBps"] = b_sweep / (sw["avg_us"] * 1e-6) / 1e9
        sw["mfma_TFLOPs"] = pos_per_launch * 2.0 * B * r * V / (sw["avg_us"] * 1e-6) / 1e12
        if "verify_rows" in per_kernel:
            # rows the accept decisions need: up to the first rejection, or K_b + 1
            vb = 4.0 * V * needed_rows
            vr = per_kernel["verify_rows"]
            vr["alg_bytes_per_step"] = vb
            vr["needed_rows_per_step"] = needed_rows
            vr["read_rows_per_step"] = read_rows
            vr["alg_GBps"] = vb / (vr["us_per_step"] * 1e-6) / 1e9
        if "verify_chain" in per_kernel:
            # one launch reads each request's rows up to its decision: exactly the needed rows
            vb = 4.0 * V * needed_rows
            vc = per_kernel["verify_chain"]
            vc["alg_bytes_per_step"] = vb
            vc["needed_rows_per_step"] = needed_rows
            vc["read_rows_per_step"] = needed_rows
            vc["alg_GBps"] = vb / (vc["us_per_step"] * 1e-6) / 1e9
        if "resid_sweep" in per_kernel:
            n_rej = float((A < Ks).sum().item()) / args.steps
            rb = 8.0 * V * n_rej + wbytes * r * V + wbytes * n_rej * r
            per_kernel["resid_sweep"]["alg_bytes"] = rb
            per_kernel["resid_sweep"]["rows"] = n_rej
            per_kernel["resid_sweep"]["alg_GBps"] = rb / (per_kernel["resid_sweep"]["avg_us"] * 1e-6) / 1e9
        for name in ("confidence", "conf_merge"):
            if name in per_kernel:
                # h rows and gathered E rows (the fused launch also reads the draft's
                # chunk partials, 24 bytes per request, position and chunk: not counted)
                cb = 2.0 * B * G * (wl.d_h + wl.d_e)
                per_kernel[name]["alg_bytes"] = cb
                per_kernel[name]["alg_GBps"] = cb / (per_kernel[name]["avg_us"] * 1e-6) / 1e9
        # what a plain read sustains on this part, for scale
        stream_gbps = stream_read_peak(ctx)
        print(f"[bench] streaming read: {stream_gbps:.1f} GB/s", file=sys.stderr, flush=True)
        for v in per_kernel.values():
            if "alg_GBps" in v:
                v["frac_hbm"] = v["alg_GBps"] / HBM_PEAK_GBPS
                v["frac_stream_read"] = v["alg_GBps"] / stream_gbps
        achieved = sw["alg_GBps"]
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": measured_traffic(wl.name, B, V, r, T) if chained else None,
                    "kernel": ("draft_chain (MFMA Markov bias + vocabulary sweep, every position in one "
                               "launch of persistent workgroups)" if chained else
                               "draft_persist (MFMA Markov bias + vocabulary sweep, all positions in one "
                               "launch, W2 held in registers)" if whole else
                               "draft_sweep (MFMA Markov bias + vocabulary sweep, one position)" if gru is None
                               else "draft_sweep (MFMA GRU-state bias + vocabulary sweep, one position)"),
                    "alg_bytes_per_launch": b_sweep, "avg_launch_us": round(sw["avg_us"], 2),
                    "timing": sweep_timing,
                    "mfma_util": round(sw["mfma_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 5),
                    "stream_read_GBps": round(stream_gbps, 1),
                    "frac_of_stream_read": round(achieved / stream_gbps, 4)}
        print(f"[bench] kernels: " + ", ".join(f"{k} {v['avg_us']:.1f}us x{v['launches_per_step']:.0f}"
                                             for k, v in per_kernel.items()), file=sys.stderr, flush=True)

    # ---- diagnostic pass (outside the step): acceptance probability of
    #      every drafted position of the last step, sum_v min(p_d, p_t) ----
    diag = None
    if T > 0 and not args.no_diag:
        alpha = torch.empty((B, G), dtype=torch.float32, device=dev)

        def diag_call():
            ctx.accept_prob(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, T, states=states,
                            out=alpha)

        diag_call()
        ctx.check()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.diag_calls):
            diag_call()
        g1.record()
        torch.cuda.synchronize()
        ctx.check()
        us = g0.elapsed_time(g1) * 1e3 / args.diag_calls
        wb = 2 if d["W2"].dtype == torch.bfloat16 else 4
        # per position: the target row twice (its log-normaliser must be known
        # before the min can be taken), U, W2 and the bias vectors
        db = G * (8.0 * B * V + sweep_bytes(B, V, r, wb, 4 if gru is not None else None))
        diag = {"kernel": "dspark_accept_prob (target rows + log-normalisers + gamma alpha sweeps + combine)",
                "us_per_call": round(us, 2), "positions_per_s": round(B * G / (us * 1e-6), 1),
                "alg_bytes_per_call": db, "alg_GBps": round(db / (us * 1e-6) / 1e9, 1),
                "frac_hbm": round(db / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "mean_alpha_per_position": [round(float(x), 4) for x in alpha.mean(0).cpu()]}
        print(f"[bench] accept_prob: {us:.1f} us/call, {diag['alg_GBps']} GB/s", file=sys.stderr, flush=True)

    # step-level algorithmic bytes (what one step must move at least: U of
    # every position, W2 once, the bias vectors of every position)
    wbytes = 2 if d["W1"].dtype == torch.bfloat16 else 4
    n_rej_all = float((A < Ks).sum().item()) / args.steps
    # the blueprint's formula: W2 once per position, every target row up to
    # K_b + 1, and the residual's rows and W2 pass
    step_bytes_formula = (G * (4.0 * B * V + wbytes * r * V + (4 if gru is not None else wbytes) * B * r)
                          + (2.0 * B * G * (wl.d_h + wl.d_e) if has_conf else 0.0)
                          + 4.0 * V * float((Ks + 1).sum().item()) / args.steps
                          + (8.0 * V * n_rej_all + wbytes * r * V if (T > 0 and n_rej_all > 0) else 0.0))
    step_bytes = (G * (4.0 * B * V + (4 if gru is not None else wbytes) * B * r) + wbytes * r * V
                  + (2.0 * B * G * (wl.d_h + wl.d_e) if has_conf else 0.0)
                  + 4.0 * V * needed_rows
                  + (8.0 * V * n_rej_all + wbytes * r * V if (T > 0 and n_rej_all > 0) else 0.0))

    # the timed steps 0 and 1 once more (the step is a deterministic function
    # of its inputs and seed), kept for the comparison with the oracle below
    gpu_steps = []
    if not args.no_cpu_baseline and not sched:
        for i in range(min(2, args.cpu_max_passes)):
            step(i, log=0)
            torch.cuda.synchronize()
            gpu_steps.append({"tok": tok.cpu().numpy(), "lse": lse.cpu().numpy(), "ytok": ytok.cpu().numpy(),
                              "conf": conf.cpu().numpy(), "surv": surv.cpu().numpy(),
                              "acc": A_log[0].cpu().numpy(), "out": out.cpu().numpy()})
        ctx.check()

    cpu = None
    parity = None
    if not args.no_cpu_baseline and not sched:
        import oracle
        from threadpoolctl import threadpool_info, threadpool_limits
        sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests"))
        from parity import Report, compare_draft, compare_confidence, compare_verify
        n = min(args.cpu_sample, B)
        rows = list(range(n))
        t = time.time()
        passes = 0
        refs = []
        while passes < args.cpu_max_passes and (passes == 0 or time.time() - t < args.cpu_seconds):
            r_ = oracle.run_step(inp, seed=args.seed ^ passes, rows=rows)
            if passes < len(gpu_steps):
                refs.append(r_)
            passes += 1
        dt = time.time() - t
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        # one host thread, on a smaller sample of the same batch
        n1 = min(args.cpu_single_sample, B)
        with threadpool_limits(limits=1):
            t1 = time.time()
            oracle.run_step(inp, seed=args.seed, rows=list(range(n1)))
            dt1 = time.time() - t1
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": round(passes * n * G / dt, 2), "unit": "verified draft positions/s", "cores": threads,
               "kind": "oracle", "sample": f"{passes} step(s) of {n} of the {B} requests (all {G} positions, "
               f"draft+confidence+verify), float64 numpy, {dt:.1f}s",
               "single_thread": {"value": round(n1 * G / dt1, 2), "cores": 1,
                                 "sample": f"1 step of {n1} of the {B} requests, {dt1:.1f}s"},
               "host": {"cpu_model": model, "nproc": os.cpu_count(),
                        "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}}
        print(f"[bench] cpu oracle: {cpu['value']} positions/s on {threads} threads, "
              f"{cpu['single_thread']['value']} on one", file=sys.stderr, flush=True)
        # the GPU's timed steps 0 and 1 against the oracle's runs of the same
        # seeds: tokens and accept lengths exact, values within 1e-3 relative,
        # near-ties (oracle decision margin below 1e-4) counted, not compared
        rep = Report()
        for g, ref in zip(gpu_steps, refs):
            sl = (lambda x: x[:n])
            rp, taint = compare_draft(sl(g["tok"]), sl(g["lse"]), sl(g["ytok"]), ref.draft, rep=rep)
            compare_confidence(sl(g["conf"]), sl(g["surv"]), ref.conf, taint, rep=rep)
            compare_verify(sl(g["acc"]), sl(g["out"]), ref.ver, taint, None, rep=rep)
        if refs:
            parity = {"steps_compared": len(refs), "requests": n, "compared": rep.compared,
                      "near_ties": rep.ties, "max_rel_err": float(f"{rep.max_rel:.3e}"), "parity_ok": rep.ok(),
                      "problems": rep.problems[:5]}
            print(f"[bench] parity vs oracle: {rep.summary()}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": "f32 logits and statistics; bf16 weights through bf16 MFMA with f32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={B} gamma={G} V={V} r={r} T={T}"
                               + (" GRU head" if gru is not None else " Markov head")
                               + (f" confidence d_h={wl.d_h} d_e={wl.d_e}" if has_conf else "")
                               + (" scheduled" if sched else " K_b=gamma"),
                   "B": B, "gamma": G, "V": V, "r": r, "temperature": T,
                   "positions_per_step": positions / args.steps,
                   "parallelism": "single GPU"},
        # the least a step must move: W2 once per step, target rows up to the
        # first rejection (or K_b + 1)
        "step_alg_bytes": step_bytes,
        "step_alg_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        # the blueprint's count: W2 once per position, target rows 1 .. K_b + 1
        "step_alg_bytes_formula": step_bytes_formula,
        "step_alg_GBps_formula": round(step_bytes_formula / (ms_per_step * 1e-3) / 1e9, 1),
        "accepted_per_step": float(A.sum().item()) / args.steps,
        # accept lengths of every (timed step, request): entry a counts the
        # requests that kept exactly a drafts (0 .. gamma), and the same for
        # the verify lengths K_b the requests were given
        "accept_hist": [int(x) for x in torch.bincount(A.flatten().long(), minlength=G + 1)[:G + 1]],
        "verify_len_hist": [int(x) for x in torch.bincount(Ks.flatten().long(), minlength=G + 1)[:G + 1]],
        # accepted drafts and emitted tokens (accepted + one correction or
        # bonus token per request) per second of the timed steps
        "accepted_tokens_per_s": round(float(A.sum().item()) / (elapsed_ms / 1e3), 1),
        "emitted_tokens_per_s": round(float(A.sum().item() + B * args.steps) / (elapsed_ms / 1e3), 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "near_ties": None if parity is None else parity["near_ties"],
        "parity_ok": None if parity is None else parity["parity_ok"],
        "accept_prob": diag,
        "per_kernel": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                       for k, v in per_kernel.items()},
        "ms_per_step_event_pass": None if ms_per_step_timed_pass is None else round(ms_per_step_timed_pass, 4),
    }
    ctx.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark: paged decode attention KV-read throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long|mixed|short|tiny]

One step = one pkv_decode call (persistent decode kernel + LSE merge when
rows are split) over the whole batch, inputs resident in HBM.  The headline
workload is the single long context (batch 1, 32/8 heads, head_dim 128,
131072 tokens, bf16, 32 splits of 4096 tokens).  Before timing, a parity gate
checks sampled (sequence, KV head) units against the float64 oracle.  The K/V
pools are kept in two copies that steps alternate between, so each step
streams from HBM rather than from the 256 MB last-level cache.

Prints one JSON line.  `value` is KV-read GB/s over the whole step (decode
+ merge, HIP events on the launch stream); `roofline` prices the decode
kernel alone (its own HIP events) against the 8 TB/s HBM peak;
`cpu_baseline` is the oracle timed on a bounded sample on the host cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode-attn KV-read GB/s (% of HBM peak); p99 step latency, 56 sessions"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long", choices=["long", "mixed", "short", "tiny"])
    ap.add_argument("--others", default="mixed,short",
                    help="extra workloads measured in the same run ('' for none; also long_tp8, the "
                         "long context's per-GPU share under 8-way head sharding)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bounded oracle sample for cpu_baseline (0 disables)")
    ap.add_argument("--order", default="canonical", choices=["canonical", "lpt"])
    ap.add_argument("--wg-per-cu", type=int, default=0)
    ap.add_argument("--merge", default="fused", choices=["fused", "separate"])
    ap.add_argument("--schedule", default="atomic", choices=["atomic", "static", "pages", "steal"],
                    help="item assignment of the one-shot launches (pages: split rows' pages "
                         "claimed from a shared cursor; steal: a quarter of each range in a "
                         "pool the row's waves drain)")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--loop-steps", type=int, default=200,
                    help="steps per run of the 56-session resident loop (0 skips the loop)")
    ap.add_argument("--loop-runs", type=int, default=3)
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny configuration's latency")
    ap.add_argument("--density-probe", action=argparse.BooleanOptionalAction, default=True,
                    help="cadenced loop with session churn at a 10 ms beat: late steps at 56 sessions "
                         "and the most sessions (up to 80) with no late step over 3 runs")
    ap.add_argument("--density", action="store_true",
                    help="cadenced loop with session churn: most sessions with no late step "
                         "at periods of 10 and 20 ms (bisection, 3 runs each)")
    ap.add_argument("--no-loop-append", action="store_true",
                    help="skip the second loop measurement, with the KV append inside each step")
    ap.add_argument("--ablations", action="store_true",
                    help="also time the scheduling ablations: static vs atomic item assignment, "
                         "and exact-length bucketed launches vs the compact queue")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "f32"],
                    help="KV-cache element type of the main workload (and of --profile-pass)")
    ap.add_argument("--no-f32", action="store_true",
                    help="skip the fp32 KV-cache measurements (long, mixed and short workloads, session loop)")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic one-shot workloads (default: the measurement seed "
                         "20260623; the session loops keep theirs)")
    ap.add_argument("--config", default="",
                    help="JSON object of pkv_config fields applied to every one-shot configuration "
                         "measured, e.g. '{\"kv_chunk_tokens\": 4096, \"order\": 1}'")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for hardware-counter runs: a few untimed decode steps of the workload, "
                         "then a 1 GiB copy probe of known size (the counter reference)")
    return ap.parse_args()


# Run settings from the command line (main): the workload seed and the
# pkv_config overrides of --config.
RUN = {"seed": None, "config": {}}


def workload(workloads, name, seed=None):
    seed = RUN["seed"] if seed is None else seed
    return workloads.CONFIGS[name]() if seed is None else workloads.CONFIGS[name](seed)


def measure(torch, pkv, workloads, name, steps, warmup, order, wg_per_cu, copies, gate, say,
            merge="fused", schedule=0, kv="bf16", chunk=0, min_warm_ms=0.0):
    wl = workload(workloads, name).with_kv_dtype(kv)
    dev = "cuda"
    q = wl.q(dev)
    pools = []
    for c in range(copies):
        pools.append((wl.pool("k", dev, poison=(c == 0)), wl.pool("v", dev, poison=(c == 0))))
    bt = wl.block_table_t(dev)
    lens = wl.ctx_lens_t(dev)
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device=dev)
    kw = dict(order=pkv.PKV_ORDER_LPT if order == "lpt" else pkv.PKV_ORDER_CANONICAL,
              wg_per_cu=wg_per_cu, schedule=schedule, kv_chunk_tokens=chunk,
              kv_dtype=pkv.PKV_KV_F32 if kv == "f32" else pkv.PKV_KV_BF16,
              merge_mode=pkv.PKV_MERGE_SEPARATE if merge == "separate" else pkv.PKV_MERGE_FUSED)
    kw["scale"] = wl.scale
    kw.update(RUN["config"])
    cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.batch,
                          wl.max_pages_per_seq, **kw)
    stream = torch.cuda.current_stream()
    dec = pkv.PagedDecoder(cfg, stream=stream)
    info = dec.build_queue(wl.ctx_lens)
    tens = [pkv.make_tensors(q, k, v, bt, lens, out, lse) for k, v in pools]

    gate_out = None
    if gate:
        # Correctness gate: one decode now, its outputs copied to the host; the
        # oracle comparison runs after the timed region, so that seconds of host
        # work do not leave the GPU idle (and its clocks down) right before it.
        pkv.pkv_decode(dec.handle, tens[0], stream)
        torch.cuda.synchronize()
        dec.query()
        gate_out = (out.float().cpu().numpy(), lse.cpu().numpy(), workloads.bits_u16(q))

    for i in range(warmup):
        pkv.pkv_decode(dec.handle, tens[i % copies], stream)
    if min_warm_ms > 0:
        # comparisons between runs: keep the GPU busy for at least min_warm_ms
        # first, since the first milliseconds after an idle gap run slower
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        i = 0
        while (time.perf_counter() - t_w) * 1e3 < min_warm_ms:
            for _ in range(10):
                pkv.pkv_decode(dec.handle, tens[i % copies], stream)
                i += 1
            torch.cuda.synchronize()
    # Timed region 1: K back-to-back steps, events only at the two ends.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        pkv.pkv_decode(dec.handle, tens[i % copies], stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    st = dec.query()
    if gate_out is not None:
        from oracle import paged_attention as pa
        o, l, qb = gate_out
        G = wl.num_q_heads // wl.num_kv_heads
        for b, hk in [(0, 0), (wl.batch - 1, wl.num_kv_heads - 1)]:
            L = int(wl.ctx_lens[b])
            npg = -(-L // 16)
            pg = wl.block_table[b, :npg]
            ks = workloads.kv_host(wl.pool_slabs("k", pg, hk))[:, None]
            vs = workloads.kv_host(wl.pool_slabs("v", pg, hk))[:, None]
            ro, rl = pa.range_state(qb[b:b + 1, hk * G:(hk + 1) * G], ks, vs,
                                    np.arange(npg)[None], 0, 0, 0, L, wl.scale, 16)
            err = np.abs(o[b, hk * G:(hk + 1) * G] - ro)
            lerr = np.abs(l[b, hk * G:(hk + 1) * G] - rl)
            if not (err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 2e-2):
                raise SystemExit(f"parity gate failed on {name} ({kv}) unit {(b, hk)}: "
                                 f"max {err.max():.3e} mean {err.mean():.3e} lse {lerr.max():.3e}")
        say(f"parity gate passed ({name}, {kv} cache)")
    ms_step = total_ms / steps
    # With the fused merge a step is one launch of the decode kernel, so the
    # step time of back-to-back launches (HIP events on the launch stream at
    # the two ends of the timed region) is the kernel's average launch
    # duration, launch gaps included.
    res = {
        "workload": name, "kv_dtype": kv, "kv_bytes": info.kv_bytes, "items": info.n_items,
        "chunk_tokens": info.chunk_tokens,
        "split": bool(info.split), "launches_per_step": info.launches_per_step,
        "partial_bytes": info.partial_bytes, "ms_per_step": ms_step,
        "gbs": info.kv_bytes / (ms_step * 1e-3) / 1e9,
        "host_wall_ms_per_step": wall * 1e3 / steps, "grid": st["grid"], "num_cus": st["num_cus"],
        "batch": wl.batch, "ctx_lens_sum": int(wl.ctx_lens.sum()),
    }
    dec.close()
    del pools, tens
    torch.cuda.empty_cache()
    return res, wl


def measure_loop(torch, pkv, workloads, steps, runs, gate, say, append=False, kv="bf16"):
    """The 56-session resident loop: 32 layers of 32/8-head, head_dim 128
    decode attention per session, contexts U[2048, 16384] growing one token
    per step.  The resident kernel is launched once per run; per step the host
    plans the queue, publishes the step and waits for its completion.  Step
    latency = pkv_decode wall time (publish -> completion observed).  With
    append, each step also writes every session's newest token into the
    cache inside the same kernel (pages from a free list), and the cache
    starts with the tokens before step 0 only.  kv = "f32": the same loop
    over an fp32 cache."""
    from oracle import paged_attention as pa
    sl = workloads.session_loop(steps=max(steps, 3), append=append, kv_dtype=kv)
    tag = ("loop+append" if append else "loop") + (" (fp32 cache)" if kv == "f32" else "")
    dev = "cuda"
    t0 = time.perf_counter()
    k, v, q = sl.pools("k", dev), sl.pools("v", dev), sl.queries(dev)
    bt = torch.as_tensor(sl.block_tables).to(dev)
    out = torch.empty((sl.steps, sl.layers, sl.sessions, sl.num_q_heads, sl.head_dim),
                      dtype=torch.bfloat16, device=dev)
    lse = torch.empty((sl.steps, sl.layers, sl.sessions, sl.num_q_heads), dtype=torch.float32,
                      device=dev)
    lens = torch.zeros(sl.sessions, dtype=torch.int32, device=dev)
    new_k = sl.new_kv("k", dev) if append else None
    new_v = sl.new_kv("v", dev) if append else None
    torch.cuda.synchronize()
    say(f"{tag} inputs generated in {time.perf_counter() - t0:.1f} s "
        f"({2 * k.numel() * sl.kv_elem_bytes / 1e9:.1f} GB of K/V)")
    S, H, D = sl.sessions, sl.num_q_heads, sl.head_dim
    strides = (S * H * D, sl.pages_per_layer * sl.num_kv_heads * 16 * D, S * sl.max_pages,
               S * H * D, S * H)
    cfg = pkv.make_config(H, sl.num_kv_heads, D, sl.pages_per_layer, S, sl.max_pages,
                          scale=sl.scale, persistent=1, num_layers=sl.layers, timeout_ms=20000,
                          append=1 if append else 0,
                          kv_dtype=pkv.PKV_KV_F32 if kv == "f32" else pkv.PKV_KV_BF16)
    G = H // sl.num_kv_heads

    def one_run(n):
        # every run starts from the same cache: a run rewrites the rows and
        # block-table entries the previous run appended with the same values
        stream = torch.cuda.Stream()
        dec = pkv.PagedDecoder(cfg, stream=stream)
        if append:
            pkv.pkv_loop_set_free_pages(dec.handle, sl.free_pages)
        lat, plan = [], []
        try:
            for t in range(n):
                a = time.perf_counter()
                info = dec.build_queue(sl.ctx_lens(t))
                b = time.perf_counter()
                extra = dict(new_k=new_k[t], new_v=new_v[t], layer_stride_new=S * sl.num_kv_heads * D) \
                    if append else {}
                tens = pkv.make_tensors(q[t], k, v, bt, lens, out[t], lse[t], batch=S,
                                        block_table_stride=sl.max_pages, layer_strides=strides, **extra)
                pkv.pkv_decode(dec.handle, tens, stream)
                c = time.perf_counter()
                plan.append(b - a)
                lat.append(c - b)
        finally:
            dec.close()
        torch.cuda.synchronize()
        return np.array(lat) * 1e3, np.array(plan) * 1e3, info

    def check(ts):
        o = out.float().cpu().numpy()
        l = lse.cpu().numpy()
        rng = np.random.default_rng(7)
        worst = 0.0
        for t in ts:
            for _ in range(2):
                layer, s, hk = int(rng.integers(sl.layers)), int(rng.integers(S)), int(rng.integers(sl.num_kv_heads))
                L = int(sl.ctx_lens(t)[s])
                npg = -(-L // 16)

                def paged(which):
                    rows = workloads.kv_host(sl.token_rows(which, t, layer, s, hk))
                    full = np.zeros((npg * 16, D), dtype=rows.dtype)
                    full[:L] = rows
                    return full.reshape(npg, 1, 16, D)

                ks, vs = paged("k"), paged("v")
                qg = workloads.bits_u16(sl.query_unit(t, layer, s))[None, hk * G:(hk + 1) * G]
                ro, rl = pa.range_state(qg, ks, vs, np.arange(npg)[None], 0, 0, 0, L, sl.scale, 16)
                err = np.abs(o[t, layer, s, hk * G:(hk + 1) * G] - ro)
                lerr = np.abs(l[t, layer, s, hk * G:(hk + 1) * G] - rl)
                if not (err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 2e-2):
                    raise SystemExit(f"loop parity failed at step {t} layer {layer} session {s} "
                                     f"kv head {hk}: max {err.max():.3e} mean {err.mean():.3e}")
                worst = max(worst, float(err.max()))
        return worst

    if gate:                                   # parity gate before timing
        one_run(3)
        say(f"{tag} parity gate passed (steps 0-2, max abs err {check([0, 1, 2]):.2e})")
    runs_out = []
    for r in range(runs):
        lat, plan, info = one_run(steps)
        runs_out.append(lat)
        say(f"{tag} run {r}: p50 {np.median(lat):.3f} ms p99 {np.percentile(lat, 99):.3f} ms "
            f"max {lat.max():.3f} ms; host planning p50 {np.median(plan):.3f} ms")
    if gate:
        say(f"{tag} parity after timing (steps 0, {steps // 2}, {steps - 1}): max abs err "
            f"{check([0, steps // 2, steps - 1]):.2e}")
    allv = np.concatenate(runs_out)
    step_bytes = np.array([sl.kv_bytes(t) for t in range(steps)])
    gbs = step_bytes / 1e9 / (np.concatenate([x[None] for x in runs_out]).mean(axis=0) * 1e-3)
    res = {"sessions": S, "layers": sl.layers, "steps": steps, "runs": runs,
           "items_per_layer": int(info.n_items), "split": bool(info.split),
           "p50_ms": round(float(np.median(allv)), 4),
           "p99_ms": round(float(np.percentile(allv, 99)), 4),
           "max_ms": round(float(allv.max()), 4),
           "p99_per_run_ms": [round(float(np.percentile(x, 99)), 4) for x in runs_out],
           "kv_gb_per_step_mean": round(float(step_bytes.mean() / 1e9), 3),
           "kv_gbs_median": round(float(np.median(gbs)), 1),
           "pct_of_hbm_peak_median": round(float(np.median(gbs)) / HBM_PEAK_GBS * 100, 2),
           "launches_per_step": 0, "append": bool(append), "kv_dtype": kv}
    del k, v, q, out, lse, new_k, new_v
    torch.cuda.empty_cache()
    return res


def density_search(torch, pkv, workloads, periods_ms, max_sessions, steps, runs, say, probe_sessions=None):
    """Cadenced session loop (WPK note: sessions served on a fixed beat, late
    beats counted, density = most sessions with none late).  Steps are
    published on a clock of period T; a step is late if it completes after its
    next tick.  Sessions come and go: each slot hosts a sequence of sessions
    (lifetimes U[40, 120] steps); when one leaves, the next joins the slot at a
    step boundary with a fresh context (drawn so that it fits the slot's
    pages).  For each T the largest session count with no late step over
    `runs` runs is found by bisection; with probe_sessions, that many sessions
    are also run `runs` times at each T and their late steps counted."""
    from oracle import paged_attention as pa
    dev = "cuda"
    sl = workloads.session_loop(sessions=max_sessions, steps=steps, name="loop_density")
    t0 = time.perf_counter()
    k, v, q = sl.pools("k", dev), sl.pools("v", dev), sl.queries(dev)
    bt = torch.as_tensor(sl.block_tables).to(dev)
    out = torch.empty((sl.steps, sl.layers, sl.sessions, sl.num_q_heads, sl.head_dim),
                      dtype=torch.bfloat16, device=dev)
    lse = torch.empty((sl.steps, sl.layers, sl.sessions, sl.num_q_heads), dtype=torch.float32,
                      device=dev)
    lens_dev = torch.zeros(sl.sessions, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    say(f"density inputs: {max_sessions} session slots, {2 * k.numel() * 2 / 1e9:.1f} GB of K/V, "
        f"{time.perf_counter() - t0:.1f} s")
    # per-slot session schedule: lengths at every step with joins and leaves
    lens, joins = sl.churn_lens(workloads.MEASURE_SEED)
    S_all, H, D = sl.sessions, sl.num_q_heads, sl.head_dim
    strides = (S_all * H * D, sl.pages_per_layer * sl.num_kv_heads * 16 * D, S_all * sl.max_pages,
               S_all * H * D, S_all * H)
    cfg = pkv.make_config(H, sl.num_kv_heads, D, sl.pages_per_layer, S_all, sl.max_pages,
                          scale=sl.scale, persistent=1, num_layers=sl.layers, timeout_ms=20000)

    def run(S, period_s):
        stream = torch.cuda.Stream()
        dec = pkv.PagedDecoder(cfg, stream=stream)
        late, lat = 0, []
        try:
            start = time.perf_counter()
            for t in range(steps):
                tick = start + t * period_s
                while time.perf_counter() < tick:
                    pass
                dec.build_queue(lens[t, :S])
                tens = pkv.make_tensors(q[t], k, v, bt, lens_dev, out[t], lse[t], batch=S,
                                        block_table_stride=sl.max_pages, layer_strides=strides)
                a = time.perf_counter()
                pkv.pkv_decode(dec.handle, tens, stream)
                done = time.perf_counter()
                lat.append(done - a)
                late += done > tick + period_s
        finally:
            dec.close()
        torch.cuda.synchronize()
        return late, np.array(lat) * 1e3

    # parity of churned steps: a slot after a join reads its new, shorter context
    n_chk = min(8, max_sessions)
    _, _ = run(n_chk, 0.0)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    G = H // sl.num_kv_heads
    for t_chk in (steps // 2, steps - 1):
        for layer in (0, sl.layers - 1):
            for s in range(n_chk):
                for hk in (0, sl.num_kv_heads - 1):
                    L = int(lens[t_chk, s])
                    npg = -(-L // 16)
                    pg = sl.block_tables[layer, s, :npg]
                    ks = workloads.bits_u16(sl.slabs("k", layer, pg, hk))[:, None]
                    vs = workloads.bits_u16(sl.slabs("v", layer, pg, hk))[:, None]
                    qg = workloads.bits_u16(sl.query_unit(t_chk, layer, s))[None, hk * G:(hk + 1) * G]
                    ro, rl = pa.range_state(qg, ks, vs, np.arange(npg)[None], 0, 0, 0, L, sl.scale, 16)
                    err = np.abs(o[t_chk, layer, s, hk * G:(hk + 1) * G] - ro)
                    lerr = np.abs(l[t_chk, layer, s, hk * G:(hk + 1) * G] - rl)
                    if not (err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 2e-2):
                        raise SystemExit(f"density loop parity failed: step {t_chk} layer {layer} slot {s} "
                                         f"head {hk}: {err.max():.3e} {lerr.max():.3e}")
    say(f"density loop parity passed ({joins} joins in the schedule)")
    res = {"max_sessions_tried": max_sessions, "steps_per_run": steps, "runs": runs,
           "session_lifetime_steps": [40, 120], "joins_per_run": joins, "periods": {}}
    for T in periods_ms:
        if probe_sessions:
            lates, p99s = [], []
            for _ in range(runs):
                late, lat = run(probe_sessions, T / 1e3)
                lates.append(late)
                p99s.append(float(np.percentile(lat, 99)))
            res[f"probe_{probe_sessions}_sessions_T{T}ms"] = {"late_steps": int(sum(lates)),
                                                              "steps": runs * steps,
                                                              "p99_ms": round(max(p99s), 4)}
            say(f"density probe T={T} ms: {probe_sessions} sessions -> {sum(lates)} late steps of "
                f"{runs * steps}, p99 {max(p99s):.2f} ms")
        lo, hi, best = 1, max_sessions, 0
        best_p99 = None
        while lo <= hi:
            S = (lo + hi) // 2
            lates, p99s = [], []
            for _ in range(runs):
                late, lat = run(S, T / 1e3)
                lates.append(late)
                p99s.append(float(np.percentile(lat, 99)))
                if late:
                    break
            ok = sum(lates) == 0
            say(f"density T={T} ms: {S} sessions -> {sum(lates)} late steps, p99 {max(p99s):.2f} ms")
            if ok:
                best, best_p99 = S, max(p99s)
                lo = S + 1
            else:
                hi = S - 1
        res["periods"][str(T)] = {"sessions": best, "p99_ms_at_density": best_p99}
        say(f"density at T={T} ms: {best} sessions with no late step over {runs} runs")
    del k, v, q, out, lse
    torch.cuda.empty_cache()
    return res


def kernel_code_digest(path):
    """sha256 prefix of a HIP source with its comments and whitespace removed:
    it changes when the code changes, not when a comment does."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


PROFILE_NAMES = {"long": "decode_kernel_long_context", "mixed": "decode_kernel_mixed_batch",
                 "short": "decode_kernel_many_short"}


def measured_traffic(root, workload="long", kv="bf16"):
    """HBM bytes per decode launch of a workload from its committed counter
    summary, if the counters were taken on the kernel code as it is now
    (else None)."""
    import re
    if workload not in PROFILE_NAMES:
        return None
    name = PROFILE_NAMES[workload] + ("_fp32_cache" if kv == "f32" else "") + "_traffic.md"
    prof = os.path.join(root, "profiles", name)
    src = os.path.join(root, "paged_kv_attention_persistent_amd", "csrc", "pkv_kernels.hip")
    try:
        text = open(prof).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        digest = kernel_code_digest(src)
    except Exception:
        return None
    if rec.get("kernel_code_sha256_prefix") != digest:
        return None
    return int(rec["traffic_bytes_per_launch"])


def measure_bucketed(torch, pkv, workloads, name, steps, warmup, say):
    """Exact-length bucketed launches (the baseline the compact queue replaces):
    rows sorted by length, one handle and one launch per distinct length, each
    with its own queue built once; a step is every bucket's launch in turn on
    one stream.  Returns the step rate and the launches and partial-state bytes
    per step."""
    from oracle import paged_attention as pa
    wl = workload(workloads, name)
    dev = "cuda"
    lens = np.asarray(wl.ctx_lens)
    order = np.argsort(lens, kind="stable")
    idx = torch.as_tensor(order, device=dev)
    q = wl.q(dev)[idx].contiguous()
    bt = wl.block_table_t(dev)[idx].contiguous()
    k, v = wl.pool("k", dev, False), wl.pool("v", dev, False)
    slens = lens[order]
    lens_dev = torch.as_tensor(slens.astype(np.int32), device=dev)
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    buckets, b0 = [], 0
    for b in range(1, wl.batch + 1):
        if b == wl.batch or slens[b] != slens[b0]:
            buckets.append((b0, b))
            b0 = b
    decs, tens, launches, partial = [], [], 0, 0
    for (a, b) in buckets:
        cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, b - a,
                              wl.max_pages_per_seq, scale=wl.scale)
        dec = pkv.PagedDecoder(cfg, stream=stream)
        info = dec.build_queue(slens[a:b].tolist())
        launches += info.launches_per_step
        partial += info.partial_bytes
        decs.append(dec)
        tens.append(pkv.make_tensors(q[a:b], k, v, bt[a:b], lens_dev[a:b], out[a:b], lse[a:b],
                                     batch=b - a, block_table_stride=bt.shape[1]))

    def step():
        for dec, t in zip(decs, tens):
            pkv.pkv_decode(dec.handle, t, stream)

    step()
    torch.cuda.synchronize()
    for dec in decs:
        dec.query()
    # parity gate on the first and the last row of the original order
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    qb = workloads.bits_u16(wl.q("cpu"))
    G = wl.num_q_heads // wl.num_kv_heads
    pos = {int(r): i for i, r in enumerate(order)}
    for b, hk in [(0, 0), (wl.batch - 1, wl.num_kv_heads - 1)]:
        L = int(wl.ctx_lens[b])
        npg = -(-L // 16)
        pg = wl.block_table[b, :npg]
        ks = workloads.bits_u16(wl.pool_slabs("k", pg, hk))[:, None]
        vs = workloads.bits_u16(wl.pool_slabs("v", pg, hk))[:, None]
        ro, rl = pa.range_state(qb[b:b + 1, hk * G:(hk + 1) * G], ks, vs, np.arange(npg)[None], 0, 0, 0,
                                L, wl.scale, 16)
        i = pos[b]
        err = np.abs(o[i, hk * G:(hk + 1) * G] - ro).max()
        lerr = np.abs(l[i, hk * G:(hk + 1) * G] - rl).max()
        if not (err <= 2e-2 and lerr <= 2e-2):
            raise SystemExit(f"bucketed parity gate failed on {name} unit {(b, hk)}: {err:.3e} {lerr:.3e}")
    for _ in range(warmup):
        step()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for dec in decs:
        dec.close()
    return {"buckets": len(buckets), "launches_per_step": launches, "partial_bytes": partial,
            "ms_per_step": ms, "gbs": wl.kv_bytes / (ms * 1e-3) / 1e9}


def ablations(torch, pkv, workloads, args, say):
    """Scheduling ablations (static vs atomic item assignment vs page claims vs
    the steal pool; exact-length bucketed launches vs the compact queue) on the one-shot
    workloads, with both cache types for the assignment."""
    res = {"schedule": {}, "bucketed": {}}
    steps = max(args.steps // 2, 10)
    scheds = (("atomic", pkv.PKV_SCHEDULE_ATOMIC), ("static", pkv.PKV_SCHEDULE_STATIC),
              ("pages", pkv.PKV_SCHEDULE_PAGES), ("steal", pkv.PKV_SCHEDULE_STEAL))
    for kv in ("bf16", "f32"):
        for name in ("long", "mixed", "short"):
            # each schedule twice, the second pass in reverse order, after at
            # least 30 ms of warm-up launches; the better run is reported
            row = {}
            for rnd, seq in enumerate((scheds, scheds[::-1])):
                for label, sched in seq:
                    r, _ = measure(torch, pkv, workloads, name, steps, args.warmup, args.order, args.wg_per_cu,
                                   args.copies, not args.no_gate and rnd == 0, say, args.merge, sched, kv=kv,
                                   min_warm_ms=30.0)
                    if label not in row or r["gbs"] > row[label]["gbs"]:
                        row[label] = {"gbs": round(r["gbs"], 1), "us_per_step": round(r["ms_per_step"] * 1e3, 2)}
            key = name if kv == "bf16" else f"{name}_f32"
            res["schedule"][key] = row
            say(f"ablation {key}: atomic {row['atomic']['gbs']} GB/s, static {row['static']['gbs']} GB/s, "
                f"page claims {row['pages']['gbs']} GB/s, steal pool {row['steal']['gbs']} GB/s")
    for name in ("mixed", "short"):
        r, _ = measure(torch, pkv, workloads, name, steps, args.warmup, args.order, args.wg_per_cu,
                       args.copies, False, say, args.merge, min_warm_ms=30.0)
        bk = measure_bucketed(torch, pkv, workloads, name, steps, args.warmup, say)
        res["bucketed"][name] = {
            "compact": {"launches_per_step": r["launches_per_step"], "partial_bytes": r["partial_bytes"],
                        "gbs": round(r["gbs"], 1), "ms_per_step": round(r["ms_per_step"], 4)},
            "bucketed": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in bk.items()}}
        say(f"ablation {name}: compact queue {r['gbs']:.1f} GB/s in {r['launches_per_step']} launch(es); "
            f"bucketed {bk['gbs']:.1f} GB/s in {bk['launches_per_step']} launches ({bk['buckets']} lengths)")
    return res


def _oracle_worker(args):
    """One process of the CPU baseline: regenerate the slabs of its (sequence,
    KV head) units (untimed), wait for the others, then run the float64
    oracle over them pass after pass for `seconds` of wall time.  Returns
    (K+V bytes of the units computed, seconds, units)."""
    root, name, kv, seed, units, seconds, barrier = args
    if root not in sys.path:
        sys.path.insert(0, root)
    from threadpoolctl import threadpool_limits
    import torch
    torch.set_num_threads(1)                         # the input generator, too, on this core only
    from oracle import paged_attention as pa
    from paged_kv_attention_persistent_amd import workloads
    wl = (workloads.CONFIGS[name]() if seed is None else workloads.CONFIGS[name](seed)).with_kv_dtype(kv)
    qb = workloads.bits_u16(wl.q("cpu"))
    G = wl.num_q_heads // wl.num_kv_heads
    data = []
    for b, hk in units:
        L = int(wl.ctx_lens[b])
        npg = -(-L // 16)
        pg = wl.block_table[b, :npg]
        data.append((b, hk, L, npg, workloads.kv_host(wl.pool_slabs("k", pg, hk))[:, None],
                     workloads.kv_host(wl.pool_slabs("v", pg, hk))[:, None]))
    done, n = 0, 0
    with threadpool_limits(limits=1):                # one core per process
        b, hk, L, npg, ks, vs = data[0]              # untimed warm-up (first-touch of temporaries)
        pa.range_state(qb[b:b + 1, hk * G:(hk + 1) * G], ks, vs, np.arange(npg)[None], 0, 0, 0, L,
                       wl.scale, 16)
        barrier.wait()
        t0 = time.perf_counter()
        while n == 0 or time.perf_counter() - t0 < seconds:
            b, hk, L, npg, ks, vs = data[n % len(data)]
            pa.range_state(qb[b:b + 1, hk * G:(hk + 1) * G], ks, vs, np.arange(npg)[None], 0, 0, 0, L,
                           wl.scale, 16)
            done += L * wl.head_dim * wl.kv_elem_bytes * 2
            n += 1
        spent = time.perf_counter() - t0
    return done, spent, n


def cpu_baseline(workloads, wl, seconds, say):
    """The float64 oracle as it stands on whole (sequence, KV head) units of
    the same workload: one process per host core available to this process
    (os.sched_getaffinity), each pinned to one BLAS thread and running its
    share of the units pass after pass for `seconds`; then the same on one
    core.  Throughput = K+V bytes of the units computed / wall seconds.  The
    worker processes are started fresh (spawn), not forked from this one."""
    import multiprocessing as mp
    root = os.path.dirname(os.path.abspath(__file__))
    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    cores = len(os.sched_getaffinity(0))
    ctx = mp.get_context("spawn")
    res = {}
    for label, n_proc in (("all", cores), ("one", 1)):
        if n_proc == 1:
            shares = [units[:1]]                     # one core: the first unit, pass after pass
        else:
            shares = [[units[(i + j * n_proc) % len(units)] for j in range(max(1, -(-len(units) // n_proc)))]
                      for i in range(n_proc)]
        with ctx.Manager() as mgr:
            barrier = mgr.Barrier(n_proc)
            with ctx.Pool(n_proc) as pool:
                out = pool.map(_oracle_worker, [(root, wl.name if wl.name in workloads.CONFIGS else "long",
                                                 wl.kv_dtype, RUN["seed"], sh, seconds, barrier) for sh in shares])
        total = sum(o[0] for o in out)
        wall = max(o[1] for o in out)
        res[label] = {"gbs": total / wall / 1e9, "processes": n_proc, "units": sum(o[2] for o in out),
                      "seconds": wall, "bytes": total}
        say(f"cpu baseline ({n_proc} process{'es' if n_proc > 1 else ''}): {res[label]['gbs']:.2f} GB/s, "
            f"{res[label]['units']} units in {wall:.1f} s")
    a, o = res["all"], res["one"]
    return {"value": round(a["gbs"], 4), "unit": "GB/s", "cores": a["processes"], "kind": "oracle",
            "affinity_cores": cores, "one_core_value": round(o["gbs"], 4),
            "sample": f"float64 NumPy oracle on whole (sequence, KV head) units of the '{wl.name}' workload "
                      f"({len(units)} units of {int(wl.ctx_lens.max())} tokens max), {a['processes']} "
                      f"processes x 1 BLAS thread for {a['seconds']:.1f} s: {a['units']} units, "
                      f"{a['bytes'] / 1e9:.2f} GB of K+V; one core: {o['units']} units in {o['seconds']:.1f} s; "
                      f"inputs regenerated in each process and excluded from the time"}


def read_ceiling(torch, pkv, say, nbytes=2 << 30, reps=5):
    """Measured HBM read ceiling: pkv_read_probe (non-temporal dwordx4 loads,
    sequential) over `nbytes`, `reps` back-to-back launches timed by HIP
    events on the launch stream, at 1, 2 and 3 workgroups per CU; the best."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(3 * cus * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best, best_grid = 0.0, 0
    for per_cu in (1, 2, 3):
        grid = per_cu * cus
        for _ in range(2):
            pkv.pkv_read_probe(src, nbytes, sink, grid, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            pkv.pkv_read_probe(src, nbytes, sink, grid, stream)
        b.record(stream)
        torch.cuda.synchronize()
        gbs = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        if gbs > best:
            best, best_grid = gbs, grid
    say(f"read ceiling: {best:.1f} GB/s ({nbytes >> 20} MiB, grid {best_grid})")
    del src, sink
    torch.cuda.empty_cache()
    return best, best_grid


def tiny_latency(torch, pkv, workloads, steps, say):
    """The tiny configuration (64 KiB of K/V, cache-resident): device time per
    call of back-to-back launches, and the host round trip of one call
    (queue build + decode + synchronise)."""
    r, wl = measure(torch, pkv, workloads, "tiny", steps, 10, "canonical", 0, 1, True, say)
    q, k, v = wl.q("cuda"), wl.pool("k", "cuda", False), wl.pool("v", "cuda", False)
    bt, lens = wl.block_table_t("cuda"), wl.ctx_lens_t("cuda")
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device="cuda")
    cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.batch,
                          wl.max_pages_per_seq, **{"scale": wl.scale, **RUN["config"]})
    dec = pkv.PagedDecoder(cfg)
    t = pkv.make_tensors(q, k, v, bt, lens, out, lse)
    rt = []
    for i in range(steps + 10):
        a = time.perf_counter()
        dec.build_queue(wl.ctx_lens)
        pkv.pkv_decode(dec.handle, t, dec.stream)
        torch.cuda.synchronize()
        if i >= 10:
            rt.append(time.perf_counter() - a)
    dec.close()
    rt = np.array(rt) * 1e6
    say(f"tiny: {r['ms_per_step'] * 1e3:.2f} us per call back to back, host round trip "
        f"p50 {np.median(rt):.1f} us")
    return {"device_us_per_call": round(r["ms_per_step"] * 1e3, 3),
            "host_round_trip_us_p50": round(float(np.median(rt)), 2),
            "host_round_trip_us_p99": round(float(np.percentile(rt, 99)), 2),
            "kv_bytes": r["kv_bytes"], "items": r["items"]}


def profile_pass(torch, pkv, workloads, args, say):
    """Untimed work for rocprofv3 counter passes: `steps` decode calls of the
    workload (alternating two pool copies), then one copy probe moving
    exactly 1 GiB (read 1 GiB, write 1 GiB), whose counter readings give the
    scale from counter units to bytes."""
    wl = workload(workloads, args.workload).with_kv_dtype(args.kv)
    dev = "cuda"
    q = wl.q(dev)
    pools = [(wl.pool("k", dev, False), wl.pool("v", dev, False)) for _ in range(2)]
    bt, lens = wl.block_table_t(dev), wl.ctx_lens_t(dev)
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device=dev)
    kw = dict(scale=wl.scale, kv_dtype=pkv.PKV_KV_F32 if args.kv == "f32" else pkv.PKV_KV_BF16,
              schedule={"atomic": pkv.PKV_SCHEDULE_ATOMIC, "static": pkv.PKV_SCHEDULE_STATIC,
                        "pages": pkv.PKV_SCHEDULE_PAGES, "steal": pkv.PKV_SCHEDULE_STEAL}[args.schedule],
              merge_mode=pkv.PKV_MERGE_SEPARATE if args.merge == "separate" else pkv.PKV_MERGE_FUSED)
    kw.update(RUN["config"])
    cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.batch,
                          wl.max_pages_per_seq, **kw)
    dec = pkv.PagedDecoder(cfg)
    info = dec.build_queue(wl.ctx_lens)
    tens = [pkv.make_tensors(q, k, v, bt, lens, out, lse) for k, v in pools]
    steps = min(args.steps, 20)
    for i in range(steps):
        pkv.pkv_decode(dec.handle, tens[i % 2], dec.stream)
    torch.cuda.synchronize()
    dec.query()
    dec.close()
    del pools, tens
    torch.cuda.empty_cache()
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    pkv.pkv_copy_probe(dst, src, n)
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": args.workload, "kv_dtype": args.kv, "decode_steps": steps,
                      "kv_bytes_per_step": info.kv_bytes, "copy_probe_bytes": n}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(this path runs on a single MI355X; no multi-GPU run exists)", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from paged_kv_attention_persistent_amd import pkv, workloads

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    RUN["seed"] = args.seed
    RUN["config"] = json.loads(args.config) if args.config else {}
    if not isinstance(RUN["config"], dict):
        raise SystemExit("--config takes a JSON object of pkv_config fields")
    pkv.lib()
    if args.profile_pass:
        profile_pass(torch, pkv, workloads, args, say)
        return
    sched = {"atomic": pkv.PKV_SCHEDULE_ATOMIC, "static": pkv.PKV_SCHEDULE_STATIC,
             "pages": pkv.PKV_SCHEDULE_PAGES, "steal": pkv.PKV_SCHEDULE_STEAL}[args.schedule]
    main_res, wl = measure(torch, pkv, workloads, args.workload, args.steps, args.warmup,
                           args.order, args.wg_per_cu, args.copies, not args.no_gate, say, args.merge,
                           sched, kv=args.kv)
    say(f"{args.workload}: {main_res['gbs']:.1f} GB/s per step ({main_res['ms_per_step'] * 1e3:.2f} us, "
        f"{main_res['launches_per_step']} launch per step)")
    keys = ("gbs", "ms_per_step", "items", "split", "chunk_tokens", "kv_bytes", "launches_per_step")
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        r, _ = measure(torch, pkv, workloads, name, max(args.steps // 2, 10), args.warmup,
                       args.order, args.wg_per_cu, args.copies, not args.no_gate, say, args.merge, sched)
        others[name] = {k: r[k] for k in keys}
        others[name]["pct_of_hbm_peak"] = 100.0 * r["gbs"] / HBM_PEAK_GBS
        others[name]["traffic"] = measured_traffic(os.path.dirname(os.path.abspath(__file__)), name)
        say(f"{name}: {r['gbs']:.1f} GB/s per step ({r['ms_per_step'] * 1e3:.2f} us, chunk {r['chunk_tokens']})")
        if name == "mixed":
            # the configuration's stated range length, beside the fitted one
            r, _ = measure(torch, pkv, workloads, name, max(args.steps // 2, 10), args.warmup,
                           args.order, args.wg_per_cu, args.copies, False, say, args.merge, sched, chunk=4096)
            others["mixed_chunk4096"] = {k: r[k] for k in keys}
            others["mixed_chunk4096"]["pct_of_hbm_peak"] = 100.0 * r["gbs"] / HBM_PEAK_GBS
            say(f"mixed at chunk 4096: {r['gbs']:.1f} GB/s per step ({r['items']} items)")
    if not args.no_tiny:
        others["tiny"] = tiny_latency(torch, pkv, workloads, max(args.steps // 2, 10), say)
    f32 = {}
    if not args.no_f32:
        for name in ("long", "mixed", "short"):
            if name == args.workload and args.kv == "f32":
                continue
            r, _ = measure(torch, pkv, workloads, name, max(args.steps // 2, 10), args.warmup,
                           args.order, args.wg_per_cu, args.copies, not args.no_gate, say, args.merge,
                           sched, kv="f32")
            f32[name] = {k: r[k] for k in keys if k != "split"}
            f32[name]["pct_of_hbm_peak"] = 100.0 * r["gbs"] / HBM_PEAK_GBS
            f32[name]["traffic"] = measured_traffic(os.path.dirname(os.path.abspath(__file__)), name, "f32")
            say(f"{name} (fp32 cache): {r['gbs']:.1f} GB/s per step ({r['ms_per_step'] * 1e3:.1f} us)")
    loop = loop_append = loop_f32 = None
    if args.loop_steps > 0:
        loop = measure_loop(torch, pkv, workloads, args.loop_steps, args.loop_runs,
                            not args.no_gate, say)
        if not args.no_loop_append:
            loop_append = measure_loop(torch, pkv, workloads, args.loop_steps, args.loop_runs,
                                       not args.no_gate, say, append=True)
        if not args.no_f32:
            loop_f32 = measure_loop(torch, pkv, workloads, args.loop_steps, args.loop_runs,
                                    not args.no_gate, say, kv="f32")
    abl = ablations(torch, pkv, workloads, args, say) if args.ablations else None
    if args.density:
        density = density_search(torch, pkv, workloads, (10, 20), 160, 100, 3, say, probe_sessions=56)
    elif args.density_probe:
        density = density_search(torch, pkv, workloads, (10,), 80, 100, 3, say, probe_sessions=56)
    else:
        density = None
    ceiling, ceiling_grid = read_ceiling(torch, pkv, say)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(workloads, wl, args.cpu_seconds, say)
    achieved = main_res["gbs"]
    one_launch = main_res["launches_per_step"] == 1
    line = {
        "metric": METRIC,
        "value": round(main_res["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.kv,
        "data": f"synthetic (seeded counter-based N(0,1) {args.kv}; permuted page pool)",
        "pct_of_hbm_peak": round(100.0 * main_res["gbs"] / HBM_PEAK_GBS, 2),
        "config": {"workload": "single long context", "batch": 1, "context_tokens": 131072,
                   "q_heads": 32, "kv_heads": 8, "head_dim": 128, "page_size": 16,
                   "kv_chunk_tokens": main_res["chunk_tokens"], "items": main_res["items"],
                   "launches_per_step": main_res["launches_per_step"],
                   "kv_bytes_per_step": main_res["kv_bytes"], "grid": main_res["grid"],
                   "order": args.order, "merge": args.merge, "schedule": args.schedule,
                   "kv_dtype": args.kv,
                   "seed": workloads.MEASURE_SEED if args.seed is None else args.seed,
                   **({"config_overrides": RUN["config"]} if RUN["config"] else {})}
                  if args.workload == "long" else
                  {"workload": args.workload, "items": main_res["items"], "kv_dtype": args.kv,
                   "kv_bytes_per_step": main_res["kv_bytes"]},
        # achieved: algorithmic K+V bytes per launch / the launch's average
        # duration, from back-to-back launches timed by HIP events on the
        # launch stream (one launch per step with the fused merge)
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__)), args.workload,
                                                 args.kv),
                     "kernel": f"decode_kernel<128,4,{'KvF32' if args.kv == 'f32' else 'KvBf16'}>",
                     "kernel_us_mean": round(main_res["ms_per_step"] * 1e3, 3) if one_launch else None,
                     "bytes_per_launch": main_res["kv_bytes"],
                     "ceiling": {"value": round(ceiling, 1), "unit": "GB/s",
                                 "kind": f"measured streaming read (pkv_read_probe, 2 GiB, grid {ceiling_grid})",
                                 "frac": round(achieved / ceiling, 4)}},
        "cpu_baseline": cpu,
        "session_loop_p99_ms": loop["p99_ms"] if loop else None,
        "session_loop": loop,
        "session_loop_append": loop_append,
        "session_loop_f32": loop_f32,
        "session_density": density,
        "other_workloads": others,
        "kv_f32": f32 or None,
        "ablations": abl,
        "host_wall_ms_per_step": round(main_res["host_wall_ms_per_step"], 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

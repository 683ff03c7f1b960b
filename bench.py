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
                    help="extra workloads measured in the same run ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bounded oracle sample for cpu_baseline (0 disables)")
    ap.add_argument("--order", default="canonical", choices=["canonical", "lpt"])
    ap.add_argument("--wg-per-cu", type=int, default=0)
    ap.add_argument("--merge", default="fused", choices=["fused", "separate"])
    ap.add_argument("--schedule", default="atomic", choices=["atomic", "static", "pages"],
                    help="item assignment of the one-shot launches (pages: split rows' pages "
                         "claimed from a shared cursor)")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--loop-steps", type=int, default=200,
                    help="steps per run of the 56-session resident loop (0 skips the loop)")
    ap.add_argument("--loop-runs", type=int, default=3)
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
    ap.add_argument("--profile-pass", action="store_true",
                    help="for hardware-counter runs: a few untimed decode steps of the workload, "
                         "then a 1 GiB copy probe of known size (the counter reference)")
    return ap.parse_args()


def measure(torch, pkv, workloads, name, steps, warmup, order, wg_per_cu, copies, gate, say,
            merge="fused", schedule=0, kv="bf16"):
    wl = workloads.CONFIGS[name]().with_kv_dtype(kv)
    dev = "cuda"
    q = wl.q(dev)
    pools = []
    for c in range(copies):
        pools.append((wl.pool("k", dev, poison=(c == 0)), wl.pool("v", dev, poison=(c == 0))))
    bt = wl.block_table_t(dev)
    lens = wl.ctx_lens_t(dev)
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device=dev)
    cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.batch,
                          wl.max_pages_per_seq, scale=wl.scale,
                          order=pkv.PKV_ORDER_LPT if order == "lpt" else pkv.PKV_ORDER_CANONICAL,
                          wg_per_cu=wg_per_cu, schedule=schedule,
                          kv_dtype=pkv.PKV_KV_F32 if kv == "f32" else pkv.PKV_KV_BF16,
                          merge_mode=pkv.PKV_MERGE_SEPARATE if merge == "separate" else pkv.PKV_MERGE_FUSED)
    stream = torch.cuda.current_stream()
    dec = pkv.PagedDecoder(cfg, stream=stream)
    info = dec.build_queue(wl.ctx_lens)
    tens = [pkv.make_tensors(q, k, v, bt, lens, out, lse) for k, v in pools]

    if gate:   # correctness gate before any timing (oracle on sampled units)
        from oracle import paged_attention as pa
        pkv.pkv_decode(dec.handle, tens[0], stream)
        torch.cuda.synchronize()
        dec.query()
        o = out.float().cpu().numpy()
        l = lse.cpu().numpy()
        qb = workloads.bits_u16(q)
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

    for i in range(warmup):
        pkv.pkv_decode(dec.handle, tens[i % copies], stream)
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
    # Timed region 2: the same steps with HIP events recorded by the library
    # right around the decode kernel on the launch stream (its own duration).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:                       # torch creates the HIP events on first record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        pkv.pkv_set_decode_events(dec.handle, ev[i][0], ev[i][1])
        pkv.pkv_decode(dec.handle, tens[i % copies], stream)
    torch.cuda.synchronize()
    pkv.pkv_set_decode_events(dec.handle, None, None)
    st = dec.query()
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_step = total_ms / steps
    res = {
        "workload": name, "kv_dtype": kv, "kv_bytes": info.kv_bytes, "items": info.n_items,
        "chunk_tokens": info.chunk_tokens,
        "split": bool(info.split), "launches_per_step": info.launches_per_step,
        "partial_bytes": info.partial_bytes, "ms_per_step": ms_step,
        "gbs": info.kv_bytes / (ms_step * 1e-3) / 1e9,
        "decode_ms_mean": float(kern_ms.mean()), "decode_ms_median": float(np.median(kern_ms)),
        "decode_ms_p99": float(np.percentile(kern_ms, 99)),
        "decode_gbs": info.kv_bytes / (kern_ms.mean() * 1e-3) / 1e9,
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


def density_search(torch, pkv, workloads, periods_ms, max_sessions, steps, runs, say):
    """Cadenced session loop (WPK note: sessions served on a fixed beat, late
    beats counted, density = most sessions with none late).  Steps are
    published on a clock of period T; a step is late if it completes after its
    next tick.  Sessions come and go: each slot hosts a sequence of sessions
    (lifetimes U[40, 120] steps); when one leaves, the next joins the slot at a
    step boundary with a fresh context (drawn so that it fits the slot's
    pages).  For each T the largest session count with no late step over
    `runs` runs is found by bisection."""
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
    rng = np.random.default_rng([workloads.MEASURE_SEED, 9])
    lens = np.zeros((steps, max_sessions), dtype=np.int32)
    joins = 0
    for s in range(max_sessions):
        cap = int(sl.l0[s])                      # the slot's pages hold cap + steps tokens
        t, L0 = 0, cap
        while t < steps:
            life = int(rng.integers(40, 121))
            for u in range(t, min(steps, t + life)):
                lens[u, s] = L0 + (u - t)
            t += life
            if t < steps:
                L0 = int(rng.integers(min(2048, cap), cap + 1))
                joins += 1
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

    # parity of a churned step: a slot after a join reads its new, shorter context
    _, _ = run(min(8, max_sessions), 0.0)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    G = H // sl.num_kv_heads
    t_chk = steps - 1
    for s in range(min(8, max_sessions)):
        L = int(lens[t_chk, s])
        npg = -(-L // 16)
        pg = sl.block_tables[0, s, :npg]
        ks = workloads.bits_u16(sl.slabs("k", 0, pg, 0))[:, None]
        vs = workloads.bits_u16(sl.slabs("v", 0, pg, 0))[:, None]
        qg = workloads.bits_u16(sl.query_unit(t_chk, 0, s))[None, :G]
        ro, rl = pa.range_state(qg, ks, vs, np.arange(npg)[None], 0, 0, 0, L, sl.scale, 16)
        err = np.abs(o[t_chk, 0, s, :G] - ro).max()
        if not err <= 2e-2:
            raise SystemExit(f"density loop parity failed for slot {s}: {err:.3e}")
    say(f"density loop parity passed ({joins} joins in the schedule)")
    res = {"max_sessions_tried": max_sessions, "steps_per_run": steps, "runs": runs,
           "session_lifetime_steps": [40, 120], "joins_per_run": joins, "periods": {}}
    for T in periods_ms:
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


def measured_traffic(root, kv="bf16"):
    """HBM bytes per decode launch of the long context from the committed
    counter summary, if it was taken on the kernel code as it is now (else
    None)."""
    import re
    name = "decode_kernel_long_context" + ("_fp32_cache" if kv == "f32" else "") + "_traffic.md"
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
    wl = workloads.CONFIGS[name]()
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
    """Scheduling ablations (static vs atomic item assignment vs page claims;
    exact-length bucketed launches vs the compact queue) on the one-shot
    workloads, with both cache types for the assignment."""
    res = {"schedule": {}, "bucketed": {}}
    steps = max(args.steps // 2, 10)
    for kv in ("bf16", "f32"):
        for name in ("long", "mixed", "short"):
            row = {}
            for label, sched in (("atomic", pkv.PKV_SCHEDULE_ATOMIC), ("static", pkv.PKV_SCHEDULE_STATIC),
                                 ("pages", pkv.PKV_SCHEDULE_PAGES)):
                r, _ = measure(torch, pkv, workloads, name, steps, args.warmup, args.order, args.wg_per_cu,
                               args.copies, not args.no_gate, say, args.merge, sched, kv=kv)
                row[label] = {"gbs": round(r["gbs"], 1), "decode_gbs": round(r["decode_gbs"], 1),
                              "decode_us": round(r["decode_ms_mean"] * 1e3, 2)}
            key = name if kv == "bf16" else f"{name}_f32"
            res["schedule"][key] = row
            say(f"ablation {key}: atomic {row['atomic']['gbs']} GB/s, static {row['static']['gbs']} GB/s, "
                f"page claims {row['pages']['gbs']} GB/s")
    for name in ("mixed", "short"):
        r, _ = measure(torch, pkv, workloads, name, steps, args.warmup, args.order, args.wg_per_cu,
                       args.copies, False, say, args.merge)
        bk = measure_bucketed(torch, pkv, workloads, name, steps, args.warmup, say)
        res["bucketed"][name] = {
            "compact": {"launches_per_step": r["launches_per_step"], "partial_bytes": r["partial_bytes"],
                        "gbs": round(r["gbs"], 1), "ms_per_step": round(r["ms_per_step"], 4)},
            "bucketed": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in bk.items()}}
        say(f"ablation {name}: compact queue {r['gbs']:.1f} GB/s in {r['launches_per_step']} launch(es); "
            f"bucketed {bk['gbs']:.1f} GB/s in {bk['launches_per_step']} launches ({bk['buckets']} lengths)")
    return res


def cpu_baseline(workloads, wl, seconds, say):
    """The oracle as it stands, on whole (sequence, KV head) units of the same
    workload, repeated pass after pass for about `seconds` of CPU time."""
    from oracle import paged_attention as pa
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threads = 1
    qb = workloads.bits_u16(wl.q("cpu"))
    G = wl.num_q_heads // wl.num_kv_heads
    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    cache = {}
    done_bytes, spent, n = 0, 0.0, 0
    while n == 0 or spent < seconds:
        b, hk = units[n % len(units)]
        L = int(wl.ctx_lens[b])
        npg = -(-L // 16)
        if (b, hk) not in cache:
            pg = wl.block_table[b, :npg]
            cache[(b, hk)] = (workloads.kv_host(wl.pool_slabs("k", pg, hk))[:, None],
                              workloads.kv_host(wl.pool_slabs("v", pg, hk))[:, None])
        ks, vs = cache[(b, hk)]
        t0 = time.perf_counter()
        pa.range_state(qb[b:b + 1, hk * G:(hk + 1) * G], ks, vs, np.arange(npg)[None], 0, 0, 0, L,
                       wl.scale, 16)
        spent += time.perf_counter() - t0
        done_bytes += L * wl.head_dim * wl.kv_elem_bytes * 2
        n += 1
    passes = n / len(units)
    say(f"cpu baseline: {n} units ({passes:.2f} passes), {spent:.1f} s")
    return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} (sequence, KV head) units = {passes:.2f} passes over the {len(units)} units "
                      f"of the '{wl.name}' workload ({done_bytes / 1e6:.1f} MB of K+V), float64 NumPy "
                      f"oracle, inputs generated on the host and excluded from the time"}


def profile_pass(torch, pkv, workloads, args, say):
    """Untimed work for rocprofv3 counter passes: `steps` decode calls of the
    workload (alternating two pool copies), then one copy probe moving
    exactly 1 GiB (read 1 GiB, write 1 GiB), whose counter readings give the
    scale from counter units to bytes."""
    wl = workloads.CONFIGS[args.workload]().with_kv_dtype(args.kv)
    dev = "cuda"
    q = wl.q(dev)
    pools = [(wl.pool("k", dev, False), wl.pool("v", dev, False)) for _ in range(2)]
    bt, lens = wl.block_table_t(dev), wl.ctx_lens_t(dev)
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device=dev)
    cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, wl.batch,
                          wl.max_pages_per_seq, scale=wl.scale,
                          kv_dtype=pkv.PKV_KV_F32 if args.kv == "f32" else pkv.PKV_KV_BF16,
                          schedule={"atomic": pkv.PKV_SCHEDULE_ATOMIC, "static": pkv.PKV_SCHEDULE_STATIC,
                                    "pages": pkv.PKV_SCHEDULE_PAGES}[args.schedule],
                          merge_mode=pkv.PKV_MERGE_SEPARATE if args.merge == "separate" else pkv.PKV_MERGE_FUSED)
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
    pkv.lib()
    if args.profile_pass:
        profile_pass(torch, pkv, workloads, args, say)
        return
    sched = {"atomic": pkv.PKV_SCHEDULE_ATOMIC, "static": pkv.PKV_SCHEDULE_STATIC,
             "pages": pkv.PKV_SCHEDULE_PAGES}[args.schedule]
    main_res, wl = measure(torch, pkv, workloads, args.workload, args.steps, args.warmup,
                           args.order, args.wg_per_cu, args.copies, not args.no_gate, say, args.merge,
                           sched, kv=args.kv)
    say(f"{args.workload}: {main_res['gbs']:.1f} GB/s per step, decode kernel "
        f"{main_res['decode_gbs']:.1f} GB/s ({main_res['decode_ms_mean'] * 1e3:.1f} us)")
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        r, _ = measure(torch, pkv, workloads, name, max(args.steps // 2, 10), args.warmup,
                       args.order, args.wg_per_cu, args.copies, not args.no_gate, say, args.merge, sched)
        others[name] = {k: r[k] for k in ("gbs", "decode_gbs", "ms_per_step", "decode_ms_mean",
                                          "items", "split", "chunk_tokens", "kv_bytes",
                                          "launches_per_step")}
        others[name]["pct_of_hbm_peak"] = 100.0 * r["gbs"] / HBM_PEAK_GBS
        say(f"{name}: {r['gbs']:.1f} GB/s per step, decode {r['decode_gbs']:.1f} GB/s")
    f32 = {}
    if not args.no_f32:
        for name in ("long", "mixed", "short"):
            if name == args.workload and args.kv == "f32":
                continue
            r, _ = measure(torch, pkv, workloads, name, max(args.steps // 2, 10), args.warmup,
                           args.order, args.wg_per_cu, args.copies, not args.no_gate, say, args.merge,
                           sched, kv="f32")
            f32[name] = {k: r[k] for k in ("gbs", "decode_gbs", "ms_per_step", "decode_ms_mean",
                                           "items", "chunk_tokens", "kv_bytes")}
            f32[name]["pct_of_hbm_peak"] = 100.0 * r["gbs"] / HBM_PEAK_GBS
            f32[name]["decode_frac"] = r["decode_gbs"] / HBM_PEAK_GBS
            if name == "long":
                f32[name]["traffic"] = measured_traffic(os.path.dirname(os.path.abspath(__file__)), "f32")
            say(f"{name} (fp32 cache): {r['gbs']:.1f} GB/s per step, decode {r['decode_gbs']:.1f} GB/s "
                f"({r['decode_ms_mean'] * 1e3:.1f} us)")
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
    density = density_search(torch, pkv, workloads, (10, 20), 160, 100, 3, say) if args.density else None
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(workloads, wl, args.cpu_seconds, say)
    achieved = main_res["decode_gbs"]
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
                   "kv_dtype": args.kv}
                  if args.workload == "long" else
                  {"workload": args.workload, "items": main_res["items"], "kv_dtype": args.kv,
                   "kv_bytes_per_step": main_res["kv_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__)), args.kv)
                     if args.workload == "long" else None,
                     "kernel": f"decode_kernel<128,4,{'KvF32' if args.kv == 'f32' else 'KvBf16'}>",
                     "decode_us_mean": round(main_res["decode_ms_mean"] * 1e3, 3)},
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

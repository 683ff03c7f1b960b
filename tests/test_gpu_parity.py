"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Tolerance (stated for bf16 inputs with fp32 accumulation): every output
element within max-abs 2e-2 and mean-abs 2e-3 of the oracle, compared in
float64 after widening the kernel's bf16 output; the same bounds apply to the
fp32 LSE.  Queue bytes and gathered K/V bits must match exactly.

Small cases compare every output; full-size workloads compare sampled
(sequence, KV head) units, each recomputed by the oracle from pages
regenerated on the CPU by the seeded generator.

The same cases run with an fp32 KV cache (kv_dtype F32: the fp32 attention
cache of the Wave Persistent Kernel note).  There the gathered K/V bits must
again match exactly, and the fp32 LSE must sit within LSE_F32 of the oracle:
with exact inputs the kernel's LSE error is fp32 rounding of the dot
products, the exponentials and the sums, of order 1e-6 here, while reading
the cache at bf16 precision would move scores by about
2^-9 * sqrt(D) * scale ~ 1e-3, so the bound tells the two apart.
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention as pa
from oracle import work_queue as wq
from paged_kv_attention_persistent_amd import pkv, workloads

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_F32 = 1e-4
KVS = ["bf16", "f32"]


def say(*a):
    print("[gpu-parity]", *a, flush=True)


def cfg_for(wl, **kw):
    kw.setdefault("kv_dtype", pkv.PKV_KV_F32 if wl.kv_dtype == "f32" else pkv.PKV_KV_BF16)
    return pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages,
                           max(wl.batch, 1), wl.max_pages_per_seq, scale=wl.scale, **kw)


class Run:
    """Inputs of one workload on the GPU plus one decode through the C ABI."""

    def __init__(self, wl, poison=True, **cfgkw):
        self.wl = wl
        dev = "cuda"
        self.q = wl.q(dev)
        self.k = wl.pool("k", dev, poison)
        self.v = wl.pool("v", dev, poison)
        self.bt = wl.block_table_t(dev)
        self.lens = wl.ctx_lens_t(dev)
        self.out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"),
                              dtype=torch.bfloat16, device=dev)
        self.lse = torch.full((wl.batch, wl.num_q_heads), float("nan"), dtype=torch.float32,
                              device=dev)
        cfgkw.setdefault("num_cus", torch.cuda.get_device_properties(0).multi_processor_count)
        self.cfg = cfg_for(wl, **cfgkw)
        self.dec = pkv.PagedDecoder(self.cfg)
        self.info = None

    def tensors(self):
        return pkv.make_tensors(self.q, self.k, self.v, self.bt, self.lens, self.out, self.lse)

    def decode(self, device_queue=False):
        if device_queue:
            self.dec.build_queue_device(self.lens)
        else:
            self.info = self.dec.build_queue(self.wl.ctx_lens)
        pkv.pkv_decode(self.dec.handle, self.tensors(), self.dec.stream)
        torch.cuda.synchronize()
        st = self.dec.query()
        assert st["error_code"] == 0
        return self.out.float().cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)

    def queue_bytes(self):
        torch.cuda.synchronize()
        lay = self.dec.layout
        ws = self.dec.workspace
        n = int(ws[lay.queue_off:lay.queue_off + 4].cpu().view(torch.int32)[0])
        items = ws[lay.items_off:lay.items_off + 16 * n].cpu().numpy().tobytes()
        B = self.wl.batch
        nch = ws[lay.n_chunks_off:lay.n_chunks_off + 4 * B].cpu().view(torch.int32).numpy()
        po = ws[lay.part_off_off:lay.part_off_off + 4 * (B + 1)].cpu().view(torch.int32).numpy()
        hdr = ws[lay.queue_off:lay.queue_off + 20].cpu().view(torch.int32).numpy()
        nm = int(hdr[1])
        mr = ws[lay.merge_rows_off:lay.merge_rows_off + 4 * nm].cpu().view(torch.int32).numpy()
        rl = ws[lay.row_len_off:lay.row_len_off + 4 * B].cpu().view(torch.int32).numpy()
        return {"items": items, "n_chunks": nch, "part_off": po, "merge_rows": mr, "hdr": hdr,
                "row_len": rl}

    def close(self):
        self.dec.close()


def oracle_full(wl, poison=True):
    q = workloads.bits_u16(wl.q("cpu"))
    k = workloads.kv_host(wl.pool("k", "cpu", poison))
    v = workloads.kv_host(wl.pool("v", "cpu", poison))
    return pa.decode_attention(q, k, v, wl.block_table, wl.ctx_lens, wl.scale, wl.page_size)


def oracle_unit(wl, q_bits, b, hk):
    """Oracle for one (sequence, KV head) from regenerated slabs."""
    L = int(wl.ctx_lens[b])
    G = wl.num_q_heads // wl.num_kv_heads
    if L == 0:
        return np.zeros((G, wl.head_dim)), np.full(G, -np.inf)
    npg = -(-L // wl.page_size)
    pages = wl.block_table[b, :npg]
    ks = workloads.kv_host(wl.pool_slabs("k", pages, hk))[:, None]      # [n][1][P][D]
    vs = workloads.kv_host(wl.pool_slabs("v", pages, hk))[:, None]
    qg = q_bits[b:b + 1, hk * G:(hk + 1) * G]                           # [1][G][D]
    bt = np.arange(npg)[None]
    return pa.range_state(qg, ks, vs, bt, 0, 0, 0, L, wl.scale, wl.page_size)


def check(o, l, ro, rl, where, lse_tol=MAX_ABS):
    err = np.abs(o - ro)
    assert np.all(np.isfinite(o)), f"{where}: non-finite output"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin), f"{where}: LSE finiteness differs"
    lerr = np.abs(l[fin] - rl[fin]) if fin.any() else np.zeros(1)
    say(f"{where}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
        f"rel_l2={np.linalg.norm(o - ro) / max(np.linalg.norm(ro), 1e-30):.3e} lse_max={lerr.max():.3e}")
    assert err.max() <= MAX_ABS, where
    assert err.mean() <= MEAN_ABS, where
    assert lerr.max() <= lse_tol, where


# ----------------------------------------------------------- small cases ----

SMALL = [
    # name, lens, Hq, Hkv, D, policy, chunk
    ("ragged_d128_nosplit", [1, 15, 16, 17, 100, 333, 0, 1024], 8, 2, 128, pkv.PKV_POLICY_NO_SPLIT, 0),
    ("ragged_d128_split64", [1, 15, 16, 17, 100, 333, 0, 1024], 8, 2, 128, pkv.PKV_POLICY_SPLIT, 64),
    ("ragged_d64_g8_split", [700, 5, 0, 2049], 16, 2, 64, pkv.PKV_POLICY_SPLIT, 256),
    ("g1_d128", [64, 257, 31], 4, 4, 128, pkv.PKV_POLICY_AUTO, 0),
    ("g2_d64", [1000, 3], 4, 2, 64, pkv.PKV_POLICY_SPLIT, 128),
    ("long_tail_many_windows", [9000, 8191], 4, 1, 128, pkv.PKV_POLICY_NO_SPLIT, 0),
    ("all_empty", [0, 0, 0], 8, 2, 128, pkv.PKV_POLICY_AUTO, 0),
]


def lse_tol(wl):
    return LSE_F32 if wl.kv_dtype == "f32" else MAX_ABS


SCHEDULES = {"atomic": pkv.PKV_SCHEDULE_ATOMIC, "pages": pkv.PKV_SCHEDULE_PAGES}


@pytest.mark.parametrize("sched", list(SCHEDULES))
@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("merge", [pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE],
                         ids=["fused_merge", "separate_merge"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_full_compare(case, merge, kv, sched):
    name, lens, hq, hkv, d, policy, chunk = case
    say("case", name, "merge", merge, "kv", kv, "schedule", sched)
    wl = workloads.custom(name, lens, hq, hkv, d, spare_pages=5, kv_dtype=kv)
    run = Run(wl, policy=policy, kv_chunk_tokens=chunk, merge_mode=merge, schedule=SCHEDULES[sched])
    ro, rl = oracle_full(wl)
    for call in range(2):                 # second call: counters and head re-armed
        o, l = run.decode()
        check(o, l, ro, rl, f"{name} {kv} call {call}", lse_tol(wl))
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))
        run.out.fill_(float("nan"))
        run.lse.fill_(float("nan"))
    if run.info.split:
        lay = run.dec.layout
        arrive = run.dec.workspace[lay.arrive_off:lay.arrive_off + 4 * len(lens) * hkv]
        assert int(arrive.cpu().view(torch.int32).abs().sum()) == 0
    run.close()


def test_tiny_workload_and_repeat_calls():
    wl = workloads.tiny()
    run = Run(wl)
    ro, rl = oracle_full(wl)
    for i in range(3):                                   # head counter re-arms each launch
        o, l = run.decode()
        check(o, l, ro, rl, f"tiny call {i}")
    st = run.dec.query()
    assert st["decode_calls"] == 3 and st["queue_head"] == 0 and st["items_done"] == 3
    run.close()


# ------------------------------------------------------ full-size cases ----

FULL = {"long": [(0, 0), (0, 5)], "mixed": [(b, (3 * b) % 8) for b in range(8)],
        "short": [(0, 0), (17, 3), (63, 7)]}


@pytest.mark.parametrize("sched", list(SCHEDULES))
@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("merge", [pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE],
                         ids=["fused_merge", "separate_merge"])
@pytest.mark.parametrize("name", ["long", "mixed", "short"])
def test_full_size_sampled_units(name, merge, kv, sched):
    say("full", name, "kv", kv, "schedule", sched)
    wl = workloads.CONFIGS[name]().with_kv_dtype(kv)
    run = Run(wl, poison=True, merge_mode=merge, schedule=SCHEDULES[sched])
    o, l = run.decode()
    info = run.info
    ref = wq.build_queue(wl.ctx_lens, wl.num_kv_heads, run.dec.query()["num_cus"], 0)
    assert info.n_items == len(ref["items"]) and bool(info.split) == ref["split"]
    qb = workloads.bits_u16(run.q)
    G = wl.num_q_heads // wl.num_kv_heads
    for b, hk in FULL[name]:
        ro, rl = oracle_unit(wl, qb, b, hk)
        check(o[b, hk * G:(hk + 1) * G], l[b, hk * G:(hk + 1) * G], ro, rl, f"{name} {kv} b={b} hk={hk}",
              lse_tol(wl))
    # every output finite: no stray read of a poisoned slot anywhere
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    run.close()


def test_split_equals_unsplit_on_gpu_partials():
    """Merge identity on the kernel's own partials: forced split vs no split,
    and each partial state vs the oracle's state for its range."""
    wl = workloads.custom("merge_id", [20000, 5000, 3], 8, 2, 128, spare_pages=2)
    a = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=1024)
    oa, la = a.decode()
    b = Run(wl, policy=pkv.PKV_POLICY_NO_SPLIT)
    ob, lb = b.decode()
    check(oa, la, ob, lb, "split vs unsplit")
    # partial states in the workspace vs oracle range_state
    lay = a.dec.layout
    ws = a.dec.workspace
    items, n_chunks, part_off, _, info = pkv.pkv_plan_queue(a.cfg, wl.ctx_lens)
    G = 4
    po = ws[lay.partial_o_off:lay.partial_o_off + 4 * lay.max_items * G * 128].cpu().view(torch.float32)
    pl = ws[lay.partial_lse_off:lay.partial_lse_off + 4 * lay.max_items * G].cpu().view(torch.float32)
    po = po.numpy().reshape(lay.max_items, G, 128)
    pl = pl.numpy().reshape(lay.max_items, G)
    q = workloads.bits_u16(wl.q("cpu"))
    k = workloads.kv_host(wl.pool("k", "cpu"))
    v = workloads.kv_host(wl.pool("v", "cpu"))
    checked = 0
    for it in items[::7]:
        if n_chunks[int(it["seq"])] <= 1:
            continue
        s = wq.partial_slot(it, part_off, 2)
        ro, rl = pa.range_state(q, k, v, wl.block_table, int(it["seq"]), int(it["kv_head"]),
                                int(it["tok_begin"]), int(it["tok_end"]), wl.scale, 16)
        assert np.abs(po[s] - ro).max() <= MAX_ABS and np.abs(pl[s] - rl).max() <= MAX_ABS
        checked += 1
    assert checked >= 3
    a.close()
    b.close()


# --------------------------------------------------- queue and gather ----

@pytest.mark.parametrize("name", ["tiny", "long", "mixed", "short"])
def test_queue_bytes_on_device_match_oracle(name):
    wl = workloads.CONFIGS[name]()
    run = Run(wl, poison=False)
    cus = run.dec.query()["num_cus"]
    ref = wq.build_queue(wl.ctx_lens, wl.num_kv_heads, cus, 0)      # chunk mode "fit"
    for device_queue in (False, True):
        if device_queue:
            run.dec.build_queue_device(run.lens)
        else:
            run.dec.build_queue(wl.ctx_lens)
        got = run.queue_bytes()
        assert got["items"] == ref["items"].tobytes(), f"{name} device={device_queue}"
        assert np.array_equal(got["n_chunks"], ref["n_chunks"])
        assert np.array_equal(got["part_off"], ref["part_off"])
        assert np.array_equal(got["merge_rows"], ref["merge_rows"])
        assert np.array_equal(got["row_len"], ref["row_len"])
        assert list(got["hdr"]) == [len(ref["items"]), len(ref["merge_rows"]), int(ref["split"]),
                                    ref["chunk_tokens"], wl.batch]
        # the C-ABI read of the same queue: the workspace bytes, header through items
        lay = run.dec.layout
        raw = pkv.pkv_queue_read(run.dec.handle, 1 << 26)
        assert len(raw) == lay.items_off - lay.queue_off + 16 * len(ref["items"])
        assert raw == run.dec.workspace[lay.queue_off:lay.queue_off + len(raw)].cpu().numpy().tobytes()
        assert raw[lay.items_off - lay.queue_off:] == ref["items"].tobytes()
        assert len(pkv.pkv_queue_read(run.dec.handle, 100)) == 100          # capped by capacity
    run.close()


def test_device_queue_random_lengths_match_oracle():
    # the device builder's bisection for chunk mode "fit", and fixed chunks,
    # against the oracle on random batches (queue only; no K/V is read)
    rng = np.random.default_rng(11)
    for trial in range(40):
        B = int(rng.integers(1, 300))
        hkv = int(rng.choice([1, 2, 8]))
        cus = int(rng.choice([8, 64, 256]))
        chunk = int(rng.choice([0, 0, 512, 4096]))
        policy = int(rng.integers(0, 3))
        maxp = int(rng.integers(1, 3000))
        lens = rng.integers(0, maxp * 16 + 1, size=B)
        lens[rng.random(B) < 0.2] = 0
        cfg = pkv.make_config(4 * hkv, hkv, 128, 64, B, maxp, policy=policy, kv_chunk_tokens=chunk,
                              num_cus=cus)
        dec = pkv.PagedDecoder(cfg)
        try:
            ref = wq.build_queue(lens.tolist(), hkv, cus, chunk, policy)
            if len(ref["items"]) > dec.layout.max_items:
                continue
            dev_lens = torch.as_tensor(lens.astype(np.int32)).cuda()
            dec.build_queue_device(dev_lens)
            torch.cuda.synchronize()
            lay, ws = dec.layout, dec.workspace
            hdr = ws[lay.queue_off:lay.queue_off + 20].cpu().view(torch.int32).numpy()
            n = int(hdr[0])
            where = f"trial {trial}: B={B} hkv={hkv} cus={cus} chunk={chunk} policy={policy}"
            assert list(hdr) == [len(ref["items"]), len(ref["merge_rows"]), int(ref["split"]),
                                 ref["chunk_tokens"], B], where
            items = ws[lay.items_off:lay.items_off + 16 * n].cpu().numpy().tobytes()
            assert items == ref["items"].tobytes(), where
            nch = ws[lay.n_chunks_off:lay.n_chunks_off + 4 * B].cpu().view(torch.int32).numpy()
            assert np.array_equal(nch, ref["n_chunks"]), where
            rl = ws[lay.row_len_off:lay.row_len_off + 4 * B].cpu().view(torch.int32).numpy()
            assert np.array_equal(rl, ref["row_len"]), where
        finally:
            dec.close()


def test_device_queue_decode_matches():
    wl = workloads.custom("devq", [5000, 0, 77, 12000], 8, 2, 128, spare_pages=3)
    run = Run(wl, policy=pkv.PKV_POLICY_AUTO)
    o, l = run.decode(device_queue=True)
    ro, rl = oracle_full(wl)
    check(o, l, ro, rl, "device-built queue")
    run.close()


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("name", ["tiny", "mixed"])
def test_gather_bits_match_oracle(name, kv):
    wl = workloads.CONFIGS[name]() if name != "mixed" else workloads.custom(
        "gather_mixed", [100, 4097, 33, 5000], 8, 2, 128, spare_pages=4)
    wl = wl.with_kv_dtype(kv)
    run = Run(wl, policy=pkv.PKV_POLICY_SPLIT if name == "mixed" else pkv.PKV_POLICY_AUTO,
              kv_chunk_tokens=1024 if name == "mixed" else 0)
    run.dec.build_queue(wl.ctx_lens)
    items, *_ = pkv.pkv_plan_queue(run.cfg, wl.ctx_lens)
    kp = workloads.kv_host(wl.pool("k", "cpu"))
    vp = workloads.kv_host(wl.pool("v", "cpu"))
    for i in range(len(items)):
        it = items[i]
        n = int(it["tok_end"] - it["tok_begin"])
        ko = torch.zeros(n, wl.head_dim, dtype=wl.kv_torch_dtype, device="cuda")
        vo = torch.zeros_like(ko)
        pkv.pkv_debug_gather(run.dec.handle, run.tensors(), i, ko, vo, run.dec.stream)
        torch.cuda.synchronize()
        rk = pa.gather_tokens(kp, wl.block_table, int(it["seq"]), int(it["kv_head"]),
                              int(it["tok_begin"]), int(it["tok_end"]), 16)
        rv = pa.gather_tokens(vp, wl.block_table, int(it["seq"]), int(it["kv_head"]),
                              int(it["tok_begin"]), int(it["tok_end"]), 16)
        gk, gv = workloads.kv_host(ko), workloads.kv_host(vo)
        assert gk.dtype == rk.dtype and gk.tobytes() == rk.tobytes(), f"K item {i}"
        assert gv.dtype == rv.dtype and gv.tobytes() == rv.tobytes(), f"V item {i}"
    run.close()


# --------------------------------------------------------- error paths ----

def test_bad_block_table_entry_is_reported_not_read():
    wl = workloads.custom("badpage", [40, 50], 4, 1, 128, spare_pages=1)
    run = Run(wl)
    bt = run.bt.clone()
    bt[1, 2] = wl.num_pages + 1000                    # outside the pool
    run.dec.build_queue(wl.ctx_lens)
    t = pkv.make_tensors(run.q, run.k, run.v, bt, run.lens, run.out, run.lse)
    pkv.pkv_decode(run.dec.handle, t, run.dec.stream)
    torch.cuda.synchronize()
    st = run.dec.query(raise_on_fault=False)
    assert st["status"] == pkv.PKV_ERR_DEVICE_FAULT
    assert st["error_code"] == pkv.PKV_DEVERR_PAGE_OOB and st["error_detail"] == wl.num_pages + 1000
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode(run.dec.handle, t, run.dec.stream)
    assert e.value.status == pkv.PKV_ERR_DEVICE_FAULT
    pkv.pkv_clear_error(run.dec.handle)
    o, l = run.decode()                                 # good table again
    ro, rl = oracle_full(wl)
    check(o, l, ro, rl, "after clear")
    run.close()


def test_argument_errors_enqueue_nothing():
    wl = workloads.tiny()
    run = Run(wl)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode(run.dec.handle, run.tensors(), run.dec.stream)   # before build
    assert e.value.status == pkv.PKV_ERR_STATE
    run.dec.build_queue(wl.ctx_lens)
    t = run.tensors()
    t.batch = 2
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode(run.dec.handle, t, run.dec.stream)
    t = run.tensors()
    t.q = t.q + 2                                      # misaligned
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode(run.dec.handle, t, run.dec.stream)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        run.dec.build_queue([10 ** 6])
    assert e.value.status == pkv.PKV_ERR_CAPACITY
    st = run.dec.query()
    assert st["decode_calls"] == 0
    run.close()


def test_generator_identical_on_cpu_and_gpu():
    idx = torch.arange(0, 1 << 20, dtype=torch.int64) * 4099 + (1 << 33)
    a = workloads.normal_bf16_bits(7, "t", idx)
    b = workloads.normal_bf16_bits(7, "t", idx.cuda()).cpu()
    assert torch.equal(a, b)


def test_fused_merge_bitwise_equals_separate_merge_over_repeats():
    """Both merge modes run the same merge arithmetic; only how partial
    states travel differs (coherent atomics inside one launch vs a kernel
    boundary).  Their outputs must agree bit for bit on every call."""
    wl = workloads.custom("fused_vs_sep", [70000, 4096 * 3 + 5, 9000, 1], 32, 8, 128, spare_pages=3)
    a = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=2048, merge_mode=pkv.PKV_MERGE_FUSED)
    b = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=2048, merge_mode=pkv.PKV_MERGE_SEPARATE)
    ob, lb = b.decode()
    ro, rl = oracle_full(wl)
    check(ob, lb, ro, rl, "separate merge")
    a.dec.build_queue(wl.ctx_lens)
    for i in range(25):
        a.out.fill_(float("nan"))
        pkv.pkv_decode(a.dec.handle, a.tensors(), a.dec.stream)
        torch.cuda.synchronize()
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16)), f"call {i}"
        assert torch.equal(a.lse.view(torch.int32), b.lse.view(torch.int32)), f"call {i}"
    assert a.dec.query()["error_code"] == 0
    a.close()
    b.close()


@pytest.mark.parametrize("name", ["long", "mixed", "short"])
def test_static_schedule_equals_atomic_bitwise(name):
    # the schedule only moves items between workgroups; each item is computed
    # the same way, so every output bit must agree
    wl = workloads.CONFIGS[name]()
    outs = []
    for schedule in (pkv.PKV_SCHEDULE_ATOMIC, pkv.PKV_SCHEDULE_STATIC):
        run = Run(wl, poison=True, schedule=schedule)
        o, l = run.decode()
        outs.append((o, l))
        assert run.dec.query()["items_done"] >= run.info.n_items
        run.close()
    say(f"{name}: static vs atomic schedule, {outs[0][0].size} outputs compared")
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_f32_cache_is_read_at_full_precision():
    """The fp32 path's LSE follows the fp32 cache, not its bf16 rounding: the
    oracle on the rounded cache lies well outside LSE_F32 somewhere, while
    the kernel stays inside it everywhere."""
    wl = workloads.custom("f32_precision", [3000, 17, 900, 4096], 16, 4, 128, spare_pages=2,
                          kv_dtype="f32")
    run = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=1024)
    o, l = run.decode()
    ro, rl = oracle_full(wl)
    check(o, l, ro, rl, "f32 cache", LSE_F32)
    wb = wl.with_kv_dtype("bf16")               # the bf16 rounding of the same values
    bo, bl = oracle_full(wb)
    gap = np.abs(bl - rl).max()
    say(f"oracle LSE gap between the fp32 cache and its bf16 rounding: {gap:.3e}")
    assert gap > 5 * LSE_F32
    run.close()


@pytest.mark.parametrize("merge", [pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE],
                         ids=["fused_merge", "separate_merge"])
def test_page_claims_with_idle_items_and_repeats(merge):
    """Page-claim schedule where most items of a row find its pages already
    claimed (16-token ranges over short rows: far more waves than page
    groups), so their partial states are empty, and repeated calls, each of
    which must start every cursor at zero again."""
    wl = workloads.custom("claims_idle", [200, 17, 0, 96, 1000], 8, 2, 128, spare_pages=3)
    run = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=16, merge_mode=merge,
              schedule=pkv.PKV_SCHEDULE_PAGES)
    ro, rl = oracle_full(wl)
    for call in range(12):
        run.out.fill_(float("nan"))
        run.lse.fill_(float("nan"))
        o, l = run.decode()
        check(o, l, ro, rl, f"idle items call {call}")
    lay = run.dec.layout
    cur = run.dec.workspace[lay.cursor_off:lay.cursor_off + 4 * 32 * len(wl.ctx_lens) * 2]
    assert int(cur.cpu().view(torch.int32).abs().sum()) == 0       # every cursor re-armed
    run.close()


@pytest.mark.parametrize("kv", KVS)
def test_page_claims_split_equals_unsplit(kv):
    # the claimed page sets differ from call to call; the merged result must
    # not: each call against the unsplit decode of the same rows
    wl = workloads.custom("claims_vs_unsplit", [20000, 5000, 3, 70000], 8, 2, 128, spare_pages=2,
                          kv_dtype=kv)
    a = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=1024, schedule=pkv.PKV_SCHEDULE_PAGES)
    b = Run(wl, policy=pkv.PKV_POLICY_NO_SPLIT)
    ob, lb = b.decode()
    ro, rl = oracle_full(wl)
    check(ob, lb, ro, rl, f"unsplit {kv}", lse_tol(wl))
    for call in range(5):
        oa, la = a.decode()
        check(oa, la, ro, rl, f"page claims {kv} call {call}", lse_tol(wl))
        check(oa, la, ob, lb, f"page claims vs unsplit {kv} call {call}", lse_tol(wl))
    a.close()
    b.close()


@pytest.mark.parametrize("sched", list(SCHEDULES))
@pytest.mark.parametrize("kv", KVS)
def test_structured_cases_count_every_token(kv, sched):
    """Closed forms on the GPU, strong enough to see one token too many or too
    few.  With q = 0 every score is 0, so LSE = ln L_b to fp32 rounding (a few
    1e-7 relative) while a dropped or repeated token moves it by about 1 / L_b
    (2e-4 at 5000 tokens); with V[t][0] = (t mod 256) / 256 and V[t][1] = 0.375
    (both bf16-exact), O[.][0] is the mean of the first column to bf16 rounding
    and O[.][1] is 0.375 exactly.  Split and unsplit rows, partial pages, a
    one-token row and an empty row."""
    lens = [5000, 17, 1, 3000, 0, 4097, 256]
    wl = workloads.custom("structured", lens, 8, 2, 128, spare_pages=3, kv_dtype=kv)
    v = wl.pool("v", "cpu", poison=True)
    for b, L in enumerate(lens):
        t = np.arange(L)
        pg = torch.as_tensor(wl.block_table[b, t // 16].astype(np.int64))
        row = torch.as_tensor(t % 16)
        v[pg, :, row, 0] = torch.as_tensor((t % 256) / 256.0, dtype=torch.float32).to(v.dtype)[:, None]
        v[pg, :, row, 1] = 0.375
    for policy, chunk in ((pkv.PKV_POLICY_SPLIT, 1024), (pkv.PKV_POLICY_NO_SPLIT, 0)):
        run = Run(wl, policy=policy, kv_chunk_tokens=chunk, schedule=SCHEDULES[sched])
        run.q.zero_()
        run.v = v.to("cuda")
        o, l = run.decode()
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))
                continue
            where = f"{kv} {sched} policy {policy} row {b} (L = {L})"
            assert np.abs(l[b] - np.log(L)).max() <= 5e-6, where
            exact = np.mean((np.arange(L) % 256) / 256.0)
            assert np.abs(o[b, :, 0] - exact).max() <= 2.0 ** -8 * exact + 1e-6, where
            assert np.all(o[b, :, 1] == 0.375), where
        run.close()

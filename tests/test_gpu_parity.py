"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Tolerance (stated for bf16 inputs with fp32 accumulation): every output
element within max-abs 2e-2 and mean-abs 2e-3 of the oracle, compared in
float64 after widening the kernel's bf16 output; the same bounds apply to the
fp32 LSE.  Queue bytes and gathered K/V bits must match exactly.

Every case compares every output: small cases, the full-size workloads
(each (sequence, KV head) of the long context, the mixed batch and the
many-short batch, with the oracle run once per workload and cache type on
pools copied back from the seeded generator), and structured cases whose
answer is known in closed form (q = 0 token counting, scores that force the
online-softmax rescale).

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


SCHEDULES = {"atomic": pkv.PKV_SCHEDULE_ATOMIC, "pages": pkv.PKV_SCHEDULE_PAGES, "steal": pkv.PKV_SCHEDULE_STEAL}


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
    for i in range(3):                                   # each launch finds its pop counter at zero
        o, l = run.decode()
        check(o, l, ro, rl, f"tiny call {i}")
    st = run.dec.query()
    assert st["decode_calls"] == 3 and st["queue_head"] == 0 and st["items_done"] == 3
    run.close()


@pytest.mark.parametrize("rows,sched,uniform", [(40, "atomic", False), (4, "atomic", False), (40, "static", False),
                                               (64, "atomic", True), (40, "atomic", True)])
def test_claim_counters_alternate_between_launches(rows, sched, uniform):
    """One-shot launches pop from two counters in turn, each launch zeroing
    the other for the next one.  Every item is followed by one claim when the
    queue has more items than workgroups (so a launch makes exactly n_items
    claims, the last grid of them empty), none when the static first round
    covers the queue, under the static schedule, or for items of one length
    in whole rounds (64 rows x 8 KV heads = 512 items: round-robin); 40 equal
    rows (320 items, not whole rounds) still claim.  Results are unchanged."""
    if uniform:
        lens = [2000] * rows
    else:
        lens = [int(x) for x in np.random.default_rng(rows).integers(1, 3000, size=rows)]
    wl = workloads.custom(f"claims{rows}{'u' if uniform else ''}", lens, 32, 8, 128)
    run = Run(wl, schedule=pkv.PKV_SCHEDULE_STATIC if sched == "static" else pkv.PKV_SCHEDULE_ATOMIC)
    ro, rl = oracle_full(wl)
    lay = run.dec.layout
    n_items, grid = None, None
    for call in range(4):
        o, l = run.decode()
        check(o, l, ro, rl, f"claims {rows} {sched} call {call}")
        st = run.dec.query()
        n_items, grid = st["n_items"], st["grid"]
        heads = run.dec.workspace[lay.ctrl_off:lay.ctrl_off + 8].cpu().view(torch.int32).numpy()
        whole_rounds = uniform and n_items % grid == 0
        claims = n_items if (sched == "atomic" and n_items > grid and not whole_rounds) else 0
        used = call % 2                                  # launch k pops from counter k mod 2
        assert heads[used] == claims and heads[1 - used] == 0, (call, heads.tolist(), n_items, grid)
        assert st["queue_head"] == 0 and st["decode_calls"] == call + 1
        assert st["items_done"] == n_items * (call + 1)
    say(f"claims rows {rows} {sched}: items {n_items}, grid {grid}")
    assert (n_items > grid) == (rows != 4), (n_items, grid)      # both regimes are covered
    if uniform and rows == 64:
        assert n_items % grid == 0, (n_items, grid)
    run.close()



@pytest.mark.parametrize("sched", list(SCHEDULES))
@pytest.mark.parametrize("device_queue", [False, True])
def test_wide_block_table_and_batch_below_capacity(sched, device_queue):
    """A block table whose rows are wider than max_pages_per_seq
    (block_table_stride) with out-of-pool ids in every padding column, and a
    batch of 5 on a configuration sized for 8: every output against the
    oracle on two calls in a row, no page fault reported (the padding is
    never read), under each schedule and both queue builders."""
    lens = [37, 1000, 0, 20000, 300]
    wl = workloads.custom("wide_bt", lens, 8, 2, 128, spare_pages=3)
    dev = "cuda"
    maxp = wl.max_pages_per_seq
    stride = maxp + 13
    bt = torch.full((wl.batch, stride), 1 << 30, dtype=torch.int32)
    bt[:, maxp:] = torch.tensor([-5, wl.num_pages, 1 << 30] * 5, dtype=torch.int32)[:stride - maxp]
    bt[:, :maxp] = torch.as_tensor(wl.block_table)
    bt = bt.to(dev)
    cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, 8, maxp, scale=wl.scale,
                          kv_chunk_tokens=2048, schedule=SCHEDULES[sched],
                          num_cus=torch.cuda.get_device_properties(0).multi_processor_count)
    dec = pkv.PagedDecoder(cfg)
    q, k, v = wl.q(dev), wl.pool("k", dev, True), wl.pool("v", dev, True)
    lens_t = wl.ctx_lens_t(dev)
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device=dev)
    t = pkv.make_tensors(q, k, v, bt, lens_t, out, lse)
    assert t.block_table_stride == stride
    ro, rl = oracle_full(wl)
    try:
        for call in range(2):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            if device_queue:
                dec.build_queue_device(lens_t)
            else:
                dec.build_queue(wl.ctx_lens)
            pkv.pkv_decode(dec.handle, t, dec.stream)
            torch.cuda.synchronize()
            assert dec.query()["error_code"] == 0
            check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                  f"wide block table {sched} device_queue={device_queue} call {call}")
    finally:
        dec.close()


TWO_LEVEL_LENS = [70 * 1024 - 100, 3000, 0, 40 * 1024 - 1024 + 17]     # 70, 3, 0 and 40 ranges of 1024


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("sched", list(SCHEDULES))
def test_two_level_merge_against_oracle_and_separate_merge(sched, kv):
    """Rows of more than 32 ranges merge in two levels in one-shot launches
    (groups of 32 ranges folded by their last workgroups, then the group
    states): every output against the oracle on three calls in a row (the
    group and row counters re-arm), a 3-range row and an empty row beside
    them, and the separate merge kernel, which runs the same two levels,
    bit for bit equal to the fused one."""
    wl = workloads.custom("two_level", TWO_LEVEL_LENS, 8, 2, 128, spare_pages=5, kv_dtype=kv)
    ro, rl = oracle_full(wl)
    res = {}
    for merge in ("fused", "separate"):
        run = Run(wl, kv_chunk_tokens=1024, schedule=SCHEDULES[sched],
                  merge_mode=pkv.PKV_MERGE_FUSED if merge == "fused" else pkv.PKV_MERGE_SEPARATE)
        run.dec.build_queue(wl.ctx_lens)
        nch = run.queue_bytes()["n_chunks"].tolist()
        assert nch == [70, 3, 0, 40], nch
        for call in range(3):
            o, l = run.decode()
            check(o, l, ro, rl, f"two-level {sched} {kv} {merge} call {call}",
                  lse_tol=LSE_F32 if kv == "f32" else MAX_ABS)
        res[merge] = (run.out.clone(), run.lse.clone())
        run.close()
    if sched == "atomic":          # the page-claim and steal schedules split pages at run time
        assert torch.equal(res["fused"][0].view(torch.int16), res["separate"][0].view(torch.int16))
        assert torch.equal(res["fused"][1].view(torch.int32), res["separate"][1].view(torch.int32))

# ------------------------------------------------------ full-size cases ----

_ORACLE_CACHE = {}


def host_inputs(run):
    """The run's query and pools as host arrays (bf16 bits / fp32 values),
    copied back from the device: they are the seeded generator's output
    (its CPU and GPU bits are identical, tested below), not the HIP path's."""
    return (workloads.bits_u16(run.q), workloads.kv_host(run.k.cpu()),
            workloads.kv_host(run.v.cpu()))


def oracle_every_unit(wl, run):
    """The oracle over every (sequence, KV head) of a full-size workload,
    computed once per (workload, cache type) and shared by the tests below."""
    key = (wl.name, wl.kv_dtype)
    if key not in _ORACLE_CACHE:
        q, k, v = host_inputs(run)
        say(f"oracle over every unit of {wl.name} ({wl.kv_dtype}): {wl.batch * wl.num_kv_heads} units")
        _ORACLE_CACHE.clear()                 # one workload's pools at a time in host memory
        _ORACLE_CACHE[key] = (pa.decode_attention(q, k, v, wl.block_table, wl.ctx_lens, wl.scale,
                                                  wl.page_size), (q, k, v))
    return _ORACLE_CACHE[key]


COMBOS = [(merge, sched) for merge in (pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE)
          for sched in SCHEDULES]


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("name", ["long", "mixed", "short"])
def test_full_size_every_unit(name, kv):
    """Every output of the full-size workloads against the oracle, for both
    merges and both schedules (the oracle is computed once per workload)."""
    wl = workloads.CONFIGS[name]().with_kv_dtype(kv)
    run = Run(wl, poison=True)
    (ro, rl), _ = oracle_every_unit(wl, run)
    cus = run.dec.query()["num_cus"]
    ref = wq.build_queue(wl.ctx_lens, wl.num_kv_heads, cus, 0)
    run.close()
    for merge, sched in COMBOS:
        run = Run(wl, poison=True, merge_mode=merge, schedule=SCHEDULES[sched])
        o, l = run.decode()
        info = run.info
        assert info.n_items == len(ref["items"]) and bool(info.split) == ref["split"]
        check(o, l, ro, rl, f"{name} {kv} merge {merge} {sched}: all {wl.batch * wl.num_kv_heads} units",
              lse_tol(wl))
        run.close()


@pytest.mark.parametrize("kv", KVS)
def test_full_size_long_context_counts_every_token(kv):
    """The long context at full size (131072 tokens, 32 ranges merged across
    256 workgroups) with q = 0 on all 32 heads: every score is 0, so
    LSE = ln 131072 to fp32 rounding, where one lost or repeated token moves
    it by 7.6e-6 and one page by 1.2e-4; O is the exact mean of each V column
    (bf16 rounding of an fp32 sum of unit-weight rows), V column 0 is set to
    (t mod 256) / 256 and column 1 to 0.375, so O[.][1] must be 0.375 bit for
    bit.  Both merges and both schedules."""
    wl = workloads.CONFIGS["long"]().with_kv_dtype(kv)
    L = int(wl.ctx_lens[0])
    t = np.arange(L)
    pg = torch.as_tensor(wl.block_table[0, t // 16].astype(np.int64))
    row = torch.as_tensor(t % 16)
    v = wl.pool("v", "cpu", poison=True)
    v[pg, :, row, 0] = torch.as_tensor((t % 256) / 256.0, dtype=torch.float32).to(v.dtype)[:, None]
    v[pg, :, row, 1] = 0.375
    vh = workloads.kv_host(v)
    q0 = np.zeros((1, wl.num_q_heads, wl.head_dim), dtype=np.uint16)       # +0.0 bits
    G = wl.num_q_heads // wl.num_kv_heads
    kz = np.zeros((1, wl.num_kv_heads, 16, wl.head_dim), dtype=vh.dtype)    # unused: q = 0
    mean = np.zeros((wl.num_q_heads, wl.head_dim))
    for hk in range(wl.num_kv_heads):
        # q = 0: the oracle's state is the plain mean of the valid V rows
        kk = np.broadcast_to(kz, (wl.num_pages, wl.num_kv_heads, 16, wl.head_dim))
        o, lse = pa.range_state(q0, kk, vh, wl.block_table, 0, hk, 0, L, wl.scale, 16)
        assert np.all(o[:, 1] == 0.375)
        assert np.allclose(lse, np.log(L), rtol=0, atol=1e-12)
        mean[hk * G:(hk + 1) * G] = o
    vd = v.to("cuda")
    for merge, sched in COMBOS:
        run = Run(wl, poison=True, merge_mode=merge, schedule=SCHEDULES[sched])
        run.q.zero_()
        run.v = vd
        o, l = run.decode()
        where = f"long {kv} merge {merge} {sched}"
        say(f"{where}: max |LSE - ln L| = {np.abs(l[0] - np.log(L)).max():.2e}, "
            f"max |O - mean| = {np.abs(o[0] - mean).max():.2e}")
        assert np.abs(l[0] - np.log(L)).max() <= 5e-6, where
        assert np.all(o[0, :, 1] == 0.375), where
        assert np.all(np.abs(o[0] - mean) <= 2.0 ** -8 * np.abs(mean) + 1e-5), where
        run.close()


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("name", ["long", "short"])
def test_full_size_gather_bits_match_oracle(name, kv):
    """The decode kernel's own gather on items of the full-size queues, bit
    for bit against the oracle's gather: the first, the last and items spread
    over the queue (both ends of every sampled row)."""
    wl = workloads.CONFIGS[name]().with_kv_dtype(kv)
    run = Run(wl, poison=True)
    run.dec.build_queue(wl.ctx_lens)
    items, *_ = pkv.pkv_plan_queue(run.cfg, wl.ctx_lens)
    _, k, v = host_inputs(run)
    pick = sorted(set([0, len(items) - 1] + list(range(0, len(items), max(1, len(items) // 24)))))
    for i in pick:
        it = items[i]
        n = int(it["tok_end"] - it["tok_begin"])
        ko = torch.zeros(n, wl.head_dim, dtype=wl.kv_torch_dtype, device="cuda")
        vo = torch.zeros_like(ko)
        pkv.pkv_debug_gather(run.dec.handle, run.tensors(), int(i), ko, vo, run.dec.stream)
        torch.cuda.synchronize()
        args = (wl.block_table, int(it["seq"]), int(it["kv_head"]), int(it["tok_begin"]),
                int(it["tok_end"]), 16)
        rk, rv = pa.gather_tokens(k, *args), pa.gather_tokens(v, *args)
        gk, gv = workloads.kv_host(ko), workloads.kv_host(vo)
        assert gk.dtype == rk.dtype and gk.tobytes() == rk.tobytes(), f"{name} K item {i}"
        assert gv.dtype == rv.dtype and gv.tobytes() == rv.tobytes(), f"{name} V item {i}"
    say(f"{name} {kv}: gather of {len(pick)} of {len(items)} items bit-exact")
    run.close()


# ------------------------------------------ online-softmax rescale cases ----

def _sign_pattern(d):
    """A fixed +-1 vector (bf16-exact): q = s_h u and K_t = r_t u make every
    dot product an exact sum of equal terms, D r_t s_h."""
    return np.where((np.arange(d) * 7 + 3) % 5 < 2, 1.0, -1.0)


def scored_workload(kind, kv, d=128, hq=8, hkv=2, lens=None):
    """Inputs whose scores force the running maximum up after the first tile.

    rising: K_t = r_t u with r_t = alpha * frac((t + 1) / period) rounded to
    bf16, per row a different period (the whole row, one 1024-token range,
    300 tokens), so scores climb by up to ~65 log2 units inside every range
    and every 8-lane group's tokens, in steps that exceed the lazy-rescale
    threshold many times.  peaked: random K, and one token per row with
    K = kappa u scoring ~30 nats (~43 log2 units above the rest) for the
    group's first head: on the last valid row of a partial last page, at the
    first token of a middle range, or mid-row.  The query heads of a group are
    u scaled by 1, 1/2, 3/4 and 5/4."""
    if lens is None:
        lens = [5000, 4099, 1030, 17, 2049, 300]
    wl = workloads.custom(f"scores_{kind}", lens, hq, hkv, d, spare_pages=3, kv_dtype=kv)
    G = hq // hkv
    u = _sign_pattern(d)
    hs = np.array([1.0, 0.5, 0.75, 1.25])[np.arange(G) % 4]
    q = np.zeros((wl.batch, hq, d), dtype=np.float32)
    for h in range(hq):
        q[:, h] = u * hs[h % G]
    k = wl.pool("k", "cpu", poison=True)
    base = float(wl.scale * d)                      # score of r_t = 1 for s_h = 1, nats
    for b, L in enumerate(lens):
        if L == 0:
            continue
        t = np.arange(L)
        pg = torch.as_tensor(wl.block_table[b, t // 16].astype(np.int64))
        row = torch.as_tensor(t % 16)
        if kind == "rising":
            period = [L, 1024, 300][b % 3]
            r = (45.0 / base) * (((t % period) + 1) / period)
            kt = torch.as_tensor(r[:, None] * u[None, :], dtype=torch.float32)
            kt = kt.to(torch.bfloat16).to(k.dtype)          # bf16-exact in both caches
            k[pg, :, row, :] = kt[:, None, :]
        else:
            peak = {0: L - 1, 1: 2048, 2: L - 1, 3: 16, 4: 1024, 5: L // 2}[b % 6]
            peak = min(peak, L - 1)
            kt = torch.as_tensor((30.0 / base) * u, dtype=torch.float32).to(torch.bfloat16).to(k.dtype)
            k[int(wl.block_table[b, peak // 16]), :, peak % 16, :] = kt
    qt = torch.as_tensor(q).to(torch.bfloat16)
    return wl, qt, k


@pytest.mark.parametrize("sched", list(SCHEDULES))
@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("kind", ["rising", "peaked"])
def test_online_softmax_rescale_cases(kind, kv, sched):
    """Scores that rise past the running maximum inside a range, on a state
    that already holds tokens, so that the lazy rescale of l and acc runs
    (PersistentKV page, Methodology 1 "Sequence Splitting": the partial
    online-softmax state).  Every output against the oracle, split (both
    merges) and unsplit, D = 128 / G = 4 and D = 64 / G = 8."""
    for d, hq, hkv, lens in ((128, 8, 2, None), (64, 16, 2, [3000, 700, 33])):
        wl, q, k = scored_workload(kind, kv, d, hq, hkv, lens)
        ro, rl = pa.decode_attention(workloads.bits_u16(q), workloads.kv_host(k),
                                     workloads.kv_host(wl.pool("v", "cpu", poison=True)),
                                     wl.block_table, wl.ctx_lens, wl.scale, wl.page_size)
        say(f"{kind} d={d}: oracle LSE range {rl.min():.2f} .. {rl.max():.2f}")
        kd = k.to("cuda")
        qd = q.to("cuda")
        for policy, chunk, merge in ((pkv.PKV_POLICY_SPLIT, 1024, pkv.PKV_MERGE_FUSED),
                                     (pkv.PKV_POLICY_SPLIT, 1024, pkv.PKV_MERGE_SEPARATE),
                                     (pkv.PKV_POLICY_NO_SPLIT, 0, pkv.PKV_MERGE_FUSED)):
            run = Run(wl, policy=policy, kv_chunk_tokens=chunk, merge_mode=merge,
                      schedule=SCHEDULES[sched])
            run.k, run.q = kd, qd
            o, l = run.decode()
            check(o, l, ro, rl, f"{kind} {kv} {sched} d={d} policy {policy} merge {merge}", lse_tol(wl))
            run.close()


# ------------------------------------------------ streams and ordering ----

def test_queue_rebuilds_and_decodes_on_other_streams_stay_ordered():
    """Queue builds (host uploads on the handle's stream, device builds on a
    third stream) alternate with decodes on a second stream, with no host
    synchronisation in between: each decode must read the queue built just
    before it, and no build may overwrite a queue a decode still reads."""
    base = [60000, 300, 41, 5000, 0, 777]
    wl = workloads.custom("streams", base, 8, 2, 128, spare_pages=2)
    run = Run(wl, poison=True, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=1024)
    s_dec, s_build = torch.cuda.Stream(), torch.cuda.Stream()
    rng = np.random.default_rng(5)
    plans, outs, dev_lens = [], [], []
    for i in range(10):
        lens = np.minimum(rng.integers(0, 4 * np.asarray(base) // 3 + 1), base).astype(np.int32)
        lens[0] = base[0] - 997 * i                 # a long row keeps every decode busy
        plans.append(lens)
        dev_lens.append(torch.as_tensor(lens).to("cuda"))
        outs.append((torch.full_like(run.out, float("nan")), torch.full_like(run.lse, float("nan"))))
    torch.cuda.synchronize()                        # inputs in place; no host sync from here on
    for i, lens in enumerate(plans):
        if i % 2 == 0:
            run.dec.build_queue(lens)
        else:
            pkv.pkv_build_queue_device(run.dec.handle, dev_lens[i], s_build)
        o, lse = outs[i]
        t = pkv.make_tensors(run.q, run.k, run.v, run.bt, run.lens, o, lse)
        pkv.pkv_decode(run.dec.handle, t, s_dec)
    torch.cuda.synchronize()
    assert run.dec.query()["error_code"] == 0
    q, k, v = host_inputs(run)
    for i, (lens, (o, lse)) in enumerate(zip(plans, outs)):
        ro, rl = pa.decode_attention(q, k, v, wl.block_table, lens, wl.scale, 16)
        check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
              ro, rl, f"call {i} ({'host' if i % 2 == 0 else 'device'} build)")
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
            assert len(ref["items"]) <= dec.layout.max_items      # the default capacity holds every queue
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


@pytest.mark.parametrize("sched", list(SCHEDULES))
def test_clear_error_restarts_the_merge_counters(sched):
    """An item the kernel refuses never counts in for its row's merge; after
    pkv_clear_error the row and group arrival counters and the page cursors
    start from zero again.  Garbage planted in that region (as a refused item
    would leave it) must not change a following decode of split rows, with
    one- and two-level merges."""
    wl = workloads.custom("clear_counters", TWO_LEVEL_LENS, 8, 2, 128, spare_pages=5)
    run = Run(wl, kv_chunk_tokens=1024, schedule=SCHEDULES[sched])
    ro, rl = oracle_full(wl)
    o, l = run.decode()
    check(o, l, ro, rl, f"clear counters {sched} before")
    lay = run.dec.layout
    region = run.dec.workspace[lay.arrive_off:lay.loop_off].view(torch.int32)
    n_counters = wl.batch * wl.num_kv_heads + lay.max_items       # row counters, then group counters
    cursors = run.dec.workspace[lay.cursor_off:lay.loop_off].view(torch.int32)
    # every counter and cursor is back at zero after a launch (the region's
    # alignment padding is never written)
    assert int(region[:n_counters].abs().sum()) == 0 and int(cursors.abs().sum()) == 0
    region.copy_(torch.randint(1, 7, region.shape, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    pkv.pkv_clear_error(run.dec.handle)
    assert int(region.abs().sum()) == 0
    for call in range(2):
        o, l = run.decode()
        check(o, l, ro, rl, f"clear counters {sched} after, call {call}")
    run.close()

def test_device_builder_reports_bad_lengths_in_the_error_word():
    """The device queue builder checks every length before it writes a queue:
    a length beyond max_pages_per_seq pages sets PKV_DEVERR_BAD_ITEM with the
    row as detail and leaves an empty queue (nothing is read: the builder
    touches only the lengths); pkv_query reports it and pkv_clear_error makes
    the handle usable again."""
    cfg = pkv.make_config(4, 1, 128, 64, 4, 100, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=256,
                          num_cus=256)
    dec = pkv.PagedDecoder(cfg)
    for lens, row in (([5, 100 * 16 + 1, 7], 1), ([3, 9, 1600, -1], 3)):
        dec.build_queue_device(torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda())
        torch.cuda.synchronize()
        st = dec.query(raise_on_fault=False)
        assert st["status"] == pkv.PKV_ERR_DEVICE_FAULT, lens
        assert st["error_code"] == pkv.PKV_DEVERR_BAD_ITEM and st["error_detail"] == row, (lens, st)
        assert st["n_items"] == 0
        pkv.pkv_clear_error(dec.handle)
    lens = [5, 100 * 16, 7, 0]
    dec.build_queue_device(torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda())
    torch.cuda.synchronize()
    st = dec.query()
    assert st["error_code"] == 0 and st["n_items"] == len(wq.build_queue(lens, 1, 256, 256, 2)["items"])
    dec.close()


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


# ------------------------------------------------------ maximum size ----

@pytest.mark.parametrize("kv", KVS)
def test_million_token_context(kv):
    """Maximum-size case: one context of 1,048,571 tokens (65,536 pages, the
    last one partial; 4.3 GB of bf16 K+V, 8.6 GB fp32) in fitted ranges of
    32,768 tokens merged across 256 workgroups.  (1) q = 0 counts every token
    under the atomic and steal schedules: LSE = ln L to fp32 rounding (one
    page more or less moves it by 1.5e-5), V column 1 = 0.375 bit for bit and
    column 0 = (t mod 256) / 256 to its exact mean within bf16 rounding;
    (2) the generator's q: every query head of the last KV head against the
    oracle."""
    L = 1_048_571
    wl = workloads.long_context(ctx=L).with_kv_dtype(kv)
    run = Run(wl, poison=True)
    say(f"million-token context ({kv}): {wl.num_pages} pages")
    o, l = run.decode()
    info = run.info
    assert info.split and info.n_items == 256 and info.chunk_tokens == 32768
    hk = wl.num_kv_heads - 1
    G = wl.num_q_heads // wl.num_kv_heads
    ro, rl = oracle_unit(wl, workloads.bits_u16(run.q), 0, hk)
    check(o[0:1, hk * G:(hk + 1) * G], l[0:1, hk * G:(hk + 1) * G], ro[None], rl[None],
          f"million {kv}: KV head {hk} against the oracle", lse_tol(wl))
    run.close()
    del run
    torch.cuda.empty_cache()
    exact = np.mean((np.arange(L) % 256) / 256.0)
    for sched in (pkv.PKV_SCHEDULE_ATOMIC, pkv.PKV_SCHEDULE_STEAL):
        run = Run(wl, poison=True, schedule=sched)
        t = torch.arange(L, device="cuda")
        pg = torch.as_tensor(wl.block_table[0].astype(np.int64), device="cuda")[t // 16]
        row = t % 16
        run.v[pg, :, row, 0] = ((t % 256).float() / 256.0).to(run.v.dtype)[:, None]
        run.v[pg, :, row, 1] = 0.375
        run.q.zero_()
        o, l = run.decode()
        where = f"million {kv} schedule {sched}"
        say(f"{where}: max |LSE - ln L| = {np.abs(l[0] - np.log(L)).max():.2e}, "
            f"max |O0 - mean| = {np.abs(o[0, :, 0] - exact).max():.2e}")
        assert np.abs(l[0] - np.log(L)).max() <= 5e-6, where
        assert np.all(o[0, :, 1] == 0.375), where
        assert np.abs(o[0, :, 0] - exact).max() <= 2.0 ** -8 * exact + 1e-6, where
        run.close()
        del run, t, pg, row
        torch.cuda.empty_cache()


@pytest.mark.parametrize("kv", KVS)
def test_queue_filling_the_default_capacity(kv):
    """Chunk mode "fit" with 1024 CUs as the policy input (the device runs the
    queue with its own workgroups, in claimed rounds): one KV head and a row
    of 32,768 pages, the last one partial, give exactly 1024 ranges of 512
    tokens, the default capacity max(Hkv * max_batch, CUs, 1024) filled to
    its last item.  The row merges in two levels (32 groups of 32 ranges);
    fused and separate merges, host- and device-built queues, every output
    against the oracle."""
    L = 32768 * 16 - 5
    wl = workloads.custom("capacity_1024", [L], 4, 1, 128, kv_dtype=kv)
    ro = rl = None
    for merge in (pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE):
        run = Run(wl, num_cus=1024, merge_mode=merge)
        assert run.dec.layout.max_items == 1024
        if ro is None:
            ro, rl = oracle_unit(wl, workloads.bits_u16(run.q), 0, 0)
        for device_queue in (False, True):
            o, l = run.decode(device_queue=device_queue)
            if not device_queue:
                assert run.info.split and run.info.n_items == 1024 and run.info.chunk_tokens == 512
            else:
                hdr = run.queue_bytes()["hdr"]
                assert list(hdr) == [1024, 1, 1, 512, 1], hdr
            check(o, l, ro[None], rl[None], f"capacity {kv} merge {merge} device queue {device_queue}",
                  lse_tol(wl))
        run.close()
        del run
        torch.cuda.empty_cache()


# ------------------------------------------------ seeded random sweep ----

def _random_case(rng, i):
    """One configuration drawn over everything the library accepts at small
    size: head_dim, group size (8 only at head_dim 64), KV heads, ragged lengths (empty rows, one
    token, page boundaries, long rows), policy, range length, queue order,
    merge, schedule and cache type."""
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8] if d == 64 else [1, 2, 4]))     # group 8 is built for head_dim 64
    hkv = int(rng.choice([1, 2, 4]))
    b = int(rng.integers(1, 7))
    pool = [0, 1, 15, 16, 17, 255, 256, 257, 1023, 2049, 3000, 4097, 9000, 20000]
    lens = [int(rng.choice(pool)) if rng.random() < 0.5 else int(rng.integers(1, 12000)) for _ in range(b)]
    policy = int(rng.choice([pkv.PKV_POLICY_AUTO, pkv.PKV_POLICY_SPLIT, pkv.PKV_POLICY_NO_SPLIT]))
    chunk = int(rng.choice([0, 0, 16, 256, 1024, 2048]))
    cfg = dict(policy=policy, kv_chunk_tokens=chunk,
               order=int(rng.choice([pkv.PKV_ORDER_CANONICAL, pkv.PKV_ORDER_LPT])),
               merge_mode=int(rng.choice([pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE])),
               schedule=int(rng.choice([pkv.PKV_SCHEDULE_ATOMIC, pkv.PKV_SCHEDULE_STATIC,
                                        pkv.PKV_SCHEDULE_PAGES, pkv.PKV_SCHEDULE_STEAL])),
               num_cus=int(rng.choice([0, 0, 8, 64])))
    kv = str(rng.choice(KVS))
    return f"random_{i}", lens, g * hkv, hkv, d, kv, cfg


@pytest.mark.parametrize("block", range(4))
def test_seeded_random_configurations_against_oracle(block):
    """Forty seeded random configurations (ten per block), every output
    against the oracle on two calls in a row, and the host queue's split
    decision and item count against the oracle's queue (num_cus = 0 is the
    device's CU count)."""
    rng = np.random.default_rng([20260623, block])
    cus_dev = torch.cuda.get_device_properties(0).multi_processor_count
    for i in range(10):
        name, lens, hq, hkv, d, kv, cfg = _random_case(rng, 10 * block + i)
        say(name, "lens", lens, "hq", hq, "hkv", hkv, "d", d, "kv", kv, cfg)
        wl = workloads.custom(name, lens, hq, hkv, d, spare_pages=3, kv_dtype=kv)
        cus = cfg.pop("num_cus") or cus_dev
        run = Run(wl, num_cus=cus, **cfg)
        ro, rl = oracle_full(wl)
        ref = wq.build_queue(lens, hkv, cus, cfg["kv_chunk_tokens"], cfg["policy"], cfg["order"])
        for call in range(2):
            run.out.fill_(float("nan"))
            run.lse.fill_(float("nan"))
            o, l = run.decode()
            assert run.info.n_items == len(ref["items"]) and bool(run.info.split) == ref["split"], name
            check(o, l, ro, rl, f"{name} call {call}", lse_tol(wl))
            for bb, L in enumerate(lens):
                if L == 0:
                    assert np.all(o[bb] == 0) and np.all(np.isneginf(l[bb])), name
        run.close()


# Rows for the steal schedule at 2048-token ranges (128 pages): every full
# range gives its first 24 pages to the row's pool (a quarter of the range,
# rounded down to whole claim rounds of 8 waves x 3 pages); the last range
# gives min(24, its pages - 1 rounded down to 24), so a last range of one
# token or one page gives none, and one of 98 pages gives 24.
STEAL_LENS = [20000, 6149, 4096, 2049, 0, 300, 16 * 128 * 3 + 16 * 25 + 7]


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("merge", [pkv.PKV_MERGE_FUSED, pkv.PKV_MERGE_SEPARATE],
                         ids=["fused_merge", "separate_merge"])
def test_steal_pool_against_oracle_and_repeats(merge, kv):
    """Steal schedule on rows whose ranges share a pool: every output against
    the oracle on repeated calls (the claimed pool pages differ from call to
    call; every cursor must start each call at zero again), and against the
    unsplit decode of the same rows."""
    wl = workloads.custom("steal_pool", STEAL_LENS, 8, 2, 128, spare_pages=3, kv_dtype=kv)
    run = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=2048, merge_mode=merge,
              schedule=pkv.PKV_SCHEDULE_STEAL)
    flat = Run(wl, policy=pkv.PKV_POLICY_NO_SPLIT)
    ob, lb = flat.decode()
    ro, rl = oracle_full(wl)
    check(ob, lb, ro, rl, f"unsplit {kv}", lse_tol(wl))
    for call in range(6):
        run.out.fill_(float("nan"))
        run.lse.fill_(float("nan"))
        o, l = run.decode()
        check(o, l, ro, rl, f"steal {kv} merge {merge} call {call}", lse_tol(wl))
        check(o, l, ob, lb, f"steal vs unsplit {kv} merge {merge} call {call}", lse_tol(wl))
        assert np.all(o[4] == 0) and np.all(np.isneginf(l[4]))
    lay = run.dec.layout
    cur = run.dec.workspace[lay.cursor_off:lay.loop_off]
    assert int(cur.cpu().view(torch.int32).abs().sum()) == 0       # every cursor re-armed
    assert run.dec.query()["error_code"] == 0
    run.close()
    flat.close()


@pytest.mark.parametrize("kv", KVS)
def test_steal_pool_counts_every_token(kv):
    """The closed forms of the structured cases (q = 0: LSE = ln L_b, V column
    means, 0.375 bit for bit) under the steal schedule with pools in use: a
    pool page read twice or never moves LSE by about 16 / L_b."""
    wl = workloads.custom("steal_structured", STEAL_LENS, 8, 2, 128, spare_pages=3, kv_dtype=kv)
    v = wl.pool("v", "cpu", poison=True)
    for b, L in enumerate(STEAL_LENS):
        t = np.arange(L)
        pg = torch.as_tensor(wl.block_table[b, t // 16].astype(np.int64))
        row = torch.as_tensor(t % 16)
        v[pg, :, row, 0] = torch.as_tensor((t % 256) / 256.0, dtype=torch.float32).to(v.dtype)[:, None]
        v[pg, :, row, 1] = 0.375
    run = Run(wl, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=2048, schedule=pkv.PKV_SCHEDULE_STEAL)
    run.q.zero_()
    run.v = v.to("cuda")
    for call in range(3):
        o, l = run.decode()
        for b, L in enumerate(STEAL_LENS):
            if L == 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))
                continue
            where = f"steal {kv} call {call} row {b} (L = {L})"
            assert np.abs(l[b] - np.log(L)).max() <= 5e-6, where
            exact = np.mean((np.arange(L) % 256) / 256.0)
            assert np.abs(o[b, :, 0] - exact).max() <= 2.0 ** -8 * exact + 1e-6, where
            assert np.all(o[b, :, 1] == 0.375), where
    run.close()


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

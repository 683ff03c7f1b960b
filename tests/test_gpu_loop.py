"""GPU tests of the resident session loop through the C ABI.

The resident kernel is launched once at pkv_create and serves every step the
host publishes; no other GPU work may be queued while it runs (it holds every
CU), so each test writes all steps' outputs into per-step buffers and reads
them only after pkv_destroy.  Parity bar as for the one-shot path: max-abs
2e-2 and mean-abs 2e-3 against the float64 oracle, for O and for the LSE.
Loops run with a bf16 and with an fp32 KV cache.
"""

import time

import numpy as np
import pytest
import torch

from oracle import paged_attention as pa
from paged_kv_attention_persistent_amd import pkv, workloads

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    print("[gpu-loop]", *a, flush=True)


class Loop:
    """Inputs of a session loop on the GPU plus a resident decoder."""

    def __init__(self, sl, timeout_ms=20000, **cfgkw):
        self.sl = sl
        dev = "cuda"
        self.k = sl.pools("k", dev)
        self.v = sl.pools("v", dev)
        self.q = sl.queries(dev)
        if sl.append:
            self.new_k = sl.new_kv("k", dev)
            self.new_v = sl.new_kv("v", dev)
            cfgkw["append"] = 1
        self.bt = torch.as_tensor(sl.block_tables).to(dev)
        self.out = torch.full((sl.steps, sl.layers, sl.sessions, sl.num_q_heads, sl.head_dim),
                              float("nan"), dtype=torch.bfloat16, device=dev)
        self.lse = torch.full((sl.steps, sl.layers, sl.sessions, sl.num_q_heads), float("nan"),
                              dtype=torch.float32, device=dev)
        self.lens = torch.zeros(sl.sessions, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        cfgkw.setdefault("num_cus", torch.cuda.get_device_properties(0).multi_processor_count)
        cfgkw.setdefault("kv_dtype", pkv.PKV_KV_F32 if sl.kv_dtype == "f32" else pkv.PKV_KV_BF16)
        self.cfg = pkv.make_config(sl.num_q_heads, sl.num_kv_heads, sl.head_dim, sl.pages_per_layer,
                                   sl.sessions, sl.max_pages, scale=sl.scale, persistent=1,
                                   num_layers=sl.layers, timeout_ms=timeout_ms, **cfgkw)
        self.stream = torch.cuda.Stream()
        self.dec = pkv.PagedDecoder(self.cfg, stream=self.stream)
        if sl.append:
            pkv.pkv_loop_set_free_pages(self.dec.handle, sl.free_pages)
        S, H, D = sl.sessions, sl.num_q_heads, sl.head_dim
        self.strides = (S * H * D, sl.pages_per_layer * sl.num_kv_heads * 16 * D,
                        S * sl.max_pages, S * H * D, S * H)

    def tensors(self, t):
        sl = self.sl
        extra = {}
        if sl.append:
            extra = dict(new_k=self.new_k[t], new_v=self.new_v[t],
                         layer_stride_new=sl.sessions * sl.num_kv_heads * sl.head_dim)
        return pkv.make_tensors(self.q[t], self.k, self.v, self.bt, self.lens, self.out[t],
                                self.lse[t], batch=sl.sessions, block_table_stride=sl.max_pages,
                                layer_strides=self.strides, **extra)

    def step(self, t):
        info = self.dec.build_queue(self.sl.ctx_lens(t))
        t0 = time.perf_counter()
        pkv.pkv_decode(self.dec.handle, self.tensors(t), self.stream)
        return time.perf_counter() - t0, info

    def close(self):
        self.dec.close()
        torch.cuda.synchronize()


def oracle_unit(sl, t, layer, s, hk):
    """The oracle over the logical token sequence of (step, layer, session, KV
    head): the cache's tokens, and with append the tokens steps 0..t wrote."""
    L = int(sl.ctx_lens(t)[s])
    G = sl.num_q_heads // sl.num_kv_heads
    if L == 0:
        return np.zeros((G, sl.head_dim)), np.full(G, -np.inf)
    npg = -(-L // 16)

    def paged(which):
        rows = workloads.kv_host(sl.token_rows(which, t, layer, s, hk))
        full = np.zeros((npg * 16, sl.head_dim), dtype=rows.dtype)
        full[:L] = rows
        return full.reshape(npg, 1, 16, sl.head_dim)

    qg = workloads.bits_u16(sl.query_unit(t, layer, s))[None, hk * G:(hk + 1) * G]
    return pa.range_state(qg, paged("k"), paged("v"), np.arange(npg)[None], 0, 0, 0, L, sl.scale, 16)


def check_all(lp, units=None):
    sl = lp.sl
    G = sl.num_q_heads // sl.num_kv_heads
    o = lp.out.float().cpu().numpy().astype(np.float64)
    l = lp.lse.cpu().numpy().astype(np.float64)
    if units is None:
        units = [(t, layer, s, hk) for t in range(sl.steps) for layer in range(sl.layers)
                 for s in range(sl.sessions) for hk in range(sl.num_kv_heads)]
    errs, lerrs = [], []
    for (t, layer, s, hk) in units:
        ro, rl = oracle_unit(sl, t, layer, s, hk)
        got_o = o[t, layer, s, hk * G:(hk + 1) * G]
        got_l = l[t, layer, s, hk * G:(hk + 1) * G]
        assert np.all(np.isfinite(got_o)), (t, layer, s, hk)
        assert np.array_equal(np.isfinite(got_l), np.isfinite(rl)), (t, layer, s, hk)
        errs.append(np.abs(got_o - ro))
        fin = np.isfinite(rl)
        lerrs.append(np.abs(got_l[fin] - rl[fin]) if fin.any() else np.zeros(1))
    err = np.concatenate([e.ravel() for e in errs])
    lerr = np.concatenate(lerrs)
    say(f"{len(units)} units: max_abs={err.max():.3e} mean_abs={err.mean():.3e} lse_max={lerr.max():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS and lerr.max() <= MAX_ABS


@pytest.mark.parametrize("variant", ["nosplit_d128", "split_d128", "nosplit_d64_g8", "many_steps", "two_level",
                                     "nosplit_d128_f32", "split_d128_f32", "nosplit_d64_g8_f32",
                                     "two_level_f32"])
def test_small_loop_every_output(variant):
    say("variant", variant)
    kv = "f32" if variant.endswith("_f32") else "bf16"
    variant = variant.removesuffix("_f32")
    if variant == "nosplit_d128":
        sl = workloads.session_loop(seed=11, sessions=5, layers=3, steps=4, lo=1, hi=60,
                                    num_q_heads=8, num_kv_heads=2, name="loop_small")
        sl.l0[2] = 0                                # an empty row at step 0
        kw = dict(policy=pkv.PKV_POLICY_NO_SPLIT)
    elif variant == "split_d128":
        sl = workloads.session_loop(seed=12, sessions=4, layers=3, steps=3, lo=30, hi=200,
                                    num_q_heads=8, num_kv_heads=2, name="loop_split")
        kw = dict(policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=32)
    elif variant == "nosplit_d64_g8":
        sl = workloads.session_loop(seed=13, sessions=6, layers=2, steps=3, lo=1, hi=90,
                                    num_q_heads=16, num_kv_heads=2, head_dim=64, name="loop_d64")
        kw = dict(policy=pkv.PKV_POLICY_NO_SPLIT)
    elif variant == "two_level":
        # rows of up to 76 ranges of 32 tokens: their merges run in two levels
        # (groups of 32 ranges, then the group states), in every layer; one
        # short row beside them merges in one level
        sl = workloads.session_loop(seed=18, sessions=3, layers=3, steps=3, lo=1200, hi=2400,
                                    num_q_heads=8, num_kv_heads=2, name="loop_two_level")
        sl.l0[1] = 40
        kw = dict(policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=32)
    else:
        # many short steps: each counter slot is reused 24 times, so a
        # workgroup that lags a step behind meets a slot in every state
        sl = workloads.session_loop(seed=17, sessions=3, layers=2, steps=48, lo=1, hi=70,
                                    num_q_heads=4, num_kv_heads=1, name="loop_many")
        kw = dict(policy=pkv.PKV_POLICY_AUTO, kv_chunk_tokens=32)
    lp = Loop(sl.with_kv_dtype(kv), **kw)
    try:
        for t in range(sl.steps):
            dt, info = lp.step(t)
            say(f"step {t}: {dt * 1e3:.2f} ms, items/layer {info.n_items}, split {info.split}")
            if variant == "two_level":
                longest = -(-int(max(sl.ctx_lens(t))) // 32)
                assert longest > 64, longest          # three groups of ranges
        st = lp.dec.query()
        assert st["loop_out_epoch"] == sl.steps and st["loop_alive"] == 1
    finally:
        lp.close()
    check_all(lp)


def test_loop_idle_timeout_is_reported_and_destroy_is_clean():
    sl = workloads.session_loop(seed=14, sessions=2, layers=2, steps=2, lo=5, hi=40,
                                num_q_heads=4, num_kv_heads=1, name="loop_idle")
    lp = Loop(sl, timeout_ms=300)
    try:
        lp.step(0)                                  # one good step
        time.sleep(1.0)                             # the kernel's idle limit passes
        with pytest.raises(pkv.PkvError) as e:
            lp.step(1)
        assert e.value.status == pkv.PKV_ERR_TIMEOUT
        st = lp.dec.query(raise_on_fault=False)
        assert st["loop_exit_reason"] == 2 and st["loop_alive"] == 0
    finally:
        lp.close()


def test_loop_create_destroy_without_steps():
    sl = workloads.session_loop(seed=15, sessions=2, layers=1, steps=1, lo=5, hi=40,
                                num_q_heads=4, num_kv_heads=1, name="loop_empty")
    lp = Loop(sl)
    time.sleep(0.05)
    lp.close()                                      # exit flag; kernel leaves its poll loop


def test_loop_rejects_one_shot_only_calls():
    sl = workloads.session_loop(seed=16, sessions=2, layers=2, steps=1, lo=5, hi=40,
                                num_q_heads=4, num_kv_heads=1, name="loop_reject")
    lp = Loop(sl)
    try:
        with pytest.raises(pkv.PkvError) as e:
            lp.dec.build_queue_device(lp.lens)
        assert e.value.status == pkv.PKV_ERR_STATE
        lp.dec.build_queue(sl.ctx_lens(0))
        t = lp.tensors(0)
        t.layer_stride_q = 0
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_decode(lp.dec.handle, t, lp.stream)
        assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    finally:
        lp.close()


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("variant", ["nosplit", "split"])
def test_loop_append_writes_tokens_and_grows_block_tables(variant, kv):
    # each step appends every session's newest token and takes a page from the
    # free list when it opens one; outputs match the oracle over the logical
    # token sequence, and the cache and block tables end up bit-exact
    say("append", variant, kv)
    sl = workloads.session_loop(seed=21, sessions=5, layers=2, steps=40, lo=1, hi=40,
                                num_q_heads=8, num_kv_heads=2, name="loop_append", append=True,
                                kv_dtype=kv)
    kw = dict(policy=pkv.PKV_POLICY_NO_SPLIT) if variant == "nosplit" else \
        dict(policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=32)
    lp = Loop(sl, **kw)
    try:
        for t in range(sl.steps):
            lp.step(t)
        assert pkv.pkv_loop_free_pages(lp.dec.handle) == 0      # every free page used once
    finally:
        lp.close()
    check_all(lp)
    want_bt = sl.appended_block_tables(sl.steps)
    assert np.array_equal(lp.bt.cpu().numpy(), want_bt)
    kb, vb = workloads.kv_host(lp.k.cpu()), workloads.kv_host(lp.v.cpu())
    for layer in range(sl.layers):
        for s in range(sl.sessions):
            for hk in range(sl.num_kv_heads):
                for t in range(sl.steps):
                    j = int(sl.l0[s]) - 1 + t
                    pg = want_bt[layer, s, j // 16]
                    want_k = workloads.kv_host(sl.new_kv_unit("k", t, layer, s, hk))
                    want_v = workloads.kv_host(sl.new_kv_unit("v", t, layer, s, hk))
                    assert kb[layer, pg, hk, j % 16].tobytes() == want_k.tobytes()
                    assert vb[layer, pg, hk, j % 16].tobytes() == want_v.tobytes()


def test_loop_append_errors():
    sl = workloads.session_loop(seed=22, sessions=3, layers=1, steps=3, lo=1, hi=20,
                                num_q_heads=4, num_kv_heads=1, name="loop_append_err", append=True)
    lp = Loop(sl)
    try:
        pkv.pkv_loop_set_free_pages(lp.dec.handle, [])            # nothing to take
        opens = [t for t in range(sl.steps) if any((int(L) - 1 + t) % 16 == 0 for L in sl.l0)]
        for t in range(sl.steps):
            if t in opens:
                with pytest.raises(pkv.PkvError) as e:
                    lp.step(t)
                assert e.value.status == pkv.PKV_ERR_CAPACITY
                break
            lp.step(t)
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_loop_set_free_pages(lp.dec.handle, [sl.pages_per_layer])   # outside the pool
        assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    finally:
        lp.close()
    plain = workloads.session_loop(seed=23, sessions=2, layers=1, steps=1, lo=5, hi=40,
                                   num_q_heads=4, num_kv_heads=1, name="loop_plain")
    lp = Loop(plain)
    try:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_loop_set_free_pages(lp.dec.handle, [0])
        assert e.value.status == pkv.PKV_ERR_STATE
    finally:
        lp.close()


def oracle_unit_len(sl, t, layer, s, hk, L):
    """The oracle over the first L tokens of a slot's pages (a session that
    joined the slot reads the slot's cache from token 0)."""
    G = sl.num_q_heads // sl.num_kv_heads
    if L == 0:
        return np.zeros((G, sl.head_dim)), np.full(G, -np.inf)
    npg = -(-L // 16)
    pages = sl.block_tables[layer, s, :npg]
    ks = workloads.kv_host(sl.slabs("k", layer, pages, hk))[:, None]
    vs = workloads.kv_host(sl.slabs("v", layer, pages, hk))[:, None]
    qg = workloads.bits_u16(sl.query_unit(t, layer, s))[None, hk * G:(hk + 1) * G]
    return pa.range_state(qg, ks, vs, np.arange(npg)[None], 0, 0, 0, L, sl.scale, 16)


@pytest.mark.parametrize("kv", ["bf16", "f32"])
@pytest.mark.parametrize("variant", ["nosplit", "split"])
def test_loop_session_churn_every_output(variant, kv):
    """Sessions leave and join at step boundaries (the Wave Persistent Kernel
    note, "Runtime and timing boundary"): a slot is reset to a new, shorter
    context, or stays empty for a step or two, and the resident kernel keeps
    running.  Every output of every step, layer and slot against the oracle
    over the slot's first L tokens; empty slots must hold the neutral state."""
    say("churn", variant, kv)
    sl = workloads.session_loop(seed=31, sessions=6, layers=2, steps=30, lo=1, hi=150,
                                num_q_heads=8, num_kv_heads=2, name="loop_churn", kv_dtype=kv)
    lens, joins = sl.churn_lens(seed=32, life=(2, 7), join_lo=1, idle_prob=0.3)
    assert joins >= 10 and (lens == 0).any()
    shorter = sum(int(lens[t, s] < lens[t - 1, s]) for t in range(1, sl.steps) for s in range(sl.sessions))
    assert shorter >= 5                                     # slots re-used with shorter contexts
    kw = dict(policy=pkv.PKV_POLICY_NO_SPLIT) if variant == "nosplit" else \
        dict(policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=32)
    lp = Loop(sl, **kw)
    try:
        for t in range(sl.steps):
            lp.dec.build_queue(lens[t])
            pkv.pkv_decode(lp.dec.handle, lp.tensors(t), lp.stream)
        st = lp.dec.query()
        assert st["loop_out_epoch"] == sl.steps and st["loop_alive"] == 1
    finally:
        lp.close()
    G = sl.num_q_heads // sl.num_kv_heads
    o = lp.out.float().cpu().numpy().astype(np.float64)
    l = lp.lse.cpu().numpy().astype(np.float64)
    errs, lerrs = [], []
    for t in range(sl.steps):
        for layer in range(sl.layers):
            for s in range(sl.sessions):
                for hk in range(sl.num_kv_heads):
                    L = int(lens[t, s])
                    got_o = o[t, layer, s, hk * G:(hk + 1) * G]
                    got_l = l[t, layer, s, hk * G:(hk + 1) * G]
                    if L == 0:
                        assert np.all(got_o == 0) and np.all(np.isneginf(got_l)), (t, layer, s)
                        continue
                    ro, rl = oracle_unit_len(sl, t, layer, s, hk, L)
                    assert np.all(np.isfinite(got_o)), (t, layer, s, hk)
                    errs.append(np.abs(got_o - ro).ravel())
                    lerrs.append(np.abs(got_l - rl))
    err = np.concatenate(errs)
    lerr = np.concatenate(lerrs)
    say(f"churn {variant} {kv}: {joins} joins, {len(errs)} units: max_abs={err.max():.3e} "
        f"mean_abs={err.mean():.3e} lse_max={lerr.max():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    assert lerr.max() <= (1e-4 if kv == "f32" else MAX_ABS)

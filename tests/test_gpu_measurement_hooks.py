"""GPU tests of the library's measurement hooks, through the C ABI: the
per-item trace (pkv_set_trace), the decode events (pkv_set_decode_events)
and the two bandwidth probes (pkv_copy_probe, pkv_read_probe).

The hooks observe a decode and must not change it: a traced or timed decode
is bit-identical to a plain one, and that plain one is held to the oracle
(max-abs 2e-2, mean-abs 2e-3, in float64, as in the parity tests).  The
trace's records must describe the run the scheduler is documented to make
(each item once, the static first round, monotone clocks on one 100 MHz
clock that agrees with the events around the kernel); the probes' outputs
have exact values computed here on the host.
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention as pa
from paged_kv_attention_persistent_amd import pkv, workloads

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
SENTINEL = -1                 # int64 all-ones: a slot no record has touched
WG_FLAG = 1 << 63


def say(*a):
    print("[gpu-hooks]", *a, flush=True)


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


class Case:
    def __init__(self, wl, **cfgkw):
        self.wl = wl
        self.q = wl.q("cuda")
        self.k = wl.pool("k", "cuda", True)
        self.v = wl.pool("v", "cuda", True)
        self.bt = wl.block_table_t("cuda")
        self.lens = wl.ctx_lens_t("cuda")
        self.out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")
        cfgkw.setdefault("num_cus", cus())
        cfg = pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, max(wl.batch, 1),
                              wl.max_pages_per_seq, scale=wl.scale, **cfgkw)
        self.dec = pkv.PagedDecoder(cfg)
        self.info = self.dec.build_queue(wl.ctx_lens)
        self.grid = int(self.dec.query()["grid"])

    def decode(self):
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        pkv.pkv_decode(self.dec.handle, pkv.make_tensors(self.q, self.k, self.v, self.bt, self.lens, self.out,
                                                         self.lse), self.dec.stream)
        torch.cuda.synchronize()
        assert self.dec.query()["error_code"] == 0
        return self.out.clone(), self.lse.clone()

    def close(self):
        self.dec.close()


def small_workload():
    # ragged lengths, an empty row, rows split into many 256-token ranges: with
    # kv_chunk_tokens 256 the queue holds 394 items, more than one per workgroup
    return workloads.custom("hooks", [37, 1000, 0, 5000, 300, 17, 2900, 40000], 8, 2, 128, spare_pages=3)


def check_oracle(wl, out, lse):
    q = workloads.bits_u16(wl.q("cpu"))
    k = workloads.kv_host(wl.pool("k", "cpu", True))
    v = workloads.kv_host(wl.pool("v", "cpu", True))
    ro, rl = pa.decode_attention(q, k, v, wl.block_table, wl.ctx_lens, wl.scale, wl.page_size)
    o = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ro)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
    l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.abs(l[fin] - rl[fin]).max() <= MAX_ABS


def trace_buffer(slots, guard=8):
    return torch.full((4 * (slots + guard),), SENTINEL, dtype=torch.int64, device="cuda")


def records(buf):
    return buf.cpu().numpy().view(np.uint64).reshape(-1, 4)


def check_item_records(rec, n_items, grid):
    idx = rec[:, 0] & 0xFFFFFFFF
    wg = (rec[:, 0] >> 32) & 0x7FFFFFFF
    assert np.array_equal(idx, np.arange(n_items, dtype=np.uint64)), "item record at the wrong slot"
    assert not (rec[:, 0] & np.uint64(WG_FLAG)).any()
    assert (wg < grid).all()
    assert (rec[:, 1] <= rec[:, 2]).all(), "item ends before it starts"
    assert ((rec[:, 3] >> 32) < 8).all(), "XCC id outside the 8 dies"
    return wg


@pytest.mark.parametrize("sched", ["atomic", "static"])
def test_trace_records_every_item_once_and_changes_nothing(sched):
    wl = small_workload()
    schedule = {"atomic": pkv.PKV_SCHEDULE_ATOMIC, "static": pkv.PKV_SCHEDULE_STATIC}[sched]
    c = Case(wl, schedule=schedule, kv_chunk_tokens=256)
    try:
        n, grid = c.info.n_items, c.grid
        say("trace", sched, "items", n, "grid", grid)
        assert n > grid, "the queue should need more than one round"
        plain_out, plain_lse = c.decode()
        check_oracle(wl, plain_out, plain_lse)

        buf = trace_buffer(n + grid)
        pkv.pkv_set_trace(c.dec.handle, buf)
        traced_out, traced_lse = c.decode()
        assert torch.equal(traced_out.view(torch.int16), plain_out.view(torch.int16))
        assert torch.equal(traced_lse.view(torch.int32), plain_lse.view(torch.int32))
        rec = records(buf)
        assert (rec[n + grid:] == np.uint64(2**64 - 1)).all(), "write past the capacity"

        wg = check_item_records(rec[:n], n, grid)
        first = np.arange(min(n, grid))
        assert np.array_equal(wg[first], first.astype(np.uint64)), "first round is not static"
        if sched == "static":
            assert np.array_equal(wg, (np.arange(n) % grid).astype(np.uint64))

        w = rec[n:n + grid]
        assert np.array_equal(w[:, 0], np.arange(grid, dtype=np.uint64) * np.uint64((1 << 32) + 1) |
                              np.uint64(WG_FLAG))
        assert (w[:, 1] <= w[:, 2]).all()
        assert ((w[:, 3] >> 32) < 8).all()
        # an item starts after its workgroup began work, on the same wave slot
        wgi = wg.astype(np.int64)
        assert (rec[:n, 1] >= w[wgi, 2]).all()
        assert np.array_equal(rec[:n, 3], w[wgi, 3])
        # items of one workgroup run one after another
        for g in np.unique(wgi):
            mine = np.sort(np.flatnonzero(wgi == g))
            starts = rec[mine, 1]
            order = np.argsort(starts, kind="stable")
            s, e = rec[mine[order], 1], rec[mine[order], 2]
            assert (s[1:] >= e[:-1]).all(), f"workgroup {g} overlaps its own items"

        pkv.pkv_set_trace(c.dec.handle, None)
        buf.fill_(SENTINEL)
        again_out, _ = c.decode()
        assert torch.equal(again_out.view(torch.int16), plain_out.view(torch.int16))
        assert (records(buf) == np.uint64(2**64 - 1)).all(), "trace written after it was cleared"
    finally:
        c.close()


def test_trace_capacity_bounds_the_records():
    wl = small_workload()
    c = Case(wl, kv_chunk_tokens=256)
    try:
        n = c.info.n_items
        cap = max(1, n // 2)
        buf = trace_buffer(n + c.grid)
        pkv.pkv_set_trace(c.dec.handle, buf[:4 * cap])
        c.decode()
        rec = records(buf)
        check_item_records(rec[:cap], cap, c.grid)
        assert (rec[cap:] == np.uint64(2**64 - 1)).all(), "record at or beyond the capacity"
    finally:
        c.close()


def test_trace_and_event_arguments_are_checked():
    c = Case(small_workload())
    try:
        buf = trace_buffer(16)
        h = pkv.C.c_void_p(c.dec.handle)
        for ptr, cap in [(buf.data_ptr() + 4, 4), (buf.data_ptr(), 0), (buf.data_ptr(), -3)]:
            assert pkv.lib().pkv_set_trace(h, pkv.C.c_void_p(ptr), cap) == pkv.PKV_ERR_INVALID_ARG
        assert (records(buf) == np.uint64(2**64 - 1)).all()
        a = torch.cuda.Event(enable_timing=True)
        a.record(c.dec.stream)
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_set_decode_events(c.dec.handle, a, None)
        assert e.value.status == pkv.PKV_ERR_INVALID_ARG
        pkv.pkv_set_decode_events(c.dec.handle, None, None)
        out, lse = c.decode()                            # the refusals left the handle usable
        check_oracle(c.wl, out, lse)
        assert (records(buf) == np.uint64(2**64 - 1)).all(), "a refused trace buffer was written"
    finally:
        c.close()


def test_decode_events_bracket_the_kernel_and_agree_with_the_trace_clock():
    wl = workloads.long_context()
    c = Case(wl)
    try:
        n, grid = c.info.n_items, c.grid
        c.decode()                                       # code object loaded, clocks up
        before = torch.cuda.Event(enable_timing=True)
        after = torch.cuda.Event(enable_timing=True)
        before.record(c.dec.stream)                      # creates the events
        after.record(c.dec.stream)
        torch.cuda.synchronize()
        buf = trace_buffer(n + grid)
        pkv.pkv_set_trace(c.dec.handle, buf)
        pkv.pkv_set_decode_events(c.dec.handle, before, after)
        out, _ = c.decode()
        ms = before.elapsed_time(after)
        rec = records(buf)
        check_item_records(rec[:n], n, grid)
        w = rec[n:n + grid]
        span_ms = (int(rec[:n, 2].max()) - int(w[:, 1].min())) / 1e5       # 100 MHz ticks
        say("events", f"{ms:.4f} ms", "trace span", f"{span_ms:.4f} ms", "items", n)
        # the kernel runs between the two events; its records span most of that time
        assert 0.0 < span_ms <= ms + 0.02
        assert span_ms >= 0.5 * ms
        # 131072 tokens x 8 KV heads x 128 x 2 B x (K, V) take well over 20 us at any HBM rate
        assert ms > 0.02

        pkv.pkv_set_decode_events(c.dec.handle, None, None)
        pkv.pkv_set_trace(c.dec.handle, None)
        again, _ = c.decode()
        assert before.elapsed_time(after) == ms, "events recorded after they were cleared"
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    finally:
        c.close()


@pytest.mark.parametrize("grid", [0, 1, 7, 64])
def test_copy_probe_copies_exactly_and_nothing_more(grid):
    nbytes = (3 << 20) + 16 * 37                       # a ragged tail after the unrolled steps
    g = torch.Generator(device="cpu").manual_seed(11 + grid)
    src_h = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    src = src_h.cuda()
    dst = torch.full((nbytes // 4 + 1024,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    say("copy probe", nbytes, "bytes, grid", grid)
    pkv.pkv_copy_probe(dst, src, nbytes, grid)
    torch.cuda.synchronize()
    d = dst.cpu()
    assert torch.equal(d[:nbytes // 4], src_h)
    assert (d[nbytes // 4:] == 0x5A5A5A5A).all()


def xor_fold(words: np.ndarray, threads: int) -> np.ndarray:
    """What each probe thread stores: the xor of the four words of every
    16-byte vector it reads (vectors t, t + threads, t + 2 * threads, ...)."""
    per_vec = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1)
    pad = (-per_vec.size) % threads
    per_vec = np.concatenate([per_vec, np.zeros(pad, dtype=per_vec.dtype)])
    return np.bitwise_xor.reduce(per_vec.reshape(-1, threads), axis=0)


@pytest.mark.parametrize("grid", [0, 1, 3, 1024])
def test_read_probe_sink_is_the_xor_fold_of_the_input(grid):
    nbytes = (5 << 20) + 16 * 101
    rng = np.random.default_rng(23 + grid)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    wg = grid if grid else 4 * cus()
    sink = torch.full((wg * 256 + 256,), 0x33, dtype=torch.int32, device="cuda")
    say("read probe", nbytes, "bytes, grid", grid)
    pkv.pkv_read_probe(src, nbytes, sink, grid)
    torch.cuda.synchronize()
    s = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(s[:wg * 256], xor_fold(words, wg * 256))
    assert (s[wg * 256:] == 0x33).all()


def test_probe_arguments_are_checked():
    a = torch.zeros(1024, dtype=torch.int32, device="cuda")
    b = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for args in [(a, b, 4008, 0), (a[1:], b, 1024, 0), (a, b[1:], 1024, 0), (a, b, 0, 0), (a, b, 1024, -1)]:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_copy_probe(*args)
        assert e.value.status == pkv.PKV_ERR_INVALID_ARG, args
    for args in [(a, 4008, b, 0), (a[1:], 1024, b, 0), (a, 0, b, 0), (a, 1024, b, -1)]:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_read_probe(*args)
        assert e.value.status == pkv.PKV_ERR_INVALID_ARG, args
    torch.cuda.synchronize()

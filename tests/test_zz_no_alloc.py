"""GPU test of pkv_decode_noalloc, the entry point for callers that cannot
allocate: its outputs must equal, bit for bit, those of pkv_decode on a
handle with a caller workspace and a device-built queue (the same kernels
over the same queue), and both must match the float64 oracle.  Calls run back
to back on one device, each later one smaller than the first, so that the
shared static scratch is re-used with stale contents from the call before."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as pa
from paged_kv_attention_persistent_amd import pkv, workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)


def inputs(wl):
    dev = "cuda"
    return dict(q=wl.q(dev), k=wl.pool("k", dev, True), v=wl.pool("v", dev, True),
                bt=wl.block_table_t(dev), lens=wl.ctx_lens_t(dev))


def outputs(wl):
    o = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    return o, torch.full((wl.batch, wl.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")


def config(wl, **kw):
    return pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages, max(wl.batch, 1),
                           wl.max_pages_per_seq, scale=wl.scale,
                           num_cus=torch.cuda.get_device_properties(0).multi_processor_count, **kw)


def with_workspace(wl, x, cfg):
    """The existing entry point: pkv_build_queue_device + pkv_decode."""
    o, l = outputs(wl)
    dec = pkv.PagedDecoder(cfg)
    dec.build_queue_device(x["lens"])
    pkv.pkv_decode(dec.handle, pkv.make_tensors(x["q"], x["k"], x["v"], x["bt"], x["lens"], o, l), dec.stream)
    torch.cuda.synchronize()
    assert dec.query()["error_code"] == 0
    dec.close()
    return o, l


def no_alloc(wl, x, cfg, err):
    o, l = outputs(wl)
    t = pkv.make_tensors(x["q"], x["k"], x["v"], x["bt"], x["lens"], o, l)
    pkv.pkv_decode_noalloc(cfg, x["lens"], t, err, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return o, l


def against_oracle(wl, o, l, where):
    ro, rl = pa.decode_attention(workloads.bits_u16(wl.q("cpu")), workloads.kv_host(wl.pool("k", "cpu")),
                                 workloads.kv_host(wl.pool("v", "cpu")), wl.block_table, wl.ctx_lens,
                                 wl.scale, wl.page_size)
    o = o.float().cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    err = np.abs(o - ro)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin), where
    lerr = np.abs(l[fin] - rl[fin]).max() if fin.any() else 0.0
    say(f"{where}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} lse_max={lerr:.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr <= 2e-2, where


CALLS = [
    # name, lens, Hq, Hkv, D, config
    ("split_rows", [20000, 5000, 3, 0, 9000, 4097], 32, 8, 128, dict(policy=pkv.PKV_POLICY_SPLIT,
                                                                     kv_chunk_tokens=1024)),
    ("smaller", [700, 0, 33], 8, 2, 128, dict()),
    ("smallest_d64", [256], 4, 1, 64, dict(merge_mode=pkv.PKV_MERGE_SEPARATE)),
    ("page_claims", [3000, 1, 1500], 8, 2, 128, dict(policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=512,
                                                     schedule=pkv.PKV_SCHEDULE_PAGES)),
    ("steal_pool", [9000, 4100, 2], 8, 2, 128, dict(policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=2048,
                                                     schedule=pkv.PKV_SCHEDULE_STEAL)),
]


def test_no_alloc_equals_workspace_entry_point_on_calls_in_a_row():
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for name, lens, hq, hkv, d, kw in CALLS:
        wl = workloads.custom(f"noalloc_{name}", lens, hq, hkv, d, spare_pages=3)
        x = inputs(wl)
        cfg = config(wl, **kw)
        a_o, a_l = no_alloc(wl, x, cfg, err)
        b_o, b_l = with_workspace(wl, x, cfg)
        assert int(err.item()) == 0, name
        if kw.get("schedule") in (pkv.PKV_SCHEDULE_PAGES, pkv.PKV_SCHEDULE_STEAL):
            # page claims differ from launch to launch: equal to rounding only
            assert (a_o.float() - b_o.float()).abs().max().item() <= 2e-2, name
            fin = torch.isfinite(b_l)
            assert torch.equal(torch.isfinite(a_l), fin)
            assert (a_l[fin] - b_l[fin]).abs().max().item() <= 2e-2, name
        else:
            assert torch.equal(a_o.view(torch.int16), b_o.view(torch.int16)), name
            assert torch.equal(a_l.view(torch.int32), b_l.view(torch.int32)), name
        against_oracle(wl, a_o, a_l, f"no-alloc {name}")
        against_oracle(wl, b_o, b_l, f"workspace {name}")


def test_no_alloc_rejects_what_it_cannot_hold():
    wl = workloads.custom("noalloc_reject", [100], 8, 2, 128, spare_pages=1)
    x = inputs(wl)
    o, l = outputs(wl)
    t = pkv.make_tensors(x["q"], x["k"], x["v"], x["bt"], x["lens"], o, l)
    big = config(wl, max_items=1 << 16)                  # partial states far beyond the scratch
    assert pkv.pkv_workspace_size(big) > 16 << 20
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_noalloc(big, x["lens"], t)
    assert e.value.status == pkv.PKV_ERR_CAPACITY
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_noalloc(config(wl, persistent=1), x["lens"], t)
    assert e.value.status == pkv.PKV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()                  # nothing was enqueued


def test_no_alloc_reports_a_bad_page_in_the_error_word():
    wl = workloads.custom("noalloc_badpage", [40, 50], 4, 1, 128, spare_pages=1)
    x = inputs(wl)
    x["bt"][1, 2] = wl.num_pages + 7
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    no_alloc(wl, x, config(wl), err)
    assert int(err.item()) == pkv.PKV_DEVERR_PAGE_OOB
    x["bt"][1, 2] = int(wl.block_table[1, 2])            # a good call after it is clean again
    err.zero_()
    o, l = no_alloc(wl, x, config(wl), err)
    assert int(err.item()) == 0
    against_oracle(wl, o, l, "no-alloc after a fault")

"""CPU tests of the C-ABI library: it loads, exports every entry point that
include/pkv.h declares, and its host-side logic (config checks, workspace
layout, the adaptive policy and the compact queue) matches the oracle's
queue byte for byte.  No kernel is launched here."""

import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import work_queue as wq
from paged_kv_attention_persistent_amd import pkv, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PKV_API\s+[\w\s\*]+?\b(pkv_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = pkv.lib()
    names = declared_symbols()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in pkv.h but not exported"
    assert set(names) == set(pkv.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (pkv_\w+)", out))
    assert exported == set(names), exported ^ set(names)


def test_struct_sizes_match_the_header():
    src = r"""
#include <stdio.h>
#include "pkv.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\n", sizeof(pkv_config), sizeof(pkv_tensors),
         sizeof(pkv_queue_info), sizeof(pkv_runtime_info), sizeof(pkv_layout));
  return 0; }
"""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "s.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "s")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        sizes = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    assert sizes == [C.sizeof(pkv.pkv_config), C.sizeof(pkv.pkv_tensors),
                     C.sizeof(pkv.pkv_queue_info), C.sizeof(pkv.pkv_runtime_info),
                     C.sizeof(pkv.pkv_layout)]


def test_status_strings():
    assert pkv.pkv_status_string(0) == "ok"
    assert pkv.pkv_status_string(pkv.PKV_ERR_DEVICE_FAULT) == "device fault"
    assert pkv.pkv_status_string(-99) == "unknown status"


def cfg_for(wl, num_cus=256, **kw):
    return pkv.make_config(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages,
                           max(wl.batch, 1), wl.max_pages_per_seq, num_cus=num_cus, **kw)


def compare_with_oracle(cfg, lens, hkv, num_cus, chunk, policy, order):
    items, n_chunks, part_off, merge_rows, info = pkv.pkv_plan_queue(cfg, lens)
    ref = wq.build_queue(lens, hkv, num_cus, chunk, policy, order)
    assert items.tobytes() == ref["items"].tobytes()
    assert np.array_equal(n_chunks[:len(lens)], ref["n_chunks"])
    assert np.array_equal(part_off, ref["part_off"])
    assert np.array_equal(merge_rows, ref["merge_rows"])
    assert bool(info.split) == ref["split"]
    assert info.chunk_tokens == ref["chunk_tokens"]
    assert info.n_items == len(ref["items"])
    sep = cfg.merge_mode == pkv.PKV_MERGE_SEPARATE
    assert info.launches_per_step == 1 + (sep and len(ref["merge_rows"]) > 0)
    return info


@pytest.mark.parametrize("name", ["tiny", "long", "mixed", "short"])
@pytest.mark.parametrize("order", [pkv.PKV_ORDER_CANONICAL, pkv.PKV_ORDER_LPT])
def test_host_queue_matches_oracle_on_workloads(name, order):
    for seed in (workloads.MEASURE_SEED, workloads.CALIBRATION_SEED):
        wl = workloads.CONFIGS[name](seed)
        cfg = cfg_for(wl, order=order)
        info = compare_with_oracle(cfg, wl.ctx_lens, wl.num_kv_heads, 256, 0,
                                   wq.POLICY_AUTO, order)
        assert info.kv_bytes == wl.kv_bytes
        fixed = cfg_for(wl, order=order, kv_chunk_tokens=4096)
        compare_with_oracle(fixed, wl.ctx_lens, wl.num_kv_heads, 256, 4096, wq.POLICY_AUTO, order)


def test_host_queue_matches_oracle_random():
    rng = np.random.default_rng(7)
    for trial in range(300):
        bsz = int(rng.integers(0, 20))
        hkv = int(rng.choice([1, 2, 8]))
        chunk = int(rng.choice([0, 16, 64, 4096]))
        maxp = int(rng.integers(1, 40))
        lens = rng.integers(0, maxp * 16 + 1, size=bsz)
        if bsz and rng.random() < 0.3:
            lens[rng.integers(0, bsz)] = 0
        policy = int(rng.integers(0, 3))
        order = int(rng.integers(0, 2))
        cus = int(rng.choice([1, 8, 256]))
        cfg = pkv.make_config(hkv * 4, hkv, 128, 1000, max(bsz, 1), maxp, policy=policy,
                              order=order, kv_chunk_tokens=chunk, num_cus=cus,
                              merge_mode=int(rng.integers(0, 2)))
        compare_with_oracle(cfg, lens.tolist(), hkv, cus, chunk, policy, order)


def test_host_fit_chunk_matches_oracle_on_long_random_rows():
    # lengths of thousands of pages, so the bisection lands above the 64-page floor
    rng = np.random.default_rng(23)
    for trial in range(200):
        bsz = int(rng.integers(1, 300))
        hkv = int(rng.choice([1, 2, 8]))
        cus = int(rng.choice([8, 64, 256, 1024]))
        maxp = int(rng.integers(1, 6000))
        lens = rng.integers(0, maxp * 16 + 1, size=bsz)
        lens[rng.random(bsz) < 0.2] = 0
        policy = int(rng.integers(0, 3))
        cfg = pkv.make_config(hkv * 4, hkv, 128, 1000, bsz, maxp, policy=policy, num_cus=cus)
        compare_with_oracle(cfg, lens.tolist(), hkv, cus, 0, policy, pkv.PKV_ORDER_CANONICAL)


def test_config_validation():
    good = pkv.make_config(32, 8, 128, 100, 4, 10, num_cus=256)
    assert pkv.pkv_workspace_size(good) > 0
    bad = [dict(num_q_heads=30), dict(head_dim=96), dict(page_size=32), dict(kv_chunk_tokens=100),
           dict(kv_chunk_tokens=-16),
           dict(num_pages=0), dict(wg_per_cu=9), dict(policy=7), dict(num_q_heads=64),
           dict(merge_mode=2), dict(persistent=1, schedule=1), dict(append=2),
           dict(append=1), dict(kv_dtype=2), dict(kv_dtype=-1),
           dict(schedule=4), dict(schedule=-1), dict(persistent=1, schedule=2),
           dict(persistent=1, schedule=3)]
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, num_pages=100, max_batch=4,
                max_pages_per_seq=10, num_cus=256)
    for b in bad:
        kw = dict(base)
        kw.update(b)
        with pytest.raises(pkv.PkvError):
            pkv.pkv_workspace_size(pkv.make_config(**kw))
    c = pkv.make_config(**base)
    c.struct_size = 4
    with pytest.raises(pkv.PkvError):
        pkv.pkv_workspace_size(c)
    c = pkv.make_config(**base)
    c.reserved[1] = 1
    with pytest.raises(pkv.PkvError):
        pkv.pkv_workspace_size(c)
    assert pkv.pkv_workspace_size(pkv.make_config(**dict(base, persistent=1, kv_dtype=1))) > 0


def test_page_claim_layout():
    # the page-claim schedule adds one 128-byte cursor per (row, KV head);
    # the queue and the other regions are unchanged
    kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, num_pages=100, max_batch=4,
              max_pages_per_seq=10, num_cus=256)
    a = pkv.pkv_workspace_layout(pkv.make_config(**kw))
    b = pkv.pkv_workspace_layout(pkv.make_config(schedule=pkv.PKV_SCHEDULE_PAGES, **kw))
    assert a.loop_off - a.cursor_off == 0
    assert b.loop_off - b.cursor_off == 4 * 8 * 128
    assert b.total_bytes - a.total_bytes == 4 * 8 * 128
    # the steal schedule: one 128-byte cursor per (row, KV head, wave), 8 waves
    c = pkv.pkv_workspace_layout(pkv.make_config(schedule=pkv.PKV_SCHEDULE_STEAL, **kw))
    assert c.loop_off - c.cursor_off == 4 * 8 * 128 * 8
    for f in ("queue_off", "n_chunks_off", "part_off_off", "row_len_off", "merge_rows_off", "items_off"):
        assert getattr(a, f) == getattr(b, f) == getattr(c, f)
    assert a.part_off_off < a.row_len_off < a.merge_rows_off < a.items_off


def test_f32_cache_plan_and_layout():
    # the fp32 cache changes neither the queue nor the workspace, only the
    # bytes a step reads
    from paged_kv_attention_persistent_amd import workloads
    wl = workloads.mixed()
    kw = dict(num_cus=256)
    a = pkv.make_config(32, 8, 128, wl.num_pages, wl.batch, wl.max_pages_per_seq, **kw)
    b = pkv.make_config(32, 8, 128, wl.num_pages, wl.batch, wl.max_pages_per_seq,
                        kv_dtype=pkv.PKV_KV_F32, **kw)
    ia, *_, infa = pkv.pkv_plan_queue(a, wl.ctx_lens)
    ib, *_, infb = pkv.pkv_plan_queue(b, wl.ctx_lens)
    assert ia.tobytes() == ib.tobytes()
    assert infb.kv_bytes == 2 * infa.kv_bytes == wl.with_kv_dtype("f32").kv_bytes
    assert pkv.pkv_workspace_size(a) == pkv.pkv_workspace_size(b)


def test_plan_rejects_bad_lengths_and_capacity():
    cfg = pkv.make_config(4, 1, 64, 100, 4, 4, num_cus=256)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan_queue(cfg, [10, 65])              # 65 > 4 pages * 16
    assert e.value.status == pkv.PKV_ERR_CAPACITY
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan_queue(cfg, [10, -1])
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan_queue(cfg, [1] * 5)                # batch > max_batch
    assert e.value.status == pkv.PKV_ERR_CAPACITY
    small = pkv.make_config(4, 1, 64, 100, 4, 4, num_cus=256, max_items=2)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan_queue(small, [1, 1, 1])
    assert e.value.status == pkv.PKV_ERR_CAPACITY


def test_layout_regions_are_ordered_and_aligned():
    cfg = pkv.make_config(32, 8, 128, 8192, 1, 8192, num_cus=256)
    lay = pkv.pkv_workspace_layout(cfg)
    # the layout does not depend on the CU count (create must accept it on any device)
    for cus in (1, 80, 256, 304):
        other = pkv.pkv_workspace_layout(pkv.make_config(32, 8, 128, 8192, 1, 8192, num_cus=cus))
        assert other.total_bytes == lay.total_bytes and other.max_items == lay.max_items
    offs = [lay.ctrl_off, lay.queue_off, lay.n_chunks_off, lay.part_off_off, lay.merge_rows_off,
            lay.items_off, lay.partial_o_off, lay.partial_lse_off, lay.arrive_off, lay.total_bytes]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.max_items == 1024                  # chunk mode "fit": max(Hkv * max_batch, 1024)
    assert lay.partial_lse_off - lay.partial_o_off >= lay.max_items * 4 * 128 * 4


def test_default_capacity_in_fit_mode_holds_every_queue():
    # a split queue in chunk mode "fit" holds at most max(1, CUs / Hkv) ranges
    # per KV head, or one range per row when no range length reaches that, so
    # max(Hkv * max_batch, CUs) items bound it whatever the rows' lengths
    big = pkv.pkv_workspace_layout(pkv.make_config(32, 8, 128, 100000, 512, 8192, num_cus=256))
    assert big.max_items == 8 * 512
    assert pkv.pkv_workspace_layout(pkv.make_config(32, 8, 128, 100000, 1, 8192, num_cus=2048)).max_items == 2048
    fixed = pkv.pkv_workspace_layout(pkv.make_config(32, 8, 128, 100000, 4, 8192, num_cus=256,
                                                     kv_chunk_tokens=4096))
    assert fixed.max_items == 8 * 4 * (8192 * 16 // 4096)
    rng = np.random.default_rng(11)
    for hkv in (1, 2, 8):
        for cus in (8, 80, 256, 304, 1024, 2048):
            for mb in (1, 3, 40, 300):
                maxp = 40000
                for policy in (pkv.PKV_POLICY_AUTO, pkv.PKV_POLICY_SPLIT):
                    cfg = pkv.make_config(hkv * 4, hkv, 128, 1000, mb, maxp, num_cus=cus, policy=policy)
                    cap = pkv.pkv_workspace_layout(cfg).max_items
                    assert cap == max(hkv * mb, cus, 1024)
                    batches = [[16 * maxp] * mb, [16 * maxp] + [1] * (mb - 1),
                               rng.integers(0, 16 * maxp + 1, size=mb).tolist(),
                               rng.integers(1, 200, size=mb).tolist()]
                    most = 0
                    for lens in batches:
                        items = pkv.pkv_plan_queue(cfg, lens)[0]
                        most = max(most, len(items))
                        assert len(items) <= max(hkv * mb, hkv * max(1, cus // hkv))
                    assert most <= cap
    # the bound is reached: one long row, one KV head, 1024 CUs
    cfg = pkv.make_config(4, 1, 128, 1000, 1, 32768, num_cus=1024)
    assert len(pkv.pkv_plan_queue(cfg, [16 * 32768])[0]) == 1024 == pkv.pkv_workspace_layout(cfg).max_items


def test_f32_stream_rounds_to_bf16_stream():
    # the fp32 cache's values round (RNE) to exactly the bf16 cache's values,
    # and carry low mantissa bits that bf16 cannot hold
    import torch
    from paged_kv_attention_persistent_amd import workloads
    wl = workloads.custom("f32_stream", [100, 37], 8, 2, 64, spare_pages=2)
    kb = wl.pool("k", "cpu", poison=True)
    kf = wl.with_kv_dtype("f32").pool("k", "cpu", poison=True)
    assert kf.dtype == torch.float32 and kb.dtype == torch.bfloat16
    fin = torch.isfinite(kf)
    assert torch.equal(fin, torch.isfinite(kb))            # the same slots poisoned
    assert torch.equal(kf[fin].to(torch.bfloat16).view(torch.int16), kb[fin].view(torch.int16))
    assert torch.equal(kf[~fin].view(torch.int32), torch.full_like(kf[~fin].view(torch.int32), 0x7FC00000))
    assert (kf[fin].view(torch.int32) & 0xFFFF).ne(0).float().mean() > 0.99
    sl = wl.with_kv_dtype("f32").pool_slabs("v", wl.block_table[0, :3], 1)
    full = wl.with_kv_dtype("f32").pool("v", "cpu", poison=False)
    assert torch.equal(sl, full[torch.as_tensor(wl.block_table[0, :3].astype(np.int64)), 1])


def test_traffic_record_follows_kernel_code_not_comments(tmp_path):
    # bench.py reports the committed traffic counters only while the kernel
    # code they were taken on is unchanged; comments and layout do not count
    import bench
    a = tmp_path / "a.hip"
    a.write_text("// note\nint f(int x) {\n  return x + 1; /* one */\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("int f(int x) { return x + 1; }  // another note\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_code_digest(a) == bench.kernel_code_digest(b) != bench.kernel_code_digest(c)
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    assert bench.measured_traffic(root) is None or bench.measured_traffic(root) > 536870912


def test_configs_whose_rows_could_need_more_than_65535_ranges_are_refused():
    # the item's range index is a 16-bit field: a config is refused when its
    # longest row at its range length would need more than 65535 ranges
    cfg = pkv.make_config(4, 1, 128, 64, 1, 65535, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=16,
                          num_cus=256, max_items=70000)
    items, n_chunks, *_ = pkv.pkv_plan_queue(cfg, [65535 * 16])
    assert n_chunks[0] == 65535 and int(items["chunk"].max()) == 65534
    ref = wq.build_queue([65535 * 16], 1, 256, 16, wq.POLICY_SPLIT)
    assert items.tobytes() == ref["items"].tobytes()
    big = pkv.make_config(4, 1, 128, 64, 1, 65536, policy=pkv.PKV_POLICY_SPLIT, kv_chunk_tokens=16,
                          num_cus=256, max_items=70000)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_workspace_size(big)
    assert e.value.status == pkv.PKV_ERR_CAPACITY


def test_plain_c_client_compiles_against_the_header():
    # include/pkv.h is plain C: the C consumer of the ABI (tests/c_abi) builds
    # with gcc -std=c11 -Wall -Wextra and links against libpkv.so and the HIP
    # runtime (it runs on the GPU in tests/test_gpu_c_abi.py)
    import shutil
    from paged_kv_attention_persistent_amd import build as b
    if not shutil.which("gcc") or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("gcc or the HIP runtime headers are missing")
    exe = b.build_c_client()
    assert os.path.exists(exe) and os.access(exe, os.X_OK)


def test_environment_overrides(monkeypatch):
    # PKV_POLICY / PKV_CHUNK_TOKENS / PKV_WG_PER_CU / PKV_SCHEDULE override the
    # config wherever the library resolves it; bad values are refused loudly
    for name in ("PKV_POLICY", "PKV_CHUNK_TOKENS", "PKV_WG_PER_CU", "PKV_SCHEDULE"):
        monkeypatch.delenv(name, raising=False)
    cfg = pkv.make_config(32, 8, 128, 8192, 1, 8192, num_cus=256)
    lens = [131072]
    *_, info = pkv.pkv_plan_queue(cfg, lens)
    assert info.split == 1 and info.chunk_tokens == 4096 and info.n_items == 256
    monkeypatch.setenv("PKV_POLICY", "nosplit")
    *_, info = pkv.pkv_plan_queue(cfg, lens)
    assert info.split == 0 and info.n_items == 8
    monkeypatch.setenv("PKV_POLICY", "split")
    monkeypatch.setenv("PKV_CHUNK_TOKENS", "8192")
    *_, info = pkv.pkv_plan_queue(cfg, lens)
    assert info.split == 1 and info.chunk_tokens == 8192 and info.n_items == 128
    monkeypatch.setenv("PKV_CHUNK_TOKENS", "")                 # empty: unset
    *_, info = pkv.pkv_plan_queue(cfg, lens)
    assert info.chunk_tokens == 4096
    monkeypatch.setenv("PKV_SCHEDULE", "steal")
    steal = pkv.pkv_workspace_layout(cfg)
    monkeypatch.delenv("PKV_SCHEDULE")
    plain = pkv.pkv_workspace_layout(cfg)
    assert steal.loop_off - steal.cursor_off == 4 * 32 * 8 * 8 and plain.loop_off == plain.cursor_off
    for name, value in (("PKV_POLICY", "sometimes"), ("PKV_CHUNK_TOKENS", "4k"), ("PKV_CHUNK_TOKENS", "100"),
                        ("PKV_WG_PER_CU", "9"), ("PKV_SCHEDULE", "random")):
        monkeypatch.setenv(name, value)
        with pytest.raises(pkv.PkvError):
            pkv.pkv_plan_queue(cfg, lens)
        monkeypatch.delenv(name)
    *_, info = pkv.pkv_plan_queue(cfg, lens)
    assert info.split == 1 and info.chunk_tokens == 4096

"""The C ABI from a plain C program: tests/c_abi/pkv_c_client.c, built with
gcc against include/pkv.h, libpkv.so and the HIP runtime only (no PyTorch in
its process), allocates its buffers with hipMalloc, creates a handle on a
stream of its own, builds the compact queue on the host, decodes twice and
reads the outputs back; it also checks that a head_dim the library does not
build and a workspace smaller than the layout are refused.  It writes its
host-side inputs (its own integer recipe: bf16-exact values, scattered pages,
NaN in every unused slot, -1 past each row's pages, an empty row) and the
outputs to a file; this test runs the oracle on those inputs and compares
every output (tolerances as in test_gpu_parity.py) and the queue's split
decision and size with the oracle's queue."""

import os
import subprocess

import numpy as np
import pytest

from oracle import paged_attention as pa
from oracle import work_queue as wq

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def client():
    from paged_kv_attention_persistent_amd import build as b
    src, exe = b.CLIENT_SRC, b.CLIENT
    lib = os.path.join(ROOT, "paged_kv_attention_persistent_amd", "libpkv.so")
    if not os.path.exists(exe) or os.path.getmtime(exe) < max(os.path.getmtime(src), os.path.getmtime(lib)):
        b.build_c_client()                      # a host-only gcc build of one small file
    return exe


def read_dump(path):
    raw = open(path, "rb").read()
    hdr = np.frombuffer(raw, dtype=np.int32, count=12)
    assert hdr[0] == 0x504B5643
    B, hq, hkv, d, p, npg, mp, n_items, split, chunk, cus = (int(x) for x in hdr[1:])
    off = 48

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a

    lens = take(np.int32, B)
    bt = take(np.int32, B * mp).reshape(B, mp)
    q = take(np.uint16, B * hq * d).reshape(B, hq, d)
    k = take(np.uint16, npg * hkv * p * d).reshape(npg, hkv, p, d)
    v = take(np.uint16, npg * hkv * p * d).reshape(npg, hkv, p, d)
    out = take(np.uint16, B * hq * d).reshape(B, hq, d)
    lse = take(np.float32, B * hq).reshape(B, hq)
    assert off == len(raw)
    return dict(B=B, hkv=hkv, d=d, lens=lens, bt=bt, q=q, k=k, v=v, out=out, lse=lse,
                n_items=n_items, split=split, chunk=chunk, cus=cus)


def test_plain_c_client_decodes_to_oracle(tmp_path):
    exe = client()
    dump = str(tmp_path / "c_client.bin")
    print("[c-abi] running", exe, flush=True)
    r = subprocess.run([exe, dump], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "refused head_dim 96" in r.stdout
    x = read_dump(dump)
    ref = wq.build_queue(x["lens"].tolist(), x["hkv"], x["cus"], 0)
    assert x["n_items"] == len(ref["items"]) and bool(x["split"]) == ref["split"]
    assert x["chunk"] == ref["chunk_tokens"]
    ro, rl = pa.decode_attention(x["q"], x["k"], x["v"], x["bt"], x["lens"], 1.0 / np.sqrt(x["d"]), 16)
    o = (x["out"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    l = x["lse"].astype(np.float64)
    assert np.all(np.isfinite(o))
    err = np.abs(o - ro)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin)
    lerr = np.abs(l[fin] - rl[fin]).max()
    print(f"[c-abi] max_abs={err.max():.3e} mean_abs={err.mean():.3e} lse_max={lerr:.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr <= 2e-2
    empty = np.where(x["lens"] == 0)[0]
    assert len(empty) == 1 and np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))

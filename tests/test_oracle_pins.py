"""Pins of the float64 oracle against things other than itself.

* a library routine: PyTorch's float64 scaled-dot-product attention on
  contiguous inputs (identity block table), with GQA by repeat-interleave;
* invariants: bitwise invariance under a permutation of the physical pages,
  insensitivity to poisoned (NaN) slots outside the valid tokens, and the
  exact split/merge identity (PersistentKV page, Methodology 1, "Sequence
  Splitting": the merge combines the split states exactly);
* a consistency law that fixes the LSE: appending one token with score s*
  and value v* must turn O into (e^LSE O + e^s* v*) / (e^LSE + e^s*);
* closed forms (hand-derived fixtures in tests/golden/closed_forms.json);
* planted mistakes: each plausible bug, planted in the oracle by
  monkeypatching it, must make at least one of the pins above fail.

The library, permutation, LSE-law and closed-form pins run for both cache
element types: bf16 bit patterns and float32 values (the fp32 attention
cache of the Wave Persistent Kernel note, "Same precision" list).  For
float32 the test widens values itself with numpy, independently of the
oracle's widening.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import paged_attention as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def f32_to_bf16_bits(x):
    """float -> bf16 bits by round-to-nearest-even (test-side input prep)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def kv_values(rng, shape, kv):
    """Random N(0,1) cache values: bf16 bits, or float32 with full mantissas."""
    x = rng.standard_normal(shape)
    return f32_to_bf16_bits(x) if kv == "bf16" else x.astype(np.float32)


def kv_f64(x):
    """Test-side widening of cache values (float32 by numpy's own cast)."""
    return np.asarray(x).astype(np.float64) if np.asarray(x).dtype == np.float32 else pa.bf16_bits_to_f64(x)


def random_case(rng, lens, hq, hkv, d, page_size, spare=3, permute=True, kv="bf16"):
    """Random inputs (q bf16, cache of element type kv); pool pages
    scattered; unused slots NaN."""
    lens = np.asarray(lens)
    need = [-(-int(L) // page_size) for L in lens]
    npg = sum(need) + spare
    maxp = max(max(need), 1)
    perm = rng.permutation(npg) if permute else np.arange(npg)
    bt = np.full((len(lens), maxp), -1, dtype=np.int64)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    k = kv_values(rng, (npg, hkv, page_size, d), kv)
    v = kv_values(rng, (npg, hkv, page_size, d), kv)
    q = f32_to_bf16_bits(rng.standard_normal((len(lens), hq, d)))
    nan = np.uint16(0x7FC0) if kv == "bf16" else np.float32("nan")
    used = np.zeros(npg, dtype=bool)
    for b, L in enumerate(lens):
        used[bt[b, :need[b]]] = True
        if L % page_size:
            k[bt[b, need[b] - 1], :, L % page_size:, :] = nan
            v[bt[b, need[b] - 1], :, L % page_size:, :] = nan
    k[~used] = nan
    v[~used] = nan
    return q, k, v, bt, lens


def sdpa_reference(q, k, v, bt, lens, scale, page_size):
    """torch float64 SDPA on K/V laid out contiguously (test-side unpaging)."""
    bsz, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((bsz, hq, d))
    for b, L in enumerate(lens):
        if L == 0:
            continue
        t = np.arange(L)
        kk = kv_f64(k[bt[b, t // page_size], :, t % page_size, :])                # [L][Hkv][D]
        vv = kv_f64(v[bt[b, t // page_size], :, t % page_size, :])
        qq = torch.from_numpy(pa.bf16_bits_to_f64(q[b]))[None, :, None, :]        # [1][Hq][1][D]
        kt = torch.from_numpy(kk).permute(1, 0, 2)[None]                          # [1][Hkv][L][D]
        vt = torch.from_numpy(vv).permute(1, 0, 2)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kt, vt, scale=scale, enable_gqa=(hq != hkv))
        out[b] = o[0, :, 0, :].numpy()
    return out


# ---------------------------------------------------------------- pins ----

def pin_sdpa(attend, seed=0, kv="bf16"):
    rng = np.random.default_rng(seed)
    for (lens, hq, hkv, d, P) in [([37, 64], 4, 2, 16, 16), ([5, 1, 33], 8, 2, 32, 4),
                                  ([70], 4, 1, 64, 16), ([9], 2, 2, 8, 2)]:
        q, k, v, bt, lens = random_case(rng, lens, hq, hkv, d, P, kv=kv)
        scale = 1.0 / math.sqrt(d)
        o, _ = attend(q, k, v, bt, lens, scale, P)
        ref = sdpa_reference(q, k, v, bt, lens, scale, P)
        if not np.allclose(o, ref, rtol=0, atol=1e-12):
            return False
    return True


def pin_permutation(attend, seed=1, kv="bf16"):
    rng = np.random.default_rng(seed)
    q, k, v, bt, lens = random_case(rng, [45, 16, 7], 4, 2, 16, 4, spare=5, kv=kv)
    o1, l1 = attend(q, k, v, bt, lens, 0.25, 4)
    perm = rng.permutation(k.shape[0])           # new physical page of old page p: perm[p]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    o2, l2 = attend(q, k2, v2, bt2, lens, 0.25, 4)
    return np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_lse_law(attend, seed=2, kv="bf16"):
    """Append a token with known score and value; O must mix by e^LSE."""
    rng = np.random.default_rng(seed)
    P, d = 4, 8
    q, k, v, bt, lens = random_case(rng, [10], 2, 1, d, P, spare=2, permute=False, kv=kv)
    scale = 0.5
    o1, l1 = attend(q, k, v, bt, lens, scale, P)
    # token 10 sits in logical page 2, row 2, currently past the end (NaN)
    phys = bt[0, 10 // P]
    kstar = kv_values(rng, d, kv)
    vstar = kv_values(rng, d, kv)
    k[phys, 0, 10 % P, :] = kstar
    v[phys, 0, 10 % P, :] = vstar
    o2, l2 = attend(q, k, v, bt, np.array([11]), scale, P)
    qf = pa.bf16_bits_to_f64(q[0])
    s = scale * (qf @ kv_f64(kstar))                            # [Hq]
    vs = kv_f64(vstar)
    for h in range(2):
        w_old, w_new = math.exp(l1[0, h]), math.exp(s[h])
        exp_o = (w_old * o1[0, h] + w_new * vs) / (w_old + w_new)
        exp_l = math.log(w_old + w_new)
        if not (np.allclose(o2[0, h], exp_o, atol=1e-12, rtol=0)
                and abs(l2[0, h] - exp_l) < 1e-12):
            return False
    return True


def pin_merge_identity(attend_range, merge, seed=3):
    rng = np.random.default_rng(seed)
    P = 4
    q, k, v, bt, lens = random_case(rng, [61], 4, 2, 16, P)
    L = int(lens[0])
    for _ in range(4):
        cuts = np.sort(rng.choice(np.arange(1, L), size=rng.integers(1, 6), replace=False))
        bounds = [0, *cuts.tolist(), L]
        for h_kv in range(2):
            whole_o, whole_l = attend_range(q, k, v, bt, 0, h_kv, 0, L, 0.3, P)
            parts = [attend_range(q, k, v, bt, 0, h_kv, lo, hi, 0.3, P)
                     for lo, hi in zip(bounds[:-1], bounds[1:])]
            parts.append(attend_range(q, k, v, bt, 0, h_kv, 5, 5, 0.3, P))  # neutral
            mo, ml = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            if not (np.allclose(mo, whole_o, atol=1e-12, rtol=0)
                    and np.allclose(ml, whole_l, atol=1e-12, rtol=0)):
                return False
    return True


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def golden_inputs(case):
    P, npg = case["page_size"], case["num_pages"]
    q = np.asarray(case["q"], dtype=np.float64)
    hq, d = q.shape
    hkv = len(case["k_tokens"])
    L = case["ctx_len"]
    k = np.full((npg, hkv, P, d), 0x7FC0, dtype=np.uint16)
    v = np.full((npg, hkv, P, d), 0x7FC0, dtype=np.uint16)
    bt = np.asarray([case["block_table"]], dtype=np.int64)
    for h in range(hkv):
        for t in range(L):
            k[bt[0, t // P], h, t % P] = f32_to_bf16_bits(case["k_tokens"][h][t])
            v[bt[0, t // P], h, t % P] = f32_to_bf16_bits(case["v_tokens"][h][t])
    return f32_to_bf16_bits(q)[None], k, v, bt, np.array([L]), case["scale"], P


def pin_golden(attend):
    for case in load_golden():
        q, k, v, bt, lens, scale, P = golden_inputs(case)
        o, l = attend(q, k, v, bt, lens, scale, P)
        eo = np.array([[float(x) for x in row] for row in case["expected_o"]])
        el = np.array([float(x) for x in case["expected_lse"]])
        if not np.allclose(o[0], eo, atol=1e-12, rtol=0):
            return False
        if not np.array_equal(np.isinf(l[0]), np.isinf(el)):
            return False
        fin = np.isfinite(el)
        if not np.allclose(l[0][fin], el[fin], atol=1e-12, rtol=0):
            return False
    return True


def pin_closed_forms(attend, seed=4, kv="bf16"):
    """q = 0 -> mean V and LSE = ln L;  constant V -> that constant;
    L = 1 -> v_0 and LSE = s_0;  equal K rows -> mean V, LSE = s + ln L."""
    rng = np.random.default_rng(seed)
    P, d = 8, 16
    q, k, v, bt, lens = random_case(rng, [57, 1, 23], 4, 1, d, P, kv=kv)
    scale = 0.25
    # q = 0
    qz = np.zeros_like(q)
    o, l = attend(qz, k, v, bt, lens, scale, P)
    for b, L in enumerate(lens):
        t = np.arange(L)
        vv = kv_f64(v[bt[b, t // P], 0, t % P, :])
        if not np.allclose(o[b], vv.mean(axis=0)[None], atol=1e-12, rtol=0):
            return False
        if not np.allclose(l[b], math.log(L), atol=1e-12, rtol=0):
            return False
    # L = 1 (row 1)
    o, l = attend(q, k, v, bt, lens, scale, P)
    k0 = kv_f64(k[bt[1, 0], 0, 0])
    v0 = kv_f64(v[bt[1, 0], 0, 0])
    s0 = scale * (pa.bf16_bits_to_f64(q[1]) @ k0)
    if not (np.allclose(o[1], v0[None], atol=1e-12, rtol=0)
            and np.allclose(l[1], s0, atol=1e-12, rtol=0)):
        return False
    # all K rows equal, V constant per dim
    k2, v2 = k.copy(), v.copy()
    row = kv_values(rng, d, kv)
    crow = kv_values(rng, d, kv)
    for b, L in enumerate(lens):
        t = np.arange(L)
        k2[bt[b, t // P], 0, t % P, :] = row
        v2[bt[b, t // P], 0, t % P, :] = crow
    o, l = attend(q, k2, v2, bt, lens, scale, P)
    for b, L in enumerate(lens):
        s = scale * (pa.bf16_bits_to_f64(q[b]) @ kv_f64(row))
        if not np.allclose(o[b], kv_f64(crow)[None], atol=1e-12, rtol=0):
            return False
        if not np.allclose(l[b], s + math.log(L), atol=1e-12, rtol=0):
            return False
    return True


def attend_oracle(q, k, v, bt, lens, scale, P):
    return pa.decode_attention(q, k, v, bt, lens, scale, P)


def all_attention_pins(attend):
    """Run every attention pin, for both cache element types where the pin
    takes one; a pin that raises counts as failed."""
    res = {}
    for name, pin, kvs in [("sdpa", pin_sdpa, KVS), ("permutation", pin_permutation, KVS),
                           ("lse_law", pin_lse_law, KVS), ("golden", pin_golden, (None,)),
                           ("closed_forms", pin_closed_forms, KVS)]:
        for kv in kvs:
            key = name if kv is None else f"{name}/{kv}"
            try:
                res[key] = bool(pin(attend) if kv is None else pin(attend, kv=kv))
            except (ValueError, IndexError, FloatingPointError, TypeError):
                res[key] = False
    return res


KVS = ("bf16", "f32")


# --------------------------------------------------------------- tests ----

def test_bf16_widening_exact():
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    got = pa.bf16_bits_to_f64(bits)
    want = [0.0, 1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38, -0.0]
    assert got.tolist() == want


def test_f32_widening_exact_and_other_types_refused():
    vals = np.array([1.0, 0.1, -3.4028234663852886e38, 1e-45, -0.0, 1.0 + 2.0 ** -23], dtype=np.float32)
    got = pa.kv_to_f64(vals)
    want = [1.0, 0.10000000149011612, -3.4028234663852886e38, 2.0 ** -149, -0.0, 1.0 + 2.0 ** -23]
    assert got.tolist() == want and np.signbit(got[4])
    assert pa.kv_to_f64(np.array([0x3F80], dtype=np.uint16)).tolist() == [1.0]
    for bad in (np.zeros(2, np.float16), np.zeros(2, np.float64), np.zeros(2, np.int32)):
        with pytest.raises(TypeError):
            pa.kv_to_f64(bad)


@pytest.mark.parametrize("kv", KVS)
def test_matches_library_sdpa(kv):
    assert pin_sdpa(attend_oracle, kv=kv)


@pytest.mark.parametrize("kv", KVS)
def test_page_permutation_invariance_bitwise(kv):
    assert pin_permutation(attend_oracle, kv=kv)


@pytest.mark.parametrize("kv", KVS)
def test_lse_consistency_law(kv):
    assert pin_lse_law(attend_oracle, kv=kv)


def test_merge_identity():
    assert pin_merge_identity(pa.range_state, pa.merge_states)


def test_golden_closed_forms():
    assert pin_golden(attend_oracle)


@pytest.mark.parametrize("kv", KVS)
def test_closed_forms_random(kv):
    assert pin_closed_forms(attend_oracle, kv=kv)


def test_f32_cache_of_bf16_values_equals_bf16_cache():
    # an fp32 cache holding exactly the bf16 values gives bit-identical results
    rng = np.random.default_rng(6)
    q, k, v, bt, lens = random_case(rng, [33, 70, 0, 5], 8, 2, 32, 16)
    o1, l1 = pa.decode_attention(q, k, v, bt, lens, 0.2, 16)
    kf = (k.astype(np.uint32) << np.uint32(16)).view(np.float32)
    vf = (v.astype(np.uint32) << np.uint32(16)).view(np.float32)
    o2, l2 = pa.decode_attention(q, kf, vf, bt, lens, 0.2, 16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_merge_all_neutral_and_empty():
    o, l = pa.merge_states(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.array_equal(o, np.zeros((2, 4))) and np.all(np.isneginf(l))
    o, l = pa.merge_states(np.zeros((0, 2, 4)), np.zeros((0, 2)))
    assert np.array_equal(o, np.zeros((2, 4))) and np.all(np.isneginf(l))


def test_bad_block_table_raises():
    rng = np.random.default_rng(5)
    q, k, v, bt, lens = random_case(rng, [9], 2, 1, 8, 4)
    bt = bt.copy()
    bt[0, 1] = k.shape[0]
    with pytest.raises(ValueError):
        pa.decode_attention(q, k, v, bt, lens, 0.5, 4)


# --------------------------------------------------- planted mistakes ----

def _mutant(monkeypatch, kind):
    """Plant one bug in the oracle module (CPU only)."""
    orig_gather = pa.gather_tokens
    orig_range = pa.range_state
    if kind == "drop_last_token":
        monkeypatch.setattr(pa, "gather_tokens", lambda pool, bt, s, h, lo, hi, P:
                            orig_gather(pool, bt, s, h, lo, max(lo, hi - 1), P))
    elif kind == "ignore_block_table":
        def g(pool, bt, s, h, lo, hi, P):
            t = np.arange(lo, hi)
            return pool[(t // P) % pool.shape[0], h, t % P, :]
        monkeypatch.setattr(pa, "gather_tokens", g)
    elif kind == "row_offset_swapped":
        def g(pool, bt, s, h, lo, hi, P):
            t = np.arange(lo, hi)
            return pool[np.asarray(bt[s])[t // P], h, (P - 1 - t % P), :]
        monkeypatch.setattr(pa, "gather_tokens", g)
    elif kind == "k_v_swapped":
        monkeypatch.setattr(pa, "range_state", lambda q, k, v, *a: orig_range(q, v, k, *a))
    elif kind == "no_scale":
        monkeypatch.setattr(pa, "range_state", lambda q, k, v, bt, s, h, lo, hi, sc, P:
                            orig_range(q, k, v, bt, s, h, lo, hi, 1.0, P))
    elif kind == "head_map_modulo":
        def r(q, k, v, bt, s, h_kv, lo, hi, sc, P):
            hq, hkv = q.shape[1], k.shape[1]
            g = hq // hkv
            idx = np.array([h for h in range(hq) if h % hkv == h_kv])   # strided groups
            q2 = q.copy()
            q2[s, h_kv * g:(h_kv + 1) * g] = q[s, idx]
            return orig_range(q2, k, v, bt, s, h_kv, lo, hi, sc, P)
        monkeypatch.setattr(pa, "range_state", r)
    elif kind == "f32_cache_rounded_to_bf16":
        orig_widen = pa.kv_to_f64

        def w(x):
            x = np.asarray(x)
            if x.dtype == np.float32:      # reads the cache as if it were bf16
                u = x.view(np.uint32).astype(np.uint64)
                x = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
            return orig_widen(x)
        monkeypatch.setattr(pa, "kv_to_f64", w)
    elif kind == "f32_cache_truncated":
        orig_widen = pa.kv_to_f64

        def w(x):
            x = np.asarray(x)
            if x.dtype == np.float32:      # drops the low 16 mantissa bits
                x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
            return orig_widen(x)
        monkeypatch.setattr(pa, "kv_to_f64", w)
    elif kind == "lse_log2":
        def r(*a):
            o, l = orig_range(*a)
            return o, l / math.log(2.0)
        monkeypatch.setattr(pa, "range_state", r)
    elif kind == "lse_missing_max":
        def r(q, k, v, bt, s, h_kv, lo, hi, sc, P):
            o, l = orig_range(q, k, v, bt, s, h_kv, lo, hi, sc, P)
            if hi <= lo:
                return o, l
            kk = pa.kv_to_f64(orig_gather(k, bt, s, h_kv, lo, hi, P))
            g = q.shape[1] // k.shape[1]
            m = (sc * (pa.bf16_bits_to_f64(q[s, h_kv * g:(h_kv + 1) * g]) @ kk.T)).max(axis=1)
            return o, l - m
        monkeypatch.setattr(pa, "range_state", r)
    else:
        raise AssertionError(kind)


@pytest.mark.parametrize("kind", ["drop_last_token", "ignore_block_table", "row_offset_swapped",
                                  "k_v_swapped", "no_scale", "head_map_modulo", "lse_log2",
                                  "lse_missing_max", "f32_cache_rounded_to_bf16",
                                  "f32_cache_truncated"])
def test_planted_attention_mistakes_are_caught(monkeypatch, kind):
    _mutant(monkeypatch, kind)
    with np.errstate(all="ignore"):
        res = all_attention_pins(attend_oracle)
    assert not all(res.values()), f"mutant {kind} passed every pin: {res}"


@pytest.mark.parametrize("kind", ["weights_not_exponentiated", "drop_max_shift_lse",
                                  "neutral_counts", "unweighted_mean"])
def test_planted_merge_mistakes_are_caught(kind):
    def merge(o_parts, lse_parts):
        if kind == "weights_not_exponentiated":
            w = np.where(np.isfinite(lse_parts), lse_parts, 0.0)
            return (w[:, :, None] * o_parts).sum(0) / w.sum(0)[:, None], pa.merge_states(o_parts, lse_parts)[1]
        if kind == "drop_max_shift_lse":
            o, l = pa.merge_states(o_parts, lse_parts)
            return o, l - np.max(np.where(np.isfinite(lse_parts), lse_parts, -1e300), axis=0)
        if kind == "neutral_counts":
            w = np.where(np.isfinite(lse_parts), np.exp(lse_parts), 1.0)
            return (w[:, :, None] * o_parts).sum(0) / w.sum(0)[:, None], np.log(w.sum(0))
        if kind == "unweighted_mean":
            return o_parts.mean(0), pa.merge_states(o_parts, lse_parts)[1]
        raise AssertionError(kind)
    with np.errstate(all="ignore"):
        assert not pin_merge_identity(pa.range_state, merge)

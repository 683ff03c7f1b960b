"""Float64 definition of decode attention over a block-table paged KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

What is computed follows the PersistentKV page ("PersistentKV: Page-Aware
Decode Scheduling for Long-Context LLM Serving on Commodity GPUs", Technical
Summary, Methodology section 1 "Native Block-Table Decode Engine"):

* GQA: G = Hq / Hkv query heads share one KV head.  Query head h reads KV
  head floor(h / G) (contiguous groups; the page gives only G, this is the
  reading taken).
* Layout: attention runs directly over the paged cache through the block
  table, with no repacking into contiguous K/V.  Pool layout (the page is
  silent; reading taken): K and V pools are separate arrays shaped
  [num_pages][Hkv][page_size][D]; ``block_table[b][j]`` is the
  physical page holding logical tokens j*page_size .. j*page_size+page_size-1
  of sequence b.
* Row-local bounds: only the true length L_b of each row is read; tokens at or
  beyond L_b are never read or weighted.
* Sequence splitting: a disjoint token range yields a partial state
  (o = normalised output, lse = log-sum-exp of the scaled scores); a separate
  merge combines such states exactly.  An empty range yields the neutral state
  (o = 0, lse = -inf), which the merge gives weight zero.

Inputs are numpy arrays of bf16 bit patterns (uint16).  The K/V pools may
instead hold float32 values: the fp32 attention cache that the Wave
Persistent Kernel note lists for its text-to-speech model ("Same precision"
list); the query stays bf16 bits.  Every value is widened exactly to float64
and all arithmetic below is float64.  Output LSE is the natural logarithm.

Because the split-and-merge scheme reaches the plain result exactly (up to
rounding order), the oracle is that plain definition written out: one softmax
over all valid tokens of a row.  ``range_state`` and ``merge_states`` exist so
that tests can pin the merge identity and check the kernel's own partials.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64.

    A bf16 value is the upper half of an IEEE binary32 word, so shifting the
    16 bits into the top of a 32-bit word gives the float32 of equal value,
    which float64 represents exactly.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def kv_to_f64(values: np.ndarray) -> np.ndarray:
    """Widen cache values exactly to float64: uint16 arrays are bf16 bit
    patterns, float32 arrays are fp32 values (float64 holds both exactly)."""
    values = np.asarray(values)
    if values.dtype == np.uint16:
        return bf16_bits_to_f64(values)
    if values.dtype == np.float32:
        return values.astype(np.float64)
    raise TypeError(f"cache values must be uint16 (bf16 bits) or float32, not {values.dtype}")


def gather_tokens(pool: np.ndarray, block_table: np.ndarray, seq: int, kv_head: int,
                  tok_begin: int, tok_end: int, page_size: int) -> np.ndarray:
    """Raw cache values of tokens [tok_begin, tok_end) of one (sequence, KV
    head).

    Token t lives in physical page ``block_table[seq][t // page_size]`` at row
    ``t % page_size`` (PersistentKV page, Methodology 1, "Layout").  Returns
    an array [tok_end - tok_begin][D] of the pool's dtype in token order.
    """
    if tok_end <= tok_begin:
        return np.zeros((0, pool.shape[-1]), dtype=pool.dtype)
    t = np.arange(tok_begin, tok_end, dtype=np.int64)
    phys = np.asarray(block_table[seq], dtype=np.int64)[t // page_size]
    if phys.min() < 0 or phys.max() >= pool.shape[0]:
        raise ValueError("block table entry outside the page pool")
    return pool[phys, kv_head, t % page_size, :]


def range_state(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                block_table: np.ndarray, seq: int, kv_head: int,
                tok_begin: int, tok_end: int, scale: float, page_size: int):
    """Partial attention state of the G query heads of ``kv_head`` over one
    token range (PersistentKV page, Methodology 1, "Sequence Splitting").

    Returns (o [G][D] float64, lse [G] float64) with
        s_t  = scale * (q_h . k_t)
        lse  = log(sum_t exp(s_t))
        o    = sum_t exp(s_t - lse) v_t
    and the neutral state (zeros, -inf) for an empty range ("Row-Local
    Bounds": empty splits write neutral states).
    """
    hq = q.shape[1]
    hkv = k_pool.shape[1]
    g = hq // hkv
    d = q.shape[2]
    if tok_end <= tok_begin:
        return np.zeros((g, d)), np.full(g, -np.inf)
    kk = kv_to_f64(gather_tokens(k_pool, block_table, seq, kv_head,
                                 tok_begin, tok_end, page_size))
    vv = kv_to_f64(gather_tokens(v_pool, block_table, seq, kv_head,
                                 tok_begin, tok_end, page_size))
    qg = bf16_bits_to_f64(q[seq, kv_head * g:(kv_head + 1) * g, :])   # [G][D]
    s = float(scale) * (qg @ kk.T)                                      # [G][n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ vv) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def merge_states(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Exact combination of partial states over disjoint ranges
    (PersistentKV page, Methodology 1: the merge "combines these states
    exactly").

    o_parts [S][G][D], lse_parts [S][G].  With M = max_i lse_i and
    w_i = exp(lse_i - M):  O = sum_i w_i o_i / sum_i w_i,
    LSE = M + log(sum_i w_i).  Neutral parts (lse = -inf) get weight 0; if
    every part is neutral (or S = 0) the result is the neutral state.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    g, d = o_parts.shape[1], o_parts.shape[2]
    out = np.zeros((g, d))
    lse = np.full(g, -np.inf)
    for h in range(g):
        ls = lse_parts[:, h] if lse_parts.shape[0] else np.zeros(0)
        if ls.size == 0 or not np.isfinite(ls).any():
            continue
        mx = ls[np.isfinite(ls)].max()
        w = np.where(np.isfinite(ls), np.exp(ls - mx), 0.0)
        out[h] = (w[:, None] * o_parts[:, h, :]).sum(axis=0) / w.sum()
        lse[h] = mx + np.log(w.sum())
    return out, lse


def decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_table: np.ndarray, ctx_lens: np.ndarray, scale: float,
                     page_size: int, units=None):
    """softmax(q K^T * scale) V and its LSE for every (sequence, query head).

    q [B][Hq][D] bf16 bits, pools [num_pages][Hkv][page_size][D] bf16 bits
    or float32 values;
    block_table int [B][max_pages]; ctx_lens int [B].  A row with L_b = 0 gets
    O = 0 and LSE = -inf (the neutral state).  ``units`` optionally restricts
    the work to a list of (seq, kv_head) pairs; rows outside it stay neutral.

    Returns (O [B][Hq][D] float64, LSE [B][Hq] float64).
    """
    bsz, hq, d = q.shape
    hkv = k_pool.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    g = hq // hkv
    out = np.zeros((bsz, hq, d))
    lse = np.full((bsz, hq), -np.inf)
    if units is None:
        units = [(b, h) for b in range(bsz) for h in range(hkv)]
    for b, h_kv in units:
        o, l = range_state(q, k_pool, v_pool, block_table, b, h_kv,
                           0, int(ctx_lens[b]), scale, page_size)
        out[b, h_kv * g:(h_kv + 1) * g] = o
        lse[b, h_kv * g:(h_kv + 1) * g] = l
    return out, lse

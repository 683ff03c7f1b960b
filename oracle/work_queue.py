"""Adaptive split policy and compact work queue, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.  The host builder (C++) and the device builder (HIP) in the
library must produce these exact bytes.

Sources (PersistentKV page, "PersistentKV: Page-Aware Decode Scheduling for
Long-Context LLM Serving on Commodity GPUs", Technical Summary):

* Methodology 1 "Row-Local Bounds": split ranges follow each row's true
  length; nothing is padded.
* Methodology 1 "Compact Workqueue": a 1-D list of tasks only for non-empty
  (row, KV head, split) intervals.
* Methodology 2 "Calibrated Adaptive Policy": split the sequence when the
  batch is too small to fill the GPU with one task per (row, KV head); use the
  compact queue for larger batches.  The page's third route (a third-party
  kernel) does not exist here, so it becomes the no-split route.

Readings taken where the page is silent:

* Split rule (AUTO): split into ``chunk_tokens``-token ranges iff
  B * Hkv < num_cus and some L_b > chunk_tokens; otherwise one item per
  (row, KV head).  ``chunk_tokens`` is a multiple of the page size.
* Range length (the page says only that ranges are disjoint): either a
  fixed ``chunk_tokens``, or, with ``chunk_tokens = 0`` ("fit"), the
  shortest whole number of pages T for which the split queue still has at
  most one range per workgroup: sum_b ceil(pages_b / T) <= K with
  K = max(1, num_cus // Hkv) and pages_b = ceil(L_b / P).  This extends the
  page's own count for one sequence (as many ranges as it takes to fill the
  GPU) to a batch, keeping the longest range as short as one round allows.
  If no T reaches the bound (more non-empty rows than K), T is the longest
  row's page count.  T is never below a floor: 16 pages (256 tokens) for
  one-shot calls, 64 pages (1024 tokens) for the resident loop, whose
  workspace sizes its per-layer partial states by this floor.  The floor is
  a measured tuning, not the page's: the shortest ranges that keep one
  range per workgroup are the fastest down to 16 pages.
* Ranges are fixed chunks from token 0: chunk c covers
  [c * C, min(L_b, (c + 1) * C)).
* Item encoding, 16 bytes little-endian:
  u32 seq, u16 kv_head, u16 chunk, u32 tok_begin, u32 tok_end.  A row that
  would need more than 65535 ranges cannot be encoded and is an error.
* n_chunks[b] = 0 for an empty row, ceil(L_b / C) for a split row, else 1.
* part_off[b] is the exclusive prefix sum over rows of n_chunks[b] counted
  only where n_chunks[b] > 1 (rows that need a merge own partial slots);
  partial slot of an item = (part_off[seq] + chunk) * Hkv + kv_head.
* merge_rows lists, ascending, the rows with n_chunks != 1 (split rows are
  merged; empty rows receive the neutral state).
* Order: canonical (seq, kv_head, chunk) ascending.  Order LPT (a named
  option) is a stable sort of the canonical list by item length, longest
  first, so ties keep canonical order.
"""

from __future__ import annotations

import numpy as np

POLICY_AUTO = 0
POLICY_NO_SPLIT = 1
POLICY_SPLIT = 2

ORDER_CANONICAL = 0
ORDER_LPT = 1

ITEM_DTYPE = np.dtype([("seq", "<u4"), ("kv_head", "<u2"), ("chunk", "<u2"),
                       ("tok_begin", "<u4"), ("tok_end", "<u4")])
assert ITEM_DTYPE.itemsize == 16


FIT_MIN_PAGES = 16           # one-shot calls
FIT_MIN_PAGES_LOOP = 64      # the resident loop


def fit_chunk(ctx_lens, num_kv_heads: int, num_cus: int, page_size: int = 16,
              min_pages: int = FIT_MIN_PAGES) -> int:
    """Range length in tokens for chunk mode "fit" (reading in the header):
    the smallest T pages with sum_b ceil(pages_b / T) <= max(1, num_cus // Hkv),
    found by trying T = 1, 2, ... in turn, and then at least ``min_pages``."""
    pages = [-(-int(L) // page_size) for L in ctx_lens]
    longest = max(pages, default=0)
    budget = max(1, num_cus // num_kv_heads)
    T = max(longest, 1)
    for t in range(1, longest + 1):
        if sum(-(-n // t) for n in pages) <= budget:
            T = t
            break
    return max(T, min_pages) * page_size


def decide_split(ctx_lens, num_kv_heads: int, num_cus: int, chunk_tokens: int,
                 policy: int = POLICY_AUTO) -> bool:
    """The adaptive split decision (PersistentKV page, Methodology 2)."""
    lens = [int(x) for x in ctx_lens]
    if policy == POLICY_NO_SPLIT:
        return False
    if policy == POLICY_SPLIT:
        return True
    if policy != POLICY_AUTO:
        raise ValueError("unknown policy")
    if not lens:
        return False
    return len(lens) * num_kv_heads < num_cus and max(lens) > chunk_tokens


def build_queue(ctx_lens, num_kv_heads: int, num_cus: int, chunk_tokens: int,
                policy: int = POLICY_AUTO, order: int = ORDER_CANONICAL,
                fit_min_pages: int = FIT_MIN_PAGES):
    """Compact work queue for one decode call.

    ``chunk_tokens = 0`` selects chunk mode "fit" (see ``fit_chunk``), with
    ranges of at least ``fit_min_pages`` pages (``FIT_MIN_PAGES_LOOP`` for
    the resident loop's steps).

    Returns a dict with
      split      bool, the policy decision
      chunk_tokens  the range length used
      items      ITEM_DTYPE array, one entry per non-empty interval
      n_chunks   int32 [B]
      part_off   int32 [B + 1]
      merge_rows int32 list of rows needing the merge/finalize pass
      row_len    int32 [B], each row's length in tokens (the input, carried
                 with the queue so a schedule that shares a row's pages
                 among its items knows where the row ends)
    """
    lens = [int(x) for x in ctx_lens]
    for L in lens:
        if L < 0:
            raise ValueError("negative context length")
    if chunk_tokens == 0:                                 # chunk mode "fit"
        chunk_tokens = fit_chunk(lens, num_kv_heads, num_cus, min_pages=fit_min_pages)
    split = decide_split(lens, num_kv_heads, num_cus, chunk_tokens, policy)
    bsz = len(lens)

    n_chunks = np.zeros(bsz, dtype=np.int32)
    for b, L in enumerate(lens):
        if L == 0:
            n_chunks[b] = 0
        elif split:
            n_chunks[b] = -(-L // chunk_tokens)          # ceil(L / C)
        else:
            n_chunks[b] = 1
        if n_chunks[b] > 65535:                          # the item's range index is 16 bits
            raise ValueError(f"row {b} needs {n_chunks[b]} ranges; an item encodes at most 65535")

    part_off = np.zeros(bsz + 1, dtype=np.int32)
    for b in range(bsz):
        owns = n_chunks[b] if n_chunks[b] > 1 else 0
        part_off[b + 1] = part_off[b] + owns

    rows = []
    for b, L in enumerate(lens):
        for h in range(num_kv_heads):
            for c in range(int(n_chunks[b])):
                if split:
                    lo = c * chunk_tokens
                    hi = min(L, (c + 1) * chunk_tokens)
                else:
                    lo, hi = 0, L
                if hi > lo:                               # non-empty only
                    rows.append((b, h, c, lo, hi))

    if order == ORDER_LPT:
        rows = sorted(rows, key=lambda r: -(r[4] - r[3]))  # stable sort
    elif order != ORDER_CANONICAL:
        raise ValueError("unknown order")

    items = np.zeros(len(rows), dtype=ITEM_DTYPE)
    for i, (b, h, c, lo, hi) in enumerate(rows):
        items[i] = (b, h, c, lo, hi)

    merge_rows = np.array([b for b in range(bsz) if n_chunks[b] != 1], dtype=np.int32)
    return {"split": split, "items": items, "n_chunks": n_chunks,
            "part_off": part_off, "merge_rows": merge_rows, "chunk_tokens": chunk_tokens,
            "row_len": np.asarray(lens, dtype=np.int32).reshape(-1)}


def partial_slot(item, part_off, num_kv_heads: int) -> int:
    """Slot of a split item's partial state (reading stated in the header)."""
    return (int(part_off[int(item["seq"])]) + int(item["chunk"])) * num_kv_heads \
        + int(item["kv_head"])

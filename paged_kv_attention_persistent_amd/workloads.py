"""Seeded synthetic inputs for paged decode attention.

This module only makes inputs: query vectors, K/V page pools, block tables
and context lengths.  It holds none of the attention arithmetic, and it is
the one module that both the HIP path's callers and the float64 oracle's
callers use, so that both see the same bits.

Values.  Every bf16 value is drawn by a counter-based generator, so any
element can be regenerated on its own on any device:

    a = mix32((i mod 2^32) xor k1),  b = mix32(a xor (i div 2^32) xor k2)
    value_i = NORMAL_TABLE[b >> 16]

``mix32`` is the "lowbias32" integer finaliser published by Chris Wellons
(hash-prospector): x ^= x>>16; x *= 0x7feb352d; x ^= x>>15; x *= 0x846ca68b;
x ^= x>>16, all modulo 2^32.  ``NORMAL_TABLE[j]`` is the bf16 rounding
(round-to-nearest-even) of the standard normal quantile at (j + 0.5) / 65536,
so each element is an N(0, 1) draw quantised to 65536 levels (tails cut at
about 4.3 sigma).  (k1, k2) come from the seed and the tensor's name.  The
arithmetic is integer-only, so CPU and GPU produce identical bits.

An fp32 KV cache (``kv_dtype="f32"``) draws from the same counters through
``NORMAL_TABLE_F32[j]``, the float32 of the same quantile: full 24-bit
mantissas, and the bf16 cache of the same workload is exactly its rounding.

Parity runs poison what must never be read: pool pages no block table points
to, and the slots of a sequence's last page at or beyond its length, hold the
quiet-NaN pattern (0x7FC0 in bf16, 0x7FC00000 in fp32).  Block-table entries past a sequence's last
page are -1.

Workload shapes are those of the decode-attention traces on the PersistentKV
page ("PersistentKV: Page-Aware Decode Scheduling ...", Evaluation Protocol:
single long context, mixed lengths, many short rows) and of the
many-session resident loop on the Wave Persistent Kernel note.  The pages do
not give their trace generators; these recipes stand in for them.
Measurement seed 20260623, calibration seed 20260622 (the PersistentKV page's
held-out and calibration seeds, Results section).
"""

from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field, replace

import numpy as np
import torch

MEASURE_SEED = 20260623
CALIBRATION_SEED = 20260622
BF16_NAN = 0x7FC0
F32_NAN = 0x7FC00000
KV_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}
_M32 = 0xFFFFFFFF


def _mix32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 on int64 tensors holding values in [0, 2^32)."""
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & _M32          # may wrap in int64; low 32 bits exact
    x = x ^ (x >> 16)
    return x


_TABLE_CACHE: dict = {}


def _quantiles_f32() -> np.ndarray:
    from scipy.special import ndtri
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(p).astype(np.float32)


def normal_table(device) -> torch.Tensor:
    """int64 tensor [65536] of bf16 bit patterns of N(0,1) quantiles."""
    key = str(device)
    if key not in _TABLE_CACHE:
        u = _quantiles_f32().view(np.uint32).astype(np.uint64)
        rne = (u + 0x7FFF + ((u >> 16) & 1)) >> 16          # float32 -> bf16 RNE
        _TABLE_CACHE[key] = torch.from_numpy(rne.astype(np.int64)).to(device)
    return _TABLE_CACHE[key]


def normal_table_f32(device) -> torch.Tensor:
    """int64 tensor [65536] of float32 bit patterns of the same quantiles."""
    key = "f32/" + str(device)
    if key not in _TABLE_CACHE:
        u = _quantiles_f32().view(np.uint32).astype(np.int64)
        _TABLE_CACHE[key] = torch.from_numpy(u).to(device)
    return _TABLE_CACHE[key]


def stream_keys(seed: int, name: str):
    """Two 32-bit keys for tensor ``name`` under ``seed``."""
    n = zlib.crc32(name.encode())
    k1 = _mix32_int(_mix32_int(seed & _M32) ^ n)
    k2 = _mix32_int(k1 ^ 0x9E3779B9)
    return k1, k2


def _table_index(seed: int, name: str, index: torch.Tensor) -> torch.Tensor:
    k1, k2 = stream_keys(seed, name)
    a = _mix32((index & _M32) ^ k1)
    b = _mix32(a ^ (index >> 32) ^ k2)
    return b >> 16


def normal_bf16_bits(seed: int, name: str, index: torch.Tensor) -> torch.Tensor:
    """bf16 bit patterns (int64 tensor, values 0..65535) for element ``index``."""
    return normal_table(index.device)[_table_index(seed, name, index)]


def normal_f32_bits(seed: int, name: str, index: torch.Tensor) -> torch.Tensor:
    """float32 bit patterns (int64 tensor, values 0..2^32-1) for element
    ``index``: the values whose bf16 rounding ``normal_bf16_bits`` gives."""
    return normal_table_f32(index.device)[_table_index(seed, name, index)]


def _to_bf16(bits: torch.Tensor) -> torch.Tensor:
    """int64 tensor of 16-bit patterns -> torch.bfloat16 with those bits."""
    return (bits - ((bits >> 15) & 1) * 65536).to(torch.int16).view(torch.bfloat16)


def _to_f32(bits: torch.Tensor) -> torch.Tensor:
    """int64 tensor of 32-bit patterns -> torch.float32 with those bits."""
    return (bits - ((bits >> 31) & 1) * (1 << 32)).to(torch.int32).view(torch.float32)


def normal_values(seed: int, name: str, index: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    """Elements ``index`` of stream ``name`` as bf16 or float32 values."""
    if dtype == torch.float32:
        return _to_f32(normal_f32_bits(seed, name, index))
    return _to_bf16(normal_bf16_bits(seed, name, index))


def fill_normal(out: torch.Tensor, seed: int, name: str, offset: int = 0,
                chunk: int = 1 << 24) -> torch.Tensor:
    """Fill a contiguous bf16 or float32 tensor with the stream ``name``
    starting at element ``offset`` (chunked to bound the int64 temporaries)."""
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(offset + s, offset + e, dtype=torch.int64, device=out.device)
        flat[s:e] = normal_values(seed, name, idx, out.dtype)
    return out


def fill_normal_bf16(out: torch.Tensor, seed: int, name: str, offset: int = 0,
                     chunk: int = 1 << 24) -> torch.Tensor:
    """Fill a contiguous bf16 tensor with the stream ``name``."""
    assert out.dtype == torch.bfloat16
    return fill_normal(out, seed, name, offset, chunk)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """Host numpy uint16 view of a bf16 tensor's bits (copies to CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def kv_host(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy of a KV tensor in the form the oracle reads: uint16 bf16
    bit patterns for a bf16 cache, float32 values for an fp32 cache."""
    if t.dtype == torch.float32:
        return t.detach().cpu().contiguous().numpy()
    return bits_u16(t)


@dataclass
class Workload:
    """One decode-attention call's shapes plus the recipe of its inputs."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    ctx_lens: np.ndarray              # int32 [B]
    block_table: np.ndarray           # int32 [B][max_pages_per_seq], -1 = unused
    num_pages: int
    seed: int
    scale: float = 0.0
    extra: dict = field(default_factory=dict)
    kv_dtype: str = "bf16"            # element type of the K/V pools: "bf16" or "f32"

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.head_dim)
        if self.kv_dtype not in KV_DTYPES:
            raise ValueError(f"kv_dtype must be one of {sorted(KV_DTYPES)}")

    @property
    def kv_torch_dtype(self):
        return KV_DTYPES[self.kv_dtype]

    @property
    def kv_elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2

    def with_kv_dtype(self, kv_dtype: str) -> "Workload":
        """The same workload (same streams, same tables) with another cache type."""
        return replace(self, kv_dtype=kv_dtype)

    @property
    def batch(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V of valid tokens: the algorithmic read volume."""
        return int(self.ctx_lens.astype(np.int64).sum()) * self.num_kv_heads \
            * self.head_dim * self.kv_elem_bytes * 2

    def q(self, device="cpu") -> torch.Tensor:
        t = torch.empty(self.batch, self.num_q_heads, self.head_dim,
                        dtype=torch.bfloat16, device=device)
        return fill_normal_bf16(t, self.seed, self.name + "/q")

    def pool(self, which: str, device="cpu", poison: bool = True) -> torch.Tensor:
        """K ('k') or V ('v') pool [num_pages][Hkv][P][D] of kv_dtype."""
        t = torch.empty(self.num_pages, self.num_kv_heads, self.page_size,
                        self.head_dim, dtype=self.kv_torch_dtype, device=device)
        fill_normal(t, self.seed, self.name + "/" + which)
        if poison:
            self.poison(t)
        return t

    def pool_pages(self, which: str, pages: np.ndarray) -> torch.Tensor:
        """Regenerate only the given pool pages on the CPU (unpoisoned values),
        shaped [len(pages)][Hkv][P][D]: the same bits ``pool`` holds there."""
        per_page = self.num_kv_heads * self.page_size * self.head_dim
        pages = torch.as_tensor(np.asarray(pages, dtype=np.int64))
        idx = pages[:, None] * per_page + torch.arange(per_page, dtype=torch.int64)[None, :]
        vals = normal_values(self.seed, self.name + "/" + which, idx.reshape(-1), self.kv_torch_dtype)
        return vals.view(len(pages), self.num_kv_heads, self.page_size, self.head_dim)

    def pool_slabs(self, which: str, pages, kv_head: int) -> torch.Tensor:
        """Regenerate on the CPU only the (page, kv_head) slabs of the given
        pages, shaped [len(pages)][P][D] (unpoisoned values)."""
        slab = self.page_size * self.head_dim
        per_page = self.num_kv_heads * slab
        pages = torch.as_tensor(np.asarray(pages, dtype=np.int64))
        idx = (pages[:, None] * per_page + kv_head * slab
               + torch.arange(slab, dtype=torch.int64)[None, :])
        vals = normal_values(self.seed, self.name + "/" + which, idx.reshape(-1), self.kv_torch_dtype)
        return vals.view(len(pages), self.page_size, self.head_dim)

    def poison(self, pool: torch.Tensor) -> None:
        """Write NaN into unreferenced pages and past-the-end slots."""
        used = np.zeros(self.num_pages, dtype=bool)
        P = self.page_size
        if pool.dtype == torch.float32:
            nan = torch.tensor(F32_NAN, dtype=torch.int32).view(torch.float32)
        else:
            nan = torch.tensor(BF16_NAN, dtype=torch.int16).view(torch.bfloat16)
        for b in range(self.batch):
            L = int(self.ctx_lens[b])
            npg = -(-L // P)
            used[self.block_table[b, :npg]] = True
            if L % P:
                last = int(self.block_table[b, npg - 1])
                pool[last, :, L % P:, :] = nan.to(pool.device)
        unused = np.nonzero(~used)[0]
        if unused.size:
            pool[torch.as_tensor(unused, device=pool.device)] = nan.to(pool.device)

    def block_table_t(self, device="cpu") -> torch.Tensor:
        return torch.as_tensor(self.block_table, dtype=torch.int32).to(device)

    def ctx_lens_t(self, device="cpu") -> torch.Tensor:
        return torch.as_tensor(self.ctx_lens, dtype=torch.int32).to(device)


def _tables(rng: np.random.Generator, lens, page_size: int, num_pages: int,
            max_pages: int | None = None):
    """Block tables that scatter every sequence over a random permutation of
    the pool (each physical page is used at most once)."""
    need = [-(-int(L) // page_size) for L in lens]
    if max_pages is None:
        max_pages = max(need) if need else 0
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((len(lens), max(max_pages, 1)), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


def tiny(seed: int = MEASURE_SEED) -> Workload:
    """Batch 1, 4 query heads / 1 KV head, head_dim 64, 256 tokens in 16 pages
    scattered over a 64-page pool."""
    rng = np.random.default_rng([seed, 1])
    lens = np.array([256], dtype=np.int32)
    return Workload("tiny", 4, 1, 64, 16, lens, _tables(rng, lens, 16, 64), 64, seed)


def long_context(seed: int = MEASURE_SEED, ctx: int = 131072) -> Workload:
    """Batch 1, 32/8 heads, head_dim 128, 131072 tokens over a permuted pool."""
    rng = np.random.default_rng([seed, 2])
    lens = np.array([ctx], dtype=np.int32)
    npg = -(-ctx // 16)
    return Workload("long", 32, 8, 128, 16, lens, _tables(rng, lens, 16, npg), npg, seed)


def long_tp8(seed: int = MEASURE_SEED, ctx: int = 131072) -> Workload:
    """One GPU's share of the long context when its 32/8 heads are split over
    8 GPUs by head: batch 1, 4 query heads / 1 KV head, head_dim 128."""
    rng = np.random.default_rng([seed, 5])
    lens = np.array([ctx], dtype=np.int32)
    npg = -(-ctx // 16)
    return Workload("long_tp8", 4, 1, 128, 16, lens, _tables(rng, lens, 16, npg), npg, seed)


def mixed(seed: int = MEASURE_SEED, batch: int = 8, lo: int = 1024, hi: int = 65536) -> Workload:
    """8 sequences, lengths log-uniform in [1024, 65536] (rounded), 32/8 heads."""
    rng = np.random.default_rng([seed, 3])
    lens = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch)))
    lens = np.clip(lens, lo, hi).astype(np.int32)
    npg = int(sum(-(-int(L) // 16) for L in lens))
    return Workload("mixed", 32, 8, 128, 16, lens, _tables(rng, lens, 16, npg), npg, seed)


def many_short(seed: int = MEASURE_SEED, batch: int = 64, ctx: int = 4096) -> Workload:
    """64 sequences of 4096 tokens, 32/8 heads."""
    rng = np.random.default_rng([seed, 4])
    lens = np.full(batch, ctx, dtype=np.int32)
    npg = batch * (-(-ctx // 16))
    return Workload("short", 32, 8, 128, 16, lens, _tables(rng, lens, 16, npg), npg, seed)


def custom(name: str, lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
           seed: int = MEASURE_SEED, spare_pages: int = 0, page_size: int = 16,
           max_pages: int | None = None, kv_dtype: str = "bf16") -> Workload:
    """Any shape: lengths given, pool = the pages needed plus ``spare_pages``
    (spare pages are poisoned)."""
    rng = np.random.default_rng([seed, zlib.crc32(name.encode())])
    lens = np.asarray(lens, dtype=np.int32)
    npg = int(sum(-(-int(L) // page_size) for L in lens)) + spare_pages
    npg = max(npg, 1)
    return Workload(name, num_q_heads, num_kv_heads, head_dim, page_size, lens,
                    _tables(rng, lens, page_size, npg, max_pages), npg, seed, kv_dtype=kv_dtype)


CONFIGS = {"tiny": tiny, "long": long_context, "mixed": mixed, "short": many_short, "long_tp8": long_tp8}


@dataclass
class SessionLoop:
    """Many concurrent real-time sessions, each a stack of decode-attention
    layers, stepped in lockstep by a resident kernel (the Wave Persistent
    Kernel note's session cohort).  Session s starts with context L0_s drawn
    uniformly from [lo, hi] and grows by one token per step: at step t its
    context is L0_s + t.  Pages for L0_s + steps tokens are allocated up front
    in every layer; each layer has its own randomly permuted pool.  K/V of the
    tokens a later step adds are generated with the rest (the append of new
    tokens is not part of the step).

    With append=True the cache starts with the L0_s - 1 tokens before step 0
    only (pages for them in every layer, every other row NaN) and step t
    appends token L0_s - 1 + t from new_kv(); a token that opens a page takes
    the next id of free_pages, in session order, the same id in every layer."""
    name: str
    sessions: int
    layers: int
    steps: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    l0: np.ndarray                    # int32 [sessions]
    block_tables: np.ndarray          # int32 [layers][sessions][max_pages]
    pages_per_layer: int
    seed: int
    page_size: int = 16
    scale: float = 0.0
    append: bool = False
    free_pages: np.ndarray = None     # append: page ids not in use before step 0
    kv_dtype: str = "bf16"            # element type of the cache (pools and new tokens)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.head_dim)
        if self.kv_dtype not in KV_DTYPES:
            raise ValueError(f"kv_dtype must be one of {sorted(KV_DTYPES)}")

    @property
    def kv_torch_dtype(self):
        return KV_DTYPES[self.kv_dtype]

    @property
    def kv_elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2

    def with_kv_dtype(self, kv_dtype: str) -> "SessionLoop":
        """The same loop (same streams, same tables) with another cache type."""
        return replace(self, kv_dtype=kv_dtype)

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[2])

    def ctx_lens(self, t: int) -> np.ndarray:
        return (self.l0 + t).astype(np.int32)

    def kv_bytes(self, t: int) -> int:
        return int(self.ctx_lens(t).astype(np.int64).sum()) * self.layers * self.num_kv_heads \
            * self.head_dim * self.kv_elem_bytes * 2

    def churn_lens(self, seed: int, life=(40, 120), join_lo: int = 2048, idle_prob: float = 0.0,
                   idle=(1, 2)):
        """Session churn over the slots (the Wave Persistent Kernel note's
        sessions joining and leaving at step boundaries): each slot hosts a
        sequence of sessions with lifetimes U[life] steps; when one leaves,
        the slot may stay empty (context 0) for U[idle] steps with probability
        idle_prob, then the next session joins with a fresh context drawn
        from [min(join_lo, L0_s), L0_s], so that it fits the pages the slot
        owns (L0_s + steps tokens).  The slot's first session is the loop's
        own (context L0_s + t).  Returns (lens int32 [steps][sessions], joins)."""
        rng = np.random.default_rng([seed, 9])
        lens = np.zeros((self.steps, self.sessions), dtype=np.int32)
        joins = 0
        for s in range(self.sessions):
            cap = int(self.l0[s])
            t, L0 = 0, cap
            while t < self.steps:
                n = int(rng.integers(life[0], life[1] + 1))
                for u in range(t, min(self.steps, t + n)):
                    lens[u, s] = L0 + (u - t)
                t += n
                if t < self.steps and idle_prob > 0 and rng.random() < idle_prob:
                    t += int(rng.integers(idle[0], idle[1] + 1))      # the slot stays empty
                if t < self.steps:
                    L0 = int(rng.integers(min(join_lo, cap), cap + 1))
                    joins += 1
        return lens, joins

    def pools(self, which: str, device) -> torch.Tensor:
        """[layers][pages][Hkv][P][D] of kv_dtype (one stream per tensor name).
        With append, rows that hold no token before step 0 are NaN."""
        t = torch.empty(self.layers, self.pages_per_layer, self.num_kv_heads, self.page_size,
                        self.head_dim, dtype=self.kv_torch_dtype, device=device)
        t = fill_normal(t, self.seed, self.name + "/" + which)
        if self.append:
            P = self.page_size
            valid = np.zeros((self.layers, self.pages_per_layer, P), dtype=bool)
            lay = np.arange(self.layers)[:, None]
            for s, L in enumerate(self.l0 - 1):
                n = -(-int(L) // P)
                if n == 0:
                    continue
                valid[lay, self.block_tables[:, s, :n - 1]] = True          # full pages
                valid[np.arange(self.layers), self.block_tables[:, s, n - 1], :int(L) - (n - 1) * P] = True
            bad = torch.as_tensor(~valid).to(device)[:, :, None, :, None].expand_as(t)
            if t.dtype == torch.float32:
                t.view(torch.int32)[bad] = F32_NAN
            else:
                t.view(torch.int16)[bad] = BF16_NAN
        return t

    def new_kv(self, which: str, device) -> torch.Tensor:
        """Append: K or V of each step's new token, [steps][layers][sessions][Hkv][D]
        of kv_dtype."""
        t = torch.empty(self.steps, self.layers, self.sessions, self.num_kv_heads, self.head_dim,
                        dtype=self.kv_torch_dtype, device=device)
        return fill_normal(t, self.seed, self.name + "/new_" + which)

    def new_kv_unit(self, which: str, t: int, layer: int, s: int, kv_head: int) -> torch.Tensor:
        """CPU regeneration of new_kv(which)[t][layer][s][kv_head] ([D])."""
        D = self.head_dim
        off = (((t * self.layers + layer) * self.sessions + s) * self.num_kv_heads + kv_head) * D
        idx = torch.arange(off, off + D, dtype=torch.int64)
        return normal_values(self.seed, self.name + "/new_" + which, idx, self.kv_torch_dtype)

    def token_rows(self, which: str, t: int, layer: int, s: int, kv_head: int) -> torch.Tensor:
        """The L_s(t) tokens of (layer, session, KV head) at step t in order, [L][D]
        of kv_dtype: the cache's tokens before step 0, then with append the
        tokens of steps 0..t."""
        L = int(self.ctx_lens(t)[s])
        P = self.page_size
        if not self.append:
            pages = self.block_tables[layer, s, :-(-L // P)]
            return self.slabs(which, layer, pages, kv_head).reshape(-1, self.head_dim)[:L]
        L0 = int(self.l0[s]) - 1
        rows = []
        if L0 > 0:
            pages = self.block_tables[layer, s, :-(-L0 // P)]
            rows.append(self.slabs(which, layer, pages, kv_head).reshape(-1, self.head_dim)[:L0])
        rows += [self.new_kv_unit(which, u, layer, s, kv_head)[None] for u in range(t + 1)]
        return torch.cat(rows)

    def appended_block_tables(self, steps: int) -> np.ndarray:
        """Append: block tables after `steps` steps (free pages taken in step,
        then session, order)."""
        bt = self.block_tables.copy()
        k = 0
        for t in range(steps):
            for s in range(self.sessions):
                j = int(self.l0[s]) - 1 + t
                if j % self.page_size == 0:
                    bt[:, s, j // self.page_size] = self.free_pages[k]
                    k += 1
        return bt

    def queries(self, device) -> torch.Tensor:
        """[steps][layers][sessions][Hq][D] bf16."""
        t = torch.empty(self.steps, self.layers, self.sessions, self.num_q_heads, self.head_dim,
                        dtype=torch.bfloat16, device=device)
        return fill_normal_bf16(t, self.seed, self.name + "/q")

    def query_unit(self, t: int, layer: int, s: int) -> torch.Tensor:
        """CPU regeneration of q[t][layer][s] ([Hq][D])."""
        per = self.num_q_heads * self.head_dim
        off = ((t * self.layers + layer) * self.sessions + s) * per
        idx = torch.arange(off, off + per, dtype=torch.int64)
        return _to_bf16(normal_bf16_bits(self.seed, self.name + "/q", idx)).view(
            self.num_q_heads, self.head_dim)

    def slabs(self, which: str, layer: int, pages, kv_head: int) -> torch.Tensor:
        """CPU regeneration of the (page, kv_head) slabs of one layer."""
        slab = self.page_size * self.head_dim
        per_page = self.num_kv_heads * slab
        base = layer * self.pages_per_layer * per_page
        pages = torch.as_tensor(np.asarray(pages, dtype=np.int64))
        idx = (base + pages[:, None] * per_page + kv_head * slab
               + torch.arange(slab, dtype=torch.int64)[None, :])
        vals = normal_values(self.seed, self.name + "/" + which, idx.reshape(-1), self.kv_torch_dtype)
        return vals.view(len(pages), self.page_size, self.head_dim)


def session_loop(seed: int = MEASURE_SEED, sessions: int = 56, layers: int = 32,
                 steps: int = 200, lo: int = 2048, hi: int = 16384, num_q_heads: int = 32,
                 num_kv_heads: int = 8, head_dim: int = 128, name: str = "loop",
                 append: bool = False, kv_dtype: str = "bf16") -> SessionLoop:
    """56 sessions x 32 layers, contexts U[2048, 16384] growing one token per
    step for 200 steps, 32/8 heads, head_dim 128.  append=True: see SessionLoop."""
    rng = np.random.default_rng([seed, 5, zlib.crc32(name.encode())])
    l0 = rng.integers(lo, hi + 1, size=sessions).astype(np.int32)
    if append:
        l0 = np.maximum(l0, 1)
        init = [-(-int(L - 1) // 16) for L in l0]
        final = [-(-int(L - 1 + steps) // 16) for L in l0]
        n_init = int(sum(init))
        n_grow = int(sum(f - i for f, i in zip(final, init)))
        maxp = max(max(final), 1)
        bts = np.full((layers, sessions, maxp), -1, dtype=np.int32)
        for layer in range(layers):
            perm = rng.permutation(n_init).astype(np.int32)
            pos = 0
            for s, n in enumerate(init):
                bts[layer, s, :n] = perm[pos:pos + n]
                pos += n
        free = np.arange(n_init, n_init + n_grow, dtype=np.int32)
        return SessionLoop(name, sessions, layers, steps, num_q_heads, num_kv_heads, head_dim,
                           l0, bts, max(n_init + n_grow, 1), seed, append=True, free_pages=free,
                           kv_dtype=kv_dtype)
    need = [-(-int(L + steps) // 16) for L in l0]
    npg = int(sum(need))
    maxp = max(need)
    bts = np.full((layers, sessions, maxp), -1, dtype=np.int32)
    for layer in range(layers):
        perm = rng.permutation(npg).astype(np.int32)
        pos = 0
        for s, n in enumerate(need):
            bts[layer, s, :n] = perm[pos:pos + n]
            pos += n
    return SessionLoop(name, sessions, layers, steps, num_q_heads, num_kv_heads, head_dim,
                       l0, bts, npg, seed, kv_dtype=kv_dtype)

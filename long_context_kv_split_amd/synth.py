"""Seeded synthetic inputs for the split-KV two-tier attention workloads.

This module is random-number and data-layout plumbing only.  It draws the
query, key and value tensors, picks outlier channels, draws ragged lengths and
deals out paged block tables.  It holds none of the method's arithmetic: it
never rotates, quantizes, attends or merges.  Both the float64 CPU oracle
(through the tests) and the HIP path (through the tests and the benchmark)
read exactly the bytes produced here.

Values are drawn N(0, 1) in float64 by numpy's PCG64 generator, one named
sub-stream per tensor (``numpy.random.SeedSequence(seed).spawn``), optionally
multiplied by 8 on the outlier channels, and rounded once to bfloat16 with
round-to-nearest-even (float64 -> float32 -> bfloat16; the float32 step is
exact for every value the bfloat16 step can distinguish except exact ties,
which this recipe defines as it is written).

The workloads are the five decode / prefill-chunk configurations of the
hybrid-tier method (ActiveKV, "Context beyond VRAM", section "What I built";
QuantForge walkthrough, section 1 for the rotated 4-bit tier):

* ``tiny``       1 x (4 q heads / 1 kv head), d=64, 384 compressed + 128 exact,
                 one split per tier
* ``exact32k``   1 x (32/4), d=128, 32,768 exact tokens, 16 fixed partitions
* ``hybrid128k`` 1 x (32/4), d=128, 123,904 compressed + 4,096 exact, 1% outliers
* ``ragged``     32 x (32/4), d=128, lengths U{4096..65536}, 2,048-token window
* ``chunk``      512-query causal chunk over 28,672 compressed + 4,096 exact,
                 then 512 tokens per kv head evicted into the compressed tier
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK = 64  # tokens per paged block

_STREAMS = (
    "q", "k_exact", "v_exact", "k_quant", "v_quant", "k_chunk", "v_chunk",
    "outliers", "table_exact", "table_quant", "lengths", "k_step", "v_step", "rotation",
)


def stream(seed: int, name: str) -> np.random.Generator:
    """Named, independent PCG64 sub-stream of ``seed``."""
    idx = _STREAMS.index(name)
    child = np.random.SeedSequence(seed).spawn(len(_STREAMS))[idx]
    return np.random.Generator(np.random.PCG64(child))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 data to bfloat16 (via float32), returning uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """Logical (token-ordered) inputs of one attention call, plus paging.

    Per-sequence arrays are uint16 bfloat16 bit patterns shaped
    ``[tokens, Hkv, d]``.  ``quant_*_src`` are the values that the compressed
    tier holds *before* encoding; each side encodes them with its own encoder.
    Block tables map a sequence's tier-local block index to a pool block.
    """

    name: str
    B: int
    Tq: int
    Hq: int
    Hkv: int
    d: int
    q: np.ndarray                      # uint16 [B, Tq, Hq, d]
    exact_k: List[np.ndarray]
    exact_v: List[np.ndarray]
    quant_k_src: List[np.ndarray]
    quant_v_src: List[np.ndarray]
    exact_table: np.ndarray            # int32 [B, max_blocks_exact], -1 = unused
    quant_table: np.ndarray            # int32 [B, max_blocks_quant], -1 = unused
    exact_pool_blocks: int
    quant_pool_blocks: int
    split_tokens_exact: int = 0        # 0 = library default
    split_tokens_quant: int = 0
    causal_tail: int = 0               # chunk: the last Tq exact tokens are the chunk
    evict: int = 0                     # chunk: tokens per kv head moved to the compressed tier
    notes: dict = field(default_factory=dict)

    @property
    def exact_len(self) -> np.ndarray:
        return np.array([x.shape[0] for x in self.exact_k], dtype=np.int32)

    @property
    def quant_len(self) -> np.ndarray:
        return np.array([x.shape[0] for x in self.quant_k_src], dtype=np.int32)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes(self, width: int = 4) -> int:
        """Algorithmic K+V bytes one call streams (bf16 exact tier + width-bit tier)."""
        per_exact = 2 * self.d * 2                      # K and V, bf16
        per_quant = 2 * (self.d * width // 8 + 2 * (self.d // 32))  # codes + fp16 scales, K and V
        return int(self.Hkv * (self.exact_len.sum() * per_exact + self.quant_len.sum() * per_quant))


def _normal_bf16(rng: np.random.Generator, n: int, hkv: int, d: int,
                 outliers: Optional[np.ndarray] = None) -> np.ndarray:
    x = rng.standard_normal((n, hkv, d))
    if outliers is not None and outliers.size:
        h, c = outliers // d, outliers % d
        x[:, h, c] *= 8.0
    return f64_to_bf16_bits(x)


def _deal_tables(rng: np.random.Generator, lengths: List[int], reserve: List[int]):
    """Random permutation of pool blocks dealt out to sequences in order.

    ``reserve[b]`` extra blocks are appended to sequence b's row (space that a
    later eviction writes into).  Returns (table, pool_blocks).
    """
    need = [(-(-n // BLOCK)) + r for n, r in zip(lengths, reserve)]
    total = int(sum(need))
    perm = rng.permutation(total).astype(np.int32)
    width = max(1, max(need))
    table = np.full((len(lengths), width), -1, dtype=np.int32)
    pos = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return table, total


def make(name: str, seed: int = 0) -> Workload:
    """Build one of the five named workloads (seed 0 is the recipe's seed)."""
    if name == "tiny":
        # two splits merged by log-sum-exp: one per tier
        return _decode(name, seed, B=1, Hq=4, Hkv=1, d=64, quant=[384], exact=[128],
                       split_quant=384, split_exact=128)
    if name == "exact32k":
        return _decode(name, seed, B=1, Hq=32, Hkv=4, d=128, quant=[0], exact=[32768],
                       split_exact=2048)
    if name == "hybrid128k":
        return _decode(name, seed, B=1, Hq=32, Hkv=4, d=128, quant=[123904], exact=[4096],
                       outlier_frac=0.01)
    if name == "ragged":
        lens = ragged_lengths(seed)
        return _decode(name, seed, B=32, Hq=32, Hkv=4, d=128,
                       quant=[int(n) - 2048 for n in lens], exact=[2048] * 32)
    if name == "chunk":
        return _chunk(name, seed)
    raise KeyError(name)


def ragged_lengths(seed: int = 0) -> np.ndarray:
    """History lengths of the ragged batch: 32 draws uniform on [4096, 65536]."""
    return stream(seed, "lengths").integers(4096, 65536, size=32, endpoint=True)


def make_small(name: str, seed: int = 0, **kw) -> Workload:
    """A reduced-size variant with the same structure (for parity at oracle speed)."""
    B = kw.get("B", 1)
    quant = kw.get("quant", [1000] * B)
    exact = kw.get("exact", [300] * B)
    return _decode(name, seed, B=B, Hq=kw.get("Hq", 32), Hkv=kw.get("Hkv", 4), d=kw.get("d", 128),
                   quant=quant, exact=exact, outlier_frac=kw.get("outlier_frac", 0.0),
                   split_exact=kw.get("split_exact", 0), split_quant=kw.get("split_quant", 0),
                   Tq=kw.get("Tq", 1), causal_tail=kw.get("causal_tail", 0),
                   reserve_exact=kw.get("reserve_exact"), reserve_quant=kw.get("reserve_quant"))


def _decode(name, seed, B, Hq, Hkv, d, quant, exact, outlier_frac=0.0,
            split_exact=0, split_quant=0, Tq=1, causal_tail=0, reserve_exact=None,
            reserve_quant=None) -> Workload:
    out_k = out_v = None
    if outlier_frac > 0:
        orng = stream(seed, "outliers")
        n_out = int(round(outlier_frac * Hkv * d))
        out_k = orng.choice(Hkv * d, n_out, replace=False)
        out_v = orng.choice(Hkv * d, n_out, replace=False)
    q = _normal_bf16(stream(seed, "q"), B * Tq, Hq, d).reshape(B, Tq, Hq, d)
    rk, rv = stream(seed, "k_quant"), stream(seed, "v_quant")
    ek, ev = stream(seed, "k_exact"), stream(seed, "v_exact")
    qk = [_normal_bf16(rk, n, Hkv, d, out_k) for n in quant]
    qv = [_normal_bf16(rv, n, Hkv, d, out_v) for n in quant]
    xk = [_normal_bf16(ek, n, Hkv, d, out_k) for n in exact]
    xv = [_normal_bf16(ev, n, Hkv, d, out_v) for n in exact]
    # reserve_*[b]: extra blocks at the end of sequence b's table row (room for
    # tokens appended or moved there later)
    et, ep = _deal_tables(stream(seed, "table_exact"), exact, reserve_exact or [0] * B)
    qt, qp = _deal_tables(stream(seed, "table_quant"), quant, reserve_quant or [0] * B)
    notes = {}
    if out_k is not None:
        notes["outliers_k"] = out_k.tolist()
        notes["outliers_v"] = out_v.tolist()
    return Workload(name, B, Tq, Hq, Hkv, d, q, xk, xv, qk, qv, et, qt, ep, qp,
                    split_tokens_exact=split_exact, split_tokens_quant=split_quant,
                    causal_tail=causal_tail, notes=notes)


def _chunk(name, seed, T=512, n_quant=28672, n_exact=4096, evict=512,
           Hq=32, Hkv=4, d=128) -> Workload:
    """Prefill chunk: T causal queries; the chunk's own K/V follow the exact window."""
    q = _normal_bf16(stream(seed, "q"), T, Hq, d).reshape(1, T, Hq, d)
    qk = [_normal_bf16(stream(seed, "k_quant"), n_quant, Hkv, d)]
    qv = [_normal_bf16(stream(seed, "v_quant"), n_quant, Hkv, d)]
    hk = _normal_bf16(stream(seed, "k_exact"), n_exact, Hkv, d)
    hv = _normal_bf16(stream(seed, "v_exact"), n_exact, Hkv, d)
    ck = _normal_bf16(stream(seed, "k_chunk"), T, Hkv, d)
    cv = _normal_bf16(stream(seed, "v_chunk"), T, Hkv, d)
    xk = [np.concatenate([hk, ck], axis=0)]
    xv = [np.concatenate([hv, cv], axis=0)]
    et, ep = _deal_tables(stream(seed, "table_exact"), [n_exact + T], [0])
    qt, qp = _deal_tables(stream(seed, "table_quant"), [n_quant], [-(-evict // BLOCK)])
    return Workload(name, 1, T, Hq, Hkv, d, q, xk, xv, qk, qv, et, qt, ep, qp,
                    causal_tail=T, evict=evict)


def contiguous(w: Workload) -> Workload:
    """Same data with identity block tables (the 'resident' layout)."""
    import copy
    c = copy.copy(w)

    def ident(table):
        t = np.full_like(table, -1)
        pos = 0
        for b in range(table.shape[0]):
            k = int((table[b] >= 0).sum())
            t[b, :k] = np.arange(pos, pos + k, dtype=np.int32)
            pos += k
        return t

    c.exact_table = ident(w.exact_table)
    c.quant_table = ident(w.quant_table)
    return c


def qr_rotation(d: int, seed: int = 0) -> np.ndarray:
    """A seeded random orthogonal matrix, float32 [d, d]: the Q factor of a
    QR factorization of an N(0,1) matrix, columns signed so that R's diagonal
    is positive (the Haar-distributed choice).  Rounded to float32 once."""
    a = stream(seed, "rotation").standard_normal((d, d))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def step_tokens(seed: int, steps: int, B: int, Hkv: int, d: int):
    """New keys and values of `steps` decode steps: bf16 [steps, B, Hkv, d] each."""
    k = _normal_bf16(stream(seed, "k_step"), steps * B, Hkv, d).reshape(steps, B, Hkv, d)
    v = _normal_bf16(stream(seed, "v_step"), steps * B, Hkv, d).reshape(steps, B, Hkv, d)
    return k, v


WORKLOADS = ("tiny", "exact32k", "hybrid128k", "ragged", "chunk")

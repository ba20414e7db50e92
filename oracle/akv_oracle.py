"""CPU oracle for split-KV two-tier attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The library path never calls it, and it shares no code,
table or constant with the HIP sources: every constant below is recomputed
here from its definition.

What it computes (plain definitions, float64 unless a step fixes another
precision):

* attention over a two-tier history (ActiveKV, "Context beyond VRAM",
  section "What I built": recent tokens kept in bf16, older ones encoded, both
  attended through one exact softmax).  The oracle does not
  split or merge at all: it takes one softmax over the whole dequantized
  history, which is what an exact merge of per-tier partials equals;
* the encoded form: a normalized Walsh-Hadamard rotation (QuantForge
  walkthrough, section 1 "Triton Fused Kernels": a Hadamard rotation keeps dot
  products, so the query can be rotated instead of the compressed blocks),
  32-element group RMS scales stored as fp16 and 4-bit indices into the
  16-level Lloyd-Max table for N(0,1).  Because its output must match the GPU
  bit for bit, the encoder emulates the float32 operation sequence of the
  encode steps E1-E9 exactly (each numpy float32 operation is one IEEE
  round-to-nearest-even operation, with no fused multiply-add);
* the same encoded form at 2 and 3 bits (``width``): the 4- and 8-level
  Lloyd-Max tables for N(0,1) in place of the 16-level one, every other step
  unchanged;
* the log-sum-exp merge of normalized partials (each partial carries the
  per-row log-sum-exp that "Bringing a serving stack up on new silicon",
  section "What I built", makes paged attention return so that partials can
  be combined), for the standalone merge entry point.

The decoded history is formed in *unrotated* space with the explicit matrix
H/sqrt(d) (not a fast transform), so the oracle's attention is ordinary
attention; the equivalence with rotated-space attention is pinned by tests.

Every function here is pinned by tests in tests/test_oracle_pins.py against
closed forms, invariants, library special cases or brute force.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

GROUP = 32      # elements per scale group
LEVELS = 16     # 4-bit codes
WIDTHS = (2, 3, 4)  # code widths in bits (2 ** width levels)


# ---------------------------------------------------------------- bit helpers

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ------------------------------------------------------------------- Hadamard

def sylvester_hadamard(d: int) -> np.ndarray:
    """Integer Sylvester-ordered Hadamard matrix H_d (natural order, no sign flips)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def normalized_hadamard(d: int) -> np.ndarray:
    """H_d / sqrt(d): symmetric and orthonormal, so it is its own inverse."""
    return sylvester_hadamard(d).astype(np.float64) / math.sqrt(d)


# ----------------------------------------------------------- Lloyd-Max table

def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper_tail(x):
    """P(X > x) for X ~ N(0,1), accurate in the upper tail."""
    return 0.5 * np.array([math.erfc(v / math.sqrt(2.0)) for v in np.atleast_1d(x)])


def lloyd_max_gaussian(levels: int = LEVELS, tol: float = 1e-15,
                       max_iter: int = 2_000_000) -> np.ndarray:
    """Minimum-MSE scalar quantizer levels for N(0,1) (Lloyd-Max), ascending.

    Lloyd's fixed point: each cell edge is the midpoint of its two levels and
    each level is the conditional mean of N(0,1) over its cell.  Solved on the
    positive half (the density is symmetric, so the levels are too) by plain
    fixed-point iteration in float64 until no level moves by more than tol.
    """
    half = levels // 2
    # start from equal-probability cell means
    edges = np.array([0.0] + [float(_inv_upper_tail(0.5 * (1 - k / half))) for k in range(1, half)]
                     + [math.inf])
    c = _cell_means(edges)
    for _ in range(max_iter):
        edges = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [math.inf]])
        c_new = _cell_means(edges)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    return np.concatenate([-c[::-1], c])


def _cell_means(edges: np.ndarray) -> np.ndarray:
    a, b = edges[:-1], edges[1:]
    pa = _phi(a)
    pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
    mass = _upper_tail(a) - np.where(np.isinf(b), 0.0, _upper_tail(np.where(np.isinf(b), 0.0, b)))
    return (pa - pb) / mass


def _inv_upper_tail(p: float) -> float:
    lo, hi = 0.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _upper_tail(mid)[0] > p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


_TABLE_CACHE: Dict[str, np.ndarray] = {}


def centroids_f32(width: int = 4) -> np.ndarray:
    """The 2**width Lloyd-Max levels rounded to float32 (the frozen table)."""
    if width not in WIDTHS:
        raise ValueError(f"code width {width} not in {WIDTHS}")
    key = f"c{width}"
    if key not in _TABLE_CACHE:
        _TABLE_CACHE[key] = lloyd_max_gaussian(2 ** width).astype(np.float32)
    return _TABLE_CACHE[key]


def zero_code(width: int = 4) -> int:
    """The code of an all-zero group (scale 0, so u = 0): the lower of the two
    levels nearest 0, as an exact tie goes to the lower index."""
    return 2 ** (width - 1) - 1


def thresholds_f32(c32: Optional[np.ndarray] = None, width: int = 4) -> np.ndarray:
    """T_k = largest float32 <= (C_k + C_{k+1}) / 2, k = 0..2**width - 2.

    The midpoint of two float32 values is exact in float64.  With these
    thresholds, code = #{k : u > T_k} is the nearest level, exact ties going
    to the lower index.
    """
    c = centroids_f32(width) if c32 is None else c32
    mid = (c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2.0
    t = mid.astype(np.float32)
    over = t.astype(np.float64) > mid
    t[over] = np.nextafter(t[over], np.float32(-np.inf))
    return t


def inv_sqrt_f32(d: int) -> np.float32:
    """RN_32(1/sqrt(d)), decided exactly with rational arithmetic."""
    # r = 1/sqrt(d) > 0;  v >= r  <=>  v*v*d >= 1  (exact with Fractions)
    v = np.float32(1.0 / math.sqrt(d))
    while Fraction(float(v)) ** 2 * d > 1:
        v = np.nextafter(v, np.float32(0))
    while Fraction(float(np.nextafter(v, np.float32(1)))) ** 2 * d <= 1:
        v = np.nextafter(v, np.float32(1))
    lo = v                                     # largest float32 <= r
    if Fraction(float(lo)) ** 2 * d == 1:
        return np.float32(lo)                  # r is exactly representable
    hi = np.nextafter(lo, np.float32(1))
    mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
    # r < mid  <=>  1 < mid^2 d ; r is irrational here, so there is no tie
    return np.float32(lo if mid * mid * d > 1 else hi)


# -------------------------------------------------------------------- encoder

def fwht_f32(x: np.ndarray) -> np.ndarray:
    """E2: unnormalized Sylvester Walsh-Hadamard transform in float32.

    Stage h = 1, 2, 4, ..., d/2; for every pair (i, i+h) with i & h == 0 the
    pair becomes (x[i] + x[i+h], x[i] - x[i+h]).  Operates on the last axis.
    """
    x = np.asarray(x, dtype=np.float32)
    n, d = x.shape[:-1], x.shape[-1]
    h = 1
    while h < d:
        y = x.reshape(*n, d // (2 * h), 2, h)
        a, b = y[..., 0, :], y[..., 1, :]
        x = np.stack([a + b, a - b], axis=-2).reshape(*n, d)
        h *= 2
    return x


def dense_rotate_f32(x: np.ndarray, rotation: np.ndarray) -> np.ndarray:
    """E2 with a caller-given rotation R (float32 [d, d]): y = R x on the last axis.

    The QuantForge walkthrough (section 5, "README Polish") sets a Hadamard
    rotation against a QR (random orthogonal) one; with R orthogonal no
    further normalization follows (there is no E3).  Each y_i is summed in
    ascending k from 0: y_i = (((0 + R_i0 x_0) + R_i1 x_1) + ...), every
    product and every sum one float32 operation, nothing fused.
    """
    x = np.asarray(x, dtype=np.float32)
    r = np.asarray(rotation, dtype=np.float32)
    acc = np.zeros(x.shape, dtype=np.float32)
    for k in range(x.shape[-1]):
        acc = acc + x[..., k:k + 1] * r[:, k]
    return acc


def group_rms_f32(y: np.ndarray) -> np.ndarray:
    """E4: per 32-group sqrt(mean(y^2)) in float32 with the fixed pairwise tree.

    sq = y*y; then for off = 16, 8, 4, 2, 1: v[i] <- v[i] + v[i+off] (i < off);
    mean = v[0] * 1/32 (exact); result = correctly rounded sqrt.
    """
    y = np.asarray(y, dtype=np.float32)
    v = (y * y).reshape(*y.shape[:-1], y.shape[-1] // GROUP, GROUP)
    off = GROUP // 2
    while off >= 1:
        v = v[..., :off] + v[..., off:2 * off]
        off //= 2
    ms = v[..., 0] * np.float32(1.0 / GROUP)
    return np.sqrt(ms)


def f32_to_f16_sat(s: np.ndarray) -> np.ndarray:
    """E5: IEEE binary16 round-to-nearest-even (subnormals kept), saturating at 65504."""
    s = np.minimum(np.asarray(s, dtype=np.float32), np.float32(65504.0))
    return s.astype(np.float16)


def encode(bits: np.ndarray, rotation: Optional[np.ndarray] = None, width: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """E1-E8 for vectors of bf16 bit patterns shaped [..., d].

    Returns (codes uint8 [..., d] in 0..2**width - 1, scales as uint16 fp16
    bit patterns [..., d/32]).  Packing (E9) is a storage detail: see
    pack_nibbles.  With ``rotation`` (float32 [d, d], orthogonal) E2 is
    dense_rotate_f32 and E3 is skipped; otherwise E2 is the Hadamard
    butterflies and E3 the 1/sqrt(d) normalization.  ``width`` picks the
    Lloyd-Max table (E8); every other step is the same at every width.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    d = bits.shape[-1]
    x = bf16_to_f32(bits)                                 # E1
    if rotation is not None:
        y = dense_rotate_f32(x, rotation)                 # E2 (dense; no E3)
    else:
        x = fwht_f32(x)                                   # E2
        y = x * inv_sqrt_f32(d)                           # E3
    s32 = group_rms_f32(y)                                # E4
    s16 = f32_to_f16_sat(s32)                             # E5
    s = s16.astype(np.float32)                            # E6
    yg = y.reshape(*y.shape[:-1], d // GROUP, GROUP)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = yg / s[..., None]                             # E7
    codes = nearest_code(u, width)                        # E8
    codes[s == 0] = zero_code(width)                      # zero scale: u == 0 -> lower of the two middle levels
    return codes.reshape(bits.shape), s16.view(np.uint16)


def nearest_code(u: np.ndarray, width: int = 4) -> np.ndarray:
    """E8: index of the nearest float32 level to float32 u, exact ties to the lower index.

    Equals #{k : u > T_k} with the round-down midpoints T_k (a binary search
    over the sorted thresholds counts them).
    """
    t = thresholds_f32(width=width)
    return np.searchsorted(t, np.asarray(u, dtype=np.float32), side="left").astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """E9: two codes per byte along the last axis, even element in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_rotated(codes: np.ndarray, scales16: np.ndarray, width: int = 4) -> np.ndarray:
    """Rotated-space reconstruction C[code] * scale, exact in float64."""
    c = centroids_f32(width).astype(np.float64)
    d = codes.shape[-1]
    s = f16_bits_to_f64(scales16)
    vals = c[codes.astype(np.int64)].reshape(*codes.shape[:-1], d // GROUP, GROUP)
    return (vals * s[..., None]).reshape(codes.shape)


def dequant(codes: np.ndarray, scales16: np.ndarray, rotation: Optional[np.ndarray] = None,
            width: int = 4) -> np.ndarray:
    """Unrotated reconstruction: (H/sqrt(d)) @ rotated with the explicit matrix, or
    R^T @ rotated for a given rotation R (orthogonal, so R^T undoes it)."""
    r = dequant_rotated(codes, scales16, width)
    d = r.shape[-1]
    if rotation is not None:
        return r @ np.asarray(rotation, dtype=np.float64)   # row-vector form of R^T @ r
    return r @ normalized_hadamard(d)   # H is symmetric: row-vector form of H @ r


# ------------------------------------------------------------------ attention

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              mask: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query-head set against one key/value set.

    q [R, d], k [N, d], v [N, d]; mask [R, N] bool (True = attend) or None.
    Returns o [R, d] (normalized) and lse [R] (natural log of the sum of
    exp(scores)); rows with nothing to attend give o = 0, lse = -inf.
    """
    s = (q @ k.T) * scale                      # [R, N]
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - safe[:, None])
    z = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(z > 0, safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    w = np.where(z[:, None] > 0, e / np.where(z > 0, z, 1.0)[:, None], 0.0)
    return w @ v, lse


def history_f64(k_exact_bits: np.ndarray, v_exact_bits: np.ndarray,
                kq_codes: Optional[np.ndarray], kq_scales: Optional[np.ndarray],
                vq_codes: Optional[np.ndarray], vq_scales: Optional[np.ndarray],
                head: int, rotation: Optional[np.ndarray] = None, width: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """Attended history of one kv head: compressed tier first, then exact tier."""
    ks, vs = [], []
    if kq_codes is not None and kq_codes.shape[0]:
        ks.append(dequant(kq_codes[:, head], kq_scales[:, head], rotation, width))
        vs.append(dequant(vq_codes[:, head], vq_scales[:, head], rotation, width))
    if k_exact_bits.shape[0]:
        ks.append(bf16_to_f64(k_exact_bits[:, head]))
        vs.append(bf16_to_f64(v_exact_bits[:, head]))
    d = k_exact_bits.shape[-1]
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks), np.concatenate(vs)


def decode_sequence(q_bits: np.ndarray, k_exact_bits, v_exact_bits,
                    kq_codes, kq_scales, vq_codes, vq_scales,
                    scale: Optional[float] = None, causal_tail: int = 0,
                    heads: Optional[Sequence[int]] = None, rotation: Optional[np.ndarray] = None,
                    width: int = 4):
    """Attention of one sequence's queries over its whole two-tier history.

    q_bits [Tq, Hq, d] bf16; exact tier [Ne, Hkv, d] bf16; compressed tier as
    codes [Nq, Hkv, d] and fp16 scale bits [Nq, Hkv, d/32].  Query head h uses
    kv head h // (Hq/Hkv).  With causal_tail = T > 0 the last T exact tokens
    are the chunk itself and query i (0-based) sees chunk tokens <= i.
    Returns o [Tq, Hq, d] float64 and lse [Tq, Hq] float64 (only the listed
    heads are filled when ``heads`` is given; the rest are NaN).
    """
    Tq, Hq, d = q_bits.shape
    Hkv = k_exact_bits.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if not scale else scale
    q = bf16_to_f64(q_bits)
    o = np.full((Tq, Hq, d), np.nan)
    lse = np.full((Tq, Hq), np.nan)
    want = set(range(Hq)) if heads is None else set(heads)
    for kv in range(Hkv):
        hs = [h for h in range(kv * G, (kv + 1) * G) if h in want]
        if not hs:
            continue
        k, v = history_f64(k_exact_bits, v_exact_bits, kq_codes, kq_scales, vq_codes, vq_scales, kv, rotation,
                           width)
        mask = None
        if causal_tail:
            n = k.shape[0]
            pos = np.arange(n)
            limit = n - causal_tail + np.arange(Tq)        # last visible index per query
            mask_t = pos[None, :] <= limit[:, None]        # [Tq, N]
        for h in hs:
            if causal_tail:
                mask = mask_t
            oh, lh = attention(q[:, h, :], k, v, scale, mask)
            o[:, h, :] = oh
            lse[:, h] = lh
    return o, lse


# ---------------------------------------------------------------------- merge

def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact merge of P normalized partials.

    o_parts [P, R, d], lse_parts [P, R].  M = max_p lse_p; if M = -inf the
    row is empty (o = 0, lse = -inf); else w_p = exp(lse_p - M), W = sum w_p,
    lse = M + ln W, o = sum_p (w_p / W) o_p.  NaN propagates.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    P, R = lse_parts.shape
    d = o_parts.shape[-1]
    o = np.zeros((R, d))
    lse = np.full(R, -np.inf)
    for r in range(R):
        col = lse_parts[:, r]
        if np.any(np.isnan(col)):
            o[r] = np.nan
            lse[r] = np.nan
            continue
        M = np.max(col)
        if M == -np.inf:
            continue
        w = np.exp(col - M)
        W = w.sum()
        lse[r] = M + math.log(W)
        o[r] = ((w / W)[:, None] * o_parts[:, r, :]).sum(axis=0)
    return o, lse


# ------------------------------------------------------------ whole workloads

def encode_tier(src_bits: List[np.ndarray]):
    """Encode every sequence's compressed-tier source; returns per-seq (codes, scales)."""
    return [encode(x) for x in src_bits]


def reference_outputs(w, encoded_k=None, encoded_v=None, heads=None, seqs=None, rotation=None, width=4):
    """o [B, Tq, Hq, d] and lse [B, Tq, Hq] (float64) for a synth.Workload-like object.

    ``w`` needs: q, exact_k, exact_v, quant_k_src, quant_v_src, causal_tail.
    Pass pre-encoded compressed tiers to avoid re-encoding.
    """
    B = len(w.exact_k)
    Tq, Hq, d = w.q.shape[1:]
    o = np.full((B, Tq, Hq, d), np.nan)
    lse = np.full((B, Tq, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        if encoded_k is None:
            kc, ks = encode(w.quant_k_src[b], rotation, width)
            vc, vs = encode(w.quant_v_src[b], rotation, width)
        else:
            kc, ks = encoded_k[b]
            vc, vs = encoded_v[b]
        ob, lb = decode_sequence(w.q[b], w.exact_k[b], w.exact_v[b], kc, ks, vc, vs,
                                 causal_tail=w.causal_tail, heads=heads, rotation=rotation, width=width)
        o[b], lse[b] = ob, lb
    return o, lse


# ------------------------------------------------------------ per-step bookkeeping

def append_evict_step(exact_k: np.ndarray, exact_v: np.ndarray, quant_k: np.ndarray, quant_v: np.ndarray,
                      new_k: np.ndarray, new_v: np.ndarray, window: int, exact_capacity: int,
                      quant_capacity: int):
    """One decode step of a sequence's two-tier history, on logical token lists.

    ActiveKV ("Context beyond VRAM", "What I built") appends each step's new
    key/value to the recent exact window and keeps the older history in the
    compact tier.  Tiers are token-ordered bf16 arrays [n, Hkv, d]; the
    compressed tier is held as its values before encoding (encoding is per
    token, so the codes of a moved token are ``encode`` of its bf16 values).

    The new token goes to the end of the exact tier.  When the exact tier then
    holds window + 64 tokens and the compressed tier has room for 64 more, the
    64 oldest exact tokens move, in order, to the end of the compressed tier,
    whatever its current length.  Capacities are in tokens.  Returns the four
    new arrays, or None when the exact tier has no room for the new token.
    """
    n = exact_k.shape[0]
    if n + 1 > exact_capacity:
        return None
    ek = np.concatenate([exact_k, new_k[None]], axis=0)
    ev = np.concatenate([exact_v, new_v[None]], axis=0)
    qk, qv = quant_k, quant_v
    m = qk.shape[0]
    if n + 1 >= window + 64 and m + 64 <= quant_capacity:
        qk = np.concatenate([qk, ek[:64]], axis=0)
        qv = np.concatenate([qv, ev[:64]], axis=0)
        ek, ev = ek[64:], ev[64:]
    return ek, ev, qk, qv

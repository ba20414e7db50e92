"""Pins of the float64 CPU oracle against things other than itself.

Each test checks an oracle function against a closed form, an invariant, a
library special case (torch's CPU scaled_dot_product_attention, scipy
quadrature) or brute force with exact rational arithmetic.  The pages print no
worked example for this method, so no test compares against printed values.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import akv_oracle as O

RNG = np.random.default_rng(12345)


def _bf16(x):
    from long_context_kv_split_amd.synth import f64_to_bf16_bits
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------------ P-1 Hadamard

@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_hadamard_orthogonal_exact(d):
    h = O.sylvester_hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
    assert np.array_equal(h, h.T)
    hn = O.normalized_hadamard(d)
    assert np.allclose(hn @ hn, np.eye(d), atol=1e-14)


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_matches_matrix_columns(d):
    h = O.sylvester_hadamard(d)
    eye = np.eye(d, dtype=np.float32)
    out = O.fwht_f32(eye)                      # row i = transform of e_i
    assert np.array_equal(out.astype(np.int64), h.T)   # = column i of H


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_involution_on_small_integers(d):
    x = RNG.integers(-50, 51, size=(20, d)).astype(np.float32)
    y = O.fwht_f32(O.fwht_f32(x))
    assert np.array_equal(y, d * x)
    # and equals the integer matrix product exactly
    assert np.array_equal(O.fwht_f32(x).astype(np.int64), x.astype(np.int64) @ O.sylvester_hadamard(d).T)


def test_fwht_float32_close_to_float64_matrix():
    x = O.bf16_to_f32(_bf16(RNG.standard_normal((50, 128))))
    ref = x.astype(np.float64) @ O.sylvester_hadamard(128).T
    got = O.fwht_f32(x).astype(np.float64)
    assert np.max(np.abs(got - ref)) < 1e-4


# --------------------------------------------------------------- P-2 Lloyd-Max

def test_lloyd_max_fixed_point_by_quadrature():
    from scipy import integrate, stats
    c = O.lloyd_max_gaussian()
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], atol=0, rtol=0)
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    n = stats.norm
    for k in range(16):
        mass = integrate.quad(n.pdf, edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * n.pdf(x), edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(mom / mass - c[k]) < 1e-12
    mse = sum(integrate.quad(lambda x: (x - c[k]) ** 2 * n.pdf(x), edges[k], edges[k + 1],
                             epsabs=1e-15)[0] for k in range(16))
    assert abs(mse - 0.0095010) < 5e-7


def test_centroids_and_thresholds_exact_rounding():
    c64 = O.lloyd_max_gaussian()
    c32 = O.centroids_f32()
    assert np.array_equal(c32, c64.astype(np.float32))
    t = O.thresholds_f32()
    for k in range(15):
        mid = (Fraction(float(c32[k])) + Fraction(float(c32[k + 1]))) / 2
        tk = Fraction(float(t[k]))
        nxt = Fraction(float(np.nextafter(t[k], np.float32(np.inf))))
        assert tk <= mid < nxt, k
    assert t[7] == 0.0


def test_inv_sqrt_rounding_decimal():
    getcontext().prec = 60
    for d in (64, 128):
        r = 1 / Decimal(d).sqrt()
        v = O.inv_sqrt_f32(d)
        cands = [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(1))]
        errs = [abs(Decimal(float(x)) - r) for x in cands]
        assert errs[1] <= min(errs)
    assert O.inv_sqrt_f32(128).view(np.uint32) == 0x3DB504F3
    assert O.inv_sqrt_f32(64) == np.float32(0.125)


# ------------------------------------------------------------ P-8 encoder steps

def _rne_f16_fraction(x: Fraction) -> Fraction:
    """Round a non-negative rational to binary16 (RNE, subnormals) -- brute force."""
    if x == 0:
        return Fraction(0)
    e = math.floor(math.log2(float(x)))
    # adjust e so that 2^e <= x < 2^(e+1)
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    q = Fraction(2) ** (max(e, -14) - 10)          # spacing (subnormal below 2^-14)
    n = x / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    return min(v, Fraction(65504))


def test_f16_rounding_brute_force():
    vals = [2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
            0.1, 1.0 / 3, 65504.0, 65519.0, 65536.0, 1e-5, 6.1e-5, 7.0e-8]
    vals += list(RNG.uniform(0, 4, 200)) + list(np.exp(RNG.uniform(-17, 11, 200)))
    x = np.array(vals, dtype=np.float32)
    got = O.f32_to_f16_sat(x).astype(np.float64)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == _rne_f16_fraction(Fraction(float(xi))), xi


def test_group_rms_tree_order_closed_form():
    # y[0] = 2^12, y[8] = y[16] = y[24] = 1: squares 2^24, 1, 1, 1.
    # tree: off=16 -> v0 = 2^24 + 1 -> 2^24 (tie to even); v8 = 1 + 1 = 2;
    #       off=8  -> v0 = 2^24 + 2 (exact); rest adds zeros.
    # a left-to-right sum would give 2^24 instead.
    y = np.zeros((1, 32), dtype=np.float32)
    y[0, 0] = 4096.0
    y[0, 8] = y[0, 16] = y[0, 24] = 1.0
    s = O.group_rms_f32(y)[0, 0]
    ms = np.float32((2.0 ** 24 + 2) / 32)          # exact: 524288.0625 is representable
    assert float(ms) == 524288.0625
    getcontext().prec = 50
    exact = Decimal(524288.0625).sqrt()
    cands = [np.float32(float(exact)), np.nextafter(np.float32(float(exact)), np.float32(0)),
             np.nextafter(np.float32(float(exact)), np.float32(1e9))]
    best = min(cands, key=lambda v: abs(Decimal(float(v)) - exact))
    assert s == best


def test_group_rms_close_to_float64():
    y = RNG.standard_normal((100, 128)).astype(np.float32)
    got = O.group_rms_f32(y).astype(np.float64)
    ref = np.sqrt((y.astype(np.float64).reshape(100, 4, 32) ** 2).mean(-1))
    assert np.max(np.abs(got / ref - 1)) < 1e-6


def test_nearest_code_brute_force_fractions():
    c = [Fraction(float(v)) for v in O.centroids_f32()]
    mids = [(c[k] + c[k + 1]) / 2 for k in range(15)]
    us = list(RNG.normal(0, 1.3, 3000).astype(np.float32))
    # exact midpoints that are float32 (ties) and their neighbours
    for m in mids:
        f = np.float32(float(m))
        us += [f, np.nextafter(f, np.float32(-9)), np.nextafter(f, np.float32(9))]
    us += [np.float32(0.0), np.float32(-0.0), np.float32(40.0), np.float32(-40.0)]
    u = np.array(us, dtype=np.float32)
    got = O.nearest_code(u)
    for ui, gi in zip(u, got):
        fu = Fraction(float(ui))
        dist = [abs(fu - ck) for ck in c]
        best = min(range(16), key=lambda k: (dist[k], k))   # ties -> lower index
        assert gi == best, (ui, gi, best)


def test_encoder_crafted_ties_through_public_path():
    # x = H y / 16 (d=128): dyadic and bf16-exact for small integers y, and the
    # float32 transform returns 8 y exactly; after the 1/sqrt(d) multiply the
    # zeros of y stay exactly 0, so u = 0 there: the C7/C8 tie -> code 7.
    d = 128
    h = O.sylvester_hadamard(d)
    for trial in range(20):
        y = RNG.integers(-3, 4, size=d)
        y[RNG.choice(d, 16, replace=False)] = 0
        x = (h @ y) / 16.0
        bits = _bf16(x)
        assert np.array_equal(O.bf16_to_f64(bits), x)      # exact in bf16
        codes, scales = O.encode(bits[None, :])
        zero = (y == 0)
        assert np.all(codes[0][zero] == 7)
        # positive y -> codes >= 8, negative y -> codes <= 7
        assert np.all(codes[0][y > 0] >= 8) and np.all(codes[0][y < 0] <= 7)


def test_encoder_all_zero_group():
    bits = np.zeros((3, 128), dtype=np.uint16)
    codes, scales = O.encode(bits)
    assert np.all(codes == 7) and np.all(scales == 0)


def test_encoder_scale_recompute_and_ideal_codes():
    d = 128
    x = _bf16(RNG.standard_normal((400, d)))
    codes, scales = O.encode(x)
    # float64-ideal pipeline
    y = O.bf16_to_f64(x) @ O.normalized_hadamard(d).T
    rms = np.sqrt((y.reshape(400, 4, 32) ** 2).mean(-1))
    s = O.f16_bits_to_f64(scales)
    assert np.max(np.abs(s / rms - 1)) < 2 ** -10            # fp16 rounding
    u = y.reshape(400, 4, 32) / s[..., None]
    c = O.centroids_f32().astype(np.float64)
    ideal = np.argmin(np.abs(u[..., None] - c), axis=-1).reshape(400, d)
    diff = ideal.astype(int) - codes.astype(int)
    assert np.all(np.abs(diff) <= 1)
    flips = np.argwhere(diff != 0)
    mids = (c[:-1] + c[1:]) / 2
    for i, j in flips:
        uu = u.reshape(400, d)[i, j]
        assert np.min(np.abs(mids - uu)) < 1e-5 * max(1.0, abs(uu))


def test_roundtrip_error_is_lloyd_max_sized():
    d = 128
    x = _bf16(RNG.standard_normal((2000, d)))
    codes, scales = O.encode(x)
    xr = O.dequant(codes, scales)
    xf = O.bf16_to_f64(x)
    rel = np.sum((xr - xf) ** 2) / np.sum(xf ** 2)
    assert 0.007 < rel < 0.013          # ~ the 16-level Gaussian MSE of 0.0095
    # dropping the inverse rotation would leave an error of order 2
    bad = O.dequant_rotated(codes, scales)
    assert np.sum((bad - xf) ** 2) / np.sum(xf ** 2) > 1.5


def test_pack_unpack_nibbles():
    codes = RNG.integers(0, 16, size=(5, 64)).astype(np.uint8)
    p = O.pack_nibbles(codes)
    assert p.shape == (5, 32)
    assert np.all(p[:, 0] == (codes[:, 0] | (codes[:, 1] << 4)))
    assert np.array_equal(O.unpack_nibbles(p), codes)


# ----------------------------------------------------- P-3 rotation exactness

def test_rotation_preserves_dots_and_attention():
    d, N = 64, 40
    hn = O.normalized_hadamard(d)
    q = RNG.standard_normal((3, d))
    k = RNG.standard_normal((N, d))
    v = RNG.standard_normal((N, d))
    assert np.allclose((q @ hn.T) @ (k @ hn.T).T, q @ k.T, rtol=1e-12, atol=1e-12)
    o, lse = O.attention(q, k, v, 0.125)
    o_r, lse_r = O.attention(q @ hn.T, k @ hn.T, v @ hn.T, 0.125)
    assert np.allclose(lse_r, lse, rtol=1e-12, atol=1e-12)
    assert np.allclose(o_r @ hn.T, o, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------- P-4 merge exactness

def test_merge_of_any_partition_equals_single_softmax():
    d, N = 32, 97
    q = RNG.standard_normal((5, d))
    k = RNG.standard_normal((N, d))
    v = RNG.standard_normal((N, d))
    o, lse = O.attention(q, k, v, 0.2)
    for cuts in ([0, 97], [0, 10, 50, 97], [0, 0, 30, 30, 97], [0, 1, 2, 3, 97, 97]):
        parts = [(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)]
        ops, lps = [], []
        for a, b in parts:
            oo, ll = O.attention(q, k[a:b], v[a:b], 0.2)
            ops.append(oo)
            lps.append(ll)
        om, lm = O.lse_merge(np.array(ops), np.array(lps))
        assert np.allclose(lm, lse, rtol=1e-12, atol=1e-12)
        assert np.allclose(om, o, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ P-5 brute force

def _brute(q, k, v, scale, mask=None):
    R, d = len(q), len(q[0])
    N = len(k)
    o = [[0.0] * d for _ in range(R)]
    lse = []
    for r in range(R):
        s = []
        for j in range(N):
            if mask is not None and not mask[r][j]:
                continue
            acc = 0.0
            for t in range(d):
                acc += q[r][t] * k[j][t]
            s.append((acc * scale, j))
        if not s:
            lse.append(-math.inf)
            continue
        m = max(x for x, _ in s)
        z = sum(math.exp(x - m) for x, _ in s)
        L = m + math.log(z)
        lse.append(L)
        for x, j in s:
            w = math.exp(x - L)
            for t in range(d):
                o[r][t] += w * v[j][t]
    return np.array(o), np.array(lse)


def test_decode_sequence_brute_force_tiny_hybrid():
    from long_context_kv_split_amd import synth
    w = synth.make_small("t", B=1, Hq=4, Hkv=2, d=64, quant=[40], exact=[24])
    kc, ks = O.encode(w.quant_k_src[0])
    vc, vs = O.encode(w.quant_v_src[0])
    o, lse = O.decode_sequence(w.q[0], w.exact_k[0], w.exact_v[0], kc, ks, vc, vs)
    q = O.bf16_to_f64(w.q[0])
    for h in range(4):
        kv = h // 2
        kk = np.concatenate([O.dequant(kc[:, kv], ks[:, kv]), O.bf16_to_f64(w.exact_k[0][:, kv])])
        vv = np.concatenate([O.dequant(vc[:, kv], vs[:, kv]), O.bf16_to_f64(w.exact_v[0][:, kv])])
        ob, lb = _brute(q[:, h].tolist(), kk.tolist(), vv.tolist(), 1 / 8)
        assert np.allclose(lb, lse[:, h], rtol=1e-12, atol=1e-12)
        assert np.allclose(ob, o[:, h], rtol=1e-12, atol=1e-12)


def test_causal_chunk_brute_force():
    from long_context_kv_split_amd import synth
    w = synth.make_small("c", B=1, Hq=2, Hkv=1, d=8 * 8, quant=[16], exact=[12], Tq=5, causal_tail=5)
    kc, ks = O.encode(w.quant_k_src[0])
    vc, vs = O.encode(w.quant_v_src[0])
    o, lse = O.decode_sequence(w.q[0], w.exact_k[0], w.exact_v[0], kc, ks, vc, vs, causal_tail=5)
    kk = np.concatenate([O.dequant(kc[:, 0], ks[:, 0]), O.bf16_to_f64(w.exact_k[0][:, 0])])
    vv = np.concatenate([O.dequant(vc[:, 0], vs[:, 0]), O.bf16_to_f64(w.exact_v[0][:, 0])])
    N = kk.shape[0]
    mask = [[j <= N - 5 + i for j in range(N)] for i in range(5)]
    q = O.bf16_to_f64(w.q[0])
    for h in range(2):
        ob, lb = _brute(q[:, h].tolist(), kk.tolist(), vv.tolist(), 1 / 8, mask)
        assert np.allclose(lb, lse[:, h], rtol=1e-12, atol=1e-12)
        assert np.allclose(ob, o[:, h], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------- P-6 library special case

def test_all_exact_matches_torch_sdpa_gqa():
    import torch
    from long_context_kv_split_amd import synth
    w = synth.make_small("e", B=1, Hq=8, Hkv=2, d=128, quant=[0], exact=[300])
    o, lse = O.decode_sequence(w.q[0], w.exact_k[0], w.exact_v[0], None, None, None, None)
    q = torch.tensor(O.bf16_to_f64(w.q[0])).permute(1, 0, 2)[None]          # [1, Hq, 1, d]
    k = torch.tensor(O.bf16_to_f64(w.exact_k[0])).permute(1, 0, 2)[None]    # [1, Hkv, N, d]
    v = torch.tensor(O.bf16_to_f64(w.exact_v[0])).permute(1, 0, 2)[None]
    k = k.repeat_interleave(4, dim=1)
    v = v.repeat_interleave(4, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    assert np.allclose(ref[0, :, 0].numpy(), o[0], rtol=1e-12, atol=1e-12)
    # lse via torch.logsumexp of the scaled scores
    s = (q @ k.transpose(-1, -2)) / math.sqrt(128)
    assert np.allclose(torch.logsumexp(s, -1)[0, :, 0].numpy(), lse[0], rtol=1e-12, atol=1e-12)


def test_causal_matches_torch_sdpa_mask():
    import torch
    from long_context_kv_split_amd import synth
    T = 7
    w = synth.make_small("e", B=1, Hq=4, Hkv=1, d=64, quant=[0], exact=[30], Tq=T, causal_tail=T)
    o, lse = O.decode_sequence(w.q[0], w.exact_k[0], w.exact_v[0], None, None, None, None,
                               causal_tail=T)
    q = torch.tensor(O.bf16_to_f64(w.q[0])).permute(1, 0, 2)[None]
    k = torch.tensor(O.bf16_to_f64(w.exact_k[0])).permute(1, 0, 2)[None].repeat_interleave(4, 1)
    v = torch.tensor(O.bf16_to_f64(w.exact_v[0])).permute(1, 0, 2)[None].repeat_interleave(4, 1)
    N = 30
    mask = torch.tensor([[j <= N - T + i for j in range(N)] for i in range(T)])
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    assert np.allclose(ref[0].permute(1, 0, 2).numpy(), o, rtol=1e-12, atol=1e-12)


def test_hybrid_with_empty_compressed_tier_is_exact_only():
    from long_context_kv_split_amd import synth
    w = synth.make_small("h", B=1, Hq=4, Hkv=1, d=64, quant=[0], exact=[50])
    e = np.zeros((0, 1, 64), dtype=np.uint16)
    kc, ks = O.encode(e)
    o1, l1 = O.decode_sequence(w.q[0], w.exact_k[0], w.exact_v[0], kc, ks, kc, ks)
    o2, l2 = O.decode_sequence(w.q[0], w.exact_k[0], w.exact_v[0], None, None, None, None)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --------------------------------------------------------------- P-7 closed forms

def test_closed_forms():
    d = 64
    N = 37
    k = RNG.standard_normal((N, d))
    v = RNG.standard_normal((N, d))
    o, lse = O.attention(np.zeros((1, d)), k, v, 0.125)
    assert abs(lse[0] - math.log(N)) < 1e-13
    assert np.allclose(o[0], v.mean(0), atol=1e-13)
    q = RNG.standard_normal((2, d))
    o, lse = O.attention(q, k[:1], v[:1], 0.125)
    assert np.allclose(o, np.repeat(v[:1], 2, 0), atol=0)
    assert np.allclose(lse, (q @ k[0]) * 0.125, atol=1e-13)
    vc = np.tile(RNG.standard_normal((1, d)), (N, 1))
    o, _ = O.attention(q, k, vc, 0.125)
    assert np.allclose(o, np.repeat(vc[:1], 2, 0), atol=1e-13)


# ------------------------------------------------------- P-9 merge special values

@pytest.mark.parametrize("P", [1, 2, 3])
def test_merge_special_values(P):
    vals = [0.3, -np.inf, 80.0, -80.0, 1e4, -1e4]
    d = 4
    import itertools
    for combo in itertools.product(vals, repeat=P):
        lse_p = np.array(combo, dtype=np.float64)[:, None]
        o_p = RNG.standard_normal((P, 1, d))
        o_p[lse_p[:, 0] == -np.inf] = 0.0
        o, l = O.lse_merge(o_p, lse_p)
        assert not np.any(np.isnan(o)) and not np.isnan(l[0])
        fin = np.isfinite(lse_p[:, 0])
        if not fin.any():
            assert l[0] == -np.inf and np.all(o == 0)
            continue
        # exact rational check of the weights for the finite parts
        M = max(lse_p[fin, 0])
        w = np.array([math.exp(x - M) if f else 0.0 for x, f in zip(lse_p[:, 0], fin)])
        assert abs(l[0] - (M + math.log(w.sum()))) <= 1e-12 * max(1, abs(l[0]))
        assert np.allclose(o[0], (w[:, None] * o_p[:, 0]).sum(0) / w.sum(), atol=1e-12)


def test_merge_nan_propagates():
    o, l = O.lse_merge(np.zeros((2, 1, 3)), np.array([[np.nan], [1.0]]))
    assert np.isnan(l[0]) and np.all(np.isnan(o))


# --------------------------------------------------------------- generator sanity

def test_generator_is_deterministic_and_shaped():
    from long_context_kv_split_amd import synth
    a = synth.make("tiny")
    b = synth.make("tiny")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.quant_k_src[0], b.quant_k_src[0])
    assert a.q.shape == (1, 1, 4, 64)
    assert list(a.quant_len) == [384] and list(a.exact_len) == [128]
    assert a.kv_bytes() == 60416
    assert sorted(a.exact_table[0][a.exact_table[0] >= 0].tolist()) == [0, 1]


# ------------------------------------------------------------ per-step append / evict

def _tokens(rng, n, hkv=2, d=64):
    return O_bits(rng.standard_normal((n, hkv, d)))


def O_bits(x):
    from long_context_kv_split_amd.synth import f64_to_bf16_bits
    return f64_to_bf16_bits(x)


def _run_steps(ek, ev, qk, qv, new_k, new_v, window, ecap, qcap):
    lens = []
    for t in range(new_k.shape[0]):
        r = O.append_evict_step(ek, ev, qk, qv, new_k[t], new_v[t], window, ecap, qcap)
        if r is None:
            lens.append(None)
            break
        ek, ev, qk, qv = r
        lens.append((ek.shape[0], qk.shape[0]))
    return ek, ev, qk, qv, lens


@pytest.mark.parametrize("e0,q0", [(128, 40), (150, 41), (191, 40), (191, 7)])
def test_append_evict_lengths_closed_form(e0, q0):
    """With room everywhere the exact tier cycles through [W, W + 63] and every
    64th append moves one block, for an even or an odd compressed length alike:
    after t steps the exact tier holds W + (e0 - W + t) mod 64 tokens and the
    compressed tier q0 + 64 * floor((e0 - W + t) / 64)."""
    rng = np.random.default_rng(1)
    W, T = 128, 150
    ek, ev = _tokens(rng, e0), _tokens(rng, e0)
    qk, qv = _tokens(rng, q0), _tokens(rng, q0)
    nk, nv = _tokens(rng, T), _tokens(rng, T)
    *_, lens = _run_steps(ek, ev, qk, qv, nk, nv, W, 10 ** 6, 10 ** 6)
    for t, (ne, nq) in enumerate(lens, start=1):
        assert ne == W + (e0 - W + t) % 64
        assert nq == q0 + 64 * ((e0 - W + t) // 64)


def test_append_evict_conserves_the_history_order():
    """Compressed tier then exact tier, concatenated, is the initial history
    followed by every appended token, in order."""
    rng = np.random.default_rng(2)
    ek, ev, qk, qv = _tokens(rng, 190), _tokens(rng, 190), _tokens(rng, 64), _tokens(rng, 64)
    nk, nv = _tokens(rng, 100), _tokens(rng, 100)
    fk, fv, gk, gv, _ = _run_steps(ek, ev, qk, qv, nk, nv, 128, 10 ** 6, 10 ** 6)
    assert np.array_equal(np.concatenate([gk, fk]), np.concatenate([qk, ek, nk]))
    assert np.array_equal(np.concatenate([gv, fv]), np.concatenate([qv, ev, nv]))
    assert gk.shape[0] > qk.shape[0]


def test_append_evict_full_compressed_tier_keeps_growing_the_window():
    rng = np.random.default_rng(3)
    ek, ev = _tokens(rng, 191), _tokens(rng, 191)
    nk, nv = _tokens(rng, 5), _tokens(rng, 5)
    # compressed tier at capacity: nothing moves, the exact tier grows by one per step
    qk, qv = _tokens(rng, 100), _tokens(rng, 100)
    fk, _, gk, _, lens = _run_steps(ek, ev, qk, qv, nk, nv, 128, 10 ** 6, 120)
    assert [l[0] for l in lens] == [192, 193, 194, 195, 196] and gk.shape[0] == 100
    # exact tier at capacity: the step is refused
    assert O.append_evict_step(ek, ev, qk, qv, nk[0], nv[0], 128, 191, 10 ** 6) is None


def test_append_evict_moves_a_block_onto_an_odd_compressed_length():
    """The tiers are token lists: how many tokens the compressed tier already
    holds has no bearing on when the window's oldest block moves.  A 99-token
    compressed tier takes the block on the step that fills the window, and the
    moved tokens follow token 98 in order."""
    rng = np.random.default_rng(5)
    ek, ev = _tokens(rng, 191), _tokens(rng, 191)
    qk, qv = _tokens(rng, 99), _tokens(rng, 99)
    nk, nv = _tokens(rng, 3), _tokens(rng, 3)
    fk, fv, gk, gv, lens = _run_steps(ek, ev, qk, qv, nk, nv, 128, 10 ** 6, 10 ** 6)
    assert lens == [(128, 163), (129, 163), (130, 163)]
    assert np.array_equal(gk, np.concatenate([qk, ek[:64]])) and np.array_equal(gv, np.concatenate([qv, ev[:64]]))
    assert np.array_equal(fk, np.concatenate([ek[64:], nk])) and np.array_equal(fv, np.concatenate([ev[64:], nv]))


def test_encoding_is_per_token():
    """The codes of tokens moved between tiers are encode() of their own values:
    encoding a concatenation equals concatenating the encodings."""
    rng = np.random.default_rng(4)
    a, b = _tokens(rng, 7, 2, 128), _tokens(rng, 9, 2, 128)
    ca, sa = O.encode(a)
    cb, sb = O.encode(b)
    cab, sab = O.encode(np.concatenate([a, b]))
    assert np.array_equal(cab, np.concatenate([ca, cb])) and np.array_equal(sab, np.concatenate([sa, sb]))


# ------------------------------------------------------------ dense (QR) rotation

def test_dense_rotation_matches_python_float32_loop():
    """E2 with a given rotation, checked against scalar float32 operations."""
    rng = np.random.default_rng(5)
    d = 8
    r = rng.standard_normal((d, d)).astype(np.float32)
    x = rng.standard_normal((3, d)).astype(np.float32)
    got = O.dense_rotate_f32(x, r)
    for n in range(3):
        for i in range(d):
            acc = np.float32(0.0)
            for k in range(d):
                acc = np.float32(acc + np.float32(r[i, k] * x[n, k]))
            assert got[n, i] == acc


def test_qr_rotation_is_orthogonal_and_seeded():
    from long_context_kv_split_amd.synth import qr_rotation
    for d in (64, 128):
        r = qr_rotation(d, 0).astype(np.float64)
        assert np.max(np.abs(r @ r.T - np.eye(d))) < 2e-6
        assert np.all(np.diag(np.linalg.qr(qr_rotation(d, 0).astype(np.float64))[1]) != 0)
        assert np.array_equal(qr_rotation(d, 0), qr_rotation(d, 0))
        assert not np.array_equal(qr_rotation(d, 0), qr_rotation(d, 1))


def test_dense_encoder_with_hadamard_matrix_differs_only_near_midpoints():
    """With R = H/sqrt(d) as a dense float32 matrix the dense encoder computes the
    same rotation in another summation order: codes differ by at most one level,
    and only where u sits within a few ulps of a threshold."""
    from long_context_kv_split_amd.synth import f64_to_bf16_bits
    rng = np.random.default_rng(6)
    d = 128
    x = f64_to_bf16_bits(rng.standard_normal((400, d)))
    h = O.normalized_hadamard(d).astype(np.float32)
    c0, s0 = O.encode(x)
    c1, s1 = O.encode(x, h)
    diff = c0.astype(int) - c1.astype(int)
    assert np.max(np.abs(diff)) <= 1
    assert np.mean(diff != 0) < 1e-3
    # scales: the same group RMS up to a few float32 ulps, so fp16 equal almost always
    assert np.mean(s0 != s1) < 5e-3


def test_qr_round_trip_and_attention_are_lloyd_max_sized():
    """Encoding under a QR rotation and undoing it with R^T gives the Lloyd-Max error,
    and attention over the reconstruction stays close to exact attention."""
    from long_context_kv_split_amd.synth import f64_to_bf16_bits, qr_rotation
    rng = np.random.default_rng(7)
    d = 128
    r = qr_rotation(d, 3)
    xb = f64_to_bf16_bits(rng.standard_normal((2000, 1, d)))
    c, s = O.encode(xb, r)
    xh = O.dequant(c[:, 0], s[:, 0], r)
    x = O.bf16_to_f64(xb[:, 0])
    rel = np.mean((xh - x) ** 2) / np.mean(x ** 2)
    assert 0.005 < rel < 0.02
    q = rng.standard_normal((4, d))
    oe, le = O.attention(q, x, x, 1 / np.sqrt(d))
    oq, lq = O.attention(q, xh, xh, 1 / np.sqrt(d))
    assert np.max(np.abs(le - lq)) < 0.5 and np.max(np.abs(oe - oq)) < 0.2


# ----------------------------------------------- code widths 2 and 3 (4 / 8 levels)

# Max (1960), "Quantizing for minimum distortion", table of the minimum
# mean-square-error quantizer for a unit Gaussian: output levels (positive
# half) and the distortion, to the printed precision.
MAX_1960 = {2: ([0.4528, 1.510], 0.1175), 3: ([0.2451, 0.7560, 1.344, 2.152], 0.03455)}


@pytest.mark.parametrize("width", [2, 3])
def test_lloyd_max_narrow_tables_match_max_1960_and_fixed_point(width):
    from scipy import integrate, stats
    n_lv = 2 ** width
    c = O.lloyd_max_gaussian(n_lv)
    assert np.all(np.diff(c) > 0) and np.array_equal(c, -c[::-1])
    levels, mse_ref = MAX_1960[width]
    assert np.allclose(c[n_lv // 2:], levels, atol=6e-4, rtol=0)
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    n = stats.norm
    mse = 0.0
    for k in range(n_lv):
        mass = integrate.quad(n.pdf, edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * n.pdf(x), edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(mom / mass - c[k]) < 1e-12
        mse += integrate.quad(lambda x: (x - c[k]) ** 2 * n.pdf(x), edges[k], edges[k + 1], epsabs=1e-15)[0]
    assert abs(mse - mse_ref) < 6e-5


@pytest.mark.parametrize("width", [2, 3])
def test_narrow_thresholds_and_nearest_code_brute_force(width):
    n_lv = 2 ** width
    c32 = O.centroids_f32(width)
    assert np.array_equal(c32, O.lloyd_max_gaussian(n_lv).astype(np.float32))
    t = O.thresholds_f32(width=width)
    assert t.shape == (n_lv - 1,) and t[n_lv // 2 - 1] == 0.0
    c = [Fraction(float(v)) for v in c32]
    for k in range(n_lv - 1):
        mid = (c[k] + c[k + 1]) / 2
        assert Fraction(float(t[k])) <= mid < Fraction(float(np.nextafter(t[k], np.float32(np.inf))))
    us = list(RNG.normal(0, 1.5, 2000).astype(np.float32))
    for k in range(n_lv - 1):
        f = np.float32(float((c[k] + c[k + 1]) / 2))
        us += [f, np.nextafter(f, np.float32(-9)), np.nextafter(f, np.float32(9))]
    us += [np.float32(0.0), np.float32(-0.0), np.float32(40.0), np.float32(-40.0)]
    u = np.array(us, dtype=np.float32)
    got = O.nearest_code(u, width)
    for ui, gi in zip(u, got):
        fu = Fraction(float(ui))
        best = min(range(n_lv), key=lambda k: (abs(fu - c[k]), k))
        assert gi == best, (width, ui, gi, best)


@pytest.mark.parametrize("width", [2, 3])
def test_narrow_encoder_zero_group_and_ties(width):
    """All-zero groups give scale 0 and the lower middle code; x = H y / 16
    puts u exactly on 0 where y = 0 (the middle tie), on the sign side elsewhere."""
    zc = O.zero_code(width)
    codes, scales = O.encode(np.zeros((2, 64), dtype=np.uint16), width=width)
    assert np.all(codes == zc) and np.all(scales == 0)
    d = 128
    h = O.sylvester_hadamard(d)
    for _ in range(10):
        y = RNG.integers(-3, 4, size=d)
        y[RNG.choice(d, 16, replace=False)] = 0
        bits = _bf16((h @ y) / 16.0)
        codes, _ = O.encode(bits[None, :], width=width)
        assert np.all(codes[0][y == 0] == zc)
        assert np.all(codes[0][y > 0] > zc) and np.all(codes[0][y < 0] <= zc)
        assert codes.max() < 2 ** width


def test_narrow_round_trip_errors_follow_the_tables():
    """Round-trip error of Gaussian vectors is near each table's distortion
    (0.1175, 0.0346, 0.0095 of the signal power), and the same vectors
    encoded at a lower width never reconstruct better."""
    d = 128
    x = _bf16(RNG.standard_normal((2000, d)))
    xf = O.bf16_to_f64(x)
    rel = {}
    for width, lo, hi in ((2, 0.10, 0.14), (3, 0.029, 0.041), (4, 0.007, 0.013)):
        codes, scales = O.encode(x, width=width)
        rel[width] = np.sum((O.dequant(codes, scales, width=width) - xf) ** 2) / np.sum(xf ** 2)
        assert lo < rel[width] < hi, (width, rel[width])
        # scales do not depend on the width
        assert np.array_equal(scales, O.encode(x)[1])
    assert rel[2] > rel[3] > rel[4]
    # decoding 2-bit codes with the 4-bit table is far off
    codes, scales = O.encode(x, width=2)
    assert np.sum((O.dequant(codes, scales) - xf) ** 2) / np.sum(xf ** 2) > 0.3

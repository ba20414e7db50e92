"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Tolerances (fixed by the method's contract): 4-bit codes and fp16 scales
bit-exact; every |lse - lse_ref| <= 1e-4; every |o - o_ref| <= 2e-3 *
max|o_ref| + 1e-3 with the max over the whole output tensor of the case.
Determinism: repeated calls are bit-identical, and a random (paged) block
table gives the same bytes as the contiguous ("resident") layout.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import akv_oracle as O
from long_context_kv_split_amd import synth

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4


def _mods():
    from long_context_kv_split_amd import akv, harness
    return akv, harness


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()   # the library must load; no fallback exists


def _say(msg):
    print(msg, flush=True)


def assert_attention(o, lse, o_ref, lse_ref, label):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    m = np.isfinite(lse_ref)
    assert np.all(np.isfinite(lse[m])), f"{label}: non-finite lse"
    dl = np.max(np.abs(lse[m] - lse_ref[m]))
    tol_o = 2e-3 * np.max(np.abs(o_ref)) + 1e-3
    do = np.max(np.abs(o - o_ref))
    _say(f"{label}: max|dlse|={dl:.3e} max|do|={do:.3e} (tol {tol_o:.3e})")
    assert dl <= LSE_TOL, f"{label}: lse error {dl}"
    assert do <= tol_o, f"{label}: o error {do} > {tol_o}"


def run_case(w, **kw):
    akv, harness = _mods()
    _say(f"case {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} quant={list(w.quant_len)[:4]} "
         f"exact={list(w.exact_len)[:4]}")
    dw = harness.DeviceWorkload(w)
    akv.check(dw.attend(**kw))
    torch.cuda.synchronize()
    return dw


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_case(w, dw=None, seqs=None, heads=None):
    """The oracle's encodings and float64 attention for sequences `seqs` (all
    by default) and query heads `heads` (all by default; the others stay NaN).
    Each sequence's encoding and each (sequence, kv head)'s attention is one
    oracle call; the calls run on a thread pool (numpy releases the GIL inside
    its array loops), which changes nothing in what each call computes."""
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    G = w.Hq // w.Hkv

    def enc(b):
        return b, O.encode(w.quant_k_src[b]), O.encode(w.quant_v_src[b])

    def att(job):
        b, kv = job
        hs = [h for h in range(kv * G, (kv + 1) * G) if heads is None or h in heads]
        if not hs:
            return b, hs, None, None
        (kc, ks), (vc, vs) = enc_k[b], enc_v[b]
        ob, lb = O.decode_sequence(w.q[b], w.exact_k[b], w.exact_v[b], kc, ks, vc, vs,
                                   causal_tail=w.causal_tail, heads=hs)
        return b, hs, ob, lb

    with ThreadPoolExecutor(_workers()) as ex:
        encs = list(ex.map(enc, seqs))
        enc_k = {b: k for b, k, _ in encs}
        enc_v = {b: v for b, _, v in encs}
        o = np.full((w.B, w.Tq, w.Hq, w.d), np.nan)
        lse = np.full((w.B, w.Tq, w.Hq), np.nan)
        for b, hs, ob, lb in ex.map(att, [(b, kv) for b in seqs for kv in range(w.Hkv)]):
            if hs:
                o[b][:, hs] = ob[:, hs]
                lse[b][:, hs] = lb[:, hs]
    return o, lse, enc_k, enc_v


def assert_codes(dw, w, enc_k, enc_v, label):
    for b, (kc, ks) in enc_k.items():
        vc, vs = enc_v[b]
        gk, gks, gv, gvs = dw.read_codes(b)
        assert np.array_equal(gk, kc), f"{label} seq {b}: K codes differ ({int((gk != kc).sum())})"
        assert np.array_equal(gks, ks), f"{label} seq {b}: K scales differ ({int((gks != ks).sum())})"
        assert np.array_equal(gv, vc), f"{label} seq {b}: V codes differ ({int((gv != vc).sum())})"
        assert np.array_equal(gvs, vs), f"{label} seq {b}: V scales differ ({int((gvs != vs).sum())})"
    _say(f"{label}: codes and scales bit-exact for {len(enc_k)} sequence(s)")


# ------------------------------------------------------------------ encoder

@pytest.mark.parametrize("d", [64, 128])
def test_compress_bit_exact_ragged(d):
    w = synth.make_small("enc", B=2, Hq=8, Hkv=2, d=d, quant=[1000, 777], exact=[64, 64], outlier_frac=0.02)
    akv, harness = _mods()
    dw = harness.DeviceWorkload(w)
    torch.cuda.synchronize()
    enc_k = {b: O.encode(w.quant_k_src[b]) for b in range(2)}
    enc_v = {b: O.encode(w.quant_v_src[b]) for b in range(2)}
    assert_codes(dw, w, enc_k, enc_v, f"compress d={d}")


def test_compress_crafted_ties():
    """x = H y / 16: u is exactly 0 where y is 0 -> code 7; all-zero vectors -> codes 7, scale 0."""
    d, n = 128, 64
    h = O.sylvester_hadamard(d)
    rng = np.random.default_rng(7)
    vals = np.zeros((n, 1, d))
    for t in range(n - 4):
        y = rng.integers(-3, 4, size=d)
        y[rng.choice(d, 20, replace=False)] = 0
        vals[t, 0] = (h @ y) / 16.0
    bits = synth.f64_to_bf16_bits(vals)
    assert np.array_equal(O.bf16_to_f64(bits), vals)
    w = synth.make_small("ties", B=1, Hq=1, Hkv=1, d=d, quant=[n], exact=[64])
    w.quant_k_src[0] = bits
    w.quant_v_src[0] = bits
    akv, harness = _mods()
    dw = harness.DeviceWorkload(w)
    torch.cuda.synchronize()
    enc = O.encode(bits)
    assert_codes(dw, w, {0: enc}, {0: enc}, "crafted ties")
    gk = dw.read_codes(0)[0]
    assert np.all(gk[-4:] == 7)


def test_compress_eviction_into_pool():
    """Evict exact tokens [0, 512) of a chunk-shaped workload into compressed positions 448*64.."""
    akv, harness = _mods()
    w = synth.make_small("ev", B=1, Hq=8, Hkv=2, d=128, quant=[448 * 64 // 8], exact=[640])
    # place the destination right after the existing compressed tokens (even start)
    n_q = int(w.quant_len[0])
    w.quant_table = np.concatenate([w.quant_table, np.full((1, 8), -1, np.int32)], axis=1)
    extra = np.arange(w.quant_pool_blocks, w.quant_pool_blocks + 8, dtype=np.int32)
    nb_used = -(-n_q // 64)
    w.quant_table[0, nb_used:nb_used + 8] = extra
    w.quant_pool_blocks += 8
    w.evict = 512
    dw = harness.DeviceWorkload(w)
    start = nb_used * 64
    akv.check(akv.akv_compress_evicted(dw.compress_desc(0, 0, 512, start), harness.stream_handle()))
    torch.cuda.synchronize()
    kc, ks = O.encode(w.exact_k[0][:512])
    vc, vs = O.encode(w.exact_v[0][:512])
    gk, gks, gv, gvs = dw.read_codes(0, start, 512)
    assert np.array_equal(gk, kc) and np.array_equal(gks, ks)
    assert np.array_equal(gv, vc) and np.array_equal(gvs, vs)


@pytest.mark.parametrize("d,width", [(128, 4), (64, 4), (128, 3), (64, 3), (128, 2), (64, 2)])
def test_compress_odd_destination_start(d, width):
    """Two compress calls into one compressed tier: tokens [0, 301), then
    [301, 551), whose first position is odd and shares its value-code byte
    with token 300.  The whole tier equals the oracle's encoding of all 551
    tokens, and position 551 (outside both ranges, sharing a byte with 550)
    keeps the codes and scales it held before."""
    akv, harness = _mods()
    w = synth.make_small("odd", B=1, Hq=8, Hkv=2, d=d, quant=[0], exact=[551], reserve_quant=[9])
    dw = harness.DeviceWorkload(w, width=width)
    P = dw.pools[0]
    g = torch.Generator(device="cpu").manual_seed(11)
    for t in (P.kc, P.vc):   # arbitrary prior contents
        t.copy_(torch.randint(0, 256, t.shape, dtype=torch.uint8, generator=g))
    for t in (P.ks, P.vs):
        t.copy_(torch.randint(0, 0x3C00, t.shape, dtype=torch.int16, generator=g))
    torch.cuda.synchronize()
    before = dw.read_codes(0, 551, 1)
    h = harness.stream_handle()
    _say(f"odd start d={d} width={width}: compress [0, 301) then [301, 551)")
    akv.check(akv.akv_compress_evicted(dw.compress_desc(0, 0, 301, 0), h))
    akv.check(akv.akv_compress_evicted(dw.compress_desc(0, 301, 250, 301), h))
    torch.cuda.synchronize()
    kc, ks = O.encode(w.exact_k[0], width=width)
    vc, vs = O.encode(w.exact_v[0], width=width)
    gk, gks, gv, gvs = dw.read_codes(0, 0, 551)
    for name, a, b in (("K codes", gk, kc), ("K scales", gks, ks), ("V codes", gv, vc), ("V scales", gvs, vs)):
        assert np.array_equal(a, b), f"{name} differ at {int((a != b).sum())} places"
    after = dw.read_codes(0, 551, 1)
    for a, b in zip(before, after):
        assert np.array_equal(a, b), "a position outside the range changed"
    _say(f"odd start d={d} width={width}: 551 tokens bit-exact, neighbour untouched")


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("cfg", [
    dict(B=2, Hq=32, Hkv=4, d=128, quant=[1000, 2500], exact=[300, 77], split_exact=128, split_quant=256),
    dict(B=3, Hq=32, Hkv=4, d=128, quant=[0, 130, 4000], exact=[1, 64, 700], split_exact=0, split_quant=0,
         outlier_frac=0.01),
    dict(B=2, Hq=4, Hkv=1, d=64, quant=[383, 64], exact=[129, 0], split_exact=64, split_quant=128),
    dict(B=1, Hq=12, Hkv=2, d=128, quant=[777], exact=[65], split_exact=64, split_quant=192),
    # one query head per kv head (15 of the 16 matrix columns are padding), ragged pair
    dict(B=2, Hq=4, Hkv=4, d=128, quant=[700, 300], exact=[200, 65], split_exact=0, split_quant=0),
    # two query heads per kv head, d 64
    dict(B=1, Hq=8, Hkv=4, d=64, quant=[900], exact=[130], split_exact=64, split_quant=256),
    # three sequences with 4 + 2 = 6 splits each (an even count in a batch: each
    # unit's splits are rotated over the XCDs), one with no compressed tier
    dict(B=3, Hq=8, Hkv=2, d=128, quant=[1000, 300, 0], exact=[256, 64, 130], split_exact=128, split_quant=256),
    # 125 + 3 = 128 splits (the most the 4-wave merge takes; the exact tier's
    # splits sit past lane 63), the short sequence leaving most of them inactive
    dict(B=2, Hq=8, Hkv=2, d=128, quant=[8000, 100], exact=[190, 64], split_exact=64, split_quant=64),
    # 141 + 16 = 157 splits: the general merge
    dict(B=2, Hq=4, Hkv=1, d=64, quant=[9000, 0], exact=[1000, 70], split_exact=64, split_quant=64),
])
def test_decode_small(cfg):
    w = synth.make_small("small", **cfg)
    dw = run_case(w)
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw, w, {b: ek[b] for b in range(w.B) if w.quant_len[b]},
                 {b: ev[b] for b in range(w.B) if w.quant_len[b]}, "small")
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, f"small {cfg}")


def test_decode_peaked_scores():
    """Queries scaled by 16 (exact in bfloat16): scores spread over tens of
    units, so each split's running maximum keeps rising and the online softmax
    rescales its sums many times, while each row's weight sits on a few
    tokens; two sequences of different lengths."""
    w = synth.make_small("peaked", B=2, Hq=32, Hkv=4, d=128, quant=[3000, 900], exact=[300, 130])
    w.q = synth.f64_to_bf16_bits(synth.bf16_bits_to_f32(w.q).astype(np.float64) * 16.0)
    dw = run_case(w)
    o_ref, lse_ref, _, _ = oracle_case(w)
    assert np.max(lse_ref) - np.min(lse_ref) > 20.0  # the scale really spreads the scores
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "decode, queries x16")


def test_tiny_two_splits():
    """The tiny config: one split per tier (384 compressed, 128 exact tokens),
    merged by log-sum-exp."""
    akv, _ = _mods()
    w = synth.make("tiny")
    dw = run_case(w)
    plan = akv.akv_split_plan(dw.desc())
    assert plan == {"split_tokens_quant": 384, "split_tokens_exact": 128, "splits_quant": 1, "splits_exact": 1}, plan
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw, w, ek, ev, "tiny")
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "tiny")


@pytest.fixture(scope="module")
def exact32k():
    w = synth.make("exact32k")
    dw = run_case(w, split_exact=2048)
    o_ref, lse_ref, _, _ = oracle_case(w)
    return w, dw, o_ref, lse_ref


def test_exact32k_parity(exact32k):
    w, dw, o_ref, lse_ref = exact32k
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "exact32k (16 splits)")


def test_exact32k_bit_identical_run_to_run(exact32k):
    akv, harness = _mods()
    w, dw, _, _ = exact32k
    o0, l0 = dw.o.clone(), dw.lse.clone()
    for _ in range(10):
        akv.check(dw.attend(split_exact=2048))
    torch.cuda.synchronize()
    assert torch.equal(dw.o, o0) and torch.equal(dw.lse, l0)


def test_exact32k_paged_equals_contiguous(exact32k):
    akv, harness = _mods()
    w, dw, _, _ = exact32k
    o0, l0 = dw.o.clone(), dw.lse.clone()
    wc = synth.contiguous(w)
    dc = harness.DeviceWorkload(wc)
    akv.check(dc.attend(split_exact=2048))
    torch.cuda.synchronize()
    assert torch.equal(dc.o, o0) and torch.equal(dc.lse, l0)


def test_exact32k_sub_splits_are_the_finer_plan(exact32k):
    """Each of the 16 partitions is attended by 4 workgroups of 512 tokens whose
    partials are merged in token order: the same bytes as 64 splits of 512."""
    akv, harness = _mods()
    w, dw, _, _ = exact32k
    assert akv.akv_decode_split_workgroups(dw.desc(split_exact=2048)) == 4
    o0, l0 = dw.o.clone(), dw.lse.clone()
    akv.check(dw.attend(split_exact=512))
    torch.cuda.synchronize()
    assert torch.equal(dw.o, o0) and torch.equal(dw.lse, l0)


def test_exact32k_single_split_within_tolerance(exact32k):
    akv, harness = _mods()
    w, dw, o_ref, lse_ref = exact32k
    akv.check(dw.attend(split_exact=32768))
    torch.cuda.synchronize()
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "exact32k (1 split)")


def _same_again(dw, label):
    """A second call (outputs cleared first) gives the same bytes: fixed split
    plan and fixed reduction order."""
    akv, _ = _mods()
    o1, l1 = dw.o.clone(), dw.lse.clone()
    dw.o.fill_(float("nan"))
    dw.lse.fill_(float("nan"))
    akv.check(dw.attend())
    torch.cuda.synchronize()
    assert torch.equal(dw.o, o1) and torch.equal(dw.lse, l1), f"{label}: not bit-identical run to run"
    _say(f"{label}: second call bit-identical")


@pytest.mark.slow
def test_hybrid128k():
    w = synth.make("hybrid128k")
    dw = run_case(w)
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw, w, ek, ev, "hybrid128k")
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "hybrid128k")
    _same_again(dw, "hybrid128k")


@pytest.mark.slow
def test_ragged_all_sequences():
    """The full ragged batch: every code and scale of all 32 sequences, and every
    output of every sequence and head, against the oracle."""
    w = synth.make("ragged")
    dw = run_case(w)
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw, w, ek, ev, "ragged")
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    assert_attention(o, lse, o_ref, lse_ref, "ragged, all 32 sequences")
    _same_again(dw, "ragged")


# ------------------------------------------------------------------ merge

def test_lse_merge_random_and_special():
    akv, harness = _mods()
    rng = np.random.default_rng(3)
    for P, R, d in [(1, 5, 64), (3, 100, 128), (17, 7, 33), (64, 3, 256)]:
        lp = rng.normal(0, 5, (P, R))
        specials = np.array([-np.inf, 80.0, -80.0, 1e4, -1e4, 0.0])
        mask = rng.random((P, R)) < 0.3
        lp[mask] = rng.choice(specials, mask.sum())
        lp[:, 0] = -np.inf            # an all-empty row
        op = rng.normal(0, 1, (P, R, d))
        op[np.isinf(lp)] = 0.0
        o_ref, l_ref = O.lse_merge(op, lp)
        top = torch.tensor(op, dtype=torch.float32, device="cuda")
        tlp = torch.tensor(lp, dtype=torch.float32, device="cuda")
        oo = torch.empty((R, d), dtype=torch.float32, device="cuda")
        ll = torch.empty((R,), dtype=torch.float32, device="cuda")
        akv.check(akv.akv_lse_merge(top.data_ptr(), tlp.data_ptr(), P, R, d, oo.data_ptr(), ll.data_ptr(),
                                    harness.stream_handle()))
        torch.cuda.synchronize()
        lg = ll.cpu().numpy().astype(np.float64)
        og = oo.cpu().numpy().astype(np.float64)
        assert lg[0] == -np.inf and np.all(og[0] == 0)
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        # fp32 merge of |lse| up to 1e4: allow the float32 spacing of the inputs
        assert np.max(np.abs(lg[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))) < 2e-6
        assert np.max(np.abs(og - o_ref)) < 1e-5 * max(1.0, np.max(np.abs(o_ref)))

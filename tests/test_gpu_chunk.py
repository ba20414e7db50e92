"""GPU parity of the prefill-chunk path (akv_attend_chunk) and the eviction after it.

Same contract as the decode tests: every |lse - lse_ref| <= 1e-4, every
|o - o_ref| <= 2e-3 * max|o_ref| + 1e-3, codes and scales bit-exact, repeated
calls and paged / contiguous block tables give identical bytes.  The oracle
applies the causal rule of the chunk: query i sees the whole compressed
tier and the exact tier up to exact token len_exact - Tq + i.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import akv_oracle as O
from long_context_kv_split_amd import synth

from test_gpu_parity import _mods, _say, assert_attention, assert_codes, oracle_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()


def run_chunk(w, **kw):
    akv, harness = _mods()
    _say(f"chunk case {w.name}: B={w.B} Tq={w.Tq} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
         f"quant={list(w.quant_len)} exact={list(w.exact_len)} {kw}")
    assert w.causal_tail == w.Tq
    dw = harness.DeviceWorkload(w)
    akv.check(dw.attend(**kw))
    torch.cuda.synchronize()
    return dw


CASES = [
    # 160 rows: two row groups, the second ragged; several splits per tier
    dict(B=1, Hq=8, Hkv=2, d=128, quant=[1000], exact=[300], Tq=40, split_exact=128, split_quant=256),
    # second sequence: no compressed tier, exact tier is the chunk alone
    dict(B=2, Hq=32, Hkv=4, d=128, quant=[700, 0], exact=[200, 130], Tq=130),
    # head dim 64, one kv head
    dict(B=1, Hq=4, Hkv=1, d=64, quant=[383], exact=[129], Tq=33, split_exact=64, split_quant=128),
    # G = 6: a row group boundary falls inside a query's heads
    dict(B=1, Hq=12, Hkv=2, d=128, quant=[300], exact=[65], Tq=17, split_quant=64),
    # outlier channels on a short history: the precision-critical case
    dict(B=1, Hq=32, Hkv=4, d=128, quant=[2000], exact=[600], Tq=64, outlier_frac=0.01),
    # one query: the chunk degenerates to decode over the whole history
    dict(B=1, Hq=32, Hkv=4, d=128, quant=[1500], exact=[100], Tq=1),
    # one query head per kv head: 50 rows per kv head, a single ragged row group
    dict(B=1, Hq=4, Hkv=4, d=128, quant=[600], exact=[200], Tq=50),
    # two query heads per kv head, d 64
    dict(B=1, Hq=8, Hkv=4, d=64, quant=[500], exact=[100], Tq=20, split_quant=128),
]


@pytest.mark.parametrize("cfg", CASES)
def test_chunk_small(cfg):
    cfg = dict(cfg)
    kw = {k: cfg.pop(k) for k in ("split_exact", "split_quant") if k in cfg}
    w = synth.make_small("chunk_small", causal_tail=cfg["Tq"], **cfg)
    dw = run_chunk(w, **kw)
    o_ref, lse_ref, ek, ev = oracle_case(w)
    qs = [b for b in range(w.B) if w.quant_len[b]]
    assert_codes(dw, w, {b: ek[b] for b in qs}, {b: ev[b] for b in qs}, "chunk small")
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, f"chunk {cfg} {kw}")


def test_chunk_peaked_scores():
    """Queries scaled by 16 (exact in bfloat16): scores spread over tens of
    units, so a split's running maximum keeps rising well past the compressed
    tier's 2^8 allowance and the softmax reference moves (rescaling O and l)
    many times per split, while each row's weight sits on a few tokens."""
    w = synth.make_small("chunk_peaked", B=1, Hq=32, Hkv=4, d=128, quant=[1500], exact=[400], Tq=64,
                         causal_tail=64)
    w.q = synth.f64_to_bf16_bits(synth.bf16_bits_to_f32(w.q).astype(np.float64) * 16.0)
    dw = run_chunk(w)
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert np.max(lse_ref) - np.min(lse_ref) > 20.0  # the scale really spreads the scores
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "chunk, queries x16")


def test_chunk_deterministic_and_paged_equals_contiguous():
    akv, harness = _mods()
    w = synth.make_small("chunk_det", B=1, Hq=32, Hkv=4, d=128, quant=[1200], exact=[400], Tq=100,
                         causal_tail=100)
    dw = run_chunk(w)
    o0, l0 = dw.o.clone(), dw.lse.clone()
    for _ in range(5):
        akv.check(dw.attend())
    torch.cuda.synchronize()
    assert torch.equal(dw.o, o0) and torch.equal(dw.lse, l0)
    dc = harness.DeviceWorkload(synth.contiguous(w))
    akv.check(dc.attend())
    torch.cuda.synchronize()
    assert torch.equal(dc.o, o0) and torch.equal(dc.lse, l0)


def test_chunk_exact_tier_shorter_than_chunk_gives_nan():
    akv, harness = _mods()
    w = synth.make_small("chunk_bad", B=2, Hq=8, Hkv=2, d=128, quant=[256, 256], exact=[64, 64], Tq=16,
                         causal_tail=16)
    dw = harness.DeviceWorkload(w)
    dw.exact_len[1] = 15          # below Tq: the chunk is not in the exact tier
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(lse[1]))
    o_ref, lse_ref, _, _ = oracle_case(w, seqs=[0])
    assert_attention(o[:1], lse[:1], o_ref[:1], lse_ref[:1], "chunk seq 0 beside a refused seq")


@pytest.fixture(scope="module")
def chunk_full():
    w = synth.make("chunk")
    dw = run_chunk(w)
    return w, dw


def test_chunk_full_size_all_heads(chunk_full):
    """512 causal queries over 28,672 compressed + 4,096 exact + 512 chunk tokens;
    every query of every one of the 32 heads against the oracle."""
    w, dw = chunk_full
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw, w, ek, ev, "chunk full")
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    assert_attention(o, lse, o_ref, lse_ref, "chunk full, all 32 heads")


def test_chunk_full_then_evict(chunk_full):
    """After the chunk: the 512 oldest exact tokens per kv head go to compressed
    positions 28,672.. (the blocks the table reserves for them), bit-exact."""
    akv, harness = _mods()
    w, dw = chunk_full
    start = int(w.quant_len[0])
    assert start == 28672 and w.evict == 512
    akv.check(akv.akv_compress_evicted(dw.compress_desc(0, 0, 512, start), harness.stream_handle()))
    torch.cuda.synchronize()
    kc, ks = O.encode(w.exact_k[0][:512])
    vc, vs = O.encode(w.exact_v[0][:512])
    gk, gks, gv, gvs = dw.read_codes(0, start, 512)
    assert np.array_equal(gk, kc) and np.array_equal(gks, ks)
    assert np.array_equal(gv, vc) and np.array_equal(gvs, vs)
    _say("chunk eviction: 512 tokens x 4 kv heads bit-exact")

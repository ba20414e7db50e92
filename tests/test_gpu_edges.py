"""GPU edge cases through the C ABI: absent tiers, and device-side problems the
kernels' own checks turn into NaN outputs for the affected sequence only
(a block id outside the pool, a length beyond the block table)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_kv_split_amd import synth

from test_gpu_parity import _mods, _say, assert_attention, oracle_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()


def _run(w, mutate=None, **kw):
    akv, harness = _mods()
    dw = harness.DeviceWorkload(w)
    if mutate is not None:
        mutate(dw)
    akv.check(dw.attend(**kw))
    torch.cuda.synchronize()
    return dw, dw.o.cpu().numpy(), dw.lse.cpu().numpy()


def test_decode_without_exact_tier():
    w = synth.make_small("noexact", B=2, Hq=32, Hkv=4, d=128, quant=[900, 64], exact=[0, 0])
    dw, o, lse = _run(w)
    assert dw.emax == 0
    o_ref, lse_ref, _, _ = oracle_case(w)
    assert_attention(o, lse, o_ref, lse_ref, "decode, compressed tier only")


def test_chunk_without_compressed_tier():
    w = synth.make_small("chunk_noq", B=1, Hq=32, Hkv=4, d=128, quant=[0], exact=[300], Tq=40, causal_tail=40)
    dw, o, lse = _run(w)
    assert dw.qmax == 0
    o_ref, lse_ref, _, _ = oracle_case(w)
    assert_attention(o, lse, o_ref, lse_ref, "chunk, exact tier only")


@pytest.mark.parametrize("tier", ["quant", "exact"])
def test_decode_bad_block_id_poisons_only_its_sequence(tier):
    w = synth.make_small("badblock", B=2, Hq=8, Hkv=2, d=128, quant=[1000, 700], exact=[300, 200])

    def mutate(dw):
        table = dw.quant_table if tier == "quant" else dw.exact_table
        table[1, 2] = 1 << 20 if tier == "quant" else -7   # outside the pool / negative
    dw, o, lse = _run(w, mutate)
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(lse[1]))
    o_ref, lse_ref, _, _ = oracle_case(w, seqs=[0])
    assert_attention(o[:1], lse[:1], o_ref[:1], lse_ref[:1], f"decode seq 0 beside a bad {tier} block id")


def test_decode_length_beyond_table_gives_nan():
    w = synth.make_small("badlen", B=2, Hq=8, Hkv=2, d=128, quant=[1000, 700], exact=[300, 200])

    def mutate(dw):
        dw.quant_len[0] = dw.qmax * 64 + 1
    dw, o, lse = _run(w, mutate)
    assert np.all(np.isnan(o[0])) and np.all(np.isnan(lse[0]))
    o_ref, lse_ref, _, _ = oracle_case(w, seqs=[1])
    assert_attention(o[1:], lse[1:], o_ref[1:], lse_ref[1:], "decode seq 1 beside a bad length")
    _say("bad length: NaN for its sequence only")


def test_chunk_bad_block_id_poisons_only_its_sequence():
    w = synth.make_small("chunk_bad_id", B=2, Hq=8, Hkv=2, d=128, quant=[500, 300], exact=[150, 100], Tq=20,
                         causal_tail=20)

    def mutate(dw):
        dw.quant_table[0, 1] = -1
    dw, o, lse = _run(w, mutate)
    assert np.all(np.isnan(o[0])) and np.all(np.isnan(lse[0]))
    o_ref, lse_ref, _, _ = oracle_case(w, seqs=[1])
    assert_attention(o[1:], lse[1:], o_ref[1:], lse_ref[1:], "chunk seq 1 beside a bad block id")

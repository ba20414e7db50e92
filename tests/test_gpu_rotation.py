"""GPU parity of the compressed tier under a given rotation (QR, random orthogonal).

The QuantForge walkthrough (section 5, "README Polish") compares the
Walsh-Hadamard rotation with a QR one.  With a rotation R passed in the
descriptors the encoder computes y = R x (float32, ascending k, no fused
multiply-add), so codes and scales are bit-exact against the oracle's dense
encoder; decode and the prefill chunk rotate the query by R and the
compressed-tier output by R^T, within the attention tolerances.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import akv_oracle as O
from long_context_kv_split_amd import synth

from test_gpu_parity import _mods, _say, assert_attention, assert_codes
from test_gpu_step import _replay

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()


def _encoded(w, R, seqs=None):
    seqs = range(w.B) if seqs is None else seqs
    ek = {b: O.encode(w.quant_k_src[b], R) for b in seqs}
    ev = {b: O.encode(w.quant_v_src[b], R) for b in seqs}
    return ek, ev


@pytest.mark.parametrize("d", [64, 128])
def test_qr_compress_bit_exact(d):
    akv, harness = _mods()
    R = synth.qr_rotation(d, seed=d)
    w = synth.make_small("qr_enc", B=2, Hq=8, Hkv=2, d=d, quant=[1000, 777], exact=[64, 64], outlier_frac=0.02)
    _say(f"QR compress d={d}: quant {list(w.quant_len)}")
    dw = harness.DeviceWorkload(w, rotation=R)
    torch.cuda.synchronize()
    ek, ev = _encoded(w, R)
    assert_codes(dw, w, ek, ev, f"QR compress d={d}")
    # the Hadamard encoding of the same tokens differs (the rotation is used)
    hk = O.encode(w.quant_k_src[0])[0]
    assert not np.array_equal(hk, ek[0][0])


@pytest.mark.parametrize("cfg", [
    dict(B=2, Hq=32, Hkv=4, d=128, quant=[1000, 2500], exact=[300, 77], split_exact=128, split_quant=256),
    dict(B=3, Hq=32, Hkv=4, d=128, quant=[0, 130, 4000], exact=[1, 64, 700], split_exact=0, split_quant=0,
         outlier_frac=0.01),
    dict(B=2, Hq=4, Hkv=1, d=64, quant=[383, 64], exact=[129, 0], split_exact=64, split_quant=128),
    dict(B=2, Hq=32, Hkv=4, d=128, quant=[20000, 5000], exact=[1000, 300], split_exact=0, split_quant=0),
])
def test_qr_decode_parity(cfg):
    akv, harness = _mods()
    w = synth.make_small("qr_dec", **cfg)
    R = synth.qr_rotation(w.d, seed=3)
    _say(f"QR decode: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} quant={list(w.quant_len)} exact={list(w.exact_len)}")
    dw = harness.DeviceWorkload(w, rotation=R)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    ek, ev = _encoded(w, R, [b for b in range(w.B) if w.quant_len[b]])
    assert_codes(dw, w, ek, ev, "QR decode")
    o_ref, lse_ref = O.reference_outputs(w, [ek.get(b, O.encode(w.quant_k_src[b], R)) for b in range(w.B)],
                                         [ev.get(b, O.encode(w.quant_v_src[b], R)) for b in range(w.B)],
                                         rotation=R)
    assert_attention(o, lse, o_ref, lse_ref, "QR decode")
    # deterministic: a second call gives the same bytes
    o1, l1 = dw.o.clone(), dw.lse.clone()
    akv.check(dw.attend())
    torch.cuda.synchronize()
    assert torch.equal(o1, dw.o) and torch.equal(l1, dw.lse)


def test_qr_append_evict_steps():
    """Per-step append/evict with a QR rotation: evicted blocks are encoded with R."""
    akv, harness = _mods()
    W, S, d = 128, 40, 128
    R = synth.qr_rotation(d, seed=11)
    w = synth.make_small("qr_step", B=2, Hq=8, Hkv=2, d=d, quant=[100, 0], exact=[W + 60, W + 30],
                         reserve_quant=[2, 2])
    dw = harness.DeviceWorkload(w, rotation=R)
    nk, nv = synth.step_tokens(5, S, w.B, w.Hkv, d)
    dk = torch.from_numpy(nk.view(np.int16)).cuda()
    dv = torch.from_numpy(nv.view(np.int16)).cuda()
    for t in range(S):
        akv.check(akv.akv_append_evict(dw.append_desc(W, dk[t], dv[t]), harness.stream_handle()))
    torch.cuda.synchronize()
    dw.o.fill_(float("nan"))
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    for b in range(w.B):
        ek_, ev_, qk, qv = _replay(w, nk, nv, W, b, S)
        assert int(dw.quant_len[b].item()) == qk.shape[0] > 0
        kc, ks = O.encode(qk, R)
        vc, vs = O.encode(qv, R)
        ck, cks, cv, cvs = dw.read_codes(b, 0, qk.shape[0])
        assert np.array_equal(ck, kc) and np.array_equal(cks, ks), f"seq {b}: K codes / scales"
        assert np.array_equal(cv, vc) and np.array_equal(cvs, vs), f"seq {b}: V codes / scales"
        o_ref, lse_ref = O.decode_sequence(w.q[b], ek_, ev_, kc, ks, vc, vs, rotation=R)
        assert_attention(o[b], lse[b], o_ref, lse_ref, f"QR step seq {b}")


def test_qr_staged_equals_resident():
    akv, harness = _mods()
    d = 128
    R = synth.qr_rotation(d, seed=5)
    w = synth.make_small("qr_staged", B=2, Hq=8, Hkv=2, d=d, quant=[3000, 900], exact=[200, 70])
    dw = harness.DeviceWorkload(w, rotation=R)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o_res, l_res = dw.o.clone(), dw.lse.clone()
    keep, tiers = dw.host_tiers()
    slots, slot_bytes = 2, -(-12 * w.Hkv * 72 * d // 256) * 256
    ring = torch.empty(slots * slot_bytes, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    sd, hold = dw.staging(tiers, ring, slots, cs)
    dw.o.fill_(float("nan"))
    akv.check(akv.akv_attend_decode_staged(dw.desc(), sd, harness.ptr(dw.ws), dw.ws_bytes, harness.stream_handle()))
    torch.cuda.synchronize()
    assert torch.equal(dw.o, o_res) and torch.equal(dw.lse, l_res)
    _say("QR staged: bit-identical to resident")
    ek, ev = _encoded(w, R, range(w.B))
    o_ref, lse_ref = O.reference_outputs(w, [ek[b] for b in range(w.B)], [ev[b] for b in range(w.B)], rotation=R)
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "QR staged vs oracle")


@pytest.mark.parametrize("cfg", [
    # 160 rows: two row groups, the second ragged; several splits per tier
    dict(B=1, Hq=8, Hkv=2, d=128, quant=[1000], exact=[300], Tq=40, split_exact=128, split_quant=256),
    # G = 6 (a row group boundary inside a query's heads) and a sequence with
    # no compressed tier
    dict(B=2, Hq=12, Hkv=2, d=128, quant=[300, 0], exact=[65, 80], Tq=17, split_quant=64),
    # head dim 64, outlier channels
    dict(B=1, Hq=4, Hkv=1, d=64, quant=[383], exact=[129], Tq=33, split_exact=64, split_quant=128,
         outlier_frac=0.02),
    # one query (the chunk degenerates to decode; its queries are rotated one per workgroup)
    dict(B=2, Hq=32, Hkv=4, d=128, quant=[1500, 64], exact=[100, 1], Tq=1),
])
def test_qr_chunk_parity(cfg):
    akv, harness = _mods()
    cfg = dict(cfg)
    kw = {k: cfg.pop(k) for k in ("split_exact", "split_quant") if k in cfg}
    w = synth.make_small("qr_chunk", causal_tail=cfg["Tq"], **cfg)
    R = synth.qr_rotation(w.d, seed=5)
    _say(f"QR chunk: B={w.B} Tq={w.Tq} Hq={w.Hq} Hkv={w.Hkv} d={w.d} quant={list(w.quant_len)} "
         f"exact={list(w.exact_len)} {kw}")
    dw = harness.DeviceWorkload(w, rotation=R)
    akv.check(dw.attend(**kw))
    torch.cuda.synchronize()
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    ek, ev = _encoded(w, R)
    qs = [b for b in range(w.B) if w.quant_len[b]]
    assert_codes(dw, w, {b: ek[b] for b in qs}, {b: ev[b] for b in qs}, "QR chunk")
    o_ref, lse_ref = O.reference_outputs(w, [ek[b] for b in range(w.B)], [ev[b] for b in range(w.B)],
                                         rotation=R)
    assert_attention(o, lse, o_ref, lse_ref, f"QR chunk {cfg} {kw}")
    # deterministic: a second call gives the same bytes
    o1, l1 = dw.o.clone(), dw.lse.clone()
    akv.check(dw.attend(**kw))
    torch.cuda.synchronize()
    assert torch.equal(o1, dw.o) and torch.equal(l1, dw.lse)

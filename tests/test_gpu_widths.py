"""GPU parity of the compressed tier at code widths 2 and 3 (4- and 8-level
Lloyd-Max tables), through the C ABI.

Codes and fp16 scales bit-exact against the oracle's encoder at the same
width (read back through the width's documented byte layout); attention
within the method's tolerances against the oracle's float64 attention over
the dequantized history; the fused per-step append / evict, the host-staged
decode, the checkpoint and the prefill chunk (also with a QR rotation) work
at every width.
"""
import copy

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


def _enc(w, width, rotation=None):
    ek = {b: O.encode(w.quant_k_src[b], rotation, width) for b in range(w.B) if w.quant_len[b]}
    ev = {b: O.encode(w.quant_v_src[b], rotation, width) for b in range(w.B) if w.quant_len[b]}
    return ek, ev


def _ref(w, width, ek, ev, rotation=None):
    kk = [ek.get(b, O.encode(w.quant_k_src[b], rotation, width)) for b in range(w.B)]
    vv = [ev.get(b, O.encode(w.quant_v_src[b], rotation, width)) for b in range(w.B)]
    return O.reference_outputs(w, kk, vv, rotation=rotation, width=width)


@pytest.mark.parametrize("width", [2, 3])
@pytest.mark.parametrize("d", [64, 128])
def test_narrow_compress_bit_exact(width, d):
    akv, harness = _mods()
    w = synth.make_small("narrow_enc", B=2, Hq=8, Hkv=2, d=d, quant=[1000, 777], exact=[64, 64], outlier_frac=0.02)
    # an all-zero token (every group's scale 0 -> the lower middle code)
    w.quant_k_src[0][5] = 0
    w.quant_v_src[1][8] = 0
    _say(f"width {width} compress d={d}: quant {list(w.quant_len)}")
    dw = harness.DeviceWorkload(w, width=width)
    torch.cuda.synchronize()
    ek, ev = _enc(w, width)
    assert_codes(dw, w, ek, ev, f"width {width} d={d}")
    assert np.all(dw.read_codes(0)[0][5] == O.zero_code(width))


@pytest.mark.parametrize("width,cfg", [
    (2, dict(B=2, Hq=32, Hkv=4, d=128, quant=[1000, 2500], exact=[300, 77], split_exact=128, split_quant=256)),
    (3, dict(B=2, Hq=32, Hkv=4, d=128, quant=[1000, 2500], exact=[300, 77], split_exact=128, split_quant=256)),
    (3, dict(B=3, Hq=32, Hkv=4, d=128, quant=[0, 130, 4000], exact=[1, 64, 700], outlier_frac=0.01)),
    (2, dict(B=2, Hq=4, Hkv=1, d=64, quant=[383, 64], exact=[129, 0], split_exact=64, split_quant=128)),
    (3, dict(B=2, Hq=4, Hkv=1, d=64, quant=[383, 64], exact=[129, 0], split_exact=64, split_quant=128)),
    (3, dict(B=1, Hq=32, Hkv=4, d=128, quant=[20000], exact=[1000])),
])
def test_narrow_decode_parity(width, cfg):
    akv, harness = _mods()
    w = synth.make_small("narrow_dec", **cfg)
    _say(f"width {width} decode: B={w.B} Hq={w.Hq} d={w.d} quant={list(w.quant_len)} exact={list(w.exact_len)}")
    dw = harness.DeviceWorkload(w, width=width)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    ek, ev = _enc(w, width)
    assert_codes(dw, w, ek, ev, f"width {width} decode")
    o_ref, lse_ref = _ref(w, width, ek, ev)
    assert_attention(o, lse, o_ref, lse_ref, f"width {width} decode")
    o1, l1 = dw.o.clone(), dw.lse.clone()
    akv.check(dw.attend())
    torch.cuda.synchronize()
    assert torch.equal(o1, dw.o) and torch.equal(l1, dw.lse)


def test_narrow_with_qr_rotation():
    akv, harness = _mods()
    w = synth.make_small("narrow_qr", B=2, Hq=16, Hkv=2, d=128, quant=[1500, 600], exact=[200, 64])
    R = synth.qr_rotation(128, seed=9)
    dw = harness.DeviceWorkload(w, rotation=R, width=3)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    ek, ev = _enc(w, 3, R)
    assert_codes(dw, w, ek, ev, "width 3 + QR")
    o_ref, lse_ref = _ref(w, 3, ek, ev, R)
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "width 3 + QR")


@pytest.mark.parametrize("width,d", [(3, 128), (2, 64)])
def test_narrow_append_evict_steps(width, d):
    akv, harness = _mods()
    W, S = 128, 40
    w = synth.make_small("narrow_step", B=2, Hq=8, Hkv=2, d=d, quant=[100, 0], exact=[W + 60, W + 30],
                         reserve_quant=[2, 2])
    dw = harness.DeviceWorkload(w, width=width)
    nk, nv = synth.step_tokens(6, S, w.B, w.Hkv, d)
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
        kc, ks = O.encode(qk, None, width)
        vc, vs = O.encode(qv, None, width)
        ck, cks, cv, cvs = dw.read_codes(b, 0, qk.shape[0])
        assert np.array_equal(ck, kc) and np.array_equal(cks, ks), f"seq {b}: K codes / scales"
        assert np.array_equal(cv, vc) and np.array_equal(cvs, vs), f"seq {b}: V codes / scales"
        o_ref, lse_ref = O.decode_sequence(w.q[b], ek_, ev_, kc, ks, vc, vs, width=width)
        assert_attention(o[b], lse[b], o_ref, lse_ref, f"width {width} step seq {b}")


def test_narrow_staged_equals_resident():
    akv, harness = _mods()
    d, width = 128, 3
    w = synth.make_small("narrow_staged", B=2, Hq=8, Hkv=2, d=d, quant=[3000, 900], exact=[200, 70])
    dw = harness.DeviceWorkload(w, width=width)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o_res, l_res = dw.o.clone(), dw.lse.clone()
    keep, tiers = dw.host_tiers()
    assert keep[0].numel() == -(-3000 // 64) * w.Hkv * (16 * width + 8) * d
    slots, slot_bytes = 2, -(-12 * w.Hkv * (16 * width + 8) * d // 256) * 256
    ring = torch.empty(slots * slot_bytes, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    sd, hold = dw.staging(tiers, ring, slots, cs)
    for rep in range(2):
        dw.o.fill_(float("nan"))
        akv.check(akv.akv_attend_decode_staged(dw.desc(), sd, harness.ptr(dw.ws), dw.ws_bytes,
                                               harness.stream_handle()))
        torch.cuda.synchronize()
        assert torch.equal(dw.o, o_res) and torch.equal(dw.lse, l_res), f"staged call {rep}"
    _say("width 3 staged: bit-identical to resident, twice")
    ek, ev = _enc(w, width)
    o_ref, lse_ref = _ref(w, width, ek, ev)
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "width 3 staged vs oracle")


def test_narrow_checkpoint_round_trip():
    """Save at width 2, restore into another placement: identical attention and
    image; restoring the same image under a width-3 descriptor is refused."""
    akv, harness = _mods()
    w = synth.make_small("narrow_ckpt", B=2, Hq=8, Hkv=2, d=128, quant=[700, 300], exact=[200, 90])
    dw = harness.DeviceWorkload(w, width=2)
    w2 = copy.copy(w)
    rng = np.random.default_rng(3)
    t = w.quant_table.copy()
    valid = t >= 0
    t[valid] = rng.permutation(w.quant_pool_blocks).astype(np.int32)[: int(valid.sum())]
    w2.quant_table = t
    dw2 = harness.DeviceWorkload(w2, width=2, fill_quant=False)
    dw2.exact_len.zero_()
    dw2.quant_len.zero_()
    d = dw.context_desc()
    n = akv.akv_checkpoint_bytes(d)
    assert n == 512 + w.B * (dw.emax * 256 + dw.qmax * (16 * 2 + 8)) * w.Hkv * w.d
    img = torch.zeros(n, dtype=torch.uint8, device="cuda")
    akv.check(akv.akv_checkpoint_save(d, img.data_ptr(), harness.stream_handle()))
    akv.check(akv.akv_checkpoint_restore(dw2.context_desc(), img.data_ptr(), harness.stream_handle()))
    torch.cuda.synchronize()
    for x in (dw, dw2):
        akv.check(x.attend())
    torch.cuda.synchronize()
    assert torch.equal(dw.o, dw2.o) and torch.equal(dw.lse, dw2.lse)
    # the restored context against the oracle over the saved tokens
    ek, ev = _enc(w, 2)
    assert_codes(dw2, w2, ek, ev, "width 2 restored")
    o_ref, lse_ref = _ref(w, 2, ek, ev)
    assert_attention(dw2.o.cpu().numpy(), dw2.lse.cpu().numpy(), o_ref, lse_ref, "width 2 restored vs oracle")
    img2 = torch.zeros_like(img)
    akv.check(akv.akv_checkpoint_save(dw2.context_desc(), img2.data_ptr(), harness.stream_handle()))
    torch.cuda.synchronize()
    assert torch.equal(img, img2)
    # the header records the width: a width-3 restore of this image is refused
    dw3 = harness.DeviceWorkload(w2, width=3, fill_quant=False)
    akv.check(akv.akv_checkpoint_restore(dw3.context_desc(), img.data_ptr(), harness.stream_handle()))
    torch.cuda.synchronize()
    assert np.all(dw3.exact_len.cpu().numpy() == -1)
    _say("width 2 checkpoint: restored bit-identically; width mismatch refused")


@pytest.mark.parametrize("width", [2, 3])
@pytest.mark.parametrize("cfg", [
    # 160 rows: two row groups, the second ragged; several splits per tier
    dict(B=1, Hq=8, Hkv=2, d=128, quant=[1000], exact=[300], Tq=40, split_exact=128, split_quant=256),
    # head dim 64, a second sequence without a compressed tier
    dict(B=2, Hq=4, Hkv=1, d=64, quant=[383, 0], exact=[129, 70], Tq=33, split_exact=64, split_quant=128),
])
def test_narrow_chunk_parity(width, cfg):
    akv, harness = _mods()
    cfg = dict(cfg)
    kw = {k: cfg.pop(k) for k in ("split_exact", "split_quant") if k in cfg}
    w = synth.make_small("narrow_chunk", causal_tail=cfg["Tq"], outlier_frac=0.01, **cfg)
    _say(f"width {width} chunk: B={w.B} Tq={w.Tq} Hq={w.Hq} Hkv={w.Hkv} d={w.d} quant={list(w.quant_len)} "
         f"exact={list(w.exact_len)} {kw}")
    dw = harness.DeviceWorkload(w, width=width)
    akv.check(dw.attend(**kw))
    torch.cuda.synchronize()
    ek, ev = _enc(w, width)
    assert_codes(dw, w, ek, ev, f"width {width} chunk")
    o_ref, lse_ref = _ref(w, width, ek, ev)
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, f"width {width} chunk {cfg}")


def test_narrow_chunk_with_qr_rotation():
    akv, harness = _mods()
    R = synth.qr_rotation(128, seed=9)
    w = synth.make_small("narrow_chunk_qr", B=1, Hq=12, Hkv=2, d=128, quant=[700], exact=[90], Tq=20,
                         causal_tail=20)
    dw = harness.DeviceWorkload(w, rotation=R, width=3)
    akv.check(dw.attend(split_quant=128))
    torch.cuda.synchronize()
    ek, ev = _enc(w, 3, R)
    assert_codes(dw, w, ek, ev, "width 3 chunk, QR")
    o_ref, lse_ref = _ref(w, 3, ek, ev, R)
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, "width 3 chunk, QR")


@pytest.mark.slow
@pytest.mark.parametrize("width,qr", [(3, False), (2, False), (4, True)])
def test_hybrid128k_variants_kv_head_0(width, qr):
    """The bench's hybrid128k decode (123,904 compressed + 4,096 exact tokens,
    the library's own split plan) at a narrow width or with a QR rotation:
    codes of kv head 0 bit-exact, and the attention of its 8 query heads
    against the oracle over that kv head's whole history."""
    akv, harness = _mods()
    w = synth.make("hybrid128k")
    R = synth.qr_rotation(w.d, seed=0) if qr else None
    _say(f"hybrid128k width {width} qr {qr}: building")
    dw = harness.DeviceWorkload(w, rotation=R, width=width)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o, lse = dw.o.cpu().numpy(), dw.lse.cpu().numpy()
    kc, ks = O.encode(w.quant_k_src[0][:, :1], R, width)
    vc, vs = O.encode(w.quant_v_src[0][:, :1], R, width)
    gk, gks, gv, gvs = dw.read_codes(0)
    assert np.array_equal(gk[:, :1], kc) and np.array_equal(gks[:, :1], ks), "K codes / scales of kv head 0"
    assert np.array_equal(gv[:, :1], vc) and np.array_equal(gvs[:, :1], vs), "V codes / scales of kv head 0"
    G = w.Hq // w.Hkv
    o_ref, lse_ref = O.decode_sequence(w.q[0][:, :G], w.exact_k[0][:, :1], w.exact_v[0][:, :1], kc, ks, vc, vs,
                                       rotation=R, width=width)
    assert_attention(o[0][:, :G], lse[0][:, :G], o_ref, lse_ref, f"hybrid128k width {width} qr {qr} kv 0")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))

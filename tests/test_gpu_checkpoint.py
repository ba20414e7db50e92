"""GPU tests of the context checkpoint (akv_checkpoint_save / _restore).

The image depends only on the tokens, so a context saved from one block
placement and restored into another (zeroed) placement must hold the saved
tokens (codes and scales bit-exact against the oracle's encoding), attend
within the decode tolerances of the float64 oracle over them and bit for bit
like the original, save back to the same bytes, and keep doing so through
further append / evict steps (replayed by the oracle).  A damaged header or a
bad table entry turns the affected sequences' attention into NaN.
"""
import copy

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_kv_split_amd import synth

from oracle import akv_oracle as O
from test_gpu_parity import _mods, _say, assert_attention, assert_codes, oracle_case
from test_gpu_step import _replay

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()


def _other_placement(w, seed):
    """Same tokens and table shapes, every valid table entry moved to another pool block."""
    rng = np.random.default_rng(seed)
    c = copy.copy(w)
    for name, nblk in (("exact_table", w.exact_pool_blocks), ("quant_table", w.quant_pool_blocks)):
        t = getattr(w, name).copy()
        valid = t >= 0
        t[valid] = rng.permutation(nblk).astype(np.int32)[: int(valid.sum())]
        setattr(c, name, t)
    return c


def _blank(dw):
    for t in (dw.pools[0].ek, dw.pools[0].ev, dw.pools[0].kc, dw.pools[0].vc, dw.pools[0].ks, dw.pools[0].vs):
        t.zero_()
    dw.exact_len.zero_()
    dw.quant_len.zero_()


def _attend(dw):
    akv, _ = _mods()
    dw.o.fill_(float("nan"))
    akv.check(dw.attend())
    torch.cuda.synchronize()
    return dw.o.clone(), dw.lse.clone()


def _save(dw):
    akv, harness = _mods()
    d = dw.context_desc()
    n = akv.akv_checkpoint_bytes(d)
    assert n > 0, akv.akv_last_error()
    img = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    akv.check(akv.akv_checkpoint_save(d, img.data_ptr(), harness.stream_handle()))
    torch.cuda.synchronize()
    return img


def _restore(dw, img):
    akv, harness = _mods()
    akv.check(akv.akv_checkpoint_restore(dw.context_desc(), img.data_ptr(), harness.stream_handle()))
    torch.cuda.synchronize()


def _pair(d=128):
    akv, harness = _mods()
    w = synth.make_small("ckpt", B=3, Hq=8, Hkv=2, d=d, quant=[700, 300, 0], exact=[200, 90, 130],
                         reserve_exact=[1, 1, 1], reserve_quant=[2, 2, 2])
    dw = harness.DeviceWorkload(w)
    w2 = _other_placement(w, 7)
    dw2 = harness.DeviceWorkload(w2)
    _blank(dw2)
    return w, dw, w2, dw2


@pytest.mark.parametrize("d", [128, 64])
def test_restore_into_another_placement_is_bit_identical(d):
    w, dw, w2, dw2 = _pair(d)
    o1, l1 = _attend(dw)
    img = _save(dw)
    _restore(dw2, img)
    assert torch.equal(dw2.exact_len, dw.exact_len) and torch.equal(dw2.quant_len, dw.quant_len)
    o2, l2 = _attend(dw2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "restored context attends differently"
    img2 = _save(dw2)
    assert torch.equal(img, img2), "image depends on the block placement"
    _say(f"checkpoint d={d}: {img.numel()} bytes, restore bit-identical, image placement-free")
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw2, w2, {b: ek[b] for b in range(w.B) if w.quant_len[b]},
                 {b: ev[b] for b in range(w.B) if w.quant_len[b]}, f"restored d={d}")
    assert_attention(o2.cpu().numpy(), l2.cpu().numpy(), o_ref, lse_ref, f"restored d={d} vs oracle")


def test_restore_then_steps_stay_identical():
    akv, harness = _mods()
    w, dw, w2, dw2 = _pair()
    W = 128
    nk, nv = synth.step_tokens(3, 20, w.B, w.Hkv, w.d)
    dk = torch.from_numpy(nk.view(np.int16)).cuda()
    dv = torch.from_numpy(nv.view(np.int16)).cuda()
    for t in range(10):
        akv.check(akv.akv_append_evict(dw.append_desc(W, dk[t], dv[t]), harness.stream_handle()))
    _restore(dw2, _save(dw))
    for t in range(10, 20):
        for x in (dw, dw2):
            akv.check(akv.akv_append_evict(x.append_desc(W, dk[t], dv[t]), harness.stream_handle()))
    torch.cuda.synchronize()
    assert torch.equal(dw.exact_len, dw2.exact_len) and torch.equal(dw.quant_len, dw2.quant_len)
    o1, l1 = _attend(dw)
    o2, l2 = _attend(dw2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _say(f"checkpoint mid-stream: lengths {dw.exact_len.tolist()} / {dw.quant_len.tolist()}, identical after 10 more steps")
    # the restored-and-stepped context against the oracle's replay of all 20 steps
    o, lse = o2.cpu().numpy(), l2.cpu().numpy()
    for b in range(w.B):
        ek, ev, qk, qv = _replay(w, nk, nv, W, b, 20)
        assert (int(dw2.exact_len[b].item()), int(dw2.quant_len[b].item())) == (ek.shape[0], qk.shape[0])
        gk, gv = dw2.read_exact(b)
        assert np.array_equal(gk, ek) and np.array_equal(gv, ev), f"seq {b}: exact tier bytes"
        kc, ks = O.encode(qk)
        vc, vs = O.encode(qv)
        if qk.shape[0]:
            ck, cks, cv, cvs = dw2.read_codes(b, 0, qk.shape[0])
            assert np.array_equal(ck, kc) and np.array_equal(cks, ks), f"seq {b}: K codes / scales"
            assert np.array_equal(cv, vc) and np.array_equal(cvs, vs), f"seq {b}: V codes / scales"
        o_ref, lse_ref = O.decode_sequence(w.q[b], ek, ev, kc, ks, vc, vs)
        assert_attention(o[b], lse[b], o_ref, lse_ref, f"restored + stepped seq {b} vs oracle")


def test_damaged_image_or_table_gives_nan():
    akv, harness = _mods()
    w, dw, w2, dw2 = _pair()
    o1, _ = _attend(dw)
    img = _save(dw)
    bad = img.clone()
    bad[0] ^= 0xFF                    # header magic
    _restore(dw2, bad)
    assert (dw2.exact_len == -1).all()
    o, lse = _attend(dw2)
    assert torch.isnan(o).all() and torch.isnan(lse).all()
    # a table entry of sequence 1 outside the pool: only sequence 1 is refused
    t = dw2.quant_table.clone()
    t[1, 0] = 10 ** 6
    dw2.quant_table.copy_(t)
    _restore(dw2, img)
    lens = dw2.exact_len.tolist()
    assert lens[1] == -1 and lens[0] == int(w.exact_len[0]) and lens[2] == int(w.exact_len[2])
    o, lse = _attend(dw2)
    assert torch.isnan(o[1]).all() and torch.equal(o[0], o1[0]) and torch.equal(o[2], o1[2])

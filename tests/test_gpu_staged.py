"""GPU tests of the host-staged decode (akv_attend_decode_staged).

The compressed tier is copied to pinned host memory in token order and
streamed back through a small device ring on a second stream.  The staged
call must meet the decode tolerances against the float64 oracle over the same
history, and since it runs the same splits, arithmetic and merge as
akv_attend_decode, its outputs must also be bit-identical to the resident
call's (and to themselves on a second call that reuses the ring).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_kv_split_amd import synth

from test_gpu_parity import _mods, _say, assert_attention, assert_codes, oracle_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()


@pytest.mark.parametrize("d,slot_blocks", [(128, 9), (64, 40)])
def test_staged_equals_resident(d, slot_blocks):
    akv, harness = _mods()
    w = synth.make_small("staged", B=3, Hq=8, Hkv=2, d=d, quant=[5000, 1800, 0], exact=[300, 140, 70])
    dw = harness.DeviceWorkload(w)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o_res, l_res = dw.o.clone(), dw.lse.clone()
    plan = akv.akv_split_plan(dw.desc())
    keep, tiers = dw.host_tiers()
    block_bytes = w.Hkv * 72 * d
    slots = 3
    slot_bytes = -(-slot_blocks * block_bytes // 256) * 256
    ring = torch.empty(slots * slot_bytes, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    sd, hold = dw.staging(tiers, ring, slots, cs)
    _say(f"staged d={d}: splits {plan['split_tokens_quant']} tokens, slot {slot_blocks} blocks x {slots}")
    for rep in range(2):
        dw.o.fill_(float("nan"))
        akv.check(akv.akv_attend_decode_staged(dw.desc(), sd, harness.ptr(dw.ws), dw.ws_bytes,
                                               harness.stream_handle()))
        torch.cuda.synchronize()
        assert torch.equal(dw.o, o_res) and torch.equal(dw.lse, l_res), f"staged call {rep} differs from resident"
    _say(f"staged d={d}: bit-identical to resident, twice")
    o_ref, lse_ref, ek, ev = oracle_case(w)
    assert_codes(dw, w, {b: ek[b] for b in range(w.B) if w.quant_len[b]},
                 {b: ev[b] for b in range(w.B) if w.quant_len[b]}, f"staged d={d}")
    assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, f"staged d={d} vs oracle")


def test_staged_ring_too_small_is_refused():
    akv, harness = _mods()
    w = synth.make_small("staged_small", B=1, Hq=8, Hkv=2, d=128, quant=[2000], exact=[100])
    dw = harness.DeviceWorkload(w)
    plan = akv.akv_split_plan(dw.desc())
    keep, tiers = dw.host_tiers()
    need = plan["split_tokens_quant"] // 64 * w.Hkv * 72 * 128
    ring = torch.empty(2 * (need - 256), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    sd, hold = dw.staging(tiers, ring, 2, cs)
    dw.ensure_ws(dw.desc())
    st = akv.akv_attend_decode_staged(dw.desc(), sd, harness.ptr(dw.ws), dw.ws_bytes, harness.stream_handle())
    assert st == akv.AKV_ERR_WORKSPACE, akv.akv_last_error()

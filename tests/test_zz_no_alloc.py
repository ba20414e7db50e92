"""GPU test of akv_attend_decode_noalloc, the decode entry point that allocates nothing.

It runs akv_attend_decode's validation and kernels with the partials in the
library's own device array instead of a caller's workspace, so its outputs
must equal akv_attend_decode's bit for bit (and so meet the oracle's
tolerances).  Two calls in a row, the second on a smaller input, check that
what the first call left in the shared array does not reach the second.
"""
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


def _both(w):
    """akv_attend_decode (with a workspace), then akv_attend_decode_noalloc on
    the same descriptor; returns the device workload and the first outputs."""
    akv, harness = _mods()
    dw = harness.DeviceWorkload(w)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o_ws, l_ws = dw.o.clone(), dw.lse.clone()
    dw.o.fill_(float("nan"))
    dw.lse.fill_(float("nan"))
    akv.check(akv.akv_attend_decode_noalloc(dw.desc(), harness.stream_handle()))
    torch.cuda.synchronize()
    return dw, o_ws, l_ws


def test_noalloc_decode_equals_workspace_decode_twice():
    big = synth.make_small("noalloc_big", B=2, Hq=32, Hkv=4, d=128, quant=[20000, 9000], exact=[2048, 700],
                           outlier_frac=0.01)
    small = synth.make_small("noalloc_small", B=1, Hq=8, Hkv=2, d=64, quant=[1000], exact=[130])
    for w in (big, small):
        _say(f"noalloc {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} quant={list(w.quant_len)} "
             f"exact={list(w.exact_len)}")
        dw, o_ws, l_ws = _both(w)
        assert torch.equal(dw.o, o_ws) and torch.equal(dw.lse, l_ws), f"{w.name}: differs from akv_attend_decode"
        o_ref, lse_ref, _, _ = oracle_case(w)
        assert_attention(dw.o.cpu().numpy(), dw.lse.cpu().numpy(), o_ref, lse_ref, f"noalloc {w.name} vs oracle")


def test_noalloc_decode_in_a_captured_graph():
    """The entry point's purpose: a decode that a HIP graph can capture.  The
    first call on the device (the array's address lookup) runs eagerly, one
    call is captured, and every replay, with eager decodes and
    synchronizations between the replays, must equal the workspace decode."""
    akv, harness = _mods()
    w = synth.make_small("noalloc_graph", B=2, Hq=32, Hkv=4, d=128, quant=[3000, 700], exact=[300, 64])
    _say(f"noalloc graph: B={w.B} quant={list(w.quant_len)} exact={list(w.exact_len)}")
    dw = harness.DeviceWorkload(w)
    akv.check(dw.attend())
    torch.cuda.synchronize()
    o_ref, l_ref = dw.o.clone(), dw.lse.clone()
    desc = dw.desc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        akv.check(akv.akv_attend_decode_noalloc(desc, side.cuda_stream))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = akv.akv_attend_decode_noalloc(desc, torch.cuda.current_stream().cuda_stream)
    assert st == 0, akv.akv_last_error()
    for r in range(4):
        dw.o.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.o, o_ref) and torch.equal(dw.lse, l_ref), f"replay {r} differs from the workspace decode"
        akv.check(dw.attend())  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(dw.o, o_ref) and torch.equal(dw.lse, l_ref)
    _say("noalloc graph: 4 replays equal to the workspace decode")

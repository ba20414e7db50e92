"""HIP-graph capture of the decode paths (a serving loop captures a step once).

The entry points enqueue kernels only: no allocation, copy, memset or
synchronization.  A captured call must therefore give, on every replay, the
bytes an eager call gives on the same inputs, and it must read its inputs at
replay time (a query changed between replays is seen).  A captured step of
append/evict + decode, fed through fixed staging buffers, must track an eager
twin bit for bit, step after step, and end in the oracle's state.  Eager work
and synchronizations run between the replays.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from long_context_kv_split_amd import synth

from test_gpu_parity import _mods, _say
from test_gpu_step import _check_state

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    _mods()


def _capture(fn):
    """Run fn(stream) once on a side stream, then capture one call into a graph."""
    akv, _ = _mods()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        akv.check(fn(side.cuda_stream))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = fn(torch.cuda.current_stream().cuda_stream)
    assert st == 0, akv.akv_last_error()
    return g


def _replays_match(g, dw, o_ref, l_ref, n, label):
    for r in range(n):
        dw.o.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.o, o_ref) and torch.equal(dw.lse, l_ref), f"{label}: replay {r} differs from eager"


@pytest.mark.parametrize("qr", [False, True])
def test_decode_graph_replays(qr):
    akv, harness = _mods()
    w = synth.make_small("graph_dec", B=2, Hq=32, Hkv=4, d=128, quant=[3000, 700], exact=[300, 64])
    dw = harness.DeviceWorkload(w, rotation=synth.qr_rotation(128, seed=2) if qr else None)
    desc = dw.desc()
    dw.ensure_ws(desc)

    def call(h):
        return akv.akv_attend_decode(desc, harness.ptr(dw.ws), dw.ws_bytes, h)

    akv.check(call(harness.stream_handle()))
    torch.cuda.synchronize()
    o_ref, l_ref = dw.o.clone(), dw.lse.clone()
    g = _capture(call)
    _replays_match(g, dw, o_ref, l_ref, 3, f"decode qr={qr}")
    # the replay reads the query at replay time: permute the heads, compare
    # with an eager call on the new query
    dw.q.copy_(dw.q.flip(-2).clone())
    akv.check(call(harness.stream_handle()))
    torch.cuda.synchronize()
    o_new, l_new = dw.o.clone(), dw.lse.clone()
    assert not torch.equal(o_new, o_ref)
    _replays_match(g, dw, o_new, l_new, 2, f"decode qr={qr}, new query")
    _say(f"decode graph (qr={qr}): 5 replays bit-identical to eager")


@pytest.mark.parametrize("variant", ["hadamard", "qr_width3"])
def test_chunk_graph_replays(variant):
    akv, harness = _mods()
    w = synth.make_small("graph_chunk", B=1, Hq=8, Hkv=2, d=128, quant=[700], exact=[300], causal_tail=96)
    if variant == "hadamard":
        dw = harness.DeviceWorkload(w)
    else:  # the rotated-query kernel, the R^T merge and the 3-bit staging inside the capture
        dw = harness.DeviceWorkload(w, rotation=synth.qr_rotation(128, seed=4), width=3)
    desc = dw.desc()
    dw.ensure_ws(desc, chunk=True)

    def call(h):
        return akv.akv_attend_chunk(desc, harness.ptr(dw.ws), dw.ws_bytes, h)

    akv.check(call(harness.stream_handle()))
    torch.cuda.synchronize()
    o_ref, l_ref = dw.o.clone(), dw.lse.clone()
    assert torch.isfinite(o_ref).all()
    g = _capture(call)
    _replays_match(g, dw, o_ref, l_ref, 3, f"chunk {variant}")
    _say(f"chunk graph ({variant}): 3 replays bit-identical to eager")


def test_serving_step_graph_tracks_eager():
    """append/evict + decode captured once, fed from fixed staging buffers."""
    akv, harness = _mods()
    W, S, d = 128, 40, 128
    w = synth.make_small("graph_step", B=2, Hq=8, Hkv=2, d=d, quant=[100, 0], exact=[W + 60, W + 30],
                         reserve_quant=[2, 2])
    dg = harness.DeviceWorkload(w)  # driven by the graph
    de = harness.DeviceWorkload(w)  # eager twin
    nk, nv = synth.step_tokens(7, S, w.B, w.Hkv, d)
    dk = torch.from_numpy(nk.view(np.int16)).cuda()
    dv = torch.from_numpy(nv.view(np.int16)).cuda()
    kbuf, vbuf = torch.empty_like(dk[0]), torch.empty_like(dv[0])
    adesc = dg.append_desc(W, kbuf, vbuf)
    ddesc = dg.desc()
    dg.ensure_ws(ddesc)
    de.ensure_ws(de.desc())

    def step(h):
        st = akv.akv_append_evict(adesc, h)
        return st if st else akv.akv_attend_decode(ddesc, harness.ptr(dg.ws), dg.ws_bytes, h)

    # the kernels run once, eagerly, on a throwaway copy before the capture
    # (a warm-up call on dg itself would append a token)
    dwarm = harness.DeviceWorkload(w)
    akv.check(akv.akv_append_evict(dwarm.append_desc(W, dk[0], dv[0]), harness.stream_handle()))
    akv.check(dwarm.attend())
    torch.cuda.synchronize()
    del dwarm
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st = step(torch.cuda.current_stream().cuda_stream)
    assert st == 0, akv.akv_last_error()
    for t in range(S):
        kbuf.copy_(dk[t])
        vbuf.copy_(dv[t])
        g.replay()
        akv.check(akv.akv_append_evict(de.append_desc(W, dk[t], dv[t]), harness.stream_handle()))
        akv.check(de.attend())
        torch.cuda.synchronize()
        assert torch.equal(dg.exact_len, de.exact_len) and torch.equal(dg.quant_len, de.quant_len), f"step {t}"
        assert torch.equal(dg.o, de.o) and torch.equal(dg.lse, de.lse), f"step {t}: graph output differs"
    _check_state(dg, w, nk, nv, W, S, "graph step")
    _say(f"serving step graph: {S} replays bit-identical to the eager twin")

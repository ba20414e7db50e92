"""C-ABI contract tests that need no GPU.

The library validates every argument on the host before anything is
enqueued, in the fixed order NULL -> SHAPE -> UNSUPPORTED -> ALIGN ->
WORKSPACE, so each refusal here returns without any HIP call.  Pointers are
fake (never dereferenced on the host).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from long_context_kv_split_amd import akv

FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def good_desc(**over):
    e = akv.ExactTier(k=FAKE, v=FAKE + 0x1000000, block_table=FAKE + 0x2000000, lengths=FAKE + 0x2100000,
                      max_blocks=64, num_blocks=64)
    q = akv.QuantTier(k_codes=FAKE + 0x3000000, v_codes=FAKE + 0x4000000, k_scales=FAKE + 0x5000000,
                      v_scales=FAKE + 0x5800000, block_table=FAKE + 0x6000000, lengths=FAKE + 0x6100000,
                      max_blocks=1936, num_blocks=1936)
    kw = dict(B=1, Hq=32, Hkv=4, d=128, Tq=1, softmax_scale=0.0, q=FAKE + 0x7000000, exact=e, quant=q,
              split_tokens_exact=0, split_tokens_quant=0, o=FAKE + 0x8000000, lse=FAKE + 0x9000000)
    kw.update(over)
    return akv.AttnDesc(**kw)


def call(desc, ws=FAKE + 0xA000000, ws_bytes=None, chunk=False):
    if ws_bytes is None:
        ws_bytes = 1 << 40
    fn = akv.akv_attend_chunk if chunk else akv.akv_attend_decode
    return fn(desc, ws, ws_bytes, 0)


def test_abi_version_and_exports():
    assert akv.akv_abi_version() == 1
    names = akv.header_functions()
    assert set(names) == {"akv_abi_version", "akv_last_error", "akv_decode_workspace_bytes",
                          "akv_chunk_workspace_bytes", "akv_attend_decode", "akv_attend_chunk",
                          "akv_split_plan", "akv_lse_merge", "akv_compress_evicted", "akv_append_evict",
                          "akv_checkpoint_bytes", "akv_checkpoint_save", "akv_checkpoint_restore",
                          "akv_attend_decode_staged", "akv_attend_decode_noalloc",
                          "akv_decode_split_workgroups"}
    for n in names:
        assert hasattr(akv.LIB, n), n


def test_exports_via_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", akv.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (akv_\w+)", out))
    assert set(akv.header_functions()) <= syms


def test_workspace_bytes_hybrid128k_shape():
    d = good_desc()
    # splits: quant ceil(1936*64/1024) = 121, exact 7 of 640 tokens -> 128 splits
    rows = 1 * 4 * 128 * 1 * 8
    po = (rows * 128 * 4 + 255) // 256 * 256
    assert akv.akv_decode_workspace_bytes(d) == po + rows * 4
    assert akv.akv_decode_workspace_bytes(good_desc(d=96)) == 0


def test_chunk_split_planner_c5_shape():
    # 512 queries x 8 heads per kv head = 32 row groups of 128; 4 kv heads ->
    # 128 units, so each tier is cut into ceil(512 / 128) = 4 runs of blocks
    e = akv.ExactTier(k=FAKE, v=FAKE + 0x1000000, block_table=FAKE + 0x2000000, lengths=FAKE + 0x2100000,
                      max_blocks=72, num_blocks=72)
    q = good_desc().quant
    q.max_blocks = q.num_blocks = 456
    d = good_desc(Tq=512, exact=e, quant=q)
    # exact: 18 blocks = 1152 tokens -> 4 splits; compressed: 114 blocks = 7296 -> 4 splits
    rows = 1 * 4 * (4 + 4) * 512 * 8
    assert akv.akv_chunk_workspace_bytes(d) == rows * 128 * 4 + rows * 4
    # explicit sizes still win
    d2 = good_desc(Tq=512, exact=e, quant=q, split_tokens_exact=4608, split_tokens_quant=29184)
    rows = 1 * 4 * 2 * 512 * 8
    assert akv.akv_chunk_workspace_bytes(d2) == rows * 128 * 4 + rows * 4
    # the decode rule on the same shape: 114 compressed splits of 256 and 12
    # exact splits of 384 tokens (one round of 504 workgroups)
    assert akv.akv_decode_workspace_bytes(good_desc(exact=e, quant=q)) == (4 * (114 + 12) * 8) * 516
    # a small chunk still gets whole-block splits, never above the maximum
    d3 = good_desc(Tq=1, Hq=4, Hkv=1, exact=e, quant=q)
    rows = 1 * 1 * (72 + 456) * 1 * 4      # 512 runs wanted -> one block per split
    assert akv.akv_chunk_workspace_bytes(d3) == (rows * 128 * 4 + 255) // 256 * 256 + rows * 4


def _plan(chunk=False, **over):
    p = akv.akv_split_plan(good_desc(**over), chunk)
    return p["split_tokens_quant"], p["split_tokens_exact"], p["splits_quant"], p["splits_exact"]


def _tiers(qblocks, eblocks):
    q = good_desc().quant
    q.max_blocks = q.num_blocks = qblocks
    e = good_desc().exact
    e.max_blocks = e.num_blocks = eblocks
    return dict(quant=q, exact=e)


def test_decode_split_planner():
    """One round of <= 512 workgroups when the shape allows it, else compressed
    splits sized for about 2,048 workgroups (at least 1,024 tokens)."""
    # 1 sequence x 4 kv heads, 123,904 + 4,096 tokens: 4 * (121 + 7) = 512 workgroups
    assert _plan() == (1024, 640, 121, 7)
    # exact tier only, 32,768 tokens: 128 splits of 256 tokens per kv head
    assert _plan(**_tiers(0, 512)) == (256, 256, 0, 128)
    # 32 sequences (tables of 1,024 + 32 blocks): no single round; compressed
    # splits for about 2,048 workgroups, ceil(65,536 * 128 / 2,048) = 4,096
    # tokens (16 splits), the exact tier at its default
    assert _plan(B=32, **_tiers(1024, 32)) == (4096, 1024, 16, 2)
    # the ragged batch's tables (880 + 32 blocks): 56,320 * 128 / 2,048 = 3,520 -> 3,584
    assert _plan(B=32, **_tiers(880, 32)) == (3584, 1024, 16, 2)
    # never below the 1,024-token default: 8 sequences of 16,384 compressed tokens
    # (512 / 32 = 16 slots per kv head, 768-token splits need 22)
    assert _plan(B=8, **_tiers(256, 32)) == (1024, 1024, 16, 2)
    # 4 query heads on 1 kv head, 384 + 128 tokens: the smallest splits
    assert _plan(Hq=4, Hkv=1, d=64, **_tiers(6, 2)) == (256, 256, 2, 1)
    # a 28,672 + 4,608-token history: 256-token compressed splits leave 16 slots
    assert _plan(**_tiers(448, 72)) == (256, 320, 112, 15)
    # explicit sizes win, and the other tier fills what is left
    assert _plan(split_tokens_quant=2048) == (2048, 256, 61, 16)
    assert _plan(split_tokens_exact=2048) == (1024, 2048, 121, 2)
    # the chunk keeps its own rule
    assert _plan(True, Tq=512, **_tiers(456, 72)) == (7296, 1152, 4, 4)
    for tq, tiers in ((1, _tiers(1936, 64)), (1, _tiers(0, 512))):
        p = akv.akv_split_plan(good_desc(Tq=tq, **tiers))
        assert 4 * (p["splits_quant"] + p["splits_exact"]) <= 512
    with pytest.raises(akv.AKVError):
        akv.akv_split_plan(good_desc(d=96))


def test_decode_sub_splits_for_small_grids():
    """A grid with fewer workgroups than compute units attends each split with
    several workgroups; the caller's partition (the split plan) is unchanged."""
    ex = _tiers(0, 512)   # 32,768 exact tokens on 4 kv heads
    d = good_desc(split_tokens_exact=2048, **ex)
    assert _plan(split_tokens_exact=2048, **ex) == (256, 2048, 0, 16)
    assert akv.akv_decode_split_workgroups(d) == 4          # 4 x 16 x 4 = 256 workgroups of 512 tokens
    rows = 4 * 64 * 8
    assert akv.akv_decode_workspace_bytes(d) == rows * 128 * 4 + rows * 4
    # 8 splits of 4,096: 8 workgroups each (256 workgroups of 512 tokens)
    assert akv.akv_decode_split_workgroups(good_desc(split_tokens_exact=4096, **ex)) == 8
    # the default plans already fill the GPU, and small splits are never cut
    assert akv.akv_decode_split_workgroups(good_desc()) == 1
    assert akv.akv_decode_split_workgroups(good_desc(**ex)) == 1
    tiny = dict(Hq=4, Hkv=1, d=64, split_tokens_quant=384, split_tokens_exact=128, **_tiers(6, 2))
    assert akv.akv_decode_split_workgroups(good_desc(**tiny)) == 1
    assert _plan(**tiny) == (384, 128, 1, 1)
    # a split whose blocks do not cut into equal runs of >= 4 blocks stays whole
    assert akv.akv_decode_split_workgroups(good_desc(split_tokens_exact=1920, **ex)) == 1
    assert akv.akv_decode_split_workgroups(good_desc(d=96)) == 0


def test_null_checks_first():
    assert akv.LIB.akv_attend_decode(None, None, 0, None) == akv.AKV_ERR_NULL
    assert call(good_desc(q=0)) == akv.AKV_ERR_NULL
    assert "q, o or lse" in akv.akv_last_error()
    e = good_desc().exact
    e.k = 0
    assert call(good_desc(exact=e)) == akv.AKV_ERR_NULL
    # NULL beats SHAPE beats UNSUPPORTED
    assert call(good_desc(q=0, Hq=33, d=96)) == akv.AKV_ERR_NULL
    assert call(good_desc(Hq=33, d=96)) == akv.AKV_ERR_SHAPE
    assert call(good_desc(d=96, q=FAKE + 2)) == akv.AKV_ERR_UNSUPPORTED


def test_noalloc_validation_and_size_limit():
    """The allocation-free decode validates like akv_attend_decode, then refuses
    a shape whose partials exceed the library's fixed scratch (nothing is
    enqueued, so no GPU is needed)."""
    f = lambda d: akv.akv_attend_decode_noalloc(d, 0)
    assert akv.LIB.akv_attend_decode_noalloc(None, None) == akv.AKV_ERR_NULL
    assert f(good_desc(q=0)) == akv.AKV_ERR_NULL
    assert f(good_desc(Hq=33)) == akv.AKV_ERR_SHAPE
    assert f(good_desc(d=96)) == akv.AKV_ERR_UNSUPPORTED
    assert f(good_desc(q=FAKE + 2)) == akv.AKV_ERR_ALIGN
    tiers = dict(quant=good_desc().quant, exact=good_desc().exact)
    tiers["quant"].max_blocks = tiers["quant"].num_blocks = 1024
    tiers["exact"].max_blocks = tiers["exact"].num_blocks = 32
    big = good_desc(B=64, split_tokens_quant=1024, **tiers)  # 64 * 4 * (64 + 2) * 8 partial rows
    assert akv.akv_decode_workspace_bytes(big) > akv.NOALLOC_SCRATCH_BYTES
    assert f(big) == akv.AKV_ERR_WORKSPACE
    assert "scratch" in akv.akv_last_error()


def test_absent_tier_may_be_null():
    q = akv.QuantTier()  # all zero: absent
    d = good_desc(quant=q)
    assert call(d, ws=0) == akv.AKV_ERR_WORKSPACE  # everything else valid


def test_shape_errors():
    for over in (dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Tq=0), dict(Hq=30), dict(softmax_scale=-1.0),
                 dict(softmax_scale=float("inf")), dict(split_tokens_exact=100), dict(split_tokens_quant=-64)):
        assert call(good_desc(**over)) == akv.AKV_ERR_SHAPE, over
    assert call(good_desc(exact=akv.ExactTier(), quant=akv.QuantTier())) == akv.AKV_ERR_SHAPE
    d = good_desc()
    d.struct_size = 8
    assert call(d) == akv.AKV_ERR_SHAPE


def test_unsupported():
    assert call(good_desc(d=256)) == akv.AKV_ERR_UNSUPPORTED
    assert call(good_desc(split_tokens_quant=65536)) == akv.AKV_ERR_UNSUPPORTED
    assert call(good_desc(split_tokens_quant=64), ws=0) == akv.AKV_ERR_WORKSPACE  # 1940 splits: served
    q = good_desc().quant
    q.max_blocks = 2100
    q.num_blocks = 2100
    assert call(good_desc(quant=q, split_tokens_quant=64)) == akv.AKV_ERR_UNSUPPORTED  # 2104 splits

    assert call(good_desc(Hq=64, Hkv=4)) == akv.AKV_ERR_UNSUPPORTED  # G = 16
    assert call(good_desc(Tq=2)) == akv.AKV_ERR_UNSUPPORTED          # decode is one query
    assert call(good_desc(Tq=513), chunk=True) == akv.AKV_ERR_UNSUPPORTED
    assert call(good_desc(Tq=4, exact=akv.ExactTier()), chunk=True) == akv.AKV_ERR_UNSUPPORTED
    # workspace sizes that would approach the size_t range are refused, not wrapped
    huge = good_desc(B=65535, Hkv=65535, Hq=8 * 65535, split_tokens_quant=1024)  # 2^32 * 125 * 8 rows
    assert call(huge) == akv.AKV_ERR_UNSUPPORTED
    assert akv.akv_decode_workspace_bytes(huge) == 0
    assert call(good_desc(B=65535, Hkv=8000, Hq=8 * 8000, Tq=512), chunk=True) == akv.AKV_ERR_UNSUPPORTED


def test_alignment():
    assert call(good_desc(q=FAKE + 8)) == akv.AKV_ERR_ALIGN
    assert call(good_desc(o=FAKE + 2)) == akv.AKV_ERR_ALIGN
    e = good_desc().exact
    e.v = FAKE + 4
    assert call(good_desc(exact=e)) == akv.AKV_ERR_ALIGN
    q = good_desc().quant
    q.k_scales = FAKE + 8
    assert call(good_desc(quant=q)) == akv.AKV_ERR_ALIGN


def test_workspace_last():
    d = good_desc()
    need = akv.akv_decode_workspace_bytes(d)
    assert call(d, ws=0) == akv.AKV_ERR_WORKSPACE
    assert call(d, ws=FAKE + 16) == akv.AKV_ERR_WORKSPACE
    assert call(d, ws_bytes=need - 1) == akv.AKV_ERR_WORKSPACE
    assert "needed" in akv.akv_last_error()
    # an alignment problem is reported before the workspace problem
    assert call(good_desc(q=FAKE + 8), ws=0) == akv.AKV_ERR_ALIGN


def test_lse_merge_validation():
    f = akv.akv_lse_merge
    assert f(0, FAKE, 2, 3, 4, FAKE, FAKE, 0) == akv.AKV_ERR_NULL
    assert f(FAKE, FAKE, 0, 3, 4, FAKE, FAKE, 0) == akv.AKV_ERR_SHAPE
    assert f(FAKE, FAKE, 5000, 3, 4, FAKE, FAKE, 0) == akv.AKV_ERR_UNSUPPORTED
    assert f(FAKE + 2, FAKE, 2, 3, 4, FAKE, FAKE, 0) == akv.AKV_ERR_ALIGN
    assert f(FAKE, FAKE, 2, 0, 4, FAKE, FAKE, 0) == akv.AKV_OK  # no rows: nothing to do


def compress_desc(**over):
    kw = dict(Hkv=4, d=128, src_k=FAKE, src_v=FAKE + 0x100000, src_block_table=FAKE + 0x200000,
              src_max_blocks=72, src_num_blocks=72, src_start=0, n_tokens=512, dst_k_codes=FAKE + 0x300000,
              dst_v_codes=FAKE + 0x400000, dst_k_scales=FAKE + 0x500000, dst_v_scales=FAKE + 0x600000,
              dst_block_table=FAKE + 0x700000, dst_max_blocks=456, dst_num_blocks=456, dst_start=28672)
    kw.update(over)
    return akv.CompressDesc(**kw)


def test_compress_validation():
    f = akv.akv_compress_evicted
    assert akv.LIB.akv_compress_evicted(None, None) == akv.AKV_ERR_NULL
    assert f(compress_desc(src_k=0)) == akv.AKV_ERR_NULL
    assert f(compress_desc(n_tokens=-1)) == akv.AKV_ERR_SHAPE
    assert f(compress_desc(src_start=72 * 64 - 511)) == akv.AKV_ERR_SHAPE
    assert f(compress_desc(dst_start=456 * 64 - 510)) == akv.AKV_ERR_SHAPE
    assert f(compress_desc(d=32)) == akv.AKV_ERR_UNSUPPORTED
    # an odd destination start is served (the shared value bytes are merged)
    assert f(compress_desc(dst_start=28671, dst_k_scales=FAKE + 0x500001)) == akv.AKV_ERR_ALIGN
    assert f(compress_desc(dst_start=28671, n_tokens=0)) == akv.AKV_OK
    assert f(compress_desc(dst_k_scales=FAKE + 0x500001)) == akv.AKV_ERR_ALIGN
    assert f(compress_desc(n_tokens=0)) == akv.AKV_OK


def test_ctypes_struct_sizes_match_header():
    # the library rejects a struct_size smaller than its own sizeof, so a
    # ctypes mirror that is too small shows up as SHAPE
    assert call(good_desc(), ws=0) == akv.AKV_ERR_WORKSPACE
    assert akv.akv_compress_evicted(compress_desc(src_k=0)) == akv.AKV_ERR_NULL


def test_frozen_device_constants_match_oracle():
    from oracle import akv_oracle as O
    src = open(os.path.join(os.path.dirname(akv.HERE), "long_context_kv_split_amd", "csrc", "akv_common.h")).read()

    def table(name):
        body = re.search(name + r"\[\d+\] = \{(.*?)\};", src, re.S).group(1)
        return np.array([int(x, 16) for x in re.findall(r"0x([0-9A-Fa-f]+)u", body)], dtype=np.uint32)

    for suffix, width in (("", 4), ("2", 2), ("3", 3)):
        levels, thresh = table("kLevelBits" + suffix), table("kThreshBits" + suffix)
        assert levels.size == 2 ** width and thresh.size == 2 ** width - 1
        assert np.array_equal(levels, O.centroids_f32(width).view(np.uint32)), f"levels, width {width}"
        assert np.array_equal(thresh, O.thresholds_f32(width=width).view(np.uint32)), f"thresholds, width {width}"
    assert "0x3DB504F3u" in src and O.inv_sqrt_f32(128).view(np.uint32) == 0x3DB504F3


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    """No fallback: with the library missing the binding raises instead of computing anything."""
    monkeypatch.setattr(akv, "LIB_PATH", str(tmp_path / "libakv.so"))
    import pytest as _pytest
    with _pytest.raises(ImportError):
        akv._load()


def append_desc(**over):
    kw = dict(B=2, Hkv=4, d=128, window=128, new_k=FAKE + 0x100, new_v=FAKE + 0x200, exact_k=FAKE,
              exact_v=FAKE + 0x1000000, exact_table=FAKE + 0x2000000, exact_lengths=FAKE + 0x2100000,
              exact_max_blocks=3, exact_num_blocks=6, k_codes=FAKE + 0x3000000, v_codes=FAKE + 0x4000000,
              k_scales=FAKE + 0x5000000, v_scales=FAKE + 0x5800000, quant_table=FAKE + 0x6000000,
              quant_lengths=FAKE + 0x6100000, quant_max_blocks=4, quant_num_blocks=8)
    kw.update(over)
    return akv.AppendDesc(**kw)


def test_append_evict_validation_order():
    """Refusals happen on the host before anything is enqueued (no GPU needed)."""
    assert akv.LIB.akv_append_evict(None, None) == akv.AKV_ERR_NULL
    assert akv.akv_append_evict(append_desc(new_k=0)) == akv.AKV_ERR_NULL
    assert akv.akv_append_evict(append_desc(quant_lengths=0, window=100)) == akv.AKV_ERR_NULL  # NULL first
    assert akv.akv_append_evict(append_desc(window=100)) == akv.AKV_ERR_SHAPE
    assert akv.akv_append_evict(append_desc(window=0)) == akv.AKV_ERR_SHAPE
    assert akv.akv_append_evict(append_desc(window=192)) == akv.AKV_ERR_SHAPE  # needs 4 exact-table entries
    assert akv.akv_append_evict(append_desc(B=0)) == akv.AKV_ERR_SHAPE
    assert akv.akv_append_evict(append_desc(d=96)) == akv.AKV_ERR_UNSUPPORTED
    assert akv.akv_append_evict(append_desc(d=96, window=100)) == akv.AKV_ERR_SHAPE  # SHAPE before UNSUPPORTED
    assert akv.akv_append_evict(append_desc(B=40000)) == akv.AKV_ERR_UNSUPPORTED
    assert akv.akv_append_evict(append_desc(exact_lengths=FAKE + 2)) == akv.AKV_ERR_ALIGN
    d = append_desc()
    d.struct_size = 8
    assert akv.akv_append_evict(d) == akv.AKV_ERR_SHAPE


def context_desc(**over):
    kw = dict(B=3, Hkv=4, d=128, exact_k=FAKE, exact_v=FAKE + 0x1000000, exact_table=FAKE + 0x2000000,
              exact_lengths=FAKE + 0x2100000, exact_max_blocks=65, exact_num_blocks=200,
              k_codes=FAKE + 0x3000000, v_codes=FAKE + 0x4000000, k_scales=FAKE + 0x5000000,
              v_scales=FAKE + 0x5800000, quant_table=FAKE + 0x6000000, quant_lengths=FAKE + 0x6100000,
              quant_max_blocks=1936, quant_num_blocks=6000)
    kw.update(over)
    return akv.ContextDesc(**kw)


def test_checkpoint_image_size_and_validation():
    """The image size is the documented layout: 256-byte header, lengths padded to
    256, 256*Hkv*d bytes per exact slot and 72*Hkv*d per compressed slot."""
    d = context_desc()
    lens_end = 256 + 256                              # 8 * B = 24 bytes, padded
    expect = lens_end + 3 * 65 * 256 * 4 * 128 + 3 * 1936 * 72 * 4 * 128
    assert akv.akv_checkpoint_bytes(d) == expect
    assert akv.akv_checkpoint_bytes(context_desc(quant_max_blocks=0, k_codes=0, v_codes=0, k_scales=0,
                                                 v_scales=0, quant_table=0)) == lens_end + 3 * 65 * 256 * 512
    assert akv.akv_checkpoint_bytes(context_desc(d=96)) == 0
    img = FAKE + 0xB000000
    assert akv.akv_checkpoint_save(context_desc(exact_lengths=0), img) == akv.AKV_ERR_NULL
    assert akv.akv_checkpoint_save(context_desc(), 0) == akv.AKV_ERR_NULL
    assert akv.akv_checkpoint_restore(context_desc(B=0), img) == akv.AKV_ERR_SHAPE
    assert akv.akv_checkpoint_restore(context_desc(d=96), img) == akv.AKV_ERR_UNSUPPORTED
    assert akv.akv_checkpoint_restore(context_desc(), img + 16) == akv.AKV_ERR_ALIGN
    assert akv.akv_checkpoint_save(context_desc(exact_k=FAKE + 8), img) == akv.AKV_ERR_ALIGN


def test_staged_decode_validation_order():
    """Staging and attention descriptors are checked together, category by category."""
    tiers = (akv.HostTier * 1)(akv.HostTier(FAKE + 0x100000, 1000))
    events = (ctypes.c_void_p * 5)(*([FAKE + 0x10] * 5))

    def sd(**over):
        kw = dict(seqs=ctypes.addressof(tiers), ring=FAKE + 0xC000000, ring_bytes=1 << 24, slots=2,
                  copy_stream=FAKE + 0x20, events=ctypes.addressof(events))
        kw.update(over)
        return akv.StagingDesc(**kw)

    def call(desc=None, st=None, ws=FAKE + 0xA000000):
        return akv.LIB.akv_attend_decode_staged(ctypes.byref(desc or good_desc()), ctypes.byref(st or sd()), ws,
                                                1 << 40, None)

    q = good_desc().quant
    q.k_codes = q.v_codes = q.k_scales = q.v_scales = q.block_table = 0   # pools are on the host here
    staged_desc = good_desc(quant=q)
    assert akv.LIB.akv_attend_decode_staged(ctypes.byref(staged_desc), None, 0, 0, None) == akv.AKV_ERR_NULL
    assert call(staged_desc, sd(ring=0)) == akv.AKV_ERR_NULL
    assert call(good_desc(q=0), sd(slots=1)) == akv.AKV_ERR_NULL            # NULL before SHAPE
    assert call(staged_desc, sd(slots=1)) == akv.AKV_ERR_SHAPE
    assert call(good_desc(quant=q, d=96), sd(slots=1)) == akv.AKV_ERR_SHAPE  # staging SHAPE before UNSUPPORTED
    assert call(good_desc(quant=q, d=96)) == akv.AKV_ERR_UNSUPPORTED
    assert call(staged_desc, sd(ring=FAKE + 0xC000010)) == akv.AKV_ERR_ALIGN
    assert call(staged_desc, ws=0) == akv.AKV_ERR_WORKSPACE
    assert call(staged_desc, sd(ring_bytes=1 << 16)) == akv.AKV_ERR_WORKSPACE  # a slot below one split


def test_rotation_field():
    """A given rotation: 16-byte aligned, and the decode and chunk workspaces
    grow by the rotated queries (4 B * Tq * Hq * d bytes, 256-aligned)."""
    d = good_desc()
    need = akv.akv_decode_workspace_bytes(d)
    dr = good_desc(rotation=FAKE + 0x800000)
    need_r = akv.akv_decode_workspace_bytes(dr)
    extra = 4 * d.B * d.Hq * d.d
    assert need + extra <= need_r <= need + extra + 256
    assert call(dr, ws_bytes=need_r - 1) == akv.AKV_ERR_WORKSPACE
    assert call(good_desc(rotation=FAKE + 8)) == akv.AKV_ERR_ALIGN
    dc, dcr = good_desc(Tq=4), good_desc(Tq=4, rotation=FAKE + 0x800000)
    need_c, need_cr = akv.akv_chunk_workspace_bytes(dc), akv.akv_chunk_workspace_bytes(dcr)
    extra_c = 4 * dc.B * dc.Tq * dc.Hq * dc.d
    assert need_c + extra_c <= need_cr <= need_c + extra_c + 256
    assert call(dcr, ws_bytes=need_cr - 1, chunk=True) == akv.AKV_ERR_WORKSPACE
    assert call(good_desc(Tq=4, rotation=FAKE + 8), chunk=True) == akv.AKV_ERR_ALIGN
    assert akv.akv_compress_evicted(compress_desc(rotation=FAKE + 4)) == akv.AKV_ERR_ALIGN
    assert akv.akv_append_evict(append_desc(rotation=FAKE + 4)) == akv.AKV_ERR_ALIGN


def test_code_width_field():
    """code_bits: 0/4, 3 and 2 served (decode and chunk); others UNSUPPORTED;
    the checkpoint image's compressed slots scale as (16 w + 8) Hkv d."""
    for cb in (0, 2, 3, 4):
        assert call(good_desc(code_bits=cb), ws=0) == akv.AKV_ERR_WORKSPACE, cb
    for cb in (1, 5, 8, -1):
        assert call(good_desc(code_bits=cb)) == akv.AKV_ERR_UNSUPPORTED, cb
    for cb in (2, 3):
        assert call(good_desc(Tq=4, code_bits=cb), chunk=True, ws=0) == akv.AKV_ERR_WORKSPACE, cb
    assert call(good_desc(Tq=4, code_bits=5), chunk=True) == akv.AKV_ERR_UNSUPPORTED
    assert akv.akv_compress_evicted(compress_desc(code_bits=5)) == akv.AKV_ERR_UNSUPPORTED
    assert akv.akv_compress_evicted(compress_desc(code_bits=3, n_tokens=0)) == akv.AKV_OK
    assert akv.akv_append_evict(append_desc(code_bits=1)) == akv.AKV_ERR_UNSUPPORTED
    sizes = {}
    for cb in (2, 3, 4):
        c = akv.ContextDesc(B=2, Hkv=4, d=128, exact_k=FAKE, exact_v=FAKE, exact_table=FAKE, exact_lengths=FAKE,
                            exact_max_blocks=3, exact_num_blocks=6, k_codes=FAKE, v_codes=FAKE, k_scales=FAKE,
                            v_scales=FAKE, quant_table=FAKE, quant_lengths=FAKE, quant_max_blocks=5,
                            quant_num_blocks=10, code_bits=cb)
        sizes[cb] = akv.akv_checkpoint_bytes(c)
        assert sizes[cb] == 512 + 2 * 3 * 256 * 4 * 128 + 2 * 5 * (16 * cb + 8) * 4 * 128, cb


@pytest.mark.parametrize("width", [2, 3])
@pytest.mark.parametrize("d", [64, 128])
def test_narrow_code_layouts_cover_each_bit_once(width, d):
    """The width-w byte layouts (as the harness reads them) give every (token,
    dim) code its own bits and use every bit of the 8 w d-byte slab once."""
    from long_context_kv_split_amd.harness import narrow_code_bits
    tok, dim = np.meshgrid(np.arange(64), np.arange(d), indexing="ij")
    for isv in (False, True):
        pb, ps, hb, hs = narrow_code_bits(d, width, tok, dim, isv)
        bits = [(8 * pb + ps).ravel(), (8 * pb + ps + 1).ravel()]
        if width == 3:
            bits.append((8 * hb + hs).ravel())
        allbits = np.concatenate(bits)
        assert np.unique(allbits).size == allbits.size == 8 * width * d * 8
        assert allbits.min() == 0 and allbits.max() == 8 * width * d * 8 - 1


@pytest.mark.parametrize("d", [64, 128])
def test_four_bit_code_layouts_cover_each_nibble_once(d):
    """The 4-bit K and V code byte layouts (as the harness reads them) give
    every (token, dim) code its own nibble of the 32 d-byte slab."""
    from long_context_kv_split_amd.harness import kcode_byte, vcode_byte
    tok, dim = np.meshgrid(np.arange(64), np.arange(d), indexing="ij")
    k = 2 * (tok * (d // 2) + kcode_byte(d, dim)) + (dim & 1)
    v = 2 * vcode_byte(d, tok, dim) + (tok & 1)
    for nib in (k.ravel(), v.ravel()):
        assert np.unique(nib).size == nib.size == 64 * d
        assert nib.min() == 0 and nib.max() == 64 * d - 1

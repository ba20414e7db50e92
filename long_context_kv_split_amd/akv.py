"""ctypes binding of libakv.so: the C entry points of include/akv.h under the same names.

Argument marshalling only -- every step of the attention path runs in the HIP
kernels of the library.  Importing this module loads the in-tree
``libakv.so``; if it is missing the import raises (there is no fallback).
Pointers are plain integers (device addresses, e.g. ``tensor.data_ptr()``)
and ``stream`` is a hipStream_t as an integer (0 = default stream).
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_float, c_int32, c_size_t, c_uint32, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libakv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "akv.h")

AKV_OK = 0
AKV_ERR_NULL = -1
AKV_ERR_SHAPE = -2
AKV_ERR_UNSUPPORTED = -3
AKV_ERR_WORKSPACE = -4
AKV_ERR_ALIGN = -5
AKV_ERR_HIP = -6
STATUS_NAMES = {0: "AKV_OK", -1: "AKV_ERR_NULL", -2: "AKV_ERR_SHAPE", -3: "AKV_ERR_UNSUPPORTED",
                -4: "AKV_ERR_WORKSPACE", -5: "AKV_ERR_ALIGN", -6: "AKV_ERR_HIP"}

BLOCK_TOKENS = 64
GROUP = 32
SPLIT_TOKENS_EXACT_DEFAULT = 1024
SPLIT_TOKENS_QUANT_DEFAULT = 1024
MAX_SPLIT_TOKENS = 32768
MIN_SPLIT_TOKENS = 256
DECODE_TARGET_WORKGROUPS = 512
MAX_SPLITS = 2048
MAX_CHUNK = 512
DECODE_MAX_SUBSPLITS = 8
MIN_SUBSPLIT_BLOCKS = 4
NOALLOC_SCRATCH_BYTES = 64 << 20


class ExactTier(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("block_table", c_void_p), ("lengths", c_void_p),
                ("max_blocks", c_int32), ("num_blocks", c_int32)]


class QuantTier(ctypes.Structure):
    _fields_ = [("k_codes", c_void_p), ("v_codes", c_void_p), ("k_scales", c_void_p), ("v_scales", c_void_p),
                ("block_table", c_void_p), ("lengths", c_void_p), ("max_blocks", c_int32),
                ("num_blocks", c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("B", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("d", c_int32),
                ("Tq", c_int32), ("softmax_scale", c_float), ("q", c_void_p), ("exact", ExactTier),
                ("quant", QuantTier), ("split_tokens_exact", c_int32), ("split_tokens_quant", c_int32),
                ("o", c_void_p), ("lse", c_void_p), ("rotation", c_void_p), ("code_bits", c_int32)]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(AttnDesc), **kw)


class CompressDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("Hkv", c_int32), ("d", c_int32), ("src_k", c_void_p),
                ("src_v", c_void_p), ("src_block_table", c_void_p), ("src_max_blocks", c_int32),
                ("src_num_blocks", c_int32), ("src_start", c_int32), ("n_tokens", c_int32),
                ("dst_k_codes", c_void_p), ("dst_v_codes", c_void_p), ("dst_k_scales", c_void_p),
                ("dst_v_scales", c_void_p), ("dst_block_table", c_void_p), ("dst_max_blocks", c_int32),
                ("dst_num_blocks", c_int32), ("dst_start", c_int32), ("rotation", c_void_p),
                ("code_bits", c_int32)]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(CompressDesc), **kw)


class AppendDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("B", c_int32), ("Hkv", c_int32), ("d", c_int32), ("window", c_int32),
                ("new_k", c_void_p), ("new_v", c_void_p), ("exact_k", c_void_p), ("exact_v", c_void_p),
                ("exact_table", c_void_p), ("exact_lengths", c_void_p), ("exact_max_blocks", c_int32),
                ("exact_num_blocks", c_int32), ("k_codes", c_void_p), ("v_codes", c_void_p),
                ("k_scales", c_void_p), ("v_scales", c_void_p), ("quant_table", c_void_p),
                ("quant_lengths", c_void_p), ("quant_max_blocks", c_int32), ("quant_num_blocks", c_int32),
                ("rotation", c_void_p), ("code_bits", c_int32)]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(AppendDesc), **kw)


class ContextDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("B", c_int32), ("Hkv", c_int32), ("d", c_int32),
                ("exact_k", c_void_p), ("exact_v", c_void_p), ("exact_table", c_void_p), ("exact_lengths", c_void_p),
                ("exact_max_blocks", c_int32), ("exact_num_blocks", c_int32), ("k_codes", c_void_p),
                ("v_codes", c_void_p), ("k_scales", c_void_p), ("v_scales", c_void_p), ("quant_table", c_void_p),
                ("quant_lengths", c_void_p), ("quant_max_blocks", c_int32), ("quant_num_blocks", c_int32),
                ("code_bits", c_int32)]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(ContextDesc), **kw)


class HostTier(ctypes.Structure):
    _fields_ = [("blocks", c_void_p), ("length", c_int32)]


class StagingDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("seqs", c_void_p), ("ring", c_void_p), ("ring_bytes", c_size_t),
                ("slots", c_int32), ("copy_stream", c_void_p), ("events", c_void_p)]

    def __init__(self, **kw):
        super().__init__(struct_size=ctypes.sizeof(StagingDesc), **kw)


class AKVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    # One HIP runtime per process: PyTorch-ROCm ships its own libamdhip64, and
    # libakv.so binds to whichever copy is already loaded.  Importing torch
    # first makes both share torch's runtime (a second runtime would not see
    # the device torch holds).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run long_context_kv_split_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.akv_abi_version.restype = ctypes.c_int
    lib.akv_abi_version.argtypes = []
    lib.akv_last_error.restype = ctypes.c_char_p
    lib.akv_last_error.argtypes = []
    for name in ("akv_decode_workspace_bytes", "akv_chunk_workspace_bytes"):
        fn = getattr(lib, name)
        fn.restype = c_size_t
        fn.argtypes = [P(AttnDesc)]
    for name in ("akv_attend_decode", "akv_attend_chunk"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P(AttnDesc), c_void_p, c_size_t, c_void_p]
    lib.akv_attend_decode_noalloc.restype = ctypes.c_int
    lib.akv_attend_decode_noalloc.argtypes = [P(AttnDesc), c_void_p]
    lib.akv_decode_split_workgroups.restype = c_int32
    lib.akv_decode_split_workgroups.argtypes = [P(AttnDesc)]
    lib.akv_split_plan.restype = ctypes.c_int
    lib.akv_split_plan.argtypes = [P(AttnDesc), c_int32, P(c_int32)]
    lib.akv_attend_decode_staged.restype = ctypes.c_int
    lib.akv_attend_decode_staged.argtypes = [P(AttnDesc), P(StagingDesc), c_void_p, c_size_t, c_void_p]
    lib.akv_lse_merge.restype = ctypes.c_int
    lib.akv_lse_merge.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.akv_compress_evicted.restype = ctypes.c_int
    lib.akv_compress_evicted.argtypes = [P(CompressDesc), c_void_p]
    lib.akv_append_evict.restype = ctypes.c_int
    lib.akv_append_evict.argtypes = [P(AppendDesc), c_void_p]
    lib.akv_checkpoint_bytes.restype = c_size_t
    lib.akv_checkpoint_bytes.argtypes = [P(ContextDesc)]
    for name in ("akv_checkpoint_save", "akv_checkpoint_restore"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P(ContextDesc), c_void_p, c_void_p]
    return lib


LIB = _load()


def header_functions() -> list:
    """Names of the functions include/akv.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:akv_status|size_t|int32_t|int|const char\*)\s+(akv_\w+)\s*\(", text, re.M)))


def akv_abi_version() -> int:
    return LIB.akv_abi_version()


def akv_last_error() -> str:
    return LIB.akv_last_error().decode()


def akv_decode_workspace_bytes(desc: AttnDesc) -> int:
    return LIB.akv_decode_workspace_bytes(ctypes.byref(desc))


def akv_chunk_workspace_bytes(desc: AttnDesc) -> int:
    return LIB.akv_chunk_workspace_bytes(ctypes.byref(desc))


def akv_split_plan(desc: AttnDesc, chunk: bool = False) -> dict:
    """Split sizes and counts the library picks for desc (raises AKVError if desc is invalid)."""
    out = (c_int32 * 4)()
    check(LIB.akv_split_plan(ctypes.byref(desc), int(bool(chunk)), out))
    return {"split_tokens_quant": out[0], "split_tokens_exact": out[1], "splits_quant": out[2],
            "splits_exact": out[3]}


def akv_decode_split_workgroups(desc: AttnDesc) -> int:
    return LIB.akv_decode_split_workgroups(ctypes.byref(desc))


def akv_attend_decode(desc: AttnDesc, ws: int, ws_bytes: int, stream: int = 0) -> int:
    return LIB.akv_attend_decode(ctypes.byref(desc), ws, ws_bytes, stream)


def akv_attend_decode_noalloc(desc: AttnDesc, stream: int = 0) -> int:
    return LIB.akv_attend_decode_noalloc(ctypes.byref(desc), stream)


def akv_attend_chunk(desc: AttnDesc, ws: int, ws_bytes: int, stream: int = 0) -> int:
    return LIB.akv_attend_chunk(ctypes.byref(desc), ws, ws_bytes, stream)


def akv_lse_merge(o_parts: int, lse_parts: int, P: int, R: int, d: int, o_out: int, lse_out: int,
                  stream: int = 0) -> int:
    return LIB.akv_lse_merge(o_parts, lse_parts, P, R, d, o_out, lse_out, stream)


def akv_compress_evicted(desc: CompressDesc, stream: int = 0) -> int:
    return LIB.akv_compress_evicted(ctypes.byref(desc), stream)


def check(status: int) -> None:
    """Raise AKVError for a non-OK status (with the library's message)."""
    if status != AKV_OK:
        raise AKVError(status, akv_last_error())


def akv_append_evict(desc: AppendDesc, stream: int = 0) -> int:
    return LIB.akv_append_evict(ctypes.byref(desc), stream)


def akv_checkpoint_bytes(desc: ContextDesc) -> int:
    return LIB.akv_checkpoint_bytes(ctypes.byref(desc))


def akv_checkpoint_save(desc: ContextDesc, image: int, stream: int = 0) -> int:
    return LIB.akv_checkpoint_save(ctypes.byref(desc), image, stream)


def akv_checkpoint_restore(desc: ContextDesc, image: int, stream: int = 0) -> int:
    return LIB.akv_checkpoint_restore(ctypes.byref(desc), image, stream)


def akv_attend_decode_staged(desc: AttnDesc, staging: StagingDesc, ws: int, ws_bytes: int, stream: int = 0) -> int:
    return LIB.akv_attend_decode_staged(ctypes.byref(desc), ctypes.byref(staging), ws, ws_bytes, stream)

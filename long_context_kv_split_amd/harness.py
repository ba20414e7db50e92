"""Device-side harness: paged pools in HBM for a synth.Workload, calls through the C ABI.

PyTorch is used only to own device memory and streams.  The compressed tier
is produced on the GPU by ``akv_compress_evicted`` from the workload's bf16
source values (staged once in an exact-tier-format pool), exactly as an
eviction would produce it.  Nothing here computes any part of the method:
the helpers only scatter/gather bytes according to the layouts documented in
include/akv.h.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import ctypes

import numpy as np
import torch

from . import akv
from .synth import BLOCK, Workload


# ------------------------------------------------------------------ layouts

def kcode_byte(d: int, dim: np.ndarray) -> np.ndarray:
    """Byte (inside a token's K-code row) holding dim `dim` (include/akv.h)."""
    m, a, b = dim >> 5, (dim >> 3) & 3, (dim >> 1) & 3
    return (d >> 3) * a + 4 * m + b


def vcode_byte(d: int, tok: np.ndarray, dim: np.ndarray) -> np.ndarray:
    """Byte (inside a V-code slab) holding token `tok` (in-block) of dim `dim`."""
    c, a, b = tok >> 5, (tok >> 3) & 3, (tok >> 1) & 3
    t, i = dim >> 4, dim & 15
    return c * 16 * d + (t >> 2) * 1024 + (a * 16 + i) * 16 + 4 * (t & 3) + b


def narrow_code_bits(d: int, w: int, tok: np.ndarray, dim: np.ndarray, isv: bool):
    """(byte, shift) pairs inside a width-w (2 or 3) code slab of the pair-plane
    bits (2 per code) and, for w = 3, of the high-plane bit of (in-block token
    `tok`, dim `dim`) (include/akv.h, "Code width")."""
    e = tok & 1 if isv else dim & 1
    if not isv:
        m, a, b = dim >> 5, (dim >> 3) & 3, (dim >> 1) & 3
        pb = tok * (d // 4) + (d // 16) * a + 4 * (m >> 1) + b
        ps = 4 * (m & 1) + 2 * e
        M = d // 32
        bit = 8 * M * a + 2 * M * b + 2 * m + e
        hb = 16 * d + tok * (d // 8) + (bit >> 3)
        hs = bit & 7
    else:
        c, a, b = tok >> 5, (tok >> 3) & 3, (tok >> 1) & 3
        t, i = dim >> 4, dim & 15
        pb = ((c * 4 + a) * 16 + i) * (d // 8) + 4 * (t >> 1) + b
        ps = 4 * (t & 1) + 2 * e
        hb = 16 * d + ((c * 4 + a) * 16 + i) * (d // 16) + 4 * (t >> 2) + b
        hs = 2 * (t & 3) + e
    return pb, ps, hb, hs


def pages_from_tokens(x: np.ndarray, n_blocks_pool: int, table_row: np.ndarray, out: np.ndarray,
                      dim_major: bool = False) -> None:
    """Scatter token-major x [n, Hkv, d] into a pool by a table row: [blocks, Hkv, 64, d]
    (exact-tier K), or [blocks, Hkv, 2, d, 32] with dim_major (exact-tier V: dim-major
    inside each 32-token half block)."""
    n, hkv, d = x.shape
    nb = -(-n // BLOCK)
    if nb == 0:
        return
    pad = np.zeros((nb * BLOCK, hkv, d), dtype=x.dtype)
    pad[:n] = x
    if dim_major:
        out[table_row[:nb]] = pad.reshape(nb, 2, BLOCK // 2, hkv, d).transpose(0, 3, 1, 4, 2)
    else:
        out[table_row[:nb]] = pad.reshape(nb, BLOCK, hkv, d).transpose(0, 2, 1, 3)


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclass
class Pools:
    """One replica of every per-call input that a decode call streams."""
    ek: Optional[torch.Tensor]
    ev: Optional[torch.Tensor]
    kc: Optional[torch.Tensor]
    vc: Optional[torch.Tensor]
    ks: Optional[torch.Tensor]
    vs: Optional[torch.Tensor]


class DeviceWorkload:
    """A workload resident in HBM, ready for akv_attend_decode / akv_attend_chunk.

    ``rotation`` (float32 [d, d] orthogonal, or None for the Walsh-Hadamard one)
    is the compressed tier's rotation and ``width`` (2, 3 or 4) its code width:
    every descriptor built here carries both."""

    def __init__(self, w: Workload, device: str = "cuda", fill_quant: bool = True,
                 rotation: Optional[np.ndarray] = None, width: int = 4):
        self.w = w
        self.device = device
        self.width = width
        self.rotation = None if rotation is None else \
            torch.from_numpy(np.ascontiguousarray(rotation, dtype=np.float32)).to(device)
        d, hkv = w.d, w.Hkv
        self.q = _dev(w.q, device)
        self.exact_len = _dev(w.exact_len, device)
        self.quant_len = _dev(w.quant_len, device)
        self.exact_table = _dev(w.exact_table, device)
        self.quant_table = _dev(w.quant_table, device)
        # a tier is present when its table holds any block (tokens or room)
        self.emax = w.exact_table.shape[1] if (w.exact_table >= 0).any() else 0
        self.qmax = w.quant_table.shape[1] if (w.quant_table >= 0).any() else 0
        ek = np.zeros((max(1, w.exact_pool_blocks), hkv, BLOCK, d), dtype=np.uint16)
        ev = np.zeros((max(1, w.exact_pool_blocks), hkv, 2, d, BLOCK // 2), dtype=np.uint16)
        for b in range(w.B):
            pages_from_tokens(w.exact_k[b], w.exact_pool_blocks, w.exact_table[b], ek)
            pages_from_tokens(w.exact_v[b], w.exact_pool_blocks, w.exact_table[b], ev, dim_major=True)
        qnb = max(1, w.quant_pool_blocks)
        self.pools = [Pools(
            _dev(ek, device), _dev(ev, device),
            torch.zeros((qnb, hkv, 8 * width * d), dtype=torch.uint8, device=device),
            torch.zeros((qnb, hkv, 8 * width * d), dtype=torch.uint8, device=device),
            torch.zeros((qnb, hkv, 2 * d), dtype=torch.int16, device=device),
            torch.zeros((qnb, hkv, 2 * d), dtype=torch.int16, device=device))]
        B, Tq, Hq = w.B, w.Tq, w.Hq
        self.o = torch.full((B, Tq, Hq, d), float("nan"), dtype=torch.float32, device=device)
        self.lse = torch.full((B, Tq, Hq), float("nan"), dtype=torch.float32, device=device)
        self.ws = None
        self.ws_bytes = 0
        if fill_quant:
            self.fill_quant_tier()

    # ----------------------------------------------------------- compressed tier
    def fill_quant_tier(self, stream: int = 0) -> None:
        """Encode every sequence's compressed-tier source into the pools (GPU)."""
        w = self.w
        if w.quant_len.max(initial=0) == 0:
            return
        for b in range(w.B):
            n = int(w.quant_len[b])
            if n == 0:
                continue
            nb = -(-n // BLOCK)
            sk = np.zeros((nb, w.Hkv, BLOCK, w.d), dtype=np.uint16)
            sv = np.zeros((nb, w.Hkv, 2, w.d, BLOCK // 2), dtype=np.uint16)
            ident = np.arange(nb, dtype=np.int32)
            pages_from_tokens(w.quant_k_src[b], nb, ident, sk)
            pages_from_tokens(w.quant_v_src[b], nb, ident, sv, dim_major=True)
            dk, dv, dt = _dev(sk, self.device), _dev(sv, self.device), _dev(ident, self.device)
            dst_t = self.quant_table[b]
            desc = akv.CompressDesc(
                Hkv=w.Hkv, d=w.d, src_k=ptr(dk), src_v=ptr(dv), src_block_table=ptr(dt),
                src_max_blocks=nb, src_num_blocks=nb, src_start=0, n_tokens=n,
                dst_k_codes=ptr(self.pools[0].kc), dst_v_codes=ptr(self.pools[0].vc),
                dst_k_scales=ptr(self.pools[0].ks), dst_v_scales=ptr(self.pools[0].vs),
                dst_block_table=ptr(dst_t), dst_max_blocks=w.quant_table.shape[1],
                dst_num_blocks=max(1, w.quant_pool_blocks), dst_start=0, rotation=ptr(self.rotation),
                code_bits=self.width)
            akv.check(akv.akv_compress_evicted(desc, stream or stream_handle()))
            torch.cuda.synchronize()
            del dk, dv, dt

    def append_desc(self, window: int, new_k: torch.Tensor, new_v: torch.Tensor, replica: int = 0) -> akv.AppendDesc:
        """Descriptor of one fused append / evict step on this workload's device state."""
        w, P = self.w, self.pools[replica]
        return akv.AppendDesc(
            B=w.B, Hkv=w.Hkv, d=w.d, window=window, new_k=ptr(new_k), new_v=ptr(new_v),
            exact_k=ptr(P.ek), exact_v=ptr(P.ev), exact_table=ptr(self.exact_table),
            exact_lengths=ptr(self.exact_len), exact_max_blocks=w.exact_table.shape[1],
            exact_num_blocks=max(1, w.exact_pool_blocks), k_codes=ptr(P.kc), v_codes=ptr(P.vc),
            k_scales=ptr(P.ks), v_scales=ptr(P.vs), quant_table=ptr(self.quant_table),
            quant_lengths=ptr(self.quant_len), quant_max_blocks=w.quant_table.shape[1],
            quant_num_blocks=max(1, w.quant_pool_blocks), rotation=ptr(self.rotation), code_bits=self.width)

    def context_desc(self, replica: int = 0) -> akv.ContextDesc:
        """Descriptor of this workload's device state for checkpoint save / restore."""
        w, P = self.w, self.pools[replica]
        return akv.ContextDesc(
            B=w.B, Hkv=w.Hkv, d=w.d, exact_k=ptr(P.ek), exact_v=ptr(P.ev), exact_table=ptr(self.exact_table),
            exact_lengths=ptr(self.exact_len), exact_max_blocks=self.emax,
            exact_num_blocks=max(1, w.exact_pool_blocks), k_codes=ptr(P.kc), v_codes=ptr(P.vc),
            k_scales=ptr(P.ks), v_scales=ptr(P.vs), quant_table=ptr(self.quant_table),
            quant_lengths=ptr(self.quant_len), quant_max_blocks=self.qmax,
            quant_num_blocks=max(1, w.quant_pool_blocks), code_bits=self.width)

    def host_tiers(self, replica: int = 0):
        """Each sequence's compressed tier copied to pinned host memory as block records
        in token order (record i = tokens 64i..: K codes, V codes, K scales, V scales of
        every kv head), as akv_attend_decode_staged reads it.  Returns the tensors (kept
        alive by the caller) and the ctypes array of akv_host_tier."""
        w, P = self.w, self.pools[replica]
        keep, tiers = [], (akv.HostTier * w.B)()
        for b in range(w.B):
            n = int(w.quant_len[b])
            nb = -(-n // BLOCK)
            rec = torch.empty(0, dtype=torch.uint8)
            if nb:
                blocks = torch.from_numpy(w.quant_table[b][:nb].astype(np.int64)).to(self.device)
                parts = [x.index_select(0, blocks).reshape(nb, -1).view(torch.uint8) for x in (P.kc, P.vc, P.ks, P.vs)]
                rec = torch.cat(parts, dim=1).cpu().pin_memory()
            keep.append(rec)
            tiers[b] = akv.HostTier(rec.data_ptr() if nb else 0, n)
        return keep, tiers

    def staging(self, tiers, ring: torch.Tensor, slots: int, copy_stream: torch.cuda.Stream):
        """A StagingDesc over `tiers` (from host_tiers) with a device ring of `slots`
        slots.  Creates its 2 * slots + 1 events; returns (desc, keep-alive objects)."""
        events = [torch.cuda.Event() for _ in range(2 * slots + 1)]
        for e in events:
            e.record(copy_stream)  # materialize the handle
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        desc = akv.StagingDesc(seqs=ctypes.addressof(tiers), ring=ring.data_ptr(), ring_bytes=ring.numel(),
                               slots=slots, copy_stream=copy_stream.cuda_stream,
                               events=ctypes.addressof(handles))
        return desc, (events, handles, tiers)

    def read_exact(self, b: int, replica: int = 0):
        """Logical exact tier (K, V), bf16 bits [n, Hkv, d] each, of sequence b as the
        device holds it now (its current length and block-table row)."""
        n = int(self.exact_len[b].item())
        table = self.exact_table[b].cpu().numpy()
        P = self.pools[replica]
        ek = P.ek.cpu().numpy().view(np.uint16)   # [blocks, Hkv, 64, d]
        ev = P.ev.cpu().numpy().view(np.uint16)   # [blocks, Hkv, 2, d, 32]
        tok = np.arange(n)
        blk, r = table[tok // BLOCK], tok % BLOCK
        return ek[blk, :, r, :], ev[blk, :, r // (BLOCK // 2), :, r % (BLOCK // 2)]

    def compress_desc(self, b: int, src_start: int, n: int, dst_start: int, replica: int = 0) -> akv.CompressDesc:
        """Descriptor moving exact tokens [src_start, +n) of sequence b to compressed [dst_start, +n)."""
        w, P = self.w, self.pools[replica]
        return akv.CompressDesc(
            Hkv=w.Hkv, d=w.d, src_k=ptr(P.ek), src_v=ptr(P.ev), src_block_table=ptr(self.exact_table[b]),
            src_max_blocks=w.exact_table.shape[1], src_num_blocks=max(1, w.exact_pool_blocks),
            src_start=src_start, n_tokens=n,
            dst_k_codes=ptr(P.kc), dst_v_codes=ptr(P.vc), dst_k_scales=ptr(P.ks), dst_v_scales=ptr(P.vs),
            dst_block_table=ptr(self.quant_table[b]), dst_max_blocks=w.quant_table.shape[1],
            dst_num_blocks=max(1, w.quant_pool_blocks), dst_start=dst_start, rotation=ptr(self.rotation),
            code_bits=self.width)

    def read_codes(self, b: int, start: int = 0, n: Optional[int] = None, replica: int = 0):
        """Logical (codes, scales) of compressed tokens [start, start+n) of sequence b.

        Returns kcodes [n, Hkv, d] u8, kscales [n, Hkv, d/32] u16 bits, vcodes, vscales.
        """
        w, P = self.w, self.pools[replica]
        d = w.d
        n = int(w.quant_len[b]) - start if n is None else n
        tok = np.arange(start, start + n)
        blocks = w.quant_table[b][tok // BLOCK].astype(np.int64)
        r = tok % BLOCK
        if self.width != 4:
            return self._read_narrow(blocks, r, replica)
        kc = P.kc.cpu().numpy().reshape(P.kc.shape[0], w.Hkv, BLOCK, d // 2)
        vc = P.vc.cpu().numpy()
        ks = P.ks.cpu().numpy().view(np.uint16).reshape(-1, w.Hkv, d // 32, BLOCK)
        vs = P.vs.cpu().numpy().view(np.uint16).reshape(-1, w.Hkv, d // 32, BLOCK)
        dims = np.arange(d)
        kb = kcode_byte(d, dims)
        krow = kc[blocks, :, r, :]                                    # [n, Hkv, d/2]
        kcodes = (krow[:, :, kb] >> (4 * (dims & 1))[None, None, :]) & 15
        vb = vcode_byte(d, (r & ~1)[:, None], dims[None, :])          # [n, d]
        vbytes = vc[blocks[:, None, None], np.arange(w.Hkv)[None, :, None], vb[:, None, :]]
        vcodes = (vbytes >> (4 * (r & 1))[:, None, None]) & 15
        kscales = ks[blocks, :, :, r]
        vscales = vs[blocks, :, :, r]
        return (kcodes.astype(np.uint8), kscales.copy(), vcodes.astype(np.uint8), vscales.copy())

    def _read_narrow(self, blocks, r, replica):
        w, P, d, wd = self.w, self.pools[replica], self.w.d, self.width
        kc = P.kc.cpu().numpy()                                       # [blocks, Hkv, 8 w d]
        vc = P.vc.cpu().numpy()
        ks = P.ks.cpu().numpy().view(np.uint16).reshape(-1, w.Hkv, d // 32, BLOCK)
        vs = P.vs.cpu().numpy().view(np.uint16).reshape(-1, w.Hkv, d // 32, BLOCK)
        dims = np.arange(d)[None, :]
        heads = np.arange(w.Hkv)[None, :, None]
        out = []
        for pool, isv in ((kc, False), (vc, True)):
            pb, ps, hb, hs = narrow_code_bits(d, wd, r[:, None], dims, isv)   # [n, d]
            blk = blocks[:, None, None]
            codes = (pool[blk, heads, pb[:, None, :]] >> ps[:, None, :]) & 3
            if wd == 3:
                codes = codes | (((pool[blk, heads, hb[:, None, :]] >> hs[:, None, :]) & 1) << 2)
            out.append(codes.astype(np.uint8))
        return out[0], ks[blocks, :, :, r].copy(), out[1], vs[blocks, :, :, r].copy()

    # ------------------------------------------------------------- attention
    def add_replicas(self, n_total: int) -> None:
        """Clone the pools so that timed calls can rotate through n_total copies."""
        base = self.pools[0]
        while len(self.pools) < n_total:
            self.pools.append(Pools(*[None if t is None else t.clone() for t in
                                      (base.ek, base.ev, base.kc, base.vc, base.ks, base.vs)]))

    def desc(self, replica: int = 0, split_exact: Optional[int] = None, split_quant: Optional[int] = None,
             tables=None) -> akv.AttnDesc:
        w, P = self.w, self.pools[replica]
        et, qt = (self.exact_table, self.quant_table) if tables is None else tables
        exact = akv.ExactTier(k=ptr(P.ek), v=ptr(P.ev), block_table=ptr(et), lengths=ptr(self.exact_len),
                              max_blocks=self.emax, num_blocks=max(1, w.exact_pool_blocks))
        quant = akv.QuantTier(k_codes=ptr(P.kc), v_codes=ptr(P.vc), k_scales=ptr(P.ks), v_scales=ptr(P.vs),
                              block_table=ptr(qt), lengths=ptr(self.quant_len), max_blocks=self.qmax,
                              num_blocks=max(1, w.quant_pool_blocks))
        se = w.split_tokens_exact if split_exact is None else split_exact
        sq = w.split_tokens_quant if split_quant is None else split_quant
        return akv.AttnDesc(B=w.B, Hq=w.Hq, Hkv=w.Hkv, d=w.d, Tq=w.Tq, softmax_scale=0.0, q=ptr(self.q),
                            exact=exact, quant=quant, split_tokens_exact=se, split_tokens_quant=sq,
                            o=ptr(self.o), lse=ptr(self.lse), rotation=ptr(self.rotation), code_bits=self.width)

    def ensure_ws(self, desc: akv.AttnDesc, chunk: bool = False) -> None:
        need = (akv.akv_chunk_workspace_bytes if chunk else akv.akv_decode_workspace_bytes)(desc)
        if need == 0:
            raise akv.AKVError(akv.AKV_ERR_SHAPE, akv.akv_last_error())
        if need > self.ws_bytes:
            self.ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
            self.ws_bytes = need

    def attend(self, replica: int = 0, stream: Optional[int] = None, **kw) -> int:
        chunk = self.w.causal_tail > 0
        d = self.desc(replica, **kw)
        self.ensure_ws(d, chunk)
        fn = akv.akv_attend_chunk if chunk else akv.akv_attend_decode
        return fn(d, ptr(self.ws), self.ws_bytes, stream_handle() if stream is None else stream)

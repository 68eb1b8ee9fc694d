"""TurboQuant / SpectralQuant KV-cache and vector codec for MI355X (gfx950).

Thin Python layer over the C ABI of libtq.so (include/tq.h): it marshals
torch tensors (device memory, the current HIP stream) into the library's
entry points.  Every step of the codec runs in the library's HIP kernels;
there is no Python or CPU fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L
from ._lib import (TQ_BF16, TQ_F32, TQ_LAYOUT_COL, TQ_LAYOUT_ROW, TQ_MSE, TQ_PROD,
                   TQ_ROT_CALIBRATE, TQ_ROT_GIVEN, TQ_ROT_HAAR, TQ_ROT_HADAMARD, TQ_TILE, TQError)

__all__ = ["Codebook", "encode", "encode_kv", "append", "score", "decode_attend", "decode_step", "search_topk", "water_fill",
           "TQError",
           "TQ_MSE", "TQ_PROD", "TQ_LAYOUT_ROW", "TQ_LAYOUT_COL", "TQ_ROT_HAAR",
           "TQ_ROT_GIVEN", "TQ_ROT_CALIBRATE", "TQ_ROT_HADAMARD", "TQ_TILE"]


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


class Codebook:
    """A built codec (rotation(s), sketch, Lloyd-Max tables) on one device.

    device=-1 builds a host-only codebook, usable for export and layout queries.
    outlier_channels ([o] or [H][o]) with outlier_bits builds an outlier-channel
    split codec (two TurboQuant instances, `bits` on the other channels)."""

    def __init__(self, d: int, mode: int, bits: int, *, bitmap: Optional[Sequence[int]] = None,
                 qjl_dims: int = 0, rotation: int = TQ_ROT_HAAR, num_heads: int = 1,
                 layout: int = TQ_LAYOUT_ROW, seed_rotation: int = 0, seed_sketch: int = 0,
                 given: Optional[np.ndarray] = None, calib: Optional[np.ndarray] = None,
                 device: int = 0, waterfill_bits: int = 0,
                 outlier_channels: Optional[np.ndarray] = None, outlier_bits: int = 0):
        desc = L.CodebookDesc()
        desc.d, desc.mode, desc.bits = d, mode, bits
        keep = []
        if bitmap is not None:
            arr = np.ascontiguousarray(np.asarray(bitmap, dtype=np.uint8))
            keep.append(arr)
            desc.bitmap = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        desc.qjl_dims, desc.rotation, desc.num_heads, desc.layout = qjl_dims, rotation, num_heads, layout
        desc.seed_rotation, desc.seed_sketch = seed_rotation, seed_sketch
        if given is not None:
            g = np.ascontiguousarray(np.asarray(given, dtype=np.float32))
            keep.append(g)
            desc.given = g.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        if calib is not None:
            if isinstance(calib, torch.Tensor) and calib.is_cuda:
                # calibration moments on the device that holds the vectors
                c = calib.contiguous()
                if c.dtype not in (torch.bfloat16, torch.float32) or c.device.index != device:
                    raise ValueError("device calib: bf16 or fp32 on the codebook's device")
                desc.calib_dtype = TQ_BF16 if c.dtype == torch.bfloat16 else TQ_F32
                desc.calib_on_device = 1
                torch.cuda.synchronize(c.device)  # the build reads it on the null stream
                keep.append(c)
                desc.calib = c.data_ptr()
                desc.calib_n = c.shape[-2]
            elif isinstance(calib, torch.Tensor):
                if calib.dtype == torch.bfloat16:
                    c = np.ascontiguousarray(calib.cpu().view(torch.int16).numpy())
                    desc.calib_dtype = TQ_BF16
                else:
                    c = np.ascontiguousarray(calib.cpu().float().numpy())
                    desc.calib_dtype = TQ_F32
            else:
                c = np.ascontiguousarray(np.asarray(calib, dtype=np.float32))
                desc.calib_dtype = TQ_F32
            if not desc.calib_on_device:
                keep.append(c)
                desc.calib = c.ctypes.data
                desc.calib_n = c.shape[-2]
        desc.device = device
        desc.waterfill_bits = waterfill_bits
        if outlier_channels is not None:
            oc = np.ascontiguousarray(np.atleast_2d(np.asarray(outlier_channels, dtype=np.int32)))
            keep.append(oc)
            desc.outlier_dims, desc.outlier_bits = oc.shape[1], outlier_bits
            desc.outlier_channels = oc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            if num_heads == 1:
                desc.num_heads = oc.shape[0]
        h = ctypes.c_void_p()
        L.check(L.lib().tq_codebook_build(ctypes.byref(desc), ctypes.byref(h)), "tq_codebook_build")
        self._h = h
        self.device = device
        info = L.CodebookInfo()
        L.check(L.lib().tq_codebook_get_info(h, ctypes.byref(info)), "tq_codebook_get_info")
        self.info = info
        self.d, self.mode, self.m = info.d, info.mode, info.m
        self.num_heads, self.tile_bytes = info.num_heads, info.tile_bytes

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                L.lib().tq_codebook_free(h)
            except Exception:
                pass
            self._h = None

    def export(self, head: int = 0):
        """(rot [d][d] f32, sketch [m][m] f32 or None, centroids [d][32] f64,
        boundaries [d][31] f64, levels [d] i32) copied from the library."""
        d, m = self.d, self.m
        rot = np.zeros((d, d), np.float32)
        sk = np.zeros((max(m, 1), max(m, 1)), np.float32)
        cen = np.zeros((d, L.TQ_MAX_LEVELS), np.float64)
        thr = np.zeros((d, L.TQ_MAX_LEVELS - 1), np.float64)
        lv = np.zeros(d, np.int32)
        L.check(L.lib().tq_codebook_export(self._h, head, rot.ctypes.data, sk.ctypes.data,
                                           cen.ctypes.data, thr.ctypes.data, lv.ctypes.data),
                "tq_codebook_export")
        return rot, (sk if self.mode == TQ_PROD else None), cen, thr, lv

    def records_bytes(self, n: int) -> int:
        return int(L.lib().tq_records_bytes(self._h, n))

    def workspace(self, op: int, a: int, b: int, c: int = 0) -> int:
        return int(L.lib().tq_workspace_size(self._h, op, a, b, c))

    def alloc_records(self, n: int, sets: int = 1) -> torch.Tensor:
        return torch.zeros(sets * self.records_bytes(n), dtype=torch.uint8, device=f"cuda:{self.device}")


def append(cb: Codebook, x: torch.Tensor, records: torch.Tensor, positions: torch.Tensor,
           capacity: int) -> None:
    """Encode x [B][H][d] (one new vector per sequence and head) into slot
    positions[b] of the records of (b, h), which hold `capacity` tokens per
    (b, h) set laid out like encode()'s output of shape [B][H][capacity]."""
    if x.stride(-1) != 1:
        x = x.contiguous()
    B, H, d = x.shape
    s = x.stride()
    per = cb.records_bytes(capacity)
    pos = positions.to(device=x.device, dtype=torch.int32).contiguous()
    L.check(L.lib().tq_append(cb.handle, x.data_ptr(), _dtype_code(x), B, H, s[0], s[1], records.data_ptr(),
                              H * per, per, pos.data_ptr(), capacity, _stream(x.device)), "tq_append")


def water_fill(lam, total_bits: int, min_bits: int = 1, max_bits: int = 5) -> np.ndarray:
    """Per-dim index bits by discrete reverse water-filling over variances lam
    (host call of the library's tq_water_fill)."""
    lam = np.ascontiguousarray(np.asarray(lam, dtype=np.float64))
    out = np.zeros(len(lam), dtype=np.uint8)
    L.check(L.lib().tq_water_fill(lam.ctypes.data, len(lam), total_bits, min_bits, max_bits, out.ctypes.data),
            "tq_water_fill")
    return out


def encode(cb: Codebook, x: torch.Tensor, records: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Encode x of shape [T][d], [H][T][d] or [B][H][T][d] (fp32 or bf16, last dim
    contiguous).  Records of set (b, h) are contiguous; returns the uint8 buffer."""
    if x.dim() == 2:
        x4 = x.unsqueeze(0).unsqueeze(0)
    elif x.dim() == 3:
        x4 = x.unsqueeze(0)
    else:
        x4 = x
    B, H, T, d = x4.shape
    per = cb.records_bytes(T)
    if records is None:
        records = torch.empty(B * H * per, dtype=torch.uint8, device=x.device)
    s = x4.stride()
    ws_bytes = cb.workspace(L.TQ_OP_ENCODE, 0, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
    L.check(L.lib().tq_encode(cb.handle, x4.data_ptr(), _dtype_code(x4), B, H, T, s[0], s[1], s[2],
                              records.data_ptr(), H * per, per,
                              ws.data_ptr() if ws is not None else None, ws_bytes,
                              _stream(x.device)), "tq_encode")
    return records


def encode_kv(kcb: Codebook, vcb: Codebook, k: torch.Tensor, v: torch.Tensor,
              k_records: Optional[torch.Tensor] = None, v_records: Optional[torch.Tensor] = None):
    """Keys k and values v of one shape ([T][d], [H][T][d] or [B][H][T][d], same
    strides, fp32 or bf16) encoded together (tq_encode_kv): the records of
    encode(kcb, k) and encode(vcb, v).  Returns (k_records, v_records)."""
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("keys and values need one shape, stride and dtype")
    if not 2 <= k.dim() <= 4:
        raise ValueError("keys and values need 2 to 4 dims")
    k4, v4 = k, v
    while k4.dim() < 4:  # leading size-1 dims: views, never copies
        k4, v4 = k4.unsqueeze(0), v4.unsqueeze(0)
    B, H, T, d = k4.shape
    kper, vper = kcb.records_bytes(T), vcb.records_bytes(T)
    if k_records is None:
        k_records = torch.empty(B * H * kper, dtype=torch.uint8, device=k.device)
    if v_records is None:
        v_records = torch.empty(B * H * vper, dtype=torch.uint8, device=v.device)
    s = k4.stride()
    L.check(L.lib().tq_encode_kv(kcb.handle, vcb.handle, k4.data_ptr(), v4.data_ptr(), _dtype_code(k4),
                                 B, H, T, s[0], s[1], s[2], k_records.data_ptr(), H * kper, kper,
                                 v_records.data_ptr(), H * vper, vper, _stream(k.device)), "tq_encode_kv")
    return k_records, v_records


def score(cb: Codebook, q: torch.Tensor, records: torch.Tensor, n: int, head: int = 0) -> torch.Tensor:
    """[nq][n] fp32 estimated inner products of fp32 queries q [nq][d] with n records."""
    q = q.contiguous()
    nq = q.shape[0]
    out = torch.empty(nq, n, dtype=torch.float32, device=q.device)
    ws_bytes = cb.workspace(L.TQ_OP_SCORE, nq, n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    L.check(L.lib().tq_score(cb.handle, q.data_ptr(), nq, head, records.data_ptr(), n,
                             out.data_ptr(), ws.data_ptr(), ws_bytes, _stream(q.device)), "tq_score")
    return out


class DecodeWorkspace:
    """Reusable workspace for decode_attend (sized for B*Hq queries and max_tokens)."""

    def __init__(self, kcb: Codebook, nq_total: int, max_tokens: int, hkv: int, device):
        self.bytes = kcb.workspace(L.TQ_OP_DECODE, nq_total, max_tokens, hkv)
        self.buf = torch.empty(max(self.bytes, 16), dtype=torch.uint8, device=device)


def _kv_view(kcb, vcb, k_records, v_records, max_tokens, hkv, seq_lens, k_strides, v_strides,
             block_table, page_tiles):
    kper, vper = kcb.records_bytes(max_tokens), vcb.records_bytes(max_tokens)
    ks = k_strides or (hkv * kper, kper)
    vs = v_strides or (hkv * vper, vper)
    bt, mp = None, 0
    if block_table is not None:
        block_table = block_table.to(dtype=torch.int32).contiguous()
        bt, mp = block_table.data_ptr(), block_table.shape[-1]
    view = L.KVView(k_records.data_ptr(), v_records.data_ptr(), ks[0], ks[1], vs[0], vs[1],
                    max_tokens, seq_lens.data_ptr() if seq_lens is not None else None, bt, page_tiles, mp)
    return view, block_table


def decode_attend(kcb: Codebook, vcb: Codebook, q: torch.Tensor, k_records: torch.Tensor,
                  v_records: torch.Tensor, max_tokens: int, hkv: int, scale: float,
                  seq_lens: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[DecodeWorkspace] = None,
                  k_strides=None, v_strides=None, block_table: Optional[torch.Tensor] = None,
                  page_tiles: int = 1) -> torch.Tensor:
    """One decode step of GQA attention over compressed K/V records.

    q: [B][Hq][d] (fp32 or bf16).  Records of (b, g) are at b*Hkv*per + g*per
    unless strides (seq, head) in bytes are given; with block_table
    ([B*Hkv][max_pages] int32) the records are pools of pages of page_tiles
    tiles."""
    B, Hq, d = q.shape
    q = q.contiguous()
    view, _bt = _kv_view(kcb, vcb, k_records, v_records, max_tokens, hkv, seq_lens, k_strides, v_strides,
                         block_table, page_tiles)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = DecodeWorkspace(kcb, B * Hq, max_tokens, hkv, q.device)
    L.check(L.lib().tq_decode_attend(kcb.handle, vcb.handle, q.data_ptr(), _dtype_code(q), B, Hq,
                                     hkv, ctypes.byref(view), scale, out.data_ptr(),
                                     workspace.buf.data_ptr(), workspace.bytes, _stream(q.device)),
            "tq_decode_attend")
    return out


def decode_attend_noalloc(kcb: Codebook, vcb: Codebook, q: torch.Tensor, k_records: torch.Tensor,
                          v_records: torch.Tensor, max_tokens: int, hkv: int, scale: float,
                          out: torch.Tensor, seq_lens: Optional[torch.Tensor] = None,
                          k_strides=None, v_strides=None, block_table: Optional[torch.Tensor] = None,
                          page_tiles: int = 1) -> torch.Tensor:
    """decode_attend through the entry point that allocates nothing (its
    workspace is the library's own device array); `out` must be given."""
    B, Hq, d = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous (this call allocates nothing)")
    view, _bt = _kv_view(kcb, vcb, k_records, v_records, max_tokens, hkv, seq_lens, k_strides, v_strides,
                         block_table, page_tiles)
    L.check(L.lib().tq_decode_attend_noalloc(kcb.handle, vcb.handle, q.data_ptr(), _dtype_code(q), B, Hq, hkv,
                                             ctypes.byref(view), scale, out.data_ptr(), _stream(q.device)),
            "tq_decode_attend_noalloc")
    return out


def decode_step(kcb: Codebook, vcb: Codebook, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                k_records: torch.Tensor, v_records: torch.Tensor, max_tokens: int, hkv: int, scale: float,
                seq_lens: torch.Tensor, out: Optional[torch.Tensor] = None,
                workspace: Optional[DecodeWorkspace] = None, k_strides=None, v_strides=None,
                block_table: Optional[torch.Tensor] = None, page_tiles: int = 1) -> torch.Tensor:
    """Append k_new / v_new ([B][Hkv][d]) at slot seq_lens[b] of each
    (sequence, KV head), then attend over seq_lens[b] + 1 tokens (seq_lens is
    not changed).  Other arguments as for decode_attend."""
    B, Hq, d = q.shape
    q = q.contiguous()
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must have the same dtype")
    k_new, v_new = k_new.contiguous(), v_new.contiguous()
    view, _bt = _kv_view(kcb, vcb, k_records, v_records, max_tokens, hkv, seq_lens, k_strides, v_strides,
                         block_table, page_tiles)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = DecodeWorkspace(kcb, B * Hq, max_tokens, hkv, q.device)
    L.check(L.lib().tq_decode_step(kcb.handle, vcb.handle, q.data_ptr(), _dtype_code(q), k_new.data_ptr(),
                                   v_new.data_ptr(), _dtype_code(k_new), B, Hq, hkv, ctypes.byref(view), scale,
                                   out.data_ptr(), workspace.buf.data_ptr(), workspace.bytes,
                                   _stream(q.device)), "tq_decode_step")
    return out


def search_topk(cb: Codebook, q: torch.Tensor, records: torch.Tensor, n: int, k: int):
    """Top-k (scores [nq][k] fp32, ids [nq][k] int64) of fp32 queries q [nq][d]."""
    q = q.contiguous()
    nq = q.shape[0]
    s = torch.empty(nq, k, dtype=torch.float32, device=q.device)
    i = torch.empty(nq, k, dtype=torch.int64, device=q.device)
    ws_bytes = cb.workspace(L.TQ_OP_TOPK, nq, n, k)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    L.check(L.lib().tq_search_topk(cb.handle, q.data_ptr(), nq, records.data_ptr(), n, k,
                                   s.data_ptr(), i.data_ptr(), ws.data_ptr(), ws_bytes,
                                   _stream(q.device)), "tq_search_topk")
    return s, i

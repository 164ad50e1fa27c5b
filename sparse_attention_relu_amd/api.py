"""Thin Python binding over the C ABI: argument marshalling only.

Every function takes torch tensors already on the GPU, checks shapes and
dtypes, passes raw pointers and the current HIP stream to libsparse_mla, and
raises on a non-zero status.  All arithmetic happens in the HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib

IDX_HEADS, IDX_DIM, HEADS, ROW, LATENT, VDIM, MAX_TOPK = 32, 128, 64, 576, 512, 256, 2048


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (the library has no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None:
        for i, (a, b) in enumerate(zip(t.shape, shape)):
            if b is not None and a != b:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if len(t.shape) != len(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A caller-side workspace buffer (256-byte aligned by the allocator)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def layer_is_full(layer: int) -> bool:
    return _lib.lib().sa_layer_is_full(int(layer)) == 1


def indexer_score(q_idx, w, k_idx, seq_start, seq_len, q_seq, q_pos, ld: int, scores=None, algo: int = 0,
                  stream=None, library=None):
    n_q = q_idx.shape[0]
    _need(q_idx, "q_idx", torch.bfloat16, (n_q, IDX_HEADS, IDX_DIM))
    _need(w, "w", torch.float32, (n_q, IDX_HEADS))
    _need(k_idx, "k_idx", torch.bfloat16, (None, IDX_DIM))
    _need(seq_start, "seq_start", torch.int64, (None,))
    _need(seq_len, "seq_len", torch.int32, (seq_start.shape[0],))
    _need(q_seq, "q_seq", torch.int32, (n_q,))
    _need(q_pos, "q_pos", torch.int32, (n_q,))
    if scores is None:
        scores = torch.empty((n_q, ld), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, (n_q, ld))
    L = library if library is not None else _lib.lib()
    st = L.sa_indexer_score_algo(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(seq_start), _ptr(seq_len), _ptr(q_seq),
                                 _ptr(q_pos), n_q, seq_start.shape[0], _ptr(scores), ld, algo, _stream(stream))
    _lib.check("sa_indexer_score", st, L)
    return scores


def topk_select(scores, q_pos, k: int = MAX_TOPK, idx=None, ws=None, algo: int = 0, stream=None):
    n_q, ld = scores.shape
    _need(scores, "scores", torch.float32, (n_q, ld))
    _need(q_pos, "q_pos", torch.int32, (n_q,))
    L = _lib.lib()
    if idx is None:
        idx = torch.empty((n_q, k), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32, (n_q, k))
    nbytes = L.sa_topk_workspace_size(n_q, ld, k)
    if ws is None:
        ws = workspace(nbytes, scores.device)
    st = L.sa_topk_select_algo(_ptr(scores), ld, _ptr(q_pos), n_q, k, _ptr(idx), _ptr(ws), ws.numel(), algo,
                               _stream(stream))
    _lib.check("sa_topk_select", st)
    return idx


def mla_split_info(n_q: int, k: int):
    """sa_mla_split_info: (slices per query, selection entries per slice) of
    the attention's split of each query's selection."""
    n_sp, kps = ctypes.c_int32(), ctypes.c_int32()
    _lib.check("sa_mla_split_info", _lib.lib().sa_mla_split_info(n_q, k, ctypes.byref(n_sp), ctypes.byref(kps)))
    return n_sp.value, kps.value


def mla_partial_bits(n_q: int, k: int) -> int:
    """sa_mla_partial_bits: 0 (no partial states), 32 (fp32) or 16 (bf16)."""
    r = _lib.lib().sa_mla_partial_bits(n_q, k)
    if r < 0:
        _lib.check("sa_mla_partial_bits", r)
    return r


def mla_sparse_attn(q_abs, kv, seq_start, q_seq, idx, w_uv, scale: float = 1.0 / 16, out=None, lse=None, ws=None,
                    stream=None):
    n_q, k = idx.shape
    _need(q_abs, "q_abs", torch.bfloat16, (n_q, HEADS, ROW))
    _need(kv, "kv", torch.bfloat16, (None, ROW))
    _need(seq_start, "seq_start", torch.int64, (None,))
    _need(q_seq, "q_seq", torch.int32, (n_q,))
    _need(idx, "idx", torch.int32, (n_q, k))
    _need(w_uv, "w_uv", torch.bfloat16, (HEADS, VDIM, LATENT))
    if out is None:
        out = torch.empty((n_q, HEADS, VDIM), dtype=torch.bfloat16, device=q_abs.device)
    _need(out, "out", torch.bfloat16, (n_q, HEADS, VDIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (n_q, HEADS))
    L = _lib.lib()
    nbytes = L.sa_mla_workspace_size(n_q, k)
    if ws is None:
        ws = workspace(nbytes, q_abs.device)
    st = L.sa_mla_sparse_attn(_ptr(q_abs), _ptr(kv), _ptr(seq_start), _ptr(q_seq), _ptr(idx), n_q, k, _ptr(w_uv),
                              float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    _lib.check("sa_mla_sparse_attn", st)
    return out


def share_selection(sel_idx, sel_of, q_pos, idx=None, stream=None):
    """sa_share_selection: row sel_of[t] of sel_idx cut at q_pos[t]."""
    n_sel, k = sel_idx.shape
    n_q = sel_of.shape[0]
    _need(sel_idx, "sel_idx", torch.int32, (n_sel, k))
    _need(sel_of, "sel_of", torch.int32, (n_q,))
    _need(q_pos, "q_pos", torch.int32, (n_q,))
    if idx is None:
        idx = torch.empty((n_q, k), dtype=torch.int32, device=sel_idx.device)
    _need(idx, "idx", torch.int32, (n_q, k))
    L = _lib.lib()
    st = L.sa_share_selection(_ptr(sel_idx), n_sel, k, _ptr(sel_of), _ptr(q_pos), n_q, _ptr(idx), _stream(stream))
    _lib.check("sa_share_selection", st)
    return idx


def quantize_rows_fp8(src, codes=None, scales=None, dst_rows=None, stream=None):
    """sa_quantize_rows_fp8: bf16 rows [n, d] (d = 576 or 128) to E4M3 codes
    (uint8 [*, d]) and one fp32 scale per row."""
    n, d = src.shape
    _need(src, "src", torch.bfloat16, (n, d))
    dev = src.device
    if codes is None:
        codes = torch.empty((n, d), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((codes.shape[0],), dtype=torch.float32, device=dev)
    _need(codes, "codes", torch.uint8, (None, d))
    _need(scales, "scales", torch.float32, (codes.shape[0],))
    if dst_rows is not None:
        _need(dst_rows, "dst_rows", torch.int64, (n,))
    elif codes.shape[0] != n:
        raise ValueError("codes must have one row per source row when dst_rows is not given")
    L = _lib.lib()
    st = L.sa_quantize_rows_fp8(_ptr(src), n, d, _ptr(dst_rows), _ptr(codes), _ptr(scales), _stream(stream))
    _lib.check("sa_quantize_rows_fp8", st)
    return codes, scales


def fp8_decode(codes, out=None, stream=None):
    """sa_fp8_decode: E4M3 codes (uint8, a multiple of 16) to bf16 values."""
    _need(codes, "codes", torch.uint8)
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    _need(out, "out", torch.bfloat16, tuple(codes.shape))
    L = _lib.lib()
    _lib.check("sa_fp8_decode", L.sa_fp8_decode(_ptr(codes), codes.numel(), _ptr(out), _stream(stream)))
    return out


def indexer_score_fp8(q_idx, w, k_codes, k_scale, seq_start, seq_len, q_seq, q_pos, ld: int, scores=None,
                      algo: int = 0, stream=None):
    n_q = q_idx.shape[0]
    _need(q_idx, "q_idx", torch.bfloat16, (n_q, IDX_HEADS, IDX_DIM))
    _need(w, "w", torch.float32, (n_q, IDX_HEADS))
    _need(k_codes, "k_codes", torch.uint8, (None, IDX_DIM))
    _need(k_scale, "k_scale", torch.float32, (k_codes.shape[0],))
    _need(seq_start, "seq_start", torch.int64, (None,))
    _need(seq_len, "seq_len", torch.int32, (seq_start.shape[0],))
    _need(q_seq, "q_seq", torch.int32, (n_q,))
    _need(q_pos, "q_pos", torch.int32, (n_q,))
    if scores is None:
        scores = torch.empty((n_q, ld), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, (n_q, ld))
    L = _lib.lib()
    st = L.sa_indexer_score_fp8_algo(_ptr(q_idx), _ptr(w), _ptr(k_codes), _ptr(k_scale), _ptr(seq_start),
                                     _ptr(seq_len), _ptr(q_seq), _ptr(q_pos), n_q, seq_start.shape[0], _ptr(scores),
                                     ld, algo, _stream(stream))
    _lib.check("sa_indexer_score_fp8", st)
    return scores


def mla_sparse_attn_fp8(q_abs, kv_codes, kv_scale, seq_start, q_seq, idx, w_uv, scale: float = 1.0 / 16, out=None,
                        lse=None, ws=None, stream=None):
    n_q, k = idx.shape
    _need(q_abs, "q_abs", torch.bfloat16, (n_q, HEADS, ROW))
    _need(kv_codes, "kv_codes", torch.uint8, (None, ROW))
    _need(kv_scale, "kv_scale", torch.float32, (kv_codes.shape[0],))
    _need(seq_start, "seq_start", torch.int64, (None,))
    _need(q_seq, "q_seq", torch.int32, (n_q,))
    _need(idx, "idx", torch.int32, (n_q, k))
    _need(w_uv, "w_uv", torch.bfloat16, (HEADS, VDIM, LATENT))
    if out is None:
        out = torch.empty((n_q, HEADS, VDIM), dtype=torch.bfloat16, device=q_abs.device)
    _need(out, "out", torch.bfloat16, (n_q, HEADS, VDIM))
    if lse is not None:
        _need(lse, "lse", torch.float32, (n_q, HEADS))
    L = _lib.lib()
    if ws is None:
        ws = workspace(L.sa_mla_workspace_size(n_q, k), q_abs.device)
    st = L.sa_mla_sparse_attn_fp8(_ptr(q_abs), _ptr(kv_codes), _ptr(kv_scale), _ptr(seq_start), _ptr(q_seq),
                                  _ptr(idx), n_q, k, _ptr(w_uv), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                  ws.numel(), _stream(stream))
    _lib.check("sa_mla_sparse_attn_fp8", st)
    return out


QLORA = 2048


def q_project(c_q, w_qb, pos, w_iq=None, w_iw=None, q=None, q_idx=None, w=None, stream=None):
    """sa_q_project: q [n,64,256] (rope part turned), and with w_iq / w_iw the
    indexer query [n,32,128] and head weights [n,32] (fp32)."""
    n = c_q.shape[0]
    _need(c_q, "c_q", torch.bfloat16, (n, QLORA))
    _need(w_qb, "w_qb", torch.bfloat16, (HEADS * 256, QLORA))
    _need(pos, "pos", torch.int32, (n,))
    dev = c_q.device
    if q is None:
        q = torch.empty((n, HEADS, 256), dtype=torch.bfloat16, device=dev)
    _need(q, "q", torch.bfloat16, (n, HEADS, 256))
    if w_iq is not None:
        _need(w_iq, "w_iq", torch.bfloat16, (IDX_HEADS * IDX_DIM, QLORA))
        _need(w_iw, "w_iw", torch.bfloat16, (IDX_HEADS, QLORA))
        if q_idx is None:
            q_idx = torch.empty((n, IDX_HEADS, IDX_DIM), dtype=torch.bfloat16, device=dev)
        if w is None:
            w = torch.empty((n, IDX_HEADS), dtype=torch.float32, device=dev)
        _need(q_idx, "q_idx", torch.bfloat16, (n, IDX_HEADS, IDX_DIM))
        _need(w, "w", torch.float32, (n, IDX_HEADS))
    L = _lib.lib()
    st = L.sa_q_project(_ptr(c_q), _ptr(w_qb), _ptr(w_iq), _ptr(w_iw), _ptr(pos), n, _ptr(q), _ptr(q_idx), _ptr(w),
                        _stream(stream))
    _lib.check("sa_q_project", st)
    return q, q_idx, w


def q_absorb(q, w_uk_t, q_abs=None, stream=None):
    """sa_q_absorb: q_abs [n,64,576] = [W_UK^T q_nope ; q_rope] per head;
    w_uk_t is [64, 512, 192] (each head's key rows of kv_b_proj, transposed)."""
    n = q.shape[0]
    _need(q, "q", torch.bfloat16, (n, HEADS, 256))
    _need(w_uk_t, "w_uk_t", torch.bfloat16, (HEADS, LATENT, 192))
    if q_abs is None:
        q_abs = torch.empty((n, HEADS, ROW), dtype=torch.bfloat16, device=q.device)
    _need(q_abs, "q_abs", torch.bfloat16, (n, HEADS, ROW))
    L = _lib.lib()
    st = L.sa_q_absorb(_ptr(q), _ptr(w_uk_t), n, _ptr(q_abs), _stream(stream))
    _lib.check("sa_q_absorb", st)
    return q_abs


def cache_write(kv_a, gamma, pos, dst, kv_cache, k_raw=None, ln_w=None, ln_b=None, k_cache=None, stream=None):
    """sa_cache_write: the cache rows (and optionally the indexer keys) of n
    new tokens, written at rows dst of kv_cache (and k_cache)."""
    n = kv_a.shape[0]
    _need(kv_a, "kv_a", torch.bfloat16, (n, ROW))
    _need(gamma, "gamma", torch.bfloat16, (LATENT,))
    _need(pos, "pos", torch.int32, (n,))
    _need(dst, "dst", torch.int64, (n,))
    _need(kv_cache, "kv_cache", torch.bfloat16, (None, ROW))
    if k_raw is not None:
        _need(k_raw, "k_raw", torch.bfloat16, (n, IDX_DIM))
        _need(ln_w, "ln_w", torch.bfloat16, (IDX_DIM,))
        _need(ln_b, "ln_b", torch.bfloat16, (IDX_DIM,))
        _need(k_cache, "k_cache", torch.bfloat16, (None, IDX_DIM))
    L = _lib.lib()
    st = L.sa_cache_write(_ptr(kv_a), _ptr(gamma), _ptr(k_raw), _ptr(ln_w), _ptr(ln_b), _ptr(pos), _ptr(dst), n,
                          _ptr(kv_cache), _ptr(k_cache), _stream(stream))
    _lib.check("sa_cache_write", st)
    return kv_cache, k_cache


class LayerStack:
    """Pre-marshalled arguments of sa_layer_stack for a fixed set of tensors,
    so a step costs one foreign call (and can be captured in a HIP graph)."""

    def __init__(self, layers: Sequence, seq_start, seq_len, q_seq, q_pos, ld: int, k: int = MAX_TOPK,
                 scale: float = 1.0 / 16, full: Optional[List[bool]] = None, outs=None, idxs=None, ws=None,
                 library=None, sel=None):
        """sel: None, or (sel_seq, sel_pos, sel_of) int32 tensors of a shared
        selection (the full layers' q_idx and w then hold len(sel_seq) rows)."""
        n_q = q_pos.shape[0]
        n_sel = 0
        if sel is not None:
            sel_seq, sel_pos, sel_of = sel
            n_sel = sel_seq.shape[0]
            _need(sel_seq, "sel_seq", torch.int32, (n_sel,))
            _need(sel_pos, "sel_pos", torch.int32, (n_sel,))
            _need(sel_of, "sel_of", torch.int32, (n_q,))
        n_rows = n_sel if n_sel else n_q
        dev = q_pos.device
        if full is None:
            full = [layer_is_full(l) for l in range(len(layers))]
        _need(seq_start, "seq_start", torch.int64, (None,))
        _need(seq_len, "seq_len", torch.int32, (seq_start.shape[0],))
        _need(q_seq, "q_seq", torch.int32, (n_q,))
        _need(q_pos, "q_pos", torch.int32, (n_q,))
        self.outs = outs if outs is not None else [
            torch.empty((n_q, HEADS, VDIM), dtype=torch.bfloat16, device=dev) for _ in layers]
        self.idxs = idxs if idxs is not None else [
            torch.empty((n_q, k), dtype=torch.int32, device=dev) if f else None for f in full]
        descs = (_lib.LayerDesc * len(layers))()
        for l, (L, f) in enumerate(zip(layers, full)):
            d = descs[l]
            d.is_full = 1 if f else 0
            k_scale = getattr(L, "k_scale", None)
            kv_scale = getattr(L, "kv_scale", None)
            if f:
                _need(L.q_idx, "q_idx", torch.bfloat16, (n_rows, IDX_HEADS, IDX_DIM))
                _need(L.w, "w", torch.float32, (n_rows, IDX_HEADS))
                if k_scale is not None:           # FP8 indexer keys: codes + one scale per key
                    _need(L.k_idx, "k_idx", torch.uint8, (None, IDX_DIM))
                    _need(k_scale, "k_scale", torch.float32, (L.k_idx.shape[0],))
                    d.k_scale = _ptr(k_scale)
                else:
                    _need(L.k_idx, "k_idx", torch.bfloat16, (None, IDX_DIM))
                d.q_idx, d.w, d.k_idx, d.idx = _ptr(L.q_idx), _ptr(L.w), _ptr(L.k_idx), _ptr(self.idxs[l])
            _need(L.q_abs, "q_abs", torch.bfloat16, (n_q, HEADS, ROW))
            if kv_scale is not None:              # FP8 cache rows: codes + one scale per row
                _need(L.kv, "kv", torch.uint8, (None, ROW))
                _need(kv_scale, "kv_scale", torch.float32, (L.kv.shape[0],))
                d.kv_scale = _ptr(kv_scale)
            else:
                _need(L.kv, "kv", torch.bfloat16, (None, ROW))
            _need(L.w_uv, "w_uv", torch.bfloat16, (HEADS, VDIM, LATENT))
            d.q_abs, d.kv, d.w_uv, d.out = _ptr(L.q_abs), _ptr(L.kv), _ptr(L.w_uv), _ptr(self.outs[l])
        self._descs = descs
        self._batch = _lib.BatchDesc(_ptr(seq_start), _ptr(seq_len), _ptr(q_seq), _ptr(q_pos), n_q,
                                     seq_start.shape[0], int(ld), n_sel,
                                     *((_ptr(x) for x in sel) if sel is not None else (None, None, None)))
        self._keep = (layers, seq_start, seq_len, q_seq, q_pos, sel)
        self.lib = lib = library if library is not None else _lib.lib()
        nbytes = lib.sa_layer_stack_workspace_size(n_q, int(ld), k)
        self.ws = ws if ws is not None else workspace(nbytes, dev)
        self.n_layers, self.k, self.scale = len(layers), k, float(scale)
        self.full = full

    def __call__(self, events=None, stream=None):
        ev = None
        if events is not None:     # six raw hipEvent_t handles (ints) or None
            ev = _lib.StageEvents(*events)
        st = self.lib.sa_layer_stack(self._descs, self.n_layers, ctypes_byref(self._batch), self.k, self.scale,
                                     _ptr(self.ws), self.ws.numel(), ctypes_byref(ev) if ev is not None else None,
                                     _stream(stream))
        _lib.check("sa_layer_stack", st, self.lib)
        return self.outs, self.idxs


def ctypes_byref(x):
    import ctypes
    return ctypes.byref(x)


def layer_stack(layers, seq_start, seq_len, q_seq, q_pos, ld: int, k: int = MAX_TOPK, scale: float = 1.0 / 16,
                full=None, stream=None):
    return LayerStack(layers, seq_start, seq_len, q_seq, q_pos, ld, k, scale, full)(stream=stream)


def debug_check(stream=None, library=None):
    """sa_debug_check of the SA_DEBUG library (default): waits for the stream
    and raises SparseMLAError if a device-side precondition check failed."""
    L = library if library is not None else _lib.debug_lib()
    _lib.check("sa_debug_check", L.sa_debug_check(_stream(stream)), L)

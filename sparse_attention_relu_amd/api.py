"""Thin Python binding over the C ABI: argument marshalling only.

Every function takes torch tensors already on the GPU, checks shapes and
dtypes, passes raw pointers and the current HIP stream to libsparse_mla, and
raises on a non-zero status.  All arithmetic happens in the HIP kernels.
"""
from __future__ import annotations

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


def indexer_score(q_idx, w, k_idx, seq_start, q_seq, q_pos, ld: int, scores=None, algo: int = 0, stream=None):
    n_q = q_idx.shape[0]
    _need(q_idx, "q_idx", torch.bfloat16, (n_q, IDX_HEADS, IDX_DIM))
    _need(w, "w", torch.float32, (n_q, IDX_HEADS))
    _need(k_idx, "k_idx", torch.bfloat16, (None, IDX_DIM))
    _need(seq_start, "seq_start", torch.int64, (None,))
    _need(q_seq, "q_seq", torch.int32, (n_q,))
    _need(q_pos, "q_pos", torch.int32, (n_q,))
    if scores is None:
        scores = torch.empty((n_q, ld), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, (n_q, ld))
    st = _lib.lib().sa_indexer_score_algo(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(seq_start), _ptr(q_seq),
                                          _ptr(q_pos), n_q, seq_start.shape[0], _ptr(scores), ld, algo,
                                          _stream(stream))
    _lib.check("sa_indexer_score", st)
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

    def __init__(self, layers: Sequence, seq_start, q_seq, q_pos, ld: int, k: int = MAX_TOPK,
                 scale: float = 1.0 / 16, full: Optional[List[bool]] = None, outs=None, idxs=None, ws=None):
        n_q = q_pos.shape[0]
        dev = q_pos.device
        if full is None:
            full = [layer_is_full(l) for l in range(len(layers))]
        _need(seq_start, "seq_start", torch.int64, (None,))
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
            if f:
                _need(L.q_idx, "q_idx", torch.bfloat16, (n_q, IDX_HEADS, IDX_DIM))
                _need(L.w, "w", torch.float32, (n_q, IDX_HEADS))
                _need(L.k_idx, "k_idx", torch.bfloat16, (None, IDX_DIM))
                d.q_idx, d.w, d.k_idx, d.idx = _ptr(L.q_idx), _ptr(L.w), _ptr(L.k_idx), _ptr(self.idxs[l])
            _need(L.q_abs, "q_abs", torch.bfloat16, (n_q, HEADS, ROW))
            _need(L.kv, "kv", torch.bfloat16, (None, ROW))
            _need(L.w_uv, "w_uv", torch.bfloat16, (HEADS, VDIM, LATENT))
            d.q_abs, d.kv, d.w_uv, d.out = _ptr(L.q_abs), _ptr(L.kv), _ptr(L.w_uv), _ptr(self.outs[l])
        self._descs = descs
        self._batch = _lib.BatchDesc(_ptr(seq_start), _ptr(q_seq), _ptr(q_pos), n_q, seq_start.shape[0], int(ld))
        self._keep = (layers, seq_start, q_seq, q_pos)
        lib = _lib.lib()
        nbytes = lib.sa_layer_stack_workspace_size(n_q, int(ld), k)
        self.ws = ws if ws is not None else workspace(nbytes, dev)
        self.n_layers, self.k, self.scale = len(layers), k, float(scale)
        self.full = full

    def __call__(self, events=None, stream=None):
        ev = None
        if events is not None:     # six raw hipEvent_t handles (ints) or None
            ev = _lib.StageEvents(*events)
        st = _lib.lib().sa_layer_stack(self._descs, self.n_layers, ctypes_byref(self._batch), self.k, self.scale,
                                       _ptr(self.ws), self.ws.numel(), ctypes_byref(ev) if ev is not None else None,
                                       _stream(stream))
        _lib.check("sa_layer_stack", st)
        return self.outs, self.idxs


def ctypes_byref(x):
    import ctypes
    return ctypes.byref(x)


def layer_stack(layers, seq_start, q_seq, q_pos, ld: int, k: int = MAX_TOPK, scale: float = 1.0 / 16, full=None,
                stream=None):
    return LayerStack(layers, seq_start, q_seq, q_pos, ld, k, scale, full)(stream=stream)

"""Seeded synthetic inputs for the sparse MLA hot path.

This module only draws tensors; it holds none of the path's arithmetic (no
indexer score, selection, attention or up-projection).  Both the HIP path and
the CPU oracle consume exactly the tensors drawn here.

Shapes and distributions follow the model the pages describe
(models.inteligile.com "GLM-5.2 / Model techniques map", section "Checked in
its code"; llm-atlas "GLM-5.2", section "Champs bruts du config.json"):

  indexer key  k_idx  [T, 128]        LayerNorm(N(0,1)^128), gamma 1, beta 0,
                                      eps 1e-5 -> bf16 (the indexer key is the
                                      LayerNorm of a projection)
  indexer q    q_idx  [n_q, 32, 128]  N(0, 1/128) -> bf16
  head weights w      [n_q, 32]       N(0, 1/32), fp32
  cache row    kv     [T, 576]        [RMSNorm(N(0,1)^512), eps 1e-5 ;
                                       RoPE(N(0,1)^64, position, theta 8e6,
                                       interleaved pairs)] -> bf16
  folded query q_abs  [n_q, 64, 576]  N(0, 1/576) -> bf16
  up-projection w_uv  [64, 256, 512]  N(0, 1/512) -> bf16

Sequences are packed: row seq_start[b] + s of a cache holds position s of
sequence b.  No dataset or trained weight is involved; these seeded tensors
stand in for real caches and activations.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

IDX_HEADS, IDX_DIM = 32, 128
HEADS, LATENT, ROPE, VDIM = 64, 512, 64, 256
ROW = LATENT + ROPE


def full_layer_pattern(n_layers: int) -> List[bool]:
    """Which layers of a stack carry indexer inputs, expanded from the layer
    layout that llm-architectures-explained "GLM-5.2" prints (section "Every
    architecture field", row "layout"): three layers with an indexer, then
    eighteen groups of (three without, one with), then three without.  A stack
    shorter than 78 layers takes the prefix."""
    groups = [(3, True)] + [(3, False), (1, True)] * 18 + [(3, False)]
    flags: List[bool] = []
    for count, has_indexer in groups:
        flags += [has_indexer] * count
    if n_layers > len(flags):
        raise ValueError("the printed layout has 78 layers")
    return flags[:n_layers]


@dataclasses.dataclass
class Workload:
    name: str
    seq_lens: List[int]
    q_seq: List[int]
    q_pos: List[int]
    full: List[bool]
    k: int = 2048
    scale: float = 1.0 / 16.0
    note: str = ""

    @property
    def n_q(self) -> int:
        return len(self.q_seq)

    @property
    def n_seq(self) -> int:
        return len(self.seq_lens)

    @property
    def n_layers(self) -> int:
        return len(self.full)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def seq_start(self) -> List[int]:
        return [int(x) for x in np.concatenate([[0], np.cumsum(self.seq_lens)[:-1]])] if self.seq_lens else []

    @property
    def ld(self) -> int:
        """Length of a score row: one past the largest query position."""
        return int(max(self.q_pos)) + 1 if self.q_pos else 0


def workload(name: str, seed: int = 0) -> Workload:
    """The five measured configurations, plus small ones for tests."""
    if name == "c0":
        return Workload("decode_b1_4q_ctx4096_1layer", [4096], [0] * 4, [4092, 4093, 4094, 4095],
                        [True], note="single layer, 4 query tokens at the end of a 4096-token cache")
    if name == "c1":
        return Workload("decode_b64_ctx32768_4layer", [32768] * 64, list(range(64)), [32767] * 64,
                        [True, False, False, False])
    if name == "c2":
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = [int(x) for x in rng.integers(65536, 131072, size=16, endpoint=True)]
        return Workload("decode_b16_ctx65536-131072_4layer", lens, list(range(16)), [L - 1 for L in lens],
                        [True, False, False, False])
    if name == "c3":
        return Workload("prefill_4096q_on_126976_cached_4layer", [131072], [0] * 4096,
                        [126976 + i for i in range(4096)], [True, False, False, False])
    if name == "c4":
        return Workload("decode_b1_ctx1048576_78layer", [1048576], [0], [1048575], full_layer_pattern(78))
    raise KeyError(name)


def ragged_workload(seq_lens, queries, n_layers=1, k=2048, name="custom", full=None) -> Workload:
    """queries: list of (sequence, position)."""
    return Workload(name, list(seq_lens), [q for q, _ in queries], [p for _, p in queries],
                    full if full is not None else full_layer_pattern(n_layers), k=k)


def _gen(device, seed: int, layer: int, tag: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 1_009 + tag) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _randn(shape, g, device, std=1.0, dtype=torch.float32):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def _fill_rows(out: torch.Tensor, g, device, make_chunk, chunk_rows: int):
    n = out.shape[0]
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        out[r0:r1] = make_chunk(r1 - r0, r0, g)


def indexer_keys(total_tokens: int, g, device, chunk_rows=1 << 16) -> torch.Tensor:
    """[T, 128] indexer keys drawn i.i.d. N(0, 1): the law of a normalised key
    (zero mean and unit variance per row in expectation), without computing
    any normalisation here."""
    out = torch.empty((total_tokens, IDX_DIM), dtype=torch.bfloat16, device=device)

    def mk(n, r0, gg):
        return torch.randn((n, IDX_DIM), generator=gg, device=device).to(torch.bfloat16)

    _fill_rows(out, g, device, mk, chunk_rows)
    return out


def cache_rows(seq_lens, g, device, chunk_rows=1 << 16) -> torch.Tensor:
    """Packed [T, 576] rows drawn i.i.d. N(0, 1): a 512-d latent of unit RMS in
    expectation, then a 64-d rope key whose pairs are isotropic Gaussians, a law
    no rotation changes.  The arithmetic that turns projections into rows is
    the cache-write kernel's, not this module's."""
    T = int(sum(seq_lens))
    out = torch.empty((T, ROW), dtype=torch.bfloat16, device=device)

    def mk(n, r0, gg):
        return torch.randn((n, ROW), generator=gg, device=device).to(torch.bfloat16)

    _fill_rows(out, g, device, mk, chunk_rows)
    return out


@dataclasses.dataclass
class LayerInputs:
    q_abs: torch.Tensor
    kv: torch.Tensor
    w_uv: torch.Tensor
    q_idx: Optional[torch.Tensor] = None
    w: Optional[torch.Tensor] = None
    k_idx: Optional[torch.Tensor] = None
    kv_scale: Optional[torch.Tensor] = None     # set when kv holds FP8 codes
    k_scale: Optional[torch.Tensor] = None      # set when k_idx holds FP8 codes


@dataclasses.dataclass
class Batch:
    wl: Workload
    seq_start: torch.Tensor     # int64 [n_seq]
    seq_len: torch.Tensor       # int32 [n_seq]
    q_seq: torch.Tensor         # int32 [n_q]
    q_pos: torch.Tensor         # int32 [n_q]
    layers: List[LayerInputs]


def make_layer(wl: Workload, layer: int, device, seed: int = 0) -> LayerInputs:
    dev = torch.device(device)
    n_q, T = wl.n_q, wl.total_tokens
    L = LayerInputs(
        q_abs=_randn((n_q, HEADS, ROW), _gen(dev, seed, layer, 1), dev, std=1 / math.sqrt(ROW),
                     dtype=torch.bfloat16),
        kv=cache_rows(wl.seq_lens, _gen(dev, seed, layer, 2), dev),
        w_uv=_randn((HEADS, VDIM, LATENT), _gen(dev, seed, layer, 3), dev, std=1 / math.sqrt(LATENT),
                    dtype=torch.bfloat16),
    )
    if wl.full[layer]:
        L.q_idx = _randn((n_q, IDX_HEADS, IDX_DIM), _gen(dev, seed, layer, 4), dev,
                         std=1 / math.sqrt(IDX_DIM), dtype=torch.bfloat16)
        L.w = _randn((n_q, IDX_HEADS), _gen(dev, seed, layer, 5), dev, std=1 / math.sqrt(IDX_HEADS))
        L.k_idx = indexer_keys(T, _gen(dev, seed, layer, 6), dev)
    return L


def make_batch(wl: Workload, device, seed: int = 0, layers=None) -> Batch:
    dev = torch.device(device)
    layer_ids = range(wl.n_layers) if layers is None else layers
    return Batch(
        wl=wl,
        seq_start=torch.tensor(wl.seq_start, dtype=torch.int64, device=dev),
        seq_len=torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev),
        q_seq=torch.tensor(wl.q_seq, dtype=torch.int32, device=dev),
        q_pos=torch.tensor(wl.q_pos, dtype=torch.int32, device=dev),
        layers=[make_layer(wl, l, dev, seed) for l in layer_ids],
    )


def to_numpy(t: Optional[torch.Tensor]):
    """Exact widening for the oracle: bf16 and fp32 become float64 arrays,
    integer tensors become int64 arrays."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.is_floating_point():
        return t.to(torch.float64).numpy()
    return t.to(torch.int64).numpy()

"""Seeded synthetic inputs for the sparse MLA hot path.

This module only draws tensors; it holds none of the path's arithmetic (no
indexer score, selection, attention or up-projection).  Both the HIP path and
the CPU oracle consume exactly the tensors drawn here.

Shapes and distributions follow the model the pages describe
(models.inteligile.com "GLM-5.2 / Model techniques map", section "Checked in
its code"; llm-atlas "GLM-5.2", section "Champs bruts du config.json"):

  indexer key  k_idx  [T, 128]        LayerNorm(N(0,1)^128), weight 1, bias 0,
                                      eps 1e-5, dims 64..127 turned by RoPE at
                                      the row's position -> bf16
  indexer q    q_idx  [n_q, 32, 128]  N(0, 1/128) -> bf16
  head weights w      [n_q, 32]       N(0, 1/32), fp32
  cache row    kv     [T, 576]        [RMSNorm(N(0,1)^512), weight 1, eps 1e-5 ;
                                       RoPE(N(0,1)^64, position, theta 8e6,
                                       interleaved pairs)] -> bf16
  folded query q_abs  [n_q, 64, 576]  N(0, 1/576) -> bf16
  up-projection w_uv  [64, 256, 512]  N(0, 1/512) -> bf16

The cache rows and indexer keys are made the way a model makes them: raw
N(0, 1) projections are drawn here and the library's cache write
(sa_cache_write, whose own parity against the oracle is tested element by
element) normalises and rotates them into rows on the device.  A caller may
pass another row writer (make_batch's write_rows).

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


def norm_params(device):
    """kv_a_layernorm weight, k_norm weight and k_norm bias at their initial
    values (1, 1, 0): the written rows are the normalised projections."""
    dev = torch.device(device)
    return (torch.ones(LATENT, dtype=torch.bfloat16, device=dev), torch.ones(IDX_DIM, dtype=torch.bfloat16, device=dev),
            torch.zeros(IDX_DIM, dtype=torch.bfloat16, device=dev))


def positions(seq_lens, device) -> torch.Tensor:
    """int32 [T]: the position of each packed cache row within its sequence."""
    dev = torch.device(device)
    if not seq_lens:
        return torch.empty(0, dtype=torch.int32, device=dev)
    return torch.cat([torch.arange(int(n), dtype=torch.int32, device=dev) for n in seq_lens])


def raw_projection_chunks(seq_lens, g_kv, g_key, device, chunk_rows=1 << 16):
    """Chunks of the raw projections of every cached token, in packed row
    order: (kv_a [n, 576], k_raw [n, 128] or None, pos int32 [n], dst int64 [n])
    with kv_a and k_raw drawn i.i.d. N(0, 1) (k_raw only when g_key is given).
    Nothing is normalised or rotated here."""
    dev = torch.device(device)
    pos = positions(seq_lens, dev)
    T = pos.shape[0]
    for r0 in range(0, T, chunk_rows):
        n = min(T, r0 + chunk_rows) - r0
        kv_a = torch.randn((n, ROW), generator=g_kv, device=dev).to(torch.bfloat16)
        k_raw = None if g_key is None else torch.randn((n, IDX_DIM), generator=g_key, device=dev).to(torch.bfloat16)
        yield kv_a, k_raw, pos[r0:r0 + n], torch.arange(r0, r0 + n, dtype=torch.int64, device=dev)


def cache_write_rows(kv_a, k_raw, pos, dst, kv, k_idx, params):
    """The default row writer: the library's cache write (sa_cache_write) turns
    the raw projections into cache rows and indexer keys on the device."""
    from sparse_attention_relu_amd import api
    gamma, ln_w, ln_b = params
    api.cache_write(kv_a, gamma, pos, dst, kv, k_raw=k_raw, ln_w=ln_w if k_raw is not None else None,
                    ln_b=ln_b if k_raw is not None else None, k_cache=k_idx if k_raw is not None else None)


def law_rows(seq_lens, g_kv, g_key, device, write_rows=None, chunk_rows=1 << 16):
    """Cache rows kv [T, 576] (and indexer keys k_idx [T, 128] when g_key is
    given) of the stated law: raw N(0, 1) projections drawn here, written into
    rows by write_rows (default: the library's cache write)."""
    dev = torch.device(device)
    T = int(sum(seq_lens))
    kv = torch.empty((T, ROW), dtype=torch.bfloat16, device=dev)
    k_idx = None if g_key is None else torch.empty((T, IDX_DIM), dtype=torch.bfloat16, device=dev)
    params = norm_params(dev)
    write = write_rows or cache_write_rows
    for kv_a, k_raw, pos, dst in raw_projection_chunks(seq_lens, g_kv, g_key, dev, chunk_rows):
        write(kv_a, k_raw, pos, dst, kv, k_idx, params)
    return kv, k_idx


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


def make_layer(wl: Workload, layer: int, device, seed: int = 0, write_rows=None) -> LayerInputs:
    dev = torch.device(device)
    n_q = wl.n_q
    kv, k_idx = law_rows(wl.seq_lens, _gen(dev, seed, layer, 2), _gen(dev, seed, layer, 6) if wl.full[layer] else None,
                         dev, write_rows)
    L = LayerInputs(
        q_abs=_randn((n_q, HEADS, ROW), _gen(dev, seed, layer, 1), dev, std=1 / math.sqrt(ROW),
                     dtype=torch.bfloat16),
        kv=kv,
        w_uv=_randn((HEADS, VDIM, LATENT), _gen(dev, seed, layer, 3), dev, std=1 / math.sqrt(LATENT),
                    dtype=torch.bfloat16),
    )
    if wl.full[layer]:
        L.q_idx = _randn((n_q, IDX_HEADS, IDX_DIM), _gen(dev, seed, layer, 4), dev,
                         std=1 / math.sqrt(IDX_DIM), dtype=torch.bfloat16)
        L.w = _randn((n_q, IDX_HEADS), _gen(dev, seed, layer, 5), dev, std=1 / math.sqrt(IDX_HEADS))
        L.k_idx = k_idx
    return L


def make_batch(wl: Workload, device, seed: int = 0, layers=None, write_rows=None) -> Batch:
    dev = torch.device(device)
    layer_ids = range(wl.n_layers) if layers is None else layers
    return Batch(
        wl=wl,
        seq_start=torch.tensor(wl.seq_start, dtype=torch.int64, device=dev),
        seq_len=torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev),
        q_seq=torch.tensor(wl.q_seq, dtype=torch.int32, device=dev),
        q_pos=torch.tensor(wl.q_pos, dtype=torch.int32, device=dev),
        layers=[make_layer(wl, l, dev, seed, write_rows) for l in layer_ids],
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

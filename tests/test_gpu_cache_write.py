"""Cache-write kernel (sa_cache_write) against the CPU oracle, element by
element.  The kernel and the oracle both compute in fp64 and round once to
bf16, so they may differ only where a value lies within the last bits of a
bf16 rounding boundary (sin, cos, pow and the order of the sums are not
bit-identical between the two): at most one bf16 ulp, on a small fraction of
the elements."""
import numpy as np
import pytest
import torch

from oracle import ref
from sparse_attention_relu_amd import api
from sparse_attention_relu_amd.synth import to_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = -7.5        # rows the call must not touch keep this value


def _dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def _ordered(x):
    """bf16 values (as float64) to integers in value order (+0 and -0 equal)."""
    u = (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
    return np.where(u & 0x8000, -(u & 0x7FFF), u)


def _assert_ulp_close(got, want, what, max_frac=0.01):
    d = np.abs(_ordered(got) - _ordered(want))
    assert d.max() <= 1, f"{what}: {int(d.max())} bf16 ulps apart"
    frac = float(np.mean(d > 0))
    assert frac <= max_frac, f"{what}: {frac:.4f} of the values differ by one ulp"


def _case(n, n_rows, positions, seed, scale=1.0, with_key=True):
    r = np.random.default_rng(seed)
    kv_a = ref.round_to_bf16(scale * r.standard_normal((n, 576)))
    gamma = ref.round_to_bf16(1.0 + 0.1 * r.standard_normal(512))
    k_raw = ref.round_to_bf16(0.5 + 2.0 * r.standard_normal((n, 128)))
    ln_w = ref.round_to_bf16(1.0 + 0.2 * r.standard_normal(128))
    ln_b = ref.round_to_bf16(0.1 * r.standard_normal(128))
    dst = r.permutation(n_rows)[:n].astype(np.int64)
    pos = np.asarray(positions, dtype=np.int32)
    assert pos.shape == (n,)
    kv_cache = torch.full((n_rows, 576), SENTINEL, dtype=torch.bfloat16, device=DEV)
    k_cache = torch.full((n_rows, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    args = dict(kv_a=_dev_bf16(kv_a), gamma=_dev_bf16(gamma), pos=torch.from_numpy(pos).to(DEV),
                dst=torch.from_numpy(dst).to(DEV), kv_cache=kv_cache)
    if with_key:
        args.update(k_raw=_dev_bf16(k_raw), ln_w=_dev_bf16(ln_w), ln_b=_dev_bf16(ln_b), k_cache=k_cache)
    print(f"[cache_write] n={n} rows={n_rows} seed={seed} scale={scale} key={with_key}", flush=True)
    api.cache_write(**args)
    torch.cuda.synchronize()
    want_rows = ref.cache_rows_from_projection(kv_a, gamma, pos)
    want_keys = ref.indexer_keys_from_projection(k_raw, ln_w, ln_b, pos)
    return to_numpy(kv_cache), to_numpy(k_cache), dst, want_rows, want_keys


def _untouched(cache, dst):
    keep = np.ones(cache.shape[0], dtype=bool)
    keep[dst] = False
    return np.all(cache[keep] == SENTINEL)


@pytest.mark.parametrize("n", [1, 5, 37])
def test_cache_write_matches_oracle(gpu_lib, n):
    r = np.random.default_rng(100 + n)
    positions = np.concatenate([[0, 1, (1 << 20) - 1], r.integers(0, 1 << 20, size=max(n - 3, 0))])[:n]
    kv, kc, dst, want_rows, want_keys = _case(n, 3 * n + 11, positions, seed=n)
    _assert_ulp_close(kv[dst], want_rows, "cache rows")
    _assert_ulp_close(kc[dst], want_keys, "indexer keys")
    assert _untouched(kv, dst) and _untouched(kc, dst)


@pytest.mark.parametrize("scale", [1e-3, 30.0])
def test_cache_write_input_scale(gpu_lib, scale):
    kv, kc, dst, want_rows, want_keys = _case(16, 40, list(range(0, 160, 10)), seed=7, scale=scale)
    _assert_ulp_close(kv[dst], want_rows, "cache rows")
    _assert_ulp_close(kc[dst], want_keys, "indexer keys")


def test_cache_write_without_indexer_key(gpu_lib):
    kv, kc, dst, want_rows, _ = _case(9, 20, [3, 1, 4, 1, 5, 9, 2, 6, 5], seed=11, with_key=False)
    _assert_ulp_close(kv[dst], want_rows, "cache rows")
    assert np.all(kc == SENTINEL)


def test_cache_write_empty(gpu_lib):
    kv_cache = torch.full((4, 576), SENTINEL, dtype=torch.bfloat16, device=DEV)
    empty = torch.empty((0, 576), dtype=torch.bfloat16, device=DEV)
    api.cache_write(empty, torch.ones(512, dtype=torch.bfloat16, device=DEV),
                    torch.empty(0, dtype=torch.int32, device=DEV), torch.empty(0, dtype=torch.int64, device=DEV),
                    kv_cache)
    torch.cuda.synchronize()
    assert bool((kv_cache == SENTINEL).all())


def test_cache_write_prefill_chunk_sampled(gpu_lib):
    # a 4096-token chunk at positions 126,976..131,071 (the chunked-prefill
    # shape), written into a 131,072-row cache; 96 rows checked one by one
    n, rows = 4096, 131072
    positions = np.arange(126976, 131072)
    kv, kc, dst, want_rows, want_keys = _case(n, rows, positions, seed=3)
    pick = np.random.default_rng(5).choice(n, size=96, replace=False)
    _assert_ulp_close(kv[dst[pick]], want_rows[pick], "cache rows")
    _assert_ulp_close(kc[dst[pick]], want_keys[pick], "indexer keys")


def test_synthetic_rows_follow_the_stated_law(gpu_lib):
    """The seeded batches' cache rows and indexer keys are the oracle's cache
    write of the raw N(0, 1) projections drawn for them (weight 1, bias 0):
    RMS-normalised latents with rotated rope keys, LayerNorm'd indexer keys."""
    from sparse_attention_relu_amd import synth
    wl = synth.ragged_workload([300, 70000, 5], [(0, 299), (1, 69999), (2, 4)], n_layers=1)
    seed = 11
    b = synth.make_batch(wl, DEV, seed=seed)
    kv, k_idx = to_numpy(b.layers[0].kv), to_numpy(b.layers[0].k_idx)
    dev = torch.device(DEV)
    chunks = synth.raw_projection_chunks(wl.seq_lens, synth._gen(dev, seed, 0, 2), synth._gen(dev, seed, 0, 6), dev)
    starts = wl.seq_start
    checked = 0
    for kv_a, k_raw, pos, dst in chunks:
        d = to_numpy(dst)
        # rows at each sequence's start and end, and a spread in between
        pick = np.unique(np.concatenate([np.arange(0, len(d), 997), [len(d) - 1]] +
                                        [np.nonzero((d >= s0) & (d < s0 + 3))[0] for s0 in starts]))
        p = to_numpy(pos)[pick]
        assert np.array_equal(p, d[pick] - np.array([starts[np.searchsorted(starts, r, side="right") - 1]
                                                     for r in d[pick]]))
        want_rows = ref.cache_rows_from_projection(to_numpy(kv_a)[pick], np.ones(512), p)
        want_keys = ref.indexer_keys_from_projection(to_numpy(k_raw)[pick], np.ones(128), np.zeros(128), p)
        _assert_ulp_close(kv[d[pick]], want_rows, "synthetic cache rows", max_frac=0.02)
        _assert_ulp_close(k_idx[d[pick]], want_keys, "synthetic indexer keys", max_frac=0.02)
        checked += len(pick)
    assert checked >= 70
    lat = kv[:, :512]
    rms = np.sqrt(np.mean(lat * lat, axis=1))
    assert np.all(np.abs(rms - 1.0) < 0.01), "latents are not RMS-normalised"
    # LayerNorm gives each key a unit mean square, which the rotation of its
    # pairs keeps
    ms = np.mean(k_idx * k_idx, axis=1)
    assert np.all(np.abs(ms - 1.0) < 0.01), "indexer keys are not LayerNorm'd"

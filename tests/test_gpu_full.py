"""Parity at the measured configurations' full sizes, in the launch
configuration the benchmark times (sa_layer_stack).  Where the oracle cannot
recompute everything in seconds, it checks sampled rows one by one."""
import numpy as np
import pytest
import torch

from oracle import ref
from sparse_attention_relu_amd import api, synth
from sparse_attention_relu_amd.synth import to_numpy
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _compact_rows(kv, seq_start_b, idx_row):
    """The selected rows of one query as a small array, and idx remapped to it."""
    sel = idx_row[idx_row >= 0]
    rows = to_numpy(kv[torch.as_tensor(sel, device=kv.device) + int(seq_start_b)])
    return rows, np.arange(len(sel))


def _check_mla_compact(L, wl, idx, out, queries):
    """Oracle attention for chosen queries using only their gathered rows."""
    qa = to_numpy(L.q_abs[list(queries)])
    wuv = to_numpy(L.w_uv)
    rows_all, idx_loc, starts = [], np.full((len(queries), idx.shape[1]), -1), []
    off = 0
    for j, t in enumerate(queries):
        rows, loc = _compact_rows(L.kv, wl.seq_start[wl.q_seq[t]], idx[t])
        rows_all.append(rows)
        idx_loc[j, :len(loc)] = loc
        starts.append(off)
        off += len(rows)
    Lnp = {"q_abs": qa, "kv": np.concatenate(rows_all), "w_uv": wuv}
    B = {"seq_start": np.array(starts), "q_seq": np.arange(len(queries)), "q_pos": None}
    return parity.check_mla(Lnp, B, idx_loc, out[list(queries)], wl.scale, n_launch=wl.n_q)


def _run_stack(wl, seed=0):
    b = synth.make_batch(wl, DEV, seed=seed)
    stack = api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    outs, idxs = stack()
    torch.cuda.synchronize()
    return b, stack, outs, idxs


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_decode_config_full(gpu_lib, name):
    wl = synth.workload(name)
    b, stack, outs, idxs = _run_stack(wl)
    L0 = b.layers[0]
    sc = api.indexer_score(L0.q_idx, L0.w, L0.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx_sep = api.topk_select(sc, b.q_pos)
    torch.cuda.synchronize()
    assert torch.equal(idx_sep, idxs[0]), "layer_stack selection differs from the separate calls"
    B = parity.np_batch(b)
    Lnp = {"q_idx": to_numpy(L0.q_idx), "w": to_numpy(L0.w), "k_idx": to_numpy(L0.k_idx)}
    sc_np = to_numpy(sc)
    worst = parity.check_scores(Lnp, B, sc_np)
    parity.check_topk_exact(sc_np, B["q_pos"], 2048, to_numpy(idxs[0]))
    parity.check_topk_band(Lnp, B, to_numpy(idxs[0]), 2048)
    idx_np = to_numpy(idxs[0])
    for l, L in enumerate(b.layers):
        _check_mla_compact(L, wl, idx_np, to_numpy(outs[l]), range(wl.n_q))
    print(f"{name}: indexer worst |err|/bound {worst:.3g}")


@pytest.mark.timeout(600)
def test_prefill_config_sampled(gpu_lib):
    wl = synth.workload("c3")
    b, stack, outs, idxs = _run_stack(wl)
    L0 = b.layers[0]
    sc = api.indexer_score(L0.q_idx, L0.w, L0.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(3))
    rows = sorted(set([0, 1, 2047, 4095] + list(rng.choice(wl.n_q, 12, replace=False))))
    B = parity.np_batch(b)
    Lnp = {"q_idx": to_numpy(L0.q_idx), "w": to_numpy(L0.w), "k_idx": to_numpy(L0.k_idx)}
    sc_rows = to_numpy(sc[rows])
    sub = lambda a: a[rows]
    Bs = {"seq_start": B["seq_start"], "q_seq": sub(B["q_seq"]), "q_pos": sub(B["q_pos"])}
    Ls = {"q_idx": sub(Lnp["q_idx"]), "w": sub(Lnp["w"]), "k_idx": Lnp["k_idx"]}
    parity.check_scores(Ls, Bs, sc_rows)
    idx_np = to_numpy(idxs[0])
    parity.check_topk_exact(sc_rows, Bs["q_pos"], 2048, idx_np[rows])
    parity.check_topk_band(Ls, Bs, idx_np[rows], 2048)
    # the whole selection: valid, ascending, within the causal set
    assert np.all(np.diff(idx_np, axis=1) > 0)
    assert np.all(idx_np[:, 0] >= 0) and np.all(idx_np.max(axis=1) <= B["q_pos"])
    for l, L in enumerate(b.layers):
        _check_mla_compact(L, wl, idx_np, to_numpy(outs[l]), rows[:8])


@pytest.mark.timeout(900)
def test_decode_1m_78_layers(gpu_lib):
    wl = synth.workload("c4")
    free, total = torch.cuda.mem_get_info()
    need = 78 * wl.total_tokens * 1152 + 21 * wl.total_tokens * 256 + (4 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free")
    b, stack, outs, idxs = _run_stack(wl)
    full_layers = [l for l in range(78) if wl.full[l]]
    assert len(full_layers) == 21 and [api.layer_is_full(l) for l in range(78)] == wl.full
    B = parity.np_batch(b)
    for l in (full_layers[0], full_layers[-1]):
        L = b.layers[l]
        sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
        torch.cuda.synchronize()
        sc_np = to_numpy(sc)
        Lnp = {"q_idx": to_numpy(L.q_idx), "w": to_numpy(L.w), "k_idx": to_numpy(L.k_idx)}
        parity.check_scores(Lnp, B, sc_np)
        parity.check_topk_exact(sc_np, B["q_pos"], 2048, to_numpy(idxs[l]))
        parity.check_topk_band(Lnp, B, to_numpy(idxs[l]), 2048)
        del Lnp, sc
    for l in range(78):
        src = ref.shared_source(l)
        _check_mla_compact(b.layers[l], wl, to_numpy(idxs[src]), to_numpy(outs[l]), [0])

"""Shared selection for speculative / multi-token-prediction decode on the GPU
against the oracle: the selecting queries' indexer scores, their exact top-k,
the per-token rows cut at each token's position (bit-exact), and every
layer's attention over those rows."""
import numpy as np
import pytest
import torch

from oracle import ref
from sparse_attention_relu_amd import _lib, api, synth
from sparse_attention_relu_amd.synth import to_numpy
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _i32(x):
    return torch.tensor(x, dtype=torch.int32, device=DEV)


def _run_and_check(wl, sel_seq, sel_pos, sel_of, seed):
    """wl: token batch; the full layers' q_idx / w are taken from the
    selecting tokens' rows (each selecting query is one of the tokens)."""
    b = synth.make_batch(wl, DEV, seed=seed)
    tok_of_sel = [next(t for t in range(wl.n_q) if wl.q_seq[t] == s and wl.q_pos[t] == p)
                  for s, p in zip(sel_seq, sel_pos)]
    layers = []
    for L in b.layers:
        L2 = synth.LayerInputs(q_abs=L.q_abs, kv=L.kv, w_uv=L.w_uv, k_idx=L.k_idx)
        if L.q_idx is not None:
            L2.q_idx = L.q_idx[tok_of_sel].contiguous()
            L2.w = L.w[tok_of_sel].contiguous()
        layers.append(L2)
    sel = (_i32(sel_seq), _i32(sel_pos), _i32(sel_of))
    stack = api.LayerStack(layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full, sel=sel)
    outs, idxs = stack()
    torch.cuda.synchronize()
    B = parity.np_batch(b)
    Bs = {"seq_start": B["seq_start"], "q_seq": np.array(sel_seq), "q_pos": np.array(sel_pos)}
    for l, L in enumerate(layers):
        if not wl.full[l]:
            continue
        # the selecting queries' scores and selection, checked as in the plain path
        sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, sel[0], sel[1], wl.ld)
        src = api.topk_select(sc, sel[1])
        torch.cuda.synchronize()
        Lnp = {"q_idx": to_numpy(L.q_idx), "w": to_numpy(L.w), "k_idx": to_numpy(L.k_idx)}
        sc_np, src_np = to_numpy(sc), to_numpy(src)
        parity.check_scores(Lnp, Bs, sc_np)
        parity.check_topk_exact(sc_np, Bs["q_pos"], 2048, src_np)
        parity.check_topk_band(Lnp, Bs, src_np, 2048)
        # the per-token rows: exactly the oracle's cut of the GPU's shared rows
        expect = ref.share_selection(src_np, sel_of, wl.q_pos)
        assert np.array_equal(to_numpy(idxs[l]), expect), f"layer {l}: shared rows differ from the oracle's cut"
    cur = None
    for l, L in enumerate(layers):
        if wl.full[l]:
            cur = to_numpy(idxs[l])
        Lm = {"q_abs": to_numpy(L.q_abs), "kv": to_numpy(L.kv), "w_uv": to_numpy(L.w_uv)}
        parity.check_mla(Lm, B, cur, to_numpy(outs[l]), wl.scale)
    return stack, outs, idxs


def test_mtp_four_drafts_share_the_last_tokens_selection(gpu_lib):
    # 4 query tokens at the end of a 4096-token cache; the last one selects
    wl = synth.workload("c0")
    wl.full = [True, False]
    _run_and_check(wl, [0], [4095], [0, 0, 0, 0], seed=41)


def test_mtp_mixed_groups(gpu_lib):
    # sequence 0: 3 drafts (the last selects), sequence 1: 2 drafts (the first
    # selects), sequence 2: one token selecting for itself; two full layers
    lens = [6000, 3000, 9000]
    queries = [(0, 5997), (0, 5998), (0, 5999), (1, 2998), (1, 2999), (2, 8999)]
    wl = synth.ragged_workload(lens, queries, name="mtp_mixed", full=[True, False, False, True])
    stack, outs, idxs = _run_and_check(wl, [0, 1, 2], [5999, 2998, 8999], [0, 0, 0, 1, 1, 2], seed=43)
    # graph replay of the shared-selection stack equals the eager call
    ref_o = [o.clone() for o in outs]
    ref_i = idxs[0].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            stack()
    torch.cuda.synchronize()
    for rep in range(2):
        idxs[0].fill_(-7)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idxs[0], ref_i), rep
        for a, c in zip(outs, ref_o):
            assert torch.equal(a, c), rep


@pytest.mark.parametrize("k", [1, 7, 300, 2048])
def test_share_selection_call_matches_oracle(gpu_lib, k):
    # rows in any order, with -1 anywhere; positions up to 9,000
    rng = np.random.Generator(np.random.PCG64(k))
    n_sel, n_q = 3, 11
    sel_idx = rng.integers(-1, 9000, size=(n_sel, k)).astype(np.int32)
    sel_idx[rng.random((n_sel, k)) < 0.2] = -1
    sel_of = rng.integers(0, n_sel, size=n_q).astype(np.int32)
    q_pos = rng.integers(0, 9000, size=n_q).astype(np.int32)
    q_pos[0] = 8999
    q_pos[1] = 0
    got = api.share_selection(torch.from_numpy(sel_idx).to(DEV), torch.from_numpy(sel_of).to(DEV),
                              torch.from_numpy(q_pos).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(got), ref.share_selection(sel_idx, sel_of, q_pos))


def test_debug_build_reports_bad_sharing(gpu_lib):
    D = _lib.debug_lib()
    sel_idx = torch.arange(16, dtype=torch.int32, device=DEV).reshape(2, 8)
    sel_of = _i32([0, 1, 5])                # 5 is outside [0, 2): the kernel clamps it
    q_pos = _i32([3, 10, 12])
    idx = torch.empty((3, 8), dtype=torch.int32, device=DEV)
    st = D.sa_share_selection(sel_idx.data_ptr(), 2, 8, sel_of.data_ptr(), q_pos.data_ptr(), 3, idx.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    _lib.check("sa_share_selection", st, D)
    with pytest.raises(_lib.SparseMLAError) as e:
        api.debug_check(library=D)
    assert "sel_of outside" in str(e.value) and "item 2" in str(e.value) and "value 5" in str(e.value)

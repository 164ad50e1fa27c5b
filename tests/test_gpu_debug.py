"""The SA_DEBUG library on the GPU: a valid stack passes its device-side checks
and gives the release library's results bit for bit; preconditions broken
from the host (in ways every kernel still handles in bounds) are reported by
sa_debug_check with the check, the item and the value."""
import numpy as np
import pytest
import torch

from sparse_attention_relu_amd import _lib, api, synth
from sparse_attention_relu_amd.synth import to_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _wl():
    lens = [3000, 700, 2500]
    return synth.ragged_workload(lens, [(0, 2999), (1, 699), (2, 1800), (0, 100)], n_layers=4)


def test_valid_stack_passes_and_matches_release(gpu_lib):
    D = _lib.debug_lib()
    assert D.sa_debug_enabled() == 1
    wl = _wl()
    b = synth.make_batch(wl, DEV, seed=3)
    rel = api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    dbg = api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full, library=D)
    o_r, i_r = rel()
    o_d, i_d = dbg()
    api.debug_check(library=D)               # raises on any recorded violation
    torch.cuda.synchronize()
    assert torch.equal(i_r[0], i_d[0])
    for a, c in zip(o_r, o_d):
        assert torch.equal(a, c)


def test_query_past_its_sequence_is_reported_and_clamped(gpu_lib):
    D = _lib.debug_lib()
    wl = _wl()
    b = synth.make_batch(wl, DEV, seed=4)
    L = b.layers[0]
    ok = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, library=D)
    api.debug_check(library=D)
    bad_pos = b.q_pos.clone()
    bad_pos[1] = 700 + 40                   # sequence 1 holds 700 keys; ld is 3000
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, bad_pos, wl.ld, library=D)
    with pytest.raises(_lib.SparseMLAError) as e:
        api.debug_check(library=D)
    assert e.value.status == -5
    msg = str(e.value)
    assert "seq_len" in msg and "item 1" in msg and "value 740" in msg, msg
    api.debug_check(library=D)               # the record was cleared by the previous check
    # the indexer read no key past the sequence: scores up to its last key
    # match the valid call, everything after is -inf
    torch.cuda.synchronize()
    assert torch.equal(sc[1, :700], ok[1, :700])
    assert torch.all(torch.isneginf(sc[1, 700:]))


def test_bad_selection_entry_is_reported(gpu_lib):
    D = _lib.debug_lib()
    wl = _wl()
    b = synth.make_batch(wl, DEV, seed=5)
    L = b.layers[0]
    idx = torch.full((wl.n_q, 16), -1, dtype=torch.int32, device=DEV)
    idx[:, 0] = 3
    idx[2, 5] = -2                          # below -1: the kernels skip it as padding
    D_out = torch.empty((wl.n_q, 64, 256), dtype=torch.bfloat16, device=DEV)
    ws = api.workspace(D.sa_mla_workspace_size(wl.n_q, 16), DEV)
    st = D.sa_mla_sparse_attn(L.q_abs.data_ptr(), L.kv.data_ptr(), b.seq_start.data_ptr(), b.q_seq.data_ptr(),
                              idx.data_ptr(), wl.n_q, 16, L.w_uv.data_ptr(), 1.0 / 16, D_out.data_ptr(), None,
                              ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    _lib.check("sa_mla_sparse_attn", st, D)
    with pytest.raises(_lib.SparseMLAError) as e:
        api.debug_check(library=D)
    msg = str(e.value)
    assert "idx entry" in msg and "item 2, slot 5, value -2" in msg, msg


def test_nan_score_is_reported(gpu_lib):
    D = _lib.debug_lib()
    sc = torch.randn((3, 5000), device=DEV)
    sc[1, 1234] = float("nan")
    sc[2, 4000] = float("nan")              # past q_pos[2]: not read, not reported
    q_pos = torch.tensor([4999, 3000, 3999], dtype=torch.int32, device=DEV)
    idx = torch.empty((3, 2048), dtype=torch.int32, device=DEV)
    ws = api.workspace(D.sa_topk_workspace_size(3, 5000, 2048), DEV)
    st = D.sa_topk_select(sc.data_ptr(), 5000, q_pos.data_ptr(), 3, 2048, idx.data_ptr(), ws.data_ptr(), ws.numel(),
                          torch.cuda.current_stream().cuda_stream)
    _lib.check("sa_topk_select", st, D)
    with pytest.raises(_lib.SparseMLAError) as e:
        api.debug_check(library=D)
    msg = str(e.value)
    assert "NaN" in msg and "item 1, slot 1234" in msg and "1 violation" in msg, msg
    idx_np = to_numpy(idx)
    assert np.all(idx_np[0] >= 0)            # the call itself still ran

"""sa_layer_stack_noalloc (static per-GPU scratch, no workspace argument)
against sa_layer_stack through the C ABI: bit-identical selections and
outputs on two calls in a row, the second with a smaller batch, and the size
limit rejected before anything runs."""
import ctypes

import pytest
import torch

from sparse_attention_relu_amd import _lib, api, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _stack(wl, seed):
    b = synth.make_batch(wl, DEV, seed=seed)
    return b, api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)


def _noalloc(L, stack):
    outs = [torch.full_like(o, 7.0) for o in stack.outs]
    idxs = [torch.full_like(i, -7) if i is not None else None for i in stack.idxs]
    descs = (_lib.LayerDesc * stack.n_layers)()
    for l in range(stack.n_layers):
        ctypes.memmove(ctypes.byref(descs[l]), ctypes.byref(stack._descs[l]), ctypes.sizeof(_lib.LayerDesc))
        descs[l].out = outs[l].data_ptr()
        if idxs[l] is not None:
            descs[l].idx = idxs[l].data_ptr()
    st = L.sa_layer_stack_noalloc(descs, stack.n_layers, ctypes.byref(stack._batch), stack.k, stack.scale, None,
                                  torch.cuda.current_stream().cuda_stream)
    _lib.check("sa_layer_stack_noalloc", st)
    return outs, idxs


def _compare(L, wl, seed):
    b, stack = _stack(wl, seed)
    assert L.sa_layer_stack_workspace_size(wl.n_q, wl.ld, 2048) <= L.sa_layer_stack_noalloc_max_bytes()
    ref_o, ref_i = stack()
    ref_o = [o.clone() for o in ref_o]
    ref_i = [i.clone() if i is not None else None for i in ref_i]
    got_o, got_i = _noalloc(L, stack)
    torch.cuda.synchronize()
    for l in range(wl.n_layers):
        if ref_i[l] is not None:
            assert torch.equal(got_i[l], ref_i[l]), f"layer {l} selection"
        assert torch.equal(got_o[l], ref_o[l]), f"layer {l} output"


def test_noalloc_matches_layer_stack_twice(gpu_lib):
    L = gpu_lib
    # first call: 16 decode queries over ragged sequences up to 40,000 keys
    lens = [40000, 25000, 33000, 12000] * 4
    big = synth.ragged_workload(lens, [(i, lens[i] - 1 - 3 * i) for i in range(16)], n_layers=4)
    _compare(L, big, seed=31)
    # second call, smaller: the scratch holds the first call's contents
    lens = [3000, 700, 2500]
    small = synth.ragged_workload(lens, [(0, 2999), (1, 699), (2, 1800), (0, 100)], n_layers=4)
    _compare(L, small, seed=32)


def test_noalloc_rejects_oversized_batch(gpu_lib):
    L = gpu_lib
    descs = (_lib.LayerDesc * 1)()
    descs[0].is_full = 1
    # 4096 queries over 131,072 positions: 2 GiB of scores alone
    batch = _lib.BatchDesc(0x10000, 0x10000, 0x10000, 0x10000, 4096, 1, 131072)
    rc = L.sa_layer_stack_noalloc(descs, 1, ctypes.byref(batch), 2048, 1.0 / 16, None, None)
    assert rc == -3 and b"static scratch" in L.sa_last_error_message()

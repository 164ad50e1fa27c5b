"""The query side on the GPU against the oracle: sa_q_project (q_b_proj with
the rope part turned, indexer query, head weights) within the derived bf16
bound, sa_q_absorb on the GPU's own q, and the produced queries through the
layer stack."""
import math

import numpy as np
import pytest
import torch

from oracle import ref
from sparse_attention_relu_amd import api, synth
from sparse_attention_relu_amd.synth import to_numpy
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _weights(seed):
    """Random-init weights scaled so q ~ N(0,1) (nope), q_abs ~ N(0, 1/576),
    q_idx ~ N(0, 1/128), w ~ N(0, 1/32) for a unit-RMS q_lora."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    w_qb = torch.randn((64, 256, 2048), generator=g, device=DEV) / math.sqrt(2048)
    w_qb[:, 192:] /= math.sqrt(576)
    w_uk = torch.randn((64, 192, 512), generator=g, device=DEV) / math.sqrt(192 * 576)
    w_iq = torch.randn((32 * 128, 2048), generator=g, device=DEV) / math.sqrt(2048 * 128)
    w_iw = torch.randn((32, 2048), generator=g, device=DEV) / math.sqrt(2048 * 32)
    bf = lambda x: x.to(torch.bfloat16).contiguous()
    w_uk = bf(w_uk)
    return bf(w_qb.reshape(64 * 256, 2048)), w_uk, w_uk.transpose(1, 2).contiguous(), bf(w_iq), bf(w_iw)


def _tokens(n, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    c = torch.randn((n, 2048), generator=g, device=DEV).to(torch.bfloat16)
    pos = torch.randint(0, 1 << 20, (n,), generator=g, device=DEV, dtype=torch.int32)
    pos[0] = 0
    if n > 1:
        pos[1] = (1 << 20) - 1
    return c, pos


@pytest.fixture(scope="module")
def weights():
    return _weights(5)


@pytest.fixture(scope="module")
def weights_np(weights):
    return [to_numpy(x) for x in weights]


@pytest.mark.parametrize("n", [1, 5, 16, 37, 64, 65, 300])
def test_q_project_and_absorb(gpu_lib, weights, weights_np, n):
    w_qb, w_uk, w_uk_t, w_iq, w_iw = weights
    c, pos = _tokens(n, 100 + n)
    q, qi, w = api.q_project(c, w_qb, pos, w_iq=w_iq, w_iw=w_iw)
    qa = api.q_absorb(q, w_uk_t)
    torch.cuda.synchronize()
    Wqb, Wuk, _, Wiq, Wiw = weights_np
    f1 = parity.check_q_project(to_numpy(c), Wqb, to_numpy(pos), to_numpy(q), Wiq, Wiw, to_numpy(qi), to_numpy(w))
    f2 = parity.check_q_absorb(to_numpy(q), Wuk, to_numpy(qa))
    print(f"n={n}: values on the other side of a rounding boundary: projections {f1:.2e}, absorption {f2:.2e}")


def test_q_project_without_indexer_part(gpu_lib, weights, weights_np):
    w_qb = weights[0]
    c, pos = _tokens(9, 7)
    q, qi, w = api.q_project(c, w_qb, pos)
    torch.cuda.synchronize()
    assert qi is None and w is None
    parity.check_q_project(to_numpy(c), weights_np[0], to_numpy(pos), to_numpy(q))


def test_prefill_shape_sampled(gpu_lib, weights, weights_np):
    # 4096 new tokens of one sequence at 126,976..131,071 (the chunked-prefill shape)
    w_qb, w_uk, w_uk_t, w_iq, w_iw = weights
    n = 4096
    g = torch.Generator(device=DEV).manual_seed(11)
    c = torch.randn((n, 2048), generator=g, device=DEV).to(torch.bfloat16)
    pos = torch.arange(126976, 131072, dtype=torch.int32, device=DEV)
    q, qi, w = api.q_project(c, w_qb, pos, w_iq=w_iq, w_iw=w_iw)
    qa = api.q_absorb(q, w_uk_t)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 2047, 2049, 4094, 4095]
    Wqb, Wuk, _, Wiq, Wiw = weights_np
    sub = lambda t: to_numpy(t[rows])
    parity.check_q_project(sub(c), Wqb, sub(pos), sub(q), Wiq, Wiw, sub(qi), sub(w))
    parity.check_q_absorb(sub(q), Wuk, sub(qa))


def test_query_side_feeds_the_layer_stack(gpu_lib, weights, weights_np):
    """Queries made by sa_q_project / sa_q_absorb at each token's position
    drive a [full, shared] stack; the path's parity checks hold on them, and
    the outputs meet the attention bar against the oracle's own chain (the
    oracle's projections, absorption and attention on the GPU's selection)."""
    w_qb, w_uk, w_uk_t, w_iq, w_iw = weights
    lens = [5000, 3000, 7000, 4100]
    queries = [(0, 4999), (1, 2999), (2, 6999), (3, 4099), (2, 3000)]
    wl = synth.ragged_workload(lens, queries, name="qside", full=[True, False])
    b = synth.make_batch(wl, DEV, seed=9)
    g = torch.Generator(device=DEV).manual_seed(13)
    c = torch.randn((wl.n_q, 2048), generator=g, device=DEV).to(torch.bfloat16)
    q, qi, w = api.q_project(c, w_qb, b.q_pos, w_iq=w_iq, w_iw=w_iw)
    layers = []
    for L in b.layers:
        qa = api.q_absorb(q, w_uk_t)
        layers.append(synth.LayerInputs(q_abs=qa, kv=L.kv, w_uv=L.w_uv, q_idx=qi if L.q_idx is not None else None,
                                        w=w if L.q_idx is not None else None, k_idx=L.k_idx))
    outs, idxs = api.layer_stack(layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    torch.cuda.synchronize()
    B = parity.np_batch(b)
    Lnp0 = {"q_idx": to_numpy(qi), "w": to_numpy(w), "k_idx": to_numpy(layers[0].k_idx)}
    sc = api.indexer_score(qi, w, layers[0].k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    torch.cuda.synchronize()
    parity.check_scores(Lnp0, B, to_numpy(sc))
    idx = to_numpy(idxs[0])
    parity.check_topk_exact(to_numpy(sc), B["q_pos"], 2048, idx)
    parity.check_topk_band(Lnp0, B, idx, 2048)
    Wqb, Wuk, _, Wiq, Wiw = weights_np
    q_o, _, _ = ref.q_project(to_numpy(c), Wqb, Wiq, Wiw, B["q_pos"])
    qa_o = ref.q_absorb(q_o, Wuk)
    for l, L in enumerate(layers):
        Lm = {"q_abs": to_numpy(L.q_abs), "kv": to_numpy(L.kv), "w_uv": to_numpy(L.w_uv)}
        parity.check_mla(Lm, B, idx, to_numpy(outs[l]), wl.scale)
        o = ref.sparse_mla(qa_o, Lm["kv"], B["seq_start"], B["q_seq"], idx, Lm["w_uv"], wl.scale)
        err = np.abs(to_numpy(outs[l]) - o)
        assert np.all(err <= 2e-2 + 1e-2 * np.abs(o)), f"layer {l}: chain max err {err.max()}"

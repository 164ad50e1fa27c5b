"""FP8 caches on the GPU against the oracle: the E4M3 decoder on every code,
the row quantizer bit for bit, and the indexer, top-k and attention over FP8
rows against the oracle on the exactly dequantized rows (the same tolerances
as the bf16 path, plus one fp32 rounding for the indexer's scale)."""
import numpy as np
import pytest
import torch

from oracle import ref
from sparse_attention_relu_amd import api, synth
from sparse_attention_relu_amd.synth import to_numpy
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCALE_ROUND = 2.0 ** -23        # the indexer's extra rounding: codes' score x scale


def test_decoder_on_every_code(gpu_lib):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    codes[0x7F] = 0
    codes[0xFF] = 0                              # NaN codes are never produced
    got = to_numpy(api.fp8_decode(codes.to(DEV)))
    expect = ref.E4M3_TABLE[to_numpy(codes)]
    assert np.array_equal(got, expect), np.nonzero(got != expect)[0][:8]


def _rows(n, d, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn((n, d), generator=g, device=DEV)
    mag = torch.tensor([1e-3, 1.0, 30.0, 1e-6, 1.0, 0.0, 1.0, 5e3], device=DEV).repeat((n + 7) // 8)[:n]
    x = x * mag[:, None]
    x[4, 3] = 200.0                              # a spike sets the scale, the rest go subnormal
    x[6] = -x[6]
    x[7, :] = 448.0 * 2.0 ** -9                  # every value on a code boundary
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("d", [576, 128])
def test_quantizer_bit_exact(gpu_lib, d):
    x = _rows(37, d, d)
    codes, scales = api.quantize_rows_fp8(x)
    # scattered destination rows
    dst = torch.randperm(100, device=DEV)[:37].to(torch.int64)
    codes2 = torch.zeros((100, d), dtype=torch.uint8, device=DEV)
    scales2 = torch.zeros(100, dtype=torch.float32, device=DEV)
    api.quantize_rows_fp8(x, codes2, scales2, dst_rows=dst)
    torch.cuda.synchronize()
    c_o, s_o = ref.quantize_rows_fp8(to_numpy(x))
    assert np.array_equal(to_numpy(scales), s_o)
    bad = np.argwhere(to_numpy(codes) != c_o)
    assert bad.size == 0, f"{len(bad)} codes differ; first {bad[0]}: gpu {to_numpy(codes)[tuple(bad[0])]:#x} " \
                          f"oracle {c_o[tuple(bad[0])]:#x} x={to_numpy(x)[tuple(bad[0])]}"
    assert torch.equal(codes2[dst], codes) and torch.equal(scales2[dst], scales)


def _fp8_layer(L):
    """The layer's caches stored as FP8 (quantized on the GPU), and their
    exactly dequantized values for the oracle."""
    kv8, kvs = api.quantize_rows_fp8(L.kv)
    out = synth.LayerInputs(q_abs=L.q_abs, kv=kv8, w_uv=L.w_uv, q_idx=L.q_idx, w=L.w, kv_scale=kvs)
    deq = {"kv": ref.dequantize_rows_fp8(to_numpy(kv8), to_numpy(kvs))}
    if L.k_idx is not None:
        k8, ks = api.quantize_rows_fp8(L.k_idx)
        out.k_idx, out.k_scale = k8, ks
        deq["k_idx"] = ref.dequantize_rows_fp8(to_numpy(k8), to_numpy(ks))
    return out, deq


def _ragged():
    lens = [3000, 17, 2100, 5000, 9000]
    queries = [(0, 2999), (1, 16), (2, 2047), (2, 2048), (3, 4999), (3, 0), (4, 8999), (4, 4500)]
    return synth.ragged_workload(lens, queries, name="ragged")


def _prefill():
    lens = [6000, 3500]
    queries = [(0, 5900 + i) for i in range(100)] + [(i % 2, 3000 + 37 * i) for i in range(12)]
    return synth.ragged_workload(lens, queries, name="prefill_small")


CASES = {"c0": lambda: synth.workload("c0"), "ragged": _ragged, "prefill": _prefill}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("algo", [1, 2])
def test_fp8_indexer_and_topk(gpu_lib, case, algo):
    wl = CASES[case]()
    b = synth.make_batch(wl, DEV, seed=3)
    L8, deq = _fp8_layer(b.layers[0])
    sc = api.indexer_score_fp8(L8.q_idx, L8.w, L8.k_idx, L8.k_scale, b.seq_start, b.seq_len, b.q_seq, b.q_pos,
                               wl.ld + 5, algo=algo)
    idx = api.topk_select(sc[:, :wl.ld].contiguous(), b.q_pos)
    torch.cuda.synchronize()
    B = parity.np_batch(b)
    Lnp = {"q_idx": to_numpy(L8.q_idx), "w": to_numpy(L8.w), "k_idx": deq["k_idx"]}
    sc_np = to_numpy(sc)
    worst = parity.check_scores(Lnp, B, sc_np, extra_rel=SCALE_ROUND)
    parity.check_topk_exact(sc_np[:, :wl.ld], B["q_pos"], 2048, to_numpy(idx))
    parity.check_topk_band(Lnp, B, to_numpy(idx), 2048, extra_rel=SCALE_ROUND)
    print(f"{case} algo {algo}: worst |err| / bound {worst:.3g}")


@pytest.mark.parametrize("n_q", [4, 8, 1, 3, 10, 24, 130])
def test_fp8_attention(gpu_lib, n_q):
    # 8: the ragged batch; 1, 3, 10: the wide merge; 24: 6 slices whose bf16
    # partial states are merged inside the W_UV launch over two query blocks;
    # 130: all 64 heads per workgroup
    if n_q == 8:
        wl = _ragged()
    elif n_q == 4:
        wl = synth.workload("c0")
    else:
        lens = [4096, 3000, 2500]
        queries = [(i % 3, lens[i % 3] - 1 - 7 * i) for i in range(n_q)]
        wl = synth.ragged_workload(lens, queries, name=f"fp8_{n_q}")
    b = synth.make_batch(wl, DEV, seed=20 + n_q)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx = api.topk_select(sc, b.q_pos)
    L8, deq = _fp8_layer(L)
    lse = torch.empty((wl.n_q, 64), dtype=torch.float32, device=DEV)
    out = api.mla_sparse_attn_fp8(L8.q_abs, L8.kv, L8.kv_scale, b.seq_start, b.q_seq, idx, L8.w_uv, wl.scale, lse=lse)
    torch.cuda.synchronize()
    Lm = {"q_abs": to_numpy(L.q_abs), "kv": deq["kv"], "w_uv": to_numpy(L.w_uv)}
    rows = None if wl.n_q <= 16 else sorted({0, 1, 2, wl.n_q // 2, wl.n_q - 2, wl.n_q - 1})
    worst = parity.check_mla(Lm, parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale, rows=rows,
                             lse_gpu=to_numpy(lse))
    print(f"n_q={n_q}: worst |err| / derived bound {worst:.3g}")


@pytest.mark.parametrize("k", [1, 300])
def test_fp8_attention_small_k_and_padding(gpu_lib, k):
    wl = _ragged()
    wl.k = k
    b = synth.make_batch(wl, DEV, seed=5)
    L8, deq = _fp8_layer(b.layers[0])
    g = torch.Generator(device="cpu").manual_seed(k)
    idx = torch.full((wl.n_q, k), -1, dtype=torch.int32)
    for t, p in enumerate(wl.q_pos):
        n = min(k, p + 1)
        idx[t, torch.randperm(k, generator=g)[:n]] = torch.randperm(p + 1, generator=g)[:n].int()
    idx = idx.to(DEV)
    out = api.mla_sparse_attn_fp8(L8.q_abs, L8.kv, L8.kv_scale, b.seq_start, b.q_seq, idx, L8.w_uv, wl.scale)
    torch.cuda.synchronize()
    Lm = {"q_abs": to_numpy(L8.q_abs), "kv": deq["kv"], "w_uv": to_numpy(L8.w_uv)}
    parity.check_mla(Lm, parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale)


def test_fp8_layer_stack_mixed(gpu_lib):
    """[F, S, S, F] with FP8 caches on layers 0, 1 and 3, bf16 on layer 2 (the
    formats are per layer), against separate FP8 calls and the oracle."""
    wl = _ragged()
    wl.full = [True, False, False, True]
    b = synth.make_batch(wl, DEV, seed=15)
    layers, deqs = [], []
    for l, L in enumerate(b.layers):
        if l == 2:
            layers.append(L)
            deqs.append({"kv": to_numpy(L.kv)})
        else:
            L8, deq = _fp8_layer(L)
            layers.append(L8)
            deqs.append(deq)
    outs, idxs = api.layer_stack(layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    torch.cuda.synchronize()
    B = parity.np_batch(b)
    cur = None
    for l, L in enumerate(layers):
        if wl.full[l]:
            sc = api.indexer_score_fp8(L.q_idx, L.w, L.k_idx, L.k_scale, b.seq_start, b.seq_len, b.q_seq, b.q_pos,
                                       wl.ld)
            cur = api.topk_select(sc, b.q_pos)
            torch.cuda.synchronize()
            assert torch.equal(cur, idxs[l]), f"layer {l}: stack selection differs from the separate calls"
            Lnp = {"q_idx": to_numpy(L.q_idx), "w": to_numpy(L.w), "k_idx": deqs[l]["k_idx"]}
            parity.check_scores(Lnp, B, to_numpy(sc), extra_rel=SCALE_ROUND)
            parity.check_topk_band(Lnp, B, to_numpy(cur), 2048, extra_rel=SCALE_ROUND)
        Lm = {"q_abs": to_numpy(L.q_abs), "kv": deqs[l]["kv"], "w_uv": to_numpy(L.w_uv)}
        parity.check_mla(Lm, B, to_numpy(cur), to_numpy(outs[l]), wl.scale)


def test_fp8_layer_stack_shared_rows(gpu_lib):
    """96 queries of one sequence with FP8 caches: the stack's attention
    gathers the codes with cached loads (queries sharing their sequence's
    rows), the separate FP8 call streams them; outputs identical bit for bit,
    and sampled queries against the oracle on the dequantized rows."""
    wl = synth.ragged_workload([5000], [(0, 4904 + i) for i in range(96)], n_layers=2, name="fp8_shared_rows")
    wl.full = [True, False]
    b = synth.make_batch(wl, DEV, seed=21)
    layers, deqs = [], []
    for L in b.layers:
        L8, deq = _fp8_layer(L)
        layers.append(L8)
        deqs.append(deq)
    outs, idxs = api.layer_stack(layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    torch.cuda.synchronize()
    B = parity.np_batch(b)
    for l, L in enumerate(layers):
        o = api.mla_sparse_attn_fp8(L.q_abs, L.kv, L.kv_scale, b.seq_start, b.q_seq, idxs[0], L.w_uv, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l]), f"layer {l}"
        Lm = {"q_abs": to_numpy(L.q_abs), "kv": deqs[l]["kv"], "w_uv": to_numpy(L.w_uv)}
        parity.check_mla(Lm, B, to_numpy(idxs[0]), to_numpy(outs[l]), wl.scale, rows=[0, 47, 95])


def test_fp8_decode_config_full(gpu_lib):
    """The 16-query, 65,536..131,072-token, 4-layer decode configuration with
    FP8 caches, in the launch configuration the benchmark times."""
    wl = synth.workload("c2")
    b = synth.make_batch(wl, DEV, seed=0)
    layers = []
    for L in b.layers:
        kv8, kvs = api.quantize_rows_fp8(L.kv)
        L8 = synth.LayerInputs(q_abs=L.q_abs, kv=kv8, w_uv=L.w_uv, q_idx=L.q_idx, w=L.w, kv_scale=kvs)
        if L.k_idx is not None:
            L8.k_idx, L8.k_scale = api.quantize_rows_fp8(L.k_idx)
        layers.append(L8)
    del b.layers
    outs, idxs = api.layer_stack(layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    L0 = layers[0]
    sc = api.indexer_score_fp8(L0.q_idx, L0.w, L0.k_idx, L0.k_scale, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    torch.cuda.synchronize()
    B = parity.np_batch(b)
    rows = [0, 7, 15]
    sub = lambda a: a[rows]
    Bs = {"seq_start": B["seq_start"], "q_seq": sub(B["q_seq"]), "q_pos": sub(B["q_pos"])}
    Lnp = {"q_idx": sub(to_numpy(L0.q_idx)), "w": sub(to_numpy(L0.w)),
           "k_idx": ref.dequantize_rows_fp8(to_numpy(L0.k_idx), to_numpy(L0.k_scale))}
    sc_np = to_numpy(sc[rows])
    idx_np = to_numpy(idxs[0])
    parity.check_scores(Lnp, Bs, sc_np, extra_rel=SCALE_ROUND)
    parity.check_topk_exact(sc_np, Bs["q_pos"], 2048, idx_np[rows])
    parity.check_topk_band(Lnp, Bs, idx_np[rows], 2048, extra_rel=SCALE_ROUND)
    for l, L in enumerate(layers):
        # the selected rows of each sampled query, dequantized
        rows_all, idx_loc, starts, off = [], np.full((len(rows), 2048), -1), [], 0
        for j, t in enumerate(rows):
            sel = idx_np[t][idx_np[t] >= 0]
            g = torch.as_tensor(sel, device=DEV) + int(wl.seq_start[wl.q_seq[t]])
            rows_all.append(ref.dequantize_rows_fp8(to_numpy(L.kv[g]), to_numpy(L.kv_scale[g])))
            idx_loc[j, :len(sel)] = np.arange(len(sel))
            starts.append(off)
            off += len(sel)
        Lm = {"q_abs": to_numpy(L.q_abs[rows]), "kv": np.concatenate(rows_all), "w_uv": to_numpy(L.w_uv)}
        Bm = {"seq_start": np.array(starts), "q_seq": np.arange(len(rows)), "q_pos": None}
        parity.check_mla(Lm, Bm, idx_loc, to_numpy(outs[l][rows]), wl.scale, n_launch=wl.n_q)

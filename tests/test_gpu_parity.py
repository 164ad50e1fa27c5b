"""HIP path against the CPU oracle, element by element, at sizes the oracle
finishes in seconds (several tiles, ragged tails, edge cases).  Every call
goes through the C ABI (libsparse_mla.so via the ctypes binding)."""
import numpy as np
import pytest
import torch

from oracle import ref
from sparse_attention_relu_amd import api, synth
from sparse_attention_relu_amd.synth import to_numpy
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _batch(wl, seed=0):
    torch.manual_seed(seed)
    return synth.make_batch(wl, DEV, seed=seed)


def ragged_wl(n_layers=1, k=2048):
    lens = [3000, 17, 2100, 5000, 9000]
    queries = [(0, 2999), (1, 16), (2, 2047), (2, 2048), (3, 4999), (3, 0), (4, 8999), (4, 4500)]
    return synth.ragged_workload(lens, queries, n_layers=n_layers, k=k, name="ragged")


def prefill_wl():
    # 100 consecutive queries of one sequence plus a block that mixes two sequences
    lens = [6000, 3500]
    queries = [(0, 5900 + i) for i in range(100)] + [(i % 2, 3000 + 37 * i) for i in range(12)]
    return synth.ragged_workload(lens, queries, name="prefill_small")


CASES = {"c0": lambda: synth.workload("c0"), "ragged": ragged_wl, "prefill": prefill_wl}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("algo", [1, 2])
def test_indexer_scores(gpu_lib, case, algo):
    wl = CASES[case]()
    b = _batch(wl)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld + 37, algo=algo)
    torch.cuda.synchronize()
    worst = parity.check_scores(parity.layer_np(L), parity.np_batch(b), to_numpy(sc))
    print(f"{case} algo {algo}: worst |err|/bound = {worst:.3g}")


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("algo", [1, 2])
def test_topk_on_gpu_scores(gpu_lib, case, algo):
    wl = CASES[case]()
    b = _batch(wl)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    for k in (2048, 1000, 1):
        idx = api.topk_select(sc, b.q_pos, k=k, algo=algo)
        torch.cuda.synchronize()
        parity.check_topk_exact(to_numpy(sc), to_numpy(b.q_pos), k, to_numpy(idx))
        parity.check_topk_band(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), k)


def _synthetic_scores(kind, n_rows, ld, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    if kind == "quantised":      # few distinct values: heavy ties everywhere
        return (torch.randint(-3, 4, (n_rows, ld), generator=g, device=DEV).float() * 0.25)
    if kind == "zeros_signed":   # +0.0 and -0.0 only: all tie
        x = torch.zeros((n_rows, ld), device=DEV)
        neg = torch.rand((n_rows, ld), generator=g, device=DEV) < 0.5
        return torch.where(neg, torch.full_like(x, -0.0), x)
    if kind == "normal":
        return torch.randn((n_rows, ld), generator=g, device=DEV)
    if kind == "spiky":          # a few huge values, many tiny ones, negatives
        x = torch.randn((n_rows, ld), generator=g, device=DEV) * 1e-3
        x[:, ::97] = 1e30
        x[:, 5::11] = -1e30
        return x
    raise KeyError(kind)


@pytest.mark.parametrize("kind", ["quantised", "zeros_signed", "normal", "spiky"])
@pytest.mark.parametrize("algo", [1, 2])
def test_topk_ties_and_edges(gpu_lib, kind, algo):
    ld = 70000
    sc = _synthetic_scores(kind, 6, ld, 7)
    q_pos = torch.tensor([ld - 1, 0, 2047, 2048, 40000, 69998], dtype=torch.int32, device=DEV)
    for k in (2048, 513, 1):
        idx = api.topk_select(sc, q_pos, k=k, algo=algo)
        torch.cuda.synchronize()
        parity.check_topk_exact(to_numpy(sc), to_numpy(q_pos), k, to_numpy(idx))


@pytest.mark.parametrize("kind", ["normal", "quantised", "spiky"])
def test_topk_rows_longer_than_the_bitmap(gpu_lib, kind):
    # rows of 262,145..900,000 positions: longer than the finish kernel's
    # one-level LDS bitmap, so the kept positions are put in order through the
    # two-level one (128-position buckets); the exact path must agree bitwise
    ld = 900000
    sc = _synthetic_scores(kind, 5, ld, 13)
    q_pos = torch.tensor([262144, 262143 + 2048, 524290, 786431, ld - 1], dtype=torch.int32, device=DEV)
    for k in (2048, 700):
        idx = api.topk_select(sc, q_pos, k=k, algo=1)
        torch.cuda.synchronize()
        parity.check_topk_exact(to_numpy(sc), to_numpy(q_pos), k, to_numpy(idx))
        assert torch.equal(idx, api.topk_select(sc, q_pos, k=k, algo=2))


def test_topk_rows_beyond_the_two_level_bitmap(gpu_lib):
    # rows longer than 2^20 positions: the kept positions are sorted instead
    ld = 1200000
    sc = _synthetic_scores("normal", 2, ld, 17)
    q_pos = torch.tensor([1048576, ld - 1], dtype=torch.int32, device=DEV)
    idx = api.topk_select(sc, q_pos, k=2048, algo=1)
    torch.cuda.synchronize()
    parity.check_topk_exact(to_numpy(sc), to_numpy(q_pos), 2048, to_numpy(idx))
    assert torch.equal(idx, api.topk_select(sc, q_pos, k=2048, algo=2))


def test_topk_clustered_selection(gpu_lib):
    # selections made of dense windows (whole 128-position buckets kept, a
    # window across a bucket boundary, one at the row's start and one ending
    # at its last position) plus scattered positions, for rows on both sides
    # of 2^18 and up to 2^20 positions
    ld = 1048576
    g = torch.Generator(device=DEV).manual_seed(41)
    sc = torch.randn((4, ld), generator=g, device=DEV)
    q_pos = torch.tensor([200000, 700000, ld - 1, 300000], dtype=torch.int32, device=DEV)
    windows = [(0, [(0, 1500)]), (1, [(300000, 301500)]), (2, [(ld - 1200, ld), (128 * 1000 - 37, 128 * 1000 + 500)]),
               (3, [(299000 - 1700, 299000)])]
    for r, ws in windows:
        for a, b in ws:
            sc[r, a:b] += 10.0
    for k in (2048, 1600):
        idx = api.topk_select(sc, q_pos, k=k, algo=1)
        torch.cuda.synchronize()
        parity.check_topk_exact(to_numpy(sc), to_numpy(q_pos), k, to_numpy(idx))
        assert torch.equal(idx, api.topk_select(sc, q_pos, k=k, algo=2))


@pytest.mark.parametrize("kind", ["normal", "quantised"])
def test_topk_many_rows_large_chunks(gpu_lib, kind):
    # 600 rows of 60,000: more than 4096 chunks of 8192, so path 1 reads 32
    # scores per thread in the histogram (chunks of 32,768) and 16 in the
    # compaction (16,384), the last chunk of each row ragged
    ld = 60000
    sc = _synthetic_scores(kind, 600, ld, 29)
    g = torch.Generator(device=DEV).manual_seed(31)
    q_pos = torch.randint(20000, ld, (600,), generator=g, device=DEV, dtype=torch.int32)
    q_pos[:3] = torch.tensor([ld - 1, 32767, 32768], dtype=torch.int32, device=DEV)
    idx = api.topk_select(sc, q_pos, k=2048, algo=1)
    assert torch.equal(idx, api.topk_select(sc, q_pos, k=2048, algo=2))
    rows = [0, 1, 2, 100, 333, 599]
    parity.check_topk_exact(to_numpy(sc), to_numpy(q_pos), 2048, to_numpy(idx), rows=rows)


def test_topk_paths_agree_bitwise(gpu_lib):
    sc = _synthetic_scores("normal", 40, 131072, 3)
    q_pos = torch.randint(0, 131072, (40,), dtype=torch.int32, device=DEV)
    a = api.topk_select(sc, q_pos, algo=1)
    b = api.topk_select(sc, q_pos, algo=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("case", ["c0", "ragged"])
def test_mla_on_gpu_selection(gpu_lib, case):
    wl = CASES[case]()
    b = _batch(wl)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx = api.topk_select(sc, b.q_pos, k=2048)
    lse = torch.empty((wl.n_q, 64), dtype=torch.float32, device=DEV)
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale, lse=lse)
    torch.cuda.synchronize()
    worst = parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale,
                             lse_gpu=to_numpy(lse))
    print(f"{case}: worst |err|/bound = {worst:.3g}")


@pytest.mark.parametrize("n_q", [1, 3, 5, 6, 10])
def test_mla_slice_counts(gpu_lib, n_q):
    # about 128 / n_q slices per query: 32, 32, 22, 22 and 13, i.e. the split
    # merge (one query) and the wide merge with 4 waves per item (even and
    # uneven slice shares) and with 2 waves (uneven)
    lens = [4096, 3000, 2500]
    queries = [(i % 3, lens[i % 3] - 1 - 7 * i) for i in range(n_q)]
    wl = synth.ragged_workload(lens, queries, name=f"slices{n_q}")
    b = _batch(wl, seed=11 + n_q)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx = api.topk_select(sc, b.q_pos, k=2048)
    lse = torch.empty((wl.n_q, 64), dtype=torch.float32, device=DEV)
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale, lse=lse)
    torch.cuda.synchronize()
    parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale,
                     lse_gpu=to_numpy(lse))


@pytest.mark.parametrize("n_q", [16, 24, 40, 63])
def test_mla_bf16_partials_merged_in_wuv(gpu_lib, n_q):
    # 16..63 queries at k = 2048: 8, 6, 4 and 3 slices whose bf16 partial
    # states are merged inside the W_UV launch, over 1..4 blocks of 16 queries
    # (the last one ragged); the bound includes the slices' rounding
    assert api.mla_partial_bits(n_q, 2048) == 16
    lens = [4096, 3000, 2500, 3500]
    queries = [(i % 4, lens[i % 4] - 1 - 5 * i) for i in range(n_q)]
    wl = synth.ragged_workload(lens, queries, name=f"bf16parts{n_q}")
    b = _batch(wl, seed=70 + n_q)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx = api.topk_select(sc, b.q_pos, k=2048)
    lse = torch.empty((wl.n_q, 64), dtype=torch.float32, device=DEV)
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale, lse=lse)
    torch.cuda.synchronize()
    parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale,
                     lse_gpu=to_numpy(lse))


@pytest.mark.parametrize("k", [100, 600, 2048])
def test_mla_single_query(gpu_lib, k):
    # one query: 2 slices merged inside the W_UV launch (bf16 partial
    # states), 10 and 32 by the split merge (fp32)
    wl = synth.ragged_workload([5000], [(0, 4321)], k=k, name=f"single_{k}")
    b = _batch(wl, seed=40 + k)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx = api.topk_select(sc, b.q_pos, k=k)
    n_sp, _ = api.mla_split_info(1, k)
    assert n_sp > 1
    lse = torch.empty((1, 64), dtype=torch.float32, device=DEV)
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale, lse=lse)
    torch.cuda.synchronize()
    parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale,
                     lse_gpu=to_numpy(lse))


@pytest.mark.parametrize("n_q", [130, 300])
def test_mla_all_heads_per_workgroup(gpu_lib, n_q):
    # from 64 queries on, one attention workgroup takes all 64 heads of a
    # (query, slice): 2 slices per query at 130 queries (partial states and
    # merge), 1 at 300; positions from 1700 up, so some rows select fewer than
    # 2048 positions
    lens = [3000, 2600]
    queries = [(i % 2, lens[i % 2] - 1 - (i // 2) % 900) for i in range(n_q)]
    wl = synth.ragged_workload(lens, queries, name=f"heads64_{n_q}")
    b = _batch(wl, seed=21 + n_q)
    L = b.layers[0]
    sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    idx = api.topk_select(sc, b.q_pos, k=2048)
    lse = torch.empty((wl.n_q, 64), dtype=torch.float32, device=DEV)
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale, lse=lse)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 2, n_q // 3, n_q // 2, n_q - 3, n_q - 2, n_q - 1})
    parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale, rows=rows,
                     lse_gpu=to_numpy(lse))


@pytest.mark.parametrize("k", [1, 7, 64, 300])
def test_mla_small_k_and_padding(gpu_lib, k):
    wl = ragged_wl(k=k)
    b = _batch(wl, seed=5)
    L = b.layers[0]
    g = torch.Generator(device="cpu").manual_seed(k)
    idx = torch.full((wl.n_q, k), -1, dtype=torch.int32)
    for t, p in enumerate(wl.q_pos):
        n = min(k, p + 1)
        pick = torch.randperm(p + 1, generator=g)[:n]
        slots = torch.randperm(k, generator=g)[:n]        # padding anywhere in the row
        idx[t, slots] = pick.int()
    idx = idx.to(DEV)
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale)
    torch.cuda.synchronize()
    parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale)


def test_mla_empty_selection_gives_zero(gpu_lib):
    wl = ragged_wl(k=8)
    b = _batch(wl, seed=9)
    L = b.layers[0]
    idx = torch.full((wl.n_q, 8), -1, dtype=torch.int32, device=DEV)
    idx[0, 3] = 5
    out = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idx, L.w_uv, wl.scale)
    torch.cuda.synchronize()
    assert torch.all(out[1:] == 0)
    parity.check_mla(parity.layer_np(L), parity.np_batch(b), to_numpy(idx), to_numpy(out), wl.scale, rows=[0])


def test_layer_stack_matches_separate_calls(gpu_lib):
    wl = ragged_wl(n_layers=4)
    wl.full = [True, False, False, True]
    b = _batch(wl, seed=11)
    stack = api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    outs, idxs = stack()
    torch.cuda.synchronize()
    cur = None
    for l, L in enumerate(b.layers):
        if wl.full[l]:
            sc = api.indexer_score(L.q_idx, L.w, L.k_idx, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
            cur = api.topk_select(sc, b.q_pos)
            assert torch.equal(cur, idxs[l])
        o = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, cur, L.w_uv, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l]), f"layer {l}"
    # layer 2 reuses layer 0's selection, checked against the oracle with its own inputs
    B = parity.np_batch(b)
    parity.check_mla(parity.layer_np(b.layers[2]), B, to_numpy(idxs[0]), to_numpy(outs[2]), wl.scale)
    parity.check_topk_band(parity.layer_np(b.layers[3]), B, to_numpy(idxs[3]), 2048)


def test_layer_stack_shared_rows_matches_separate_calls(gpu_lib):
    # 600 queries of one sequence: the stack's attention gathers with cached
    # loads (queries sharing their sequence's rows) and W_UV takes its
    # 128-row, two-way query split; the separate call streams its gathers,
    # and the outputs must be identical bit for bit
    lens = [9000]
    queries = [(0, 8400 + i) for i in range(600)]
    wl = synth.ragged_workload(lens, queries, n_layers=2, name="shared_rows")
    wl.full = [True, False]
    b = _batch(wl, seed=19)
    outs, idxs = api.layer_stack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full)
    torch.cuda.synchronize()
    for l, L in enumerate(b.layers):
        o = api.mla_sparse_attn(L.q_abs, L.kv, b.seq_start, b.q_seq, idxs[0], L.w_uv, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l]), f"layer {l}"
    B = parity.np_batch(b)
    rows = [0, 1, 299, 598, 599]
    sel = to_numpy(idxs[0])
    for l in range(2):
        parity.check_mla(parity.layer_np(b.layers[l]), B, sel, to_numpy(outs[l]), wl.scale, rows=rows)


def test_deterministic(gpu_lib):
    wl = ragged_wl(n_layers=2)
    b = _batch(wl, seed=13)
    stack = api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    o1, i1 = stack()
    o1 = [x.clone() for x in o1]
    i1 = i1[0].clone()
    o2, i2 = stack()
    torch.cuda.synchronize()
    assert torch.equal(i1, i2[0])
    for a, c in zip(o1, o2):
        assert torch.equal(a, c)


def test_graph_replay_matches_eager(gpu_lib):
    wl = ragged_wl(n_layers=4)
    b = _batch(wl, seed=17)
    stack = api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld)
    outs, idxs = stack()
    torch.cuda.synchronize()
    ref_o = [o.clone() for o in outs]
    ref_i = idxs[0].clone()
    for o in outs:
        o.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            stack()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        idxs[0].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idxs[0], ref_i), rep
        for a, c in zip(outs, ref_o):
            assert torch.equal(a, c), rep

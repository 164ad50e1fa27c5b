"""Pins for the CPU oracle: checks against facts the pages and mathematics fix,
never against the oracle's own formula retyped.

Each ``check_*`` takes the oracle module (or a stand-in with a planted
mistake) and raises AssertionError when the oracle disagrees with the fact.
``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutations.py`` plants plausible mistakes in copies of the
oracle's functions and requires some check to fail for each.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bf16_grid(x):
    """Snap to values exactly representable in bf16 (8 significant bits) so
    the oracle sees the same kind of inputs as the GPU."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256) / 256, e)


# ----------------------------------------------------------------- indexer
def check_indexer_one_hot_closed_form(ref):
    """One head with weight w, query e_i: the score is w * max(0, k_s[i]).
    Keys are chosen so the expected row is printed below by hand."""
    n = 8
    k = np.zeros((n, 128))
    k[:, 5] = [-2.0, -0.5, 0.0, 0.25, 0.5, 1.0, 3.0, -1.0]
    q = np.zeros((1, 32, 128))
    q[0, 7, 5] = 1.0                       # head 7 looks at key dim 5
    w = np.zeros((1, 32))
    w[0, 7] = 2.0
    s = ref.indexer_scores(q, w, k, [0], [0], [n - 1], ld=n + 2)
    expect = [0.0, 0.0, 0.0, 0.5, 1.0, 2.0, 6.0, 0.0, -np.inf, -np.inf]
    assert np.array_equal(s[0], expect), s[0]
    # a negative head weight multiplies after the ReLU: w * ReLU(d), not ReLU(w d)
    w[0, 7] = -0.5
    s = ref.indexer_scores(q, w, k, [0], [0], [n - 1])
    expect = [0.0, 0.0, 0.0, -0.125, -0.25, -0.5, -1.5, 0.0]
    assert np.array_equal(s[0], expect), s[0]


def check_indexer_two_heads_closed_form(ref):
    """Two heads on opposite signs of the same key coordinate: exactly one
    of them is active per key, so the score is w_a k or -w_b k."""
    k = np.zeros((4, 128))
    k[:, 0] = [1.0, -1.0, 2.0, -3.0]
    q = np.zeros((1, 32, 128))
    q[0, 0, 0] = 1.0
    q[0, 31, 0] = -1.0
    w = np.zeros((1, 32))
    w[0, 0], w[0, 31] = 1.0, 10.0
    s = ref.indexer_scores(q, w, k, [0], [0], [3])
    assert np.array_equal(s[0], [1.0, 10.0, 2.0, 30.0]), s[0]


def check_indexer_gemv_reduction(ref):
    """With non-negative q and k every ReLU is the identity, so
    I[t, s] = (sum_h w_h q_h) . k_s: a plain matrix-vector product computed
    through a different association.  Covers head/dim indexing, w per query,
    sequence offsets and the causal bound, on two packed sequences."""
    rng = _rng(11)
    lens = [37, 53]
    starts = [0, 37]
    k = _bf16_grid(np.abs(rng.standard_normal((sum(lens), 128))))
    queries = [(1, 52), (0, 36), (1, 0), (0, 10)]
    q = _bf16_grid(np.abs(rng.standard_normal((4, 32, 128))) / 11)
    w = rng.standard_normal((4, 32))
    s = ref.indexer_scores(q, w, k, starts, [b for b, _ in queries], [p for _, p in queries], ld=60)
    for t, (b, p) in enumerate(queries):
        v = np.einsum("h,hi->i", w[t], q[t])
        expect = np.matmul(k[starts[b]:starts[b] + p + 1], v)
        np.testing.assert_allclose(s[t, :p + 1], expect, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(s[t, p + 1:]))


def check_indexer_zero_weights(ref):
    """w = 0 gives an all-zero row over the causal set."""
    rng = _rng(3)
    k = rng.standard_normal((20, 128))
    q = rng.standard_normal((2, 32, 128))
    s = ref.indexer_scores(q, np.zeros((2, 32)), k, [0], [0, 0], [19, 4], ld=20)
    assert np.all(s[0] == 0.0) and np.all(s[1, :5] == 0.0) and np.all(np.isneginf(s[1, 5:]))


def check_indexer_sampled_matches_rows(ref):
    """The sampled-position entry point agrees with the full row."""
    rng = _rng(5)
    k = rng.standard_normal((30, 128))
    q = rng.standard_normal((2, 32, 128))
    w = rng.standard_normal((2, 32))
    s = ref.indexer_scores(q, w, k, [0, 10], [1, 0], [19, 9])
    pos = np.array([0, 3, 19])
    np.testing.assert_allclose(ref.indexer_scores_at(q, w, k, [0, 10], [1, 0], [19, 9], 0, pos),
                               s[0, pos], rtol=1e-13, atol=1e-13)


def check_score_error_bound_covers_fp32(ref):
    """The fp32 error bound must cover fp32 evaluations in several summation
    orders (forward, reverse, pairwise) of a real score row."""
    rng = _rng(17)
    k = _bf16_grid(rng.standard_normal((64, 128)))
    q = _bf16_grid(rng.standard_normal((1, 32, 128)) / 11.3)
    w = rng.standard_normal((1, 32)).astype(np.float32).astype(np.float64) / 5.7
    exact = ref.indexer_scores(q, w, k, [0], [0], [63])[0]
    bound = ref.score_error_bound(q[0], w[0], k)
    q32, k32, w32 = q[0].astype(np.float32), k.astype(np.float32), w[0].astype(np.float32)
    prods = q32[:, None, :] * k32[None, :, :]                      # exact in fp32
    for order in ("fwd", "rev", "pair"):
        if order == "pair":
            d = prods
            while d.shape[-1] > 1:
                d = (d[..., 0::2] + d[..., 1::2]).astype(np.float32)
            d = d[..., 0]
        else:
            seq = range(128) if order == "fwd" else range(127, -1, -1)
            d = np.zeros((32, 64), dtype=np.float32)
            for i in seq:
                d = (d + prods[:, :, i]).astype(np.float32)
        r = np.maximum(d, np.float32(0))
        acc = np.zeros(64, dtype=np.float32)
        for h in (range(32) if order != "rev" else range(31, -1, -1)):
            acc = (acc + w32[h] * r[h]).astype(np.float32)
        assert np.all(np.abs(acc.astype(np.float64) - exact) <= bound), order
    assert np.all(bound < 1e-3 * (np.abs(exact).max() + 1e-30))
    # Cancellation: products 512, 2^-16, -512 summed left to right lose the
    # middle term entirely (fp32 ulp at 512 is 2^-14), so the dot-product
    # term of the bound must carry the error.
    kc = np.zeros((1, 128))
    kc[0, :3] = [512.0, 2.0 ** -16, 512.0]
    qc = np.zeros((1, 32, 128))
    qc[0, 0, :3] = [1.0, 1.0, -1.0]
    wc = np.zeros((1, 32))
    wc[0, 0] = 1.0
    exact_c = ref.indexer_scores(qc, wc, kc, [0], [0], [0])[0, 0]
    fwd = np.float32(np.float32(np.float32(512.0) + np.float32(2.0 ** -16)) - np.float32(512.0))
    assert exact_c == 2.0 ** -16 and fwd == 0.0
    assert abs(float(fwd) - exact_c) <= ref.score_error_bound(qc[0], wc[0], kc)[0]


# ------------------------------------------------------------------- top-k
def check_topk_full_sort(ref):
    """Top-k equals the first k of a full sort by (score desc, position asc),
    on many tiny rows with forced ties (scores quantised to few levels)."""
    rng = _rng(23)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        levels = int(rng.integers(1, 6))
        row = rng.integers(-levels, levels + 1, size=n).astype(np.float64) / 4
        k = int(rng.integers(1, n + 6))
        got = ref.topk_select(np.concatenate([row, [-np.inf] * 3]), n - 1, k)
        brute = sorted(range(n), key=lambda s: (-row[s], s))[:min(k, n)]
        expect = sorted(brute) + [-1] * (k - min(k, n))
        assert list(got) == expect, (trial, row, k, got)


def check_topk_order_invariant(ref):
    """Every selected position beats every unselected one: a higher score, or
    an equal score at a lower position; the set has min(k, n) members."""
    rng = _rng(29)
    for trial in range(100):
        n = int(rng.integers(1, 200))
        row = np.round(rng.standard_normal(n) * 3) / 2
        k = int(rng.integers(1, 64))
        got = ref.topk_select(row, n - 1, k)
        sel = [int(s) for s in got if s >= 0]
        assert len(sel) == min(k, n) and len(set(sel)) == len(sel)
        assert all(got[len(sel):] == -1)
        uns = sorted(set(range(n)) - set(sel))
        for s in sel:
            for u in uns:
                assert row[s] > row[u] or (row[s] == row[u] and s < u)


def check_topk_hand_example(ref):
    """Hand example: scores at positions 0..5 = [1, 3, 3, 2, 3, -0.0] and
    k = 2 keep the two lowest positions among the three 3's, {1, 2}; k = 5
    keeps {0, 1, 2, 3, 4}; -0.0 and +0.0 tie (the +0.0 at position 6 loses
    to the -0.0 at position 5 when one of them must go)."""
    row = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -0.0, 0.0])
    assert list(ref.topk_select(row, 6, 2)) == [1, 2]
    assert list(ref.topk_select(row, 6, 5)) == [0, 1, 2, 3, 4]
    assert list(ref.topk_select(row, 6, 6)) == [0, 1, 2, 3, 4, 5]
    assert list(ref.topk_select(row, 3, 6)) == [0, 1, 2, 3, -1, -1]


def check_topk_degenerate(ref):
    """All-equal rows keep positions 0..k-1; rows no longer than k keep all."""
    assert list(ref.topk_select(np.zeros(100), 99, 8)) == list(range(8))
    assert list(ref.topk_select(np.arange(5.0), 4, 8)) == [0, 1, 2, 3, 4, -1, -1, -1]
    assert list(ref.topk_select(np.array([7.0]), 0, 2048))[:2] == [0, -1]


def check_topk_respects_causal_bound(ref):
    """Only positions <= q_pos are eligible, even if later entries are larger."""
    row = np.array([0.0, 1.0, 2.0, 100.0, 200.0])
    assert list(ref.topk_select(row, 2, 2)) == [1, 2]


# --------------------------------------------------------------- sparse MLA
def _mla_inputs(seed, n_q, lens, k, n_heads=64, scale_q=1.0):
    rng = _rng(seed)
    T = sum(lens)
    starts = list(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int))
    kv = _bf16_grid(rng.standard_normal((T, 576)))
    q = _bf16_grid(rng.standard_normal((n_q, n_heads, 576)) * scale_q / 24)
    wuv = _bf16_grid(rng.standard_normal((n_heads, 256, 512)) / 22.6)
    q_seq = [int(rng.integers(0, len(lens))) for _ in range(n_q)]
    q_pos = [int(rng.integers(0, lens[b])) for b in q_seq]
    idx = np.full((n_q, k), -1)
    for t in range(n_q):
        n = q_pos[t] + 1
        pick = rng.choice(n, size=min(k, n), replace=False)
        idx[t, :len(pick)] = pick
        rng.shuffle(idx[t])                  # padding slots anywhere in the row
    return q, kv, starts, q_seq, q_pos, idx, wuv


def _dense_masked_reference(q, kv, starts, q_seq, q_pos, idx, wuv, scale):
    """The additive-mask mechanism of the reference code: score every cached
    position of the sequence, add 0 for selected positions and -inf for the
    rest, softmax over the whole row in one pass, multiply by all latents."""
    n_q, n_h = q.shape[0], q.shape[1]
    out = np.zeros((n_q, n_h, 256))
    for t in range(n_q):
        b = q_seq[t]
        end = starts[b + 1] if b + 1 < len(starts) else kv.shape[0]
        rows = kv[starts[b]:end]
        mask = np.full(rows.shape[0], -np.inf)
        sel = idx[t][idx[t] >= 0]
        mask[sel] = 0.0
        logits = scale * np.einsum("hd,sd->hs", q[t], rows) + mask[None, :]
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        attn = z / z.sum(axis=1, keepdims=True)
        lat = np.einsum("hs,sc->hc", attn, rows[:, :512])
        out[t] = np.einsum("hvc,hc->hv", wuv, lat)
    return out


def check_mla_equals_dense_masked(ref):
    q, kv, starts, q_seq, q_pos, idx, wuv = _mla_inputs(31, 5, [40, 70, 9], 16)
    got = ref.sparse_mla(q, kv, starts, q_seq, idx, wuv, 1.0 / 16)
    exp = _dense_masked_reference(q, kv, starts, q_seq, q_pos, idx, wuv, 1.0 / 16)
    np.testing.assert_allclose(got, exp, rtol=1e-10, atol=1e-12)


def check_mla_take_all_equals_dense_causal(ref):
    """k >= n: attention over all of 0..p, i.e. dense causal attention."""
    q, kv, starts, q_seq, q_pos, _, wuv = _mla_inputs(37, 4, [25, 30], 64)
    idx = np.full((4, 64), -1)
    for t in range(4):
        idx[t, :q_pos[t] + 1] = np.arange(q_pos[t] + 1)[::-1]
    got = ref.sparse_mla(q, kv, starts, q_seq, idx, wuv, 1.0 / 16)
    for t in range(4):
        rows = kv[starts[q_seq[t]]:starts[q_seq[t]] + q_pos[t] + 1]
        for h in (0, 17, 63):
            z = (q[t, h] @ rows.T) / 16
            a = np.exp(z - z.max())
            a /= a.sum()
            np.testing.assert_allclose(got[t, h], wuv[h] @ (a @ rows[:, :512]), rtol=1e-10, atol=1e-12)


def check_mla_absorbed_equals_explicit(ref):
    """Draw a kv_b_proj [64 * (192 + 256), 512]; per head its first 192 rows
    are W_UK and the next 256 are W_UV.  The explicit form computes, per head,
    keys [W_UK c ; k_rope] (256 wide), values W_UV c and scale 1/sqrt(256);
    the absorbed oracle gets q_abs = [W_UK^T q_nope ; q_rope] and the cache
    rows [c ; k_rope]."""
    rng = _rng(41)
    n_tok, n_q, k = 50, 3, 20
    kvb = rng.standard_normal((64 * 448, 512)) / 22.6
    w_uk = np.stack([kvb[h * 448:h * 448 + 192] for h in range(64)])          # [64, 192, 512]
    w_uv = np.stack([kvb[h * 448 + 192:(h + 1) * 448] for h in range(64)])    # [64, 256, 512]
    c = rng.standard_normal((n_tok, 512))
    kr = rng.standard_normal((n_tok, 64))
    q_nope = rng.standard_normal((n_q, 64, 192)) / 13.9
    q_rope = rng.standard_normal((n_q, 64, 64)) / 8
    q_pos = [49, 30, 19]
    idx = np.stack([rng.choice(p + 1, size=k, replace=False) for p in q_pos])
    scale = 1.0 / math.sqrt(192 + 64)
    explicit = np.zeros((n_q, 64, 256))
    for t in range(n_q):
        sel = idx[t]
        for h in range(64):
            keys = np.concatenate([c[sel] @ w_uk[h].T, kr[sel]], axis=1)     # [k, 256]
            vals = c[sel] @ w_uv[h].T                                          # [k, 256]
            z = scale * (keys @ np.concatenate([q_nope[t, h], q_rope[t, h]]))
            a = np.exp(z - z.max())
            explicit[t, h] = (a / a.sum()) @ vals
    q_abs = np.concatenate([np.einsum("hnc,thn->thc", w_uk, q_nope), q_rope], axis=2)
    rows = np.concatenate([c, kr], axis=1)
    got = ref.sparse_mla(q_abs, rows, [0], [0] * n_q, idx, w_uv, scale)
    np.testing.assert_allclose(got, explicit, rtol=1e-9, atol=1e-12)


def check_mla_single_row(ref):
    """One selected row: its weight is 1, so out = W_UV c_s."""
    q, kv, starts, q_seq, q_pos, _, wuv = _mla_inputs(43, 3, [30, 12], 4)
    idx = np.full((3, 4), -1)
    for t in range(3):
        idx[t, 2] = q_pos[t] // 2
    got = ref.sparse_mla(q, kv, starts, q_seq, idx, wuv, 1.0 / 16)
    for t in range(3):
        c_s = kv[starts[q_seq[t]] + q_pos[t] // 2, :512]
        np.testing.assert_allclose(got[t], np.einsum("hvc,c->hv", wuv, c_s), rtol=1e-12, atol=1e-13)


def check_mla_zero_query_mean(ref):
    """q = 0: all logits equal, weights uniform, the latent average is the
    mean of the selected rows; and the result ignores the order of idx."""
    q, kv, starts, q_seq, q_pos, idx, wuv = _mla_inputs(47, 3, [64], 10)
    q[:] = 0.0
    got = ref.sparse_mla(q, kv, starts, q_seq, idx, wuv, 1.0 / 16)
    perm = idx[:, ::-1].copy()
    got2 = ref.sparse_mla(q, kv, starts, q_seq, perm, wuv, 1.0 / 16)
    np.testing.assert_allclose(got, got2, rtol=1e-12, atol=1e-14)
    for t in range(3):
        sel = idx[t][idx[t] >= 0]
        mean = kv[sel, :512].mean(axis=0)
        np.testing.assert_allclose(got[t], np.einsum("hvc,c->hv", wuv, mean), rtol=1e-12, atol=1e-13)


def check_mla_hand_example(ref):
    """Two rows, hand-computed.  One head sees dim 0 of the rope part:
    q = 16 ln 3 at dim 512, row A has 0 there and row B has 1, so the logits
    are 0 and ln 3 (scale 1/16) and the weights 1/4 and 3/4.  Latents:
    A = (0, 4, 0, ...), B = (4, 0, 8, ...), so obar = (3, 1, 6, 0, ...).
    W_UV of that head copies latent dims to value dims (v = c for c < 256),
    so out = (3, 1, 6, 0, ...)."""
    q = np.zeros((1, 64, 576))
    q[0, 5, 512] = 16 * math.log(3.0)
    kv = np.zeros((2, 576))
    kv[0, 1] = 4.0
    kv[1, 0], kv[1, 2], kv[1, 512] = 4.0, 8.0, 1.0
    wuv = np.zeros((64, 256, 512))
    wuv[5, np.arange(256), np.arange(256)] = 1.0
    got = ref.sparse_mla(q, kv, [0], [0], np.array([[1, -1, 0]]), wuv, 1.0 / 16)
    expect = np.zeros(256)
    expect[:3] = [3.0, 1.0, 6.0]
    np.testing.assert_allclose(got[0, 5], expect, rtol=1e-14, atol=1e-14)
    assert np.all(got[0, :5] == 0.0) and np.all(got[0, 6:] == 0.0)


def _simulate_fp32_bf16(ref, q_t, rows, wuv, scale):
    """One allowed evaluation: fp32 logits and exp, weights rounded to bf16
    for the value product, fp32 normaliser, latent average rounded to bf16,
    fp32 up-projection, output rounded to bf16."""
    r32 = rows.astype(np.float32)
    z = (q_t.astype(np.float32) @ r32.T) * np.float32(scale)
    e = np.exp(z - z.max(axis=1, keepdims=True)).astype(np.float32)
    lsum = e.sum(axis=1, dtype=np.float32)
    e16 = ref.round_to_bf16(e).astype(np.float32)
    ob = (e16 @ r32[:, :512]) / lsum[:, None]
    ob16 = ref.round_to_bf16(ob).astype(np.float32)
    o = np.einsum("hvc,hc->hv", wuv.astype(np.float32), ob16)
    return ref.round_to_bf16(o)


def check_mla_error_bound_sane(ref):
    """Both derived tolerances cover an allowed fp32 / bf16 re-evaluation;
    the probabilistic one is small against the output's scale, so it can see
    mistakes the worst-case one would hide."""
    q, kv, starts, q_seq, q_pos, idx, wuv = _mla_inputs(53, 2, [3000], 2048)
    out, obar, m, l, rows, p = ref.sparse_mla(q, kv, starts, q_seq, idx, wuv, 1.0 / 16, return_parts=True)
    worst = ref.mla_error_bound(out, q, wuv, rows, p, 1.0 / 16, model="worst")
    prob = ref.mla_error_bound(out, q, wuv, rows, p, 1.0 / 16)
    for t in range(2):
        sim = _simulate_fp32_bf16(ref, q[t], rows[t], wuv, 1.0 / 16)
        assert np.all(np.abs(sim - out[t]) <= prob[t])
        assert np.all(np.abs(sim - out[t]) <= worst[t])
    assert np.all(prob <= worst)
    assert np.max(prob - 2.0 ** -8 * np.abs(out)) < 0.25 * np.sqrt(np.mean(out ** 2))


def _simulate_sliced_bf16(ref, q_t, rows, wuv, scale, kps):
    """Another allowed evaluation: the rows processed in slices of kps, each
    slice's unnormalised weighted row sum (fp32 weights against its own
    maximum, bf16 weights in the product) rounded to bf16, the slices
    combined with fp32 factors exp(m_s - max m), then as above."""
    r32 = rows.astype(np.float32)
    z = (q_t.astype(np.float32) @ r32.T) * np.float32(scale)           # [64, k]
    n = rows.shape[0]
    parts = []
    for j0 in range(0, n, kps):
        zs = z[:, j0:j0 + kps]
        ms = zs.max(axis=1, keepdims=True)
        e = np.exp(zs - ms).astype(np.float32)
        os16 = ref.round_to_bf16(ref.round_to_bf16(e).astype(np.float32) @ r32[j0:j0 + kps, :512]).astype(np.float32)
        parts.append((ms, e.sum(axis=1, dtype=np.float32)[:, None], os16))
    M = np.max([m for m, _, _ in parts], axis=0)
    num = sum(np.exp(m - M).astype(np.float32) * o for m, _, o in parts)
    den = sum(np.exp(m - M).astype(np.float32) * l for m, l, _ in parts)
    ob16 = ref.round_to_bf16((num / den).astype(np.float32)).astype(np.float32)
    o = np.einsum("hvc,hc->hv", wuv.astype(np.float32), ob16)
    return ref.round_to_bf16(o)


def check_mla_error_bound_sliced(ref):
    """With part_slices the derived tolerances also cover slice partials
    rounded to bf16 before the merge (8 slices of 256 over k = 2048), and
    they only grow against the unsliced ones."""
    q, kv, starts, q_seq, q_pos, idx, wuv = _mla_inputs(59, 2, [3000], 2048)
    out, obar, m, l, rows, p = ref.sparse_mla(q, kv, starts, q_seq, idx, wuv, 1.0 / 16, return_parts=True)
    sl = [np.arange(r.shape[0]) // 256 for r in rows]
    worst = ref.mla_error_bound(out, q, wuv, rows, p, 1.0 / 16, model="worst", part_slices=sl)
    prob = ref.mla_error_bound(out, q, wuv, rows, p, 1.0 / 16, part_slices=sl)
    prob0 = ref.mla_error_bound(out, q, wuv, rows, p, 1.0 / 16)
    for t in range(2):
        sim = _simulate_sliced_bf16(ref, q[t], rows[t], wuv, 1.0 / 16, 256)
        assert np.all(np.abs(sim - out[t]) <= prob[t])
        assert np.all(np.abs(sim - out[t]) <= worst[t])
    assert np.all(prob >= prob0) and np.any(prob > prob0)
    assert np.all(prob <= worst)


def check_round_to_bf16(ref):
    """Round to nearest, ties to even, on hand-picked binary32 values:
    1 + 2^-8 is a tie between 1 and 1 + 2^-7 and goes to the even 1;
    1 + 3 * 2^-8 ties between 1 + 2^-7 and 1 + 2^-6 and goes up;
    1 + 2^-8 + 2^-20 is above the tie and goes up."""
    vals = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -2.5, 0.0])
    expect = [1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -2.5, 0.0]
    assert list(ref.round_to_bf16(vals)) == expect


# --------------------------------------------------------------- layer stack
def check_layer_pattern_matches_pages(ref):
    g = json.load(open(os.path.join(GOLDEN, "layer_layout.json")))
    printed = []
    for count, flag in g["groups"]:
        printed += [bool(flag)] * count
    assert ref.layer_pattern(78) == printed
    assert sum(printed) == g["indexer_types_full"] and len(printed) - sum(printed) == g["indexer_types_shared"]
    for l in range(78):
        src = ref.shared_source(l)
        assert printed[src] and src <= l and all(not printed[j] for j in range(src + 1, l + 1))


def check_cache_bytes_match_modelled_costs(ref):
    """One 576-wide bf16 row per layer plus one 128-d bf16 indexer key per
    full layer reproduces the pages' modelled 93 KiB per token and 93 GiB at
    1M tokens."""
    g = json.load(open(os.path.join(GOLDEN, "modelled_costs.json")))
    n_full = sum(ref.layer_pattern(78))
    per_tok = 78 * ref.ROW_DIM * 2 + n_full * ref.INDEX_HEAD_DIM * 2
    assert round(per_tok / 1024) == g["kv_cache_per_token_kib"]
    assert round(per_tok * g["context_tokens"] / 2 ** 30) == g["kv_cache_1m_tokens_gib"]


def check_layer_stack_shares_selection(ref):
    """A 4-layer stack [full, shared, shared, shared]: each shared layer's
    output equals sparse_mla over the full layer's selection with the shared
    layer's own inputs; a stack starting with a shared layer is refused."""
    rng = _rng(59)
    lens, qs, ps = [40, 33], [0, 1, 1], [39, 32, 20]
    T = sum(lens)
    layers = []
    for l in range(4):
        L = dict(q_abs=rng.standard_normal((3, 64, 576)) / 24, kv=rng.standard_normal((T, 576)),
                 w_uv=rng.standard_normal((64, 256, 512)) / 22.6)
        if l == 0:
            L.update(q_idx=rng.standard_normal((3, 32, 128)) / 11, w=rng.standard_normal((3, 32)),
                     k_idx=rng.standard_normal((T, 128)))
        layers.append(L)
    outs, idxs, _ = ref.layer_stack(layers, [0, 40], qs, ps, k=16, full=[True, False, False, False])
    sc = ref.indexer_scores(layers[0]["q_idx"], layers[0]["w"], layers[0]["k_idx"], [0, 40], qs, ps)
    sel = np.stack([sorted(range(ps[t] + 1), key=lambda s: (-sc[t, s], s))[:16] for t in range(3)])
    assert np.array_equal(np.sort(sel, axis=1), idxs[0])
    for l in range(4):
        np.testing.assert_allclose(outs[l], ref.sparse_mla(layers[l]["q_abs"], layers[l]["kv"], [0, 40], qs, sel,
                                                           layers[l]["w_uv"], 1.0 / 16), rtol=1e-12, atol=1e-14)
    try:
        ref.layer_stack(layers, [0, 40], qs, ps, k=16, full=[False, True, False, False])
    except ValueError:
        pass
    else:
        raise AssertionError("stack starting with a shared layer accepted")


# ------------------------------------------------------ MTP shared selection
# [GLM-5.2 llm-atlas] index_share_for_mtp_iteration; the reading: one
# selection per group of draft tokens, cut at each token's own position.

def check_mtp_share_hand_example(ref):
    sel = np.array([[2, 5, 9, 12, -1, -1],
                    [0, 1, 3, -1, -1, -1]])
    sel_of = [0, 0, 0, 0, 1, 1]
    q_pos = [9, 5, 4, 12, 3, 0]
    expect = np.array([[2, 5, 9, -1, -1, -1],
                       [2, 5, -1, -1, -1, -1],
                       [2, -1, -1, -1, -1, -1],
                       [2, 5, 9, 12, -1, -1],
                       [0, 1, 3, -1, -1, -1],
                       [0, -1, -1, -1, -1, -1]])
    assert np.array_equal(ref.share_selection(sel, sel_of, q_pos), expect)


def _mtp_layers(rng, n_sel, n_q, T, n_layers=2):
    layers = []
    for l in range(n_layers):
        L = dict(q_abs=_bf16_grid(rng.standard_normal((n_q, 64, 576)) / 24),
                 kv=_bf16_grid(rng.standard_normal((T, 576))),
                 w_uv=_bf16_grid(rng.standard_normal((64, 256, 512)) / 22.6))
        if l == 0:
            L.update(q_idx=_bf16_grid(rng.standard_normal((n_sel, 32, 128)) / 11),
                     w=rng.standard_normal((n_sel, 32)), k_idx=_bf16_grid(rng.standard_normal((T, 128))))
        layers.append(L)
    return layers


def check_mtp_share_equals_dense_masked(ref):
    """Two sequences, each verifying 4 draft tokens at its last positions; the
    group's last token selects 12 positions.  Each token's output equals
    dense additive-mask attention whose 0 entries are the selected positions
    at or before the token's own position (built here from sets)."""
    rng = _rng(71)
    lens = [40, 33]
    starts = [0, 40]
    q_seq = [0, 0, 0, 0, 1, 1, 1, 1]
    q_pos = [36, 37, 38, 39, 29, 30, 31, 32]
    sel_seq, sel_pos, sel_of = [0, 1], [39, 32], [0, 0, 0, 0, 1, 1, 1, 1]
    layers = _mtp_layers(rng, 2, 8, sum(lens))
    outs, idxs = ref.layer_stack_mtp(layers, starts, q_seq, q_pos, sel_seq, sel_pos, sel_of, k=12,
                                     full=[True, False])
    L0 = layers[0]
    sc = ref.indexer_scores(L0["q_idx"], L0["w"], L0["k_idx"], starts, sel_seq, sel_pos)
    chosen = [set(sorted(range(sel_pos[s] + 1), key=lambda p: (-sc[s, p], p))[:12]) for s in range(2)]
    for t in range(8):
        allowed = sorted(p for p in chosen[sel_of[t]] if p <= q_pos[t])
        assert sorted(idxs[0][t][idxs[0][t] >= 0].tolist()) == allowed
        mask_idx = np.array([allowed])
        for l in range(2):
            exp = _dense_masked_reference(layers[l]["q_abs"][t:t + 1], layers[l]["kv"], starts, [q_seq[t]],
                                          [q_pos[t]], mask_idx, layers[l]["w_uv"], 1.0 / 16)
            np.testing.assert_allclose(outs[l][t], exp[0], rtol=1e-10, atol=1e-12)


def check_mtp_take_all_equals_unshared(ref):
    """When every causal set fits in k, the shared selection cut at a token's
    position is that token's whole causal set: the same as each token
    selecting for itself."""
    rng = _rng(73)
    lens = [20, 15]
    q_seq, q_pos = [0, 0, 0, 1, 1], [16, 17, 19, 13, 14]
    sel_seq, sel_pos, sel_of = [0, 1], [19, 14], [0, 0, 0, 1, 1]
    layers = _mtp_layers(rng, 2, 5, sum(lens))
    outs, idxs = ref.layer_stack_mtp(layers, [0, 20], q_seq, q_pos, sel_seq, sel_pos, sel_of, k=32,
                                     full=[True, False])
    own = [dict(L) for L in layers]
    own[0]["q_idx"] = layers[0]["q_idx"][sel_of]
    own[0]["w"] = layers[0]["w"][sel_of]
    outs2, idxs2, _ = ref.layer_stack(own, [0, 20], q_seq, q_pos, k=32, full=[True, False])
    assert np.array_equal(idxs[0], idxs2[0])
    for a, b in zip(outs, outs2):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def check_mtp_identity_sharing_is_plain_stack(ref):
    """Each token its own selecting query: the plain layer stack."""
    rng = _rng(79)
    lens = [50, 30]
    q_seq, q_pos = [0, 1, 1], [49, 29, 12]
    layers = _mtp_layers(rng, 3, 3, sum(lens))
    outs, idxs = ref.layer_stack_mtp(layers, [0, 50], q_seq, q_pos, q_seq, q_pos, [0, 1, 2], k=8,
                                     full=[True, False])
    outs2, idxs2, _ = ref.layer_stack(layers, [0, 50], q_seq, q_pos, k=8, full=[True, False])
    assert np.array_equal(idxs[0], idxs2[0])
    for a, b in zip(outs, outs2):
        np.testing.assert_allclose(a, b, rtol=0, atol=0)


# ---------------------------------------------------------------- cache write
# [GLM-5.2 techniques map] rows "Multi-head latent attention", "QK
# normalization", "Partial RoPE", "YaRN RoPE scaling"; [GLM-5.2 llm-atlas]
# rope_theta 8e6, rms_norm_eps 1e-5, rope_interleave true.

def check_rope_position_zero_is_identity(ref):
    x = _rng(40).standard_normal((3, 64))
    assert np.array_equal(ref.rope_interleaved(x, [0, 0, 0]), x)


def check_rope_frequencies_from_theta(ref):
    # One-hot input on the first slot of pair i at position 1: the pair turns
    # by exactly that pair's frequency into its second slot (the interleaved
    # layout), pair 0 turns by 1 radian, and consecutive frequencies fall by
    # the factor theta^(-2/64), theta = 8e6.
    d = 64
    freqs = []
    for i in range(d // 2):
        x = np.zeros((1, d))
        x[0, 2 * i] = 1.0
        y = ref.rope_interleaved(x, [1])[0]
        others = np.delete(y, [2 * i, 2 * i + 1])
        assert np.all(others == 0.0), "rotation leaves its pair"
        freqs.append(math.atan2(y[2 * i + 1], y[2 * i]))
    freqs = np.array(freqs)
    assert abs(freqs[0] - 1.0) < 1e-15
    assert np.allclose(freqs[1:] / freqs[:-1], 8.0e6 ** (-2.0 / 64), rtol=1e-12, atol=0)


def check_rope_is_a_rotation_by_relative_position(ref):
    # Pair norms are kept, turning by a then b equals turning by a + b, and the
    # product of two rotated vectors depends only on their distance.
    r = _rng(41)
    q, k = r.standard_normal((1, 64)), r.standard_normal((1, 64))
    for a, b in [(3, 11), (1000, 17), (1 << 20, 5)]:
        qa = ref.rope_interleaved(q, [a])
        assert np.allclose(qa[0, 0::2] ** 2 + qa[0, 1::2] ** 2, q[0, 0::2] ** 2 + q[0, 1::2] ** 2, rtol=1e-12)
        assert np.allclose(ref.rope_interleaved(qa, [b]), ref.rope_interleaved(q, [a + b]), atol=1e-9)
        lhs = float(ref.rope_interleaved(q, [a + b])[0] @ ref.rope_interleaved(k, [b])[0])
        rhs = float(ref.rope_interleaved(q, [a])[0] @ k[0])
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def check_rms_norm_closed_forms(ref):
    n = 512
    for c in [1e-3, 0.5, 7.0]:
        y = ref.rms_norm(np.full((1, n), c), np.ones(n))
        assert np.allclose(y, c / math.sqrt(c * c + 1e-5), rtol=1e-14)
    x = _rng(42).standard_normal((4, n))
    ms = np.mean(x ** 2, axis=1)
    y = ref.rms_norm(x, np.ones(n))
    assert np.allclose(np.mean(y ** 2, axis=1), ms / (ms + 1e-5), rtol=1e-12)
    g = _rng(43).standard_normal(n)
    assert np.allclose(ref.rms_norm(x, g), ref.rms_norm(x, np.ones(n)) * g, rtol=1e-14)
    assert np.allclose(ref.rms_norm(1e3 * x, np.ones(n)), ref.rms_norm(x, np.ones(n)), rtol=1e-5)


def check_layer_norm_closed_forms(ref):
    n = 128
    r = _rng(44)
    x = 3.0 + 2.0 * r.standard_normal((5, n))
    y = ref.layer_norm(x, np.ones(n), np.zeros(n))
    var = np.var(x, axis=1)           # population variance
    assert np.allclose(np.mean(y, axis=1), 0.0, atol=1e-12)
    assert np.allclose(np.mean(y ** 2, axis=1), var / (var + 1e-5), rtol=1e-12)
    w, b = r.standard_normal(n), r.standard_normal(n)
    assert np.allclose(ref.layer_norm(x, w, b), y * w + b, rtol=1e-13, atol=1e-13)
    assert np.allclose(ref.layer_norm(np.full((1, n), 4.25), w, b), b, atol=1e-12)


def check_cache_rows_structure(ref):
    r = _rng(45)
    n = 6
    kv_a = _bf16_grid(r.standard_normal((n, 576)))
    gamma = np.ones(512)
    pos = [0, 1, 7, 4096, 131071, 1048575]
    rows = ref.cache_rows_from_projection(kv_a, gamma, pos)
    assert rows.shape == (n, 576)
    assert np.array_equal(ref.round_to_bf16(rows), rows)
    lat = kv_a[:, :512]
    ms = np.mean(lat ** 2, axis=1, keepdims=True)
    assert np.allclose(rows[:, :512], lat / np.sqrt(ms + 1e-5), rtol=2 ** -8)
    rot, k = rows[:, 512:], kv_a[:, 512:]
    assert np.allclose(rot[:, 0::2] ** 2 + rot[:, 1::2] ** 2, k[:, 0::2] ** 2 + k[:, 1::2] ** 2, rtol=2 ** -6, atol=1e-4)
    assert np.array_equal(rot[0], k[0])           # position 0: no turn (k is bf16 already)


def check_indexer_keys_structure(ref):
    r = _rng(46)
    n = 4
    k_raw = _bf16_grid(r.standard_normal((n, 128)))
    w, b = r.standard_normal(128), r.standard_normal(128)
    pos = [0, 3, 65536, 1048575]
    keys = ref.indexer_keys_from_projection(k_raw, w, b, pos)
    mean = np.mean(k_raw, axis=1, keepdims=True)
    var = np.mean((k_raw - mean) ** 2, axis=1, keepdims=True)
    ln = (k_raw - mean) / np.sqrt(var + 1e-5) * w + b
    assert np.allclose(keys[:, :64], ln[:, :64], rtol=2 ** -8, atol=1e-6)    # first half: not turned
    assert np.allclose(keys[0], ln[0], rtol=2 ** -8, atol=1e-6)              # position 0: not turned
    rot = keys[:, 64:]
    assert np.allclose(rot[:, 0::2] ** 2 + rot[:, 1::2] ** 2, ln[:, 64::2] ** 2 + ln[:, 65::2] ** 2, rtol=2 ** -6, atol=1e-4)
    assert not np.allclose(rot[1:], ln[1:, 64:], rtol=1e-3)                  # later positions: turned


# ----------------------------------------------------------------- query side
# [GLM-5.2 techniques map] rows "Multi-head latent attention" (q_lora
# bottleneck, kv_b_proj key/value rows per head) and "Partial RoPE" (192
# unturned + 64 turned query dims per head); [GLM-5.2 architectures]
# q_lora_rank 2,048; [GLM-5.2 llm-atlas] qk_head_dim 256, rope_theta 8e6.

def _q_weights(rng, scale=1.0):
    w_qb = _bf16_grid(rng.standard_normal((64 * 256, 2048)) * scale)
    w_iq = _bf16_grid(rng.standard_normal((32 * 128, 2048)) * scale)
    w_iw = rng.standard_normal((32, 2048)).astype(np.float32).astype(np.float64)
    return w_qb, w_iq, w_iw


def check_qproj_one_hot_columns(ref):
    """c_q = e_j: every projection returns column j; at position 0 nothing
    turns; at position p > 0 only the rope part of each head turns (pairs
    keep their length, pair 0 turns by p radians)."""
    rng = _rng(81)
    w_qb, w_iq, w_iw = _q_weights(rng)
    j = 1234
    c = np.zeros((2, 2048))
    c[:, j] = 1.0
    q, qi, w = ref.q_project(c, w_qb, w_iq, w_iw, [0, 5])
    assert np.array_equal(q[0].reshape(-1), w_qb[:, j])
    assert np.array_equal(qi[0].reshape(-1), w_iq[:, j])
    assert np.array_equal(w[0], w_iw[:, j]) and np.array_equal(w[1], w_iw[:, j])
    col = w_qb[:, j].reshape(64, 256)
    assert np.array_equal(q[1, :, :192], col[:, :192])                    # nope part: not turned
    a, b = col[:, 192], col[:, 193]
    np.testing.assert_allclose(q[1, :, 192], a * np.cos(5.0) - b * np.sin(5.0), rtol=2 ** -7, atol=1e-30)
    np.testing.assert_allclose(q[1, :, 193], a * np.sin(5.0) + b * np.cos(5.0), rtol=2 ** -7, atol=1e-30)
    r = q[1, :, 192:]
    np.testing.assert_allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, col[:, 192::2] ** 2 + col[:, 193::2] ** 2,
                               rtol=2 ** -6)
    icol = w_iq[:, j].reshape(32, 128)
    assert np.array_equal(qi[1, :, :64], icol[:, :64])                    # indexer: first half not turned
    assert not np.allclose(qi[1, :, 64:], icol[:, 64:], rtol=1e-3)


def check_qproj_rounds_to_nearest_even(ref):
    """Two-hot c_q whose exact sums fall between bf16 values: 1 + 2^-8 + 2^-10
    rounds up to 1 + 2^-7, 1 + 2^-9 down to 1, the tie 1 + 2^-8 to even (1)."""
    w_qb = np.zeros((64 * 256, 2048))
    w_iq = np.zeros((32 * 128, 2048))
    w_iw = np.zeros((32, 2048))
    w_qb[:, 0] = 1.0
    w_iq[:, 0] = 1.0
    c = np.zeros((3, 2048))
    c[:, 0] = 1.0
    c[:, 1] = [2.0 ** -8 + 2.0 ** -10, 2.0 ** -9, 2.0 ** -8]
    w_qb[:, 1] = 1.0
    w_iq[:, 1] = 1.0
    q, qi, _ = ref.q_project(c, w_qb, w_iq, w_iw, [0, 0, 0])
    for t, v in enumerate([1 + 2.0 ** -7, 1.0, 1.0]):
        assert np.all(q[t] == v) and np.all(qi[t] == v), t
    # The rope pair is rounded before it turns: at position 2 the pair
    # (1.0078125, 1.0078125) (the bf16 value of 1 + 2^-8 + 2^-10) turns to
    # (cos 2 - sin 2, sin 2 + cos 2) * 1.0078125 = (-1.33573..., 0.49621...),
    # stored as (-1.3359375, 0.49609375); turning the unrounded sum would give
    # -1.328125 for the first.
    q2, _, _ = ref.q_project(c[:1], w_qb, w_iq, w_iw, [2])
    assert np.all(q2[0, :, 192] == -1.3359375) and np.all(q2[0, :, 193] == 0.49609375)


def check_qabsorb_integer_exact_explicit_logits(ref):
    """With small-integer inputs every step is exact: the absorbed query's
    logit against [latent ; k_rope] equals the explicit form
    q_nope . (W_UK latent) + q_rope . k_rope, head by head."""
    rng = _rng(83)
    n = 3
    q = rng.integers(-1, 2, size=(n, 64, 256)).astype(np.float64)
    w_uk = rng.integers(-1, 2, size=(64, 192, 512)).astype(np.float64)
    rows = rng.integers(-2, 3, size=(5, 576)).astype(np.float64)
    qa = ref.q_absorb(q, w_uk)
    assert qa.shape == (n, 64, 576)
    for t in range(n):
        for h in range(64):
            k_nope = w_uk[h] @ rows[:, :512].T                  # [192, 5]: explicit keys
            explicit = q[t, h, :192] @ k_nope + q[t, h, 192:] @ rows[:, 512:].T
            assert np.array_equal(qa[t, h] @ rows.T, explicit), (t, h)


def check_qproj_turned_query_scores_by_relative_position(ref):
    """The turned query against keys turned by the cache write scores by
    relative position: (p, s) and (p + d, s + d) give the same rope logit."""
    rng = _rng(87)
    w_qb, w_iq, w_iw = _q_weights(rng, scale=0.05)
    c = _bf16_grid(rng.standard_normal((1, 2048)))
    kv_a = _bf16_grid(rng.standard_normal((1, 576)))
    gamma = np.ones(512)
    for p, s, d in [(1000, 900, 5000), (70000, 3, 400000)]:
        q1, _, _ = ref.q_project(c, w_qb, w_iq, w_iw, [p])
        q2, _, _ = ref.q_project(c, w_qb, w_iq, w_iw, [p + d])
        k1 = ref.cache_rows_from_projection(kv_a, gamma, [s])[0, 512:]
        k2 = ref.cache_rows_from_projection(kv_a, gamma, [s + d])[0, 512:]
        l1 = q1[0, :, 192:] @ k1
        l2 = q2[0, :, 192:] @ k2
        scale = np.abs(q1[0, :, 192:]) @ np.abs(k1)
        assert np.all(np.abs(l1 - l2) <= 2 ** -6 * scale), (p, s, d)


def check_projection_error_bound_covers_fp32(ref):
    rng = _rng(89)
    a = _bf16_grid(rng.standard_normal((4, 2048)))
    b = _bf16_grid(rng.standard_normal((6, 2048)))
    exact = a @ b.T
    bound = ref.projection_error_bound(a, b)
    prods = (a[:, None, :] * b[None, :, :]).astype(np.float32)          # exact: bf16 x bf16 fits fp32
    for order in (slice(None), slice(None, None, -1)):
        acc = np.zeros((4, 6), dtype=np.float32)
        for k in range(2048)[order]:
            acc = acc + prods[:, :, k]
        assert np.all(np.abs(acc.astype(np.float64) - exact) <= bound)
    pair = prods.copy()
    while pair.shape[-1] > 1:
        pair = (pair[..., 0::2] + pair[..., 1::2]).astype(np.float32)
    assert np.all(np.abs(pair[..., 0].astype(np.float64) - exact) <= bound)
    # near the worst case: 1 followed by 2047 products of 2^-24, each lost
    # against the running fp32 sum (a tie to even at 1.0): error 2047 u
    a1 = np.full((1, 2048), 2.0 ** -12)
    a1[0, 0] = 1.0
    acc = np.float32(0.0)
    for k in range(2048):
        acc = np.float32(acc + np.float32(a1[0, k] * a1[0, k]))
    err = abs(float(acc) - float(a1[0] @ a1[0]))
    assert err > 2000 * 2.0 ** -24 and err <= ref.projection_error_bound(a1, a1)[0, 0]


# ------------------------------------------------------------------ FP8 caches
# [GLM-5.2 techniques map] "inference quantization" (FP8 inference); the
# format facts below are the OCP 8-bit floating point specification's E4M3.

def check_e4m3_published_values(ref):
    v = ref.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest finite magnitude
    assert v(0x08) == 2.0 ** -6 and v(0x07) == 7 * 2.0 ** -9 and v(0x01) == 2.0 ** -9   # smallest normal, subnormals
    assert v(0x38) == 1.0 and v(0x3F) == 1.875 and v(0x40) == 2.0
    assert v(0x00) == 0.0 and np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    mags = np.array([v(c) for c in range(127)])
    assert np.all(np.diff(mags) > 0)                       # 127 finite magnitudes, increasing


def check_e4m3_encode_rounding(ref):
    enc = ref.e4m3_encode
    codes = np.arange(127)
    vals = np.array([ref.e4m3_value(c) for c in codes])
    assert np.array_equal(enc(vals), codes) and np.array_equal(enc(-vals[1:]), codes[1:] | 0x80)
    # midpoints between neighbours go to the even code
    mid = (vals[:-1] + vals[1:]) / 2
    got = enc(mid).astype(np.int64)
    assert np.all(got % 2 == 0) and np.all((got == codes[:-1]) | (got == codes[1:]))
    # just above / below a midpoint go to the nearer code
    assert np.array_equal(enc(mid * (1 + 1e-9)), codes[1:]) and np.array_equal(enc(mid * (1 - 1e-9)), codes[:-1])
    assert enc(np.array([1e6]))[0] == 0x7E and enc(np.array([-500.0]))[0] == 0xFE and enc(np.array([449.0]))[0] == 0x7E
    assert enc(np.array([2.0 ** -11]))[0] == 0 and enc(np.array([3 * 2.0 ** -11]))[0] == 1   # 2^-10 ties to 0; 1.5 * 2^-10 up


def check_quantize_rows_fp8(ref):
    rng = _rng(91)
    x = _bf16_grid(rng.standard_normal((6, 576)) * np.array([[1e-3], [1], [30], [1], [1], [0]]))
    x[3, 7] = 100.0                                        # a spike sets the scale
    x[4] = -x[4]
    codes, scales = ref.quantize_rows_fp8(x)
    deq = ref.dequantize_rows_fp8(codes, scales)
    for r in range(5):
        am = np.max(np.abs(x[r]))
        assert np.float32(scales[r]) == np.float32(np.float32(am) / np.float32(448))
        i = np.argmax(np.abs(x[r]))
        assert codes[r, i] & 0x7F == 0x7E                  # the row maximum lands on +-448
        # per element: at most half a step of the format at the element's size
        # (relative 2^-4 for normal codes, 2^-10 scale for subnormals), plus the
        # fp32 division's rounding
        err = np.abs(deq[r] - x[r])
        assert np.all(err <= 2.0 ** -4 * np.abs(x[r]) + 2.0 ** -10 * scales[r] + 1e-6 * np.abs(x[r]))
    assert np.all(codes[5] == 0) and scales[5] == 1.0 and np.all(deq[5] == 0)
    assert np.array_equal(ref.quantize_rows_fp8(deq[:5])[0], codes[:5])   # quantizing the decoded rows is stable


def check_fp8_indexer_scores_scale_out(ref):
    """ReLU commutes with a positive scale: the score of a key stored as
    (codes, scale) is scale times the score of the decoded codes alone."""
    rng = _rng(93)
    T = 50
    k = _bf16_grid(rng.standard_normal((T, 128)))
    codes, scales = ref.quantize_rows_fp8(k)
    q = _bf16_grid(rng.standard_normal((2, 32, 128)) / 11)
    w = rng.standard_normal((2, 32))
    full = ref.indexer_scores(q, w, ref.dequantize_rows_fp8(codes, scales), [0], [0, 0], [49, 30])
    unit = ref.indexer_scores(q, w, ref.E4M3_TABLE[codes.astype(np.int64)], [0], [0, 0], [49, 30])
    np.testing.assert_allclose(full[:, :31], unit[:, :31] * scales[None, :31], rtol=1e-12, atol=1e-300)


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]

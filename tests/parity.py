"""Parity checks of the HIP path against the CPU oracle (used by the gpu tests).

Tolerances (written here, derived in the oracle):
  indexer scores   |gpu - exact| <= score_error_bound (worst-case fp32
                   summation bound over any order), entries past q_pos are -inf.
  top-k            the oracle's selection run on the GPU's own fp32 scores must
                   equal the GPU's idx exactly (an integer decision taken in the
                   kernel's precision); against the oracle's exact scores, every
                   position in the symmetric difference must score within
                   1e-3 * |I(sigma_k)| + eps(sigma_k) + eps(s) of the oracle's
                   k-th pick sigma_k (eps = the score error bound).
  attention        the benchmark spec bar: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|;
                   and the derived probabilistic bound of mla_error_bound.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import ref
from sparse_attention_relu_amd.synth import to_numpy


def np_batch(batch):
    return dict(seq_start=to_numpy(batch.seq_start), q_seq=to_numpy(batch.q_seq), q_pos=to_numpy(batch.q_pos))


def check_scores(L, B, scores_gpu, rows=None, extra_rel=0.0):
    """L: numpy layer dict (q_idx, w, k_idx); B: numpy batch dict; scores_gpu float64 [n_q, ld].
    extra_rel: one more fp32 rounding of the score (FP8 keys: the codes' score
    times the key's scale), added as extra_rel * |exact|."""
    n_q, ld = scores_gpu.shape
    rows = range(n_q) if rows is None else rows
    worst = 0.0
    for t in rows:
        p = int(B["q_pos"][t])
        exact = ref.indexer_scores_at(L["q_idx"], L["w"], L["k_idx"], B["seq_start"], B["q_seq"], B["q_pos"], t,
                                      np.arange(p + 1))
        base = int(B["seq_start"][B["q_seq"][t]])
        bound = ref.score_error_bound(L["q_idx"][t], L["w"][t], L["k_idx"][base:base + p + 1]) + extra_rel * np.abs(exact)
        err = np.abs(scores_gpu[t, :p + 1] - exact)
        bad = np.nonzero(err > bound)[0]
        assert bad.size == 0, f"row {t}: {bad.size} scores outside the fp32 bound, first at s={bad[0]}: " \
                              f"gpu={scores_gpu[t, bad[0]]!r} exact={exact[bad[0]]!r} bound={bound[bad[0]]!r}"
        assert np.all(np.isneginf(scores_gpu[t, p + 1:])), f"row {t}: entries past q_pos are not -inf"
        worst = max(worst, float(np.max(err / np.maximum(bound, 1e-300))))
    return worst


def check_topk_exact(scores_gpu, q_pos, k, idx_gpu, rows=None):
    """The oracle's selection on the GPU's own scores equals the GPU's idx."""
    rows = range(scores_gpu.shape[0]) if rows is None else rows
    for t in rows:
        expect = ref.topk_select(scores_gpu[t], int(q_pos[t]), k)
        got = idx_gpu[t]
        if not np.array_equal(expect, got):
            d = np.setxor1d(expect[expect >= 0], got[got >= 0])
            raise AssertionError(f"row {t}: top-k differs from the oracle on the GPU's scores "
                                 f"({d.size} positions differ, first {d[:8]}); got head {got[:8]} tail {got[-4:]}")


def check_topk_band(L, B, idx_gpu, k, rows=None, extra_rel=0.0):
    """The GPU's selection against the oracle's exact scores, with the tie band."""
    n_q = idx_gpu.shape[0]
    rows = range(n_q) if rows is None else rows
    for t in rows:
        p = int(B["q_pos"][t])
        exact = ref.indexer_scores_at(L["q_idx"], L["w"], L["k_idx"], B["seq_start"], B["q_seq"], B["q_pos"], t,
                                      np.arange(p + 1))
        row = np.full(p + 1, -np.inf)
        row[:] = exact
        orc = ref.topk_select(row, p, k)
        got = idx_gpu[t]
        k_eff = min(k, p + 1)
        assert np.all(got[k_eff:] == -1) and np.all(got[:k_eff] >= 0) and np.all(got[:k_eff] <= p)
        assert np.all(np.diff(got[:k_eff]) > 0), f"row {t}: idx not strictly ascending"
        diff = np.setxor1d(orc[orc >= 0], got[got >= 0])
        if diff.size == 0:
            continue
        sel = orc[orc >= 0]
        sigma = sel[np.lexsort((-sel, exact[sel]))[0]]      # the oracle's k-th pick
        base = int(B["seq_start"][B["q_seq"][t]])
        keys = L["k_idx"][base:base + p + 1]
        pts = np.concatenate([[sigma], diff])
        eps = ref.score_error_bound(L["q_idx"][t], L["w"][t], keys[pts]) + extra_rel * np.abs(exact[pts])
        tau = 1e-3 * abs(exact[sigma]) + eps[0] + eps[1:]
        gap = np.abs(exact[diff] - exact[sigma])
        assert np.all(gap <= tau), f"row {t}: swapped positions outside the tie band: {diff[gap > tau][:8]}"


def part_slices(idx_rows, n_launch, k):
    """The slice of each selected entry (valid entries of each idx row, in
    order) when the attention launch of n_launch queries with k entries
    rounds its partial states to bf16 (sa_mla_partial_bits), else None."""
    from sparse_attention_relu_amd import api
    if api.mla_partial_bits(n_launch, k) != 16:
        return None
    kps = api.mla_split_info(n_launch, k)[1]
    return [np.nonzero(np.asarray(r) >= 0)[0] // kps for r in idx_rows]


def check_mla(Lnp, B, idx_gpu, out_gpu, scale, rows=None, lse_gpu=None, n_launch=None):
    """out_gpu float64 [n_q, 64, 256] (bf16 widened); idx_gpu int64 [n_q, k].
    n_launch: the query count of the attention launch when idx_gpu holds only
    some of its rows (default: every row of idx_gpu)."""
    rows = list(range(idx_gpu.shape[0])) if rows is None else list(rows)
    sub = lambda a: a[rows]
    out, obar, m, l, rows_l, p_l = ref.sparse_mla(sub(Lnp["q_abs"]), Lnp["kv"], B["seq_start"], sub(B["q_seq"]),
                                                  sub(idx_gpu), Lnp["w_uv"], scale, return_parts=True)
    slices = part_slices(sub(idx_gpu), n_launch or idx_gpu.shape[0], idx_gpu.shape[1])
    got = out_gpu[rows]
    err = np.abs(got - out)
    ns = 2e-2 + 1e-2 * np.abs(out)
    assert np.all(err <= ns), f"outside the 2e-2 + 1e-2|x| bar: max err {err.max()}"
    bound = ref.mla_error_bound(out, sub(Lnp["q_abs"]), Lnp["w_uv"], rows_l, p_l, scale, part_slices=slices)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{len(bad)} outputs outside the derived bound; first {bad[0]}: " \
                          f"gpu={got[tuple(bad[0])]} oracle={out[tuple(bad[0])]} bound={bound[tuple(bad[0])]}"
    if lse_gpu is not None:
        np.testing.assert_allclose(lse_gpu[rows], m + np.log(l), rtol=1e-5, atol=1e-5)
    return float(np.max(err / np.maximum(bound, 1e-300)))


def layer_np(L):
    return {k: to_numpy(getattr(L, k)) for k in ("q_idx", "w", "k_idx", "q_abs", "kv", "w_uv")}


# ----------------------------------------------------------------- query side
# Derived tolerances.  A stored bf16 value y = rnd(sum) where the GPU's fp32
# sum differs from the exact one by at most eps = projection_error_bound
# (gamma_{K+1} sum |a_k b_k|); the oracle rounds the exact sum (through fp32).
# Both roundings move a value by at most half a bf16 ulp (<= 2^-8 |x|), so
#   |gpu - oracle| <= eps + 2^-7 (|s| + eps) + 2^-23 |s|.
# A turned pair starts from two such values (errors d0, d1), turns in fp64
# (error ~1e-16, allowed 2^-20 of the pair's size) and is rounded again:
#   |gpu - oracle| <= d0 + d1 + 2^-7 (|y| + d0 + d1) + 2^-20 (|x0| + |x1|).

def _bf16_bound(s, eps):
    return eps + 2.0 ** -7 * (np.abs(s) + eps) + 2.0 ** -23 * np.abs(s) + 1e-30


def _check_bf16_part(name, got, exact, eps, rope_first, d, pos, ref_rounded):
    """got / ref_rounded [n, H, d]; exact / eps [n, H, d] before rounding."""
    b_pre = _bf16_bound(exact, eps)
    bound = b_pre.copy()
    if rope_first is not None:
        d0, d1 = b_pre[..., rope_first::2], b_pre[..., rope_first + 1::2]
        x0, x1 = np.abs(exact[..., rope_first::2]), np.abs(exact[..., rope_first + 1::2])
        for off, y in ((0, ref_rounded[..., rope_first::2]), (1, ref_rounded[..., rope_first + 1::2])):
            bound[..., rope_first + off::2] = d0 + d1 + 2.0 ** -7 * (np.abs(y) + d0 + d1) + 2.0 ** -20 * (x0 + x1)
    err = np.abs(got - ref_rounded)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{name}: {len(bad)} values outside the derived bound; first {tuple(bad[0])}: " \
                          f"gpu={got[tuple(bad[0])]} oracle={ref_rounded[tuple(bad[0])]} bound={bound[tuple(bad[0])]}"
    return float(np.mean(err > 0))


def check_q_project(c_q, w_qb, pos, q_gpu, w_iq=None, w_iw=None, qi_gpu=None, w_gpu=None):
    """All numpy float64 (bf16 values widened); returns the fraction of
    stored values that differ from the oracle's (a rounding-boundary rate)."""
    n = c_q.shape[0]
    if w_iq is None:
        w_iq, w_iw = np.zeros((32 * 128, 2048)), np.zeros((32, 2048))
    q_o, qi_o, w_o = ref.q_project(c_q, w_qb, w_iq, w_iw, pos)
    s = (c_q @ w_qb.T).reshape(n, 64, 256)
    eps = ref.projection_error_bound(c_q, w_qb).reshape(n, 64, 256)
    frac = _check_bf16_part("q", q_gpu, s, eps, 192, 256, pos, q_o)
    if qi_gpu is not None:
        si = (c_q @ w_iq.T).reshape(n, 32, 128)
        epsi = ref.projection_error_bound(c_q, w_iq).reshape(n, 32, 128)
        frac = max(frac, _check_bf16_part("q_idx", qi_gpu, si, epsi, 64, 128, pos, qi_o))
        epsw = ref.projection_error_bound(c_q, w_iw)
        err = np.abs(w_gpu - c_q @ w_iw.T)
        assert np.all(err <= epsw), f"w: max err {err.max()} against bound {epsw[err > epsw][:4]}"
    return frac


def check_q_absorb(q_gpu, w_uk, qa_gpu):
    """q_abs on the GPU's own q (the absorption alone); w_uk [64, 192, 512]."""
    qa_o = ref.q_absorb(q_gpu, w_uk)
    n = q_gpu.shape[0]
    exact = np.einsum("nhd,hdc->nhc", q_gpu[:, :, :192], w_uk)
    eps = np.stack([ref.projection_error_bound(q_gpu[:, h, :192], w_uk[h].T) for h in range(64)], axis=1)
    frac = _check_bf16_part("q_abs", qa_gpu[:, :, :512], exact, eps, None, 512, None, qa_o[:, :, :512])
    assert np.array_equal(qa_gpu[:, :, 512:], q_gpu[:, :, 192:]), "q_abs rope part is not q's rope part"
    return frac

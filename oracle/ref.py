"""Plain CPU oracle for the indexer-selected sparse MLA hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the only thing both sides
consume is the seeded input tensors.

Everything here is written for a reader to check against the pages by eye:
NumPy in float64, a matmul or a sort as the only library primitives, no
blocking, fusion or reordering beyond what the definition states.  Inputs that
the GPU consumes as bf16 are handed in already widened (exactly) to float.

Sources, cited by page title and section:
  [GLM-5.2 techniques map]  models.inteligile.com "GLM-5.2 / Model techniques
      map", section "Checked in its code", rows "Multi-head latent attention",
      "Indexer-selected sparse attention (DeepSeek Sparse Attention)",
      "Learnable attention sink", "Gated attention output", "QK normalization",
      "Partial RoPE", "YaRN RoPE scaling".
  [GLM-5.2 architectures]   llm-architectures-explained "GLM-5.2", section
      "Every architecture field" (row "layout") and "Modelled costs".
  [GLM 5.2 hermosaai]       hermosaai "GLM 5.2", sections "78 layers,
      IndexShare pattern" and "MLA + DSA with IndexShare".
  [GLM-5.2 llm-atlas]       llm-atlas "GLM-5.2", section "Champs bruts du
      config.json" (index_topk, index_n_heads, index_head_dim, indexer_types,
      index_topk_freq, index_skip_topk_offset, kv_lora_rank, qk_rope_head_dim,
      qk_nope_head_dim, v_head_dim, qk_head_dim).

Where the pages leave a step open, the reading taken is stated next to the
code that takes it.

Pin status (what checks this module against something other than itself, all
under ``tests/`` marked ``not gpu``):
  indexer_scores     closed-form one-hot cases, the non-negative GEMV
                     reduction, w = 0, causal bound, sequence offsets.
  topk_select        full-sort brute force, pairwise order invariant, hand
                     example with ties, degenerate (all equal, n <= k).
  sparse_mla         dense additive-mask attention, dense causal attention
                     when k >= n, explicit (non-absorbed) kv_b_proj form,
                     k_eff = 1, zero query, hand-computed two-row example.
  layer_pattern      the pages' printed 78-layer layout and the 21/57 counts.
  q_project,         one- and two-hot closed forms (the nope/rope split, the
  q_absorb           bf16 rounding), integer-exact absorbed = explicit logits,
                     the relative-position property of the turned query
                     against keys turned by the cache write, the indexer
                     query's unturned first half.
  e4m3_value,        the format's published values (0x7E = 448, 0x08 = 2^-6,
  e4m3_encode,       0x01 = 2^-9, 0x38 = 1), 127 finite magnitudes in order,
  quantize_rows_fp8  round trips, midpoints to the even code, saturation, the
                     row maximum at +-448, the per-element error bound.
  share_selection,   hand example, dense additive-mask attention over the
  layer_stack_mtp    shared selection cut at each token's position, and the
                     take-all case (sharing changes nothing when every causal
                     set fits in k).
  score_error_bound  pinned against exhaustive fp32 re-summation orders on
                     small cases (the bound must cover every order).
No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# --- constants printed on the pages --------------------------------------
# [GLM-5.2 llm-atlas] config.json fields; [GLM-5.2 techniques map] MLA row.
INDEX_N_HEADS = 32        # index_n_heads
INDEX_HEAD_DIM = 128      # index_head_dim
INDEX_TOPK = 2048         # index_topk
N_HEADS = 64              # num_attention_heads
KV_LORA_RANK = 512        # kv_lora_rank (latent width)
QK_ROPE_DIM = 64          # qk_rope_head_dim
QK_NOPE_DIM = 192         # qk_nope_head_dim
V_HEAD_DIM = 256          # v_head_dim
ROW_DIM = KV_LORA_RANK + QK_ROPE_DIM   # 576: one cache row per token
N_LAYERS = 78             # num_hidden_layers
INDEX_TOPK_FREQ = 4       # index_topk_freq
INDEX_SKIP_TOPK_OFFSET = 3  # index_skip_topk_offset


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --- a1: indexer score -----------------------------------------------------
def indexer_scores(q_idx, w, k_idx, seq_start, q_seq, q_pos, ld=None):
    """Indexer scores I[t, s] for every query t and every cached position s.

    [GLM-5.2 techniques map] "Indexer-selected sparse attention": a per-query
    indexer with index_n_heads heads of index_head_dim scores past tokens
    against one key per token shared by all heads (the key has shape
    [B, S, 1, D]).  The pages give shapes only; the score taken is

        I[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[b_t, s, :])

    for s in the causal set {0 .. q_pos[t]} (diagonal included: the single
    causal mask of the "layer_types" row), and -inf for s > q_pos[t] so that
    every row of length ``ld`` is self-contained.

    q_idx [n_q, 32, 128], w [n_q, 32], k_idx [total_tokens, 128] (packed by
    sequence, row seq_start[b] + s holds position s of sequence b),
    q_seq / q_pos [n_q].  Returns float64 [n_q, ld].
    """
    q_idx, w, k_idx = _f64(q_idx), _f64(w), _f64(k_idx)
    q_seq = np.asarray(q_seq, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    seq_start = np.asarray(seq_start, dtype=np.int64)
    n_q = q_idx.shape[0]
    if ld is None:
        ld = int(q_pos.max()) + 1 if n_q else 0
    out = np.full((n_q, ld), -np.inf, dtype=np.float64)
    for t in range(n_q):
        n_t = int(q_pos[t]) + 1
        base = int(seq_start[q_seq[t]])
        keys = k_idx[base:base + n_t]                 # [n_t, 128]
        dots = q_idx[t] @ keys.T                      # [32, n_t]: q_h . k_s
        out[t, :n_t] = w[t] @ np.maximum(dots, 0.0)   # sum_h w_h ReLU(.)
    return out


def indexer_scores_at(q_idx, w, k_idx, seq_start, q_seq, q_pos, t, positions):
    """The same score as :func:`indexer_scores` for one query t at chosen
    positions only (used at sizes where a full row is too slow on the CPU).
    Positions must lie in the causal set of t."""
    positions = np.asarray(positions, dtype=np.int64)
    assert positions.size == 0 or (positions.min() >= 0 and positions.max() <= int(q_pos[t]))
    base = int(seq_start[int(q_seq[t])])
    keys = _f64(k_idx[base + positions])
    dots = _f64(q_idx[t]) @ keys.T
    return _f64(w[t]) @ np.maximum(dots, 0.0)


def score_error_bound(q_idx_t, w_t, keys, unit_roundoff=2.0 ** -23):
    """Rigorous bound on |fp32 score - exact score| for scores computed with
    exact bf16 products, fp32 sums of the 128 products per head in any order,
    fp32 ReLU, and an fp32 weighted sum over the 32 heads in any order.

    Standard worst-case summation bound (Higham, "Accuracy and Stability of
    Numerical Algorithms", ch. 3): a sum of n terms in floating point, any
    order, has error <= gamma_{n-1} * sum |terms| with
    gamma_n = n u / (1 - n u).  The per-head dot product d_h gets
    gamma_127 * sum_i |q_hi k_i|; ReLU is 1-Lipschitz so that error passes
    through; the weighted sum of 32 products w_h * r_h (each one rounding)
    adds gamma_33 * sum_h |w_h| |r_h|, and the dot-product errors enter scaled
    by |w_h|.  unit_roundoff defaults to 2^-23 (covers truncating as well as
    round-to-nearest accumulators).  Returns float64 [n_keys].
    """
    q = np.abs(_f64(q_idx_t))            # [32, 128]
    wa = np.abs(_f64(w_t))               # [32]
    k = _f64(keys)                        # [n, 128]
    u = unit_roundoff

    def gamma(n):
        return n * u / (1.0 - n * u)

    abs_dots = q @ np.abs(k).T            # [32, n]: sum_i |q_hi k_i|
    relu = np.maximum(_f64(q_idx_t) @ k.T, 0.0)
    err_dot = gamma(INDEX_HEAD_DIM) * (wa @ abs_dots)
    err_sum = gamma(INDEX_N_HEADS + 1) * (wa @ (relu + gamma(INDEX_HEAD_DIM) * abs_dots))
    return err_dot + err_sum


# --- a2: top-k selection -----------------------------------------------------
def topk_select(scores_row, q_pos_t, k=INDEX_TOPK):
    """Exact top-k of one indexer row over its causal set.

    [GLM-5.2 techniques map] "Indexer-selected sparse attention": the kept
    count is min(index_topk, number of scores), returned as int32 positions.
    The pages do not state a tie order; the reading taken is that equal scores
    go to the lower position.  Scores of -0.0 and +0.0 compare equal (numeric
    comparison), so they tie.

    Returns the selected positions in ascending order, padded with -1 to k.
    """
    n_t = int(q_pos_t) + 1
    row = _f64(scores_row)[:n_t]
    k_eff = min(int(k), n_t)
    positions = np.arange(n_t)
    order = np.lexsort((positions, -row))   # primary: score desc; then position asc
    chosen = np.sort(order[:k_eff])
    out = np.full(int(k), -1, dtype=np.int64)
    out[:k_eff] = chosen
    return out


def topk_select_rows(scores, q_pos, k=INDEX_TOPK):
    return np.stack([topk_select(scores[t], q_pos[t], k) for t in range(scores.shape[0])]) \
        if scores.shape[0] else np.zeros((0, int(k)), dtype=np.int64)


# --- a3 + a4: absorbed sparse MLA and the W_UV up-projection ------------------
def sparse_mla(q_abs, kv, seq_start, q_seq, idx, w_uv, scale, return_parts=False):
    """Attention of each query over only its selected cache rows, absorbed
    form, then the per-head value up-projection.

    [GLM-5.2 techniques map] "Multi-head latent attention": keys and values
    come from one kv_lora_rank latent per token (after kv_a_layernorm) plus a
    decoupled qk_rope_head_dim key; kv_b_proj maps the latent to, per head,
    qk_nope_head_dim key rows and v_head_dim value rows.  Folding the key
    half of kv_b_proj (W_UK) into the query and applying the value half (W_UV)
    after attention is the same product re-associated; the cache row is then
    [latent (512) ; k_rope (64)] and the folded query is 576 wide.
    "Learnable attention sink" / "Gated attention output": plain softmax with
    no extra logit and no gate.  "Indexer-selected sparse attention": each
    query attends only to its selected positions (an additive 0 / -inf mask
    in the reference code; here the selected rows are gathered).

    For each query t and head h, over the selected rows R_j (slots with
    idx = -1 are ignored):
        z_j   = scale * (q_abs[t, h] . R_j)               (all 576 dims)
        p_j   = exp(z_j - max z) / sum_j exp(z_j - max z)
        obar  = sum_j p_j * R_j[:512]
        out[t, h] = W_UV[h] @ obar                          ([256, 512] @ [512])

    Returns out float64 [n_q, 64, 256] (unrounded).  With return_parts also
    returns obar [n_q, 64, 512], the row max m [n_q, 64], the sum l [n_q, 64],
    and the per-query gathered rows (list of [k_eff, 576]) and weights (list
    of [64, k_eff]) for error-bound computations.
    """
    q_abs, kv, w_uv = _f64(q_abs), kv, _f64(w_uv)
    seq_start = np.asarray(seq_start, dtype=np.int64)
    q_seq = np.asarray(q_seq, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    n_q, n_h = q_abs.shape[0], q_abs.shape[1]
    lat = w_uv.shape[2]
    out = np.zeros((n_q, n_h, w_uv.shape[1]))
    obar_all = np.zeros((n_q, n_h, lat))
    m_all = np.zeros((n_q, n_h))
    l_all = np.zeros((n_q, n_h))
    rows_all, p_all = [], []
    for t in range(n_q):
        sel = idx[t][idx[t] >= 0]
        rows = _f64(kv[int(seq_start[q_seq[t]]) + sel])      # [k_eff, 576]
        z = scale * (q_abs[t] @ rows.T)                        # [64, k_eff]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        lsum = e.sum(axis=1, keepdims=True)
        p = e / lsum
        obar = p @ rows[:, :lat]                               # [64, 512]
        for h in range(n_h):
            out[t, h] = w_uv[h] @ obar[h]
        obar_all[t], m_all[t], l_all[t] = obar, m[:, 0], lsum[:, 0]
        rows_all.append(rows)
        p_all.append(p)
    if return_parts:
        return out, obar_all, m_all, l_all, rows_all, p_all
    return out


def round_to_bf16(x):
    """Round float values to the nearest bfloat16 (ties to even), returned as
    float64.  bfloat16 keeps the top 16 bits of an IEEE binary32; the value is
    first rounded to binary32 (exact for inputs that are binary32 already)."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    nan = np.isnan(f)
    rounded = np.where(nan, (bits >> 16) | 0x40, rounded)
    out = (rounded.astype(np.uint32) << 16).view(np.float32)
    return out.astype(np.float64)


def mla_error_bound(out, q_abs, w_uv, rows_list, p_list, scale, n_lat=KV_LORA_RANK,
                    model="probabilistic", lam=8.0, part_slices=None):
    """Per-element tolerance for the GPU's sparse MLA output, derived from the
    arithmetic the kernels are allowed (not fitted to results).

    Allowed deviations from the exact value (u32 = 2^-24 with slack 2^-23,
    ub = 2^-8 is the bf16 unit roundoff):
      * logits summed in fp32 over 576 products, scaled and moved to base 2 in
        fp32, exponentiated with a 1-2 ulp exp:
        |dz_j| <= gamma_576 scale sum_i |q_i R_ji| + 2^-21 (|z_j| + 1);
        a softmax weight then moves by at most a factor exp(2 max|dz|);
      * weights fed to the value product in bf16 and the normaliser formed
        from the unrounded fp32 weights: relative 2 ub per weight;
      * fp32 accumulation of up to 2048 weighted rows;
      * with part_slices (per query, the slice of each gathered row, in the
        order of rows_list): the selection is processed in slices whose
        partial weighted row sums are each rounded once to bf16 before they
        are combined; slice s holds a positive multiple of
        a_s = sum over its rows of p_j R_j[:512], so the latent average moves
        by at most ub sum_s |a_s| (worst) or lam ub sqrt(sum_s a_s^2);
      * the latent average fed to the up-projection in bf16 (relative 2 ub)
        and summed in fp32 over 512 terms;
      * the final rounding of the output to bf16 (ub |out|, rigorous).

    model="worst": every rounding error at its worst case and aligned
    (Higham, "Accuracy and Stability of Numerical Algorithms", ch. 3).  It is
    rigorous but of the order of the output itself.
    model="probabilistic": independent, mean-zero rounding errors (Higham and
    Mary, "A new approach to probabilistic rounding error analysis", SISC
    2019): a sum of n rounded terms errs by at most lam * u * sqrt(sum of
    squared terms) (for the per-term roundings) or lam * sqrt(n) * u * sum of
    |terms| (for the accumulation), each holding with probability at least
    1 - 2 exp(-lam^2 / 2); lam = 8 makes a false alarm ~1e-14 per element.

    Returns float64 [n_q, 64, 256].
    """
    u = 2.0 ** -23
    ub = 2.0 ** -8

    def gamma(n):
        return n * u / (1 - n * u)

    w = _f64(w_uv)
    wa = np.abs(w)
    q_abs = _f64(q_abs)
    bound = np.zeros_like(out)
    for t, (rows, p) in enumerate(zip(rows_list, p_list)):
        n_sel = rows.shape[0]
        z = scale * (q_abs[t] @ rows.T)                                # [64, k]
        dz = gamma(rows.shape[1]) * scale * (np.abs(q_abs[t]) @ np.abs(rows).T) \
            + 2.0 ** -21 * (np.abs(z) + 1.0)
        rel_z = 2.2 * dz.max(axis=1, keepdims=True)                  # [64, 1]
        v = rows[:, :n_lat]
        pv_abs = p @ np.abs(v)                                        # [64, 512]: sum_j p_j |R_j[c]|
        obar = p @ v                                                  # [64, 512]
        a_sl = None
        if part_slices is not None and n_sel > 0:
            sl = np.asarray(part_slices[t])
            a_sl = np.stack([p[:, sl == s] @ v[sl == s] for s in np.unique(sl)])   # [slices, 64, 512]
        if model == "worst":
            d_obar = (2 * ub + rel_z) * pv_abs + gamma(max(n_sel, 1)) * pv_abs
            if a_sl is not None:
                d_obar = d_obar + ub * np.abs(a_sl).sum(axis=0)
            for h in range(out.shape[1]):
                bound[t, h] = wa[h] @ d_obar[h] + (2 * ub + gamma(n_lat)) * (wa[h] @ np.abs(obar[h])) \
                    + ub * np.abs(out[t, h])
        else:
            pv_sq = np.sqrt((p ** 2) @ (v ** 2))                      # [64, 512]
            d_obar = lam * 2 * ub * pv_sq + rel_z * pv_abs + lam * np.sqrt(max(n_sel, 1)) * u * pv_abs
            if a_sl is not None:
                d_obar = d_obar + lam * ub * np.sqrt((a_sl ** 2).sum(axis=0))
            for h in range(out.shape[1]):
                prop = np.sqrt((w[h] ** 2) @ (d_obar[h] ** 2))        # errors of obar through W_UV
                rnd = lam * 2 * ub * np.sqrt((w[h] ** 2) @ (obar[h] ** 2))
                acc = lam * np.sqrt(n_lat) * u * (wa[h] @ np.abs(obar[h]))
                bound[t, h] = prop + rnd + acc + ub * np.abs(out[t, h])
    return bound


# --- a5: IndexShare layer stack ----------------------------------------------
def layer_is_full(layer: int) -> bool:
    """Whether layer l runs its own indexer.

    [GLM 5.2 hermosaai] "78 layers, IndexShare pattern": 21 of 78 layers run a
    full indexer, the rest reuse one, in groups of four after the first three.
    [GLM-5.2 llm-atlas] config fields index_topk_freq = 4 and
    index_skip_topk_offset = 3.  [GLM-5.2 architectures] "layout" row prints
    the sequence.  The reading that fits all three: layers 0, 1, 2 are full;
    after them the layers form groups of four whose last layer is full
    (layers 6, 10, ..., 74), i.e. l < 3 or l mod 4 == 2.
    """
    if layer < INDEX_SKIP_TOPK_OFFSET:
        return True
    return (layer - INDEX_SKIP_TOPK_OFFSET) % INDEX_TOPK_FREQ == INDEX_TOPK_FREQ - 1


def layer_pattern(n_layers=N_LAYERS):
    return [layer_is_full(l) for l in range(n_layers)]


def shared_source(layer: int) -> int:
    """The full layer whose selection a layer uses: itself if full, else the
    latest full layer before it."""
    l = layer
    while not layer_is_full(l):
        l -= 1
    return l


def layer_stack(layers, seq_start, q_seq, q_pos, k=INDEX_TOPK, scale=1.0 / 16, full=None):
    """Run the hot path over a stack of layers in order.

    ``layers`` is a list of dicts with keys q_idx, w, k_idx (full layers only),
    q_abs, kv, w_uv.  ``full`` gives each layer's kind (default: the pages'
    pattern).  Each layer keeps its own queries, cache and W_UV; only the
    selected positions are shared ([GLM 5.2 hermosaai] "MLA + DSA with
    IndexShare": the next layers reuse the selection instead of scoring
    again).  Returns (outs, idxs, scores) with idxs / scores holding an entry
    for every full layer (None for shared layers).
    """
    if full is None:
        full = layer_pattern(len(layers))
    if len(layers) and not full[0]:
        raise ValueError("the first layer of a stack must run its own indexer")
    outs, idxs, scores_all = [], [], []
    cur = None
    for l, L in enumerate(layers):
        if full[l]:
            sc = indexer_scores(L["q_idx"], L["w"], L["k_idx"], seq_start, q_seq, q_pos)
            cur = topk_select_rows(sc, q_pos, k)
            idxs.append(cur)
            scores_all.append(sc)
        else:
            idxs.append(None)
            scores_all.append(None)
        outs.append(sparse_mla(L["q_abs"], L["kv"], seq_start, q_seq, cur, L["w_uv"], scale))
    return outs, idxs, scores_all


# --------------------------------------------------------------------------
# MTP / speculative decode: one selection shared by several query tokens.
#
# [GLM-5.2 llm-atlas] config field index_share_for_mtp_iteration = true;
# [GLM 5.2 hermosaai] "78 layers, IndexShare pattern": one Multi-Token
# Prediction layer, tuned for a longer speculative accept length;
# [GLM-5.2 techniques map] "decoding strategy": speculative decoding and
# multi-token prediction.  The pages name the flag only.  Reading taken: in a
# speculative decode step a sequence brings several consecutive query tokens
# (the drafts being verified); the indexer and the top-k run once, for one
# selecting query of the group (normally the group's last token, whose causal
# set holds every other token's), and each token of the group attends over
# that selection restricted to its own causal set: selected positions past
# the token's own position are dropped, the rest keep their order.

def share_selection(sel_idx, sel_of, q_pos):
    """Per-token selection rows built from shared ones.

    sel_idx [n_sel, k]: the selecting queries' rows (positions, -1 padding).
    Token t uses row sel_of[t] and keeps its positions p with 0 <= p <=
    q_pos[t], in the row's order, followed by -1 padding.  Returns int64
    [n_q, k]."""
    sel_idx = np.asarray(sel_idx, dtype=np.int64)
    n_q, k = len(sel_of), sel_idx.shape[1]
    out = np.full((n_q, k), -1, dtype=np.int64)
    for t in range(n_q):
        row = sel_idx[int(sel_of[t])]
        keep = row[(row >= 0) & (row <= int(q_pos[t]))]
        out[t, :len(keep)] = keep
    return out


def layer_stack_mtp(layers, seq_start, q_seq, q_pos, sel_seq, sel_pos, sel_of, k=INDEX_TOPK, scale=1.0 / 16,
                    full=None):
    """:func:`layer_stack` with a selection shared inside groups of tokens.

    Full layers score and select for the selecting queries only (sequence
    sel_seq[s], position sel_pos[s]; their layer inputs q_idx and w have
    n_sel rows); token t then uses the selection of selecting query
    sel_of[t], restricted to its own causal set (:func:`share_selection`).
    Attention runs for every token with its own q_abs.  Returns (outs, idxs)
    with idxs holding the per-token rows of every full layer (None for shared
    layers)."""
    if full is None:
        full = layer_pattern(len(layers))
    if len(layers) and not full[0]:
        raise ValueError("the first layer of a stack must run its own indexer")
    outs, idxs = [], []
    cur = None
    for l, L in enumerate(layers):
        if full[l]:
            sc = indexer_scores(L["q_idx"], L["w"], L["k_idx"], seq_start, sel_seq, sel_pos)
            cur = share_selection(topk_select_rows(sc, sel_pos, k), sel_of, q_pos)
            idxs.append(cur)
        else:
            idxs.append(None)
        outs.append(sparse_mla(L["q_abs"], L["kv"], seq_start, q_seq, cur, L["w_uv"], scale))
    return outs, idxs


# --------------------------------------------------------------------------
# Cache write: the step before the path.  Each new token's kv_a_proj output
# (512 latent + 64 rope-key values) becomes its 576-wide cache row, and its
# indexer-key projection becomes its 128-wide indexer key.
#
# [GLM-5.2 techniques map] row "Multi-head latent attention": the latent goes
# through kv_a_layernorm, an RMSNorm over kv_lora_rank = 512 values, and the
# decoupled 64-dim key is rotated.  Row "QK normalization": the indexer key
# is the LayerNorm (k_norm) of the wk output.  Rows "Partial RoPE" and "YaRN
# RoPE scaling": rotary embedding of the 64-dim part, rope_type "default"
# (no scaling), rope_theta 8,000,000.  [GLM-5.2 llm-atlas] config fields:
# rms_norm_eps 1e-5, rope_interleave true, indexer_rope_interleave true.
#
# Readings where the pages are silent (each stated again in the design notes):
#   * RMSNorm is x / sqrt(mean(x^2) + eps) * gamma; LayerNorm is
#     (x - mean) / sqrt(var + eps) * weight + bias with the population
#     variance; both with eps = rms_norm_eps (the pages give none for k_norm).
#   * "Interleaved" RoPE rotates the adjacent pairs (2i, 2i + 1) in place by
#     the angle p * theta^(-2i / 64); the output keeps that layout.
#   * The indexer key is rotated on its last 64 dims (64..127) with the same
#     frequencies, the order the main attention uses for its nope/rope split.
#   * Everything is exact here (float64); the stored row is rounded once to
#     bfloat16.

ROPE_THETA = 8.0e6        # rope_parameters.rope_theta
RMS_NORM_EPS = 1e-5       # rms_norm_eps


def rms_norm(x, gamma, eps=RMS_NORM_EPS):
    """RMSNorm of each row of x (last axis), scaled by gamma."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gamma)


def layer_norm(x, weight, bias, eps=RMS_NORM_EPS):
    """LayerNorm of each row of x (last axis) with an affine weight and bias."""
    x = _f64(x)
    mean = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mean) ** 2, axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * _f64(weight) + _f64(bias)


def rope_interleaved(x, pos, theta=ROPE_THETA):
    """Rotate the adjacent pairs (2i, 2i + 1) of each row of x (shape [n, d])
    by pos[n] * theta^(-2i / d)."""
    x = _f64(x)
    d = x.shape[-1]
    inv_freq = np.power(float(theta), -np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = x0 * c - x1 * s
    out[:, 1::2] = x0 * s + x1 * c
    return out


def cache_rows_from_projection(kv_a, gamma, pos):
    """The 576-wide cache rows of n new tokens: RMSNorm(latent) * gamma, then
    the rotated 64-dim key; rounded to bfloat16.  kv_a: [n, 576]."""
    kv_a = _f64(kv_a)
    lat = rms_norm(kv_a[:, :KV_LORA_RANK], gamma)
    rot = rope_interleaved(kv_a[:, KV_LORA_RANK:], pos)
    return round_to_bf16(np.concatenate([lat, rot], axis=1))


def indexer_keys_from_projection(k_raw, ln_weight, ln_bias, pos):
    """The 128-wide indexer keys of n new tokens: LayerNorm, then the last 64
    dims rotated; rounded to bfloat16.  k_raw: [n, 128]."""
    k = layer_norm(k_raw, ln_weight, ln_bias)
    half = INDEX_HEAD_DIM - QK_ROPE_DIM
    k[:, half:] = rope_interleaved(k[:, half:], pos)
    return round_to_bf16(k)


# --------------------------------------------------------------------------
# Query side: the projections that produce the path's query inputs.
#
# [GLM-5.2 techniques map] row "Multi-head latent attention": the query goes
# through a q_lora_rank bottleneck; kv_b_proj maps the 512-wide latent to, per
# head, qk_nope_head_dim key rows and v_head_dim value rows.  Row "Partial
# RoPE": each head's query splits into a 192-dim part without rotation and a
# 64-dim rotated part, in that order.  [GLM-5.2 architectures] "Every
# architecture field": q_lora_rank 2,048, qk_nope 192, qk_rope 64; [GLM-5.2
# llm-atlas] qk_head_dim 256, rope_interleave, indexer_rope_interleave, and
# rope_theta 8e6 ([GLM-5.2 techniques map] row "YaRN RoPE scaling": default
# rope type).  Row "Indexer-selected sparse attention": 32 indexer heads of
# 128 against one shared key.
#
# Readings where the pages are silent (each stated again in the design notes):
#   * The input c_q is the q_lora activation as the attention receives it
#     (after its normalisation, which the pages do not print).
#   * q = q_b_proj(c_q) holds, per head, [192 nope ; 64 rope]; the rope part
#     turns with the cache key's convention (interleaved pairs, position p).
#   * Absorption: the key half of kv_b_proj for head h, W_UK[h] ([192, 512],
#     nope rows of the head), folds into the query: q_abs[h] =
#     [W_UK[h]^T q_nope[h] ; q_rope[h]], so q_abs[h] . row =
#     q_nope[h] . (W_UK[h] latent) + q_rope[h] . k_rope.
#   * The indexer query and the head weights are projections of the same
#     q_lora activation (the pages print the key's source only); the indexer
#     query turns dims 64..127 of each head, as the indexer key does.  No
#     extra scale on the weights (a positive factor leaves every selection
#     unchanged).
#   * Rounding as a bf16 model stores activations: each projection's output
#     is rounded to bf16 once, the rope part is turned from those bf16 values
#     and rounded again, the absorbed query is rounded once; the head weights
#     stay fp32.

Q_LORA_RANK = 2048        # q_lora_rank
QK_HEAD_DIM = QK_NOPE_DIM + QK_ROPE_DIM   # 256 = qk_head_dim


def _rope_heads(x, pos, first):
    """Turn dims first.. of every head of x [n, H, d] at the token positions."""
    x = _f64(x).copy()
    n, H, d = x.shape
    part = x[:, :, first:].reshape(n * H, d - first)
    x[:, :, first:] = rope_interleaved(part, np.repeat(np.asarray(pos), H)).reshape(n, H, d - first)
    return x


def q_project(c_q, w_qb, w_iq, w_iw, pos):
    """The query projections of n tokens.

    c_q  [n, 2048] q_lora activation; w_qb [64 * 256, 2048] (q_b_proj);
    w_iq [32 * 128, 2048] (indexer query); w_iw [32, 2048] (head weights);
    pos  [n] token positions.
    Returns q [n, 64, 256] (per head [192 nope ; 64 turned rope], bf16
    values), q_idx [n, 32, 128] (dims 64..127 turned, bf16 values) and
    w [n, 32] (float32 values)."""
    c_q = _f64(c_q)
    n = c_q.shape[0]
    q = round_to_bf16(c_q @ _f64(w_qb).T).reshape(n, N_HEADS, QK_HEAD_DIM)
    q = round_to_bf16(_rope_heads(q, pos, QK_NOPE_DIM))
    qi = round_to_bf16(c_q @ _f64(w_iq).T).reshape(n, INDEX_N_HEADS, INDEX_HEAD_DIM)
    qi = round_to_bf16(_rope_heads(qi, pos, INDEX_HEAD_DIM - QK_ROPE_DIM))
    w = (c_q @ _f64(w_iw).T).astype(np.float32).astype(np.float64)
    return q, qi, w


def q_absorb(q, w_uk):
    """Fold the key half of kv_b_proj into the query.

    q [n, 64, 256] from :func:`q_project`; w_uk [64, 192, 512], the nope rows
    of kv_b_proj for each head.  Returns q_abs [n, 64, 576] (bf16 values):
    [W_UK[h]^T q_nope[h] ; q_rope[h]] per head."""
    q, w_uk = _f64(q), _f64(w_uk)
    n = q.shape[0]
    out = np.empty((n, N_HEADS, ROW_DIM))
    for h in range(N_HEADS):
        out[:, h, :KV_LORA_RANK] = round_to_bf16(q[:, h, :QK_NOPE_DIM] @ w_uk[h])
        out[:, h, KV_LORA_RANK:] = q[:, h, QK_NOPE_DIM:]
    return out


def projection_error_bound(a, b):
    """|fp32 sum - exact| bound for each entry of a @ b.T summed in fp32 in
    any order: gamma_K * sum_k |a_k b_k| (Higham, ch. 3), K = a.shape[-1]."""
    K = a.shape[-1]
    u = 2.0 ** -24
    g = (K + 1) * u / (1 - (K + 1) * u)
    return g * (np.abs(_f64(a)) @ np.abs(_f64(b)).T)


# --------------------------------------------------------------------------
# FP8 caches.
#
# [GLM-5.2 techniques map] "inference quantization": FP8 inference;
# [GLM-5.2 llm-atlas] "Faits clés": precision fp8.  The pages name FP8 only.
# Readings taken (each stated again in the design notes):
#   * The format is OCP 8-bit E4M3 ("fn"): 1 sign bit, 4 exponent bits (bias
#     7), 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; the
#     largest finite magnitude is 448 (code 0x7E); 0x7F and 0xFF are NaN and
#     never produced.
#   * Each cache row (a 576-wide latent + rope row, or a 128-wide indexer key)
#     is stored as codes with one fp32 scale: scale = amax / 448 computed in
#     fp32 (1 for an all-zero row); code_i = the E4M3 value nearest to
#     x_i / scale (the division in fp32), ties to the even code, magnitudes
#     above 448 saturating to 448.  The stored row means scale * value(code).
#   * What gets quantized is the bf16 row the cache write produces.
#   * The queries stay bf16; the path computes on the exactly dequantized rows,
#     so the indexer, top-k and attention oracles above apply unchanged to
#     dequantize_rows_fp8's output.

E4M3_MAX = 448.0


def e4m3_value(code):
    """The value of an E4M3 code (0..255), from the format's definition."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)])


def e4m3_encode(y):
    """Nearest E4M3 code of each value (float64 array), ties to the even code,
    saturating at +-448.  Brute force over the 127 finite magnitudes."""
    y = np.asarray(y, dtype=np.float64)
    mags = E4M3_TABLE[:127]                       # codes 0x00..0x7E, increasing
    a = np.minimum(np.abs(y), E4M3_MAX)
    d = np.abs(a[..., None] - mags)               # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                              # one or two nearest codes
    codes = np.arange(127)
    even = cand & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    neg = np.signbit(y) & (pick > 0)              # -0 encodes as 0x00
    return (pick | (neg.astype(np.int64) << 7)).astype(np.uint8)


def quantize_rows_fp8(x):
    """Codes (uint8 [n, d]) and scales (float32-valued [n]) of rows x [n, d]
    (bf16 values)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[:, None]).astype(np.float32)
    return e4m3_encode(y.astype(np.float64)), scale.astype(np.float64)


def dequantize_rows_fp8(codes, scales):
    """The rows the path computes on: scale * value(code), exact in float64."""
    return np.asarray(scales, dtype=np.float64)[:, None] * E4M3_TABLE[np.asarray(codes, dtype=np.int64)]

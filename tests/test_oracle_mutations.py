"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that at least one pin catches each of them.  This shows the pins constrain
every step of the oracle, not only its happy path."""
import inspect
import types

import pytest

from oracle import ref
from tests import oracle_pins

SOURCE = inspect.getsource(ref)

# (name, original text, planted mistake)
MUTATIONS = [
    ("relu_after_weight", "out[t, :n_t] = w[t] @ np.maximum(dots, 0.0)",
     "out[t, :n_t] = np.maximum(w[t][:, None] * dots, 0.0).sum(axis=0)"),
    ("no_relu", "out[t, :n_t] = w[t] @ np.maximum(dots, 0.0)", "out[t, :n_t] = w[t] @ dots"),
    ("causal_excludes_diagonal", "        n_t = int(q_pos[t]) + 1\n        base", "        n_t = int(q_pos[t])\n        base"),
    ("head_weights_reversed", "out[t, :n_t] = w[t] @ np.maximum(dots, 0.0)",
     "out[t, :n_t] = w[t][::-1] @ np.maximum(dots, 0.0)"),
    ("ignores_sequence_offset", "        base = int(seq_start[q_seq[t]])\n        keys", "        base = 0\n        keys"),
    ("key_dims_reversed", "dots = q_idx[t] @ keys.T ", "dots = q_idx[t] @ keys[:, ::-1].T "),
    ("query_of_wrong_token", "dots = q_idx[t] @ keys.T ", "dots = q_idx[(t + 1) % n_q] @ keys.T "),
    ("ties_to_higher_position", "order = np.lexsort((positions, -row))", "order = np.lexsort((-positions, -row))"),
    ("topk_smallest", "order = np.lexsort((positions, -row))", "order = np.lexsort((positions, row))"),
    ("topk_ignores_causal_bound", "row = _f64(scores_row)[:n_t]", "row = _f64(scores_row)[:n_t + 1]"),
    ("topk_off_by_one_k", "k_eff = min(int(k), n_t)", "k_eff = min(int(k) - 1, n_t)"),
    ("mla_no_scale", "z = scale * (q_abs[t] @ rows.T)  ", "z = (q_abs[t] @ rows.T)  "),
    ("mla_value_slice_wrong", "obar = p @ rows[:, :lat] ", "obar = p @ rows[:, -lat:] "),
    ("mla_logits_drop_rope", "z = scale * (q_abs[t] @ rows.T)  ", "z = scale * (q_abs[t][:, :lat] @ rows[:, :lat].T)  "),
    ("mla_head_mismatch", "out[t, h] = w_uv[h] @ obar[h]", "out[t, h] = w_uv[n_h - 1 - h] @ obar[h]"),
    ("mla_softmax_over_heads", "m = z.max(axis=1, keepdims=True)\n        e = np.exp(z - m)\n        lsum = e.sum(axis=1, keepdims=True)",
     "m = z.max(axis=0, keepdims=True)\n        e = np.exp(z - m)\n        lsum = e.sum(axis=0, keepdims=True)"),
    ("mla_padding_not_skipped", "sel = idx[t][idx[t] >= 0]", "sel = idx[t]"),
    ("mla_sequence_offset_ignored", "rows = _f64(kv[int(seq_start[q_seq[t]]) + sel])", "rows = _f64(kv[sel])"),
    ("mla_no_normalisation", "p = e / lsum", "p = e"),
    ("bound_drops_slice_rounding", "d_obar = d_obar + lam * ub * np.sqrt((a_sl ** 2).sum(axis=0))",
     "d_obar = d_obar + 0.0 * ub * np.sqrt((a_sl ** 2).sum(axis=0))"),
    ("pattern_offset_wrong", "== INDEX_TOPK_FREQ - 1", "== 0"),
    ("pattern_no_prefix", "if layer < INDEX_SKIP_TOPK_OFFSET:\n        return True", "if layer < 1:\n        return True"),
    ("stack_shares_wrong_layer", "            cur = topk_select_rows(sc, q_pos, k)", "            cur = topk_select_rows(sc, q_pos, k - 1)"),
    ("bf16_truncates", "rounded = (bits + 0x7FFF + lsb) >> 16", "rounded = bits >> 16"),
    ("bf16_ties_away", "rounded = (bits + 0x7FFF + lsb) >> 16", "rounded = (bits + 0x8000) >> 16"),
    ("bound_drops_dot_term", "return err_dot + err_sum", "return err_sum"),
    ("rope_turns_backwards", "out[:, 1::2] = x0 * s + x1 * c", "out[:, 1::2] = -x0 * s + x1 * c"),
    ("rope_half_split_layout", "x0, x1 = x[:, 0::2], x[:, 1::2]", "x0, x1 = x[:, : d // 2], x[:, d // 2:]"),
    ("rope_wrong_theta", "ROPE_THETA = 8.0e6", "ROPE_THETA = 1.0e4"),
    ("rope_exponent_over_half_dim", "-np.arange(0, d, 2, dtype=np.float64) / d)", "-np.arange(0, d, 2, dtype=np.float64) / (d // 2))"),
    ("rms_without_eps", "return x / np.sqrt(ms + eps) * _f64(gamma)", "return x / np.sqrt(ms) * _f64(gamma)"),
    ("rms_sum_not_mean", "ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    ("ln_sample_variance", "var = np.mean((x - mean) ** 2, axis=-1, keepdims=True)",
     "var = np.sum((x - mean) ** 2, axis=-1, keepdims=True) / (x.shape[-1] - 1)"),
    ("ln_drops_bias", "* _f64(weight) + _f64(bias)", "* _f64(weight)"),
    ("indexer_key_turns_first_half", "k[:, half:] = rope_interleaved(k[:, half:], pos)", "k[:, :half] = rope_interleaved(k[:, :half], pos)"),
    ("mtp_cut_excludes_own_position", "keep = row[(row >= 0) & (row <= int(q_pos[t]))]",
     "keep = row[(row >= 0) & (row < int(q_pos[t]))]"),
    ("mtp_no_causal_cut", "keep = row[(row >= 0) & (row <= int(q_pos[t]))]", "keep = row[row >= 0]"),
    ("mtp_first_row_for_all", "row = sel_idx[int(sel_of[t])]", "row = sel_idx[0]"),
    ("mtp_selects_at_token_positions", "cur = share_selection(topk_select_rows(sc, sel_pos, k), sel_of, q_pos)",
     "cur = share_selection(topk_select_rows(sc, np.minimum(sel_pos, min(q_pos)), k), sel_of, q_pos)"),
    ("q_rope_on_first_dims", "q = round_to_bf16(_rope_heads(q, pos, QK_NOPE_DIM))",
     "q = round_to_bf16(_rope_heads(q[:, :, ::-1], pos, QK_NOPE_DIM)[:, :, ::-1])"),
    ("q_not_rounded_before_rope", "q = round_to_bf16(c_q @ _f64(w_qb).T).reshape(n, N_HEADS, QK_HEAD_DIM)",
     "q = (c_q @ _f64(w_qb).T).reshape(n, N_HEADS, QK_HEAD_DIM)"),
    ("q_turned_backwards", "x[:, :, first:] = rope_interleaved(part, np.repeat(np.asarray(pos), H))",
     "x[:, :, first:] = rope_interleaved(part, -np.repeat(np.asarray(pos), H))"),
    ("indexer_q_turns_first_half", "qi = round_to_bf16(_rope_heads(qi, pos, INDEX_HEAD_DIM - QK_ROPE_DIM))",
     "qi = round_to_bf16(_rope_heads(qi, pos, 0))"),
    ("absorb_one_head_for_all", "out[:, h, :KV_LORA_RANK] = round_to_bf16(q[:, h, :QK_NOPE_DIM] @ w_uk[h])",
     "out[:, h, :KV_LORA_RANK] = round_to_bf16(q[:, h, :QK_NOPE_DIM] @ w_uk[0])"),
    ("absorb_drops_rope", "out[:, h, KV_LORA_RANK:] = q[:, h, QK_NOPE_DIM:]", "out[:, h, KV_LORA_RANK:] = 0.0"),
    ("head_weights_wrong_matrix", "w = (c_q @ _f64(w_iw).T).astype(np.float32).astype(np.float64)",
     "w = (c_q @ _f64(w_iw).T)[:, ::-1].astype(np.float32).astype(np.float64)"),
    ("projection_bound_too_small", "g = (K + 1) * u / (1 - (K + 1) * u)", "g = 8 * u"),
    ("e4m3_wrong_bias", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    ("e4m3_subnormal_scale", "return sign * m * 2.0 ** -9", "return sign * m * 2.0 ** -10"),
    ("e4m3_ties_to_lower", "pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))",
     "pick = np.argmax(cand, axis=-1)"),
    ("e4m3_drops_sign", "return (pick | (neg.astype(np.int64) << 7)).astype(np.uint8)", "return pick.astype(np.uint8)"),
    ("fp8_scale_over_max_code", "amax / np.float32(E4M3_MAX)", "amax / np.float32(240.0)"),
    ("fp8_scale_not_applied", "return np.asarray(scales, dtype=np.float64)[:, None] * E4M3_TABLE",
     "return 1.0 * E4M3_TABLE"),
    ("cache_row_latent_not_normalised", "lat = rms_norm(kv_a[:, :KV_LORA_RANK], gamma)", "lat = kv_a[:, :KV_LORA_RANK] * _f64(gamma)"),
]


def mutated_module(orig, new):
    assert SOURCE.count(orig) >= 1, f"mutation anchor not found: {orig!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SOURCE.replace(orig, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_some_pin_catches(name, orig, new):
    mod = mutated_module(orig, new)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"


def test_unmutated_source_passes():
    mod = mutated_module("import numpy as np", "import numpy as np")
    for check in oracle_pins.ALL_CHECKS:
        check(mod)

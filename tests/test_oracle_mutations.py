"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
at least one pin catches each of them: evidence that the pins constrain every
part of the oracle, not just the parts that happened to be exercised."""
import inspect
import types

import pytest

from oracle import dflash_oracle
from tests.oracle_pins import ALL_PINS

SRC = inspect.getsource(dflash_oracle)

# (name, text in the oracle, replacement)
MUTANTS = [
    ("bf16_truncates", "np.rint(m * 256.0)", "np.trunc(m * 256.0)"),
    ("bf16_ties_away", "np.rint(m * 256.0)", "np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5)"),
    ("rms_no_eps", "np.sqrt(ms + eps)", "np.sqrt(ms)"),
    ("rms_sum_not_mean", "ms = np.mean(x * x, axis=-1, keepdims=True)",
     "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    ("rms_no_gain", "return np.asarray(g, dtype=F64) * (x / np.sqrt(ms + eps))",
     "return (x / np.sqrt(ms + eps))"),
    ("silu_is_sigmoid", "return x / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(-x))"),
    ("fuse_reversed_sources", "for h in h_tgt], axis=1)", "for h in h_tgt[::-1]], axis=1)"),
    ("fuse_no_norm", "return store(rmsnorm(u, g_c, eps), storage)", "return store(u, storage)"),
    ("inject_k_v_swapped", "_, wk, wv = split_qkv(w_qkv, Hq, Hkv, d)",
     "_, wv, wk = split_qkv(w_qkv, Hq, Hkv, d)"),
    ("inject_uses_wq", "_, wk, wv = split_qkv(w_qkv, Hq, Hkv, d)",
     "wk, _, wv = split_qkv(w_qkv, Hq, Hkv, d)"),
    ("attn_head_map_mod", "j = h // G", "j = h % Hkv"),
    ("attn_no_scale", "/ np.sqrt(d)          # [R, n]", "# [R, n]"),
    ("attn_causal", "s = s - np.max(s, axis=1, keepdims=True)",
     "s = s + np.triu(np.full(s.shape, -1e30), 1 + s.shape[1] - s.shape[0]); "
     "s = s - np.max(s, axis=1, keepdims=True)"),
    ("attn_no_normalise", "p = p / np.sum(p, axis=1, keepdims=True)", "p = p"),
    ("draft_block_kv_unrounded",
     "kb = store(qkv[..., Hq * d:(Hq + Hkv) * d], storage)", "kb = (qkv[..., Hq * d:(Hq + Hkv) * d])"),
    ("draft_context_ignored",
     "keys = np.concatenate([cache.k[l][b], kb[b]], axis=0)\n"
     "            vals = np.concatenate([cache.v[l][b], vb[b]], axis=0)",
     "keys = kb[b]\n            vals = vb[b]"),
    ("draft_no_attn_residual", "h = h + o @ np.asarray(w[\"w_o\"], dtype=F64).T",
     "h = o @ np.asarray(w[\"w_o\"], dtype=F64).T"),
    ("draft_gains_swapped", "a = rmsnorm(h, w[\"g_attn\"], eps)", "a = rmsnorm(h, w[\"g_ffn\"], eps)"),
    ("draft_gate_up_swapped", "s = silu(gu[..., :F]) * gu[..., F:]", "s = silu(gu[..., F:]) * gu[..., :F]"),
    ("draft_no_final_norm", "return rmsnorm(h, g_final, eps), block_kv", "return h, block_kv"),
    ("draft_ffn_on_unnormed", "gu = f @ np.asarray(w[\"w_gateup\"], dtype=F64).T",
     "gu = h @ np.asarray(w[\"w_gateup\"], dtype=F64).T"),
    ("lm_includes_anchor", "z = np.asarray(h_final, dtype=F64)[:, 1:, :]",
     "z = np.asarray(h_final, dtype=F64)[:, :-1, :]"),
    ("argmax_last_tie", "draft = np.argmax(logits, axis=-1).astype(np.int32)",
     "draft = (logits.shape[-1] - 1 - np.argmax(logits[..., ::-1], axis=-1)).astype(np.int32)"),
    ("accept_no_bonus", "tau[b] = m + 1", "tau[b] = m"),
    ("accept_counts_all_matches", "while m < n and int(draft[b, m]) == int(target[b, m]):\n            m += 1",
     "m = int(np.sum(draft[b] == target[b, :n]))"),
    ("accept_next_is_draft", "nxt[b] = target[b, m]", "nxt[b] = draft[b, min(m, n - 1)]"),
    ("gumbel_sign", "key = np.asarray(logw, dtype=F64) - np.log(-np.log(",
     "key = np.asarray(logw, dtype=F64) + np.log(-np.log("),
    ("gumbel_plain_uniform", "key = np.asarray(logw, dtype=F64) - np.log(-np.log(np.asarray(u, dtype=F64)))",
     "key = np.asarray(logw, dtype=F64) + np.asarray(u, dtype=F64)"),
    ("gumbel_last_tie", "idx = np.argmax(key, axis=-1)",
     "idx = key.shape[-1] - 1 - np.argmax(key[..., ::-1], axis=-1)"),
    ("log_softmax_no_temperature", "x = np.asarray(logits, dtype=F64) / float(T)\n    mx = np.max(x, axis=-1, keepdims=True)",
     "x = np.asarray(logits, dtype=F64)\n    mx = np.max(x, axis=-1, keepdims=True)"),
    ("lse_drops_max", "return mx + np.log(np.sum(np.exp(x - mx[..., None]), axis=-1))",
     "return np.log(np.sum(np.exp(x - mx[..., None]), axis=-1))"),
    ("sample_no_temperature", "draft, gap = gumbel_pick(z / float(T), u)", "draft, gap = gumbel_pick(z, u)"),
    ("sample_includes_anchor", "z = np.asarray(h_final, dtype=F64)[:, 1:, :] @ np.asarray(lm_head",
     "z = np.asarray(h_final, dtype=F64)[:, :-1, :] @ np.asarray(lm_head"),
    ("accept_ratio_inverted", "log_ratio = lp[:, :n][bi, ji, draft] - lq[bi, ji, draft]",
     "log_ratio = lq[bi, ji, draft] - lp[:, :n][bi, ji, draft]"),
    ("accept_ratio_next_row", "log_ratio = lp[:, :n][bi, ji, draft] - lq[bi, ji, draft]",
     "log_ratio = lp[:, 1:][bi, ji, draft] - lq[bi, ji, draft]"),
    ("accept_always_capped_half", "accepted = np.asarray(accept_u, dtype=F64) < np.exp(log_ratio)",
     "accepted = np.asarray(accept_u, dtype=F64) < np.minimum(0.5, np.exp(log_ratio))"),
    ("resid_from_p", "logw = lp[b, m] if empty[b] else np.log(r)", "logw = lp[b, m]"),
    ("resid_q_minus_p", "r = np.maximum(0.0, np.exp(lp[b, m]) - np.exp(lq[b, m]))",
     "r = np.maximum(0.0, np.exp(lq[b, m]) - np.exp(lp[b, m]))"),
    ("bonus_from_draft_row", "logw = lp[b, n]", "logw = lq[b, n - 1]"),
    ("sample_tau_no_bonus", "m_all[b], tau[b], nxt[b], key_gap[b] = m, m + 1, tok, gap",
     "m_all[b], tau[b], nxt[b], key_gap[b] = m, max(m, 1), tok, gap"),
    ("ragged_wrong_sequence_cache", "hf, kv = draft_forward(dims, layers, g_final, cache.sequence(b), int(g),",
     "hf, kv = draft_forward(dims, layers, g_final, cache.sequence(0), int(g),"),
    ("ragged_uniform_gamma", "hf, kv = draft_forward(dims, layers, g_final, cache.sequence(b), int(g),",
     "hf, kv = draft_forward(dims, layers, g_final, cache.sequence(b), int(gammas[0]),"),
    ("ragged_accept_shifted_targets", "res = [accept(np.asarray(d)[None], np.asarray(t)[None]) for d, t in zip(drafts, targets)]",
     "res = [accept(np.asarray(d)[None], np.asarray(t)[None][:, ::-1]) for d, t in zip(drafts, targets)]"),
    ("blocks_see_anchor_feature", "cache.prefix(int(sq), int(a)), gamma, embed=embed,",
     "cache.prefix(int(sq), int(a) + 1), gamma, embed=embed,"),
    ("blocks_see_whole_context", "cache.prefix(int(sq), int(a)), gamma, embed=embed,",
     "cache.sequence(int(sq)), gamma, embed=embed,"),
    ("blocks_wrong_sequence", "cache.prefix(int(sq), int(a)), gamma, embed=embed,",
     "cache.prefix(0, int(a)), gamma, embed=embed,"),
    ("sample_counts_all_accepts", "while m < n and accepted[b, m]:\n            m += 1",
     "m = int(np.sum(accepted[b]))"),
    ("taps_from_first_layer", "first, last = 1, L_t - 3", "first, last = 0, L_t - 3"),
    ("taps_to_second_last", "first, last = 1, L_t - 3", "first, last = 1, L_t - 2"),
    ("taps_round_down", "(n - 1) + 0.5))", "(n - 1)))"),
    ("target_not_causal", "seen = n_ctx + i + 1", "seen = k.shape[0]"),
    ("target_skips_own_row", "seen = n_ctx + i + 1", "seen = max(n_ctx + i, 1)"),
    ("target_tap_normed", "kept[l] = store(x, tap_storage)",
     "kept[l] = store(rmsnorm(x, w[\"g_ffn\"], eps), tap_storage)"),
    ("target_tap_before_ffn", "x = x + (silu(up[..., :F]) * up[..., F:]) @ np.asarray(w[\"w_down\"], dtype=F64).T\n"
     "        if l in taps:\n            kept[l] = store(x, tap_storage)",
     "if l in taps:\n            kept[l] = store(x, tap_storage)\n"
     "        x = x + (silu(up[..., :F]) * up[..., F:]) @ np.asarray(w[\"w_down\"], dtype=F64).T"),
    ("target_no_final_norm", "logits = rmsnorm(x, g_final, eps) @", "logits = x @"),
    ("target_context_keys_zeroed", "np.concatenate([cache.k[l][b], kt[b]], axis=0)",
     "np.concatenate([0 * cache.k[l][b], kt[b]], axis=0)"),
]


def _mutant_module(old, new):
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = SRC.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant_module(old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} survived every pin"

"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case takes one oracle function's own source, makes one plausible
mistake in it (a sign, an index, a dropped term, a widened or transposed
mask, a wrong constant), swaps the mutant in for the duration of the test,
and runs the pins that should notice: at least one must fail with an
assertion.  This shows the pins are not restatements of the code they pin."""

import importlib
import inspect
import textwrap

import pytest

import oracle
import test_oracle_e2etv as te
import test_oracle_gdn as tg
import test_oracle_lmhead as tl
import test_oracle_prefill as tp
import test_oracle_qsa as tq
import test_oracle_tree_attention as tt

# (oracle module, function, text in its source, replacement, pins)
CASES = {
    "overlap takes the max": (
        "oracle.e2etv", "overlap", "np.minimum(np.exp(lq), np.exp(lp))",
        "np.maximum(np.exp(lq), np.exp(lp))",
        [te.test_eq13_worked_example, te.test_appC2_first_overlap]),
    "prefix product reads the parent's overlap": (
        "oracle.e2etv", "prefix_products", "(1.0 if p < 0 else P[r, p])",
        "(1.0 if p < 0 else alpha[r, p])",
        [lambda: te.test_constant_alpha_chain_closed_form(0.7, 7)]),
    "suffix sum drops the child's overlap": (
        "oracle.e2etv", "suffix_sums", "S[r, p] += alpha[r, j] * S[r, j]", "S[r, p] += S[r, j]",
        [te.test_division_free_equals_descendant_sum]),
    "log-sum-exp drops its shift": (
        "oracle.e2etv", "logsumexp", "return m + np.log(", "return np.log(",
        [te.test_eq13_worked_example]),
    "gradient indicator reversed": (
        "oracle.e2etv", "e2etv", "ind = (lq < lp).astype(np.float64)",
        "ind = (lq > lp).astype(np.float64)", [te.test_gradient_finite_difference]),
    "gradient adds G instead of subtracting": (
        "oracle.e2etv", "e2etv", "q * (ind - Gf[r0:r1, None])", "q * (ind + Gf[r0:r1, None])",
        [te.test_gradient_finite_difference, te.test_grad_scale_and_row_sums]),
    "gradient drops the parent's prefix product": (
        "oracle.e2etv", "e2etv", "c = -grad_scale * Ppar * S / count", "c = -grad_scale * S / count",
        [te.test_gradient_finite_difference, te.test_division_free_equals_descendant_sum]),
    "loss divides by the wrong count": (
        "oracle.e2etv", "e2etv", '"loss": 1.0 - numer / count', '"loss": 1.0 - numer / (count + 1.0)',
        [lambda: te.test_constant_alpha_chain_closed_form(0.3, 2)]),
    "rotation sign flipped": (
        "oracle.rope", "rope", "x1 * c - x2 * s", "x1 * c + x2 * s",
        [tt.test_rope_pair_is_complex_rotation, tt.test_rope_hand_values]),
    "rotation frequencies halved": (
        "oracle.rope", "rope_angles", "-2.0 * i / D", "-1.0 * i / D",
        [tt.test_rope_pair_is_complex_rotation, tt.test_rope_hand_values]),
    "anchor token masked": (
        "oracle.tree_attention", "branch_mask", "m[j, : int(anchor) + 1] = True",
        "m[j, : int(anchor)] = True", [tt.test_fig3_toy_tree]),
    "every earlier node visible (siblings leak)": (
        "oracle.tree_attention", "branch_mask", "for k in walk_ancestors(parent, j):",
        "for k in range(j + 1):", [tt.test_each_row_is_plain_attention_over_its_history]),
    "scores scaled by 1/D": (
        "oracle.tree_attention", "tree_attention_branch", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D",
        [tt.test_each_row_is_plain_attention_over_its_history]),
    "query heads dealt to kv heads round robin": (
        "oracle.tree_attention", "tree_attention_branch", "for h in range(g * G, (g + 1) * G):",
        "for h in range(g, Hq, Hkv):", [tt.test_gqa_head_mapping]),
    "prefill sees one token ahead": (
        "oracle.prefill", "trunk_prefill", "np.arange(L)[None, :] <= todo[:, None]",
        "np.arange(L)[None, :] <= todo[:, None] + 1",
        [lambda: tp.test_prefill_is_library_causal_attention(0, 37, 4, 2, 16)]),
    "prefill kv head transposed": (
        "oracle.prefill", "trunk_prefill", "g = h // G", "g = h % Hkv",
        [lambda: tp.test_prefill_is_library_causal_attention(0, 37, 4, 2, 16)]),
    "delta rule adds the old association": (
        "oracle.gdn", "gated_delta_update", "(S - float(beta) * np.outer(Sk, k))",
        "(S + float(beta) * np.outer(Sk, k))",
        [tg.test_update_is_the_linear_map_on_the_flattened_state, tg.test_full_strength_write_reads_back_the_value]),
    "gate applied after the write": (
        "oracle.gdn", "gated_delta_update",
        "float(alpha) * (S - float(beta) * np.outer(Sk, k)) + float(beta) * np.outer(v, k)",
        "float(alpha) * (S - float(beta) * np.outer(Sk, k) + float(beta) * np.outer(v, k))",
        [tg.test_update_is_the_linear_map_on_the_flattened_state, tg.test_first_token_from_zero_state]),
    "replay starts one token late": (
        "oracle.gdn", "replay_span", "return m - 1, m * C", "return m - 1, m * C + 1",
        [lambda: tg.test_replayed_anchor_state_equals_the_full_history(9), tg.test_figure5_replay_spans]),
    "checkpoint taken a token early": (
        "oracle.gdn", "trunk_checkpoints", "if (t + 1) % C == 0:", "if (t + 2) % C == 0 and t + 2 <= L:",
        [tg.test_checkpoints_are_states_after_every_C_tokens]),
    "node output reads its parent's state": (
        "oracle.gdn", "gdn_branch", "out[j, h] = gdn_read(Sj, q[j][h])", "out[j, h] = gdn_read(Sp, q[j][h])",
        [lambda: tg.test_branch_equals_full_recomputation_of_its_history(8)]),
    "branch nodes chained in index order": (
        "oracle.gdn", "gdn_branch", "Sp = Sa if parent[j] < 0 else states[int(parent[j])]",
        "Sp = Sa if j == 0 else states[j - 1]",
        [tg.test_sibling_subtrees_do_not_see_each_other]),
    "conv window walks node indices, not parents": (
        "oracle.gdn", "conv_history", "x = int(parent[x])", "x = x - 1",
        [tg.test_fork_history_follows_the_parent_map, tg.test_conv_ignores_nodes_outside_the_window]),
    "conv trunk history starts a token early": (
        "oracle.gdn", "conv_history", "s = int(a)\n", "s = int(a) - 1\n",
        [lambda: tg.test_chain_conv_is_the_causal_convolution_of_its_history(4, 37)]),
    "conv activation sign flipped": (
        "oracle.gdn", "branch_conv", "y = z / (1.0 + np.exp(-z))", "y = z / (1.0 + np.exp(z))",
        [tg.test_width_one_is_silu_of_the_scaled_input]),
    "conv weights applied newest-last": (
        "oracle.gdn", "branch_conv", "z += w[:, i] *", "z += w[:, K - 1 - i] *",
        [lambda: tg.test_chain_conv_is_the_causal_convolution_of_its_history(3, 5)]),
    "score row of the node itself": (
        "oracle.rows", "score_row_source", 'else ("node", p)', 'else ("node", int(j))',
        [tt.test_fig3_toy_tree]),
    "boundary group filled with reference tokens after the anchor": (
        "oracle.qsa", "branch_group_keys", "if q > anchor:", "if q > anchor + GROUP:",
        [lambda: tq.test_branch_rows_equal_plain_sequence(1),
         lambda: tq.test_reference_tokens_after_the_anchor_do_not_leak(0)]),
    "incomplete group is a candidate": (
        "oracle.qsa", "qsa_branch_select", "G = (p + 1) // GROUP", "G = (p + GROUP) // GROUP",
        [lambda: tq.test_branch_rows_equal_plain_sequence(2)]),
    "query read unrotated": (
        "oracle.qsa", "qsa_branch_select", "s = keys @ rnd(rope(y[j], p, base))", "s = keys @ rnd(y[j])",
        [lambda: tq.test_branch_rows_equal_plain_sequence(4)]),
    "branch group rotated at its last token": (
        "oracle.qsa", "branch_group_keys", "gamma, p - (GROUP - 1), base, eps)",
        "gamma, p, base, eps)", [tq.test_siblings_share_keys_before_the_fork_only]),
    "boundary group shifted one trunk token": (
        "oracle.qsa", "branch_group_keys", "toks.append(trunk_raw[q])", "toks.append(trunk_raw[q - 1])",
        [tq.test_siblings_share_keys_before_the_fork_only]),
    "RMSNorm by the sum of squares": (
        "oracle.qsa", "rms_norm", "np.mean(u * u, axis=-1, keepdims=True)",
        "np.sum(u * u, axis=-1, keepdims=True)", [tq.test_hand_values_two_dims]),
    "top-k in score order": (
        "oracle.qsa", "select_topk", "return np.sort(order[:k])", "return order[:k]",
        [lambda: tq.test_topk_matches_sorting_rule(3)]),
    "head applied transposed": (
        "oracle.lmhead", "lmhead_logits", "@ np.asarray(W, np.float64).T", "@ np.asarray(W, np.float64).T[::-1]",
        [tl.test_logits_are_the_linear_map, tl.test_identity_head_is_e2etv_on_the_hidden_states]),
    "target rows not gathered": (
        "oracle.lmhead", "lmhead_e2etv", "ht = np.asarray(h_target, np.float64)[np.asarray(target_row).reshape(-1)]",
        "ht = np.asarray(h_target, np.float64)[: R * Wn]", [tl.test_siblings_read_their_parents_row]),
    "bf16 rounding ties away from even": (
        "oracle.qsa", "round_bf16", "b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000",
        "b = (b + 0x8000) & 0xFFFF0000", [tq.test_round_bf16_ties_to_even]),
}


def _mutant(mod, name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(mod, name)))
    assert src.count(old) == 1, f"{name}: the planted text must occur once"
    ns = dict(vars(mod))
    exec(compile(src.replace(old, new), f"<planted {name}>", "exec"), ns)
    return ns[name]


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_mistake_is_caught(case, monkeypatch):
    modname, name, old, new, pins = CASES[case]
    mod = importlib.import_module(modname)
    orig = getattr(mod, name)
    bad = _mutant(mod, name, old, new)
    monkeypatch.setattr(mod, name, bad)
    if getattr(oracle, name, None) is orig:
        monkeypatch.setattr(oracle, name, bad)
    caught = []
    for pin in pins:
        try:
            pin()
        except AssertionError as e:
            caught.append(str(e)[:80])
    assert caught, f"no pin caught: {case}"


def test_unplanted_pins_pass():
    """The same pins pass on the oracle as written (so a catch above is the
    planted mistake's doing)."""
    for case in CASES.values():
        for pin in case[4]:
            pin()

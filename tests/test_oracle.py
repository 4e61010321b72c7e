"""The CPU oracle against its pins, plus planted-mistake checks on copies of it.

Runs on the CPU only (no GPU marker).
"""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import attn_ref
from tests import oracle_pins

PINS = dict(oracle_pins.ALL_PINS)


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    PINS[name](oracle)


def test_block_rows_match_whole_rows():
    """Splitting the query rows into blocks only splits the sums over queries."""
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((2, 45, 16))
    v, do = rng.standard_normal((2, 45, 8))
    for causal in (True, False):
        a = attn_ref.head_backward(q, k, v, do, 0.3, causal, None)
        b = attn_ref.head_backward(q, k, v, do, 0.3, causal, 7)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_selected_heads_match_full_run():
    rng = np.random.default_rng(4)
    q, k, v, do = rng.standard_normal((4, 2, 9, 3, 8))
    full = attn_ref.attn_ref_bwd(q, k, v, do, True)
    part = attn_ref.attn_ref_heads(q, k, v, do, True, heads=[(0, 1), (1, 2)])
    assert sorted(part) == [(0, 1), (1, 2)]
    for (b, h), r in part.items():
        for name in ("dq", "dk", "dv", "o"):
            np.testing.assert_array_equal(r[name], full[name][b, :, h])
        np.testing.assert_array_equal(r["lse"], full["lse"][b, h])


# ---------------------------------------------------------------------------------
# Planted mistakes: each is a one-place edit of the oracle's source text, built into
# a fresh module.  Every one of them must make at least one pin fail.
# ---------------------------------------------------------------------------------
MUTANTS = {
    "drop_D_term": ("dS = P * (dP - Dr[:, None])", "dS = P * dP"),
    "dS_sign": ("dS = P * (dP - Dr[:, None])", "dS = P * (Dr[:, None] - dP)"),
    "dV_untransposed": ("dV[:nk] += Pk.T @ do[r0:r1]", "dV[:nk] += Pk @ do[r0:r1]"),
    "dQ_no_scale": ("dQ[r0:r1] = scale * (dS @ k[:nk])", "dQ[r0:r1] = (dS @ k[:nk])"),
    "dK_no_scale": ("dK[:nk] += scale * (dS.T @ q[r0:r1])", "dK[:nk] += (dS.T @ q[r0:r1])"),
    "dK_uses_k": ("dK[:nk] += scale * (dS.T @ q[r0:r1])", "dK[:nk] += scale * (dS.T @ k[r0:r1])"),
    "dP_uses_q": ("dP = do[r0:r1] @ v[:nk].T", "dP = do[r0:r1] @ v[:nk].T + 1e-3 * q[r0:r1] @ k[:nk].T"),
    "mask_off_by_one": ("S = np.where(kj > qi, -np.inf, S)", "S = np.where(kj > qi + 1, -np.inf, S)"),
    "lse_log2": ("return e / l, (m + np.log(l))[:, 0]", "return e / l, (m + np.log2(l))[:, 0]"),
    "lse_no_max": ("return e / l, (m + np.log(l))[:, 0]", "return e / l, (np.log(l))[:, 0]"),
    "D_from_dP_only": ("Dr = (dP * P).sum(axis=1)", "Dr = dP.sum(axis=1)"),
    "scores_no_scale": ("S = scale * (q @ k.T)", "S = (q @ k.T)"),
    "varlen_keys_cut_at_query_length": ("qh, kh, vh = q[b, :lq, h], k[b, :lk, h], v[b, :lk, h]",
                                        "qh, kh, vh = q[b, :lq, h], k[b, :lq, h], v[b, :lq, h]"),
    "varlen_padding_lse_zero": ('"lse": np.full((B, NH, T), -np.inf)}', '"lse": np.zeros((B, NH, T))}'),
    "window_off_by_one": ("S = np.where(qi - kj >= window, -np.inf, S)", "S = np.where(qi - kj > window, -np.inf, S)"),
    "window_ignored": ("S = np.where(qi - kj >= window, -np.inf, S)", "S = S"),
    "alibi_sign": ("S = S - slope * (qi - kj)", "S = S + slope * (qi - kj)"),
    "keybias_sign": ("            S = S + key_bias[None, :nk]\n        allowed = _block_allowed(block_map, block, r0, r1, nk)\n        if allowed is not None:\n            S = np.where(allowed, S, -np.inf)\n        P, lse[r0:r1] = _softmax_rows_or_empty(S)\n        Pk = P if keep is None",
                     "            S = S - key_bias[None, :nk]\n        allowed = _block_allowed(block_map, block, r0, r1, nk)\n        if allowed is not None:\n            S = np.where(allowed, S, -np.inf)\n        P, lse[r0:r1] = _softmax_rows_or_empty(S)\n        Pk = P if keep is None"),
    "keybias_on_queries": ("            S = S + key_bias[None, :nk]\n        allowed = _block_allowed(block_map, block, r0, r1, nk)\n        if allowed is not None:\n            S = np.where(allowed, S, -np.inf)\n        P, lse[r0:r1] = _softmax_rows_or_empty(S)\n        Pk = P if keep is None",
                           "            S = S + key_bias[r0:r1, None]\n        allowed = _block_allowed(block_map, block, r0, r1, nk)\n        if allowed is not None:\n            S = np.where(allowed, S, -np.inf)\n        P, lse[r0:r1] = _softmax_rows_or_empty(S)\n        Pk = P if keep is None"),
    "dbias_from_dP": ("dbias[:nk] += dS.sum(axis=0)", "dbias[:nk] += dP.sum(axis=0)"),
    "dbias_scaled": ("dbias[:nk] += dS.sum(axis=0)", "dbias[:nk] += scale * dS.sum(axis=0)"),
    "dbias_shared_not_summed": ('out["dbias"][b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0] += x',
                                'out["dbias"][b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0] = x'),
    "e4m3_bias_8": ("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)"),
    "e4m3_no_subnormals": ("np.where(e == 0, m / 8.0 * 2.0 ** -6,", "np.where(e == 0, 0.0 * m,"),
    "e4m3_mantissa_quarters": ("(1.0 + m / 8.0) * np.exp2", "(1.0 + m / 4.0) * np.exp2"),
    "fp8_descale_v_dropped": ("    v = e4m3_to_f64(v8) * descale_v\n", "    v = e4m3_to_f64(v8)\n"),
    "dropout_no_rescale": ("Pk = P if keep is None else P * (keep[r0:r1, :nk] / (1.0 - p_drop))",
                           "Pk = P if keep is None else P * keep[r0:r1, :nk]"),
    "dropout_dP_unmasked": ("            dP = dP * (keep[r0:r1, :nk] / (1.0 - p_drop))  # through the dropout",
                            "            dP = dP / (1.0 - p_drop)  # through the dropout"),
    "philox_bump_first_round": ("        if r > 0:\n            k0 = (k0 + np.uint64(PHILOX_W0)) & mask",
                                "        if r >= 0:\n            k0 = (k0 + np.uint64(PHILOX_W0)) & mask"),
    "philox_swapped_words": ("c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & mask,", "c = [p1 & mask, (p1 >> np.uint64(32)) ^ c[1] ^ k0,"),
    "keep_counter_fields_swapped": ("np.broadcast_arrays(g, i, np.uint64(b * NH + h)", "np.broadcast_arrays(i, g, np.uint64(b * NH + h)"),
    "keep_halves_swapped": ("u[:, :, e] = (x[:, :, e // 2] >> (16 * (e % 2))) & 0xFFFF",
                            "u[:, :, e] = (x[:, :, e // 2] >> (16 * (1 - e % 2))) & 0xFFFF"),
    "blocksparse_map_transposed": ("return np.asarray(block_map)[qi[:, None], kj[None, :]] != 0",
                                   "return np.asarray(block_map).T[qi[:, None], kj[None, :]] != 0"),
    "blocksparse_block_index_off": ("qi = np.arange(r0, r1) // block", "qi = np.arange(r0 + 1, r1 + 1) // block"),
    "blocksparse_empty_row_lse_zero": ("lse = np.full(S.shape[0], -np.inf)", "lse = np.zeros(S.shape[0])"),
    "blocksparse_map_ignored": ("            S = np.where(allowed, S, -np.inf)\n        P, lse[r0:r1] = _softmax_rows_or_empty(S)\n        O[r0:r1] = P @ v[:nk]\n    return O, lse",
                                "            pass\n        P, lse[r0:r1] = _softmax_rows_or_empty(S)\n        O[r0:r1] = P @ v[:nk]\n    return O, lse"),
    "alibi_slope_index": ("2.0 ** (-8.0 * (h + 1) / NH)", "2.0 ** (-8.0 * h / NH)"),
}


def _mutant(old: str, new: str):
    src = open(attn_ref.__file__).read()
    assert src.count(old) == 1, f"planted-mistake anchor not found once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = os.path.join(os.path.dirname(attn_ref.__file__), "mutant.py")
    exec(compile(src.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistake_is_caught(mutant):
    mod = _mutant(*MUTANTS[mutant])
    failed = []
    for name, pin in oracle_pins.ALL_PINS:
        if name.startswith("finite_differences"):
            continue  # the slowest pins; the others must already catch every mutant
        try:
            pin(mod)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(name)
    assert failed, f"no pin caught the planted mistake {mutant}"

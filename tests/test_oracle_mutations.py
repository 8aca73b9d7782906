"""Planted mistakes in the oracle (on the CPU) must each be caught by at least one pin.

Each mutant is a copy of the oracle's source with one plausible error (a dropped term, a
wrong sign or index, a transposed operand, a wrong order of steps), loaded as a separate
module; the real oracle is never modified.
"""
import importlib.util
import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sdm_oracle.py")

MUTANTS = {
    # residual against the undecayed read
    "raw_residual": ("rho = alpha[t] * (a @ old)", "rho = (a @ old)"),
    # input gate dropped
    "no_beta": ("delta = beta[t] * (v[t] - rho)", "delta = (v[t] - rho)"),
    # sign of the residual flipped
    "sign_flip": ("delta = beta[t] * (v[t] - rho)", "delta = beta[t] * (rho - v[t])"),
    # written rows not decayed
    "no_decay_on_write": ("round_mem(alpha[t] * old + a[:, None] * delta[None, :]", "round_mem(old + a[:, None] * delta[None, :]"),
    # every row of the table decays, not only the written ones
    "decay_all_rows": ("        old = M[n]\n", "        old = M[n].copy()\n        M *= alpha[t]\n"),
    # read taken before the write
    "read_before_write": (
        "        M[n] = round_mem(alpha[t] * old + a[:, None] * delta[None, :], mem_dtype)\n        m = np.asarray(ridx[t])\n        o[t] = np.asarray(rgt[t], dtype=np.float64) @ M[m]\n",
        "        m = np.asarray(ridx[t])\n        o[t] = np.asarray(rgt[t], dtype=np.float64) @ M[m]\n        M[n] = round_mem(alpha[t] * old + a[:, None] * delta[None, :], mem_dtype)\n"),
    # halves scored against the wrong sub-key sets
    "swapped_halves": ("s1 = x[..., :h] @ np.asarray(C1", "s1 = x[..., h:] @ np.asarray(C1"),
    # slot number transposed
    "slot_transposed": ("slots = (I1[:, :, None] * s + I2[:, None, :])", "slots = (I1[:, :, None] + I2[:, None, :] * s)"),
    # ties broken by descending index
    "tie_desc": ("order = np.lexsort((ids, -scores), axis=-1)", "order = np.lexsort((-ids, -scores), axis=-1)"),
    # ascending instead of descending scores
    "min_instead_of_max": ("order = np.lexsort((ids, -scores), axis=-1)", "order = np.lexsort((ids, scores), axis=-1)"),
    # weights not normalised
    "unnormalised_weights": ("return e / np.sum(e, axis=-1, keepdims=True)", "return e"),
    # softmax with a temperature
    "temperature": ("e = np.exp(z - np.max(z, axis=-1, keepdims=True))", "e = np.exp(0.5 * (z - np.max(z, axis=-1, keepdims=True)))"),
    # table not rounded to bf16 on write
    "no_bf16_rounding": ("    if mem_dtype == \"bf16\":\n        return round_bf16(x)", "    if mem_dtype == \"bf16\":\n        return np.asarray(x, dtype=np.float64)"),
    # bf16 rounding by truncation
    "bf16_truncate": ("y = np.ldexp(np.rint(np.ldexp(x, -q)), q)", "y = np.ldexp(np.trunc(np.ldexp(x, -q)), q)"),
    # read weights taken from the write weights
    "read_uses_write_weights": ("o[t] = np.asarray(rgt[t], dtype=np.float64) @ M[m]", "o[t] = np.asarray(wgt[t], dtype=np.float64)[:len(m)] @ M[m]"),
    # reads addressed by keys
    "reads_from_keys": ("ridx, rgt, rsc = address(q, C1, C2, kappa, R)", "ridx, rgt, rsc = address(k, C1, C2, kappa, R)"),
    # whole-table decay applied after the write (written rows decay twice)
    "table_decay_after_write": (
        "        if decay == \"table\":\n            M *= alpha[t]\n        M[n] = round_mem(alpha[t] * old + a[:, None] * delta[None, :], mem_dtype)\n",
        "        M[n] = round_mem(alpha[t] * old + a[:, None] * delta[None, :], mem_dtype)\n        if decay == \"table\":\n            M *= alpha[t]\n"),
    # whole-table decay never applied
    "table_decay_missing": ("            M *= alpha[t]\n", "            pass\n"),
    # decay gate without the time-step bias
    "gate_no_dt_bias": ("g = -A * _softplus(a + np.asarray(dt_bias, dtype=np.float64)[:, None])", "g = -A * _softplus(a)"),
    # input gate not squashed
    "gate_beta_raw": ("return np.exp(g), 1.0 / (1.0 + np.exp(-b))", "return np.exp(g), b"),
    # RMS without the mean (L2 norm)
    "norm_l2": ("r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)", "r = 1.0 / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps)"),
    # sigmoid gate instead of SiLU
    "gate_sigmoid": ("(z / (1.0 + np.exp(-z)))", "(1.0 / (1.0 + np.exp(-z)))"),
    # head mixing with the untransposed weight
    "mix_transposed": ("@ np.asarray(Wo, dtype=np.float64).T", "@ np.asarray(Wo, dtype=np.float64).T[::-1]"),
    # backward: the read's gradient added after the write part
    "bwd_read_after_write": ("        np.add.at(G, m, u[:, None] * g[None, :])\n", "\n"),
    # backward: the residual's decay dropped from the weight gradient
    "bwd_dw_no_alpha": ("dw[t] += alpha[t] * (x @ drho)", "dw[t] += (x @ drho)"),
    # backward: the table's gradient accumulated instead of replaced at the written rows
    "bwd_g_accumulate": ("        G[n] = dx\n", "        G[n] += dx\n"),
    # addressing backward: the softmax Jacobian without its centring term
    "abwd_no_centring": ("dsc = w * (dw - np.sum(w * dw, axis=-1, keepdims=True))", "dsc = w * dw"),
    # addressing backward: the second half's gradient taken from the first sub-key set
    "abwd_wrong_codebook": ('dx[:, h:] = np.einsum("tk,tkc->tc", dsc, C2[i2])', 'dx[:, h:] = np.einsum("tk,tkc->tc", dsc, C1[i2])'),
    # addressing backward: sub-key gradients scattered with the other half's index
    "abwd_swapped_index": ("np.add.at(dC1, i1.ravel(),", "np.add.at(dC1, i2.ravel(),"),
    # chunkwise form: reads miss the chunk's own writes
    "chunk_no_q": ("        o[tok] = O0 + Q @ delta\n", "        o[tok] = O0\n"),
    # chunkwise form: a read sees its token's write undecayed by nothing (window one short)
    "chunk_q_window": ("Q[i, k] += w * dec(slot, k, i + 1) * wk", "Q[i, k] += w * dec(slot, k, i) * wk"),
    # chunkwise form: the interaction without the token's own gate
    "chunk_k_no_alpha": ("K[i, k] += al[i] * w * dec(slot, k, i) * wk", "K[i, k] += w * dec(slot, k, i) * wk"),
    # chunkwise form: the written-back row forgets the decay of its chunk-start value
    "chunk_no_start_decay": ("row = dec(slot, -1, L) * M[slot]", "row = M[slot]"),
    # per-half top-k keeps too few sub-keys
    "kappa_off_by_one": ("I1 = np.take_along_axis(sub, top_order(s1, sub, kappa), axis=-1)", "I1 = np.take_along_axis(sub, top_order(s1, sub, max(1, kappa - 1)), axis=-1)"),
    # chunkwise form, bf16 table: the chunk-start row rounded after its decay, before the
    # deltas are added
    "chunk_round_start_early": ("row = dec(slot, -1, L) * M[slot]", "row = round_mem(dec(slot, -1, L) * M[slot], mem_dtype)"),
    # chunkwise form: the written-back row is not rounded to the table dtype
    "chunk_no_writeback_rounding": ("            M[slot] = round_mem(row, mem_dtype)\n", "            M[slot] = row\n"),
    # chunkwise form: the chunk-start row's decay taken up to the last writer only
    "chunk_start_decay_short": ("row = dec(slot, -1, L) * M[slot]", "row = dec(slot, -1, L - 1) * M[slot]"),
    # selection by the first half's scores alone
    "select_first_half_only": ("pick = top_order(cand, slots, n_sel)", "pick = top_order(np.repeat(np.take_along_axis(s1, I1, -1), kappa, axis=-1), slots, n_sel)"),
}


def load_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = SRC
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = load_mutant(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"

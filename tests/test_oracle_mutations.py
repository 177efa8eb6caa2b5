"""Each pin must fail when a plausible mistake is planted in the oracle.

The mistakes are planted on the CPU by swapping an oracle function for a
subtly wrong copy; the pin tests are then re-run against it.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
import test_oracle_assign as ta
import test_oracle_bank as tbk
import test_oracle_capacity as tc
import test_oracle_forward as tf
import test_oracle_router as tr


def _fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def test_float_capacity_is_caught(monkeypatch):
    real = om.capacity_plan

    def float_caps(T, top_k, E, P, W, send_cap=(11, 10), recv_cap=(23, 20), cap_send_rows=0, cap_recv_rows=0):
        p = real(T, top_k, E, P, W, send_cap, recv_cap, cap_send_rows, cap_recv_rows)
        p["cap_send"] = math.ceil(send_cap[0] / send_cap[1] * p["Tw"] * top_k / P)
        return p
    monkeypatch.setattr(oracle, "capacity_plan", float_caps)
    assert _fails(tc.test_exact_rational_not_float)


def test_floor_instead_of_ceil_is_caught(monkeypatch):
    real = om.capacity_plan

    def floor_caps(*a, **k):
        p = real(*a, **k)
        p["cap_recv"] = math.floor(Fraction(23, 20) * Fraction(p["Tw"] * a[1], a[2]))
        return p
    monkeypatch.setattr(oracle, "capacity_plan", floor_caps)
    assert _fails(tc.test_recv_share_printed_capacity)


def test_high_index_tie_break_is_caught(monkeypatch):
    def bad_topk(l, b, k):
        s = om.selection_scores(l, b).astype(np.float64)
        T, E = s.shape
        idx = np.broadcast_to(np.arange(E), (T, E))
        return np.lexsort((-idx, -s), axis=-1)[:, :k]
    monkeypatch.setattr(oracle, "route_topk", bad_topk)
    assert _fails(tr.test_topk_bruteforce_with_ties, 0)
    assert _fails(tr.test_all_equal_logits_pick_lowest_indices)


def test_fp64_score_is_caught(monkeypatch):
    def bad_topk(l, b, k):
        s = np.asarray(l, np.float64) + np.asarray(b, np.float64)[None, :]
        T, E = s.shape
        idx = np.broadcast_to(np.arange(E), (T, E))
        return np.lexsort((idx, -s), axis=-1)[:, :k]
    monkeypatch.setattr(oracle, "route_topk", bad_topk)
    assert _fails(tr.test_selection_decided_in_fp32)


def test_biased_gates_are_caught(monkeypatch):
    def bad_gates(l, idx):
        sel = np.take_along_axis(np.asarray(l, np.float64), idx, axis=1)
        sel = sel + 0.01 * np.arange(idx.shape[1])   # a stray additive term
        ex = np.exp(sel - sel.max(1, keepdims=True))
        return ex / ex.sum(1, keepdims=True)
    monkeypatch.setattr(oracle, "gates", bad_gates)
    assert _fails(tr.test_gates_closed_forms)


def test_receiver_cap_first_is_caught(monkeypatch):
    real = om.assign_slots

    def recv_first(idx, E, P, W, cs, cr):
        # wrong order: the receiver cap is checked first, so a row the
        # receiver would refuse never takes a pool slot
        idx = np.asarray(idx)
        T, k = idx.shape
        epp = E // P
        a = real(idx, E, P, W, cs, cr)
        ps = np.full((T, k), -1)
        rs = np.full((T, k), -1)
        for t0, t1 in om.wave_ranges(T, W):
            pc, ec = [0] * P, [0] * E
            for t in range(t0, t1):
                for j in range(k):
                    e = int(idx[t, j])
                    p = e // epp
                    if ec[e] >= cr or pc[p] >= cs:
                        continue
                    ps[t, j] = pc[p]
                    pc[p] += 1
                    rs[t, j] = ec[e]
                    ec[e] += 1
        a["pool_slot"], a["recv_slot"] = ps, rs
        return a
    monkeypatch.setattr(oracle, "assign_slots", recv_first)
    assert _fails(ta.test_brute_force_tiny, 0, 16, 4, 2, 3)


def test_global_counters_across_waves_are_caught(monkeypatch):
    def one_wave(idx, E, P, W, cs, cr):
        # wrong: counters not reset per wave (waves ignored)
        return om.assign_slots(idx, E, P, 1, cs, cr) if W == 1 else _reshape(om.assign_slots(idx, E, P, 1, cs, cr), W)

    def _reshape(a, W):
        a = dict(a)
        a["pool_count"] = np.repeat(a["pool_count"], W, axis=0)
        a["expert_count"] = np.repeat(a["expert_count"], W, axis=0)
        a["bank_rows"] = np.repeat(a["bank_rows"], W, axis=0)
        a["ids"] = np.repeat(a["ids"], W, axis=0)
        return a
    monkeypatch.setattr(oracle, "assign_slots", one_wave)
    assert _fails(ta.test_waves_are_independent_chunks)


def test_renormalised_gates_are_caught(monkeypatch):
    real = om.combine

    def renorm(g, recv_slot, o):
        keep = (np.asarray(recv_slot) >= 0)
        g = np.asarray(g) * keep
        s = g.sum(1, keepdims=True)
        g = np.where(s > 0, g / np.where(s > 0, s, 1), 0)
        return real(g, recv_slot, o)
    monkeypatch.setattr(om, "combine", renorm)
    assert _fails(tf.test_combine_then_project_is_project_then_combine)


def test_transposed_weight_is_caught(monkeypatch):
    def bad_swiglu(u, wg, wu, wd):
        u = np.asarray(u, np.float64)
        return (om.silu(u @ np.asarray(wg).T) * (u @ np.asarray(wu).T)) @ np.asarray(wd).reshape(np.asarray(wd).T.shape)
    monkeypatch.setattr(om, "swiglu", bad_swiglu)
    monkeypatch.setattr(oracle, "swiglu", bad_swiglu)
    assert _fails(tf.test_swiglu_matches_library)
    assert _fails(tf.test_single_expert_is_a_dense_mlp_stack)


def test_wrong_pool_map_is_caught(monkeypatch):
    real = om.assign_slots

    def strided_pools(idx, E, P, W, cs, cr):
        # wrong map e -> e mod P, emulated by relabelling experts
        idx = np.asarray(idx)
        perm = np.array([(e % P) * (E // P) + e // P for e in range(E)])
        a = real(perm[idx], E, P, W, cs, cr)
        inv = np.argsort(perm)
        a["ids"] = np.where(a["ids"] >= 0, inv[np.maximum(a["ids"], 0)], -1)
        a["expert_count"] = a["expert_count"][:, perm]
        a["bank_rows"] = a["bank_rows"][:, perm]
        return a
    monkeypatch.setattr(oracle, "assign_slots", strided_pools)
    assert _fails(ta.test_closed_forms_tiny_workload, 0)


# --- backward of the routed path -------------------------------------------

import oracle.moe_backward as ob  # noqa: E402
import test_oracle_backward as tb  # noqa: E402


def test_silu_derivative_without_the_a_term_is_caught(monkeypatch):
    def wrong(u, w_gate, w_up, w_down, d_o):
        u, wg, wu, wd, d_o = (np.asarray(x, dtype=np.float64) for x in (u, w_gate, w_up, w_down, d_o))
        a, b = u @ wg.T, u @ wu.T
        s = 1 / (1 + np.exp(-a))
        h = a * s * b
        dh = d_o @ wd
        da = dh * b * s          # drops the a (1 - s) term of silu'
        db = dh * a * s
        return da @ wg + db @ wu, da.T @ u, db.T @ u, d_o.T @ h
    monkeypatch.setattr(ob, "swiglu_backward", wrong)
    monkeypatch.setattr(oracle, "swiglu_backward", wrong)
    assert _fails(tb.test_dz_matches_finite_differences, 0)
    assert _fails(tb.test_swiglu_backward_matches_torch_autograd)


def test_transposed_down_gradient_is_caught(monkeypatch):
    real = ob.swiglu_backward

    def wrong(*a):
        du, dwg, dwu, dwd = real(*a)
        return du, dwg, dwu, dwd[::-1].copy()   # rows of dW_d out of order
    monkeypatch.setattr(ob, "swiglu_backward", wrong)
    assert _fails(tb.test_weight_gradients_match_finite_differences, "wd")


def test_gate_left_out_of_d_o_is_caught(monkeypatch):
    def wrong(gate_w, recv_slot, o, dy_lat):
        keep = (np.asarray(recv_slot) >= 0).astype(np.float64)
        dy = np.asarray(dy_lat, dtype=np.float64)
        d_gates = np.einsum("tl,tjl->tj", dy, np.asarray(o, dtype=np.float64)) * keep
        return d_gates, keep[:, :, None] * dy[:, None, :]
    monkeypatch.setattr(ob, "combine_backward", wrong)
    assert _fails(tb.test_dz_matches_finite_differences, 1)


def test_softmax_backward_sign_is_caught(monkeypatch):
    def wrong(gate_w, d_gates):
        g, dg = np.asarray(gate_w), np.asarray(d_gates)
        return g * (dg + (g * dg).sum(axis=1, keepdims=True))
    monkeypatch.setattr(ob, "gates_backward", wrong)
    monkeypatch.setattr(oracle, "gates_backward", wrong)
    assert _fails(tb.test_logit_gradient_matches_finite_differences, 0)
    assert _fails(tb.test_logit_gradient_closed_forms)


def test_dropped_rows_sent_back_is_caught(monkeypatch):
    def wrong_combine(gate_w, recv_slot, o, dy_lat):
        dy = np.asarray(dy_lat, dtype=np.float64)
        return (np.einsum("tl,tjl->tj", dy, np.asarray(o, dtype=np.float64)),
                np.asarray(gate_w, dtype=np.float64)[:, :, None] * dy[:, None, :])
    monkeypatch.setattr(ob, "combine_backward", wrong_combine)
    assert _fails(tb.test_dropped_assignments_get_nothing)


# --------------------------------------------------------------- router bias
import oracle.router_bias as rbm
import test_oracle_bias as tbias

_BIAS_PINS = [tbias.test_worked_example_by_hand, tbias.test_rank_on_a_bin_edge_takes_that_bin,
              tbias.test_rank_before_an_empty_bin_is_the_generalised_inverse,
              lambda: tbias.test_quantile_inverts_the_interpolated_cdf(4096, 16, 2, 16),
              tbias.test_histogram_matches_numpy_on_exact_edges, tbias.test_quantile_within_one_bin_of_the_sample_quantile,
              tbias.test_shift_equivariance_is_exact, tbias.test_zero_mean, tbias.test_special_levels,
              tbias.test_the_bias_balances_a_skewed_router]


def _some_bias_pin_fails():
    return any(_fails(f) for f in _BIAS_PINS)


def _quantile_variant(level_of=None, strict=False, width_div=0):
    def q(hist, lo, hi, T, top_k):
        hist = np.asarray(hist, dtype=np.int64)
        E, nb = hist.shape
        level = level_of(E, top_k) if level_of else Fraction(E - top_k, E)
        r = float(level * T)
        out = np.empty(E)
        for e in range(E):
            c = np.cumsum(hist[e])
            j = int(np.argmax(c > r)) if strict else int(np.argmax(c >= r))
            cp = int(c[j - 1]) if j > 0 else 0
            w = (float(hi[e]) - float(lo[e])) / (nb - width_div if nb > width_div else 1)
            out[e] = float(lo[e]) + (j + (r - cp) / int(hist[e, j])) * w
        return out
    return q


def test_bias_pins_pass_on_the_real_oracle():
    assert not _some_bias_pin_fails()


def test_lower_tail_level_is_caught(monkeypatch):
    monkeypatch.setattr(rbm, "histogram_quantile", _quantile_variant(level_of=lambda E, k: Fraction(k, E)))
    assert _some_bias_pin_fails()


def test_strict_rank_search_is_caught(monkeypatch):
    monkeypatch.setattr(rbm, "histogram_quantile", _quantile_variant(strict=True))
    assert _some_bias_pin_fails()


def test_bin_width_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(rbm, "histogram_quantile", _quantile_variant(width_div=1))
    assert _some_bias_pin_fails()


def test_missing_mean_removal_is_caught(monkeypatch):
    def no_centre(logits32, top_k, n_bins):
        l = np.asarray(logits32, dtype=np.float32)
        hist, lo, hi = rbm.histograms(l, n_bins)
        q = rbm.histogram_quantile(hist, lo, hi, l.shape[0], top_k)
        return (-q).astype(np.float32), hist, lo, hi, q
    monkeypatch.setattr(rbm, "bias_update", no_centre)
    monkeypatch.setattr(tbias.rb, "bias_update", no_centre)
    assert _some_bias_pin_fails()


def test_bias_sign_flip_is_caught(monkeypatch):
    real = rbm.bias_update

    def flipped(logits32, top_k, n_bins):
        b, *rest = real(logits32, top_k, n_bins)
        return (-b).astype(np.float32), *rest
    monkeypatch.setattr(tbias.rb, "bias_update", flipped)
    assert _some_bias_pin_fails()


def test_global_range_instead_of_per_expert_is_caught(monkeypatch):
    real_range = rbm.logit_range

    def global_range(logits32):
        lo, hi = real_range(logits32)
        return np.full_like(lo, lo.min()), np.full_like(hi, hi.max())
    monkeypatch.setattr(rbm, "logit_range", global_range)
    assert _some_bias_pin_fails()


def test_round_to_nearest_bin_is_caught(monkeypatch):
    def nearest(logits32, lo, scale, n_bins):
        l = np.asarray(logits32, dtype=np.float32)
        p = ((l - lo[None, :]) * scale[None, :]).astype(np.float32)
        return np.minimum(np.rint(p).astype(np.int64), n_bins - 1)
    monkeypatch.setattr(rbm, "bin_index", nearest)
    assert _some_bias_pin_fails()


# ------------------------------------------------------------------ receiver side
def _bank_variant(pick):
    """bank_expert_rows with the (w, r) -> (row wave, slot) map replaced."""
    def bad(rows, bank_rows, expert_count, expert_weights, experts, row_filter=None):
        out = {}
        W, _, C = bank_rows.shape
        for e in experts:
            wg, wu, wd = expert_weights(int(e))
            sel = [x for w in range(W) for x in pick(bank_rows, expert_count, w, int(e), C)]
            sel = [(w, s) for (w, s) in sel if row_filter is None or row_filter(w, s)]
            if not sel:
                continue
            o = om.swiglu(np.stack([np.asarray(rows[w][s], np.float64) for w, s in sel]), wg, wu, wd)
            out.update({ws: v for ws, v in zip(sel, o)})
        return out
    return bad


def test_bank_rows_pins_pass_on_the_real_oracle():
    tbk.test_bank_rows_equal_forward_expert_outputs()
    tbk.test_bank_rows_single_wave_by_hand()


def test_bank_rows_swapped_waves_are_caught(monkeypatch):
    # the row lists of wave w read against the pool block of another wave
    pick = lambda br, ec, w, e, C: [(w, int(br[(w + 1) % br.shape[0], e, r]))
                                    for r in range(int(ec[(w + 1) % br.shape[0], e]))]
    monkeypatch.setattr(oracle, "bank_expert_rows", _bank_variant(pick))
    assert _fails(tbk.test_bank_rows_equal_forward_expert_outputs)


def test_bank_rows_read_past_count_are_caught(monkeypatch):
    # every entry of the row list, not just the first expert_count
    pick = lambda br, ec, w, e, C: [(w, int(br[w, e, r])) for r in range(C)]
    monkeypatch.setattr(oracle, "bank_expert_rows", _bank_variant(pick))
    assert _fails(tbk.test_bank_rows_equal_forward_expert_outputs)


def test_bank_rows_off_by_one_slot_is_caught(monkeypatch):
    pick = lambda br, ec, w, e, C: [(w, int(br[w, e, r]) + 1) for r in range(int(ec[w, e]))]
    monkeypatch.setattr(oracle, "bank_expert_rows", _bank_variant(pick))
    assert _fails(tbk.test_bank_rows_single_wave_by_hand)


def test_bank_rows_receiver_slot_as_pool_slot_is_caught(monkeypatch):
    # the receiver slot r taken as the pool slot (no bank_rows lookup)
    pick = lambda br, ec, w, e, C: [(w, r) for r in range(int(ec[w, e]))]
    monkeypatch.setattr(oracle, "bank_expert_rows", _bank_variant(pick))
    assert _fails(tbk.test_bank_rows_equal_forward_expert_outputs)


def test_drop_fractions_swapped_ends_are_caught(monkeypatch):
    def bad(a, T, k):
        n = T * k
        return dict(sender=a["receiver_dropped"] / n, receiver=a["sender_dropped"] / n,
                    total=(a["sender_dropped"] + a["receiver_dropped"]) / n)
    monkeypatch.setattr(oracle, "drop_fractions", bad)
    assert _fails(tbk.test_drop_fractions_hand_count)
    assert _fails(tbk.test_drop_fractions_conservation)


def test_drop_fractions_per_token_denominator_is_caught(monkeypatch):
    def bad(a, T, k):
        sd, rd = a["sender_dropped"], a["receiver_dropped"]
        return dict(sender=sd / T, receiver=rd / T, total=(sd + rd) / T)
    monkeypatch.setattr(oracle, "drop_fractions", bad)
    assert _fails(tbk.test_drop_fractions_hand_count)

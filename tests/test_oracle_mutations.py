"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that at least one pin fails for each.  This is what makes the pins worth
trusting: a dropped term, a flipped tie rule, a swapped operand or an
off-by-one scan would not slip through."""
import numpy as np
import pytest

import oracle as O
import oracle.moe_oracle as M
from tests import test_formats_pins as F
from tests import test_oracle_pins as P
from tests import test_prenorm_pins as N
from tests import test_lora_pins as LP
from tests import test_backward_pins as BP


def patch(monkeypatch, name, fn):
    monkeypatch.setattr(M, name, fn)
    if hasattr(O, name):          # private helpers are not re-exported
        monkeypatch.setattr(O, name, fn)


def ties_to_higher_index(logits32, k):
    T, E = logits32.shape
    idx = np.broadcast_to(-np.arange(E), (T, E))
    return np.lexsort((idx, -logits32.astype(np.float64)), axis=-1)[:, :k].astype(np.int32)


def no_renormalisation(logits32, ids):
    l = np.asarray(logits32, dtype=np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids.astype(np.int64), axis=1)


def renormalised_anyway(logits32, ids):
    l = np.asarray(logits32, dtype=np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def sigmoid_not_silu(z):
    return 1.0 / (1.0 + np.exp(-z))


def inclusive_scan(counts):
    c = np.cumsum(counts)
    return np.concatenate([c, [c[-1]]]).astype(np.int32)


def unstable_permute(ids_flat, offsets):
    perm, pos = ORIG_STABLE(ids_flat, offsets)
    for e in range(len(offsets) - 1):
        a, b = offsets[e], offsets[e + 1]
        perm[a:b] = perm[a:b][::-1].copy()
    pos[perm] = np.arange(len(perm))
    return perm, pos


def bias_ignored(x_bits, wr_bits, bias=None, exact=False):
    return ORIG_LOGITS(x_bits, wr_bits, None, exact)


def swapped_nibbles(packed):
    out = ORIG_UNPACK(packed)
    out[..., 0::2], out[..., 1::2] = out[..., 1::2].copy(), out[..., 0::2].copy()
    return out


def rne_through_fp32(v):
    return ORIG_RNE(np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64))


def norm_variant(kind):
    def f(residual_bits, delta_bits, gamma_bits, eps):
        r = M.bf16_bits_to_f64(residual_bits)
        if delta_bits is not None and kind != "delta_dropped":
            r = r + M.bf16_bits_to_f64(delta_bits)
        r_bits = M.f64_to_bf16_rne(r)
        r = M.bf16_bits_to_f64(r_bits)
        if kind == "sum_not_mean":
            ms = np.sum(r * r, axis=1, keepdims=True)
        else:
            ms = np.mean(r * r, axis=1, keepdims=True)
        e = 0.0 if kind == "eps_ignored" else float(eps)
        g = 1.0 if kind == "gamma_ignored" else M.bf16_bits_to_f64(gamma_bits)[None, :]
        return r_bits, r / np.sqrt(ms + e) * g
    return f


def lora_scale_ignored(lora, e, I):
    t = ORIG_LORA_OF(lora, e, I)
    return None if t is None else (*t[:5], 1.0)


def lora_variant(kind):
    def mlp(x64, wg, wu, wd, lora=None):
        if lora is None:
            return ORIG_MLP(x64, wg, wu, wd)
        a_gu, b_g, b_u, a_d, b_d, s = lora
        g, u = x64 @ wg.T, x64 @ wu.T
        z = x64 @ a_gu.T
        if kind == "after_silu":
            h = M.silu(g) * u + s * (z @ b_g.T)
        else:
            h = M.silu(g + s * (z @ b_g.T)) * (u + s * (z @ b_u.T))
        y = h @ wd.T
        if kind != "down_dropped":
            y = y + s * ((h @ a_d.T) @ b_d.T)
        return y
    return mlp


def silu_grad_is_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def backward_uncentred_softmax(inp, d_out, weights=None, routing=None):
    """The backward with d_l = w * d_w (the softmax Jacobian's centring term
    dropped): only the router part of d_x changes."""
    b = ORIG_BACKWARD(inp, d_out, weights, routing)
    ids, w = b["routing"]["ids"], b["routing"]["w"]
    wr = M.bf16_bits_to_f64(inp.w_router)
    wrong = w * b["d_w"]
    d_x = b["d_x"].copy()
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            d_x[t] += (wrong[t, j] - b["d_logits"][t, j]) * wr[int(ids[t, j])]
    return dict(b, d_x=d_x, d_logits=wrong)


def backward_lora_variant(kind):
    """LoRA backward mistakes: the adapter gradients without the scale, or
    d_x taken through the frozen weights alone (adapter path dropped)."""
    def f(inp, d_out, weights=None, routing=None, lora=None):
        b = ORIG_BACKWARD(inp, d_out, weights, routing, lora)
        if lora is None:
            return b
        if kind == "scale_dropped":
            return dict(b, **{n: b[n] / lora.scale for n in ("d_a_gate_up", "d_b_gate_up", "d_a_down", "d_b_down")})
        return dict(b, d_x=ORIG_BACKWARD(inp, d_out, weights, routing)["d_x"])
    return f


def backward_wgrad_variant(kind):
    """Expert-weight gradient mistakes: gate and up halves swapped, or the
    down gradient taken with d_out instead of w * d_out."""
    def f(inp, d_out, weights=None, routing=None, lora=None, weight_grads=False):
        b = ORIG_BACKWARD(inp, d_out, weights, routing, lora, weight_grads)
        if not weight_grads:
            return b
        if kind == "halves_swapped":
            g = b["d_w_gate_up"]
            return dict(b, d_w_gate_up=np.concatenate([g[:, inp.I:], g[:, :inp.I]], axis=1))
        r = dict(b["routing"], w=np.ones_like(b["routing"]["w"]))
        return dict(b, d_w_down=ORIG_BACKWARD(inp, d_out, weights, r, lora, True)["d_w_down"])
    return f


def backward_unrenorm_chosen_only(inp, d_out, weights=None, routing=None, lora=None, weight_grads=False,
                                  wgrad_experts=None, renorm=True):
    """The un-renormalised backward with the softmax gradient kept on the k
    chosen logits only (the experts not chosen dropped from the router share)."""
    b = ORIG_BACKWARD(inp, d_out, weights, routing, lora, weight_grads, wgrad_experts, renorm)
    if renorm:
        return b
    ids = b["routing"]["ids"].astype(np.int64)
    wr = M.bf16_bits_to_f64(inp.w_router)
    keep = np.zeros_like(b["d_logits"], dtype=bool)
    np.put_along_axis(keep, ids, True, axis=1)
    dropped = np.where(keep, 0.0, b["d_logits"])
    return dict(b, d_x=b["d_x"] - dropped @ wr, d_logits=np.where(keep, b["d_logits"], 0.0))


ORIG_BACKWARD = M.backward_per_token
ORIG_LORA_OF = M._lora_of
ORIG_MLP = M.expert_mlp
ORIG_RNE = M.f64_to_bf16_rne
ORIG_STABLE = M.stable_permute
ORIG_LOGITS = M.router_logits
ORIG_UNPACK = M.nf4_unpack


def swap_gate_up(monkeypatch):
    orig = M.ExpertWeights._convert

    def conv(self, e):
        orig(self, e)
        g, u, d = self._pending[e]
        self._pending[e] = (u, g, d)

    monkeypatch.setattr(M.ExpertWeights, "_convert", conv)


def uniform_combine(monkeypatch):
    orig = M.route

    def route(*a, **kw):
        ids, w, l = orig(*a, **kw)
        return ids, np.full_like(w, 1.0 / w.shape[1]), l

    patch(monkeypatch, "route", route)


MUTATIONS = {
    "ties_to_higher_index": (lambda mp: patch(mp, "topk_lowest_index", ties_to_higher_index),
                             [P.test_hand_worked_block_closed_form, P.test_identical_router_rows_lower_index_wins]),
    "no_renormalisation": (lambda mp: patch(mp, "renormalised_weights", no_renormalisation),
                           [P.test_hand_worked_block_closed_form, P.test_weights_sum_to_one_and_are_positive]),
    "unrenormalised_variant_renormalises": (lambda mp: patch(mp, "softmax_weights", renormalised_anyway),
                                            [P.test_unrenormalised_hand_closed_form,
                                             P.test_unrenormalised_weights_are_softmax_mass_of_the_chosen]),
    "bf16_rounding_through_fp32": (lambda mp: patch(mp, "f64_to_bf16_rne", rne_through_fp32),
                                   [N.test_rne_is_nearest_with_ties_to_even]),
    "norm_delta_dropped": (lambda mp: patch(mp, "residual_rmsnorm", norm_variant("delta_dropped")),
                           [N.test_residual_add_matches_torch_bf16_add]),
    "norm_sum_not_mean": (lambda mp: patch(mp, "residual_rmsnorm", norm_variant("sum_not_mean")),
                          [N.test_rmsnorm_matches_torch_rms_norm, N.test_rmsnorm_constant_row_closed_form]),
    "norm_eps_ignored": (lambda mp: patch(mp, "residual_rmsnorm", norm_variant("eps_ignored")),
                         [N.test_rmsnorm_constant_row_closed_form]),
    "norm_gamma_ignored": (lambda mp: patch(mp, "residual_rmsnorm", norm_variant("gamma_ignored")),
                           [N.test_rmsnorm_matches_torch_rms_norm, N.test_rmsnorm_constant_row_closed_form]),
    "lora_scale_ignored": (lambda mp: patch(mp, "_lora_of", lora_scale_ignored),
                           [LP.test_lora_hand_closed_form, LP.test_lora_equals_merged_weights]),
    "lora_delta_after_silu": (lambda mp: patch(mp, "expert_mlp", lora_variant("after_silu")),
                              [LP.test_lora_hand_closed_form, LP.test_lora_equals_merged_weights]),
    "lora_down_dropped": (lambda mp: patch(mp, "expert_mlp", lora_variant("down_dropped")),
                          [LP.test_lora_hand_closed_form, LP.test_lora_equals_merged_weights]),
    "backward_silu_grad_is_sigmoid": (lambda mp: patch(mp, "silu_grad", silu_grad_is_sigmoid),
                                      [BP.test_backward_matches_torch_autograd,
                                       BP.test_backward_finite_differences]),
    "backward_softmax_not_centred": (lambda mp: patch(mp, "backward_per_token", backward_uncentred_softmax),
                                     [BP.test_backward_matches_torch_autograd,
                                      BP.test_backward_finite_differences]),
    "backward_lora_grad_scale_dropped": (lambda mp: patch(mp, "backward_per_token",
                                                          backward_lora_variant("scale_dropped")),
                                         [BP.test_backward_with_lora_matches_torch_autograd]),
    "backward_lora_d_x_through_frozen_weights": (lambda mp: patch(mp, "backward_per_token",
                                                                  backward_lora_variant("dx_frozen")),
                                                 [BP.test_backward_with_lora_matches_torch_autograd]),
    "backward_wgrad_gate_up_halves_swapped": (lambda mp: patch(mp, "backward_per_token",
                                                               backward_wgrad_variant("halves_swapped")),
                                              [BP.test_backward_weight_grads_match_torch_autograd]),
    "backward_wgrad_down_without_routing_weight": (lambda mp: patch(mp, "backward_per_token",
                                                                    backward_wgrad_variant("unweighted")),
                                                   [BP.test_backward_weight_grads_match_torch_autograd]),
    "backward_unrenormalised_chosen_only": (lambda mp: patch(mp, "backward_per_token",
                                                             backward_unrenorm_chosen_only),
                                            [BP.test_backward_unrenormalised_matches_torch_autograd]),
    "sigmoid_not_silu": (lambda mp: patch(mp, "silu", sigmoid_not_silu),
                         [P.test_hand_worked_block_closed_form, P.test_single_expert_reduces_to_swiglu_mlp]),
    "gate_up_swapped": (swap_gate_up,
                        [P.test_hand_worked_block_closed_form, P.test_single_expert_reduces_to_swiglu_mlp]),
    "routing_weights_ignored": (uniform_combine, [P.test_hand_worked_block_closed_form]),
    "inclusive_scan": (lambda mp: patch(mp, "exclusive_scan", inclusive_scan),
                       [P.test_bucketing_random_and_adversarial]),
    "unstable_permute": (lambda mp: patch(mp, "stable_permute", unstable_permute),
                         [P.test_bucketing_random_and_adversarial, P.test_bucketing_zero_input_closed_form]),
    "bias_ignored": (lambda mp: patch(mp, "router_logits", bias_ignored),
                     [P.test_router_bias_added_in_fp32]),
    "nibbles_swapped": (lambda mp: patch(mp, "nf4_unpack", swapped_nibbles),
                        [F.test_nf4_pack_unpack_round_trip_and_nibble_order,
                         F.test_nf4_dequant_is_codebook_times_absmax_in_fp32]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    apply, pins = MUTATIONS[name]
    apply(monkeypatch)
    for pin in pins:
        with pytest.raises((AssertionError, IndexError, ValueError)):
            pin()

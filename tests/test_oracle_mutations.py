"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of an oracle module (a textual edit
of its source, executed as a fresh module on the CPU), points one pin test at
the copy and expects that pin to fail. The real oracle is never modified."""

import inspect
import types

import pytest

import oracle.bf16
import oracle.loss
import oracle.objectives
import oracle.philox
import oracle.schedule
import oracle.truncate
import oracle.verify

from . import test_oracle_bf16 as t_bf16
from . import test_oracle_loss as t_loss
from . import test_oracle_loss_logits as t_logits
from . import test_oracle_margins as t_margin
from . import test_oracle_objectives as t_obj
from . import test_oracle_philox as t_philox
from . import test_oracle_schedule as t_sched
from . import test_oracle_truncate as t_trunc
from . import test_oracle_verify as t_verify


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) == 1, f"mutation anchor not unique in {module.__name__}: {old!r}"
    mod = types.ModuleType(module.__name__)
    mod.__package__ = "oracle"
    mod.__file__ = module.__file__
    exec(compile(src.replace(old, new), module.__file__, "exec"), mod.__dict__)
    return mod


# (oracle module, anchor, replacement, test module, its alias for the oracle
#  module, pin test, args)
CASES = [
    ("accept compares with <=", oracle.verify,
     "return bool(u < r), abs(u - r)", "return bool(u <= r), abs(u - r)",
     t_verify, "ov", "test_accept_rule_threshold_on_the_24_bit_lattice", ()),
    ("accept when q(y) = 0 and p(y) = 0", oracle.verify,
     "return bool(p_y > 0.0), np.inf", "return True, np.inf",
     t_verify, "ov", "test_accept_rule_threshold_on_the_24_bit_lattice", ()),
    ("residual drawn from p instead of max(0, p - q)", oracle.verify,
     "w = np.maximum(0.0, p[j] - q[j])", "w = p[j]",
     t_verify, "ov", "test_residual_support_invariant", ()),
    ("residual drawn from max(0, q - p)", oracle.verify,
     "w = np.maximum(0.0, p[j] - q[j])", "w = np.maximum(0.0, q[j] - p[j])",
     t_verify, "ov", "test_single_position_law_rebuilds_target", ()),
    ("bonus drawn from the last draft position", oracle.verify,
     "        w = p[k_b]\n", "        w = p[k_b - 1]\n",
     t_verify, "ov", "test_chi_square_emitted_law_two_positions", ()),
    ("inverse CDF takes the first C[v] >= target", oracle.verify,
     'side="right"', 'side="left"',
     t_verify, "ov", "test_draw_counts_on_the_24_bit_lattice", ()),
    ("overlap sums max instead of min", oracle.verify,
     "np.sum(np.minimum(p, q))", "np.sum(np.maximum(p, q))",
     t_verify, "ov", "test_alpha_is_one_minus_tv", (1.0,)),
    ("temperature multiplies instead of divides", oracle.verify,
     "inv_t = np.float32(1.0) / np.float32(temperature)",
     "inv_t = np.float32(temperature)",
     t_verify, "ov", "test_alpha_is_one_minus_tv", (0.6,)),
    ("greedy correction takes the draft argmax", oracle.verify,
     'out["tokens"][j] = g[j]', 'out["tokens"][j] = h[j] if j < k_b else g[j]',
     t_verify, "ov", "test_greedy_literal_rule_with_arbitrary_tokens", ()),
    ("scan continues past a rejection", oracle.verify,
     "            j = k\n            break\n\n    _, u_draw",
     "            j = k\n\n    _, u_draw",
     t_verify, "ov", "test_chi_square_emitted_law_two_positions", ()),
    ("gradient weight uses P_k instead of P_{k-1}", oracle.loss,
     "g = -prev * suffix", "g = -prefix * suffix",
     t_loss, "ol", "test_gradient_matches_torch_autograd", ()),
    ("gradient sign flipped on the q >= p side", oracle.loss,
     "-coef * q * s_below[:, None]", "coef * q * s_below[:, None]",
     t_loss, "ol", "test_gradient_central_differences", ()),
    ("suffix recursion drops alpha", oracle.loss,
     "suffix[k] = 1.0 + alpha[k + 1] * suffix[k + 1]",
     "suffix[k] = 1.0 + suffix[k + 1]",
     t_loss, "ol", "test_gradient_matches_torch_autograd", ()),
    ("branches summed instead of averaged", oracle.loss,
     '"loss": total / n_br,', '"loss": total,',
     t_loss, "ol", "test_worked_examples",
     ({"alphas": [0.8, 0.8, 0.8, 0.8], "expected_emitted": 3.3616},)),
    ("CE gradient drops the sum of p", oracle.objectives,
     "dz = (q * np.sum(p64, axis=1, keepdims=True) - p64) / n_branches",
     "dz = (q - p64) / n_branches",
     t_obj, "ob", "test_gradient_central_differences", ("ce",)),
    ("KL drops the p log p term", oracle.objectives,
     "per_pos = ce + np.sum(plogp, axis=1)", "per_pos = ce",
     t_obj, "ob", "test_kl_vanishes_at_q_equal_p", ()),
    ("per-step TV gradient sign flipped", oracle.objectives,
     "dz = np.where(below, -q * s_above, q * s_below) / n_branches",
     "dz = np.where(below, q * s_above, -q * s_below) / n_branches",
     t_obj, "ob", "test_gradient_central_differences", ("step_tv",)),
    ("per-step TV loss sums alpha", oracle.objectives,
     "loss_n = float(np.sum(1.0 - alpha))", "loss_n = float(np.sum(alpha))",
     t_obj, "ob", "test_step_tv_is_half_l1_and_matches_e2e_at_one_position", ()),
    ("logits-target gradient drops the 1/T chain factor", oracle.objectives,
     "return loss_n, alpha, float(inv_t) * ds", "return loss_n, alpha, ds",
     t_logits, "ob", "test_gradient_central_differences_through_the_scaling", ("e2e_tv",)),
    ("target logits left unscaled by the temperature", oracle.objectives,
     "scaled_logits(target_logits_bf16[n], temperature)",
     "bf16.decode(target_logits_bf16[n]).astype(np.float64)",
     t_logits, "ob", "test_alpha_is_the_verify_overlap_at_the_same_temperature", (0.6,)),
    ("target softmax taken over the draft row", oracle.objectives,
     "p = np.stack([e2e.softmax64(s_t[k])", "p = np.stack([e2e.softmax64(np.asarray(s_z)[k])",
     t_logits, "ob", "test_matches_torch_autograd_at_an_exact_temperature", ("ce",)),
    ("schedule takes the smallest survivals first", oracle.schedule,
     "order = np.lexsort((np.arange(flat.size), -flat.astype(np.float64)))",
     "order = np.lexsort((np.arange(flat.size), flat.astype(np.float64)))",
     t_sched, "osch", "test_matches_exhaustive_search", ("steps", 3, 3)),
    ("schedule prices the batch without the bonus tokens", oracle.schedule,
     "theta = (R + s) * sps[R + np.arange(flat.size + 1)]",
     "theta = (R + s) * sps[np.arange(flat.size + 1)]",
     t_sched, "osch", "test_matches_exhaustive_search", ("steps", 3, 3)),
    ("schedule drops the guaranteed token per request", oracle.schedule,
     "theta = (R + s) * sps[R + np.arange(flat.size + 1)]",
     "theta = s * sps[R + np.arange(flat.size + 1)]",
     t_sched, "osch", "test_flat_curve_verifies_everything_and_collapse_verifies_nothing", ()),
    ("top-p keeps one token too few", oracle.truncate,
     'n = int(np.searchsorted(c, target, side="left")) + 1',
     'n = int(np.searchsorted(c, target, side="left"))',
     t_trunc, "ot", "test_top_p_matches_the_ascending_formulation", (0.5,)),
    ("top-p measured against the untruncated mass", oracle.truncate,
     "w = np.exp(s[idx[:m]] - np.max(s))", "w = np.exp(s[idx] - np.max(s))",
     t_trunc, "ot", "test_top_k_then_top_p_uses_the_top_k_mass", ()),
    ("equal logits kept in reverse token order", oracle.truncate,
     "return np.lexsort((np.arange(s.size), -s))",
     "return np.lexsort((-np.arange(s.size), -s))",
     t_trunc, "ot", "test_equal_logits_kept_in_token_order", ()),
    ("Philox key not bumped between rounds", oracle.philox,
     "k0 = (k0 + _WEYL_A) & _MASK64", "k0 = k0",
     t_philox, "philox", "test_block_matches_numpy_random_counters", ()),
    ("Philox words permuted wrongly", oracle.philox,
     "c0, c1, c2, c3 = hi_b ^ c1 ^ k0, lo_b, hi_a ^ c3 ^ k1, lo_a",
     "c0, c1, c2, c3 = hi_a ^ c1 ^ k0, lo_b, hi_b ^ c3 ^ k1, lo_a",
     t_philox, "philox", "test_block_matches_numpy_random_counters", ()),
    ("uniform from the low bits", oracle.philox,
     "float(int(word) >> 40)", "float(int(word) & 0xFFFFFF)",
     t_philox, "philox", "test_uniforms_are_top_24_bits", ()),
    ("draw margin not normalised by the total", oracle.verify,
     "margin = min(float(target) - below, c[v] - float(target)) / total",
     "margin = min(float(target) - below, c[v] - float(target))",
     t_margin, "ov", "test_draw_margin_exact", (0.5, 1, 0.25)),
    ("draw margin measured from the wrong lower bound", oracle.verify,
     "below = c[v - 1] if v > 0 else 0.0", "below = c[v - 2] if v > 1 else 0.0",
     t_margin, "ov", "test_draw_margin_exact", (0.75 + 2.0 ** -12, 2, 2.0 ** -12)),
    ("accept margin measured against p(y) instead of p/q", oracle.verify,
     "return bool(u < r), abs(u - r)", "return bool(u < r), abs(u - p_y)",
     t_margin, "ov", "test_accept_margin_exact", (0.25, 0.5, 0.5 - 3 * 2.0 ** -24, True,
                                                   3 * 2.0 ** -24)),
    ("top-p margin not normalised", oracle.truncate,
     "margin = min(abs(c[n - 1] - target), abs(target - below)) / c[-1]",
     "margin = min(abs(c[n - 1] - target), abs(target - below))",
     t_margin, "ot", "test_top_p_margin_exact", (0.5 + 2.0 ** -6, 3, 2.0 ** -6)),
    ("top-p margin normalised by the whole row", oracle.truncate,
     "margin = min(abs(c[n - 1] - target), abs(target - below)) / c[-1]",
     "margin = min(abs(c[n - 1] - target), abs(target - below)) / np.sum(np.exp(s - np.max(s)))",
     t_margin, "ot", "test_top_p_margin_is_normalised_by_the_top_k_total", ()),
    ("top-p margin taken one token late", oracle.truncate,
     "below = c[n - 2] if n >= 2 else 0.0", "below = c[n - 1]",
     t_margin, "ot", "test_top_p_margin_exact", (0.5 + 2.0 ** -6, 3, 2.0 ** -6)),
    ("schedule lets a NaN throughput win", oracle.schedule,
     "theta = np.where(np.isnan(theta), -np.inf, theta)", "pass",
     t_margin, "osch", "test_schedule_never_picks_a_nan_throughput", ()),
    ("bf16 ties rounded away from zero", oracle.bf16,
     "np.rint(scaled)", "np.floor(scaled + 0.5)",
     t_bf16, "bf16", "test_ties_round_to_even", ()),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pin_catches_planted_mistake(case, monkeypatch):
    _, module, old, new, test_mod, alias, test_name, args = case
    mutant = _mutant(module, old, new)
    monkeypatch.setattr(test_mod, alias, mutant)
    with pytest.raises(AssertionError):
        getattr(test_mod, test_name)(*args)

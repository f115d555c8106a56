"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each case rewrites one expression in the source of an oracle function, runs
the pins that should catch it against the mutated module, and requires at
least one of them to fail.  The oracle module is restored afterwards.
"""
import importlib
import inspect
import textwrap

import pytest

import oracle.fp8 as fp8_mod
import oracle.qat_attention as qa_mod
from tests import test_oracle_attention as TA
from tests import test_oracle_fp8 as TF
from tests import test_oracle_quant as TQ
from tests import test_oracle_qkv_wiring as TW


def _pins_attention():
    yield lambda: TA.test_quant_off_is_textbook_attention(37, 37, True)
    yield lambda: TA.test_quant_off_is_textbook_attention(20, 70, False)
    yield lambda: TA.test_quant_off_backward_is_autograd(False)
    yield lambda: TA.test_quant_off_backward_is_autograd(True)
    yield lambda: TA.test_dk_sums_to_zero(False, False)
    yield lambda: TA.test_ste_gradients_equal_finite_differences(False, False, "e4m3")
    yield lambda: TA.test_ste_gradients_equal_finite_differences(True, False, "e4m3")
    yield lambda: TA.test_zero_q_closed_form("e4m3")
    yield lambda: TA.test_single_key_closed_form()
    yield lambda: TA.test_causal_first_row_and_future_independence()
    yield lambda: TA.test_p_groups_are_64_absolute_columns()
    yield lambda: TA.test_fp8_v_path()


def _pins_quant():
    yield TQ.test_worked_example_e4m3
    yield TQ.test_worked_example_e5m2
    yield lambda: TQ.test_absmax_element_maps_to_fmax("e4m3")
    yield lambda: TQ.test_error_bound("e4m3", 3)
    yield TQ.test_groups_are_independent_and_absolute
    yield TQ.test_zero_and_underflow_groups
    yield TQ.test_token_and_channel_helpers


def _pins_qkv():
    for which in "qkv":
        for causal in (False, True):
            yield lambda w=which, c=causal: TW.test_qkv_quant_equals_attention_on_hand_quantized_inputs(w, c)


def _pins_fp8():
    yield lambda: TF.test_rounding_vs_brute_force_at_boundaries("e4m3")
    yield lambda: TF.test_rounding_vs_brute_force_at_boundaries("e5m2")
    yield lambda: TF.test_decode_matches_torch_float8("e4m3")
    yield lambda: TF.test_decode_matches_torch_float8("e5m2")
    yield TF.test_ties_to_even_examples
    yield TF.test_saturation_and_signed_zero


MUTANTS = [
    # (module, function, original snippet, mutated snippet, pin family)
    (qa_mod, "backward_head", "float(sm_scale) * (dS.T @ qh[r])", "(dS.T @ qh[r])", "attn"),
    (qa_mod, "backward_head", "float(sm_scale) * (dS_q @ kh)", "(dS_q @ kh)", "attn"),
    (qa_mod, "backward_head", "Delta = np.sum(do[r] * O_hp, axis=1)", "Delta = np.sum(do[r] * (_p_hat(P, p_quant, p_fmt, group) @ vh), axis=1)", "attn"),
    (qa_mod, "backward_head", "dS = P[:, k_rows] * (dP - Delta[:, None])", "dS = P[:, k_rows] * (dP + Delta[:, None])", "attn"),
    (qa_mod, "backward_head", "dS_q = P[sel] * (dP_q - Delta[sel, None])", "dS_q = P[sel] * dP_q", "attn"),
    (qa_mod, "backward_head", "dS = P[:, k_rows] * (dP - Delta[:, None])", "dS = Ph[:, k_rows] * (dP - Delta[:, None])", "attn"),
    (qa_mod, "backward_head", "dV += Ph[:, k_rows].T @ do[r]", "dV += P[:, k_rows].T @ do[r]", "attn"),
    (qa_mod, "backward_head", "dP = do[r] @ vh[k_rows].T", "dP = do[r] @ vh[k_rows][::-1].T", "attn"),
    (qa_mod, "backward_head", "c = slice(g * group, min(Nkv, (g + 1) * group))", "c = slice(g * group + 1, min(Nkv, (g + 1) * group))", "attn"),
    (qa_mod, "_scores", "cols[None, :] > rows[:, None]", "cols[None, :] > rows[:, None] + 1", "attn"),
    (qa_mod, "_scores", "float(sm_scale) * (qh[rows] @ kh.T)", "(qh[rows] @ kh.T)", "attn"),
    (qa_mod, "_softmax_rows", "lse = m[:, 0] + np.log(", "lse = m[:, 0] + np.log2(", "attn"),
    (qa_mod, "forward_head", "O[b0:b0 + r.size] = Ph @ vh", "O[b0:b0 + r.size] = P @ vh", "attn"),
    (qa_mod, "fake_quant_groups", "s = _to_f32(a / FMAX)", "s = _to_f32(a / (FMAX - 1))", "quant"),
    (qa_mod, "fake_quant_groups", "a = np.max(np.abs(blk), axis=1)", "a = np.max(blk, axis=1)", "quant"),
    (qa_mod, "fake_quant_groups", "c0, c1 = g * group, min((g + 1) * group, cols)", "c0, c1 = g * group + (g > 0), min((g + 1) * group + 1, cols)", "quant"),
    (qa_mod, "quantize_v_channels", "fake_quant_groups(vt, fmt, N)", "fake_quant_groups(vt, fmt, max(1, N // 2))", "quant"),
    # Q/K/V fake-quant wiring: a tensor left unquantized, the e5m2 grid, one
    # scale per channel instead of per token
    (qa_mod, "_prepare_head", 'vh = quantize_token_rows(vh, "e4m3")[2].astype(np.float64)', "vh = vh", "qkv"),
    (qa_mod, "_prepare_head", 'qh = quantize_token_rows(qh, "e4m3")[2].astype(np.float64)', "qh = qh", "qkv"),
    (qa_mod, "_prepare_head", 'qh = quantize_token_rows(qh, "e4m3")', 'qh = quantize_token_rows(qh, "e5m2")', "qkv"),
    (qa_mod, "_prepare_head", 'kh = quantize_token_rows(kh, "e4m3")', 'kh = quantize_token_rows(kh, "e5m2")', "qkv"),
    (qa_mod, "_prepare_head", 'kh = quantize_token_rows(kh, "e4m3")[2].astype(np.float64)',
     'kh = quantize_token_rows(kh.T, "e4m3")[2].T.astype(np.float64)', "qkv"),
    (qa_mod, "_prepare_head", 'vh = quantize_token_rows(vh, "e4m3")[2].astype(np.float64)',
     'vh = quantize_token_rows(vh.T, "e4m3")[2].T.astype(np.float64)', "qkv"),
    (fp8_mod, "round_rne_sat", "n = np.rint(a / quantum)", "n = np.floor(a / quantum + 0.5)", "fp8"),
    (fp8_mod, "round_rne_sat", "e = np.maximum(ex - 1, emin)", "e = np.maximum(ex, emin)", "fp8"),
    (fp8_mod, "decode", "(1 - bias - mbits)", "(-bias - mbits)", "fp8"),
]


def _mutate(module, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, fname)))
    assert old in src, f"snippet not found in {fname}: {old}"
    ns = module.__dict__
    exec(compile(src.replace(old, new), module.__file__, "exec"), ns)


@pytest.mark.parametrize("case", MUTANTS,
                         ids=lambda m: f"{m[1]}:{m[3][:40]}")
def test_planted_mistake_is_caught(case):
    module, fname, old, new, family = case
    pins = {"attn": _pins_attention, "quant": _pins_quant, "fp8": _pins_fp8, "qkv": _pins_qkv}[family]
    try:
        _mutate(module, fname, old, new)
        caught = False
        for pin in pins():
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught = True
                break
        assert caught, f"no pin caught the mutation of {fname}"
    finally:
        importlib.reload(fp8_mod)
        importlib.reload(qa_mod)

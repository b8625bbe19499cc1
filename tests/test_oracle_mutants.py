"""Plant plausible mistakes in the oracle (on the CPU) and require that the pins catch
each one: a dropped term, a wrong sign, a wrong index or mask bound, a transposed
operand, a missing scale, the wrong logarithm, a missing max shift."""
import numpy as np
import pytest

import oracle
from oracle import attention as A
from tests import pins


def _probs_variant(q_blk, k, scale, causal, kv_len_b, row0, *, causal_off=0, pad_off=0,
                   shift=True, scale_in_s=True):
    s = (scale if scale_in_s else 1.0) * (q_blk @ k.T)
    i = np.arange(row0, row0 + q_blk.shape[0])[:, None]
    j = np.arange(k.shape[0])[None, :]
    a = np.ones(s.shape, bool)
    if causal:
        a &= j <= i + causal_off
    if kv_len_b is not None:
        a &= j < int(kv_len_b) + pad_off
    s = np.where(a, s, -np.inf)
    m = s.max(axis=1) if shift else np.zeros(s.shape[0])
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def _fwd_variant(**kw):
    log = kw.pop("log", np.log)

    def head_forward(q, k, v, scale, causal=False, kv_len_b=None):
        p, m, l = _probs_variant(q, k, scale, causal, kv_len_b, 0, **kw)
        return p @ v, m + log(l)
    return head_forward


def _bwd_variant(kind):
    def head_backward(q, k, v, dout, scale, causal=False, kv_len_b=None, check_d=True):
        p, _, _ = _probs_variant(q, k, scale, causal, kv_len_b, 0)
        dv = p.T @ dout
        dp = dout @ v.T
        dsum = (p * dp).sum(1)
        ds = p * (dp - dsum[:, None])
        dq = scale * ds @ k
        dk = scale * ds.T @ q
        if kind == "drop_D":
            ds = p * dp
            dq, dk = scale * ds @ k, scale * ds.T @ q
        elif kind == "sign_D":
            ds = p * (dsum[:, None] - dp)
            dq, dk = scale * ds @ k, scale * ds.T @ q
        elif kind == "dk_untransposed":
            dk = scale * ds @ q
        elif kind == "dv_untransposed":
            dv = p @ dout
        elif kind == "dq_no_scale":
            dq = ds @ k
        elif kind == "dp_wrong_operand":
            dp = dout @ k.T
            ds = p * (dp - (p * dp).sum(1)[:, None])
            dq, dk = scale * ds @ k, scale * ds.T @ q
        elif kind == "D_from_wrong_rows":
            ds = p * (dp - np.roll(dsum, 1)[:, None])
            dq, dk = scale * ds @ k, scale * ds.T @ q
        return dq, dk, dv
    return head_backward


FWD_MUTANTS = {
    "causal_excludes_diagonal_plus1": _fwd_variant(causal_off=1),
    "causal_excludes_diagonal": _fwd_variant(causal_off=-1),
    "padding_off_by_one": _fwd_variant(pad_off=1),
    "no_max_shift": _fwd_variant(shift=False),
    "lse_log2": _fwd_variant(log=np.log2),
    "scale_dropped": _fwd_variant(scale_in_s=False),
}
BWD_MUTANTS = ["drop_D", "sign_D", "dk_untransposed", "dv_untransposed", "dq_no_scale",
               "dp_wrong_operand", "D_from_wrong_rows"]


def _run_all_checks():
    failed = []
    for check in pins.ALL_CHECKS:
        if check is pins.check_finite_differences:
            continue  # slow; the other pins already catch every planted mistake
        try:
            with np.errstate(all="ignore"):
                check(oracle.attention_forward, oracle.attention_backward)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(monkeypatch, name):
    monkeypatch.setattr(A, "head_forward", FWD_MUTANTS[name])
    assert _run_all_checks(), f"no pin caught forward mutant {name}"


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_backward_mutant_is_caught(monkeypatch, kind):
    monkeypatch.setattr(A, "head_backward", _bwd_variant(kind))
    assert _run_all_checks(), f"no pin caught backward mutant {kind}"


def test_finite_differences_catch_drop_D(monkeypatch):
    """The finite-difference pin on its own catches a dropped -D term."""
    monkeypatch.setattr(A, "head_backward", _bwd_variant("drop_D"))
    with pytest.raises(AssertionError):
        pins.check_finite_differences(oracle.attention_forward, oracle.attention_backward)

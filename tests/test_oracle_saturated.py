"""Pins of the oracle's gradient on saturated rows against 60-digit decimal
arithmetic.

When one vocabulary entry holds nearly all of the student's mass (q_max =
1 - 1e-15 and beyond, as on the heavy-head workload), the centring of the
reverse-KL and mixture gradients subtracts numbers of the size of the
log-sum-exps to leave a value of order 1e-12 or less, and forward KL's
q_a - p_a subtracts two numbers near one when both models saturate. Here
every entry of the oracle's dL/ds must match the definitions evaluated with
Python's decimal module at 60 significant digits (exp and ln of the exactly
converted fp64 logits) to a relative 1e-9, the dominant entry included;
the formula evaluated as written in fp64 misses the dominant entry by far
more, which the last test shows.
"""
from decimal import Decimal, localcontext

import numpy as np
import pytest

from oracle import kd_oracle as O


def exact_grad(s_row, t_row, beta):
    """dL/ds of the beta table (forward KL, reverse KL, mixture), in decimal."""
    with localcontext() as ctx:
        ctx.prec = 60
        S = [Decimal(float(x)) for x in s_row]
        T = [Decimal(float(x)) for x in t_row]

        def log_softmax(x):
            m = max(x)
            lse = m + sum((xi - m).exp() for xi in x).ln()
            return [xi - lse for xi in x]

        lq, lp = log_softmax(S), log_softmax(T)
        q = [x.exp() for x in lq]
        p = [x.exp() for x in lp]
        if beta == 0.0:
            return np.array([float(a - b) for a, b in zip(q, p)])
        if beta == 1.0:
            kl = sum(qi * (a - b) for qi, a, b in zip(q, lq, lp))
            return np.array([float(qi * (a - b - kl)) for qi, a, b in zip(q, lq, lp)])
        b = Decimal(float(beta))
        lm = [(b * pi + (1 - b) * qi).ln() for pi, qi in zip(p, q)]
        kl = sum(qi * (a - m) for qi, a, m in zip(q, lq, lm))
        return np.array([float((1 - b) * qi * (a - m - kl)) for qi, a, m in zip(q, lq, lm)])


def _rows():
    g = np.random.default_rng(71)
    V = 64
    s, t = g.normal(0, 1, (4, V)), g.normal(0, 2, (4, V))
    s[0, 7] = 45.0               # saturated student, teacher not
    s[1, 7], t[1, 7] = 40.0, 38.0  # both saturated on the same entry
    s[2, 3] = 30.0               # saturated student, teacher's mass elsewhere
    t[2, 11] = 25.0
    s[3, 5] = 2.5                # q_max about 0.5: not saturated
    return s, t


@pytest.mark.parametrize("beta", [0.0, 0.3, 0.5, 1.0])
def test_gradient_matches_decimal_on_saturated_rows(beta):
    s, t = _rows()
    got = O.grad_student_logits(s, t, beta)
    for r in range(s.shape[0]):
        want = exact_grad(s[r], t[r], beta)
        err = np.abs(got[r] - want)
        assert np.all(err <= 1e-9 * np.abs(want) + 1e-300), (r, np.max(err / (np.abs(want) + 1e-300)))
        assert abs(np.sum(want)) <= 1e-12 * np.sum(np.abs(want))  # the exact gradient sums to zero


def test_direct_fp64_evaluation_loses_the_dominant_entry():
    # the plain fp64 evaluation of q (log q - log p - KL) on the saturated row
    s, t = _rows()
    lq, lp = O.log_softmax(s[:1]), O.log_softmax(t[:1])
    q = np.exp(lq)
    kl = np.sum(q * (lq - lp), axis=-1, keepdims=True)
    naive = (q * (lq - lp - kl))[0]
    want = exact_grad(s[0], t[0], 1.0)
    a = int(np.argmax(s[0]))
    assert abs(naive[a] - want[a]) > 1e-6 * abs(want[a])
    assert abs(O.grad_student_logits(s[:1], t[:1], 1.0)[0, a] - want[a]) <= 1e-9 * abs(want[a])

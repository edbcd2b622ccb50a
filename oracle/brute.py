"""Pure-Python brute force for tiny inputs (lists and ``math`` only).

TEST INFRASTRUCTURE (same import rule as ``kd_oracle``). It recomputes the
same definitions element by element, with no numpy, so that a slip in the
vectorised oracle (an axis, a broadcast, a dropped term) shows up as a
disagreement. Definitions as cited in ``kd_oracle``: [White-box OPD, 2.3] for
the beta family and the temperature, [Top-K KD, 一.2] for the three terms,
[White-box OPD, 2.4] for the tail bucket.
"""
from __future__ import annotations

import math


def dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def row_logits(h_row, W):
    return [dot(h_row, w) for w in W]


def log_softmax(x):
    m = max(x)
    s = math.fsum(math.exp(v - m) for v in x)
    L = m + math.log(s)
    return [v - L for v in x], L


def divergence_row(s, t, beta):
    lq, _ = log_softmax(s)
    lp, _ = log_softmax(t)
    if beta == 0.0:
        return math.fsum(math.exp(a) * (a - b) for a, b in zip(lp, lq))
    if beta == 1.0:
        return math.fsum(math.exp(b) * (b - a) for a, b in zip(lp, lq))
    tot = 0.0
    parts = []
    for a, b in zip(lp, lq):
        m = beta * math.exp(a) + (1.0 - beta) * math.exp(b)
        lm = math.log(m)
        parts.append(beta * math.exp(a) * (a - lm) + (1.0 - beta) * math.exp(b) * (b - lm))
    tot = math.fsum(parts)
    return tot


def loss_rows(h_s, W_s, h_t, W_t, beta, tau):
    out = []
    for hs, ht in zip(h_s, h_t):
        s = [z / tau for z in row_logits(hs, W_s)]
        t = [z / tau for z in row_logits(ht, W_t)]
        out.append(divergence_row(s, t, beta))
    return out


def fd_grad_h(h_s, W_s, h_t, W_t, beta, tau, eps=1e-5):
    """Central finite differences of each row's loss w.r.t. its student hidden state."""
    grads = []
    for hs, ht in zip(h_s, h_t):
        g = []
        for i in range(len(hs)):
            hp = list(hs)
            hm = list(hs)
            hp[i] += eps
            hm[i] -= eps
            lp = loss_rows([hp], W_s, [ht], W_t, beta, tau)[0]
            lm = loss_rows([hm], W_s, [ht], W_t, beta, tau)[0]
            g.append((lp - lm) / (2 * eps))
        grads.append(g)
    return grads


def fd_grad_W(h_s, W_s, h_t, W_t, beta, tau, eps=1e-5):
    """Central finite differences of the summed loss w.r.t. each entry of W_s."""
    grads = []
    for v in range(len(W_s)):
        g = []
        for i in range(len(W_s[v])):
            Wp = [list(r) for r in W_s]
            Wm = [list(r) for r in W_s]
            Wp[v][i] += eps
            Wm[v][i] -= eps
            lp = math.fsum(loss_rows(h_s, Wp, h_t, W_t, beta, tau))
            lm = math.fsum(loss_rows(h_s, Wm, h_t, W_t, beta, tau))
            g.append((lp - lm) / (2 * eps))
        grads.append(g)
    return grads


def topk_row(keys, k):
    """k indices of the largest keys, ties broken by the lower index."""
    return [i for _, i in sorted(((-v, i) for i, v in enumerate(keys)))[:k]]


def three_terms_row(zs, zt, sel, tau):
    """binary, cond for one row from (already rounded) logits."""
    s = [z / tau for z in zs]
    t = [z / tau for z in zt]
    lq, _ = log_softmax(s)
    lp, _ = log_softmax(t)
    P = math.fsum(math.exp(lp[i]) for i in sel)
    Q = math.fsum(math.exp(lq[i]) for i in sel)
    binary = P * math.log(P / Q)
    if P < 1.0:
        binary += (1.0 - P) * math.log((1.0 - P) / (1.0 - Q))
    cond = math.fsum((math.exp(lp[i]) / P) * (math.log(math.exp(lp[i]) / P) - math.log(math.exp(lq[i]) / Q))
                     for i in sel)
    return binary, cond, P, Q


def fd_grad_topk_row(zs, zt, sel, tau, label, wb, wc, we, eps=1e-6):
    """Central finite differences of wb*binary + wc*cond + we*ce for one row
    w.r.t. each student logit (selection and teacher fixed)."""
    def loss(z):
        b, c, _, _ = three_terms_row(z, zt, sel, tau)
        out = wb * b + wc * c
        if label is not None and label != -100:
            m = max(z)
            ce = m + math.log(math.fsum(math.exp(x - m) for x in z)) - z[label]
            out += we * ce
        return out
    g = []
    for i in range(len(zs)):
        zp = list(zs)
        zm = list(zs)
        zp[i] += eps
        zm[i] -= eps
        g.append((loss(zp) - loss(zm)) / (2 * eps))
    return g


def tail_loss_row(zs, zt, sup, beta, tau):
    """Beta-divergence over the buckets {each support entry} + {the rest}
    for one row ((already rounded) logits; sup: support indices)."""
    s = [z / tau for z in zs]
    t = [z / tau for z in zt]
    lq, _ = log_softmax(s)
    lp, _ = log_softmax(t)
    pb = [math.exp(lp[i]) for i in sup]
    qb = [math.exp(lq[i]) for i in sup]
    if len(set(sup)) < len(zs):
        rest = [i for i in range(len(zs)) if i not in set(sup)]
        pb.append(math.fsum(math.exp(lp[i]) for i in rest))
        qb.append(math.fsum(math.exp(lq[i]) for i in rest))
    terms = []
    for p, q in zip(pb, qb):
        if beta == 0.0:
            terms.append(p * math.log(p / q))
        elif beta == 1.0:
            terms.append(q * math.log(q / p))
        else:
            m = beta * p + (1.0 - beta) * q
            terms.append(beta * p * math.log(p / m) + (1.0 - beta) * q * math.log(q / m))
    return math.fsum(terms)


def fd_grad_tail_row(zs, zt, sup, beta, tau, eps=1e-6):
    """Central finite differences of ``tail_loss_row`` w.r.t. each student
    logit (support and teacher fixed)."""
    g = []
    for i in range(len(zs)):
        zp = list(zs)
        zm = list(zs)
        zp[i] += eps
        zm[i] -= eps
        g.append((tail_loss_row(zp, zt, sup, beta, tau) - tail_loss_row(zm, zt, sup, beta, tau)) / (2 * eps))
    return g

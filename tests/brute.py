"""Independent brute-force statement of the sampled estimator for tiny inputs.

Pure Python loops, written separately from the C oracle to pin it:
  * bf16 rounding comes from torch's cast, not the oracle's bit routine;
  * each code bit is sign(x . w) with a Python float dot product;
  * the sampling probability enumerates every subset of the L tables
    (P = sum over subsets with at least T members, the pages' T = 2, of
     prod p * prod (1 - p)), instead of a binomial formula;
  * the estimator is Equation 9 literally: sum (w_i / u_i) v_i / sum (w_i / u_i)
    with w_i = exp(q.k_i / sqrt(d)).
MagicPIG, arXiv 2410.16179v2: Section 2.2 (SimHash), Section 4.3 (Equations 9-11),
Algorithm 1; the centring of Section 4.3 "Data pre-processing".
"""
import itertools
import math

import numpy as np
import torch


def bf16(v: float) -> float:
    return float(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float()[0])


def mean_f32(keys):
    d = len(keys[0])
    return [float(np.float32(math.fsum(float(k[t]) for k in keys) / len(keys))) for t in range(d)]


def code_of(vec, mu, W, K, L, lift_r=None):
    """Code bits of one vector; with ``lift_r`` (Equation 8) the vector gets the
    extra coordinate sqrt(r^2 - |x|^2) (rounded to fp32, then bf16) and W has
    d + 1 rows; a lifted query passes lift_r = 0.0 (extra coordinate 0)."""
    d = len(vec)
    if mu is None:
        x = [bf16(float(np.float32(vec[t]))) for t in range(d)]
    else:
        x = [bf16(float(np.float32(vec[t]) - np.float32(mu[t]))) for t in range(d)]
    if lift_r is not None:
        rem = float(lift_r) ** 2 - math.fsum(v * v for v in x) if lift_r else 0.0
        x = x + [bf16(float(np.float32(math.sqrt(rem)))) if rem > 0 else 0.0]
        d += 1
    codes = []
    for l in range(L):
        c = 0
        for b in range(K):
            j = l * K + b
            z = 0.0
            for t in range(d):
                z += x[t] * bf16(float(W[t][j]))
            if z > 0:
                c += 1 << b
        codes.append(c)
    return codes


def prob_at_least(p: float, L: int, T: int = 2) -> float:
    total = 0.0
    for hits in itertools.product([0, 1], repeat=L):
        if sum(hits) >= T:
            term = 1.0
            for h in hits:
                term *= p if h else (1.0 - p)
            total += term
    return total


def prob_at_least_two(p: float, L: int) -> float:
    return prob_at_least(p, L, 2)


def lift_radius(keys, mu):
    """Largest |bf16(k - mu)| over the keys, rounded to fp32 (Equation 8's r)."""
    best = 0.0
    for k in keys:
        x = [bf16(float(np.float32(k[t]) - np.float32(mu[t]))) for t in range(len(k))]
        best = max(best, math.fsum(v * v for v in x))
    return float(np.float32(math.sqrt(best)))


def decode_head(q, keys, vals, W, K, L, n_static_head=0, n_static_tail=0, T=2, lift=False):
    """Returns (sampled index list, out vector, lse) for one query head; a key
    is sampled when it collides in at least T tables.  With ``lift`` the keys
    are hashed lifted (Equation 8; W has d + 1 rows) and the sampling angle is
    taken against the lifted key, whose norm is r."""
    n, d = len(keys), len(q)
    mu = mean_f32(keys)
    R = lift_radius(keys, mu) if lift else None
    kc = [code_of(k, mu, W, K, L, R) for k in keys]
    qc = code_of(q, None, W, K, L, 0.0 if lift else None)
    S, forced = [], []
    for i in range(n):
        f = i < n_static_head or i >= n - n_static_tail
        m = sum(1 for l in range(L) if kc[i][l] == qc[l])
        if f or m >= T:
            S.append(i)
            forced.append(f)
    qn = math.sqrt(sum(float(a) * float(a) for a in q))
    num = [0.0] * d
    den = 0.0
    for i, f in zip(S, forced):
        k = [float(a) for a in keys[i]]
        c = [k[t] - mu[t] for t in range(d)]
        cn = R if lift else math.sqrt(sum(a * a for a in c))
        if f:
            u = 1.0
        else:
            cosv = sum(float(q[t]) * c[t] for t in range(d)) / (qn * cn) if qn > 0 and cn > 0 else 0.0
            cosv = max(-1.0, min(1.0, cosv))
            p = (1.0 - math.acos(cosv) / math.pi) ** K
            u = prob_at_least(p, L, T)
        w = math.exp(sum(float(q[t]) * k[t] for t in range(d)) / math.sqrt(d))
        den += w / u
        for t in range(d):
            num[t] += (w / u) * float(vals[i][t])
    if not S:
        return S, [0.0] * d, -math.inf
    return S, [a / den for a in num], math.log(den)

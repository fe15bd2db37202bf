"""50-digit decimal brute force of softmax attention for tiny problems.

Independent of the C oracle: pure Python ``decimal`` arithmetic on the exact
values of the stored inputs. It materialises the full masked score matrix of
each segment and head, so it is only for a handful of tokens.

Visibility of key j to query row i of a segment with Sq queries and Sk keys
(bottom-right alignment, inclusive window, -1 = unbounded):
the query sits at key position pos = i + Sk - Sq; j is visible iff
0 <= j < Sk, (not causal or j <= pos), (left < 0 or j >= pos - left) and
(right < 0 or j <= pos + right).
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np

PREC = 50


def _to_float(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _dec_tanh(x: Decimal) -> Decimal:
    e2 = (2 * x).exp()
    return (e2 - 1) / (e2 + 1)


def visible(i, j, sq, sk, causal, left, right) -> bool:
    pos = i + sk - sq
    if j < 0 or j >= sk:
        return False
    if causal and j > pos:
        return False
    if left >= 0 and j < pos - left:
        return False
    if right >= 0 and j > pos + right:
        return False
    return True


def attention(q, k, v, cu_q, cu_k, *, causal=False, window=(-1, -1), softcap=0.0, scale=None):
    """Returns (O [total_q, Hq, d_v], LSE [total_q, Hq]) as float64 arrays."""
    qf, kf, vf = _to_float(np.asarray(q)), _to_float(np.asarray(k)), _to_float(np.asarray(v))
    total_q, hq, dqk = qf.shape
    hkv = kf.shape[1]
    dv = vf.shape[2]
    group = hq // hkv
    if scale is None:
        scale = dqk ** -0.5
    out = np.zeros((total_q, hq, dv), dtype=np.float64)
    lse = np.full((total_q, hq), -np.inf, dtype=np.float64)
    with localcontext() as ctx:
        ctx.prec = PREC
        dscale = Decimal(float(scale))
        dcap = Decimal(float(softcap))
        for b in range(len(cu_q) - 1):
            q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
            k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
            sq, sk = q1 - q0, k1 - k0
            for h in range(hq):
                g = h // group
                for i in range(sq):
                    keys = [j for j in range(sk) if visible(i, j, sq, sk, causal, window[0], window[1])]
                    if not keys:
                        continue
                    scores = []
                    for j in keys:
                        dot = sum(Decimal(float(qf[q0 + i, h, c])) * Decimal(float(kf[k0 + j, g, c]))
                                  for c in range(dqk))
                        t = dscale * dot
                        if softcap > 0:
                            t = dcap * _dec_tanh(t / dcap)
                        scores.append(t)
                    m = max(scores)
                    es = [(s - m).exp() for s in scores]
                    z = sum(es)
                    for c in range(dv):
                        acc = sum(e * Decimal(float(vf[k0 + j, g, c])) for e, j in zip(es, keys))
                        out[q0 + i, h, c] = float(acc / z)
                    lse[q0 + i, h] = float(m + z.ln())
    return out, lse

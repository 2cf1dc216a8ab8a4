"""Pure-Python brute force for tiny GQA inputs -- TEST INFRASTRUCTURE ONLY.

A second, independent spelling of the oracle for toy sizes (pure Python floats,
no numpy, no C): it materialises the broadcast of each KV head to its R query heads
(the ``repeat_interleave`` over the head axis that the page "Hands-on: implementing
GQA in PyTorch", section 1.3, applies to K), builds an explicit mask matrix
(the upper triangle above the diagonal, as in "LLM principles -- code implementation
of multi-head attention (MQA and GQA)", section 3), and applies the softmax from its
textbook form without subtracting the maximum. Inputs are nested lists.
"""

from __future__ import annotations

import math


def _materialise(kv, H):
    """kv[b][g][t][d] with G heads -> [b][h][t][d] with H heads, head h taking g = h // (H/G)."""
    out = []
    for per_b in kv:
        G = len(per_b)
        R = H // G
        out.append([per_b[h // R] for h in range(H)])
    return out


def attention(q, k, v, causal, scale, q_offset=0):
    """q[b][h][i][d], k/v[b][g][j][d] (lists of Python floats).

    Query row i sits at absolute position ``q_offset + i``; with ``causal`` it sees
    keys j <= q_offset + i. Returns out[b][h][i][d].
    """
    B = len(q)
    H = len(q[0])
    kh = _materialise(k, H)
    vh = _materialise(v, H)
    out = []
    for b in range(B):
        ob = []
        for h in range(H):
            Tq = len(q[b][h])
            Tk = len(kh[b][h])
            mask = [[(causal and j > q_offset + i) for j in range(Tk)] for i in range(Tq)]
            oh = []
            for i in range(Tq):
                w = []
                for j in range(Tk):
                    if mask[i][j]:
                        w.append(0.0)
                    else:
                        dot = 0.0
                        for d in range(len(q[b][h][i])):
                            dot += q[b][h][i][d] * kh[b][h][j][d]
                        w.append(math.exp(scale * dot))
                z = sum(w)
                D = len(vh[b][h][0])
                oh.append([sum(w[j] * vh[b][h][j][d] for j in range(Tk)) / z for d in range(D)])
            ob.append(oh)
        out.append(ob)
    return out

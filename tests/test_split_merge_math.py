"""The split-KV merge the decode kernels rely on, as an fp64 model on the CPU, against the unsplit
oracle ("GQA revolution: how xformers speeds up LLM inference", section on split-KV block
computation: the cache is cut into key ranges whose partial results are reduced; the page gives
no formula).

A key range s leaves, per query head, a reference m_s, l_s = sum_j 2^(t_j - m_s) and
acc_s = sum_j 2^(t_j - m_s) v_j, with t_j the base-2 score of key j; an empty range leaves
m = -inf, l = 0, acc = 0. With M = max_s m_s and w_s = 2^(m_s - M) (0 for an empty range),
out = (sum_s w_s acc_s) / (sum_s w_s l_s). The kernels take m_s lazily (a reference that lags the
running maximum by up to 2^8 in probability) and merge the four waves of a workgroup the same
way before the ranges; any reference gives the same result in exact arithmetic, and in fp64 to
1e-12 here. This tests the algorithm's mathematics, not the oracle (whose decode is the
reference) and not the kernels.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as W

LOG2E = 1.0 / math.log(2.0)


def _partial(t, v, lo, hi, ref_drop):
    """(m, l, acc) of keys lo..hi-1 for one head; t base-2 scores [L], v values [L, D]. The
    reference is the range's maximum lowered by ref_drop (a lazy reference), -inf when empty."""
    if hi <= lo:
        return -math.inf, 0.0, np.zeros(v.shape[1])
    m = float(np.max(t[lo:hi])) - ref_drop
    p = np.exp2(t[lo:hi] - m)
    return m, float(p.sum()), p @ v[lo:hi]


def _merge(parts):
    M = max(m for m, _, _ in parts)
    num, den = 0.0, 0.0
    for m, l, acc in parts:
        if m == -math.inf:
            continue
        w = 2.0 ** (m - M)
        num = num + w * acc
        den += w * l
    return num / den


def _split_decode(case, cuts_of, rng, lazy):
    """The decode of `case` through split partials: cuts_of(L) gives the range boundaries of a
    sequence of L keys; each range is further cut in four interleaved 32-key blocks sets (the
    waves of a workgroup), merged first, as in the kernels."""
    q = oracle.to_f64(case.q)
    k, v = oracle.decode_kv_f64(case)
    B, H, D = q.shape
    G = k.shape[1]
    R = H // G
    out = np.zeros((B, H, D))
    for b in range(B):
        L = int(min(max(int(case.seq_lens[b]), 0), k.shape[2]))
        if L == 0:
            continue
        cuts = cuts_of(L)
        for h in range(H):
            g = h // R
            t = (k[b, g, :L] @ q[b, h]) * case.scale * LOG2E
            ranges = []
            for lo, hi in zip(cuts[:-1], cuts[1:]):
                # four waves: blocks w, w+4, ... of 32 keys inside the range
                waves = []
                for w in range(4):
                    rows = [r for r in range(lo, hi) if ((r - lo) // 32) % 4 == w]
                    if not rows:
                        waves.append((-math.inf, 0.0, np.zeros(D)))
                        continue
                    drop = float(rng.uniform(0, 8)) if lazy else 0.0
                    m = float(np.max(t[rows])) - drop
                    p = np.exp2(t[rows] - m)
                    waves.append((m, float(p.sum()), p @ v[b, g, rows]))
                if hi <= lo:
                    ranges.append((-math.inf, 0.0, np.zeros(D)))
                    continue
                # the workgroup's partial: its waves merged to a common reference
                Mw = max(m for m, _, _ in waves)
                l = sum(2.0 ** (m - Mw) * lw for m, lw, _ in waves if m != -math.inf)
                acc = sum(2.0 ** (m - Mw) * a for m, _, a in waves if m != -math.inf)
                ranges.append((Mw, l, acc))
            out[b, h] = _merge(ranges)
    return out


CASES = [
    # B, H, G, lens, T_cap
    (2, 8, 2, [300, 77], 320),
    (3, 4, 1, [1, 64, 129], 160),
    (1, 16, 16, [513], 513),
    (4, 8, 4, [0, 5, 200, 33], 256),
]


@pytest.mark.parametrize("B,H,G,lens,T_cap", CASES)
@pytest.mark.parametrize("lazy", [False, True])
def test_uniform_ranges_merge_to_the_oracle(B, H, G, lens, T_cap, lazy):
    """Uniform ranges of split_len keys, S of them, empty ones included (as the uniform layout)."""
    c = W.make_decode(B, H, G, 32, lens, T_cap=T_cap, q_dtype=W.F32, kv_dtype=W.F32, seed=B + H)
    want = oracle.decode(c)
    rng = np.random.default_rng(7)
    for S in (1, 2, 3, 7, 64):
        split_len = -(-T_cap // S)
        got = _split_decode(c, lambda L: [min(s * split_len, L) for s in range(S)] + [L], rng, lazy)
        assert np.max(np.abs(got - want)) <= 1e-12, (S, lazy)


@pytest.mark.parametrize("lazy", [False, True])
def test_ragged_pieces_merge_to_the_oracle(lazy):
    """Arbitrary cut points, as the flat layout's pieces fall wherever a workgroup's run ends."""
    c = W.make_decode(3, 8, 2, 32, [700, 45, 260], T_cap=700, q_dtype=W.F32, kv_dtype=W.F32, seed=5)
    want = oracle.decode(c)
    rng = np.random.default_rng(11)

    def cuts(L):
        inner = sorted(set(int(x) for x in rng.integers(1, L, size=min(5, max(L - 1, 0)))))
        return [0] + inner + [L]

    got = _split_decode(c, cuts, rng, lazy)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_a_dropped_weight_is_caught():
    """The model is sensitive: merging without the 2^(m_s - M) weights is far off."""
    c = W.make_decode(1, 4, 2, 32, [200], T_cap=200, q_dtype=W.F32, kv_dtype=W.F32, seed=3)
    want = oracle.decode(c)
    q = oracle.to_f64(c.q)
    k, v = oracle.decode_kv_f64(c)
    t = (k[0, 0, :200] @ q[0, 0]) * c.scale * LOG2E
    parts = [_partial(t, v[0, 0, :200], lo, hi, 0.0) for lo, hi in ((0, 100), (100, 200))]
    wrong = sum(acc for _, _, acc in parts) / sum(l for _, l, _ in parts)
    assert np.max(np.abs(wrong - want[0, 0])) > 1e-3
    assert np.max(np.abs(_merge(parts) - want[0, 0])) <= 1e-12

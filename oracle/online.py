"""The online-softmax (m, l, o) recurrence and the merge of partial states, in float64.

Test infrastructure only (see the package docstring).

This is not the oracle (``attention`` is).  It spells out the algebra the
paged kernel relies on, so that the algebra itself is checked against dense
attention before it is trusted in HIP:

  [Budgets] eq. (4): for a new chunk of scores s_j,
      m' = max(m, max_j s_j),   l' = e^(m - m') l + sum_j e^(s_j - m'),
  and the weighted-value accumulator is rescaled by the same factor:
      o' = e^(m - m') o + sum_j e^(s_j - m') v_j            (reading: o unnormalised)
  [Slides] slide "分页以后，attention 仍然按完整历史归一化" and quiz
  "逻辑顺序没错…": blocks are combined through mergeable (m, l, o) state, never by
  averaging per-block softmaxes; slots past the length are masked out.

Readings:
  * Empty state: m = -inf, l = 0, o = 0.  A chunk with no valid score leaves
    the state unchanged (never evaluates -inf - (-inf)).
  * Merging states (m_p, l_p, o_p): M = max m_p, L = sum e^(m_p - M) l_p,
    O = sum e^(m_p - M) o_p; the result is O / L, or 0 when every part is empty.
"""

import math

import numpy as np

NEG_INF = -math.inf


def empty_state(d):
    return NEG_INF, 0.0, np.zeros(d, dtype=np.float64)


def update(state, scores, values, valid):
    """One step of eq. (4) over a chunk; ``valid`` masks slots past the length."""
    m, l, o = state
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    keep = np.asarray(valid, dtype=bool)
    if not keep.any():
        return state
    s = scores[keep]
    v = values[keep]
    m_new = max(m, float(s.max()))
    alpha = math.exp(m - m_new) if m != NEG_INF else 0.0
    p = np.exp(s - m_new)
    l_new = alpha * l + float(p.sum())
    o_new = alpha * o + p @ v
    return m_new, l_new, o_new


def merge(states, d):
    """Combine partial states computed over disjoint key ranges; returns o / l."""
    live = [st for st in states if st[0] != NEG_INF]
    if not live:
        return np.zeros(d, dtype=np.float64)
    M = max(st[0] for st in live)
    L = sum(math.exp(st[0] - M) * st[1] for st in live)
    O = sum(math.exp(st[0] - M) * st[2] for st in live)
    return O / L


def blockwise_attention_head(q_h, K, V, scale, n, B, splits=1):
    """One head over a contiguous history [N>=n, d], chunked into blocks of B.

    Logical blocks 0..ceil(n/B)-1 are divided into ``splits`` contiguous ranges
    of ceil(nb/splits) blocks; each range runs the recurrence from the empty
    state and the partial states are merged.  Slots at positions >= n inside a
    block are masked.  Returns out_h [d].
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = q_h.shape[0]
    nb = -(-n // B)
    per = -(-nb // splits) if nb else 0
    states = []
    for p in range(splits):
        st = empty_state(d)
        for j in range(p * per, min(nb, (p + 1) * per)):
            rows = range(j * B, j * B + B)
            valid = [t < n for t in rows]
            idx = [min(t, K.shape[0] - 1) for t in rows]
            scores = scale * (K[idx] @ q_h)
            st = update(st, scores, V[idx], valid)
        states.append(st)
    return merge(states, d)

"""Paged gather + dense softmax attention in float64: what the decode kernel computes.

Test infrastructure only (see the package docstring).

Paging changes where K/V live, not what attention reads ([Serving] §1;
[Slides] "读 token 6，先查表，再找偏移").  So the oracle first rebuilds each
request's history as a contiguous array through the block table, then runs
plain dense attention on it, which is the comparison the pages prescribe
([Slides] quiz "逻辑顺序没错，为什么 attention 输出还是错？": shuffle the
physical ids and compare against dense attention on contiguous KV).

Array conventions (any float dtype in, float64 out):
  q            [S, Hq, d]
  k_pool/v_pool [NB, B, Hkv, d]   physical block, slot, KV head, dim
                                  ([Slides] "把 token 6 变成真正的内存地址")
  block_tables [S, MB]  integer, logical block -> physical block
  seq_lens     [S]      tokens attended by each request

Readings of points the pages leave open:
  * GQA mapping: query head h reads KV head h // (Hq / Hkv) (contiguous groups).
  * A request with no tokens attends to nothing: its output is exactly 0.
  * Table entries at or beyond ceil(n / B) are never used.
"""

import numpy as np


def token_location(block_table_row, t, B):
    """(physical block, slot) of logical token t.

    Token t lies in logical block t // B at offset t % B; the table maps the
    logical block to a physical one ([Slides] "读 token 6，先查表，再找偏移",
    "把 token 6 变成真正的内存地址").  Tokens are numbered from 0.
    """
    return int(block_table_row[t // B]), t % B


def gather_sequence(pool, block_table_row, n, B):
    """Contiguous copy [n, Hkv, d] (pool dtype) of the first n tokens of one request.

    Built from an explicit per-token list of (block, slot) pairs, in logical order.
    """
    pool = np.asarray(pool)
    if n == 0:
        return pool[:0, 0]
    locs = [token_location(block_table_row, t, B) for t in range(n)]
    blocks = np.array([b for b, _ in locs], dtype=np.int64)
    slots = np.array([s for _, s in locs], dtype=np.int64)
    return pool[blocks, slots]


def dense_attention(q_s, K_s, V_s, scale):
    """Softmax attention of one new token over n contiguous history tokens.

    q_s [Hq, d]; K_s, V_s [n, Hkv, d].  For head h with KV head g = h // (Hq/Hkv):
        z_t = scale * <q_h, k_t>,  w = softmax(z),  out_h = sum_t w_t v_t.
    Subtracting max(z) before exp does not change the softmax and keeps the
    exponentials finite for large logits ([Budgets] §6 asks exactly this of
    an implementation).  n = 0 gives a zero output.
    """
    q_s = np.asarray(q_s, dtype=np.float64)
    K_s = np.asarray(K_s, dtype=np.float64)
    V_s = np.asarray(V_s, dtype=np.float64)
    Hq, d = q_s.shape
    n, Hkv = K_s.shape[0], K_s.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    out = np.zeros((Hq, d), dtype=np.float64)
    if n == 0:
        return out
    for h in range(Hq):
        g = h // group
        z = float(scale) * (K_s[:, g, :] @ q_s[h])
        z = z - z.max()
        w = np.exp(z)
        w = w / w.sum()
        out[h] = w @ V_s[:, g, :]
    return out


def paged_decode(q, k_pool, v_pool, block_tables, seq_lens, B, scale):
    """Oracle for one decode step of one layer: [S, Hq, d] float64."""
    q = np.asarray(q)
    S, Hq, d = q.shape
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        n = int(seq_lens[s])
        K_s = gather_sequence(k_pool, block_tables[s], n, B)
        V_s = gather_sequence(v_pool, block_tables[s], n, B)
        out[s] = dense_attention(q[s], K_s, V_s, scale)
    return out


def paged_decode_rows(q, k_pool, v_pool, block_tables, seq_lens, B, scale, rows):
    """Oracle output for selected requests only: {s: [Hq, d]}.

    Used at full workload sizes where the oracle computes sampled outputs.
    """
    res = {}
    for s in rows:
        n = int(seq_lens[s])
        K_s = gather_sequence(k_pool, block_tables[s], n, B)
        V_s = gather_sequence(v_pool, block_tables[s], n, B)
        res[s] = dense_attention(np.asarray(q)[s], K_s, V_s, scale)
    return res


def extend_attention(q_s, K_s, V_s, scale):
    """T new tokens of one request, each attending causally over the request's history.

    [Serving] §5 places speculative decoding beside paging: a verification
    step scores several new tokens against one history, and the same holds
    for a prompt fed in chunks.  Readings of what the pages leave open:
      * the T new tokens are already in the history (appended first, as for
        a single decode token), so they are its last T positions;
      * query i (0-based) sits at logical position n - T + i and attends
        tokens 0 .. n - T + i: itself and everything before it, nothing after
        (the causal order of a left-to-right model);
      * a query whose position would be negative (n < T) attends nothing and
        gets 0, as a request of length 0 does.
    q_s [T, Hq, d]; K_s, V_s [n, Hkv, d].  Returns [T, Hq, d] float64; each row
    is ``dense_attention`` over that query's own prefix of the history.
    """
    q_s = np.asarray(q_s)
    T = q_s.shape[0]
    n = np.asarray(K_s).shape[0]
    out = np.zeros(q_s.shape, dtype=np.float64)
    for i in range(T):
        pos = n - T + i
        if pos < 0:
            continue
        out[i] = dense_attention(q_s[i], K_s[: pos + 1], V_s[: pos + 1], scale)
    return out


def paged_extend(q, k_pool, v_pool, block_tables, seq_lens, B, scale):
    """Oracle for T query tokens per request over paged KV: [S, T, Hq, d] float64.

    q is [S, T, Hq, d]; seq_lens counts the whole history including the T
    new tokens.  Each request's history is gathered through its table, then
    ``extend_attention`` runs on it.
    """
    q = np.asarray(q)
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(q.shape[0]):
        n = int(seq_lens[s])
        K_s = gather_sequence(k_pool, block_tables[s], n, B)
        V_s = gather_sequence(v_pool, block_tables[s], n, B)
        out[s] = extend_attention(q[s], K_s, V_s, scale)
    return out


def paged_extend_rows(q, k_pool, v_pool, block_tables, seq_lens, B, scale, rows):
    """``paged_extend`` for selected requests only: {s: [T, Hq, d]}."""
    res = {}
    for s in rows:
        n = int(seq_lens[s])
        K_s = gather_sequence(k_pool, block_tables[s], n, B)
        V_s = gather_sequence(v_pool, block_tables[s], n, B)
        res[s] = extend_attention(np.asarray(q)[s], K_s, V_s, scale)
    return res

"""Pins for the multi-token (causal) attention and multi-token append oracle (CPU only).

T new tokens of a request, already appended as its last T positions, each
attend to the history up to and including themselves ([Serving] §5:
speculative verification and chunked prompts read the same paged history as
a decode step).  The pins are fixed by something other than the oracle: plain
Python loops, torch's scaled_dot_product_attention with an explicit mask or
its own causal flag, closed forms (a zero query averages exactly the values
it may see), and invariants (future tokens cannot move a result).  The last
test plants plausible mistakes in copies of the oracle and checks that a pin
catches each.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import kvcache as kvc


def rand_extend_case(seed, S, T, Hq, Hkv, d, B, lens, spare=1, poison=True):
    """Tiny paged case built by hand (independent of the workload package): q is [S, T, Hq, d]."""
    rng = np.random.default_rng(seed)
    need = [-(-n // B) for n in lens]
    MB = max(1, max(need))
    NB = sum(need) + spare
    perm = rng.permutation(NB)
    tables = np.full((S, MB), perm[-1] if spare else 0, dtype=np.int64)
    cur = 0
    for s, nb in enumerate(need):
        tables[s, :nb] = perm[cur:cur + nb]
        cur += nb
    k = rng.standard_normal((NB, B, Hkv, d))
    v = rng.standard_normal((NB, B, Hkv, d))
    if poison:
        for s, n in enumerate(lens):
            for t in range(n, need[s] * B):
                k[tables[s, t // B], t % B] = np.nan
                v[tables[s, t // B], t % B] = np.nan
        for b in perm[sum(need):]:
            k[b] = np.nan
            v[b] = np.nan
    q = rng.standard_normal((S, T, Hq, d))
    return q, k, v, tables, np.array(lens)


def brute_extend(q, k, v, tables, lens, B, scale):
    """Plain Python: query i of request s sums exp over tokens t <= n - T + i only."""
    S, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    out = np.zeros((S, T, Hq, d))
    for s in range(S):
        n = int(lens[s])
        for i in range(T):
            last = n - T + i
            for h in range(Hq):
                g = h // G
                ws, rows = [], []
                for t in range(last + 1):
                    blk, slot = int(tables[s][t // B]), t % B
                    z = scale * math.fsum(float(q[s, i, h, e]) * float(k[blk, slot, g, e]) for e in range(d))
                    ws.append(math.exp(z))
                    rows.append(v[blk, slot, g])
                if not ws:
                    continue
                tot = math.fsum(ws)
                for e in range(d):
                    out[s, i, h, e] = math.fsum(w * float(r[e]) for w, r in zip(ws, rows)) / tot
    return out


@pytest.mark.parametrize("seed,T,Hq,Hkv,d,B,lens", [
    (1, 3, 4, 2, 3, 4, [3, 4, 9, 10]),
    (2, 4, 2, 1, 4, 2, [7, 2, 0]),  # n < T: the first queries see nothing
    (3, 1, 3, 3, 2, 3, [8, 5]),
    (4, 5, 4, 1, 2, 4, [5, 13]),
])
def test_extend_matches_brute_force_tiny(seed, T, Hq, Hkv, d, B, lens):
    q, k, v, tab, n = rand_extend_case(seed, len(lens), T, Hq, Hkv, d, B, lens)
    got = att.paged_extend(q, k, v, tab, n, B, 0.6)
    want = brute_extend(q, k, v, tab, n, B, 0.6)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= 1e-14 * max(1.0, np.max(np.abs(want)))


def _dense_kv(k, v, n, B):
    NB, _, Hkv, d = k.shape
    K = torch.from_numpy(k.reshape(NB * B, Hkv, d)[:n]).permute(1, 0, 2)
    V = torch.from_numpy(v.reshape(NB * B, Hkv, d)[:n]).permute(1, 0, 2)
    return K, V


@pytest.mark.parametrize("T,n", [(5, 23), (8, 8), (16, 40)])
def test_extend_matches_library_sdpa(T, n):
    """Identity table: torch SDPA in float64 with a boolean mask (or its causal flag when T = n)."""
    rng = np.random.default_rng(11 + T)
    Hq, Hkv, d, B = 8, 2, 16, 4
    G = Hq // Hkv
    NB = -(-n // B)
    k = rng.standard_normal((NB, B, Hkv, d))
    v = rng.standard_normal((NB, B, Hkv, d))
    q = rng.standard_normal((1, T, Hq, d))
    scale = 1 / math.sqrt(d)
    got = att.paged_extend(q, k, v, [list(range(NB))], [n], B, scale)[0]  # [T, Hq, d]
    K, V = _dense_kv(k, v, n, B)
    K = K.repeat_interleave(G, dim=0).contiguous()
    V = V.repeat_interleave(G, dim=0).contiguous()
    Q = torch.from_numpy(q[0]).permute(1, 0, 2).contiguous()  # [Hq, T, d]
    if T == n:
        want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    else:
        pos = torch.arange(n - T, n).unsqueeze(1)
        mask = torch.arange(n).unsqueeze(0) <= pos  # [T, n], True = may attend
        want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    want = want.permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - want)) < 1e-13


def test_zero_query_averages_exactly_its_own_prefix():
    """q = 0: query i's output is the mean of V over positions 0 .. n-T+i, no more, no fewer."""
    q, k, v, tab, n = rand_extend_case(21, 3, 4, 4, 2, 8, 4, [4, 7, 13])
    q[:] = 0.0
    out = att.paged_extend(q, k, v, tab, n, 4, 1.0)
    for s in range(3):
        hist = att.gather_sequence(v, tab[s], int(n[s]), 4)
        for i in range(4):
            last = int(n[s]) - 4 + i
            for h in range(4):
                assert np.allclose(out[s, i, h], hist[: last + 1, h // 2].mean(axis=0), rtol=0, atol=1e-15)
    assert np.all(np.isfinite(out))


def test_future_tokens_cannot_reach_earlier_queries():
    """NaN in every position after query i's own leaves query i finite and unchanged."""
    q, k, v, tab, n = rand_extend_case(22, 2, 5, 4, 1, 8, 4, [9, 17], poison=False)
    base = att.paged_extend(q, k, v, tab, n, 4, 0.5)
    for s in range(2):
        for i in range(5):
            kk, vv = k.copy(), v.copy()
            for t in range(int(n[s]) - 5 + i + 1, int(n[s])):
                kk[tab[s][t // 4], t % 4] = np.nan
                vv[tab[s][t // 4], t % 4] = np.nan
            got = att.paged_extend(q, kk, vv, tab, n, 4, 0.5)
            assert np.array_equal(got[s, : i + 1], base[s, : i + 1])


def test_first_position_and_empty_queries():
    """n < T: queries at negative positions give exactly 0; the query at position 0 returns v_0."""
    q, k, v, tab, n = rand_extend_case(23, 2, 4, 2, 2, 8, 4, [2, 1])
    out = att.paged_extend(q, k, v, tab, n, 4, 0.9)
    for s in range(2):
        first = 4 - int(n[s])  # index of the query at position 0
        assert np.all(out[s, :first] == 0.0)
        for h in range(2):
            assert np.array_equal(out[s, first, h], v[tab[s][0], 0, h])  # G = 1: head h reads KV head h


def test_single_query_token_is_the_decode_step():
    q, k, v, tab, n = rand_extend_case(24, 3, 1, 4, 2, 8, 4, [1, 6, 12])
    got = att.paged_extend(q, k, v, tab, n, 4, 0.4)[:, 0]
    want = att.paged_decode(q[:, 0], k, v, tab, n, 4, 0.4)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- multi-token append


def test_append_tokens_crosses_a_block_boundary():
    """B = 4, table [5, 1, 7], start 3, four tokens: (5, 3), (1, 0), (1, 1), (1, 2)."""
    pool = np.zeros((8, 4, 1, 2))
    new = np.arange(1, 9, dtype=float).reshape(1, 4, 1, 2)
    out = kvc.append_tokens(pool, new, [[5, 1, 7]], [3], 4)
    assert np.array_equal(out[5, 3, 0], [1, 2])
    assert np.array_equal(out[1, 0, 0], [3, 4])
    assert np.array_equal(out[1, 1, 0], [5, 6])
    assert np.array_equal(out[1, 2, 0], [7, 8])
    assert np.count_nonzero(out) == 8
    assert np.count_nonzero(pool) == 0


def test_append_tokens_equals_repeated_single_appends_and_skips():
    rng = np.random.default_rng(5)
    pool = rng.standard_normal((10, 4, 2, 3))
    new = rng.standard_normal((3, 3, 2, 3))
    tabs = [[2, 7, 9], [4, 0, 1], [3, 5, 6]]
    pos = [2, -1, 5]
    got = kvc.append_tokens(pool, new, tabs, pos, 4)
    want = pool
    for i in range(3):
        want = kvc.append(want, new[:, i], tabs, [p + i if p >= 0 else -1 for p in pos], 4)
    assert np.array_equal(got, want)
    assert np.array_equal(got[[4, 0, 1]], pool[[4, 0, 1]])  # the skipped request's blocks


# ---------------------------------------------------------------- planted mistakes


def _extend_pins_pass(paged_extend):
    try:
        q, k, v, tab, n = rand_extend_case(1, 4, 3, 4, 2, 3, 4, [3, 4, 9, 10])
        if np.max(np.abs(paged_extend(q, k, v, tab, n, 4, 0.6) - brute_extend(q, k, v, tab, n, 4, 0.6))) > 1e-13:
            return False
        q, k, v, tab, n = rand_extend_case(21, 3, 4, 4, 2, 8, 4, [4, 7, 13])
        q[:] = 0.0
        out = paged_extend(q, k, v, tab, n, 4, 1.0)
        for s in range(3):
            hist = att.gather_sequence(v, tab[s], int(n[s]), 4)
            for i in range(4):
                if not np.allclose(out[s, i, 0], hist[: int(n[s]) - 4 + i + 1, 0].mean(axis=0), atol=1e-14):
                    return False
    except (IndexError, ValueError, FloatingPointError):
        return False
    return True


def _extend_mutant(kind):
    def paged(q, k, v, tab, n, B, scale):
        S, T = q.shape[:2]
        out = np.zeros(q.shape)
        for s in range(S):
            m = int(n[s])
            K_s = att.gather_sequence(k, tab[s], m, B)
            V_s = att.gather_sequence(v, tab[s], m, B)
            for i in range(T):
                last = {"none": m - T + i, "exclusive": m - T + i - 1, "one_ahead": min(m - 1, m - T + i + 1),
                        "reversed": m - 1 - i, "not_causal": m - 1, "from_zero": i}[kind]
                if last < 0:
                    continue
                out[s, i] = att.dense_attention(q[s, i], K_s[: last + 1], V_s[: last + 1], scale)
        return out

    return paged


def test_extend_reference_passes_and_planted_mistakes_are_caught():
    assert _extend_pins_pass(att.paged_extend)
    assert _extend_pins_pass(_extend_mutant("none"))
    for kind in ("exclusive", "one_ahead", "reversed", "not_causal", "from_zero"):
        assert not _extend_pins_pass(_extend_mutant(kind)), kind


# ---------------------------------------------------------------- sampled rows


def _extend_rows_case():
    # n < T for request 1, T = n for request 3; tails and spares poisoned
    return rand_extend_case(41, 5, 3, 4, 2, 3, 4, [10, 2, 7, 3, 13], spare=2), [4, 1, 3, 0]


def test_extend_rows_match_brute_force_and_full_oracle():
    """paged_extend_rows is the reference for the sampled requests of large
    several-token batches: each row equals the brute force, and bit for bit
    the full oracle's row."""
    (q, k, v, tab, n), rows = _extend_rows_case()
    got = att.paged_extend_rows(q, k, v, tab, n, 4, 0.6, rows)
    assert sorted(got) == sorted(rows)
    want = brute_extend(q, k, v, tab, n, 4, 0.6)
    full = att.paged_extend(q, k, v, tab, n, 4, 0.6)
    for s in rows:
        assert np.all(np.isfinite(got[s]))
        assert np.max(np.abs(got[s] - want[s])) <= 1e-14 * max(1.0, np.max(np.abs(want[s])))
        assert np.array_equal(got[s], full[s])
    assert np.array_equal(got[1][0], np.zeros_like(got[1][0]))  # position -1 attends nothing


def _extend_rows_pins_pass(rows_fn):
    (q, k, v, tab, n), rows = _extend_rows_case()
    try:
        got = rows_fn(q, k, v, tab, n, 4, 0.6, rows)
    except (IndexError, ValueError):
        return False
    want = brute_extend(q, k, v, tab, n, 4, 0.6)
    return sorted(got) == sorted(rows) and all(
        np.all(np.isfinite(got[s])) and np.max(np.abs(got[s] - want[s])) <= 1e-13 for s in rows)


def _extend_rows_mutant(kind):
    def rows_fn(q, k, v, tab, lens, B, scale, rows):
        res = {}
        for i, s in enumerate(rows):
            qs = q[i] if kind == "q_by_position" else q[s]
            row = tab[(s + 1) % len(lens)] if kind == "table_of_next" else tab[s]
            m = int(lens[rows[0]]) if kind == "length_of_first" else int(lens[s])
            K_s = att.gather_sequence(k, row, m, B)
            V_s = att.gather_sequence(v, row, m, B)
            res[s] = att.extend_attention(qs, K_s, V_s, scale)
        return res

    return rows_fn


def test_extend_rows_planted_mistakes_are_caught():
    assert _extend_rows_pins_pass(att.paged_extend_rows)
    assert _extend_rows_pins_pass(_extend_rows_mutant("none"))
    for kind in ("q_by_position", "table_of_next", "length_of_first"):
        assert not _extend_rows_pins_pass(_extend_rows_mutant(kind)), kind

"""Pins for the attention, online-softmax and KV-cache oracle (CPU only).

Each pin is fixed by something other than the oracle itself: a worked example
the pages print, a brute-force sum in plain Python, a library routine on a
special case, a closed form, or an invariant.  The last test plants plausible
mistakes in copies of the oracle and checks that some pin catches each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import kvcache as kvc
from oracle import online

with open(os.path.join(os.path.dirname(__file__), "golden", "pages_accounting.json")) as _f:
    GOLD = json.load(_f)


def rand_case(seed, S, Hq, Hkv, d, B, lens, spare=1, q_scale=1.0, poison=True):
    """Tiny paged case built by hand here (independent of the workload package)."""
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
    q = rng.standard_normal((S, Hq, d)) * q_scale
    return q, k, v, tables, np.array(lens)


def brute_attention(q, k, v, tables, lens, B, scale):
    """Pure-Python loops: exp and fsum, no max subtraction, no numpy arithmetic."""
    S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(S)]
    for s in range(S):
        n = int(lens[s])
        for h in range(Hq):
            g = h // G
            ws = []
            rows = []
            for t in range(n):
                blk = int(tables[s][t // B])
                slot = t % B
                z = scale * math.fsum(float(q[s, h, e]) * float(k[blk, slot, g, e]) for e in range(d))
                ws.append(math.exp(z))
                rows.append(v[blk, slot, g])
            tot = math.fsum(ws)
            for e in range(d):
                out[s][h][e] = math.fsum(w * float(r[e]) for w, r in zip(ws, rows)) / tot if n else 0.0
    return np.array(out)


# ---------------------------------------------------------------- addressing


def test_token6_address_example():
    g = GOLD["token6_address"]
    blk, slot = att.token_location(g["table"], g["token"], g["B"])
    assert g["token"] // g["B"] == g["expect_logical_block"]
    assert (blk, slot) == (g["expect_physical"], g["expect_slot"])


def test_identity_table_gather_is_contiguous_history():
    rng = np.random.default_rng(1)
    B, NB, Hkv, d = 4, 5, 2, 3
    pool = rng.standard_normal((NB, B, Hkv, d))
    flat = pool.reshape(NB * B, Hkv, d)
    for n in (0, 1, 4, 5, 19, 20):
        got = att.gather_sequence(pool, list(range(NB)), n, B)
        assert np.array_equal(got, flat[:n])


def test_gather_follows_shuffled_table():
    rng = np.random.default_rng(2)
    B, NB = 4, 6
    pool = rng.standard_normal((NB, B, 1, 2))
    table = [5, 1, 3]
    got = att.gather_sequence(pool, table, 10, B)
    want = np.concatenate([pool[5], pool[1], pool[3][:2]])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- dense attention


@pytest.mark.parametrize("seed,Hq,Hkv,d,B,lens", [
    (3, 4, 2, 3, 4, [1, 4, 5, 9]),
    (4, 2, 1, 4, 2, [3, 7, 0]),
    (5, 3, 3, 2, 3, [8, 6]),
])
def test_matches_brute_force_tiny(seed, Hq, Hkv, d, B, lens):
    q, k, v, tab, n = rand_case(seed, len(lens), Hq, Hkv, d, B, lens)
    scale = 0.7
    got = att.paged_decode(q, k, v, tab, n, B, scale)
    want = brute_attention(q, k, v, tab, n, B, scale)
    assert np.max(np.abs(got - want)) <= 1e-15 * max(1.0, np.max(np.abs(want))) * 8


def test_matches_library_sdpa_identity_table():
    """Special case: identity table, no poison; torch SDPA in float64 with K/V repeated per group."""
    rng = np.random.default_rng(6)
    Hq, Hkv, d, B, n = 8, 2, 16, 4, 23
    G = Hq // Hkv
    NB = -(-n // B)
    k = rng.standard_normal((NB, B, Hkv, d))
    v = rng.standard_normal((NB, B, Hkv, d))
    q = rng.standard_normal((1, Hq, d))
    scale = 1 / math.sqrt(d)
    got = att.paged_decode(q, k, v, [list(range(NB))], [n], B, scale)[0]
    K = torch.from_numpy(k.reshape(NB * B, Hkv, d)[:n]).permute(1, 0, 2)  # [Hkv, n, d]
    V = torch.from_numpy(v.reshape(NB * B, Hkv, d)[:n]).permute(1, 0, 2)
    K = K.repeat_interleave(G, dim=0).contiguous()
    V = V.repeat_interleave(G, dim=0).contiguous()
    Q = torch.from_numpy(q[0]).unsqueeze(1)  # [Hq, 1, d]
    want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0].numpy()
    assert np.max(np.abs(got - want)) < 1e-13


def test_single_token_returns_its_value_exactly():
    q, k, v, tab, n = rand_case(7, 3, 4, 2, 8, 4, [1, 1, 1])
    out = att.paged_decode(q, k, v, tab, n, 4, 0.3)
    for s in range(3):
        blk = tab[s][0]
        for h in range(4):
            assert np.array_equal(out[s, h], v[blk, 0, h // 2])


def test_zero_query_gives_mean_of_valid_values():
    """q = 0 weights every valid token equally; NaN-poisoned tails would leak into the mean."""
    q, k, v, tab, n = rand_case(8, 4, 4, 2, 8, 4, [3, 4, 5, 13])
    q[:] = 0.0
    out = att.paged_decode(q, k, v, tab, n, 4, 1.0)
    for s in range(4):
        hist = att.gather_sequence(v, tab[s], int(n[s]), 4)
        for h in range(4):
            assert np.allclose(out[s, h], hist[:, h // 2].mean(axis=0), rtol=0, atol=1e-15)
    assert np.all(np.isfinite(out))


def test_identical_keys_give_mean_of_values():
    q, k, v, tab, n = rand_case(9, 1, 2, 1, 4, 4, [7])
    for t in range(7):
        k[tab[0][t // 4], t % 4] = k[tab[0][0], 0]
    out = att.paged_decode(q, k, v, tab, n, 4, 1.0)
    hist = att.gather_sequence(v, tab[0], 7, 4)
    assert np.allclose(out[0], hist[:, 0].mean(axis=0)[None, :], atol=1e-15)


def test_gqa_group_mapping():
    """KV head g holds the constant value g+1 everywhere: head h must read h // (Hq/Hkv)."""
    q, k, v, tab, n = rand_case(10, 2, 8, 4, 4, 4, [5, 9])
    for g in range(4):
        v[..., g, :] = g + 1.0
    out = att.paged_decode(q, k, v, tab, n, 4, 1.0)
    for h in range(8):
        assert np.allclose(out[:, h], h // 2 + 1.0, atol=1e-14)


def test_logit_shift_invariance():
    """An extra dimension with q = c/scale and k = 1 shifts every logit by c: output unchanged."""
    q, k, v, tab, n = rand_case(11, 3, 4, 2, 6, 4, [4, 9, 16], poison=False)
    scale = 0.5
    base = att.paged_decode(q, k, v, tab, n, 4, scale)
    c = 37.0
    q2 = np.concatenate([q, np.full(q.shape[:2] + (1,), c / scale)], axis=2)
    k2 = np.concatenate([k, np.ones(k.shape[:3] + (1,))], axis=3)
    v2 = np.concatenate([v, np.zeros(v.shape[:3] + (1,))], axis=3)
    shifted = att.paged_decode(q2, k2, v2, tab, n, 4, scale)[..., :6]
    assert np.max(np.abs(shifted - base)) < 1e-14


def test_physical_permutation_gives_identical_output():
    q, k, v, tab, n = rand_case(12, 3, 4, 2, 8, 4, [6, 11, 16])
    base = att.paged_decode(q, k, v, tab, n, 4, 0.4)
    rng = np.random.default_rng(99)
    NB = k.shape[0]
    perm = rng.permutation(NB)            # new id of old block b is perm[b]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    tab2 = perm[np.asarray(tab)]
    again = att.paged_decode(q, k2, v2, tab2, n, 4, 0.4)
    assert np.array_equal(base, again)


def test_large_logits_stay_finite_and_shift_invariant():
    """Logits near +-100: exp(z) alone overflows float32 past ~88.7; the oracle must not."""
    q, k, v, tab, n = rand_case(13, 2, 4, 2, 32, 16, [40, 77], q_scale=40.0)
    scale = 1 / math.sqrt(32)
    out = att.paged_decode(q, k, v, tab, n, 16, scale)
    assert np.all(np.isfinite(out))
    zmax = max(float(np.max(np.abs(scale * (att.gather_sequence(k, tab[s], int(n[s]), 16)[:, h // 2] @ q[s, h]))))
               for s in range(2) for h in range(4))
    assert zmax > 89  # past float32 exp overflow
    # binary64 exp does not overflow here, so the unshifted brute force is exact enough
    want = brute_attention(q / 4, k * 4, v, tab, n, 16, scale)  # same logits, different factoring
    assert np.max(np.abs(out - want)) < 1e-12


def test_edge_lengths():
    B = 4
    lens = [0, 1, B, B + 1, 3 * B]
    q, k, v, tab, n = rand_case(14, len(lens), 2, 1, 3, B, lens)
    out = att.paged_decode(q, k, v, tab, n, B, 0.9)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.all(np.isfinite(out))
    want = brute_attention(q, k, v, tab, n, B, 0.9)
    assert np.max(np.abs(out - want)) < 1e-14


# ---------------------------------------------------------------- online recurrence


@pytest.mark.parametrize("B,splits", [(1, 1), (4, 1), (4, 3), (16, 5), (3, 7)])
def test_online_recurrence_matches_dense(B, splits):
    rng = np.random.default_rng(20 + B + splits)
    d, n = 8, 29
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    want = att.dense_attention(q[None], K[:, None], V[:, None], 0.6)[0]
    got = online.blockwise_attention_head(q, K, V, 0.6, n, B, splits)
    # the page's own binary64 check reports a largest error of one ulp of 1
    assert np.max(np.abs(got - want)) <= 8 * GOLD["online_vs_dense_witness"]["largest_absolute_error"]


def test_online_empty_splits_and_length_zero():
    rng = np.random.default_rng(30)
    d = 4
    q, K, V = rng.standard_normal(d), rng.standard_normal((5, d)), rng.standard_normal((5, d))
    # more splits than blocks: trailing splits are empty and must be identities
    got = online.blockwise_attention_head(q, K, V, 1.0, 5, 4, splits=6)
    want = att.dense_attention(q[None], K[:, None], V[:, None], 1.0)[0]
    assert np.max(np.abs(got - want)) < 1e-15
    assert np.array_equal(online.blockwise_attention_head(q, K, V, 1.0, 0, 4, 3), np.zeros(d))
    st = online.empty_state(d)
    assert online.update(st, [1.0, 2.0], np.ones((2, d)), [False, False]) is st


def test_online_large_logits():
    rng = np.random.default_rng(31)
    d, n = 16, 50
    q = rng.standard_normal(d) * 30
    K = rng.standard_normal((n, d)) * 3
    V = rng.standard_normal((n, d))
    got = online.blockwise_attention_head(q, K, V, 1.0, n, 16, 3)
    want = att.dense_attention(q[None], K[:, None], V[:, None], 1.0)[0]
    assert np.all(np.isfinite(got)) and np.max(np.abs(got - want)) < 1e-13


# ---------------------------------------------------------------- append / COW


def test_append_token6_example():
    B = 4
    pool = np.zeros((8, B, 1, 2), dtype=np.uint16)
    new = np.array([[[7, 9]]], dtype=np.uint16)
    out = kvc.append(pool, new, [[5, 1, 7]], [6], B)
    changed = np.argwhere(out != pool)
    assert {(int(a), int(b)) for a, b, *_ in changed} == {(1, 2)}
    assert np.array_equal(out[1, 2], new[0])
    assert np.array_equal(pool, np.zeros_like(pool))  # input untouched


def test_append_skip_and_new_block():
    B = 4
    pool = np.arange(6 * B * 2 * 3, dtype=np.uint16).reshape(6, B, 2, 3)
    new = np.full((3, 2, 3), 60000, dtype=np.uint16)
    tables = [[2, 4], [1, 5], [0, 3]]
    out = kvc.append(pool, new, tables, [4, -1, 3], B)  # first write into a fresh block, a skip, a tail fill
    assert np.array_equal(out[4, 0], new[0]) and np.array_equal(out[0, 3], new[2])
    mask = np.ones(pool.shape[:2], bool)
    mask[4, 0] = mask[0, 3] = False
    assert np.array_equal(out[mask], pool[mask])


def test_cow_isolation_protocol():
    """Two branches share a tail with 3 valid slots; each copies then writes its own token."""
    B = 4
    rng = np.random.default_rng(40)
    pool = rng.integers(0, 65535, size=(6, B, 2, 3), dtype=np.uint16)
    pool[2, 3] = 0xFFFF  # unwritten slot of the shared tail
    shared = pool[2].copy()
    # branch A copies into block 3, branch B keeps the original (its refcount falls to 1)
    after = kvc.cow_copy(pool, [2], [3], [3])
    assert np.array_equal(after[3, :3], shared[:3])
    assert np.array_equal(after[3, 3], pool[3, 3])            # slot >= n_valid untouched
    mask = np.ones(6, bool)
    mask[3] = False
    assert np.array_equal(after[mask], pool[mask])            # every other block untouched
    X = np.full((2, 3), 111, np.uint16)
    Y = np.full((2, 3), 222, np.uint16)
    after = kvc.append(after, np.stack([X, Y]), [[0, 3], [0, 2]], [7, 7], B)
    assert np.array_equal(after[3, 3], X) and np.array_equal(after[2, 3], Y)
    assert np.array_equal(after[2, :3], shared[:3]) and np.array_equal(after[3, :3], shared[:3])


def test_cow_layers_copies_every_layer():
    rng = np.random.default_rng(41)
    pools = rng.integers(0, 65535, size=(3, 5, 4, 1, 2), dtype=np.uint16)
    out = kvc.cow_copy_layers(pools, [0, 1], [2, 3], [2, 4])
    for layer in range(3):
        assert np.array_equal(out[layer, 2, :2], pools[layer, 0, :2])
        assert np.array_equal(out[layer, 3], pools[layer, 1])
        assert np.array_equal(out[layer, 2, 2:], pools[layer, 2, 2:])


def test_gather_padded_matches_gather_sequence():
    q, k, v, tab, n = rand_case(42, 3, 2, 1, 2, 4, [0, 5, 8])
    g = kvc.gather_padded(k, tab, n, 4, fill=-7.0)
    for s in range(3):
        m = int(n[s])
        assert np.array_equal(g[s, :m], att.gather_sequence(k, tab[s], m, 4), equal_nan=True)
        assert np.all(g[s, m:] == -7.0)


# ---------------------------------------------------------------- planted mistakes


def _pins_pass(paged_decode):
    """Re-run a subset of the pins above against a candidate implementation."""
    try:
        q, k, v, tab, n = rand_case(3, 4, 4, 2, 3, 4, [1, 4, 5, 9])
        if np.max(np.abs(paged_decode(q, k, v, tab, n, 4, 0.7) - brute_attention(q, k, v, tab, n, 4, 0.7))) > 1e-13:
            return False
        q, k, v, tab, n = rand_case(10, 2, 8, 4, 4, 4, [5, 9])
        for g in range(4):
            v[..., g, :] = g + 1.0
        out = paged_decode(q, k, v, tab, n, 4, 1.0)
        if not all(np.allclose(out[:, h], h // 2 + 1.0) for h in range(8)):
            return False
        q, k, v, tab, n = rand_case(13, 2, 4, 2, 32, 16, [40, 77], q_scale=40.0)
        if not np.all(np.isfinite(paged_decode(q, k, v, tab, n, 16, 1 / math.sqrt(32)))):
            return False
    except (IndexError, ValueError, FloatingPointError):
        return False
    return True


def _mutant(kind):
    def loc(row, t, B):
        if kind == "slot_swap":
            return int(row[t % B]), t // B
        if kind == "off_by_one":
            return int(row[(t + 1) // B]), (t + 1) % B
        return int(row[t // B]), t % B

    def dense(q_s, K_s, V_s, scale):
        Hq, d = q_s.shape
        Hkv = K_s.shape[1]
        G = Hq // Hkv
        out = np.zeros((Hq, d))
        if K_s.shape[0] == 0:
            return out
        for h in range(Hq):
            g = h % Hkv if kind == "gqa_modulo" else h // G
            sc = 1.0 if kind == "no_scale" else scale
            z = sc * (K_s[:, g, :] @ q_s[h])
            if kind != "no_max_shift":
                z = z - z.max()
            with np.errstate(over="ignore", invalid="ignore"):
                w = np.exp(z.astype(np.float32) if kind == "no_max_shift" else z)
                w = w / w.sum()
            if kind == "transposed_pv":
                out[h] = (V_s[:, g, :].T @ w[:d])[:d] if w.shape[0] >= d else np.zeros(d)
            else:
                out[h] = w @ V_s[:, g, :]
        return out

    def paged(q, k, v, tab, n, B, scale):
        S, Hq, d = q.shape
        o = np.zeros((S, Hq, d))
        for s in range(S):
            m = int(n[s])
            locs = [loc(tab[s], t, B) for t in range(m)]
            Ks = np.array([k[b, sl] for b, sl in locs]).reshape(m, k.shape[2], k.shape[3])
            Vs = np.array([v[b, sl] for b, sl in locs]).reshape(m, v.shape[2], v.shape[3])
            o[s] = dense(q[s], Ks, Vs, scale)
        return o

    return paged


def test_reference_mutant_passes_and_planted_mistakes_are_caught():
    assert _pins_pass(att.paged_decode)
    assert _pins_pass(_mutant("none"))
    for kind in ("slot_swap", "off_by_one", "gqa_modulo", "no_scale", "no_max_shift", "transposed_pv"):
        assert not _pins_pass(_mutant(kind)), kind


def test_swap_round_trip_and_isolation():
    """swap_out then swap_in into other ids copies exactly those blocks, in every layer."""
    rng = np.random.default_rng(9)
    k = rng.standard_normal((2, 6, 4, 1, 2))
    v = rng.standard_normal((2, 6, 4, 1, 2))
    buf = kvc.swap_out(k, v, [4, 1])
    assert buf.shape == (2, 2, 2, 4, 1, 2)
    assert np.array_equal(buf[1, 0, 0], k[1, 4]) and np.array_equal(buf[0, 1, 1], v[0, 1])
    k2, v2 = kvc.swap_in(k, v, [0, 5], buf)
    assert np.array_equal(k2[:, 0], k[:, 4]) and np.array_equal(v2[:, 5], v[:, 1])
    assert np.array_equal(k2[:, 1:5], k[:, 1:5]) and np.array_equal(v2[:, 1:5], v[:, 1:5])


# ---------------------------------------------------------------- sampled rows


def _rows_case():
    # five requests with distinct lengths (one empty, one of a single token),
    # NaN-poisoned tails and spare blocks, asked for out of order
    return rand_case(31, 5, 4, 2, 3, 4, [9, 0, 5, 1, 12], spare=2), [4, 0, 2, 1]


def test_decode_rows_match_brute_force_and_full_oracle():
    """paged_decode_rows is the reference for the sampled requests of large batches.

    Each returned row equals the brute-force sum for that request, and is bit
    for bit the full oracle's row for the same request.
    """
    (q, k, v, tab, n), rows = _rows_case()
    got = att.paged_decode_rows(q, k, v, tab, n, 4, 0.7, rows)
    assert sorted(got) == sorted(rows)
    want = brute_attention(q, k, v, tab, n, 4, 0.7)
    full = att.paged_decode(q, k, v, tab, n, 4, 0.7)
    for s in rows:
        assert np.all(np.isfinite(got[s]))
        assert np.max(np.abs(got[s] - want[s])) <= 1e-14 * max(1.0, np.max(np.abs(want[s])))
        assert np.array_equal(got[s], full[s])
    assert np.array_equal(got[1], np.zeros_like(got[1]))  # length 0


def _rows_pins_pass(rows_fn):
    (q, k, v, tab, n), rows = _rows_case()
    try:
        got = rows_fn(q, k, v, tab, n, 4, 0.7, rows)
    except (IndexError, ValueError):
        return False
    want = brute_attention(q, k, v, tab, n, 4, 0.7)
    return sorted(got) == sorted(rows) and all(
        np.all(np.isfinite(got[s])) and np.max(np.abs(got[s] - want[s])) <= 1e-13 for s in rows)


def _rows_mutant(kind):
    """Copies of the sampled-row wrapper with one plausible indexing slip each."""
    def rows_fn(q, k, v, tab, lens, B, scale, rows):
        res = {}
        for i, s in enumerate(rows):
            qs = q[i] if kind == "q_by_position" else q[s]
            row = tab[(s + 1) % len(lens)] if kind == "table_of_next" else tab[s]
            m = int(lens[rows[0]]) if kind == "length_of_first" else int(lens[s])
            K_s = att.gather_sequence(k, row, m, B)
            V_s = att.gather_sequence(v, row, m, B)
            res[s] = att.dense_attention(qs, K_s, V_s, scale)
        return res

    return rows_fn


def test_decode_rows_planted_mistakes_are_caught():
    assert _rows_pins_pass(att.paged_decode_rows)
    assert _rows_pins_pass(_rows_mutant("none"))
    for kind in ("q_by_position", "table_of_next", "length_of_first"):
        assert not _rows_pins_pass(_rows_mutant(kind)), kind

"""Accounting oracle pinned to every figure the pages print (tests/golden/pages_accounting.json)."""

import json
import os
from fractions import Fraction

import pytest

from oracle import accounting as acc

with open(os.path.join(os.path.dirname(__file__), "golden", "pages_accounting.json")) as _f:
    GOLD = json.load(_f)


def pct2(fr):
    return f"{float(fr) * 100:.2f}"


def test_bytes_per_token_teaching_model():
    g = GOLD["bytes_per_token_teaching_model"]
    b = acc.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert b == g["expect_bytes"]
    assert b == g["expect_kib"] * acc.KiB


def test_request_4096_tokens():
    g = GOLD["request_4096_tokens"]
    for kv_heads, gib in g["kv_heads_cases"]:
        b = acc.kv_bytes(g["layers"], g["tokens"], kv_heads, g["head_dim"], g["elem_bytes"])
        assert Fraction(b, acc.GiB) == Fraction(gib)


def test_five_sequences():
    g = GOLD["five_sequences"]
    L = g["lengths"]
    assert sum(L) == g["useful"]
    assert acc.fixed_reservation_slots(L, 512) == g["fixed_512_slots"]
    assert sum(acc.allocated_slots(n, 16) for n in L) == g["B16_slots"]
    assert sum(acc.allocated_slots(n, 32) for n in L) == g["B32_slots"]
    u = g["utilisation_percent_2dp"]
    assert pct2(Fraction(g["useful"], acc.fixed_reservation_slots(L, 512))) == u["fixed_512"]
    assert pct2(acc.utilisation(L, 16)) == u["B16"]
    assert pct2(acc.utilisation(L, 32)) == u["B32"]


def test_pool_24gib():
    g = GOLD["pool_24gib"]
    blocks = acc.pool_blocks(g["pool_gib"] * acc.GiB, g["B"], g["bytes_per_token"])
    assert blocks == g["expect_blocks"]
    assert g["requests"] * g["blocks_per_request"] == g["blocks_used_by_47"]
    fit, left = acc.requests_that_fit(blocks, g["blocks_per_request"])
    assert fit == g["requests"] and left == g["blocks_left"]
    assert g["blocks_per_request"] - left == g["short_for_48th"]
    # any length needing 257 blocks of 16 tokens (the page does not state it)
    assert acc.blocks_for(4097, 16) == 257 and acc.blocks_for(4112, 16) == 257


def test_pool_8gib_quiz():
    g = GOLD["pool_8gib_quiz"]
    bpt = acc.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert bpt == g["expect_bytes_per_token"]
    assert g["B"] * bpt == g["expect_block_kib"] * acc.KiB
    pool = g["pool_gib"] * acc.GiB
    blocks = acc.pool_blocks(pool, g["B"], bpt)
    assert blocks == g["expect_blocks"]
    per = acc.blocks_for(g["request_tokens"], g["B"])
    assert per == g["expect_blocks_per_request"]
    assert acc.requests_that_fit(blocks, per) == (g["expect_requests"], g["expect_blocks_left"])
    assert acc.pool_leftover_bytes(pool, g["B"], bpt) == g["expect_leftover_kib"] * acc.KiB


def test_tail_waste_table_B16():
    g = GOLD["tail_waste_table_B16"]
    B = g["B"]
    for n, blocks, slots, empty in g["rows"]:
        assert (acc.blocks_for(n, B), acc.allocated_slots(n, B), acc.tail_waste(n, B)) == (blocks, slots, empty)
    lens = [r[0] for r in g["rows"]]
    tot = [sum(lens), sum(acc.blocks_for(n, B) for n in lens),
           sum(acc.allocated_slots(n, B) for n in lens), acc.total_tail_waste(lens, B)]
    assert tot == g["total"]


def test_block_size_table_and_lab_output():
    g = GOLD["block_size_table"]
    for B_s, col in g["columns"].items():
        B = int(B_s)
        lens = g["lengths"]
        assert sum(acc.blocks_for(n, B) for n in lens) == col["blocks"]
        assert sum(acc.allocated_slots(n, B) for n in lens) == col["slots"]
        empty = acc.total_tail_waste(lens, B)
        assert empty == col["empty"]
        assert Fraction(empty * g["bytes_per_token"], acc.MiB) == Fraction(col["empty_mib"]).limit_denominator()
        assert empty <= acc.tail_waste_bound(lens, B)
    lab = GOLD["lab_output"]
    lens = g["lengths"]
    assert sum(acc.blocks_for(n, 16) for n in lens) == lab["B16"]["blocks"]
    assert sum(acc.allocated_slots(n, 16) for n in lens) == lab["B16"]["slots"]
    assert sum(lens) == lab["B16"]["useful"]
    assert acc.total_tail_waste(lens, 16) == lab["B16"]["tail_waste"]
    assert sum(acc.blocks_for(n, 4) for n in lens) == lab["B4"]["blocks"]
    assert acc.total_tail_waste(lens, 4) == lab["B4"]["tail_waste"]


def test_length10_B4():
    g = GOLD["length10_B4"]
    assert acc.blocks_for(g["n"], g["B"]) == g["expect_blocks"]
    assert acc.allocated_slots(g["n"], g["B"]) == g["expect_slots"]
    assert acc.tail_waste(g["n"], g["B"]) == g["expect_tail_empty"]


def test_mean_tail_waste():
    g = GOLD["mean_tail_waste"]
    assert acc.mean_fixed_reservation_waste(g["max_len"]) == Fraction(g["fixed_reservation_mean"])
    for B in g["page_sizes"]:
        # enumeration over [1, 512] equals the closed form (B-1)/2
        assert acc.mean_tail_waste_uniform(B, g["max_len"] // B) == Fraction(B - 1, 2)


def test_decode_read_volume():
    g = GOLD["decode_read_volume"]
    total = g["requests"] * g["history"] * g["bytes_per_token"]
    assert total == g["expect_gib_all_layers"] * acc.GiB
    assert total // g["layers"] == g["expect_mib_per_layer"] * acc.MiB


def test_tail_waste_bound_and_edge_cases():
    assert acc.blocks_for(0, 16) == 0 and acc.tail_waste(0, 16) == 0
    for B in (1, 4, 16, 64):
        for n in range(1, 200):
            w = acc.tail_waste(n, B)
            assert 0 <= w <= B - 1
    with pytest.raises(ValueError):
        acc.blocks_for(-1, 16)


def _bound_pins_pass(bound):
    """The tail-waste bound of [Budgets] eq. (2) is N(B-1) over the N non-empty
    requests.  Pinned by what the inequality must satisfy: it holds for every
    length list, it is attained (the largest total tail waste over all lists
    with the same number of empty and non-empty requests equals it, found here
    by exhaustive enumeration), and empty requests add nothing."""
    from itertools import product

    for B in (1, 2, 3, 4):
        for S in (1, 2, 3):
            by_zeros = {}
            for lens in product(range(0, 2 * B + 2), repeat=S):
                w = acc.total_tail_waste(lens, B)
                b = bound(list(lens), B)
                if w > b:
                    return False
                z = sum(1 for n in lens if n == 0)
                by_zeros.setdefault(z, []).append((w, b))
            for z, pairs in by_zeros.items():
                bs = {b for _, b in pairs}
                if len(bs) != 1 or max(w for w, _ in pairs) != bs.pop():
                    return False
    # lengths all one past a block boundary attain it exactly; empty requests are not counted
    for B in (16, 64):
        lens = [1 + B * j for j in range(7)] + [0, 0, 0]
        if not (acc.total_tail_waste(lens, B) == 7 * (B - 1) == bound(lens, B)):
            return False
    return bound([0, 0], 16) == 0


def test_tail_waste_bound_is_attained_and_skips_empty_requests():
    assert _bound_pins_pass(acc.tail_waste_bound)


def test_tail_waste_bound_planted_mistakes_are_caught():
    mutants = {
        "counts_empty": lambda lens, B: len(lens) * (B - 1),
        "N_times_B": lambda lens, B: sum(1 for n in lens if n > 0) * B,
        "B_minus_one_total": lambda lens, B: (B - 1) if any(lens) else 0,
        "ceil_of_sum": lambda lens, B: acc.tail_waste(sum(lens), B),
    }
    for kind, fn in mutants.items():
        assert not _bound_pins_pass(fn), kind

"""The seeded workload generators build the batches their descriptions promise (CPU)."""

import numpy as np
import pytest
import torch

from oracle import accounting as acc
from oracle import attention as att
from oracle import kvcache as kvc
import workloads as W


def _blocks_used(b):
    return sum(acc.blocks_for(int(n), b.B) for n in b.seq_lens.tolist())


def _check_tables(b):
    tab = b.block_tables.numpy()
    lens = b.seq_lens.numpy()
    owned = []
    for s in range(b.S):
        nb = acc.blocks_for(int(lens[s]), b.B)
        owned += tab[s, :nb].tolist()
        if b.spare_block >= 0:
            assert np.all(tab[s, nb:] == b.spare_block)
    assert np.all((tab >= 0) & (tab < b.NB))
    return owned


def test_config1_shape_and_poison():
    b = W.config1()
    assert b.k_pool.shape == (1, 64, 16, 2, 128) and b.dtype == torch.float32
    assert b.seq_lens.tolist() == [37, 91, 128, 201, 511]
    owned = _check_tables(b)
    assert len(owned) == len(set(owned)) == 62 == _blocks_used(b)
    # valid history finite, everything else NaN
    for s in range(b.S):
        n = int(b.seq_lens[s])
        hist = att.gather_sequence(b.k_pool[0].numpy(), b.block_tables[s].numpy(), n, 16)
        assert np.all(np.isfinite(hist))
        nb = acc.blocks_for(n, 16)
        last = int(b.block_tables[s, nb - 1])
        assert torch.isnan(b.k_pool[0, last, n - (nb - 1) * 16:]).all()
    assert torch.isnan(b.k_pool[0, b.spare_block]).all()
    assert b.rounds == 0 and b.cow_src.numel() == 0


def test_config1_is_seeded():
    a, b = W.config1(), W.config1()
    assert torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.q, b.q) and torch.equal(a.k_pool.nan_to_num(), b.k_pool.nan_to_num())


def test_config3_lengths_and_layout():
    _, h = W.decode.config3_lengths()
    assert h[:4].tolist() == [0, 1, 16, 17]
    assert len(h) == 256 and h[4:].min() >= 1 and h[4:].max() <= 512
    b = W.config3(layers=1)
    assert b.NB == 12288 and b.MB == 33
    assert np.array_equal(b.seq_lens.numpy(), h + 1)
    assert np.array_equal(b.append_positions[0].numpy(), h)
    owned = _check_tables(b)
    assert len(owned) == len(set(owned))
    # the append slot is unwritten before the step
    for s in range(4):
        pos = int(h[s])
        blk = int(b.block_tables[s, pos // 16])
        assert torch.isnan(b.k_pool[0, blk, pos % 16]).all()
    # 24 GiB over 32 layers at 128 KiB/token: 384 MiB per K (or V) pool per layer
    per_layer = b.k_pool[0].numel() * 2
    assert per_layer * 2 * 32 == 24 * acc.GiB


def test_config4_cow_structure():
    b = W.config4()
    t = b.info["t"]
    c = np.array(b.info["c"])
    assert 1 <= t <= 15 and c.min() >= 1 and c.max() <= 64
    assert b.cow_src.numel() == 63 and len(set(b.cow_dst.tolist())) == 63
    assert set(b.cow_src.tolist()) == {b.info["shared_tail"]}
    assert np.all(b.cow_n.numpy() == t)
    tab = b.block_tables.numpy()
    assert np.all(tab[:, :128] == tab[0, :128])                      # shared prefix, refcount 64
    assert tab[63, 128] == b.info["shared_tail"]                     # last branch writes in place
    assert np.array_equal(b.seq_lens.numpy(), 2048 + t + c)
    assert b.MB <= 133
    # q scaled by 20
    assert 10 < float(b.q.float().std()) < 30
    # replaying COW + rounds in the oracle leaves no NaN inside any attended history
    k = b.k_pool[0].view(torch.int16).numpy()
    k = kvc.cow_copy(k, b.cow_src.numpy(), b.cow_dst.numpy(), b.cow_n.numpy())
    for r in range(b.rounds):
        k = kvc.append(k, b.k_new[r, 0].view(torch.int16).numpy(), tab, b.append_positions[r].numpy(), 16)
    kf = torch.from_numpy(k).view(torch.bfloat16).float().numpy()
    for s in range(b.S):
        assert np.all(np.isfinite(att.gather_sequence(kf, tab[s], int(b.seq_lens[s]), 16)))


@pytest.mark.parametrize("t", [1, 15])
def test_config4_forced_tail_fill(t):
    b = W.config4(t=t)
    assert b.info["t"] == t and np.all(b.cow_n.numpy() == t)


def test_config5_pool_matches_quiz():
    b = W.config5(layers=1)
    assert b.NB == 10922 and b.MB == 65 and b.S == 168
    assert _blocks_used(b) == 168 * 65 == 10920
    assert np.all(b.append_positions[0].numpy() == 1024)
    assert np.all(b.seq_lens.numpy() == 1025)
    owned = _check_tables(b)
    assert len(set(owned)) == 10920


def test_config2_fills_pool():
    b = W.config2(S=2, n=64)  # same construction at a small size
    assert b.NB == 8 and _blocks_used(b) == 8 and b.spare_block == -1
    assert b.dtype == torch.bfloat16 and b.Hq == 32 and b.Hkv == 8


def test_custom_append_round():
    b = W.custom([0, 1, 5, 16, 17], append=True)
    assert b.append_positions[0].tolist() == [-1, 0, 4, 15, 16]
    assert b.hist_lens.tolist() == [0, 0, 4, 15, 16]

"""Token append and copy-on-write of a tail block (bit-exact references).

Test infrastructure only (see the package docstring).

Pools are numpy arrays [NB, B, Hkv, d] (or [L, NB, B, Hkv, d] for the
multi-layer COW) of any dtype; bf16 pools are passed as their uint16 bit
patterns so that comparisons are bitwise.  Every function returns a new
array and leaves its input untouched.
"""

import numpy as np


def append(pool, new, block_tables, positions, B):
    """Write request s's new token (``new[s]``, [Hkv, d]) at logical position positions[s].

    The token goes to slot pos % B of physical block table[s][pos // B]; no
    other slot moves ([Slides] "写满一块，再拿下一块").  A negative position
    means the request writes nothing this step.
    """
    out = np.array(pool, copy=True)
    for s in range(len(positions)):
        pos = int(positions[s])
        if pos < 0:
            continue
        blk = int(block_tables[s][pos // B])
        out[blk, pos % B] = new[s]
    return out


def append_tokens(pool, new, block_tables, positions, B):
    """Write T consecutive tokens per request: ``new[s, i]`` ([Hkv, d]) at position positions[s] + i.

    The multi-token form of ``append`` (a verification step or a prompt chunk
    adds several tokens at once, [Serving] §5); token i lands in slot
    (p + i) % B of block table[s][(p + i) // B].  A negative start position
    skips the request.
    """
    out = np.array(pool, copy=True)
    for s in range(len(positions)):
        p = int(positions[s])
        if p < 0:
            continue
        for i in range(np.asarray(new).shape[1]):
            blk = int(block_tables[s][(p + i) // B])
            out[blk, (p + i) % B] = new[s][i]
    return out


def cow_copy(pool, src_blocks, dst_blocks, n_valid):
    """Copy slots [0, n_valid) of each source block into its destination block.

    The copy-on-write step of [Slides] "先确保分配成功，再改变可见状态"
    (``copy_valid_kv(tail, new)``): only the valid range is copied; slots at or
    beyond n_valid of the destination, and every other block, keep their bytes.
    Pairs are applied in order.
    """
    out = np.array(pool, copy=True)
    for a, b, n in zip(src_blocks, dst_blocks, n_valid):
        out[int(b), : int(n)] = out[int(a), : int(n)]
    return out


def cow_copy_layers(pools, src_blocks, dst_blocks, n_valid):
    """The COW copy applied in every layer of a [L, NB, B, Hkv, d] pool.

    All layers share one token -> block numbering, so a copied block must be
    copied in each layer's storage ([Slides] "128 KiB：每新增一个位置的账单").
    """
    return np.stack([cow_copy(p, src_blocks, dst_blocks, n_valid) for p in pools])


def gather_padded(pool, block_tables, seq_lens, B, fill):
    """[S, MB*B, Hkv, d]: token t of request s at [s, t]; positions >= n_s hold ``fill``.

    The contiguous view a block table describes, for checking the device-side
    address computation bit for bit.
    """
    pool = np.asarray(pool)
    S, MB = np.asarray(block_tables).shape
    out = np.full((S, MB * B) + pool.shape[2:], fill, dtype=pool.dtype)
    for s in range(S):
        for t in range(int(seq_lens[s])):
            out[s, t] = pool[int(block_tables[s][t // B]), t % B]
    return out


def swap_out(k_pools, v_pools, blocks):
    """Whole blocks of every layer into one buffer [L, 2, n, B, Hkv, d] (K then V).

    [Slides] "腾出显存以后，还要付一次恢复成本": moving a preempted request's KV
    out (and back in, below) instead of recomputing it.  Pools are [L, NB, ...].
    """
    k_pools, v_pools = np.asarray(k_pools), np.asarray(v_pools)
    idx = [int(b) for b in blocks]
    return np.stack([np.stack([k_pools[l][idx], v_pools[l][idx]]) for l in range(k_pools.shape[0])])


def swap_in(k_pools, v_pools, blocks, buf):
    """The inverse: block blocks[i] of layer l takes buf[l, 0/1, i]; new arrays returned."""
    k, v = np.array(k_pools, copy=True), np.array(v_pools, copy=True)
    for l in range(k.shape[0]):
        for i, b in enumerate(blocks):
            k[l, int(b)] = buf[l, 0, i]
            v[l, int(b)] = buf[l, 1, i]
    return k, v

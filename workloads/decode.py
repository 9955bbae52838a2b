"""Synthetic paged-decode workloads (seeded), shaped like the five benchmark batches.

Conventions
-----------
* Pools are [L, NB, B, Hkv, D]: layer, physical block, slot, KV head, dim.
  Every layer has its own storage; all layers share one block table.
* Physical ids are a seeded permutation of range(NB), handed out in order as
  logical blocks are assigned, so tables point all over the pool.
* Slots nobody has written, blocks nobody owns, and table entries past a
  request's last block (they point at a spare block) hold NaN, so any read of
  them shows up in the output.
* q, K, V are N(0, 1) drawn in float32 and rounded to the storage dtype
  (round-to-nearest-even for bf16).
* A decode step applies, in order: the copy-on-write pairs (every layer), each
  append round (every layer), then attention over ``seq_lens`` tokens.
  ``hist_lens`` are the tokens written before the step.

Structure (lengths, ids, fills) comes from numpy PCG64(seed); values come from
a torch generator seeded the same way on the device the tensors live on.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

SCALE_D128 = float(np.float32(1.0 / np.sqrt(128.0)))


@dataclass
class Batch:
    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    B: int
    NB: int
    MB: int
    L: int
    dtype: torch.dtype
    scale: float
    q: torch.Tensor               # [L, S, Hq, D]
    k_pool: torch.Tensor          # [L, NB, B, Hkv, D]
    v_pool: torch.Tensor
    block_tables: torch.Tensor    # int32 [S, MB]
    seq_lens: torch.Tensor        # int32 [S]  tokens attended after the step
    hist_lens: np.ndarray         # tokens written before the step
    append_positions: torch.Tensor  # int32 [R, S], -1 = no write in that round
    k_new: torch.Tensor           # [R, L, S, Hkv, D]
    v_new: torch.Tensor
    cow_src: torch.Tensor         # int32 [P]
    cow_dst: torch.Tensor
    cow_n: torch.Tensor
    spare_block: int
    info: dict = field(default_factory=dict)

    @property
    def rounds(self):
        return int(self.append_positions.shape[0])

    @property
    def elem_bytes(self):
        return torch.tensor([], dtype=self.dtype).element_size()

    def valid_kv_bytes_per_layer(self):
        """K+V bytes of the attended (valid) slots of one layer."""
        return int(self.seq_lens.sum().item()) * 2 * self.Hkv * self.D * self.elem_bytes


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, dtype, scale=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def _fill_pools(L, NB, B, Hkv, D, dtype, gen, device):
    k = torch.empty((L, NB, B, Hkv, D), dtype=dtype, device=device)
    v = torch.empty_like(k)
    for pool in (k, v):
        for layer in range(L):  # one layer at a time bounds the float32 temporary
            pool[layer] = _randn((NB, B, Hkv, D), gen, device, dtype)
    return k, v


def _poison(k, v, blocks, slots, whole_blocks, device):
    """NaN-fill (block, slot) pairs and whole blocks in every layer."""
    nan = float("nan")
    if len(blocks):
        bi = torch.as_tensor(np.asarray(blocks, np.int64), device=device)
        si = torch.as_tensor(np.asarray(slots, np.int64), device=device)
        for pool in (k, v):
            pool[:, bi, si] = nan
    if len(whole_blocks):
        wi = torch.as_tensor(np.asarray(whole_blocks, np.int64), device=device)
        for pool in (k, v):
            pool[:, wi] = nan


def _assemble(name, *, S, Hq, Hkv, D, B, NB, L, dtype, seed, device, hist, seq_lens,
              tables_np, spare_ids, rounds_pos, cow=None, q_scale=1.0, info=None):
    """Materialise values for a laid-out batch.

    ``hist[s]`` tokens of request s are written; slots from hist[s] up to the
    end of its last allocated block are unwritten (NaN), as is every block in
    ``spare_ids`` and every copy-on-write destination (written by the copy).
    """
    gen = _gen(seed, device)
    MB = tables_np.shape[1]
    k_pool, v_pool = _fill_pools(L, NB, B, Hkv, D, dtype, gen, device)
    pb, ps = [], []
    for s in range(S):
        nblk = -(-int(max(seq_lens[s], hist[s])) // B)
        for t in range(int(hist[s]), nblk * B):
            pb.append(int(tables_np[s, t // B]))
            ps.append(t % B)
    whole = list(spare_ids) + ([] if cow is None else [int(x) for x in cow[1]])
    _poison(k_pool, v_pool, pb, ps, whole, device)
    q = _randn((L, S, Hq, D), gen, device, dtype, q_scale)
    R = len(rounds_pos)
    k_new = _randn((R, L, S, Hkv, D), gen, device, dtype)
    v_new = _randn((R, L, S, Hkv, D), gen, device, dtype)
    pos = torch.as_tensor(np.asarray(rounds_pos, np.int32).reshape(R, S), device=device)
    if cow is None:
        cow = (np.zeros(0, np.int32),) * 3
    cs, cd, cn = (torch.as_tensor(np.asarray(a, np.int32), device=device) for a in cow)
    return Batch(
        name=name, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, NB=NB, MB=MB, L=L, dtype=dtype,
        scale=SCALE_D128 if D == 128 else float(np.float32(1.0 / np.sqrt(D))),
        q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.as_tensor(tables_np.astype(np.int32), device=device),
        seq_lens=torch.as_tensor(np.asarray(seq_lens, np.int32), device=device),
        hist_lens=np.asarray(hist, np.int64),
        append_positions=pos, k_new=k_new, v_new=v_new,
        cow_src=cs, cow_dst=cd, cow_n=cn,
        spare_block=int(spare_ids[0]) if len(spare_ids) else -1,
        info=dict(info or {}, seed=int(seed)),
    )


def _layout(rng, NB, B, lens_alloc, MB=None):
    """Assign physical blocks for requests needing ceil(lens_alloc[s]/B) blocks.

    Returns (tables [S, MB] int64, spare ids).  Entries past a request's last
    block point at the first spare block (or block 0 when the pool is full).
    """
    need = [-(-int(n) // B) for n in lens_alloc]
    if MB is None:
        MB = max(1, max(need))
    if max(need) > MB or sum(need) > NB:
        raise ValueError("workload does not fit its pool / table width")
    perm = rng.permutation(NB)
    spare = perm[sum(need):]
    filler = int(spare[0]) if len(spare) else 0
    tables = np.full((len(need), MB), filler, dtype=np.int64)
    cur = 0
    for s, nb in enumerate(need):
        tables[s, :nb] = perm[cur:cur + nb]
        cur += nb
    return tables, spare


def custom(lengths, *, Hq=8, Hkv=2, D=128, B=16, dtype=torch.float32, NB=None, MB=None,
           L=1, seed=0, device="cpu", append=False, q_scale=1.0, spare_blocks=2, name="custom"):
    """Any batch: ``lengths`` are tokens attended; with ``append`` the step first
    writes token lengths[s]-1 of every non-empty request."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lengths, np.int64)
    S = len(lens)
    hist = np.maximum(lens - 1, 0) if append else lens.copy()
    used = sum(-(-int(n) // B) for n in lens)
    if NB is None:
        NB = used + spare_blocks
    tables, spare = _layout(rng, NB, B, lens, MB)
    rounds = [np.where(lens > 0, hist, -1)] if append else []
    return _assemble(name, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, NB=NB, L=L, dtype=dtype, seed=seed,
                     device=device, hist=hist, seq_lens=lens, tables_np=tables, spare_ids=spare,
                     rounds_pos=rounds, q_scale=q_scale)


def config1(device="cpu", seed=353):
    """5 requests of 37/91/128/201/511 tokens, Hq 8 / Hkv 2, d 128, B 16, fp32, 64-block pool."""
    lens = np.array([37, 91, 128, 201, 511])
    rng = np.random.Generator(np.random.PCG64(seed))
    tables, spare = _layout(rng, 64, 16, lens, MB=32)
    return _assemble("config1_fp32_5seq", S=5, Hq=8, Hkv=2, D=128, B=16, NB=64, L=1,
                     dtype=torch.float32, seed=seed, device=device, hist=lens, seq_lens=lens,
                     tables_np=tables, spare_ids=spare, rounds_pos=[])


def config2(device="cpu", seed=354, S=32, n=4096, B=16):
    """32 requests x 4096 tokens, Hq 32 / Hkv 8, d 128, B 16 (or another block
    size), bf16; a pool of exactly the blocks the histories fill (8192 at B 16)."""
    lens = np.full(S, n)
    NB = S * (-(-n // B))
    rng = np.random.Generator(np.random.PCG64(seed))
    tables, spare = _layout(rng, NB, B, lens)
    return _assemble(f"config2_bf16_{S}x{n}_B{B}", S=S, Hq=32, Hkv=8, D=128, B=B, NB=NB, L=1,
                     dtype=torch.bfloat16, seed=seed, device=device, hist=lens, seq_lens=lens,
                     tables_np=tables, spare_ids=spare, rounds_pos=[])


def config3_lengths(seed=355):
    """History lengths h: forced 0, 1, 16, 17, then 252 draws uniform on [1, 512]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    h = np.concatenate([[0, 1, 16, 17], rng.integers(1, 513, size=252)])
    return rng, h.astype(np.int64)


def config3(device="cpu", seed=355, layers=32):
    """256 requests, Hq 32 / Hkv 8, d 128, B 16, bf16, 12,288-block pool per layer.

    Each request has h tokens of history; the step appends token h in every
    layer and attends over h + 1 tokens.
    """
    rng, h = config3_lengths(seed)
    lens = h + 1
    tables, spare = _layout(rng, 12288, 16, lens, MB=33)
    return _assemble("config3_bf16_256req", S=256, Hq=32, Hkv=8, D=128, B=16, NB=12288,
                     L=layers, dtype=torch.bfloat16, seed=seed, device=device, hist=h,
                     seq_lens=lens, tables_np=tables, spare_ids=spare, rounds_pos=[h])


def config4(device="cpu", seed=356, t=None, branches=64):
    """Prefix sharing + copy-on-write, one layer, q scaled by 20.

    64 branches share 128 full prefix blocks (2048 tokens) and one tail block
    holding t tokens.  Branches 0..62 find the tail shared and copy its t valid
    slots into a fresh block; branch 63 is then its only reader and writes in
    place.  Branch i then appends c_i ~ U[1, 64] tokens, one per round,
    taking a fresh block whenever its tail fills.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, NB, P = 16, 1024, 128
    if t is None:
        t = int(rng.integers(1, B))
    c = rng.integers(1, 65, size=branches).astype(np.int64)
    perm = rng.permutation(NB)
    cur = 0

    def take(k):
        nonlocal cur
        ids = perm[cur:cur + k]
        cur += k
        return [int(x) for x in ids]

    prefix = take(P)
    shared_tail = take(1)[0]
    lens = P * B + t + c
    MB = int(max(-(-int(n) // B) for n in lens))
    rows = []
    cow_src, cow_dst, cow_n = [], [], []
    for i in range(branches):
        row = list(prefix)
        if i < branches - 1:
            fresh = take(1)[0]
            cow_src.append(shared_tail)
            cow_dst.append(fresh)
            cow_n.append(t)
            row.append(fresh)
        else:
            row.append(shared_tail)
        row += take(-(-int(lens[i]) // B) - len(row))
        rows.append(row)
    spare = perm[cur:]
    tables = np.full((branches, MB), int(spare[0]), dtype=np.int64)
    for i, row in enumerate(rows):
        tables[i, :len(row)] = row
    hist = np.full(branches, P * B + t)
    rounds = [np.where(c > r, P * B + t + r, -1) for r in range(int(c.max()))]
    # Unwritten: everything past the shared tail's t slots, the fresh COW
    # targets and the continuation blocks (poisoned via the tables).
    b = _assemble(f"config4_bf16_cow_t{t}", S=branches, Hq=32, Hkv=8, D=128, B=B, NB=NB, L=1,
                  dtype=torch.bfloat16, seed=seed, device=device, hist=hist, seq_lens=lens,
                  tables_np=tables, spare_ids=spare, rounds_pos=rounds,
                  cow=(cow_src, cow_dst, cow_n), q_scale=20.0,
                  info={"t": t, "c": c.tolist(), "prefix_blocks": P, "shared_tail": shared_tail})
    return b


def config5(device="cpu", seed=357, layers=24):
    """168 requests x 1025 tokens, Hq 16 / Hkv 4, d 128, B 16, bf16, 10,922-block pool.

    The 1024-token history fills 64 blocks; the step appends token 1024 into
    the 65th block of every layer and attends over 1025 tokens.
    """
    S, n = 168, 1025
    lens = np.full(S, n)
    h = lens - 1
    rng = np.random.Generator(np.random.PCG64(seed))
    tables, spare = _layout(rng, 10922, 16, lens, MB=65)
    return _assemble("config5_bf16_168x1025", S=S, Hq=16, Hkv=4, D=128, B=16, NB=10922,
                     L=layers, dtype=torch.bfloat16, seed=seed, device=device, hist=h,
                     seq_lens=lens, tables_np=tables, spare_ids=spare, rounds_pos=[h])


def make_config(idx, device="cpu", **kw):
    return {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}[idx](device=device, **kw)

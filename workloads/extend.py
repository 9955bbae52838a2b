"""Synthetic batches with several new query tokens per request (seeded).

A speculative-verification step or one chunk of a prompt: each request has
``lengths[s]`` tokens in all after the step, the last T of them new.  The
step appends the T new tokens (when the request has at least T tokens) and
then runs attention for all T of them over the paged history.

Conventions are those of ``workloads.decode`` (one layer here): pools
[NB, B, Hkv, D] with shuffled physical ids, NaN in every slot nobody wrote,
in spare blocks and in table entries past a request's last block; q, K, V
drawn N(0, 1) in float32 and rounded to the storage dtype.
"""

from dataclasses import dataclass

import numpy as np
import torch

from .decode import SCALE_D128, _fill_pools, _gen, _layout, _poison, _randn


@dataclass
class ExtendBatch:
    name: str
    S: int
    T: int
    Hq: int
    Hkv: int
    D: int
    B: int
    NB: int
    MB: int
    dtype: torch.dtype
    scale: float
    q: torch.Tensor              # [S, T, Hq, D]
    k_pool: torch.Tensor         # [NB, B, Hkv, D]
    v_pool: torch.Tensor
    block_tables: torch.Tensor   # int32 [S, MB]
    seq_lens: torch.Tensor       # int32 [S]  tokens in all after the step (the T new ones last)
    positions: torch.Tensor      # int32 [S]  where the T new tokens go; -1 = already written
    k_new: torch.Tensor          # [S, T, Hkv, D]
    v_new: torch.Tensor
    spare_block: int

    @property
    def elem_bytes(self):
        return torch.tensor([], dtype=self.dtype).element_size()

    def valid_kv_bytes(self):
        """K+V bytes of the valid slots: the history every pass over it must read once."""
        return int(self.seq_lens.sum().item()) * 2 * self.Hkv * self.D * self.elem_bytes


def extend_batch(lengths, T, *, Hq=32, Hkv=8, D=128, B=16, dtype=torch.bfloat16, NB=None, MB=None, seed=0,
                 device="cpu", spare_blocks=2, q_scale=1.0, name=None):
    """``lengths[s]`` tokens per request after the step, the last T new.

    Requests with at least T tokens hold lengths[s] - T written tokens and get
    the T new ones appended by the step at positions[s] = lengths[s] - T.
    Shorter requests (the first queries then have no position) are written
    whole beforehand and skip the append (positions[s] = -1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lengths, np.int64)
    S = len(lens)
    appended = lens >= T
    hist = np.where(appended, lens - T, lens)
    used = sum(-(-int(n) // B) for n in lens)
    if NB is None:
        NB = used + spare_blocks
    tables, spare = _layout(rng, NB, B, lens, MB)
    gen = _gen(seed, device)
    k_pool, v_pool = _fill_pools(1, NB, B, Hkv, D, dtype, gen, device)
    pb, ps = [], []
    for s in range(S):
        for t in range(int(hist[s]), -(-int(lens[s]) // B) * B):
            pb.append(int(tables[s, t // B]))
            ps.append(t % B)
    _poison(k_pool, v_pool, pb, ps, list(spare), device)
    q = _randn((S, T, Hq, D), gen, device, dtype, q_scale)
    k_new = _randn((S, T, Hkv, D), gen, device, dtype)
    v_new = _randn((S, T, Hkv, D), gen, device, dtype)
    pos = np.where(appended, hist, -1).astype(np.int32)
    return ExtendBatch(
        name=name or f"extend_T{T}_{S}req",
        S=S, T=T, Hq=Hq, Hkv=Hkv, D=D, B=B, NB=NB, MB=tables.shape[1], dtype=dtype,
        scale=SCALE_D128 if D == 128 else float(np.float32(1.0 / np.sqrt(D))),
        q=q, k_pool=k_pool[0], v_pool=v_pool[0],
        block_tables=torch.as_tensor(tables.astype(np.int32), device=device),
        seq_lens=torch.as_tensor(lens.astype(np.int32), device=device),
        positions=torch.as_tensor(pos, device=device),
        k_new=k_new, v_new=v_new,
        spare_block=int(spare[0]) if len(spare) else -1,
    )


def verify_batch(device="cpu", seed=358, S=32, n=4096, T=4, B=16):
    """Speculative verification: 32 requests, 4096 tokens each after the step
    (4092 of history + 4 draft tokens), Hq 32 / Hkv 8, d 128, B 16, bf16."""
    return extend_batch(np.full(S, n), T, B=B, NB=S * (-(-n // B)) + 1, seed=seed, device=device,
                        name=f"verify_bf16_{S}x{n}_T{T}")


def prefill_chunk_batch(device="cpu", seed=359, S=8, n=4096, T=512, B=16):
    """One prompt chunk: 8 requests, 4096 tokens each after the step (3584 of
    history + a 512-token chunk), Hq 32 / Hkv 8, d 128, B 16, bf16."""
    return extend_batch(np.full(S, n), T, B=B, NB=S * (-(-n // B)) + 1, seed=seed, device=device,
                        name=f"prefill_chunk_bf16_{S}x{n}_T{T}")

"""Helpers for the GPU parity tests: run a decode step through the C ABI, and
the same step through the oracle on host copies of the pre-step inputs."""

import numpy as np
import torch

import paged_kv_cache_352_amd as pa
from oracle import attention as att
from oracle import kvcache as kvc

BF16_REL_TOL = 5e-3   # max |gpu - oracle| <= 5e-3 * max |oracle|, bf16 K/V, fp32 accumulation
FP32_ABS_TOL = 1e-5   # max |gpu - oracle| for fp32 K/V


def banner(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def host_f32(t):
    """Exact float32 host copy (bf16 widens exactly)."""
    return t.float().cpu().numpy()


def host_bits(t):
    """Bit patterns of a tensor (for bitwise comparisons)."""
    view = {2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.contiguous().view(view).cpu().numpy()


def gpu_step(b, layers=None, num_splits=0):
    """COW pairs, append rounds, then decode, all through libpagedattn on one stream.

    Returns {layer: out [S, Hq, D] float32 (device)}.
    """
    layers = range(b.L) if layers is None else layers
    if b.cow_src.numel():
        pa.kv_cow_copy(b.k_pool, b.v_pool, b.cow_src, b.cow_dst, b.cow_n, b.B)
    for r in range(b.rounds):
        for layer in range(b.L):
            pa.kv_append(b.k_pool[layer], b.v_pool[layer], b.k_new[r, layer], b.v_new[r, layer],
                         b.block_tables, b.append_positions[r], b.B)
    return {layer: pa.paged_attn_decode(b.q[layer], b.k_pool[layer], b.v_pool[layer], b.block_tables,
                                        b.seq_lens, b.B, b.scale, num_splits=num_splits)
            for layer in layers}


class HostLayer:
    """Host copy of one layer's pre-step inputs, for the oracle."""

    def __init__(self, b, layer):
        self.k = host_f32(b.k_pool[layer])
        self.v = host_f32(b.v_pool[layer])
        self.q = host_f32(b.q[layer])
        self.k_new = host_f32(b.k_new[:, layer]) if b.rounds else None
        self.v_new = host_f32(b.v_new[:, layer]) if b.rounds else None
        self.tables = b.block_tables.cpu().numpy()
        self.lens = b.seq_lens.cpu().numpy()
        self.pos = b.append_positions.cpu().numpy()
        self.cow = tuple(t.cpu().numpy() for t in (b.cow_src, b.cow_dst, b.cow_n))
        self.B, self.scale = b.B, b.scale

    def pools_after_step(self):
        k, v = self.k, self.v
        if len(self.cow[0]):
            k = kvc.cow_copy(k, *self.cow)
            v = kvc.cow_copy(v, *self.cow)
        for r in range(self.pos.shape[0]):
            k = kvc.append(k, self.k_new[r], self.tables, self.pos[r], self.B)
            v = kvc.append(v, self.v_new[r], self.tables, self.pos[r], self.B)
        return k, v

    def oracle(self, rows=None):
        k, v = self.pools_after_step()
        if rows is None:
            return att.paged_decode(self.q, k, v, self.tables, self.lens, self.B, self.scale)
        return att.paged_decode_rows(self.q, k, v, self.tables, self.lens, self.B, self.scale, rows)


class HostRows:
    """Host copy of one layer's pre-step inputs for the listed requests only.

    Holds just the blocks those requests' tables reference (renumbered), so
    every layer of a large multi-layer batch can be checked on a handful of
    requests without copying its pools.  Batches with copy-on-write pairs are
    not supported (a copy may read blocks outside the listed requests)."""

    def __init__(self, b, layer, rows):
        assert not b.cow_src.numel()
        self.rows = list(rows)
        tab = b.block_tables.cpu().numpy()
        lens = b.seq_lens.cpu().numpy()
        pos = b.append_positions.cpu().numpy()
        nblk = {s: -(-max(int(lens[s]), int(max(pos[:, s].max(initial=-1) + 1, 0))) // b.B) for s in self.rows}
        used = sorted({int(tab[s, j]) for s in self.rows for j in range(nblk[s])})
        remap = {blk: i for i, blk in enumerate(used)}
        ids = torch.as_tensor(used, dtype=torch.long, device=b.k_pool.device)
        self.k = host_f32(b.k_pool[layer].index_select(0, ids))
        self.v = host_f32(b.v_pool[layer].index_select(0, ids))
        sel = torch.as_tensor(self.rows, dtype=torch.long, device=b.q.device)
        self.q = host_f32(b.q[layer].index_select(0, sel))
        self.tables = np.zeros((len(self.rows), b.MB), dtype=np.int64)
        for i, s in enumerate(self.rows):
            self.tables[i, :nblk[s]] = [remap[int(tab[s, j])] for j in range(nblk[s])]
        self.lens = lens[self.rows]
        self.pos = pos[:, self.rows]
        self.k_new = host_f32(b.k_new[:, layer].index_select(1, sel)) if b.rounds else None
        self.v_new = host_f32(b.v_new[:, layer].index_select(1, sel)) if b.rounds else None
        self.B, self.scale = b.B, b.scale

    def oracle(self):
        """[len(rows), Hq, d] float64, in the order the rows were listed."""
        k, v = self.k, self.v
        for r in range(self.pos.shape[0]):
            k = kvc.append(k, self.k_new[r], self.tables, self.pos[r], self.B)
            v = kvc.append(v, self.v_new[r], self.tables, self.pos[r], self.B)
        return att.paged_decode(self.q, k, v, self.tables, self.lens, self.B, self.scale)


# Largest error against the oracle per recorded case, written out at the end
# of the session when PA_ACCURACY_REPORT names a file (tests/conftest.py).
ACCURACY = []


def assert_close(got, want, dtype, what="", record=None):
    """Element-wise check against the oracle at the tolerance for ``dtype``.

    ``record`` names the case in the accuracy report (largest absolute error,
    largest |oracle|, their ratio and the tolerance)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    ref = float(np.max(np.abs(want))) if want.size else 0.0
    if record is not None:
        ACCURACY.append({"case": record, "dtype": str(dtype).replace("torch.", ""), "elements": int(got.size),
                         "max_abs_err": err, "max_abs_oracle": ref, "err_over_max_out": err / ref if ref else 0.0,
                         "tolerance": (f"abs {FP32_ABS_TOL}" if dtype == torch.float32
                                       else f"{BF16_REL_TOL} * max|oracle|")})
    if dtype == torch.float32:
        assert err <= FP32_ABS_TOL, f"{what}: max abs err {err:.3e} > {FP32_ABS_TOL}"
    else:
        assert err <= BF16_REL_TOL * ref, f"{what}: max abs err {err:.3e} > {BF16_REL_TOL} * {ref:.3e}"
    return err

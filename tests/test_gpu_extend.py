"""Several query tokens per request on the GPU: kv_append_tokens and paged_attn_extend
against the float64 oracle (causal attention of the last T tokens over the paged
history), fp32 within 1e-5 absolute and bf16 within 5e-3 * max|out|; the
multi-token append bit for bit; bitwise-identical output under a permutation of
physical ids; and a speculative-decoding loop driven by the block manager
(grow by T drafts, verify, roll back the rejected ones)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_352_amd as pa
import workloads as W
from oracle import attention as att
from oracle import kvcache as kvc
from tests.gpu_util import assert_close, banner, host_bits, host_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_extend(b, num_splits=0, bf16_weights=False):
    """The step through libpagedattn on one stream: append the T new tokens, then attend."""
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    return pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                                num_splits=num_splits, bf16_weights=bf16_weights)


class HostExtend:
    """Host copies of a batch's pre-step inputs, and the oracle's answer for them."""

    def __init__(self, b):
        self.k, self.v = host_f32(b.k_pool), host_f32(b.v_pool)
        self.q = host_f32(b.q)
        self.k_new, self.v_new = host_f32(b.k_new), host_f32(b.v_new)
        self.tables = b.block_tables.cpu().numpy()
        self.lens = b.seq_lens.cpu().numpy()
        self.pos = b.positions.cpu().numpy()
        self.B, self.scale = b.B, b.scale

    def pools_after_step(self):
        return (kvc.append_tokens(self.k, self.k_new, self.tables, self.pos, self.B),
                kvc.append_tokens(self.v, self.v_new, self.tables, self.pos, self.B))

    def oracle(self, rows=None):
        k, v = self.pools_after_step()
        if rows is None:
            return att.paged_extend(self.q, k, v, self.tables, self.lens, self.B, self.scale)
        return att.paged_extend_rows(self.q, k, v, self.tables, self.lens, self.B, self.scale, rows)


# lengths around tile (16) and block boundaries, shorter than T, and a few hundred
RAGGED = [1, 2, 3, 4, 5, 15, 16, 17, 19, 31, 32, 33, 100, 257, 300]


def check(b, dtype, what, num_splits=0, bf16_weights=False):
    host = HostExtend(b)
    out = gpu_extend(b, num_splits=num_splits, bf16_weights=bf16_weights)
    torch.cuda.synchronize()
    return assert_close(host_f32(out), host.oracle(), dtype, what)


@pytest.mark.parametrize("T", [2, 3, 4, 5, 8])
def test_bf16_one_item_per_group(T):
    """G = 4: up to 8 tokens share one pass over the history (one or two sets of
    16 MFMA columns per wave)."""
    banner(f"extend bf16 G=4 T={T} ragged")
    b = W.extend_batch(RAGGED, T, Hq=16, Hkv=4, seed=10 + T, device=DEV)
    check(b, torch.bfloat16, f"bf16 T={T}")


@pytest.mark.parametrize("G,T", [(4, 7), (4, 16), (1, 17), (1, 40), (16, 3), (8, 5), (2, 9),
                                 (4, 40), (16, 9), (2, 70), (8, 33), (4, 17), (4, 24), (2, 36), (1, 65),
                                 (4, 33), (1, 150), (4, 12), (4, 70)])
def test_bf16_several_items_per_group(G, T):
    """Separate items per column set up to two sets; the shared-tile kernel above,
    with one 16-column set per wave, or two once one set per wave would need a
    second workgroup (then some waves may hold no live column); past 128 columns
    the 8-wave ping-pong form (4 x 33: 132 columns, one live column past the
    first four waves; 1 x 150: 32 tokens per wave).  Waves whose tokens all lie
    past T skip their arithmetic: 4 x 12 (the 16-column kernel's last wave),
    4 x 24 (the 32-column kernel's), 4 x 70 (the ping-pong kernel's second
    workgroup, live in wave 0 only, idle waves in both phase groups)."""
    banner(f"extend bf16 G={G} T={T} ragged")
    b = W.extend_batch(RAGGED, T, Hq=2 * G, Hkv=2, seed=20 + G + T, device=DEV)
    check(b, torch.bfloat16, f"bf16 G={G} T={T}")


# PA_FLAG_BF16_WEIGHTS on the shared-tile path: group sizes, one and two
# column sets, forced splits (l leaves through the split workspace), block sizes.
@pytest.mark.parametrize("G,T,splits,B", [(4, 17, 0, 16), (4, 40, 0, 16), (1, 40, 0, 16), (2, 70, 0, 16),
                                          (8, 33, 0, 16), (16, 9, 0, 16), (4, 24, 0, 16), (4, 40, 4, 16),
                                          (2, 36, 3, 16), (4, 40, 0, 4), (4, 40, 0, 64)])
def test_bf16_weights_flag(G, T, splits, B):
    """Weights rounded once to bf16, l summed from the rounded weights: within the
    bf16 tolerance of the oracle, and not the default form's result."""
    banner(f"extend bf16 weights G={G} T={T} splits={splits} B={B}")
    lens = RAGGED + [2 * B + 1, 4 * B - 1]
    b = W.extend_batch(lens, T, Hq=2 * G, Hkv=2, B=B, seed=200 + G + T + B, device=DEV)
    host = HostExtend(b)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    fast = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                                num_splits=splits, bf16_weights=True)
    exact = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                                 num_splits=splits)
    torch.cuda.synchronize()
    ref = host.oracle()
    err_fast = assert_close(host_f32(fast), ref, torch.bfloat16, "bf16 weights")
    err_exact = assert_close(host_f32(exact), ref, torch.bfloat16, "head + remainder")
    print(f"  max abs err: bf16 weights {err_fast:.3e}, head + remainder {err_exact:.3e}", flush=True)
    assert not torch.equal(fast, exact)


@pytest.mark.parametrize("T,bf16_weights,splits", [(4, False, 0), (40, False, 0), (40, True, 0), (300, False, 0),
                                                   (16, False, 4), (24, True, 4)])
def test_negative_scale(T, bf16_weights, splits):
    """A negative scale (legal, if unusual) reverses the order of the logits, and a
    zero scale weighs every visible position the same: the decode-kernel form (T = 4)
    and the shared-tile kernel (also as four parts of one workgroup), which feeds q
    negated and the scale's magnitude to its unmasked steps, both match the oracle."""
    for factor in (-3.0, 0.0):  # a zero scale: every visible position weighs the same
        banner(f"extend bf16 scale x {factor} T={T} bf16_weights={bf16_weights} splits={splits}")
        b = W.extend_batch([T + 1, T + 60, T + 700], T, Hq=8, Hkv=2, seed=250 + T, device=DEV)
        b.scale = abs(b.scale) * factor
        check(b, torch.bfloat16, f"scale x {factor} T={T}", num_splits=splits, bf16_weights=bf16_weights)


@pytest.mark.parametrize("dtype,G,T", [(torch.bfloat16, 4, 1), (torch.bfloat16, 4, 5), (torch.bfloat16, 4, 8),
                                       (torch.bfloat16, 1, 16), (torch.float32, 4, 20)])
def test_bf16_weights_flag_ignored_off_the_shared_tile_path(dtype, G, T):
    """Decode-kernel forms (up to two column sets) and float32 keep the head and
    remainder: bitwise the same output with and without the flag."""
    banner(f"extend flag ignored {dtype} G={G} T={T}")
    b = W.extend_batch(RAGGED, T, Hq=2 * G, Hkv=2, dtype=dtype, seed=230 + G + T, device=DEV)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    a = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale, bf16_weights=True)
    c = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(a), host_bits(c))


@pytest.mark.parametrize("G,T", [(4, 2), (4, 5), (1, 9), (8, 3), (2, 4)])
def test_fp32(G, T):
    banner(f"extend fp32 G={G} T={T} ragged")
    b = W.extend_batch(RAGGED, T, Hq=2 * G, Hkv=2, dtype=torch.float32, seed=30 + G + T, device=DEV)
    check(b, torch.float32, f"fp32 G={G} T={T}")


@pytest.mark.parametrize("dtype,splits,T", [(torch.bfloat16, 2, 5), (torch.bfloat16, 3, 5), (torch.bfloat16, 7, 5),
                                            (torch.float32, 2, 5), (torch.float32, 5, 5), (torch.bfloat16, 3, 12),
                                            (torch.bfloat16, 4, 40)])
def test_forced_splits(dtype, splits, T):
    """Split boundaries inside the causal region: later splits of early tokens hold nothing."""
    banner(f"extend {dtype} splits={splits} T={T}")
    b = W.extend_batch([16, 17, 40, 64, 65, 200, 300], T, Hq=8, Hkv=2, dtype=dtype, seed=40 + splits + T,
                       device=DEV)
    check(b, dtype, f"splits={splits} T={T}", num_splits=splits)


@pytest.mark.parametrize("B", [4, 8, 32, 64])
def test_block_sizes(B):
    banner(f"extend bf16 B={B} T=4 and fp32 T=3")
    lens = [1, 3, 4, 5, B - 1, B, B + 1, 2 * B + 3, 150]
    check(W.extend_batch(lens, 4, Hq=16, Hkv=4, B=B, seed=50 + B, device=DEV), torch.bfloat16, f"bf16 B={B}")
    check(W.extend_batch(lens, 3, Hq=8, Hkv=2, B=B, dtype=torch.float32, seed=60 + B, device=DEV),
          torch.float32, f"fp32 B={B}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_one_token_is_the_decode_step_bitwise(dtype):
    banner(f"extend T=1 vs decode {dtype}")
    b = W.extend_batch(RAGGED, 1, Hq=8, Hkv=2, dtype=dtype, seed=70, device=DEV)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    ext = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale)
    dec = pa.paged_attn_decode(b.q[:, 0].contiguous(), b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B,
                               b.scale)
    torch.cuda.synchronize()
    assert torch.equal(ext[:, 0], dec)


@pytest.mark.parametrize("dtype,T", [(torch.bfloat16, 4), (torch.bfloat16, 6), (torch.bfloat16, 9),
                                     (torch.bfloat16, 40), (torch.float32, 3)])
def test_physical_permutation_is_bitwise_invisible(dtype, T):
    banner(f"extend permutation {dtype} T={T}")
    b = W.extend_batch(RAGGED, T, Hq=8, Hkv=2, dtype=dtype, seed=80 + T, device=DEV)
    out1 = gpu_extend(b).clone()
    perm = torch.randperm(b.NB, generator=torch.Generator().manual_seed(5)).to(DEV)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(b.NB, device=DEV)
    k2 = torch.empty_like(b.k_pool)
    v2 = torch.empty_like(b.v_pool)
    k2[inv] = b.k_pool  # block p moves to inv[p]
    v2[inv] = b.v_pool
    t2 = inv[b.block_tables.long()].to(torch.int32)
    out2 = pa.paged_attn_extend(b.q, k2, v2, t2, b.seq_lens, b.B, b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out1), host_bits(out2))


@pytest.mark.parametrize("T,splits", [(4, 0), (8, 3), (40, 0), (40, 2), (16, 2), (16, 4), (24, 2), (24, 4)])
def test_graph_capture_replays_match_eager(T, splits):
    """A captured paged_attn_extend replays bit-identically, several times, with
    eager work between the replays (decode-kernel and shared-tile variants, with
    and without the split merge, and the splits run as two halves or four parts
    of one workgroup)."""
    banner(f"extend graph capture T={T} splits={splits}")
    b = W.extend_batch([9, 40, 300, 77, 130], T, Hq=8, Hkv=2, seed=95 + T, device=DEV)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    eager = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                                 num_splits=splits).clone()
    launch = pa.DecodeLaunch(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale, num_splits=splits)
    launch.launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch.launch()
    for _ in range(4):
        launch.out.fill_(-1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(launch.out.view(torch.int32), eager.view(torch.int32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_tokens_bit_exact(dtype):
    banner(f"kv_append_tokens bit-exact {dtype}")
    b = W.extend_batch(RAGGED, 6, Hq=8, Hkv=2, dtype=dtype, seed=90, device=DEV)
    k0, v0 = host_bits(b.k_pool), host_bits(b.v_pool)
    kn, vn = host_bits(b.k_new), host_bits(b.v_new)
    tab, pos = b.block_tables.cpu().numpy(), b.positions.cpu().numpy()
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(b.k_pool), kvc.append_tokens(k0, kn, tab, pos, b.B))
    assert np.array_equal(host_bits(b.v_pool), kvc.append_tokens(v0, vn, tab, pos, b.B))


def test_verify_32x4096_T4_sampled():
    """The verification batch at full size (the launch the benchmark times), sampled requests."""
    banner("verify bf16 32x4096 T=4 (bench launch configuration), sampled rows")
    b = W.verify_batch(device=DEV)
    host = HostExtend(b)
    out = host_f32(gpu_extend(b))
    rows = [0, 13, 31]
    ref = host.oracle(rows)
    assert_close(np.stack([out[s] for s in rows]), np.stack([ref[s] for s in rows]), torch.bfloat16, "verify",
                 record=f"bf16 verification 32 x 4096 tokens, T = 4, rows {rows}")
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("T,bf16_weights,parts", [(16, False, 4), (16, True, 2), (13, False, 4), (12, False, 2),
                                                  (24, False, 4), (24, True, 4), (20, False, 4)])
def test_verify_32x4096_shared_tile_sampled(T, bf16_weights, parts):
    """The verification batch at full size with 12-24 draft tokens, in the
    automatic plan the benchmark times: four parts of one workgroup on the
    32-column kernel (two waves each for 13-16 tokens of 4-head groups with
    the default weights, three each for 17-24 tokens), two halves otherwise;
    sampled requests against the oracle."""
    banner(f"verify bf16 32x4096 T={T} bf16_weights={bf16_weights} ({parts} parts), sampled rows")
    b = W.verify_batch(device=DEV, T=T)
    assert pa.paged_attn_extend_plan(b.S, b.Hq, b.Hkv, b.D, b.MB, b.NB, b.dtype, b.B, T,
                                     bf16_weights=bf16_weights) == (parts, 0)
    host = HostExtend(b)
    out = host_f32(gpu_extend(b, bf16_weights=bf16_weights))
    rows = [0, 13, 31]
    ref = host.oracle(rows)
    assert_close(np.stack([out[s] for s in rows]), np.stack([ref[s] for s in rows]), torch.bfloat16, "verify",
                 record=f"bf16 verification 32 x 4096 tokens, T = {T}, bf16_weights={bf16_weights}, rows {rows}")
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("bf16_weights", [False, True])
def test_prefill_chunk_512_sampled(bf16_weights):
    """A 512-token prompt chunk over 3584 tokens of history, 8 requests; three sampled requests."""
    banner(f"prefill chunk bf16 8x4096 T=512 bf16_weights={bf16_weights}, sampled rows")
    b = W.prefill_chunk_batch(device=DEV)
    host = HostExtend(b)
    out = host_f32(gpu_extend(b, bf16_weights=bf16_weights))
    rows = [0, 5, 7]
    ref = host.oracle(rows)
    assert_close(np.stack([out[s] for s in rows]), np.stack([ref[s] for s in rows]), torch.bfloat16, "chunk",
                 record=f"bf16 prompt chunk 8 x 4096 tokens, T = 512, bf16_weights={bf16_weights}, rows {rows}")
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_chunked_prefill_matches_one_pass(dtype):
    """A whole prompt in chunks, as when a swapped-out request's KV is recomputed:
    chunk c attends the request's pages up to its own last token, and the chunks
    together equal one causal pass over the prompt.  Chunks of 256, 256, 83 and 5
    tokens take the shared-tile kernel and then the decode kernel's causal form."""
    banner(f"extend {dtype} chunked prefill 600 = 256 + 256 + 83 + 5")
    n, bounds = 600, [0, 256, 512, 595, 600]
    b = W.extend_batch([n], n, Hq=8, Hkv=2, dtype=dtype, seed=61, device=DEV)  # every token new
    host = HostExtend(b)
    ref = host.oracle()  # [1, n, Hq, d]: causal over the whole prompt
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    outs = []
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        lens_c = torch.tensor([c1], dtype=torch.int32, device=DEV)
        outs.append(pa.paged_attn_extend(b.q[:, c0:c1].contiguous(), b.k_pool, b.v_pool, b.block_tables, lens_c,
                                         b.B, b.scale))
    torch.cuda.synchronize()
    assert_close(host_f32(torch.cat(outs, dim=1)), ref, dtype, "chunked prefill")


@pytest.mark.parametrize("T,bf16_weights,splits", [(5, False, 0), (40, False, 0), (40, True, 0), (16, False, 4),
                                                   (16, True, 2), (24, False, 4), (24, True, 4)])
def test_rising_logits(T, bf16_weights, splits):
    """Logits climbing along the history in stairs of 10 (14.4 in base 2, beyond the
    reference-move threshold of the matrix-core kernels), for the decode kernel's causal
    form (T = 5), the shared-tile kernel (T = 40), and its splits run as two halves or
    four parts of one workgroup, each part with its own reference max until the merge."""
    from tests.test_gpu_decode import _ramp_keys

    banner(f"extend bf16 rising logits T={T} bf16_weights={bf16_weights} splits={splits}")
    b = W.extend_batch([100, 600, 1500], T, Hq=8, Hkv=2, seed=71 + T, device=DEV)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    lens = b.seq_lens.cpu().numpy()
    rows = _ramp_keys(b, b.q[:, -1], b.k_pool, lens, 10.0)  # aimed at the last query token's heads
    for (s, g), r in rows.items():  # the new tokens' K as now in the pool, for the host's re-append
        b.k_new[s, :, g] = r[int(lens[s]) - T:]
    host = HostExtend(b)
    out = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale,
                               bf16_weights=bf16_weights, num_splits=splits)
    torch.cuda.synchronize()
    assert_close(host_f32(out), host.oracle(), torch.bfloat16, f"rising logits T={T}")


def test_speculative_loop_with_rollback():
    """Branches over a shared 1029-token prefix; each step reserves T = 4 draft
    positions (copying a shared partial tail first), appends the drafts, verifies
    them with one paged_attn_extend, then keeps a random number of them and rolls
    the rest back.  Every step's output is compared with dense attention on the
    branch's own accepted history plus its drafts, kept on the host."""
    banner("speculative loop: 4 branches, 10 steps, T=4 drafts, rollback")
    rng = np.random.default_rng(91)
    NB, B, MB, Hq, Hkv, D, T = 256, 16, 80, 16, 4, 128, 4
    scale = float(np.float32(1.0 / np.sqrt(D)))
    bm = pa.BlockManager(NB, B, MB, rng.permutation(NB).astype(np.int32))
    k_pool = torch.full((NB, B, Hkv, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.full_like(k_pool, float("nan"))

    def rand(*shape):
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)

    parent = bm.add_request()
    n0 = 1024 + 5
    bm.reserve(parent, n0)
    tab, _ = bm.export([parent])
    k_hist, v_hist = rand(n0, Hkv, D), rand(n0, Hkv, D)
    t = np.arange(n0)
    blk = torch.as_tensor(tab[0][t // B], dtype=torch.long, device=DEV)
    slot = torch.as_tensor(t % B, dtype=torch.long, device=DEV)
    k_pool[blk, slot] = k_hist.to(DEV)  # prefill placement is test set-up
    v_pool[blk, slot] = v_hist.to(DEV)
    branches = [parent] + [bm.fork(parent) for _ in range(3)]
    hist = {r: (k_hist.clone(), v_hist.clone()) for r in branches}
    copies = 0
    for step in range(10):
        pos, (cs, cd, cn) = bm.prepare_extend(branches, T)
        copies += len(cs)
        tables, lens = bm.export(branches)
        S = len(branches)
        if len(cs):
            pa.kv_cow_copy(k_pool, v_pool, *(torch.as_tensor(x, device=DEV) for x in (cs, cd, cn)), B)
        k_new, v_new, q = rand(S, T, Hkv, D), rand(S, T, Hkv, D), rand(S, T, Hq, D)
        t_tab = torch.as_tensor(tables, device=DEV)
        pa.kv_append_tokens(k_pool, v_pool, k_new.to(DEV), v_new.to(DEV), t_tab, torch.as_tensor(pos, device=DEV), B)
        out = pa.paged_attn_extend(q.to(DEV), k_pool, v_pool, t_tab, torch.as_tensor(lens, device=DEV), B, scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for i, r in enumerate(branches):
            kh = torch.cat([hist[r][0], k_new[i]])
            vh = torch.cat([hist[r][1], v_new[i]])
            assert lens[i] == kh.shape[0] == pos[i] + T
            ref = att.extend_attention(q[i].float().numpy(), kh.float().numpy(), vh.float().numpy(), scale)
            err = float(np.max(np.abs(got[i] - ref)))
            assert np.all(np.isfinite(got[i])) and err <= 5e-3 * float(np.max(np.abs(ref))), (step, i, err)
            keep = int(rng.integers(0, T + 1))  # drafts accepted this step
            bm.truncate(r, int(pos[i]) + keep)
            hist[r] = (kh[: int(pos[i]) + keep], vh[: int(pos[i]) + keep])
        bm.check()
    # the first step copies the shared 5-token tail for all but the last branch
    assert copies >= 3


@pytest.mark.parametrize("T", [4, 24, 40])
def test_table_padding_past_the_history_may_hold_anything(T):
    """Entries at or past ceil(n/B) never address the pools in the several-token
    kernels either (decode-kernel causal form, 4-wave and ping-pong shared-tile
    forms): ids outside the pool there change no output bit."""
    banner(f"extend garbage table padding T={T}")
    lens = [T, T + 1, T + 15, T + 16, T + 33, T + 300]
    b = W.extend_batch(lens, T, Hq=8, Hkv=2, seed=120 + T, device=DEV)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    base = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, b.block_tables, b.seq_lens, b.B, b.scale)
    tab = b.block_tables.cpu().numpy()
    garbage = np.array([-7, b.NB, b.NB + 12345, 2**31 - 1, -2**31], dtype=np.int64)
    for s_, n in enumerate(lens):
        need = -(-n // b.B)
        tab[s_, need:] = garbage[(np.arange(tab.shape[1] - need) + s_) % len(garbage)]
    t2 = torch.as_tensor(tab.astype(np.int32), device=DEV)
    out = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, t2, b.seq_lens, b.B, b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), host_bits(base))
    assert np.all(np.isfinite(host_f32(out)))


@pytest.mark.parametrize("T", [4, 40])
def test_bad_lengths_and_out_of_pool_entries_poison_only_their_request(T):
    """As for the decode: NaN for the request with a bad length or an out-of-pool
    entry inside its history, the oracle's answer for the others (decode-kernel and
    shared-tile variants)."""
    banner(f"extend bad inputs T={T}")
    lens = [60, 90, 50, 45, 120]
    b = W.extend_batch(lens, T, Hq=8, Hkv=2, seed=97 + T, device=DEV)
    host = HostExtend(b)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    ref = host.oracle()
    tab = b.block_tables.clone()
    tab[1, 1] = -9
    ln = b.seq_lens.clone()
    ln[2] = b.MB * b.B + 16
    ln[3] = -1
    out = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, tab, ln, b.B, b.scale)
    torch.cuda.synchronize()
    got = host_f32(out)
    for s_ in (1, 2, 3):
        assert np.all(np.isnan(got[s_])), s_
    for s_ in (0, 4):
        assert_close(got[s_], ref[s_], torch.bfloat16, f"request {s_}")


@pytest.mark.parametrize("G,T,B,bf16_weights", [(4, 9, 16, False), (4, 12, 16, True), (4, 16, 16, False),
                                                (4, 16, 4, False), (4, 16, 64, True), (4, 24, 16, False),
                                                (4, 32, 8, True), (2, 40, 32, False), (1, 100, 16, False)])
def test_two_splits_as_one_workgroup_of_two_halves(G, T, B, bf16_weights):
    """Two splits of the 4-wave shared-tile kernels (one 16-column set per wave
    up to 16 tokens of a 4-head group, the 32-column kernel up to 128 columns)
    run as one workgroup whose two 4-wave halves take a split each and merge in
    LDS: no workspace, no merge kernel.  Requests shorter than a split leave the
    second half nothing of its own (it still passes every barrier); lengths cross
    tile, block and split boundaries; T = 24 leaves a whole wave idle."""
    banner(f"extend two halves G={G} T={T} B={B} bf16_weights={bf16_weights}")
    lens = [T, T + 5, 140, 300, 1000, 1031, 2049, 16 * 64 + 1]
    b = W.extend_batch(lens, T, Hq=2 * G, Hkv=2, B=B, seed=400 + T + B, device=DEV)
    P, ws = pa.paged_attn_extend_plan(b.S, b.Hq, b.Hkv, b.D, b.MB, b.NB, b.dtype, b.B, T, num_splits=2)
    assert (P, ws) == (2, 0)
    check(b, torch.bfloat16, f"two halves T={T} B={B}", num_splits=2, bf16_weights=bf16_weights)


@pytest.mark.parametrize("T", [16, 24])
def test_two_halves_poison_only_their_request(T):
    """An out-of-pool entry in either split's range, a bad length: NaN for that
    request only, through the halves' merge (16-column and 32-column kernels)."""
    banner(f"extend two halves bad inputs T={T}")
    lens = [1500, 1600, 1400, 1700, 1650]
    b = W.extend_batch(lens, T, Hq=8, Hkv=2, seed=431 + T, device=DEV)
    host = HostExtend(b)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    ref = host.oracle()
    tab = b.block_tables.clone()
    tab[1, 3] = -9                 # in the first split
    tab[2, 80] = b.NB + 5          # in the second split
    ln = b.seq_lens.clone()
    ln[3] = -1
    out = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, tab, ln, b.B, b.scale, num_splits=2)
    torch.cuda.synchronize()
    got = host_f32(out)
    for s_ in (1, 2, 3):
        assert np.all(np.isnan(got[s_])), s_
    for s_ in (0, 4):
        assert_close(got[s_], ref[s_], torch.bfloat16, f"request {s_}")


@pytest.mark.parametrize("G,T,B,bf16_weights", [(4, 9, 16, False), (4, 12, 16, True), (4, 16, 16, False),
                                                (4, 16, 4, False), (4, 16, 64, True), (4, 13, 8, False),
                                                (4, 16, 32, False), (2, 32, 32, False), (1, 64, 16, False),
                                                (8, 8, 16, True), (16, 4, 16, False),
                                                (4, 17, 16, False), (4, 20, 16, True), (4, 24, 16, False),
                                                (4, 24, 4, False), (4, 24, 64, True), (4, 21, 8, False),
                                                (4, 24, 32, True), (1, 96, 16, False), (2, 40, 32, False),
                                                (8, 12, 16, True), (16, 6, 16, False)])
def test_four_splits_as_one_workgroup_of_four_parts(G, T, B, bf16_weights):
    """Four splits of up to 64 (token, head) columns per KV head run on the
    32-column kernel as one workgroup of four 2-wave parts, one split each,
    every wave loading 16 rows of each step; 65-96 columns as four 3-wave parts
    (12 waves, q read from LDS, 3 row groups per wave and 2 for the last, the
    states handed over in two rounds).  The parts merge in LDS: no workspace,
    no merge kernel.  Requests shorter than a split leave later parts nothing
    of their own (they still pass every barrier); lengths cross tile, block and
    split boundaries; T = 9, 13 and 17 leave the last wave of each part mostly
    padding columns."""
    banner(f"extend four parts G={G} T={T} B={B} bf16_weights={bf16_weights}")
    lens = [T, T + 5, 140, 300, 1000, 1031, 2049, 16 * 64 + 1]
    b = W.extend_batch(lens, T, Hq=2 * G, Hkv=2, B=B, seed=500 + T + B, device=DEV)
    P, ws = pa.paged_attn_extend_plan(b.S, b.Hq, b.Hkv, b.D, b.MB, b.NB, b.dtype, b.B, T, num_splits=4)
    assert (P, ws) == (4, 0)
    check(b, torch.bfloat16, f"four parts T={T} B={B}", num_splits=4, bf16_weights=bf16_weights)


@pytest.mark.parametrize("T", [12, 16, 24])
def test_four_parts_poison_only_their_request(T):
    """An out-of-pool entry in the first, third or last split's range, a bad
    length: NaN for that request only, through the four parts' merge."""
    banner(f"extend four parts bad inputs T={T}")
    lens = [1500, 1600, 1400, 1700, 1650, 1690]
    b = W.extend_batch(lens, T, Hq=8, Hkv=2, seed=531 + T, device=DEV)
    host = HostExtend(b)
    pa.kv_append_tokens(b.k_pool, b.v_pool, b.k_new, b.v_new, b.block_tables, b.positions, b.B)
    ref = host.oracle()
    P = 4
    assert pa.paged_attn_extend_plan(b.S, b.Hq, b.Hkv, b.D, b.MB, b.NB, b.dtype, b.B, T, num_splits=P) == (4, 0)
    tab = b.block_tables.clone()
    tab[1, 3] = -9                 # in the first split
    tab[2, 60] = b.NB + 5          # in the third split (blocks 54-80 of 107)
    tab[5, 100] = -1               # in the last split
    ln = b.seq_lens.clone()
    ln[3] = -1
    out = pa.paged_attn_extend(b.q, b.k_pool, b.v_pool, tab, ln, b.B, b.scale, num_splits=P)
    torch.cuda.synchronize()
    got = host_f32(out)
    for s_ in (1, 2, 3, 5):
        assert np.all(np.isnan(got[s_])), s_
    for s_ in (0, 4):
        assert_close(got[s_], ref[s_], torch.bfloat16, f"request {s_}")

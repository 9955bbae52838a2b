"""The C-ABI library loads, exports what include/pagedattn.h declares, and rejects
bad host-side arguments before enqueuing anything (CPU; no kernel is launched).

Every call here is built to fail a host-side check.  Pointer arguments are
NULL or fake, so these tests are skipped where a GPU is visible: a check that
wrongly passed must never launch on fake addresses.
"""

import ctypes
import os

import pytest
import torch

import paged_kv_cache_352_amd as pa
from paged_kv_cache_352_amd import _lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_352_amd.build import build

        build()
    return pa.load()


no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer checks run only without a GPU")


def dims(S=4, Hq=8, Hkv=2, D=128, MB=4, NB=16, dtype=pa.PA_BF16, splits=0, ws=None, ws_bytes=0):
    d = pa.make_dims(S, Hq, Hkv, D, MB, NB, dtype, splits)
    if ws is not None:
        d.workspace = ws
        d.workspace_bytes = ws_bytes
    return d


FAKE = ctypes.c_void_p(0x7F0000000000)  # 256-byte aligned, never dereferenced


def decode(lib, d, q=FAKE, k=FAKE, v=FAKE, t=FAKE, n=FAKE, B=16, scale=0.1, out=FAKE):
    return lib.paged_attn_decode(q, k, v, t, n, B, ctypes.c_float(scale), out, None,
                                 ctypes.byref(d) if d is not None else None)


def test_exports_every_declared_symbol(lib):
    names = pa.declared_functions()
    assert {"paged_attn_decode", "kv_append", "kv_cow_copy", "paged_kv_gather", "paged_attn_plan",
            "paged_attn_extend", "paged_attn_extend_plan", "kv_append_tokens", "pa_bm_truncate",
            "paged_attn_decode_append", "paged_attn_workspace_bytes", "paged_attn_order",
            "pa_bm_prepare_extend"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.pa_abi_version() == 4


def test_status_strings(lib):
    for code, name in [(0, "PA_OK"), (-1, "PA_ERR_INVALID_ARG"), (-2, "PA_ERR_UNSUPPORTED"),
                       (-3, "PA_ERR_WORKSPACE"), (-4, "PA_ERR_LAUNCH")]:
        assert lib.pa_status_string(code).decode() == name


def test_plan_is_deterministic_and_covers_table(lib):
    for shape in [(32, 32, 8, 256), (5, 8, 2, 32), (256, 32, 8, 33), (168, 16, 4, 65), (64, 32, 8, 133), (1, 8, 8, 1)]:
        S, Hq, Hkv, MB = shape
        a = pa.paged_attn_plan(S, Hq, Hkv, 128, MB, 10000, torch.bfloat16, 16)
        b = pa.paged_attn_plan(S, Hq, Hkv, 128, MB, 10000, torch.bfloat16, 16)
        assert a == b
        P, ws = a
        assert 1 <= P <= MB
        assert ws == (S * Hq * P * 130 * 4 if P > 1 else 0)
    # float32: up to 4 splits need no workspace (merged in LDS); 16 splits leave 4 groups, 6 splits 2
    assert pa.paged_attn_plan(5, 8, 2, 128, 32, 64, torch.float32, 16, num_splits=4) == (4, 0)
    assert pa.paged_attn_plan(5, 8, 2, 128, 32, 64, torch.float32, 16, num_splits=16) == (16, 5 * 8 * 4 * 130 * 4)
    assert pa.paged_attn_plan(5, 8, 2, 128, 96, 64, torch.float32, 16, num_splits=6) == (6, 5 * 8 * 2 * 130 * 4)
    # forced split counts are honoured (clamped to the table width)
    assert pa.paged_attn_plan(5, 8, 2, 128, 32, 64, torch.float32, 16, num_splits=3)[0] == 3
    assert pa.paged_attn_plan(5, 8, 2, 128, 32, 64, torch.float32, 16, num_splits=1)[0] == 1
    assert pa.paged_attn_plan(5, 8, 2, 128, 4, 64, torch.float32, 16, num_splits=9)[0] == 4


def test_automatic_bf16_splits_are_never_shorter_than_256_tokens(lib):
    # bf16 decode: a table of 19 blocks (304 tokens) stays one split, 32 blocks take two of 256
    assert pa.paged_attn_plan(3, 16, 2, 128, 19, 64, torch.bfloat16, 16)[0] == 1
    assert pa.paged_attn_plan(3, 16, 2, 128, 32, 64, torch.bfloat16, 16)[0] == 2
    assert pa.paged_attn_plan(3, 16, 2, 128, 15, 64, torch.bfloat16, 16)[0] == 1
    for MB in (1, 17, 19, 33, 47, 64, 250):
        P, _ = pa.paged_attn_plan(1, 32, 8, 128, MB, 10000, torch.bfloat16, 16)
        tokens = MB * 16
        assert P == 1 or -(-tokens // P) >= 256, (MB, P)


def test_plan_rejects_bad_shapes(lib):
    p, w = ctypes.c_int32(), ctypes.c_size_t()
    cases = [
        (dims(Hq=6, Hkv=4), INVALID),      # Hq not a multiple of Hkv
        (dims(Hq=6, Hkv=2), UNSUPPORTED),  # group of 3
        (dims(D=64), UNSUPPORTED),
        (dims(Hkv=0), INVALID),
        (dims(S=-1), INVALID),
        (dims(MB=0), INVALID),
        (dims(dtype=7), UNSUPPORTED),
        (dims(splits=-2), INVALID),
    ]
    for d, want in cases:
        assert lib.paged_attn_plan(ctypes.byref(d), 16, ctypes.byref(p), ctypes.byref(w)) == want
        assert lib.pa_last_error().decode() != ""
    for B in (2, 12, 24, 128):  # block sizes are powers of two from 4 to 64
        assert lib.paged_attn_plan(ctypes.byref(dims()), B, ctypes.byref(p), ctypes.byref(w)) == UNSUPPORTED
    for B in (4, 8, 16, 32, 64):
        assert lib.paged_attn_plan(ctypes.byref(dims()), B, ctypes.byref(p), ctypes.byref(w)) == OK
    assert lib.paged_attn_plan(None, 16, ctypes.byref(p), ctypes.byref(w)) == INVALID


@no_gpu
def test_decode_rejects_before_launch(lib):
    assert decode(lib, None) == INVALID
    assert decode(lib, dims(Hq=6, Hkv=2)) == UNSUPPORTED
    assert decode(lib, dims(), q=None) == INVALID
    assert decode(lib, dims(), out=None) == INVALID
    assert decode(lib, dims(), q=ctypes.c_void_p(0x7F0000000008)) == INVALID  # not 16-byte aligned
    assert decode(lib, dims(), scale=float("nan")) == INVALID
    assert decode(lib, dims(), B=24) == UNSUPPORTED
    # a split plan with no workspace, then a too-small and a misaligned one
    d = dims(S=1, Hkv=1, Hq=4, MB=64, splits=4)
    assert decode(lib, d) == WORKSPACE
    d = dims(S=1, Hkv=1, Hq=4, MB=64, splits=4, ws=0x7F0000100000, ws_bytes=100)
    assert decode(lib, d) == WORKSPACE
    d = dims(S=1, Hkv=1, Hq=4, MB=64, splits=4, ws=0x7F0000100010, ws_bytes=1 << 20)
    assert decode(lib, d) == WORKSPACE
    assert "workspace" in lib.pa_last_error().decode()


@no_gpu
def test_unknown_flags_are_rejected_before_launch(lib):
    """pa_dims.flags carries PA_FLAG_BF16_WEIGHTS (1) only; any other bit is refused
    by every attention entry point before anything is enqueued."""
    assert lib.pa_abi_version() == _lib.ABI_VERSION == 4
    for bad in (2, 4, 1 << 30, -1):
        d = dims()
        d.flags = bad
        assert decode(lib, d) == INVALID
        assert "flags" in lib.pa_last_error().decode()
        assert lib.paged_attn_extend(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 16, ctypes.c_float(0.1), FAKE, None,
                                     ctypes.byref(d)) == INVALID
    # the defined bit passes the flag check (and then fails on the NULL q, as without it)
    d = dims()
    d.flags = _lib.FLAG_BF16_WEIGHTS
    assert decode(lib, d, q=None) == INVALID
    assert "NULL" in lib.pa_last_error().decode()


def test_empty_batch_is_a_noop(lib):
    d = dims(S=0)
    assert decode(lib, d, q=None, k=None, v=None, t=None, n=None, out=None) == OK
    assert lib.kv_append(None, None, None, None, None, None, 16, None, ctypes.byref(d)) == OK
    assert lib.kv_cow_copy(FAKE, FAKE, None, None, None, 0, 16, 1, 0, None, ctypes.byref(d)) == OK


@no_gpu
def test_kv_ops_reject_before_launch(lib):
    d = dims()
    assert lib.kv_append(None, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, ctypes.byref(d)) == INVALID
    assert lib.kv_append(FAKE, FAKE, None, FAKE, FAKE, FAKE, 16, None, ctypes.byref(d)) == INVALID
    assert lib.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, ctypes.byref(d)) == INVALID
    assert lib.kv_cow_copy(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 16, 1, 0, None, ctypes.byref(d)) == INVALID
    assert lib.kv_cow_copy(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 16, 0, 0, None, ctypes.byref(d)) == INVALID
    # a layer stride shorter than one layer's pool
    assert lib.kv_cow_copy(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 16, 2, 10, None, ctypes.byref(d)) == INVALID
    assert lib.kv_cow_copy(FAKE, FAKE, None, FAKE, FAKE, 3, 16, 1, 0, None, ctypes.byref(d)) == INVALID
    assert lib.paged_kv_gather(FAKE, FAKE, None, FAKE, 16, FAKE, FAKE, None, ctypes.byref(d)) == INVALID
    # Hkv*d*2 bytes not a multiple of 16
    assert lib.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, ctypes.byref(dims(Hkv=1, D=4))) == UNSUPPORTED
    # the all-layer append: layer count and stride checked like kv_cow_copy's
    app = lambda layers, stride, d=d: lib.kv_append_layers(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, layers, stride,
                                                           None, ctypes.byref(d))
    assert app(0, 0) == INVALID
    assert app(70000, 0) == INVALID
    assert app(2, 10) == INVALID  # stride shorter than one layer's pool
    assert app(2, 16 * 16 * 2 * 128 + 3) == INVALID  # stride not a multiple of 16 bytes
    assert lib.kv_append_layers(FAKE, FAKE, None, FAKE, FAKE, FAKE, 16, 2, 16 * 16 * 2 * 128, None,
                                ctypes.byref(d)) == INVALID
    assert app(2, 0, d=dims(S=0)) == OK  # nothing to append, nothing launched


def test_binding_refuses_host_tensors(lib):
    q = torch.zeros(2, 8, 128)
    k = torch.zeros(4, 16, 2, 128)
    t = torch.zeros(2, 2, dtype=torch.int32)
    n = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(_lib.PagedAttnError):
        pa.paged_attn_decode(q, k, k, t, n, 16, 0.1)


@no_gpu
def test_swap_rejects_bad_arguments(lib):
    d = dims()
    args = lambda n=2, buf=FAKE, layers=1, stride=0: (FAKE, FAKE, FAKE, n, buf, 16, layers, stride, None, ctypes.byref(d))
    assert lib.kv_swap_out(*args(n=-1)) == INVALID
    assert lib.kv_swap_out(*args(buf=None)) == INVALID
    assert lib.kv_swap_in(*args(buf=ctypes.c_void_p(0x7F0000000008))) == INVALID  # misaligned buffer
    assert lib.kv_swap_in(*args(layers=0)) == INVALID
    assert lib.kv_swap_out(*args(layers=2, stride=5)) == INVALID  # stride smaller than one pool
    assert lib.kv_swap_out(*args(n=0)) == OK  # nothing to do, nothing launched


def shared_tile_halves(dt, G, T, P):
    """Two splits of the 4-wave shared-tile kernels (bf16, more tokens than two
    16-column sets hold, at most 128 (token, head) columns) run as one workgroup
    of two halves that merge in LDS: no workspace."""
    if dt != torch.bfloat16:
        return False
    per_wave = 1 if G >= 16 else 16 // G
    return T > 2 * per_wave and T * G <= 128 and P == 2


def shared_tile_quarters(dt, G, T, P):
    """Four splits of the shared-tile case (bf16, more tokens than two 16-column
    sets hold) with at most 64 (token, head) columns, or at most 96 once they
    need two sets per wave, run as one workgroup of four parts of the 32-column
    kernel that merge in LDS: no workspace."""
    if dt != torch.bfloat16:
        return False
    per_wave = 1 if G >= 16 else 16 // G
    return T > 2 * per_wave and (T <= 4 * per_wave or T * G <= 96) and P == 4


def shared_tile_parts(dt, G, T, P):
    return 4 if shared_tile_quarters(dt, G, T, P) else (2 if shared_tile_halves(dt, G, T, P) else 1)


def merged_splits(P, dt):
    """Partial states per output row that reach the split workspace: float32 runs
    groups of up to 4 splits (the next power of two) as the waves of one
    workgroup and merges each group in LDS, so only the groups' states are written."""
    if dt != torch.float32:
        return P
    w = 1
    while w < P and w < 4:
        w *= 2
    return -(-P // w)


def test_extend_plan_matches_decode_at_one_token_and_scales_workspace(lib):
    for S, Hq, Hkv, MB, dt in [(32, 32, 8, 256, torch.bfloat16), (5, 8, 2, 32, torch.float32), (7, 16, 1, 9, torch.bfloat16),
                               (2, 8, 2, 4096, torch.float32)]:
        assert pa.paged_attn_extend_plan(S, Hq, Hkv, 128, MB, 10000, dt, 16, 1) == pa.paged_attn_plan(
            S, Hq, Hkv, 128, MB, 10000, dt, 16)
        for T in (2, 4, 7, 16, 33):
            for w in (False, True):
                P, ws = pa.paged_attn_extend_plan(S, Hq, Hkv, 128, MB, 10000, dt, 16, T, bf16_weights=w)
                Pm = 1 if shared_tile_parts(dt, Hq // Hkv, T, P) > 1 else merged_splits(P, dt)
                assert P >= 1 and ws == (S * T * Hq * Pm * 130 * 4 if Pm > 1 else 0)
            for P0 in (2, 3, 4, 5):
                P, ws = pa.paged_attn_extend_plan(S, Hq, Hkv, 128, MB, 10000, dt, 16, T, num_splits=P0)
                Pm = 1 if shared_tile_parts(dt, Hq // Hkv, T, P) > 1 else merged_splits(P, dt)
                assert ws == (S * T * Hq * Pm * 130 * 4 if Pm > 1 else 0)
            # forced splits are honoured as in the one-token plan
            assert pa.paged_attn_extend_plan(S, Hq, Hkv, 128, MB, 10000, dt, 16, T, num_splits=2)[0] == min(2, MB)
    p, w = ctypes.c_int32(), ctypes.c_size_t()
    assert lib.paged_attn_extend_plan(ctypes.byref(dims()), 16, 0, ctypes.byref(p), ctypes.byref(w)) == INVALID


def test_extend_plan_takes_four_parts_for_one_set_per_wave_with_default_weights(lib):
    """32 requests of 4096 tokens, 4-head groups: the automatic plan for 13-16
    query tokens (49-64 columns per KV head) takes 4 splits, run as the parts
    of one workgroup (no workspace); with PA_FLAG_BF16_WEIGHTS, and for 9-12
    tokens, it keeps 2 (two halves, no workspace); 17-24 tokens (65-96
    columns) take 4 with either weights (three waves per part); 8 and 25-32
    tokens are unchanged; a history too short for four 256-slot splits is not
    promoted."""
    plan = lambda T, w=False, MB=256, S=32: pa.paged_attn_extend_plan(S, 32, 8, 128, MB, 40000, torch.bfloat16, 16,
                                                                      T, bf16_weights=w)
    for T in range(13, 17):
        assert plan(T) == (4, 0)
        assert plan(T, True) == (2, 0)
    for T in range(9, 13):  # the second 32-column wave at most half full: two halves
        assert plan(T) == plan(T, True) == (2, 0)
    for T in range(17, 25):
        assert plan(T) == plan(T, True) == (4, 0)
    for T in (25, 32):
        assert plan(T) == plan(T, True) == (2, 0)
    assert plan(8) == plan(8, True)
    assert plan(16, MB=32) == plan(16, True, MB=32)  # 512 slots: at most 2 splits of 256
    # G = 1, 2, 8 and 16 take the same rule on their own column counts
    for Hq, T, P in ((8, 40, 2), (8, 49, 4), (16, 24, 2), (16, 25, 4), (64, 6, 2), (64, 7, 4), (128, 3, 2),
                     (128, 4, 4), (8, 96, 4), (8, 97, 2), (16, 48, 4), (16, 49, 2), (64, 12, 4), (64, 13, 2),
                     (128, 6, 4), (128, 7, 2)):
        assert pa.paged_attn_extend_plan(32, Hq, 8, 128, 256, 40000, torch.bfloat16, 16, T) == (P, 0), (Hq, T)


@no_gpu
def test_extend_and_token_append_reject_before_launch(lib):
    def extend(d, T=4, q=FAKE, out=FAKE, B=16):
        return lib.paged_attn_extend(q, FAKE, FAKE, FAKE, FAKE, T, B, ctypes.c_float(0.1), out, None,
                                     ctypes.byref(d))
    assert extend(dims(), T=0) == INVALID
    assert extend(dims(), q=None) == INVALID
    assert extend(dims(Hq=6, Hkv=2)) == UNSUPPORTED
    assert extend(dims(), B=12) == UNSUPPORTED
    assert extend(dims(S=1, Hkv=1, Hq=4, MB=64, splits=4)) == WORKSPACE
    assert extend(dims(S=0), q=None, out=None) == OK
    d = dims()
    assert lib.kv_append_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, None, ctypes.byref(d)) == INVALID
    assert lib.kv_append_tokens(FAKE, FAKE, None, FAKE, FAKE, FAKE, 3, 16, None, ctypes.byref(d)) == INVALID
    assert lib.kv_append_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 0, None, ctypes.byref(d)) == INVALID


@no_gpu
def test_decode_append_rejects_before_launch(lib):
    d = dims()
    f = lambda kn=FAKE, vn=FAKE, pos=FAKE, B=16: lib.paged_attn_decode_append(
        FAKE, FAKE, FAKE, kn, vn, FAKE, pos, FAKE, B, ctypes.c_float(0.1), FAKE, None, ctypes.byref(d))
    assert f(kn=None) == INVALID
    assert f(pos=None) == INVALID
    assert f(vn=ctypes.c_void_p(0x7F0000000008)) == INVALID  # misaligned
    assert f(B=12) == UNSUPPORTED
    e = dims(S=0)
    assert lib.paged_attn_decode_append(None, None, None, None, None, None, None, None, 16, ctypes.c_float(0.1),
                                        None, None, ctypes.byref(e)) == OK


# The five decode workloads' shapes (S, Hq, Hkv, MB, NB, dtype) at B = 16.
CONFIG_SHAPES = [
    (5, 8, 2, 32, 64, torch.float32),        # 5 sequences of 37-511 tokens, fp32
    (32, 32, 8, 256, 8192, torch.bfloat16),  # 32 x 4096 tokens
    (256, 32, 8, 33, 12288, torch.bfloat16),  # 256 mixed lengths (one layer)
    (64, 32, 8, 133, 1024, torch.bfloat16),  # prefix sharing
    (168, 16, 4, 65, 10922, torch.bfloat16),  # 168 x 1025 tokens (one layer)
]


def test_workspace_bytes_agrees_with_plan_on_the_workload_shapes(lib):
    size_max = ctypes.c_size_t(-1).value
    for S, Hq, Hkv, MB, NB, dt in CONFIG_SHAPES:
        for splits in (0, 1, 2, 3, 4, 7, 16, 64):
            d = pa.make_dims(S, Hq, Hkv, 128, MB, NB, dt, splits)
            P, want = pa.paged_attn_plan(S, Hq, Hkv, 128, MB, NB, dt, 16, num_splits=splits)
            got = lib.paged_attn_workspace_bytes(ctypes.byref(d), 16)
            assert got == want, (S, splits, got, want)
            assert got == pa.paged_attn_workspace_bytes(S, Hq, Hkv, 128, MB, NB, dt, 16, num_splits=splits)
            assert got == (S * Hq * merged_splits(P, dt) * 130 * 4 if merged_splits(P, dt) > 1 else 0)
    # rejected arguments: SIZE_MAX and a reason, for the same cases paged_attn_plan refuses
    for d in (dims(Hq=6, Hkv=4), dims(D=64), dims(splits=-2), dims(MB=0)):
        assert lib.paged_attn_workspace_bytes(ctypes.byref(d), 16) == size_max
        assert lib.pa_last_error().decode() != ""
    assert lib.paged_attn_workspace_bytes(ctypes.byref(dims()), 12) == size_max
    assert lib.paged_attn_workspace_bytes(None, 16) == size_max
    with pytest.raises(pa.PagedAttnError):
        pa.paged_attn_workspace_bytes(4, 6, 4, 128, 4, 16, torch.bfloat16, 16)
    assert lib.paged_attn_workspace_bytes(ctypes.byref(dims()), 16) == 0 and lib.pa_last_error().decode() == ""


def test_forced_split_counts_round_to_whole_units(lib):
    # MB * B = 160 slots at B = 16 is 10 units of 16: 6 or 7 splits of ceil(10/P) units leave 5
    for P0, want in [(1, 1), (2, 2), (3, 3), (4, 4), (5, 5), (6, 5), (7, 5), (9, 5), (10, 10), (40, 10)]:
        assert pa.paged_attn_plan(3, 8, 2, 128, 10, 64, torch.bfloat16, 16, num_splits=P0)[0] == want, P0


@no_gpu
def test_noalloc_decode_refuses_before_launch(lib):
    def call(d):
        return lib.paged_attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 16, ctypes.c_float(0.1), FAKE, None,
                                             ctypes.byref(d) if d is not None else None)

    assert call(None) == INVALID
    assert call(dims(Hq=6, Hkv=4)) == INVALID
    assert call(dims(D=64)) == UNSUPPORTED
    # 64 requests x 32 heads in 19 splits need 20.2 MB of partial states: more than the static scratch
    d = pa.make_dims(64, 32, 8, 128, 38, 4096, pa.PA_BF16, 32)
    assert pa.paged_attn_plan(64, 32, 8, 128, 38, 4096, torch.bfloat16, 16, num_splits=32)[1] > pa.NOALLOC_SCRATCH_BYTES
    assert call(d) == WORKSPACE
    assert "static scratch" in lib.pa_last_error().decode()
    assert call(dims(S=0)) == OK  # nothing to do, nothing launched


def test_pa_dims_mirror_matches_the_c_layout(tmp_path):
    """The binding's PaDims has the size and field offsets of the header's pa_dims
    (checked with the host C compiler against include/pagedattn.h)."""
    import shutil
    import subprocess
    from paged_kv_cache_352_amd._lib import PaDims

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    names = [f[0] for f in PaDims._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'  printf("%zu\\n", offsetof(pa_dims, {n}));\n' for n in names)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "pagedattn.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(pa_dims));\n' + body + '  return 0;\n}\n')
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(PaDims)
    assert got[1:] == [getattr(PaDims, n).offset for n in names]


def test_order_rejections_before_launch(lib):
    """paged_attn_order: S = 0 is a no-op, bad arguments fail before any launch."""
    fn = lib.paged_attn_order
    assert fn(None, 0, None, None) == 0
    assert fn(None, -1, None, None) == -1
    assert fn(None, 4, None, None) == -1
    assert "required" in lib.pa_last_error().decode()
    fake = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    assert fn(fake, 65537, fake, None) == -2
    assert "65536" in lib.pa_last_error().decode()

"""Host-side checks of the C-ABI library (no GPU work is enqueued).

The library loads without a GPU; these tests cover the exported symbols,
argument validation (which returns before any HIP call), the selector's plan,
the tile-traffic model against the table printed by page "Operator &
Runtime" §5.2.2, and the workgroup -> tile map (a bijection).
"""
import ctypes
import os
import re

import pytest

import dense_gemm_05_amd as g5
from dense_gemm_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(g5.LIB_PATH):
        from dense_gemm_05_amd.build import build_library
        build_library()
    return g5.lib()


def test_exports_every_declared_symbol(L):
    with open(os.path.join(ROOT, "include", "gemm05.h")) as fh:
        text = fh.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gemm_[a-z_0-9]+)\s*\(", text, re.M))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5):
        assert g5.status_string(st).startswith("GEMM_")
    assert "unknown" in g5.status_string(7)


CR = g5.GEMM_WORKSPACE_COUNTER_BYTES   # the workspace's counter region


def ws_bytes(part=0, rows_a=0, rows_b=0):
    """Workspace a plan needs (include/gemm05.h, gemm_run): the counter region
    counters, then the partial sums and the realigned row copies, each
    rounded up to 256 bytes; nothing when none of them is needed."""
    r = lambda b: (b + 255) // 256 * 256
    return 0 if part == rows_a == rows_b == 0 else CR + r(part) + r(rows_a) + r(rows_b)


P = 0x7F0000000000  # fake, well-aligned, non-overlapping addresses (never dereferenced)
A_ADDR, B_ADDR, C_ADDR = P, P + (1 << 34), P + (2 << 34)


def call_bf16(L, M, N, K, a=A_ADDR, lda=None, b=B_ADDR, ldb=None, c=C_ADDR, ldc=None, ct=0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return L.gemm_bf16(M, N, K, a, lda, b, ldb, c, ldc, ct, None)


@pytest.mark.parametrize("args", [
    dict(M=-1, N=4, K=4), dict(M=4, N=-1, K=4), dict(M=4, N=4, K=-2),
    dict(M=4, N=4, K=8, lda=7), dict(M=4, N=8, K=4, ldb=7), dict(M=4, N=8, K=4, ldc=7),
    dict(M=4, N=4, K=4, a=0), dict(M=4, N=4, K=4, b=0), dict(M=4, N=4, K=4, c=0),
    dict(M=4, N=4, K=4, ct=2), dict(M=4, N=4, K=4, ct=-1),
    dict(M=4, N=4, K=4, c=A_ADDR + 8),            # C overlaps A
    dict(M=4, N=4, K=4, c=B_ADDR),                # C overlaps B
])
def test_invalid_arguments_rejected_before_launch(L, args):
    assert call_bf16(L, **args) == g5.GEMM_ERR_INVALID_ARG


def test_invalid_sgemm_and_batched(L):
    assert L.gemm_sgemm(4, 4, 4, 0, 4, B_ADDR, 4, C_ADDR, 4, None) == g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_sgemm(4, 4, 4, A_ADDR, 3, B_ADDR, 4, C_ADDR, 4, None) == g5.GEMM_ERR_INVALID_ARG
    # batch entries of C overlap: strideC < (M-1)*ldc + N
    assert L.gemm_bf16_batched(2, 4, 4, 4, A_ADDR, 4, 16, B_ADDR, 4, 16, C_ADDR, 4, 15, 0, None) == \
        g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_bf16_batched(-1, 4, 4, 4, A_ADDR, 4, 16, B_ADDR, 4, 16, C_ADDR, 4, 16, 0, None) == \
        g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_bf16_batched(2, 4, 4, 4, A_ADDR, 4, -16, B_ADDR, 4, 16, C_ADDR, 4, 16, 0, None) == \
        g5.GEMM_ERR_INVALID_ARG


def test_empty_problems_are_noops_without_device(L):
    # M, N or batch of zero: nothing is enqueued, even with NULL pointers.
    assert L.gemm_bf16(0, 5, 5, None, 5, None, 5, None, 5, 0, None) == g5.GEMM_OK
    assert L.gemm_bf16(5, 0, 5, None, 5, None, 0, None, 0, 0, None) == g5.GEMM_OK
    assert L.gemm_sgemm(0, 0, 0, None, 0, None, 0, None, 0, None) == g5.GEMM_OK
    assert L.gemm_bf16_batched(0, 4, 4, 4, None, 4, 0, None, 4, 0, None, 4, 0, 0, None) == g5.GEMM_OK


def test_k_zero_plans_a_fill(L):
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 3, 5, 0)
    assert st == 0 and p.name == b"zero"


def test_force_config_unsupported(L, monkeypatch):
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "f32_128x128")
    st, _ = g5.plan_query(g5.GEMM_OP_BF16, 64, 64, 64)
    assert st == g5.GEMM_ERR_UNSUPPORTED
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "no_such_config")
    st, _ = g5.plan_query(g5.GEMM_OP_BF16, 64, 64, 64)
    assert st == g5.GEMM_ERR_UNSUPPORTED
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "decode_64")
    st, _ = g5.plan_query(g5.GEMM_OP_BF16, 64, 64, 64)   # M > 16
    assert st == g5.GEMM_ERR_UNSUPPORTED
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "generic")
    st, p = g5.plan_query(g5.GEMM_OP_SGEMM, 64, 64, 64)
    assert st == 0 and p.name == b"generic"
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "f32_32x32_wholek")
    for (M, N, K) in ((100, 256, 256), (256, 256, 288), (256, 250, 256)):   # M % 32, K > 256, N % 32
        st, _ = g5.plan_query(g5.GEMM_OP_SGEMM, M, N, K)
        assert st == g5.GEMM_ERR_UNSUPPORTED
    st, _ = g5.plan_query(g5.GEMM_OP_SGEMM, 256, 256, 256, lda=258)   # A rows 8-byte aligned
    assert st == g5.GEMM_ERR_UNSUPPORTED
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "decode_splitk")
    for (M, N, K) in ((4, 256, 31), (4, 250, 64)):            # K % 32, N % 128
        st, _ = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
        assert st == g5.GEMM_ERR_UNSUPPORTED
    st, _ = g5.plan_query(g5.GEMM_OP_BF16, 4, 256, 64, lda=72)  # X rows 144 bytes apart: 16-byte aligned
    assert st == 0
    st, _ = g5.plan_query(g5.GEMM_OP_BF16, 4, 256, 64, lda=68)  # 136 bytes: not 16-byte aligned
    assert st == g5.GEMM_ERR_UNSUPPORTED


def test_selector_choices_for_the_workloads(L):
    # FFN projection: 256x192 tiles give 4 x 64 = 256 workgroups, one per CU.
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.grid == 256 and p.even == 1
    # decode rows go to the small-M path, whatever M <= 16 is: 128-column
    # strips with K split in 2 (96 x 2 workgroups) when N % 128 == 0 and the
    # rows are 16-byte aligned; else whole-K strips of 64 columns.  M = 1:
    # the two slices meet in exchange slots, one word per output inside the
    # counter region (no partial-sum buffer) for every M <= 16 here
    for M in (1, 4, 16):
        st, p = g5.plan_query(g5.GEMM_OP_BF16, M, 12288, 4096)
        assert st == 0 and p.family == 4 and p.name == b"decode_splitk" and p.grid == 96 * 2
        want = CR if M * 12288 * 4 <= CR else ws_bytes(96 * 2 * 16 * 128 * 4)
        assert p.variant == 1 and p.workspace_bytes == want, (M, p.workspace_bytes)
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 4, 12290, 4096)
    assert st == 0 and p.name == b"decode_64" and p.variant == 0 and p.workspace_bytes == 0
    # 192 or more strips: one slice each, stored directly (no partial sums,
    # no workspace), 256 bytes of each W row per workgroup -- faster than
    # the whole-K 64-column strips (N = 24576: 35.8 against 44.2 us)
    for N, grid in ((24576, 192), (32768, 256)):
        for with_ws in (True, False):
            st, p = g5.plan_query(g5.GEMM_OP_BF16, 1, N, 4096, with_workspace=with_ws)
            assert st == 0 and p.name == b"decode_splitk" and p.grid == grid and p.workspace_bytes == 0
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1, 12288, 4096, with_workspace=False)   # 96 strips: too few
    assert st == 0 and p.name == b"decode_64" and p.grid == 192
    # a bf16 4096^3 product: 256x256 tiles fill the 256 CUs exactly once
    # (256x192 would need 352 tiles, two waves; measured 116.6 against
    # 164.9 us); an output with too few large tiles for the 256 CUs takes
    # 128x128 tiles, the least operand bytes per CU (2048x2048x8192: 93.7
    # against 149.7 us with 256x192; the 1024x1536x4096 shard of an 8-way
    # split FFN: 45.4 against 78.5 us)
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 4096, 4096, 4096)
    assert st == 0 and p.name == b"bf16_256x256" and p.grid == 256 and p.variant == 1
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 8192, 4096, 2048)
    assert st == 0 and p.name == b"bf16_256x256" and p.grid == 512
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 2048, 2048, 8192)
    assert st == 0 and p.name == b"bf16_128x128" and p.grid == 256
    # ... and with K split in 2 over workgroups (96 tiles -> 192 workgroups;
    # the slices' FP32 tiles and a counter per tile in the workspace)
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1024, 1536, 4096)
    assert st == 0 and p.name == b"bf16_128x128" and p.ksplit == 2 and p.grid == 192
    assert p.workspace_bytes == ws_bytes(96 * 2 * 128 * 128 * 4)
    st, p = g5.plan_query(g5.GEMM_OP_SGEMM, 4096, 4096, 4096)
    assert st == 0 and p.family == 3 and p.even == 1
    # FP32 256^3: 32x32 tiles with all of K staged at once; K = 288 (9 slabs)
    # or a 4096^3 problem go to the double-buffered kernels
    st, p = g5.plan_query(g5.GEMM_OP_SGEMM, 256, 256, 256)
    assert st == 0 and p.name == b"f32_32x32_wholek" and p.grid == 64 and p.variant == 1
    st, p = g5.plan_query(g5.GEMM_OP_SGEMM, 256, 256, 288)
    assert st == 0 and p.name == b"f32_64x64"
    # batched scores, K = 128 (4 stages): 128x128 tiles, two workgroups per CU
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1024, 1024, 128, batch=32, c_type=1)
    assert st == 0 and p.name == b"bf16_128x128" and p.grid == 32 * 8 * 8 and p.variant == 1
    # ragged: K=4100 bf16 rows are only 8-byte aligned; the product is large,
    # so A's rows are first copied to 4104-element (16-byte aligned) rows
    # and the masked ring kernel copies A 16 bytes per lane (variant 2)
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1000, 12280, 4100, c_type=1)
    assert st == 0 and p.family == 2 and p.even == 0 and p.vec_a == 16 and p.vec_b == 16
    assert p.variant == 2 and p.workspace_bytes == ws_bytes(0, 1000 * 4104 * 2)
    # a small product keeps A as it is (4-byte copies, variant 3)
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 300, 392, 262)
    assert st == 0 and p.variant == 3 and p.vec_a == 4 and p.workspace_bytes == 0
    # every plan fits the 160 KiB LDS of a gfx950 CU
    for args in [(1024, 12288, 4096), (1000, 12280, 4100), (17, 33, 65)]:
        st, p = g5.plan_query(g5.GEMM_OP_BF16, *args)
        assert p.lds_bytes <= 160 * 1024


def _golden_rows():
    rows, extra = [], {}
    with open(os.path.join(GOLDEN, "op_runtime_5_2_2_tile_traffic.txt")) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] in ("flops", "once_MiB"):
                extra[parts[0]] = int(parts[1])
            else:
                rows.append((int(parts[0]), int(parts[1]), int(parts[2]), int(parts[3]), float(parts[4])))
    return rows, extra


def test_traffic_model_reproduces_op_runtime_table(L):
    M, K, N = 1024, 4096, 12288
    rows, extra = _golden_rows()
    flops = 2 * M * K * N
    assert flops == extra["flops"]
    once = (2 * (M * K + K * N + M * N)) / 2 ** 20
    assert once == extra["once_MiB"]
    for m, n, kib, mib, fpb in rows:
        assert L.gemm_model_local_bytes(m, n, 32, 2) == kib * 1024
        v = L.gemm_model_traffic_bytes(M, N, K, m, n, 2)
        assert v == mib * 2 ** 20
        # The page's intensity column is 103e9 FLOP (its rounded figure) over V,
        # to one decimal; the exact 2MKN gives the same within 0.06.
        assert round(103e9 / v, 1) == fpb
        assert abs(flops / v - fpb) < 0.06


def test_tile_map_is_a_bijection(L):
    i64 = ctypes.c_int64
    b, tm, tn = i64(), i64(), i64()
    for batch, tiles_m, tiles_n, group in [(1, 4, 64, 4), (1, 7, 5, 3), (3, 3, 11, 8), (2, 13, 9, 8),
                                           (1, 1, 1, 1), (32, 4, 6, 4), (1, 16, 16, 8), (5, 1, 13, 1),
                                           (1, 4, 64, 0), (3, 3, 11, 0), (1, 4, 64, -4), (2, 13, 9, -8)]:
        seen = set()
        total = batch * tiles_m * tiles_n
        for w in range(total):
            assert L.gemm_tile_map(w, batch, tiles_m, tiles_n, group, ctypes.byref(b), ctypes.byref(tm),
                                   ctypes.byref(tn)) == 0
            assert 0 <= b.value < batch and 0 <= tm.value < tiles_m and 0 <= tn.value < tiles_n
            seen.add((b.value, tm.value, tn.value))
        assert len(seen) == total
        assert L.gemm_tile_map(total, batch, tiles_m, tiles_n, group, ctypes.byref(b), ctypes.byref(tm),
                               ctypes.byref(tn)) == -1


def test_tile_map_gives_each_xcd_a_compact_block(L):
    """FFN grid (4 x 64 tiles of 256x192): the 32 workgroups on XCD x
    (ids x, x+8, ...) cover all 4 row tiles of 8 adjacent column tiles."""
    i64 = ctypes.c_int64
    b, tm, tn = i64(), i64(), i64()
    for x in range(8):
        cols, rowset = set(), set()
        for w in range(x, 256, 8):
            L.gemm_tile_map(w, 1, 4, 64, 4, ctypes.byref(b), ctypes.byref(tm), ctypes.byref(tn))
            cols.add(tn.value)
            rowset.add(tm.value)
        assert rowset == {0, 1, 2, 3} and cols == set(range(8 * x, 8 * x + 8))


def test_tile_map_diagnostic_orders(L):
    """The orders the XCD-aware map is compared with: group 0 is plain
    row-major (workgroup w -> tile row w / tiles_n, column w % tiles_n); a
    negative group is the column-band walk without the per-XCD gathering,
    so XCD x then holds every 8th tile of the walk, spread over 32 column
    tiles of the FFN grid instead of 8."""
    i64 = ctypes.c_int64
    b, tm, tn = i64(), i64(), i64()
    for w in range(256):
        L.gemm_tile_map(w, 1, 4, 64, 0, ctypes.byref(b), ctypes.byref(tm), ctypes.byref(tn))
        assert (tm.value, tn.value) == (w // 64, w % 64)
        L.gemm_tile_map(w, 1, 4, 64, -4, ctypes.byref(b), ctypes.byref(tm), ctypes.byref(tn))
        assert (tm.value, tn.value) == (w % 4, w // 4)
    for x in range(8):
        cols = set()
        for w in range(x, 256, 8):
            L.gemm_tile_map(w, 1, 4, 64, -4, ctypes.byref(b), ctypes.byref(tm), ctypes.byref(tn))
            cols.add(tn.value)
        assert len(cols) == 32


@pytest.mark.parametrize("M,N,K,batch", [(1, 12288, 4096, 1), (5, 1664, 4160, 1), (16, 384, 1024, 3),
                                         (9, 1024, 1024, 5), (1, 256, 8192, 1)])
def test_split_small_m_workspace_covers_every_slot(M, N, K, batch):
    """The split small-M kernel's workgroup (strip, slice) of batch entry b
    writes partial-sum slot (b*strips + strip)*KS + slice of 16 x 128 floats
    and counter b*strips + strip; the workspace the plan reports must hold
    the largest of each, for the KS the launch uses (grid = strips*KS*batch).
    Two slices whose batch x M x N outputs fit the counter region
    meet in one exchange word per output there instead."""
    st, p = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, batch=batch)
    assert st == 0 and p.name == b"decode_splitk", p.name
    strips = N // 128
    ks = p.grid // (strips * batch)
    assert p.grid == strips * ks * batch and 2 <= ks <= 8
    if ks == 2 and batch * M * N * 4 <= CR:
        assert p.workspace_bytes == CR
        return
    top_slot = ((batch - 1) * strips + strips - 1) * ks + ks - 1
    top_cnt = (batch - 1) * strips + strips - 1
    assert (top_cnt + 1) * 4 <= CR and CR + (top_slot + 1) * 16 * 128 * 4 <= p.workspace_bytes


def call_fused(L, op, M, N, K, a=A_ADDR, lda=None, b=B_ADDR, ldb=None, c=C_ADDR, ldc=None):
    lda = K if lda is None else lda
    ldb = (N if op == "silu" else 2 * N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    fn = L.gemm_bf16_silu if op == "silu" else L.gemm_bf16_swiglu
    return fn(M, N, K, a, lda, b, ldb, c, ldc, None)


@pytest.mark.parametrize("op", ["silu", "swiglu"])
def test_fused_arguments(L, op):
    """Fused epilogues: the same validation as gemm_bf16 with B spanning 2N
    columns for SwiGLU; unaligned output rows or N % 8 are unsupported."""
    nb = 1 if op == "silu" else 2
    assert call_fused(L, op, -1, 8, 4) == g5.GEMM_ERR_INVALID_ARG
    assert call_fused(L, op, 4, 8, 4, ldb=nb * 8 - 1) == g5.GEMM_ERR_INVALID_ARG
    assert call_fused(L, op, 4, 8, 4, lda=3) == g5.GEMM_ERR_INVALID_ARG
    assert call_fused(L, op, 4, 8, 4, ldc=7) == g5.GEMM_ERR_INVALID_ARG
    assert call_fused(L, op, 4, 8, 4, b=0) == g5.GEMM_ERR_INVALID_ARG
    # C starting inside B's last row: overlaps only if B spans nb*N columns
    assert call_fused(L, op, 4, 8, 4, c=B_ADDR + (3 * nb * 8 + nb * 8 - 4) * 2) == g5.GEMM_ERR_INVALID_ARG
    assert call_fused(L, op, 4, 12, 4) == g5.GEMM_ERR_UNSUPPORTED          # N % 8
    assert call_fused(L, op, 4, 8, 4, c=C_ADDR + 2) == g5.GEMM_ERR_UNSUPPORTED  # C rows 2-byte aligned
    assert call_fused(L, op, 0, 8, 4) == g5.GEMM_OK                          # empty: nothing to do
    opc = g5.GEMM_OP_BF16_SILU if op == "silu" else g5.GEMM_OP_BF16_SWIGLU
    st, p = g5.plan_query(opc, 4, 8, 0)
    assert st == 0 and p.family == 1                                         # K = 0: fill with zeros
    st, p = g5.plan_query(opc, 4, 8, 4, batch=2)
    assert st == 0 and p.family == 4                                         # batched, small M: small-M kernels
    st, p = g5.plan_query(opc, 32, 8, 4, batch=2)
    assert st == 0 and p.family == 2                                         # batched (e.g. MoE experts)
    st, _ = g5.plan_query(opc, 4, 8, 4, batch=2, sC=8 * 4 - 1)
    assert st == g5.GEMM_ERR_INVALID_ARG                                     # output entries overlap


def test_swiglu_e4m3_arguments(L):
    """E4M3FN SwiGLU output: the range must be finite and positive; the
    output type belongs to SwiGLU alone; output rows are bytes, so 16-byte
    aligned rows need ldz % 16 == 0 (N = 8 with ldz = 8 is unsupported where
    bf16 rows of 16 bytes were fine)."""
    f = L.gemm_bf16_swiglu_e4m3
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert f(4, 16, 4, A_ADDR, 4, B_ADDR, 32, C_ADDR, 16, bad, None) == g5.GEMM_ERR_INVALID_ARG
    assert f(4, 16, 4, A_ADDR, 4, B_ADDR, 31, C_ADDR, 16, 1.0, None) == g5.GEMM_ERR_INVALID_ARG   # ldw < 2N
    assert f(4, 16, 4, A_ADDR, 4, B_ADDR, 32, C_ADDR, 15, 1.0, None) == g5.GEMM_ERR_INVALID_ARG   # ldz < N
    assert f(4, 8, 4, A_ADDR, 4, B_ADDR, 16, C_ADDR, 8, 1.0, None) == g5.GEMM_ERR_UNSUPPORTED     # 8-byte rows
    assert f(4, 16, 4, A_ADDR, 4, B_ADDR, 32, C_ADDR + 8, 16, 1.0, None) == g5.GEMM_ERR_UNSUPPORTED
    assert f(0, 16, 4, A_ADDR, 4, B_ADDR, 32, C_ADDR, 16, 1.0, None) == g5.GEMM_OK               # empty
    # the codes take N bytes per row: C may start N bytes (not 2N) after B's end
    b_end = B_ADDR + (3 * 32 + 32) * 2
    assert f(4, 16, 4, A_ADDR, 4, B_ADDR, 32, b_end - 8, 16, 1.0, None) == g5.GEMM_ERR_INVALID_ARG
    fb = L.gemm_bf16_swiglu_e4m3_batched
    assert fb(2, 4, 16, 4, A_ADDR, 4, 16, B_ADDR, 32, 128, C_ADDR, 16, 63, 1.0, None) == g5.GEMM_ERR_INVALID_ARG
    assert fb(2, 4, 16, 4, A_ADDR, 4, 16, B_ADDR, 32, 128, C_ADDR, 16, 64, 0.0, None) == g5.GEMM_ERR_INVALID_ARG
    # GEMM_OUT_E4M3 is SwiGLU's alone
    for op in (g5.GEMM_OP_BF16, g5.GEMM_OP_BF16_NT, g5.GEMM_OP_FP8_NT, g5.GEMM_OP_BF16_AFFINE, g5.GEMM_OP_BF16_TN):
        st, _ = g5.plan_query(op, 64, 64, 64, c_type=g5.GEMM_OUT_E4M3)
        assert st == g5.GEMM_ERR_INVALID_ARG, op
    # SiLU ignores c_type (bf16 always), as before
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SILU, 64, 64, 64, c_type=g5.GEMM_OUT_E4M3)
    assert st == 0
    # gemm_run: the range travels in alpha
    args = (g5.GEMM_OP_BF16_SWIGLU, 1, 4, 16, 4, A_ADDR, 4, 0, B_ADDR, 32, 0, C_ADDR, 16, 0, g5.GEMM_OUT_E4M3)
    assert L.gemm_run(*args, 0.0, None, 0.0, None, None, None, 0, None) == g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_run(*args[:1], 0, *args[2:], 1.0, None, 0.0, None, None, None, 0, None) == g5.GEMM_OK


def test_act_chain_arguments(L):
    """gemm_act_chain validates before any device call: the step, sizes,
    pointers, strides, element alignment, the output overlapping an input,
    and the range of the quantizing steps (ignored by the others)."""
    f = L.gemm_act_chain
    G, U, O = A_ADDR, B_ADDR, C_ADDR
    INV = g5.GEMM_ERR_INVALID_ARG
    assert f(5, 4, 16, G, 16, U, 16, O, 16, 1.0, None) == INV                  # unknown step
    assert f(-1, 4, 16, G, 16, U, 16, O, 16, 1.0, None) == INV
    assert f(g5.GEMM_ACT_SILU, -1, 16, G, 16, None, 0, O, 16, 1.0, None) == INV
    assert f(g5.GEMM_ACT_SILU, 4, 16, G, 15, None, 0, O, 16, 1.0, None) == INV  # ld0 < N
    assert f(g5.GEMM_ACT_SILU, 4, 16, G, 16, None, 0, O, 15, 1.0, None) == INV  # ldo < N
    assert f(g5.GEMM_ACT_MUL, 4, 16, G, 16, None, 16, O, 16, 1.0, None) == INV  # missing U
    assert f(g5.GEMM_ACT_MUL, 4, 16, G, 16, U, 15, O, 16, 1.0, None) == INV     # ld1 < N
    assert f(g5.GEMM_ACT_SILU, 4, 16, G + 1, 16, None, 0, O, 16, 1.0, None) == INV   # odd bf16 address
    assert f(g5.GEMM_ACT_SILU, 4, 16, G, 16, None, 0, O + 1, 16, 1.0, None) == INV   # odd bf16 output
    assert f(g5.GEMM_ACT_SILU, 4, 16, G, 16, None, 0, G + 64, 16, 1.0, None) == INV  # out inside G
    assert f(g5.GEMM_ACT_MUL, 4, 16, G, 16, U, 16, U, 16, 1.0, None) == INV         # in place on U
    for step in (g5.GEMM_ACT_QUANT, g5.GEMM_ACT_SWIGLU_E4M3):
        for bad in (0.0, -2.0, float("nan"), float("inf")):
            assert f(step, 4, 16, G, 16, U, 16, O, 16, bad, None) == INV, (step, bad)
    # codes are bytes: an odd output address passes validation (the call
    # then needs a device)
    assert f(g5.GEMM_ACT_QUANT, 4, 16, G, 16, None, 0, O + 1, 16, 1.0, None) != INV
    # (M == 0 or N == 0: nothing to do, no device needed)
    assert f(g5.GEMM_ACT_SWIGLU_E4M3, 0, 16, G, 16, U, 16, O, 16, 1.0, None) == g5.GEMM_OK
    assert f(g5.GEMM_ACT_SILU, 4, 0, 0, 0, None, 0, 0, 0, 0.0, None) == g5.GEMM_OK
    assert f(g5.GEMM_ACT_SILU, 0, 16, G, 16, None, 0, O, 16, float("nan"), None) == g5.GEMM_OK


def test_swiglu_e4m3_plans(L):
    """The E4M3FN output runs on the same kernels as the bf16 one: the FFN
    gate/up shape on the 256x192 ring kernel (grid 4 x 128), decode on the
    split small-M path with the same workspace (exchange slots only)."""
    e4 = dict(c_type=g5.GEMM_OUT_E4M3)
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 1024, 12288, 4096, **e4)
    assert st == 0 and p.name == b"bf16_256x192" and p.grid == 4 * 128 and p.variant == 1
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 1, 12288, 4096, **e4)
    assert st == 0 and p.name == b"decode_splitk" and p.grid == 192 and p.workspace_bytes == CR
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 300, 392, 261, lda=266, ldb=792, ldc=400, **e4)
    assert st == 0 and p.variant == 3
    # 392-byte code rows are 8-byte, not 16-byte, aligned (bf16 rows of 392
    # elements, 784 bytes, are 16-byte aligned)
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 300, 392, 261, lda=266, ldb=792, ldc=392, **e4)
    assert st == g5.GEMM_ERR_UNSUPPORTED
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 300, 392, 261, lda=266, ldb=792, ldc=392)
    assert st == 0 and p.variant == 3


def test_fused_plans(L):
    """Ring-kernel variants of the fused calls (the epilogues exist in the
    ring kernels only): 4-byte A copies for 4-byte aligned rows, 16-byte for
    aligned ones, and 2-byte aligned A rows realigned first at any size;
    SwiGLU output tiles of half the B tile's columns."""
    for op in (g5.GEMM_OP_BF16_SILU, g5.GEMM_OP_BF16_SWIGLU):
        nb = 392 if op == g5.GEMM_OP_BF16_SILU else 784
        st, p = g5.plan_query(op, 300, 392, 261, lda=266, ldb=nb + 8, ldc=400)
        assert st == 0 and p.variant == 3 and p.workspace_bytes == 0
        st, p = g5.plan_query(op, 300, 392, 264, lda=272, ldb=nb + 8, ldc=400)
        assert st == 0 and p.variant == 2
        st, p = g5.plan_query(op, 257, 96, 33)
        assert st == 0 and p.variant == 2 and p.workspace_bytes == ws_bytes(0, 257 * 40 * 2)
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.grid == 4 * 128 and p.variant == 1
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SILU, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.grid == 256


def test_fused_small_m_plans(L):
    """M <= 16: SiLU and SwiGLU run on the small-M kernels.  With a workspace
    the K-split path (SwiGLU: separate workgroups for a strip's gate and up
    columns, 2 x 96 strips for N = 12288; SiLU: 96 strips x 2 slices), its
    two members of a strip meeting in exchange slots in the workspace's
    counter region (no partial sums); without one the whole-K 64-column
    kernel; K % 32 != 0 only the latter."""
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 1, 12288, 4096)
    assert st == 0 and p.name == b"decode_splitk" and p.grid == 192
    assert p.workspace_bytes == CR
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SILU, 16, 12288, 4096)
    assert st == 0 and p.name == b"decode_splitk" and p.grid == 192
    assert p.workspace_bytes == CR
    for op in (g5.GEMM_OP_BF16_SILU, g5.GEMM_OP_BF16_SWIGLU):
        st, p = g5.plan_query(op, 1, 12288, 4096, with_workspace=False)
        assert st == 0 and p.name == b"decode_64" and p.grid == 192 and p.workspace_bytes == 0
        st, p = g5.plan_query(op, 8, 384, 4100, lda=4104)
        assert st == 0 and p.name == b"decode_64" and p.variant == 1
        st, p = g5.plan_query(op, 8, 200, 64)
        assert st == 0 and p.name == b"decode_64" and p.variant == 0
        st, p = g5.plan_query(op, 17, 384, 640)
        assert st == 0 and p.family == 2


def test_ksplit_plans(L, monkeypatch):
    """K split over workgroups: only for outputs with fewer tiles than CUs,
    each slice at least 4 stages of 32; forcing follows the same rule."""
    for args, ks in [((1024, 12288, 4096), 1), ((4096, 4096, 4096), 1), ((2048, 2048, 8192), 1),
                     ((512, 512, 4096), 5), ((256, 256, 16384), 8), ((1000, 1000, 1000), 3)]:
        st, p = g5.plan_query(g5.GEMM_OP_BF16, *args)
        assert st == 0 and p.ksplit == ks, (args, p.ksplit)
        tiles = -(-args[0] // p.tile_m) * -(-args[1] // p.tile_n)
        assert p.grid == tiles * ks
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1024, 1024, 128, batch=32, c_type=1)
    assert st == 0 and p.ksplit == 1
    # SiLU, SwiGLU and FP32 never split
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SILU, 512, 512, 4096)
    assert st == 0 and p.ksplit == 1
    st, p = g5.plan_query(g5.GEMM_OP_SGEMM, 512, 512, 4096)
    assert st == 0 and p.ksplit == 1
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", "3")
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 300, 392, 400)      # 12 stages: 3 slices of 4
    assert st == 0 and p.ksplit == 3 and p.grid == 3 * 12
    st, _ = g5.plan_query(g5.GEMM_OP_BF16, 300, 392, 380)      # 11 stages: too few for 3
    assert st == g5.GEMM_ERR_UNSUPPORTED


def test_nt_arguments_and_plans(L):
    """Transposed B: ldbt >= K, Bt spans N rows of K; every bf16 tile config
    runs it on its ring kernel; Bt rows that are not 16-byte aligned are
    realigned first (the general kernel takes no transposed B); small M stays
    on the tiled kernels."""
    def nt(M, N, K, lda=None, ldb=None, ldc=None, c=C_ADDR, b=B_ADDR):
        return L.gemm_bf16_nt(M, N, K, A_ADDR, K if lda is None else lda, b, K if ldb is None else ldb, c,
                              N if ldc is None else ldc, 0, None)
    assert nt(4, 8, 16, ldb=15) == g5.GEMM_ERR_INVALID_ARG
    assert nt(4, 8, 16, b=0) == g5.GEMM_ERR_INVALID_ARG
    assert nt(4, 8, 16, c=B_ADDR + (7 * 16 + 15) * 2) == g5.GEMM_ERR_INVALID_ARG   # C inside Bt's last row
    assert nt(0, 8, 16) == g5.GEMM_OK
    st, p = g5.plan_query(g5.GEMM_OP_BF16_NT, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.variant == 1 and p.grid == 256
    # small M: a GEMV over the rows of Bt (decode_nt), 16 rows per workgroup,
    # 48 (three blocks sharing X) when M > 1; unaligned Bt rows: tiled kernels
    st, p = g5.plan_query(g5.GEMM_OP_BF16_NT, 1, 12288, 4096)
    assert st == 0 and p.name == b"decode_nt" and p.grid == 768 and p.variant == 1
    st, p = g5.plan_query(g5.GEMM_OP_BF16_NT, 16, 12288, 4096)
    assert st == 0 and p.name == b"decode_nt" and p.grid == 256 and p.variant == 2
    st, p = g5.plan_query(g5.GEMM_OP_BF16_NT, 16, 12288, 4100)
    assert st == 0 and p.family == 2
    st, p = g5.plan_query(g5.GEMM_OP_BF16_NT, 300, 392, 264, ldb=265)
    assert st == 0 and p.variant >= 1 and p.vec_b == 16
    assert p.workspace_bytes >= 392 * 264 * 2
    st, p = g5.plan_query(g5.GEMM_OP_BF16_NT, 1024, 1024, 128, batch=32, c_type=1)
    assert st == 0 and p.name == b"bf16_128x128" and p.variant == 1 and p.workspace_bytes == 0


def test_tn_arguments_and_plans(L, monkeypatch):
    """Transposed A: ldat >= M, At spans K rows of M; the ring kernels of the
    256x192, 256x256 and 128x128 configs run it (variants 1 and 2 only); At
    rows not 16-byte aligned, or M % 8 != 0, are realigned into rows of
    ceil(M/8)*8 elements first; small M stays on the tiled kernels."""
    def tn(M, N, K, lda=None, ldb=None, ldc=None, a=A_ADDR, c=C_ADDR):
        return L.gemm_bf16_tn(M, N, K, a, M if lda is None else lda, B_ADDR, N if ldb is None else ldb, c,
                              N if ldc is None else ldc, 0, None)
    assert tn(4, 8, 16, lda=3) == g5.GEMM_ERR_INVALID_ARG
    assert tn(4, 8, 16, a=0) == g5.GEMM_ERR_INVALID_ARG
    assert tn(4, 8, 16, c=A_ADDR + (15 * 4 + 2) * 2) == g5.GEMM_ERR_INVALID_ARG    # C inside At's last row
    assert tn(0, 8, 16) == g5.GEMM_OK
    op = g5.GEMM_OP_BF16_TN
    st, p = g5.plan_query(op, 4096, 12288, 1024)
    assert st == 0 and p.family == 2 and p.variant == 1 and p.workspace_bytes == 0
    assert p.name in (b"bf16_256x192", b"bf16_256x256", b"bf16_128x128")
    st, p = g5.plan_query(op, 300, 392, 262)                       # M % 8 != 0
    assert st == 0 and p.variant == 2 and p.workspace_bytes >= 262 * 304 * 2
    st, p = g5.plan_query(op, 304, 392, 262, lda=306)              # 4-byte aligned At rows
    assert st == 0 and p.variant == 2 and p.workspace_bytes >= 262 * 304 * 2
    st, p = g5.plan_query(op, 304, 392, 264, lda=312, ldb=400)     # aligned: no copy
    assert st == 0 and p.variant == 2 and p.workspace_bytes == 0
    st, p = g5.plan_query(op, 1, 4096, 4096, lda=8)
    assert st == 0 and p.family == 2
    st, p = g5.plan_query(op, 512, 512, 4096)
    assert st == 0 and p.name == b"bf16_128x128" and p.ksplit > 1
    for bad in ("bf16_256x128", "decode_64", "f32_128x128"):
        monkeypatch.setenv("GEMM_FORCE_CONFIG", bad)
        st, _ = g5.plan_query(op, 304, 392, 264)
        assert st == g5.GEMM_ERR_UNSUPPORTED, bad


def test_fp8_arguments_and_plans(L):
    """FP8: factors 4-byte aligned and not overlapping C; Bt rows 16-byte
    aligned and, on the ring kernels (M > 16), A rows 4-byte aligned; 64 K
    values per stage; quantization arguments."""
    def f8(M, N, K, lda=None, ldb=None, sa=0, sb=0, c=C_ADDR):
        return L.gemm_fp8_nt(M, N, K, A_ADDR, K if lda is None else lda, sa, B_ADDR, K if ldb is None else ldb, sb,
                             c, N, 0, None)
    assert f8(4, 8, 16, ldb=15) == g5.GEMM_ERR_INVALID_ARG
    assert f8(4, 8, 16, sa=C_ADDR + 2) == g5.GEMM_ERR_INVALID_ARG             # misaligned factor vector
    assert f8(4, 8, 16, sb=C_ADDR + 8) == g5.GEMM_ERR_INVALID_ARG             # factors inside C
    assert f8(4, 8, 20) == g5.GEMM_ERR_UNSUPPORTED                            # Bt rows 4-byte aligned
    assert f8(20, 8, 20, lda=22, ldb=32) == g5.GEMM_ERR_UNSUPPORTED           # A rows 2-byte aligned (tiled)
    # M <= 16 with 16-byte Bt rows: the FP8 GEMV over Bt rows, any A alignment
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 4, 8, 20, lda=22, ldb=32)
    assert st == 0 and p.name == b"decode_nt"
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 1, 12288, 4096)
    assert st == 0 and p.name == b"decode_nt" and p.variant == 1 and p.grid == 768
    assert f8(0, 8, 16) == g5.GEMM_OK
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.variant == 1 and p.even == 1
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 1024, 12288, 4128)              # K % 64 = 32: masked
    assert st == 0 and p.variant == 2
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 300, 392, 260, ldb=272)
    assert st == 0 and p.variant == 3
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 1024, 1536, 4096)
    assert st == 0 and p.name == b"bf16_128x128" and p.ksplit == 2
    q = L.gemm_fp8_quantize_rows
    assert q(-1, 8, A_ADDR, 8, B_ADDR, 8, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG
    assert q(4, 8, A_ADDR, 7, B_ADDR, 8, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG
    assert q(4, 8, A_ADDR, 8, A_ADDR + 8, 8, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG   # Q inside X
    assert q(4, 8, A_ADDR, 8, B_ADDR, 8, C_ADDR + 1, None) == g5.GEMM_ERR_INVALID_ARG   # misaligned factors
    assert q(0, 8, A_ADDR, 8, B_ADDR, 8, C_ADDR, None) == g5.GEMM_OK


def test_quant_traffic_model_reproduces_example_5_8(L):
    """gemm_model_quant_traffic against the page's Example 5-8: 444 MiB when
    the input is quantized before the GEMM, 620 MiB when inside it."""
    import ctypes
    rows = {}
    vals = None
    with open(os.path.join(GOLDEN, "op_runtime_5_4_3_quant_traffic.txt")) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if vals is None:
                vals = [int(v) for v in parts]
            else:
                rows[parts[0]] = int(parts[1])
    M, K, N, m, n, inb, qb, wb, ob = vals
    sep, fus = ctypes.c_double(), ctypes.c_double()
    L.gemm_model_quant_traffic(M, N, K, m, n, inb, qb, wb, ob, ctypes.byref(sep), ctypes.byref(fus))
    MiB = 2.0 ** 20
    assert sep.value / MiB == rows["total_separate"] and fus.value / MiB == rows["total_fused"]
    common = (-(-M // m)) * wb * K * N + ob * M * N
    assert common / MiB == rows["common"]
    assert (sep.value - common) / MiB == rows["input_separate"] and (fus.value - common) / MiB == rows["input_fused"]


def test_act_chain_traffic_model_reproduces_example_5_4(L):
    """gemm_model_act_chain_bytes summed over each program's calls gives the
    page's Example 5-4 figures: 120 -> 72 MiB for SiLU and the product,
    156 -> 108 -> 60 MiB with the quantization."""
    rows, shape = {}, None
    with open(os.path.join(GOLDEN, "op_runtime_5_3_1_act_chain_traffic.txt")) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if shape is None:
                shape = [int(v) for v in parts]
            else:
                rows[parts[0]] = int(parts[1])
    M, N = shape
    b = lambda step: L.gemm_model_act_chain_bytes(step, M, N) / 2.0 ** 20
    S, P, F, Q, F3 = (g5.GEMM_ACT_SILU, g5.GEMM_ACT_MUL, g5.GEMM_ACT_SWIGLU, g5.GEMM_ACT_QUANT,
                      g5.GEMM_ACT_SWIGLU_E4M3)
    assert b(S) + b(P) == rows["silu_then_product"]
    assert b(F) == rows["fused_silu_product"]
    assert b(S) + b(P) + b(Q) == rows["three_steps"]
    assert b(F) + b(Q) == rows["fused_two_then_quantize"]
    assert b(F3) == rows["fused_three"]
    assert L.gemm_model_act_chain_bytes(5, M, N) == 0.0 and L.gemm_model_act_chain_bytes(S, -1, N) == 0.0


def call_affine(L, M, N, K, batch=1, a=A_ADDR, lda=None, b=B_ADDR, ldb=None, c=C_ADDR, ldc=None, alpha=1.0,
                bias=0, beta=0.0, c_type=0, sA=None, sB=None, sC=None):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    sA = M * lda if sA is None else sA
    sB = K * ldb if sB is None else sB
    sC = M * ldc if sC is None else sC
    return L.gemm_bf16_affine(batch, M, N, K, a, lda, sA, b, ldb, sB, alpha, bias or None, beta, c, ldc, sC,
                              c_type, None)


def test_affine_arguments(L):
    """Affine epilogue: gemm_bf16_batched's validation plus finite alpha and
    beta and a 2-byte aligned bias outside C; the fused-epilogue store's
    preconditions when a product is formed (not for alpha == 0 or K == 0,
    which read neither A nor B)."""
    assert call_affine(L, -1, 8, 4) == g5.GEMM_ERR_INVALID_ARG
    assert call_affine(L, 4, 8, 4, alpha=float("nan")) == g5.GEMM_ERR_INVALID_ARG
    assert call_affine(L, 4, 8, 4, beta=float("inf")) == g5.GEMM_ERR_INVALID_ARG
    assert call_affine(L, 4, 8, 4, bias=0x7000001) == g5.GEMM_ERR_INVALID_ARG      # odd address
    assert call_affine(L, 4, 8, 4, bias=C_ADDR + 6) == g5.GEMM_ERR_INVALID_ARG     # inside C
    assert call_affine(L, 4, 8, 4, c_type=2) == g5.GEMM_ERR_INVALID_ARG
    assert call_affine(L, 4, 8, 4, b=0) == g5.GEMM_ERR_INVALID_ARG
    assert call_affine(L, 2, 8, 4, batch=2, sC=8) == g5.GEMM_ERR_INVALID_ARG       # C entries overlap
    assert call_affine(L, 4, 12, 4) == g5.GEMM_ERR_UNSUPPORTED                     # N % 8
    assert call_affine(L, 4, 8, 4, c=C_ADDR + 2) == g5.GEMM_ERR_UNSUPPORTED        # C rows 2-byte aligned
    assert call_affine(L, 0, 8, 4) == g5.GEMM_OK                                    # empty: nothing to do
    st, p = g5.plan_query(g5.GEMM_OP_BF16_AFFINE, 4, 8, 0)
    assert st == 0 and p.family == 1                                                # K = 0: element-wise pass
    st, p = g5.plan_query(g5.GEMM_OP_BF16_AFFINE, 4, 12, 0, c_addr=C_ADDR + 2)
    assert st == 0 and p.family == 1                                                # ... at any alignment


def test_affine_plans(L):
    """The affine epilogue runs on the fused-epilogue ring kernels, batched,
    with either output type, and splits K for small outputs like gemm_bf16;
    M <= 16 takes the small-M kernels."""
    op = g5.GEMM_OP_BF16_AFFINE
    for ct in (0, 1):
        st, p = g5.plan_query(op, 1024, 12288, 4096, c_type=ct)
        assert st == 0 and p.family == 2 and p.variant == 1 and p.ksplit == 1
        assert p.name in (b"bf16_256x192", b"bf16_256x256", b"bf16_128x128")
    st, p = g5.plan_query(op, 512, 512, 4096)
    assert st == 0 and p.name == b"bf16_128x128" and p.ksplit == 5
    st, p = g5.plan_query(op, 1, 4096, 4096)
    assert st == 0 and p.name == b"decode_splitk"                                  # small M: the small-M kernels
    st, p = g5.plan_query(op, 5, 200, 64, batch=2)
    assert st == 0 and p.name == b"decode_64" and p.variant == 0
    st, p = g5.plan_query(op, 17, 4096, 4096)
    assert st == 0 and p.family == 2
    st, p = g5.plan_query(op, 300, 392, 261, lda=266, ldb=400, ldc=400, batch=3)
    assert st == 0 and p.variant == 3
    st, p = g5.plan_query(op, 257, 96, 33)
    assert st == 0 and p.variant == 2 and p.workspace_bytes == ws_bytes(0, 257 * 40 * 2)        # A realigned


def test_nt_affine_plans(L):
    """The affine epilogue with B transposed: the transposed-B ring kernels
    of the fused configs (with K split for small outputs), the small-M
    transposed-B kernel for M <= 16, Bt rows realigned when not 16-byte
    aligned; the affine argument checks apply."""
    op = g5.GEMM_OP_BF16_NT_AFFINE
    st, p = g5.plan_query(op, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.variant == 1
    st, p = g5.plan_query(op, 1, 12288, 4096)
    assert st == 0 and p.name == b"decode_nt"
    st, p = g5.plan_query(op, 512, 512, 4096)
    assert st == 0 and p.name == b"bf16_128x128" and p.ksplit > 1
    st, p = g5.plan_query(op, 300, 392, 264, ldb=265)
    assert st == 0 and p.variant >= 1 and p.workspace_bytes >= 392 * 264 * 2
    st, _ = g5.plan_query(op, 4, 12, 16)
    assert st == g5.GEMM_ERR_UNSUPPORTED                                          # N % 8
    args = (1, 4, 8, 16, A_ADDR, 16, 64, B_ADDR, 16, 128)
    assert L.gemm_bf16_nt_affine(*args, float("nan"), None, 0.0, C_ADDR, 8, 32, 0, None) == g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_bf16_nt_affine(*args, 1.0, C_ADDR + 4, 0.0, C_ADDR, 8, 32, 0, None) == g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_bf16_nt_affine(1, 4, 8, 16, A_ADDR, 16, 64, B_ADDR, 15, 128, 1.0, None, 0.0, C_ADDR, 8, 32, 0,
                                 None) == g5.GEMM_ERR_INVALID_ARG                  # ldbt < K


def test_operands_over_2gib_plans(L):
    """An operand whose byte extent reaches 2^31 cannot be addressed by the
    ring kernels' 32-bit buffer offsets: plain products take the general
    kernel (variant 0); calls that exist only on the ring kernels report
    GEMM_ERR_UNSUPPORTED instead of launching."""
    M, N, K = 270000, 128, 4096                     # A: 2.2e9 bytes
    far = dict(a_addr=A_ADDR, b_addr=B_ADDR, c_addr=C_ADDR)
    st, p = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, **far)
    assert st == 0 and p.family == 2 and p.variant == 0
    for op in (g5.GEMM_OP_BF16_SILU, g5.GEMM_OP_BF16_NT, g5.GEMM_OP_BF16_TN, g5.GEMM_OP_BF16_AFFINE):
        st, _ = g5.plan_query(op, M, N, K, **far)
        assert st == g5.GEMM_ERR_UNSUPPORTED, op
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1, 64, 64, batch=70000, **far)
    assert st == 0 and p.family == 2                # more entries than the small-M grid takes


def test_tn_affine_plans(L):
    """The affine epilogue with A transposed runs on the transposed-A ring
    kernels at every M (no small-M path), with K split for small outputs and
    At rows realigned as for gemm_bf16_tn."""
    op = g5.GEMM_OP_BF16_TN_AFFINE
    st, p = g5.plan_query(op, 4096, 12288, 1024, c_type=1)
    assert st == 0 and p.family == 2 and p.variant == 1
    st, p = g5.plan_query(op, 8, 4096, 4096)
    assert st == 0 and p.family == 2
    st, p = g5.plan_query(op, 512, 512, 4096)
    assert st == 0 and p.name == b"bf16_128x128" and p.ksplit > 1
    st, p = g5.plan_query(op, 300, 392, 262)                       # M % 8 != 0: At rows realigned
    assert st == 0 and p.variant == 2 and p.workspace_bytes >= 262 * 304 * 2
    args = (1, 8, 8, 16, A_ADDR, 8, 128, B_ADDR, 8, 128)
    assert L.gemm_bf16_tn_affine(*args, float("inf"), None, 1.0, C_ADDR, 8, 64, 0, None) == g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_bf16_tn_affine(1, 8, 8, 16, A_ADDR, 7, 128, B_ADDR, 8, 128, 1.0, None, 1.0, C_ADDR, 8, 64, 0,
                                 None) == g5.GEMM_ERR_INVALID_ARG          # ldat < M


# ---- the ownership contract: caller workspaces, nothing allocated inside ----

def test_named_calls_plan_without_workspace(L):
    """The named entry points run the plans of a call without a workspace:
    whole K per workgroup (no split small-M path, no K split over
    workgroups) and no realigned row copies."""
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1, 12288, 4096, with_workspace=False)
    assert st == 0 and p.name == b"decode_64" and p.workspace_bytes == 0
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1024, 1536, 4096, with_workspace=False)
    assert st == 0 and p.ksplit == 1 and p.workspace_bytes == 0
    # ragged 1000x12280x4100: A rows (8200 bytes) realigned only with a workspace
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1000, 12280, 4100, c_type=1, with_workspace=False)
    assert st == 0 and p.variant == 3 and p.workspace_bytes == 0
    st, p = g5.plan_query(g5.GEMM_OP_BF16, 1000, 12280, 4100, c_type=1)
    assert st == 0 and p.variant == 2 and p.workspace_bytes == ws_bytes(0, 1000 * 4104 * 2)
    # a fused epilogue with 2-byte aligned A rows runs only from a realigned copy
    st, _ = g5.plan_query(g5.GEMM_OP_BF16_SILU, 300, 256, 130, lda=131, with_workspace=False)
    assert st == g5.GEMM_ERR_UNSUPPORTED
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SILU, 300, 256, 130, lda=131)
    assert st == 0 and p.workspace_bytes > 0
    # GEMM_FORCE_KSPLIT needs a workspace
    for M, N, K in ((1024, 1536, 4096), (4096, 4096, 4096)):
        st, p = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, with_workspace=False)
        assert st == 0 and p.ksplit == 1


def test_workspace_size_matches_plan(L):
    for args in ((g5.GEMM_OP_BF16, 1, 1, 12288, 4096), (g5.GEMM_OP_BF16, 1, 1024, 1536, 4096),
                 (g5.GEMM_OP_BF16, 1, 1024, 12288, 4096), (g5.GEMM_OP_BF16_TN, 1, 300, 392, 262)):
        op, batch, M, N, K = args
        st, p = g5.plan_query(op, M, N, K, batch=batch)
        lda, ldb, ldc, sA, sB, sC = g5.gemm._plan_args(op, M, N, K, batch, None, None, None, None, None, None)
        n = g5.workspace_size(op, batch, M, N, K, 0x10000, lda, sA, 0x20000000, ldb, sB, 0x40000000, ldc, sC, 0)
        assert st == 0 and n == p.workspace_bytes


def test_run_rejects_small_or_unaligned_workspace(L):
    """gemm_run checks the workspace on the host, before any GPU call: too
    small is GEMM_ERR_WORKSPACE, not 256-byte aligned GEMM_ERR_INVALID_ARG
    (fake device addresses; nothing is enqueued)."""
    M, N, K = 1, 12288, 4096
    st, p = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
    need = p.workspace_bytes
    assert need >= CR
    WS = P + (3 << 34)
    run = lambda ws, n: L.gemm_run(g5.GEMM_OP_BF16, 1, M, N, K, A_ADDR, K, 0, B_ADDR, N, 0, C_ADDR, N, 0, 0,
                                   1.0, None, 0.0, None, None, ws, n, None)
    assert run(WS, need - 1) == g5.GEMM_ERR_WORKSPACE
    assert run(WS + 16, need) == g5.GEMM_ERR_INVALID_ARG
    assert L.gemm_run(99, 1, M, N, K, A_ADDR, K, 0, B_ADDR, N, 0, C_ADDR, N, 0, 0, 1.0, None, 0.0, None, None,
                      None, 0, None) == g5.GEMM_ERR_INVALID_ARG


def test_library_source_allocates_nothing():
    """The library's sources name no allocation, free, copy or
    synchronisation call: the caller owns every byte of device memory."""
    csrc = os.path.join(ROOT, "dense_gemm_05_amd", "csrc")
    banned = re.compile(r"\bhip(Malloc|MallocAsync|Free|FreeAsync|HostMalloc|Memcpy\w*|Memset\w*|StreamSynchronize|"
                        r"DeviceSynchronize|EventSynchronize|ExtMallocWithFlags|MallocManaged)\b")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".cpp", ".hip", ".h")):
            with open(os.path.join(csrc, name)) as fh:
                for i, line in enumerate(fh, 1):
                    assert not banned.search(line), f"{name}:{i}: {line.strip()}"


def test_fp8_batched_affine_and_cols_arguments(L):
    """FP8: batched products and the affine op plan like their bf16
    counterparts (small M on the GEMV over Bt's rows); factor vectors are
    checked against C over every batch entry; the column quantizer
    validates before touching the GPU."""
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 300, 392, 256, batch=3)
    assert st == 0 and p.family == 2
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT, 5, 392, 256, batch=3)
    assert st == 0 and p.name == b"decode_nt"
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT_AFFINE, 7, 200, 144)
    assert st == 0 and p.name == b"decode_nt"
    st, p = g5.plan_query(g5.GEMM_OP_FP8_NT_AFFINE, 1024, 12288, 4096)
    assert st == 0 and p.name == b"bf16_256x192" and p.grid == 256
    st, _ = g5.plan_query(g5.GEMM_OP_FP8_NT_AFFINE, 300, 392, 256, ldc=396, c_addr=C_ADDR + 8)
    assert st == g5.GEMM_ERR_UNSUPPORTED                       # tiled affine: C rows 16-byte aligned
    # C (3 x 8 x 16 floats) overlapping the last entry's factors of A
    M, N, K, batch = 8, 16, 64, 3
    run = lambda sa, sb, sA=M * K: L.gemm_run(g5.GEMM_OP_FP8_NT, batch, M, N, K, A_ADDR, K, sA, B_ADDR, K, N * K,
                                            C_ADDR, N, M * N, 1, 1.0, None, 0.0, sa, sb, None, 0, None)
    before_c = C_ADDR - 4 * (M + 1)            # M factors end 4 bytes before C; 3 M reach into it
    assert run(before_c, None) == g5.GEMM_ERR_INVALID_ARG                        # one vector per entry
    assert run(before_c, None, sA=0) != g5.GEMM_ERR_INVALID_ARG                  # broadcast A: M factors only
    assert run(None, C_ADDR + 2) == g5.GEMM_ERR_INVALID_ARG                      # unaligned factors
    q = L.gemm_fp8_quantize_cols
    assert q(64, 32, A_ADDR, 31, B_ADDR, 64, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG    # ldw < N
    assert q(64, 32, A_ADDR, 32, B_ADDR, 63, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG    # ldq < K
    assert q(64, 32, A_ADDR + 1, 32, B_ADDR, 64, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG  # W not 2-byte aligned
    assert q(64, 32, A_ADDR, 32, A_ADDR + 100, 64, C_ADDR, None) == g5.GEMM_ERR_INVALID_ARG  # Qt overlaps W
    assert q(64, 0, None, 0, None, 64, None, None) == g5.GEMM_OK                       # nothing to do


def test_fp8_quant_a_arguments(L):
    """The FP8 product with X quantized inside the GEMM validates before
    touching the GPU: whole 64-deep stages and 16-byte rows, a workspace of
    the counter region (untouched) plus M floats, 256-byte aligned, and no
    overlaps."""
    M, N, K = 64, 128, 256
    W = P + (3 << 34)
    def call(K=K, ldx=K, x=A_ADDR, ws=W, wsb=CR + 4 * M, sx=P + (4 << 34), c=C_ADDR):
        return L.gemm_fp8_nt_quant_a(M, N, K, x, ldx, sx, B_ADDR, K, None, c, N, 0, ws, wsb, None)
    assert call(K=200, ldx=200) == g5.GEMM_ERR_UNSUPPORTED           # K % 64
    assert call(ldx=260) == g5.GEMM_ERR_UNSUPPORTED                  # X rows 8-byte aligned
    assert call(wsb=CR + 4 * M - 4) == g5.GEMM_ERR_WORKSPACE
    assert call(wsb=4 * M) == g5.GEMM_ERR_WORKSPACE                  # no room past the counters
    assert call(ws=None, wsb=0) == g5.GEMM_ERR_WORKSPACE
    assert call(ws=W + 64) == g5.GEMM_ERR_INVALID_ARG                # workspace not 256-byte aligned
    assert call(ldx=100) == g5.GEMM_ERR_INVALID_ARG                  # ldx < K
    assert call(sx=C_ADDR + 16) == g5.GEMM_ERR_INVALID_ARG           # factors inside C
    assert call(ws=C_ADDR - CR) == g5.GEMM_ERR_INVALID_ARG           # the maxima would land in C
    assert L.gemm_fp8_nt_quant_a(0, N, K, None, K, None, None, K, None, None, N, 0, None, 0, None) == g5.GEMM_OK

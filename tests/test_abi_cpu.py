"""The C-ABI library loads on a machine without a GPU, exports every entry
point include/tiledq.h declares, and rejects bad arguments on the host before
any HIP call (no compute is launched by these tests)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "tiledq.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b(tq_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from block_quantized_matmul_repack_amd import _lib
    return _lib.lib()


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("tq_repack_tiles", "tq_quantize_act", "tq_qgemv", "tq_qgemm", "tq_block_dots"):
        assert name in syms


def test_library_exports_every_declared_symbol(L):
    from block_quantized_matmul_repack_amd import _lib
    syms = declared_symbols()
    assert syms
    for name in syms:
        assert hasattr(L, name), name
        assert name in _lib.SIGNATURES, name


def test_sizes_match_oracle(L, orc):
    for t in (0, 1, 2, 3, 4, 5):
        assert L.tq_tile_bytes(t) == orc.tile_bytes(t)
        assert L.tq_block_bytes(t) == orc.block_bytes(t)
        for K, N in ((32, 1), (4096, 4096), (4096, 14336), (4096, 128001), (96, 70), (768, 3)):
            if t == 5 and K % 256:
                assert L.tq_tiled_bytes(t, K, N) == 0 and L.tq_flat_bytes(t, K, N) == 0
                continue
            assert L.tq_tiled_bytes(t, K, N) == orc.tiled_bytes(t, K, N)
            assert L.tq_flat_bytes(t, K, N) == orc.flat_bytes(t, K, N)
    assert L.tq_tile_bytes(7) == 0
    assert L.tq_tiled_bytes(0, 33, 4) == 0 and L.tq_flat_bytes(0, 16, 4) == 0


def test_supported_static_properties(L):
    assert L.tq_supported(0, 4096, 4096, 8, 0) == 1
    assert L.tq_supported(0, 4096, 4096, 9, 0) == 0
    assert L.tq_supported(2, 4096, 4096, 512, 1) == 1
    assert L.tq_supported(3, 4096, 4096, 1, 0) == 1          # MXFP4
    assert L.tq_supported(4, 4096, 4096, 1, 0) == 1          # Q4_1
    assert L.tq_supported(5, 4096, 4096, 1, 0) == 1          # Q4_K
    assert L.tq_supported(5, 4128, 4096, 1, 0) == 0          # K % 256 != 0
    assert L.tq_supported(6, 4096, 4096, 1, 0) == 0
    assert L.tq_supported(0, 4096, 4096, 8, 2) == 1          # flat GEMV
    assert L.tq_supported(0, 4096, 4096, 9, 2) == 0
    assert L.tq_supported(5, 4096, 4096, 512, 3) == 1        # flat GEMM
    assert L.tq_supported(0, 4096, 4096, 1, 4) == 0          # block-scaled path: MXFP4 only
    assert L.tq_supported(3, 4096, 4096, 512, 4) == 1
    assert L.tq_supported(3, 4001, 4096, 512, 4) == 0
    assert L.tq_supported(0, 4001, 4096, 1, 0) == 0
    assert L.tq_supported(0, 4096, 4096, 1, 5) == 0


# Fake, never-dereferenced device addresses: validation fails before any use.
A16 = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x10002)
NUL = None
LUT = (ctypes.c_int8 * 16)(*range(-8, 8))


def test_workspace_bytes(L):
    # K=N=4096, M=1: 128 stripes, each split S ways (S a power of two): the
    # pairwise tree needs (S - 1) * 32 slots of 8 bytes per stripe
    ws = L.tq_qgemv_workspace_bytes(1, 4096, 4096, 1)
    assert ws % (128 * 32 * 8) == 0 and ws // (128 * 32 * 8) + 1 in (2, 4, 8)
    assert L.tq_qgemv_workspace_bytes(1, 4096, 128001, 1) == 0      # enough stripes
    assert L.tq_qgemv_workspace_bytes(1, 4096, 4096, 9) == 0
    assert L.tq_qgemv_workspace_bytes(1, 4000 + 1, 4096, 1) == 0
    assert L.tq_qgemv_workspace_bytes(1, 4096, 0, 1) == 0           # empty: no division by 0
    assert L.tq_qgemv_workspace_bytes(1, 4096, 4096, 0) == 0


def test_status_strings(L):
    for s in range(6):
        assert L.tq_status_string(s).startswith(b"TQ_")


def test_repack_validation(L):
    assert L.tq_repack_tiles(9, A16, 64, 32, A16, NUL) == 2
    assert L.tq_repack_tiles(0, A16, 48, 32, A16, NUL) == 3
    assert L.tq_repack_tiles(0, A16, 0, 32, A16, NUL) == 3
    assert L.tq_repack_tiles(0, A16, 64, -1, A16, NUL) == 3
    assert L.tq_repack_tiles(0, NUL, 64, 32, A16, NUL) == 1
    assert L.tq_repack_tiles(0, A16, 64, 32, A2, NUL) == 4
    assert L.tq_repack_tiles(0, ctypes.c_void_p(0x10001), 64, 32, A16, NUL) == 4
    assert L.tq_repack_tiles(0, NUL, 64, 0, NUL, NUL) == 0       # empty: OK, no launch
    assert L.tq_repack_tiles(3, A2, 64, 32, A16, NUL) == 4       # MXFP4 flat: 4-byte aligned
    assert L.tq_repack_tiles(4, A2, 64, 32, A16, NUL) == 4       # Q4_1 flat: 4-byte aligned
    assert L.tq_repack_tiles(5, ctypes.c_void_p(0x10004), 256, 32, A16, NUL) == 4   # Q4_K: 16
    assert L.tq_repack_tiles(5, A16, 288, 32, A16, NUL) == 3     # Q4_K: K % 256
    assert L.tq_qgemv(5, A16, 288, 32, A16, A16, 1, NUL, A16, 32, NUL, 0, NUL) == 3


def test_quantize_validation(L):
    assert L.tq_quantize_act(5, A16, 1, 64, 64, A16, A16, NUL) == 2
    assert L.tq_quantize_act(0, A16, 1, 60, 64, A16, A16, NUL) == 3
    assert L.tq_quantize_act(0, A16, 1, 64, 32, A16, A16, NUL) == 3   # ldx < K
    assert L.tq_quantize_act(0, A16, -1, 64, 64, A16, A16, NUL) == 3
    assert L.tq_quantize_act(0, NUL, 1, 64, 64, A16, A16, NUL) == 1
    assert L.tq_quantize_act(0, A2, 1, 64, 64, A16, A16, NUL) == 4    # fp32 needs 4 B
    assert L.tq_quantize_act(0, NUL, 0, 64, 64, NUL, NUL, NUL) == 0


@pytest.mark.parametrize("fn", ["tq_qgemv", "tq_qgemm", "tq_matmul"])
def test_matmul_validation(L, fn):
    if fn in ("tq_qgemv", "tq_matmul"):
        def f(*a):
            return getattr(L, fn)(*a[:10], None, 0, a[10])
    else:
        f = L.tq_qgemm
    assert f(9, A16, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 2
    assert f(0, A16, 48, 32, A16, A16, 1, NUL, A16, 32, NUL) == 3
    assert f(0, A16, 64, 32, A16, A16, 1, NUL, A16, 31, NUL) == 3     # ldy < N
    assert f(0, NUL, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 1
    assert f(0, A16, 64, 32, NUL, A16, 1, NUL, A16, 32, NUL) == 1
    assert f(0, A16, 64, 32, A16, NUL, 1, NUL, A16, 32, NUL) == 1
    assert f(0, A16, 64, 32, A16, A16, 1, NUL, NUL, 32, NUL) == 1
    assert f(2, A16, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 1     # IQ4_NL needs the table
    assert f(0, A2, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 4
    assert f(0, A16, 64, 32, A2, A16, 1, NUL, A16, 32, NUL) == 4
    assert f(0, A16, 64, 32, A16, A16, 1, NUL, A2, 32, NUL) == 4
    assert f(0, NUL, 64, 32, NUL, NUL, 0, NUL, NUL, 32, NUL) == 0     # M == 0
    assert f(0, NUL, 64, 0, NUL, NUL, 4, NUL, NUL, 0, NUL) == 0       # N == 0
    assert f(2, NUL, 64, 0, NUL, NUL, 4, LUT, NUL, 0, NUL) == 0


def test_matmul_mx_validation_and_workspace(L):
    """tq_matmul_mx checks its arguments before any launch; its workspace
    holds S partial planes after the 1 MiB slot region, S = 2, 4 or 8 where
    the cost model estimates the split faster (few 64 x 128 output blocks;
    none at M = 256 or 512, N = 4096)."""
    ws = ctypes.c_void_p(0x20000)
    f = L.tq_matmul_mx
    assert f(A16, 48, 32, A16, A16, 1, A16, 32, ws, 0, NUL) == 3           # K % 32
    assert f(A16, 64, 32, A16, A16, 1, A16, 31, ws, 0, NUL) == 3           # ldy < N
    assert f(NUL, 64, 32, A16, A16, 1, A16, 32, ws, 0, NUL) == 1
    assert f(A16, 64, 32, A16, NUL, 1, A16, 32, ws, 0, NUL) == 1
    assert f(A2, 64, 32, A16, A16, 1, A16, 32, ws, 0, NUL) == 4
    assert f(A16, 64, 32, A16, A16, 1, A16, 32, ctypes.c_void_p(0x20010), 64, NUL) == 4
    assert f(NUL, 64, 32, NUL, NUL, 0, NUL, 32, NUL, 0, NUL) == 0          # M == 0
    W = L.tq_matmul_mx_workspace_bytes
    assert W(4096, 4096, 512) == 0
    assert W(4096, 4096, 128) == (1 << 20) + 4 * 128 * 4096 * 4
    assert W(4096, 4096, 64) == (1 << 20) + 4 * 64 * 4096 * 4
    assert W(8192, 512, 200) == (1 << 20) + 8 * 200 * 512 * 4
    assert W(4096, 14336, 8) == (1 << 20) + 2 * 8 * 14336 * 4
    assert W(1024, 300, 40) == 0 and W(4096, 4096, 256) == 0      # estimated no faster
    assert W(48, 64, 8) == 0 and W(64, 64, 0) == 0


def test_qgemv_x_validation(L):
    f = L.tq_qgemv_x
    # (type, tiles, K, N, dtype, x, ldx, M, lut, y, ldy, ws, ws_bytes, stream)
    assert f(0, A16, 64, 32, 7, A16, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 2      # bad dtype
    assert f(9, A16, 64, 32, 0, A16, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 2      # bad type
    assert f(0, A16, 64, 32, 0, A16, 64, 9, NUL, A16, 32, NUL, 0, NUL) == 3      # M > 8
    assert f(0, A16, 64, 32, 0, A16, 32, 1, NUL, A16, 32, NUL, 0, NUL) == 3      # ldx < K
    assert f(0, A16, 64, 32, 0, NUL, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 1      # x NULL
    assert f(0, A16, 64, 32, 0, A2, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 4       # fp32 x at 2 B
    assert f(2, A16, 64, 32, 1, A16, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 1      # IQ4_NL, no table
    assert f(0, NUL, 64, 0, 0, NUL, 64, 1, NUL, NUL, 0, NUL, 0, NUL) == 0        # N == 0


def test_matmul_dispatch_validation(L):
    # M > 8 goes to the GEMM's checks: no M limit, same shape / pointer rules
    f = L.tq_matmul
    assert f(0, A16, 64, 32, A16, A16, 9, NUL, A16, 31, NUL, 0, NUL) == 3        # ldy < N
    assert f(0, A16, 64, 32, A16, NUL, 9, NUL, A16, 32, NUL, 0, NUL) == 1        # d NULL
    assert f(0, NUL, 64, 0, NUL, NUL, 9, NUL, NUL, 0, NUL, 0, NUL) == 0          # N == 0
    # 9 <= M <= 16 on the two-pass GEMV path (K = N = 4096): the whole call
    # is checked before any launch
    assert L.tq_matmul_path(0, 4096, 4096, 12) == 0 and L.tq_matmul_path(2, 4096, 4096, 16) == 0
    assert f(0, A16, 4096, 4096, A16, A16, 12, NUL, A16, 4096, ctypes.c_void_p(0x10010), 4096,
             NUL) == 4                                                            # workspace
    assert f(0, A16, 4096, 4096, A2, A16, 16, NUL, A16, 4096, NUL, 0, NUL) == 4  # q
    assert f(2, A16, 4096, 4096, A16, A16, 12, NUL, A16, 4096, NUL, 0, NUL) == 1  # IQ4_NL table
    assert f(0, A16, 4096, 4096, A16, A16, 16, NUL, A16, 4095, NUL, 0, NUL) == 3  # ldy < N
    # the split GEMM path (M = 128): checked the same way
    assert L.tq_matmul_path(0, 4096, 4096, 128) == 5
    assert f(0, A16, 4096, 4096, A16, A16, 128, NUL, A16, 4096, ctypes.c_void_p(0x10010), 1 << 24,
             NUL) == 4                                                            # workspace
    assert f(0, A16, 4096, 4096, A16, NUL, 128, NUL, A16, 4096, NUL, 0, NUL) == 1  # d NULL


def test_matmul_path(L):
    """tq_matmul's path: GEMV for M <= 8; above, the least estimated time of
    decode passes (9 <= M <= 64), the GEMM, and the GEMM with K split over
    workgroups.  The expected paths are the fastest measured on MI355X for
    these shapes (graph-replayed, per call, us): e.g. Q4_0 K=N=4096 M=16:
    passes 12.5, split GEMM 13.8, GEMM 25.7; M=128: split 18.3, GEMM 26.3;
    N=14336: no split fits (224 blocks), M=16 passes 21.6 vs GEMM 27.8,
    M=32 GEMM 28.2 vs passes 43.8; K=1024 M=128: GEMM 10.4 vs split 12.4."""
    G, GEMM, SPLIT = 0, 1, 5
    assert L.tq_matmul_path(1, 4096, 4096, 8) == G
    assert L.tq_matmul_path(0, 4096, 4096, 16) == G
    assert L.tq_matmul_path(2, 4096, 4096, 9) == G
    assert L.tq_matmul_path(0, 4096, 4096, 32) == SPLIT
    assert L.tq_matmul_path(0, 4096, 4096, 128) == SPLIT
    assert L.tq_matmul_path(2, 4096, 4096, 256) == SPLIT
    assert L.tq_matmul_path(0, 4096, 1024, 9) == SPLIT
    assert L.tq_matmul_path(0, 4096, 14336, 16) == G
    assert L.tq_matmul_path(0, 4096, 14336, 32) == GEMM
    assert L.tq_matmul_path(1, 4096, 14336, 16) == GEMM
    assert L.tq_matmul_path(0, 1024, 4096, 128) == GEMM
    assert L.tq_matmul_path(0, 8192, 4096, 16) == G
    assert L.tq_matmul_path(2, 8192, 4096, 128) == SPLIT
    assert L.tq_matmul_path(2, 4096, 4096, 512) == GEMM        # 256 blocks: a full round
    assert L.tq_matmul_path(1, 4096, 128001, 128) == GEMM      # 2001 blocks
    assert L.tq_matmul_path(9, 4096, 4096, 12) == -1
    assert L.tq_matmul_path(0, 4000 + 1, 4096, 12) == -1


def test_matmul_workspace_bytes(L):
    """Slots for up to 8 rows at the front (the first 1 MiB holds them for
    every shape); on the split path 1 MiB + S * M * N fp32 planes; for
    tq_matmul_x the unfused path adds q and d after the first 1 MiB."""
    MiB = 1 << 20
    for t, K, N, M in ((0, 4096, 4096, 128), (2, 4096, 1024, 9), (1, 8192, 4096, 128)):
        assert L.tq_matmul_path(t, K, N, M) == 5
        ws = L.tq_matmul_workspace_bytes(t, K, N, M)
        S = (ws - MiB) // (M * N * 4)
        assert S in (2, 4, 8) and ws == MiB + S * M * N * 4
        wx = L.tq_matmul_x_workspace_bytes(t, K, N, M)
        assert wx >= MiB + M * K + M * (K // 32) * 2 + S * M * N * 4
    for t, K, N, M in ((0, 4096, 4096, 8), (0, 4096, 14336, 32), (2, 4096, 4096, 512)):
        assert L.tq_matmul_workspace_bytes(t, K, N, M) == L.tq_qgemv_workspace_bytes(t, K, N, min(M, 8))
    # the fused decode needs only the slots; the unfused path q and d too
    assert L.tq_matmul_x_workspace_bytes(0, 4096, 4096, 1) == L.tq_qgemv_workspace_bytes(0, 4096, 4096, 1)
    assert L.tq_matmul_x_workspace_bytes(0, 4096, 14336, 4) >= MiB + 4 * 4096 + 4 * 128 * 2
    assert L.tq_matmul_workspace_bytes(9, 4096, 4096, 16) == 0
    assert L.tq_matmul_x_workspace_bytes(0, 4096, 4096, 0) == 0


def test_matmul_x_validation(L):
    f = L.tq_matmul_x
    assert f(0, A16, 64, 32, 3, A16, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 2        # dtype
    assert f(0, A16, 64, 32, 0, A16, 63, 1, NUL, A16, 32, NUL, 0, NUL) == 3        # ldx < K
    assert f(0, NUL, 64, 32, 0, A16, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 1        # tiles
    assert f(0, A16, 64, 32, 0, NUL, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 1        # x
    assert f(0, A16, 64, 32, 0, A2, 64, 1, NUL, A16, 32, NUL, 0, NUL) == 4         # fp32 x
    assert f(0, NUL, 64, 32, 0, NUL, 64, 0, NUL, NUL, 32, NUL, 0, NUL) == 0        # M == 0
    # the unfused path (M = 40) needs a workspace for q and d
    assert f(0, A16, 1024, 4096, 0, A16, 1024, 40, NUL, A16, 4096, NUL, 0, NUL) == 1
    assert f(0, A16, 1024, 4096, 0, A16, 1024, 40, NUL, A16, 4096, A16, 4096, NUL) == 3


def test_gemv_m_limit(L):
    assert L.tq_qgemv(0, A16, 64, 32, A16, A16, 9, NUL, A16, 32, NUL, 0, NUL) == 3
    assert L.tq_qgemv(0, A16, 64, 32, A16, A16, 1, NUL, A16, 32, ctypes.c_void_p(0x10010), 4096, NUL) == 4
    assert L.tq_block_dots(0, A16, 64, 32, A16, 9, NUL, A16, 0, NUL) == 3
    assert L.tq_block_dots(0, A16, 64, 32, A16, 9, NUL, A16, 7, NUL) == 2


def test_shape_limits(L):
    """N <= 2^27 and M * K < 2^34 (every grid then fits a dispatch's 32-bit
    work-item count): one past either limit is TQ_E_SHAPE before any launch."""
    big_n = 2 ** 27 + 1
    assert L.tq_supported(0, 32, 2 ** 27, 1, 0) == 1
    assert L.tq_supported(0, 32, big_n, 1, 0) == 0
    assert L.tq_supported(1, 32, big_n, 512, 1) == 0
    assert L.tq_supported(0, 2 ** 20, 2 ** 20 - 32, 2 ** 14 - 1, 1) == 1
    assert L.tq_supported(0, 2 ** 20, 2 ** 20 - 32, 2 ** 14, 1) == 0      # M * K = 2^34
    assert L.tq_tiled_bytes(0, 32, big_n) == 0
    assert L.tq_repack_tiles(0, A16, 32, big_n, A16, NUL) == 3
    assert L.tq_qgemm(0, A16, 32, big_n, A16, A16, 1, NUL, A16, big_n, NUL) == 3
    assert L.tq_qgemv(0, A16, 32, big_n, A16, A16, 1, NUL, A16, big_n, NUL, 0, NUL) == 3
    assert L.tq_quantize_act(0, A16, 2 ** 14, 2 ** 20, 2 ** 20, A16, A16, NUL) == 3
    assert L.tq_quantize_act_mx(0, A16, 2 ** 14, 2 ** 20, 2 ** 20, A16, A16, NUL) == 3
    assert L.tq_qgemm_mx(A16, 32, big_n, A16, A16, 1, A16, big_n, NUL) == 3


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import block_quantized_matmul_repack_amd as tq
    x = torch.zeros(2, 64)
    with pytest.raises(tq.TiledqError):
        tq.quantize_act(x)
    with pytest.raises(tq.TiledqError):
        tq.repack_tiles(0, torch.zeros(36, dtype=torch.uint8), 64, 1)


def test_product_code_never_touches_oracle():
    """The HIP path and its binding neither import nor load the oracle."""
    pkg = os.path.join(ROOT, "block_quantized_matmul_repack_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in src.lower(), fn
                assert "synth" not in src, fn


def test_flat_validation(L):
    A4 = ctypes.c_void_p(0x10004)
    # unpack: Q4_K has no inverse; alignment as the repack's flat buffer
    assert L.tq_unpack_tiles(5, A16, 256, 32, A16, NUL) == 2
    assert L.tq_unpack_tiles(9, A16, 64, 32, A16, NUL) == 2
    assert L.tq_unpack_tiles(0, A16, 48, 32, A16, NUL) == 3
    assert L.tq_unpack_tiles(0, A2, 64, 32, A16, NUL) == 4          # tiles need 16
    assert L.tq_unpack_tiles(4, A16, 64, 32, A2, NUL) == 4          # Q4_1 flat needs 4
    assert L.tq_unpack_tiles(0, NUL, 64, 0, NUL, NUL) == 0
    for fn in ("tq_qgemv_flat", "tq_qgemm_flat", "tq_matmul_flat"):
        f = getattr(L, fn)
        # (type, flat, K, N, q, d, M, lut, y, ldy, stream)
        assert f(9, A16, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 2, fn
        assert f(5, A16, 288, 32, A16, A16, 1, NUL, A16, 32, NUL) == 3, fn     # Q4_K: K % 256
        assert f(5, A4, 256, 32, A16, A16, 1, NUL, A16, 32, NUL) == 4, fn      # Q4_K flat: 16
        assert f(3, A2, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 4, fn       # MXFP4 flat: 4
        assert f(2, A16, 64, 32, A16, A16, 1, NUL, A16, 32, NUL) == 1, fn      # IQ4_NL table
        assert f(0, A16, 64, 32, A16, A16, 1, NUL, A16, 31, NUL) == 3, fn      # ldy < N
        assert f(0, NUL, 64, 0, NUL, NUL, 3, NUL, NUL, 0, NUL) == 0, fn
    assert L.tq_qgemv_flat(0, A16, 64, 32, A16, A16, 9, NUL, A16, 32, NUL) == 3
    assert L.tq_block_dots(0, A16, 64, 32, A16, 1, NUL, A16, 4, NUL) == 2       # unknown path
    assert L.tq_block_dots(0, A16, 64, 32, A16, 9, NUL, A16, 2, NUL) == 3       # flat GEMV, M > 8
    assert L.tq_block_dots(5, A4, 256, 32, A16, 1, NUL, A16, 3, NUL) == 4       # Q4_K flat: 16


def test_mx_validation(L):
    q = L.tq_quantize_act_mx
    assert q(5, A16, 1, 64, 64, A16, A16, NUL) == 2
    assert q(0, A16, 1, 60, 64, A16, A16, NUL) == 3
    assert q(0, A16, 1, 64, 32, A16, A16, NUL) == 3         # ldx < K
    assert q(0, NUL, 1, 64, 64, A16, A16, NUL) == 1
    assert q(0, A16, 1, 64, 64, A16, NUL, NUL) == 1
    assert q(0, A2, 1, 64, 64, A16, A16, NUL) == 4          # fp32 needs 4 B
    assert q(0, A16, 1, 64, 64, A2, A16, NUL) == 4          # q needs 8 B
    assert q(0, NUL, 0, 64, 64, NUL, NUL, NUL) == 0
    g = L.tq_qgemm_mx
    assert g(A16, 48, 32, A16, A16, 1, A16, 32, NUL) == 3
    assert g(A16, 64, 32, A16, A16, 1, A16, 31, NUL) == 3   # ldy < N
    assert g(NUL, 64, 32, A16, A16, 1, A16, 32, NUL) == 1
    assert g(A16, 64, 32, NUL, A16, 1, A16, 32, NUL) == 1
    assert g(A16, 64, 32, A16, NUL, 1, A16, 32, NUL) == 1
    assert g(A16, 64, 32, A16, A16, 1, NUL, 32, NUL) == 1
    assert g(A2, 64, 32, A16, A16, 1, A16, 32, NUL) == 4
    assert g(A16, 64, 32, A2, A16, 1, A16, 32, NUL) == 4
    assert g(A16, 64, 32, A16, A16, 1, A2, 32, NUL) == 4
    assert g(NUL, 64, 32, NUL, NUL, 0, NUL, 32, NUL) == 0   # M == 0
    assert g(NUL, 64, 0, NUL, NUL, 4, NUL, 0, NUL) == 0     # N == 0


# --- the torch binding checks every buffer against the sizes the call will
# touch before anything reaches the library: CPU tensors of the wrong size get
# a size error (a launch would read or write past them); of the right size,
# the GPU-only error.  Nothing here launches a kernel.

def _raises(fn, words):
    from block_quantized_matmul_repack_amd import TiledqError
    with pytest.raises(TiledqError) as e:
        fn()
    assert any(w in str(e.value) for w in words), str(e.value)


def test_binding_rejects_short_buffers_before_launch():
    import torch
    import block_quantized_matmul_repack_amd as tq
    K, N, M = 256, 70, 3
    tb = tq.tiled_bytes(tq.Q4_0, K, N)
    fb = tq.flat_bytes(tq.Q4_0, K, N)
    tiles = torch.zeros(tb, dtype=torch.uint8)
    short = torch.zeros(tb - 1, dtype=torch.uint8)
    q = torch.zeros((M, K), dtype=torch.int8)
    d = torch.zeros((M, K // 32), dtype=torch.float16)
    x = torch.zeros((M, K), dtype=torch.float32)
    size = ("holds", "needs", "must be", "exceeds", "columns", "too small")
    gpu = ("GPU tensors only",)
    for fn in (tq.qgemv, tq.qgemm, tq.matmul):
        _raises(lambda: fn(tq.Q4_0, short, K, N, q, d), size)
        _raises(lambda: fn(tq.Q4_0, tiles, K + 32, N, q, d), size)            # q width != K
        _raises(lambda: fn(tq.Q4_0, tiles, K, N, q, d[:2]), size)             # d short
        _raises(lambda: fn(tq.Q4_0, tiles, K, N, q, d.float()), size)         # d dtype
        _raises(lambda: fn(tq.Q4_0, tiles, K, N, q.to(torch.uint8), d), size)
        _raises(lambda: fn(tq.Q4_0, tiles, K, N, q, d,
                           out=torch.zeros((M - 1, N), dtype=torch.float32)), size)
        _raises(lambda: fn(tq.Q4_0, tiles, K, N, q, d,
                           out=torch.zeros((M, N - 1), dtype=torch.float32)), size)
        _raises(lambda: fn(tq.Q4_0, tiles, K, N, q, d), gpu)
    _raises(lambda: tq.qgemv_x(tq.Q4_0, short, K, N, x), size)
    _raises(lambda: tq.qgemv_x(tq.Q4_0, tiles, K + 32, N, x), size)
    _raises(lambda: tq.qgemv_x(tq.Q4_0, tiles, K, N, x), gpu)
    flat = torch.zeros(fb, dtype=torch.uint8)
    for fn in (tq.qgemv_flat, tq.qgemm_flat, tq.matmul_flat):
        _raises(lambda: fn(tq.Q4_0, flat[:-1], K, N, q, d), size)
        _raises(lambda: fn(tq.Q4_0, flat, K, N, q, d[:1]), size)
        _raises(lambda: fn(tq.Q4_0, flat, K, N, q, d), gpu)
    _raises(lambda: tq.quantize_act(x, q=q[:2]), size)
    _raises(lambda: tq.quantize_act(x, d=d[:2]), size)
    _raises(lambda: tq.quantize_act(x, K=K + 32), size)
    _raises(lambda: tq.quantize_act(x, q=q, d=d), gpu)
    isum = torch.zeros((M, N, K // 32), dtype=torch.int32)
    _raises(lambda: tq.block_dots(tq.Q4_0, tiles, K, N, q, out=isum[:, :-1]), size)
    _raises(lambda: tq.block_dots(tq.Q4_0, short, K, N, q), size)
    _raises(lambda: tq.block_dots(tq.Q4_0, flat[:-1], K, N, q, path=tq.PATH_GEMV_FLAT), size)
    _raises(lambda: tq.block_dots(tq.Q4_0, tiles, K, N, q, out=isum), gpu)
    _raises(lambda: tq.repack_tiles(tq.Q4_0, flat[:-1], K, N), size)
    _raises(lambda: tq.repack_tiles(tq.Q4_0, flat, K, N, out=short), size)
    _raises(lambda: tq.unpack_tiles(tq.Q4_0, short, K, N), size)
    _raises(lambda: tq.unpack_tiles(tq.Q4_0, tiles, K, N, out=flat[:-1]), size)
    _raises(lambda: tq.repack_tiles(tq.Q4_0, flat, K, N, out=tiles), gpu)
    sink = torch.zeros(tq.ops.STREAM_READ_BLOCKS, dtype=torch.int32)
    _raises(lambda: tq.stream_read(tiles, tb + 16), size)
    _raises(lambda: tq.stream_read(tiles, sink=sink[:-1]), size)
    _raises(lambda: tq.stream_read(tiles, sink=sink.float()), size)
    _raises(lambda: tq.stream_read(tiles, sink=sink), gpu)


def test_noalloc_scratch_covers_every_split(L):
    """tq_qgemv_noalloc's device array holds the K-split workspace of every
    shape tq_qgemv accepts (the entry point rejects larger needs with
    TQ_E_SHAPE, which no accepted shape reaches)."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+TQ_NOALLOC_SCRATCH_BYTES\s+\(1u\s*<<\s*(\d+)\)", text)
    assert m
    cap = 1 << int(m.group(1))
    worst = 0
    for K in (64, 128, 512, 1024, 4096, 1 << 20):
        for nct in range(1, 600):
            for M in (1, 8):
                worst = max(worst, L.tq_qgemv_workspace_bytes(0, K, 32 * nct, M))
    assert 0 < worst <= cap


def test_stream_read_validation(L):
    """The streaming-read instrument rejects bad arguments on the host: the
    byte count is checked first, an empty read is OK with no launch, then
    pointers and alignment."""
    V = ctypes.c_void_p
    assert L.tq_stream_read(None, 0, None, None) == 0
    assert L.tq_stream_read(V(4096), 20, V(4096), None) == 3       # not whole 16-byte chunks
    assert L.tq_stream_read(None, 16, V(4096), None) == 1
    assert L.tq_stream_read(V(4096), 16, None, None) == 1
    assert L.tq_stream_read(V(4104), 16, V(4096), None) == 4       # src not 16-byte aligned
    assert L.tq_stream_read(V(4096), 16, V(4098), None) == 4       # sink not 4-byte aligned

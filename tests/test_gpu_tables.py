"""IQ4_NL through every kernel with other 16-entry tables.

Page: "Block-32 Quantized Formats", IQ4_NL -- each 4-bit index selects an
entry of a 16-entry non-linear table, then the row scale applies.  The page
names the table without printing it, and the library takes it as an input
(16 int8), so the kernels must be right for any table, not only for the
stand-in the other tests use.  Tables here: the int8 extremes (-128 and 127
mixed), all -128 (with sign activations every code is +-127, so the block
dot reaches -128 * 127 * 32 = -520192), seeded random tables with repeats,
and one with a single non-zero entry.  Bit-exact block dots of the GEMV,
GEMM and both flat kernels; fp32 y of every product entry point within the
tolerance of gpu_helpers, against the oracle called with the same table.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_y, make

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

IQ4_NL = synth.IQ4_NL


def _tables():
    rng = np.random.default_rng(20261202)
    t = {
        "extremes": np.array([-128, 127] * 8, dtype=np.int8),
        "all_min": np.full(16, -128, dtype=np.int8),
        "one_entry": np.array([0] * 15 + [-128], dtype=np.int8),
    }
    for i in range(2):
        t[f"random{i}"] = rng.integers(-128, 128, size=16).astype(np.int8)
    t["random_repeats"] = rng.choice(np.array([-128, -1, 0, 1, 127], dtype=np.int8), size=16)
    return t


TABLES = _tables()


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_matmul_repack_amd as tq
    tq.lib()
    return tq


def _inputs(name, M, K, N, seed):
    inp = make(IQ4_NL, K, N, M, seed=seed)
    x = inp.x.copy()
    if name == "all_min":
        # every block's amax is 1: all codes +-127; row 0 all +1 makes each
        # of its block dots -520192 exactly
        x = np.where(np.random.default_rng(seed).random(x.shape) < 0.5, -1.0, 1.0).astype(np.float32)
        x[0] = 1.0
    return inp, x


CASES = [(1, 96, 33), (4, 512, 65), (8, 4096, 40), (33, 1024, 97), (130, 256, 64)]


@pytest.mark.parametrize("name", list(TABLES))
@pytest.mark.parametrize("M,K,N", CASES)
def test_tiled_any_table(tq, name, M, K, N):
    lut = TABLES[name]
    inp, x = _inputs(name, M, K, N, seed=M * 7919 + K + N)
    tiles = oracle.repack(IQ4_NL, inp.flat, K, N)
    tdev = torch.from_numpy(tiles).cuda()
    q, d = oracle.quantize_act(x)
    qd, dd = tq.quantize_act(torch.from_numpy(x).cuda())
    assert np.array_equal(qd.cpu().numpy(), q)
    ref = oracle.block_dots(IQ4_NL, tiles, K, N, q, lut)
    if name == "all_min":
        assert (ref[0] == -128 * 127 * 32).all()
    paths = [tq.PATH_GEMM] + ([tq.PATH_GEMV] if M <= 8 else [])
    for path in paths:
        got = tq.block_dots(IQ4_NL, tdev, K, N, qd, lut=lut, path=path).cpu().numpy()
        assert np.array_equal(got, ref), (name, path, np.argwhere(got != ref)[:4])
    y_ref, acond = oracle.matmul(IQ4_NL, tiles, K, N, q, d, lut)
    what = (name, M, K, N)
    check_y(tq.qgemm(IQ4_NL, tdev, K, N, qd, dd, lut=lut).cpu().numpy(), y_ref, acond, what)
    check_y(tq.matmul(IQ4_NL, tdev, K, N, qd, dd, lut=lut).cpu().numpy(), y_ref, acond, what)
    if M <= 8:
        for split in (False, True):
            check_y(tq.qgemv(IQ4_NL, tdev, K, N, qd, dd, lut=lut, split=split).cpu().numpy(),
                    y_ref, acond, what + (split,))
        xd = torch.from_numpy(x).cuda()
        check_y(tq.qgemv_x(IQ4_NL, tdev, K, N, xd, lut=lut).cpu().numpy(), y_ref, acond, what)
        check_y(tq.matmul_x(IQ4_NL, tdev, K, N, xd, lut=lut).cpu().numpy(), y_ref, acond, what)


@pytest.mark.parametrize("name", list(TABLES))
@pytest.mark.parametrize("M,K,N", [(1, 96, 33), (8, 512, 65), (33, 1024, 40)])
def test_flat_any_table(tq, name, M, K, N):
    lut = TABLES[name]
    inp, x = _inputs(name, M, K, N, seed=M * 104729 + K + N)
    q, d = oracle.quantize_act(x)
    flat = torch.from_numpy(inp.flat).cuda()
    qd, dd = torch.from_numpy(q).cuda(), tq.quantize_act(torch.from_numpy(x).cuda())[1]
    ref = oracle.block_dots_flat(IQ4_NL, inp.flat, K, N, q, lut)
    paths = [tq.PATH_GEMM_FLAT] + ([tq.PATH_GEMV_FLAT] if M <= 8 else [])
    for path in paths:
        got = tq.block_dots(IQ4_NL, flat, K, N, qd, lut=lut, path=path).cpu().numpy()
        assert np.array_equal(got, ref), (name, path, np.argwhere(got != ref)[:4])
    y_ref, acond = oracle.matmul_flat(IQ4_NL, inp.flat, K, N, q, d, lut)
    what = ("flat", name, M, K, N)
    check_y(tq.qgemm_flat(IQ4_NL, flat, K, N, qd, dd, lut=lut).cpu().numpy(), y_ref, acond, what)
    check_y(tq.matmul_flat(IQ4_NL, flat, K, N, qd, dd, lut=lut).cpu().numpy(), y_ref, acond, what)
    if M <= 8:
        check_y(tq.qgemv_flat(IQ4_NL, flat, K, N, qd, dd, lut=lut).cpu().numpy(), y_ref, acond,
                what)

"""Shared helpers of the GPU parity tests: seeded inputs (synth), the oracle's
reference values, and the tolerance of the fp32 output.

Tolerance (fp32 y against the oracle's fp64 y_ref): an element passes iff
|y - y_ref| <= 1e-3 * max(|y_ref|, 1e-2 * A), A = sum_k |W*A| the sum of the
magnitudes of the terms.  1e-3 is the stated relative bound; the floor keeps
elements whose terms cancel from demanding more than fp32 can give.  With
exact int32 block dots the fp32 error is below about K/32 * 2^-24 * A.
"""
import numpy as np
import torch

import oracle
import synth

TOL = 1e-3
FLOOR = 1e-2


def seed_for(*parts):
    return abs(hash(tuple(parts))) % (2 ** 31)


def make(qtype, K, N, M, seed=0, dist=None, act="f32"):
    dist = dist or {synth.Q8_0: "absnormal", synth.MXFP4: "e8m0",
                    synth.Q4_1: "minmax", synth.Q4_K: "q4k"}.get(qtype, "uniform")
    w = synth.Workload("t", qtype, K, N, M, dist, act_dtype=act, seed=seed)
    return synth.make_inputs(w)


def to_dev_act(x, act):
    if act == "f32":
        return torch.from_numpy(x).cuda()
    t = torch.from_numpy(x.view(np.int16)).cuda()
    return t.view(torch.bfloat16 if act == "bf16" else torch.float16)


def check_y(y, y_ref, acond, what="", floor=FLOOR):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = TOL * np.maximum(np.abs(y_ref), floor * acond)
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, (what, [(int(i), int(j), float(y[i, j]), float(y_ref[i, j]))
                                     for i, j in zip(*bad)][:5])
    nrm = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / nrm) if nrm else 0.0


def oracle_matmul_rows(qtype, tiles, K, N, q, d, lut=None, n0=0, n1=None, threads=None):
    """oracle.matmul over output rows n0..n1, the rows cut into one range per
    host thread (the oracle's C call releases the GIL): what lets a test
    check a full-size GEMM output in seconds.  Returns (y_ref, acond) for
    all N columns, zero outside n0..n1."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    n1 = N if n1 is None else n1
    T = threads or min(16, len(os.sched_getaffinity(0)))
    cuts = [n0 + (n1 - n0) * i // T for i in range(T + 1)]
    with ThreadPoolExecutor(T) as ex:
        parts = list(ex.map(lambda j: oracle.matmul(qtype, tiles, K, N, q, d, lut,
                                                    n0=cuts[j], n1=cuts[j + 1]), range(T)))
    y = sum(p[0] for p in parts)
    a = sum(p[1] for p in parts)
    return y, a


def tiles_slice(tiles, qtype, K, s0, s1):
    ts = oracle.tile_bytes(qtype)
    nkt = K // 32
    return tiles[s0 * nkt * ts: s1 * nkt * ts]


# The block-scaled MXFP4 x MXFP8 path (tq_qgemm_mx): its bound is derived in
# test_gpu_mx.py's docstring.
def mx_bound(K, acond, adds=1):
    """Elementwise bound of the block-scaled path: 2^-14 * A + (K/64 + adds)
    * 2^-24 * A, A = sum of |terms|; `adds` bounds the fp32 additions of
    partial sums after the matrix core's accumulation: 1 without a split
    (the two wave groups' sums), at most 2 S with K split into S ranges (one
    group sum per range, then S - 1 plane additions)."""
    return (2.0 ** -14 + (-(-K // 64) + adds) * 2.0 ** -24) * acond


def check_mx(y, y_ref, acond, what, K, adds=1):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    ok = (err <= 1e-3 * np.abs(y_ref)) | (err <= mx_bound(K, acond, adds))
    bad = np.nonzero(~ok)
    assert bad[0].size == 0, (what, [(int(i), int(j), float(y[i, j]), float(y_ref[i, j]),
                                      float(err[i, j] / acond[i, j]))
                                     for i, j in zip(*bad)][:5])
    assert np.linalg.norm(y - y_ref) <= 1e-4 * np.linalg.norm(y_ref), what

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


def tiles_slice(tiles, qtype, K, s0, s1):
    ts = oracle.tile_bytes(qtype)
    nkt = K // 32
    return tiles[s0 * nkt * ts: s1 * nkt * ts]

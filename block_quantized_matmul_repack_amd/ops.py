"""Torch-facing binding of the tiledq C ABI.

Argument marshalling only: device pointers, sizes and the current HIP stream
go to libtiledq.so; every step of the computation runs in its HIP kernels.
Tensors must live on the GPU; outputs are allocated with torch unless given.
"""
import ctypes
import functools

import torch

from ._lib import TiledqError, check, lib

Q4_0, Q8_0, IQ4_NL, MXFP4, Q4_1, Q4_K = 0, 1, 2, 3, 4, 5
F32, BF16, F16 = 0, 1, 2
PATH_GEMV, PATH_GEMM, PATH_GEMV_FLAT, PATH_GEMM_FLAT, PATH_GEMM_MX, PATH_GEMM_SPLIT = 0, 1, 2, 3, 4, 5

_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def _ptr(t):
    """Device address as an int (the C-ABI's pointer arguments take ints)."""
    return t.data_ptr() if t is not None else None


# torch's raw handle of a device's current stream (what
# torch.cuda.current_stream(device).cuda_stream returns, without building a
# Stream object on every call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    """The current HIP stream of tensor t's device, as an int handle."""
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


@functools.lru_cache(maxsize=4096)
def _size_query(name, *args):
    """A size / workspace query of the C ABI; they depend on their arguments
    alone, so results are cached."""
    return getattr(lib(), name)(*args)


def _need_cuda(*ts, out=None):
    """Inputs must be contiguous GPU tensors; `out` a GPU tensor (its row
    stride is passed to the library as ldy, checked by _check_out)."""
    for t in ts:
        if t is not None and not t.is_cuda:
            raise TiledqError("tiledq operates on GPU tensors only")
        if t is not None and not t.is_contiguous():
            raise TiledqError("tiledq expects contiguous tensors")
    if out is not None and not out.is_cuda:
        raise TiledqError("tiledq operates on GPU tensors only")


def _nbytes(t):
    return t.numel() * t.element_size()


def _need_bytes(name, what, t, nbytes):
    if t is not None and _nbytes(t) < nbytes:
        raise TiledqError(f"{name}: {what} holds {_nbytes(t)} bytes, needs {nbytes}")


def _check_weights(name, qtype, w, K, N, flat=False):
    """The weight buffer covers the tiles (or flat blocks) of (qtype, K, N)."""
    nbytes = _size_query("tq_flat_bytes" if flat else "tq_tiled_bytes", qtype, K, N)
    if nbytes == 0 and N > 0:
        raise TiledqError(f"{name}: type {qtype} with K={K}, N={N} is not a valid shape")
    _need_bytes(name, "flat" if flat else "tiles", w, nbytes)


def _check_act(name, q, d, K):
    """q is int8 [M, K] and d fp16 with M * K/32 elements; returns M."""
    if q.dim() != 2 or q.dtype != torch.int8 or q.shape[1] != K:
        raise TiledqError(f"{name}: q must be int8 [M, K={K}], got {q.dtype} {tuple(q.shape)}")
    M = q.shape[0]
    if d is not None:
        if d.dtype != torch.float16:
            raise TiledqError(f"{name}: d must be float16, got {d.dtype}")
        if d.numel() < M * (K // 32):
            raise TiledqError(f"{name}: d holds {d.numel()} scales, needs {M * (K // 32)}")
    return M


def _check_out(name, out, M, N):
    """out is fp32 with unit column stride, at least M rows and N columns."""
    if out is None:
        return
    if out.dim() != 2 or out.dtype != torch.float32 or out.stride(1) != 1 or \
            out.shape[0] < M or out.shape[1] < N:
        raise TiledqError(f"{name}: out must be float32 [>={M}, >={N}] with unit column "
                          f"stride, got {out.dtype} {tuple(out.shape)}")


def _lut_arg(lut):
    if lut is None:
        return None
    vals = [int(v) for v in (lut.tolist() if hasattr(lut, "tolist") else lut)]
    if len(vals) != 16 or any(v < -128 or v > 127 for v in vals):
        raise TiledqError("lut must hold 16 int8 values")
    return (ctypes.c_int8 * 16)(*vals)


def tile_bytes(qtype):
    return lib().tq_tile_bytes(qtype)


def block_bytes(qtype):
    return lib().tq_block_bytes(qtype)


def tiled_bytes(qtype, K, N):
    return lib().tq_tiled_bytes(qtype, K, N)


def flat_bytes(qtype, K, N):
    return lib().tq_flat_bytes(qtype, K, N)


def supported(qtype, K, N, M, path=PATH_GEMV):
    return bool(lib().tq_supported(qtype, K, N, M, path))


def repack_tiles(qtype, flat, K, N, out=None):
    """Flat GGML blocks (uint8 GPU tensor) -> tiles (uint8 GPU tensor)."""
    nbytes = tiled_bytes(qtype, K, N)
    _check_weights("repack_tiles", qtype, flat, K, N, flat=True)
    _need_bytes("repack_tiles", "out", out, nbytes)
    _need_cuda(flat, out)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=flat.device)
    check(lib().tq_repack_tiles(qtype, _ptr(flat), K, N, _ptr(out), _stream(flat)),
          "tq_repack_tiles")
    return out


def quantize_act(x, K=None, q=None, d=None):
    """x [M, >=K] fp32 / bf16 / fp16 -> (q int8 [M, K], d fp16 [M, K/32])."""
    if x.dim() != 2 or x.dtype not in _DTYPES:
        raise TiledqError("quantize_act: x must be 2-D fp32, bf16 or fp16")
    if x.stride(1) != 1:
        raise TiledqError("quantize_act: x must have unit column stride")
    M, Kx = x.shape
    K = Kx if K is None else K
    if K > Kx:
        raise TiledqError(f"quantize_act: K={K} exceeds the {Kx} columns of x")
    if q is not None and q.dtype != torch.int8:
        raise TiledqError("quantize_act: q must be int8")
    if d is not None and d.dtype != torch.float16:
        raise TiledqError("quantize_act: d must be float16")
    _need_bytes("quantize_act", "q", q, M * K)
    _need_bytes("quantize_act", "d", d, 2 * M * (K // 32))
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((M, K // 32), dtype=torch.float16, device=x.device)
    if not x.is_cuda:
        raise TiledqError("tiledq operates on GPU tensors only")
    _need_cuda(q, d)
    check(lib().tq_quantize_act(_DTYPES[x.dtype], _ptr(x), M, K, x.stride(0), _ptr(q), _ptr(d),
                                _stream(x)), "tq_quantize_act")
    return q, d


def _out(q, N, out):
    """`out` as given (the caller has checked it with _check_out), else a new
    fp32 [M, N] tensor on q's device."""
    if out is None:
        out = torch.empty((q.shape[0], N), dtype=torch.float32, device=q.device)
    return out


# Zero-filled qgemv workspaces, one per (device, stream): every call leaves
# its workspace zero-filled, so it is reused by later calls on the same stream
# without clearing (calls on one stream never overlap).  A HIP graph captured
# on a stream keeps that stream's workspace: replaying it on another stream
# while calls run on the capture stream would share the workspace, so replay
# it on the capture stream or keep the two apart in time.
_workspaces = {}


def workspace(device, stream_handle, nbytes):
    key = (device, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def qgemv(qtype, tiles, K, N, q, d, lut=None, out=None, split=True):
    """Decode product y [M, N] = W (tiles) x A (q, d), M <= 8.  split=False
    runs one workgroup per stripe (no workspace)."""
    M = _check_act("tq_qgemv", q, d, K)
    _check_weights("tq_qgemv", qtype, tiles, K, N)
    _check_out("tq_qgemv", out, M, N)
    _need_cuda(tiles, q, d, out=out)
    out = _out(q, N, out)
    st = _stream(q)
    need = _size_query("tq_qgemv_workspace_bytes", qtype, K, N, M) if split else 0
    ws = workspace(q.device, st, need) if need else None
    check(lib().tq_qgemv(qtype, _ptr(tiles), K, N, _ptr(q), _ptr(d), M, _lut_arg(lut),
                         _ptr(out), out.stride(0), _ptr(ws), need, st), "tq_qgemv")
    return out


def qgemv_noalloc(qtype, tiles, K, N, q, d, lut=None, out=None):
    """qgemv through the entry point that allocates nothing (its K-split
    scratch is a device array inside the library, shared by all calls on a
    GPU: calls that overlap on one GPU race).  Pass `out` to allocate
    nothing here either."""
    M = _check_act("tq_qgemv_noalloc", q, d, K)
    _check_weights("tq_qgemv_noalloc", qtype, tiles, K, N)
    _check_out("tq_qgemv_noalloc", out, M, N)
    _need_cuda(tiles, q, d, out=out)
    out = _out(q, N, out)
    check(lib().tq_qgemv_noalloc(qtype, _ptr(tiles), K, N, _ptr(q), _ptr(d), M, _lut_arg(lut),
                                 _ptr(out), out.stride(0), _stream(q)), "tq_qgemv_noalloc")
    return out


def qgemv_x(qtype, tiles, K, N, x, lut=None, out=None, split=True):
    """Decode in one launch: quantize x [M, >=K] (fp32 / bf16 / fp16) and
    multiply, y [M, N]; bit-identical to quantize_act followed by qgemv."""
    if x.dim() != 2 or x.dtype not in _DTYPES or x.stride(1) != 1:
        raise TiledqError("qgemv_x: x must be 2-D fp32, bf16 or fp16 with unit column stride")
    if x.shape[1] < K:
        raise TiledqError(f"qgemv_x: x has {x.shape[1]} columns, K={K}")
    _check_weights("tq_qgemv_x", qtype, tiles, K, N)
    _check_out("tq_qgemv_x", out, x.shape[0], N)
    _need_cuda(tiles, out=out)
    if not x.is_cuda:
        raise TiledqError("tiledq operates on GPU tensors only")
    M = x.shape[0]
    out = _out(x, N, out)
    st = _stream(x)
    need = _size_query("tq_qgemv_workspace_bytes", qtype, K, N, M) if split else 0
    ws = workspace(x.device, st, need) if need else None
    check(lib().tq_qgemv_x(qtype, _ptr(tiles), K, N, _DTYPES[x.dtype], _ptr(x), x.stride(0), M,
                           _lut_arg(lut), _ptr(out), out.stride(0), _ptr(ws), need, st),
          "tq_qgemv_x")
    return out


def qgemm(qtype, tiles, K, N, q, d, lut=None, out=None):
    """Prefill product y [M, N] on int8 MFMA, any M."""
    M = _check_act("tq_qgemm", q, d, K)
    _check_weights("tq_qgemm", qtype, tiles, K, N)
    _check_out("tq_qgemm", out, M, N)
    _need_cuda(tiles, q, d, out=out)
    out = _out(q, N, out)
    check(lib().tq_qgemm(qtype, _ptr(tiles), K, N, _ptr(q), _ptr(d), q.shape[0], _lut_arg(lut),
                         _ptr(out), out.stride(0), _stream(q)), "tq_qgemm")
    return out


def matmul_path(qtype, K, N, M):
    """The path matmul takes: PATH_GEMV, PATH_GEMM_SPLIT or PATH_GEMM."""
    return lib().tq_matmul_path(qtype, K, N, M)


def matmul(qtype, tiles, K, N, q, d, lut=None, out=None):
    """y [M, N] for any M: the library picks qgemv (M <= 8), one qgemv pass
    per 8 rows (up to 64 rows, where estimated faster), the GEMM with K split
    over workgroups (small output grids) or qgemm (matmul_path)."""
    M = _check_act("tq_matmul", q, d, K)
    _check_weights("tq_matmul", qtype, tiles, K, N)
    _check_out("tq_matmul", out, M, N)
    _need_cuda(tiles, q, d, out=out)
    out = _out(q, N, out)
    st = _stream(q)
    need = _size_query("tq_matmul_workspace_bytes", qtype, K, N, M)
    ws = workspace(q.device, st, need) if need else None
    check(lib().tq_matmul(qtype, _ptr(tiles), K, N, _ptr(q), _ptr(d), M, _lut_arg(lut),
                          _ptr(out), out.stride(0), _ptr(ws), need, st), "tq_matmul")
    return out


def matmul_x(qtype, tiles, K, N, x, lut=None, out=None):
    """y [M, N] from fp32 / bf16 / fp16 activations x [M, >=K], any M: the
    fused decode where it is cheaper, else quantize_act into the workspace
    followed by matmul's path."""
    if x.dim() != 2 or x.dtype not in _DTYPES or x.stride(1) != 1:
        raise TiledqError("matmul_x: x must be 2-D fp32, bf16 or fp16 with unit column stride")
    if x.shape[1] < K:
        raise TiledqError(f"matmul_x: x has {x.shape[1]} columns, K={K}")
    M = x.shape[0]
    _check_weights("tq_matmul_x", qtype, tiles, K, N)
    _check_out("tq_matmul_x", out, M, N)
    _need_cuda(tiles, out=out)
    if not x.is_cuda:
        raise TiledqError("tiledq operates on GPU tensors only")
    out = _out(x, N, out)
    st = _stream(x)
    need = _size_query("tq_matmul_x_workspace_bytes", qtype, K, N, M)
    ws = workspace(x.device, st, need) if need else None
    check(lib().tq_matmul_x(qtype, _ptr(tiles), K, N, _DTYPES[x.dtype], _ptr(x), x.stride(0), M,
                            _lut_arg(lut), _ptr(out), out.stride(0), _ptr(ws), need, st),
          "tq_matmul_x")
    return out


def unpack_tiles(qtype, tiles, K, N, out=None):
    """Tiles (uint8 GPU tensor) -> flat GGML blocks (uint8 GPU tensor)."""
    nbytes = flat_bytes(qtype, K, N)
    _check_weights("unpack_tiles", qtype, tiles, K, N)
    _need_bytes("unpack_tiles", "out", out, nbytes)
    _need_cuda(tiles, out)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=tiles.device)
    check(lib().tq_unpack_tiles(qtype, _ptr(tiles), K, N, _ptr(out), _stream(tiles)),
          "tq_unpack_tiles")
    return out[:nbytes]


def quantize_act_mx(x, K=None, q=None, e=None):
    """x [M, >=K] fp32 / bf16 / fp16 -> MXFP8 (q uint8 E4M3 codes [M, K],
    e uint8 E8M0 scales [M, K/32])."""
    if x.dim() != 2 or x.dtype not in _DTYPES:
        raise TiledqError("quantize_act_mx: x must be 2-D fp32, bf16 or fp16")
    if x.stride(1) != 1:
        raise TiledqError("quantize_act_mx: x must have unit column stride")
    M, Kx = x.shape
    K = Kx if K is None else K
    if K > Kx:
        raise TiledqError(f"quantize_act_mx: K={K} exceeds the {Kx} columns of x")
    _need_bytes("quantize_act_mx", "q", q, M * K)
    _need_bytes("quantize_act_mx", "e", e, M * (K // 32))
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if e is None:
        e = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    if not x.is_cuda:
        raise TiledqError("tiledq operates on GPU tensors only")
    _need_cuda(q, e)
    check(lib().tq_quantize_act_mx(_DTYPES[x.dtype], _ptr(x), M, K, x.stride(0), _ptr(q),
                                   _ptr(e), _stream(x)), "tq_quantize_act_mx")
    return q, e


def qgemm_mx(tiles, K, N, q, e, out=None):
    """MXFP4 tiles x MXFP8 activations on the block-scaled matrix cores:
    y [M, N] fp32, any M."""
    M = q.shape[0]
    if tiles.numel() * tiles.element_size() < tiled_bytes(MXFP4, K, N) or \
            q.numel() < M * K or e.numel() < M * (K // 32):
        raise TiledqError("qgemm_mx: buffer too small")
    _check_out("tq_qgemm_mx", out, M, N)
    _need_cuda(tiles, q, e, out=out)
    out = _out(q, N, out)
    check(lib().tq_qgemm_mx(_ptr(tiles), K, N, _ptr(q), _ptr(e), M, _ptr(out), out.stride(0),
                            _stream(q)), "tq_qgemm_mx")
    return out


def matmul_mx(tiles, K, N, q, e, out=None):
    """qgemm_mx with K split over workgroups where the output grid is small
    (tq_matmul_mx; the per-stream workspace holds the partial planes)."""
    M = q.shape[0]
    if tiles.numel() * tiles.element_size() < tiled_bytes(MXFP4, K, N) or \
            q.numel() < M * K or e.numel() < M * (K // 32):
        raise TiledqError("matmul_mx: buffer too small")
    _check_out("tq_matmul_mx", out, M, N)
    _need_cuda(tiles, q, e, out=out)
    out = _out(q, N, out)
    st = _stream(q)
    need = _size_query("tq_matmul_mx_workspace_bytes", K, N, M)
    ws = workspace(q.device, st, need) if need else None
    check(lib().tq_matmul_mx(_ptr(tiles), K, N, _ptr(q), _ptr(e), M, _ptr(out), out.stride(0),
                             _ptr(ws), need, st), "tq_matmul_mx")
    return out


def _flat_product(name, qtype, flat, K, N, q, d, lut, out):
    M = _check_act(name, q, d, K)
    _check_weights(name, qtype, flat, K, N, flat=True)
    _check_out(name, out, M, N)
    _need_cuda(flat, q, d, out=out)
    out = _out(q, N, out)
    check(getattr(lib(), name)(qtype, _ptr(flat), K, N, _ptr(q), _ptr(d), q.shape[0],
                               _lut_arg(lut), _ptr(out), out.stride(0), _stream(q)), name)
    return out


def qgemv_flat(qtype, flat, K, N, q, d, lut=None, out=None):
    """Decode product over flat (un-repacked) GGML blocks, M <= 8."""
    return _flat_product("tq_qgemv_flat", qtype, flat, K, N, q, d, lut, out)


def qgemm_flat(qtype, flat, K, N, q, d, lut=None, out=None):
    """Prefill product over flat GGML blocks, any M."""
    return _flat_product("tq_qgemm_flat", qtype, flat, K, N, q, d, lut, out)


def matmul_flat(qtype, flat, K, N, q, d, lut=None, out=None):
    """Product over flat GGML blocks for any M (qgemv_flat for M <= 8)."""
    return _flat_product("tq_matmul_flat", qtype, flat, K, N, q, d, lut, out)


def block_dots(qtype, tiles, K, N, q, lut=None, path=PATH_GEMV, out=None):
    """Integer block dots int32 [M, N, K/32] as computed inside qgemv / qgemm
    (paths PATH_GEMV_FLAT / PATH_GEMM_FLAT: `tiles` holds flat blocks)."""
    M = _check_act("tq_block_dots", q, None, K)
    _check_weights("tq_block_dots", qtype, tiles, K, N,
                   flat=path in (PATH_GEMV_FLAT, PATH_GEMM_FLAT))
    if out is not None and out.dtype != torch.int32:
        raise TiledqError("tq_block_dots: out must be int32")
    _need_bytes("tq_block_dots", "out", out, 4 * M * N * (K // 32))
    _need_cuda(tiles, q, out)
    if out is None:
        out = torch.empty((M, N, K // 32), dtype=torch.int32, device=q.device)
    check(lib().tq_block_dots(qtype, _ptr(tiles), K, N, _ptr(q), M, _lut_arg(lut), _ptr(out),
                              path, _stream(q)), "tq_block_dots")
    return out


STREAM_READ_BLOCKS = 2048       # TQ_STREAM_READ_BLOCKS: words of the sink


def stream_read(buf, nbytes=None, sink=None):
    """Measurement instrument: read the first `nbytes` bytes of `buf` (all of
    it by default) once with the library's streaming-read kernel.  Returns
    the int32 sink [STREAM_READ_BLOCKS]; the XOR of its words is the XOR of
    every 32-bit word read."""
    nbytes = _nbytes(buf) if nbytes is None else nbytes
    _need_bytes("tq_stream_read", "buf", buf, nbytes)
    if sink is not None and sink.dtype != torch.int32:
        raise TiledqError("tq_stream_read: sink must be int32")
    _need_bytes("tq_stream_read", "sink", sink, 4 * STREAM_READ_BLOCKS)
    _need_cuda(buf, sink)
    if sink is None:
        sink = torch.empty(STREAM_READ_BLOCKS, dtype=torch.int32, device=buf.device)
    check(lib().tq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf)), "tq_stream_read")
    return sink

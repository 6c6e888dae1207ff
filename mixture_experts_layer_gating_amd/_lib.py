"""Thin ctypes binding of ``libmoe.so``: one Python function per C symbol,
same names, argument marshalling only.

Tensors are torch tensors on the GPU (or ``None`` where the C argument may be
NULL); they are passed as raw device pointers.  Every call enqueues on
``stream`` (default: torch's current stream of the tensor's device) and
raises :class:`MoEError` with the library's message on a non-zero status.

The library must have been built (``mixture_experts_layer_gating_amd.build``);
importing this module without it raises ``ImportError`` -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_F32 = 0
MOE_BF16 = 1
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 32
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
MOE_IDXERR_EXPERT = 1
MOE_IDXERR_ROW = 2
MOE_IDXERR_GROUP = 4
MOE_IDXERR_GATHER = 8

# Every exported symbol of include/moe.h.
SYMBOLS = (
    "moe_last_error", "moe_version", "moe_index_errors", "moe_route_topk", "moe_route_topk_bwd",
    "moe_count_index_workspace_size", "moe_count_index", "moe_count_index_noalloc",
    "moe_permute",
    "moe_unpermute", "moe_unpermute_bwd", "moe_grouped_gemm_workspace_size",
    "moe_grouped_gemm_plan",
    "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd", "moe_grouped_gemm_swiglu_fwd",
    "moe_grouped_gemm_swiglu_fwd_gather", "moe_grouped_gemm_bwd_gather",
    "moe_act_fwd", "moe_act_bwd", "moe_gather_scale", "moe_grouped_gemm_bwd_scaled_gather",
    "moe_act_bwd_scaled",
)


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"status {status}: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -m mixture_experts_layer_gating_amd.build` (or __graft_entry__.build())")

# PyTorch (ROCm build) ships its own HIP runtime.  Load torch first so that
# libmoe.so's dependency on libamdhip64.so.7 resolves to that already-loaded
# runtime (same SONAME) instead of pulling in a second one, then check that
# exactly one HIP runtime is mapped into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and os.path.basename(parts[5]).startswith("libamdhip64.so"):
                    paths.add(os.path.realpath(parts[5]))
    except OSError:  # pragma: no cover
        pass
    return sorted(paths)


_RUNTIMES = _hip_runtimes()
if len(_RUNTIMES) > 1:
    raise ImportError("two HIP runtimes are loaded into this process "
                      f"({', '.join(_RUNTIMES)}); import torch before loading libmoe.so")

_p = ctypes.c_void_p
_i = ctypes.c_int
_z = ctypes.c_size_t

_SIG = {
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_version": ([], ctypes.c_char_p),
    "moe_index_errors": ([_p, _i, _p], _i),
    "moe_route_topk": ([_p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p], _i),
    "moe_route_topk_bwd": ([_p, _p, _p, _i, _i, _i, _i, _p, _i, _p], _i),
    "moe_count_index_workspace_size": ([_i, _i, _i], _z),
    "moe_count_index": ([_p, _i, _i, _i, _p, _p, _p, _p, _p, _z, _p], _i),
    "moe_count_index_noalloc": ([_p, _i, _i, _i, _p, _p, _p, _p, _p], _i),
    "moe_permute": ([_p, _p, _i, _i, _i, _i, _p, _p], _i),
    "moe_unpermute": ([_p, _p, _p, _i, _i, _i, _i, _p, _p], _i),
    "moe_unpermute_bwd": ([_p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _p], _i),
    "moe_grouped_gemm_workspace_size": ([_i, _i, _i, _i, _i], _z),
    "moe_grouped_gemm_plan": ([_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p], _i),
    "moe_grouped_gemm_fwd": ([_p, _p, _p, _i, _i, _i, _i, _i, _p, _i, _p, _z, _p], _i),
    "moe_grouped_gemm_bwd": ([_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _z, _p], _i),
    "moe_grouped_gemm_swiglu_fwd": ([_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p], _i),
    "moe_grouped_gemm_swiglu_fwd_gather": ([_p, _p, _i, _i, _p, _p, _i, _i, _i, _i, _i, _p, _p,
                                            _p], _i),
    "moe_grouped_gemm_bwd_gather": ([_p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p,
                                     _p, _z, _p], _i),
    "moe_act_fwd": ([_p, _i, _i, _i, _p, _p], _i),
    "moe_act_bwd": ([_p, _p, _i, _i, _i, _p, _p], _i),
    "moe_gather_scale": ([_p, _p, _i, _p, _p], _i),
    "moe_grouped_gemm_bwd_scaled_gather": ([_p, _p, _p, _p, _i, _i, _p, _p, _i, _i, _i, _i, _i,
                                            _p, _p, _p, _z, _p], _i),
    "moe_act_bwd_scaled": ([_p, _p, _p, _i, _i, _i, _p, _p, _p], _i),
}
for _name, (_args, _res) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def lib():
    return _lib


def _ptr(t):
    """Device pointer of a tensor (or raw int pointer / None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    if t.device.type != "cuda":
        raise ValueError("tensors passed to the library must live on the GPU")
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int):
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, _lib.moe_last_error().decode())


def dtype_code(torch_dtype):
    import torch
    if torch_dtype == torch.bfloat16:
        return MOE_BF16
    if torch_dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {torch_dtype}")


def moe_last_error():
    return _lib.moe_last_error().decode()


def moe_version():
    return _lib.moe_version().decode()


def moe_index_errors(clear=True, stream=None):
    """MOE_IDXERR_* bits recorded by the kernels (waits for the stream)."""
    mask = ctypes.c_uint(0)
    _check(_lib.moe_index_errors(ctypes.byref(mask), 1 if clear else 0, _stream(stream)))
    return mask.value


def moe_route_topk(logits, bias, T, E, k, renorm, forced_idx, topk_idx, topk_w, probs,
                   stream=None):
    _check(_lib.moe_route_topk(_ptr(logits), _ptr(bias), T, E, k, int(renorm),
                               _ptr(forced_idx), _ptr(topk_idx), _ptr(topk_w), _ptr(probs),
                               _stream(stream, logits)))


def moe_route_topk_bwd(probs, topk_idx, dtopk_w, T, E, k, renorm, dlogits, dlogits_dtype,
                       stream=None):
    _check(_lib.moe_route_topk_bwd(_ptr(probs), _ptr(topk_idx), _ptr(dtopk_w), T, E, k,
                                   int(renorm), _ptr(dlogits), dlogits_dtype,
                                   _stream(stream, probs)))


def moe_count_index_workspace_size(T, k, E):
    return int(_lib.moe_count_index_workspace_size(T, k, E))


def moe_count_index(topk_idx, T, k, E, counts, offsets, dest, src, ws, ws_bytes, stream=None):
    _check(_lib.moe_count_index(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets),
                                _ptr(dest), _ptr(src), _ptr(ws), ws_bytes,
                                _stream(stream, topk_idx)))


def moe_count_index_noalloc(topk_idx, T, k, E, counts, offsets, dest, src, stream=None):
    _check(_lib.moe_count_index_noalloc(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets),
                                        _ptr(dest), _ptr(src), _stream(stream, topk_idx)))


def moe_permute(x, dest, T, k, d, dtype, xp, stream=None):
    _check(_lib.moe_permute(_ptr(x), _ptr(dest), T, k, d, dtype, _ptr(xp), _stream(stream, x)))


def moe_unpermute(yp, dest, w, T, k, d, dtype, y, stream=None):
    _check(_lib.moe_unpermute(_ptr(yp), _ptr(dest), _ptr(w), T, k, d, dtype, _ptr(y),
                              _stream(stream, yp)))


def moe_unpermute_bwd(dy, yp, dest, w, T, k, d, dtype, dyp, dw, stream=None):
    _check(_lib.moe_unpermute_bwd(_ptr(dy), _ptr(yp), _ptr(dest), _ptr(w), T, k, d, dtype,
                                  _ptr(dyp), _ptr(dw), _stream(stream, dy)))


def moe_grouped_gemm_workspace_size(M, K, N, E, dtype):
    return int(_lib.moe_grouped_gemm_workspace_size(M, K, N, E, dtype))


def moe_grouped_gemm_plan(product, M, K, N, E, dtype):
    """Returns dict(tile_m, tile_n, waves_m, waves_n, split, mfma) chosen for
    this shape."""
    keys = ("tile_m", "tile_n", "waves_m", "waves_n", "split", "mfma")
    vals = [ctypes.c_int() for _ in keys]
    _check(_lib.moe_grouped_gemm_plan(product, M, K, N, E, dtype,
                                      *[ctypes.byref(v) for v in vals]))
    return dict(zip(keys, (v.value for v in vals)))


def moe_grouped_gemm_fwd(a, b, offsets, M, K, N, E, ab_dtype, c, c_dtype, ws=None, ws_bytes=0,
                         stream=None):
    _check(_lib.moe_grouped_gemm_fwd(_ptr(a), _ptr(b), _ptr(offsets), M, K, N, E, ab_dtype,
                                     _ptr(c), c_dtype, _ptr(ws), ws_bytes, _stream(stream, a)))


def moe_grouped_gemm_bwd(a, b, dc, offsets, M, K, N, E, dtype, da, da_add, db, ws=None,
                         ws_bytes=0, stream=None):
    _check(_lib.moe_grouped_gemm_bwd(_ptr(a), _ptr(b), _ptr(dc), _ptr(offsets), M, K, N, E,
                                     dtype, _ptr(da), _ptr(da_add), _ptr(db), _ptr(ws), ws_bytes,
                                     _stream(stream, dc)))


def moe_grouped_gemm_swiglu_fwd(a, b, offsets, M, K, F, E, dtype, h, act, stream=None):
    _check(_lib.moe_grouped_gemm_swiglu_fwd(_ptr(a), _ptr(b), _ptr(offsets), M, K, F, E, dtype,
                                            _ptr(h), _ptr(act), _stream(stream, a)))


def moe_grouped_gemm_swiglu_fwd_gather(x, x_rows, x_div, x_phys, b, offsets, M, K, F, E, dtype,
                                       h, act, stream=None):
    _check(_lib.moe_grouped_gemm_swiglu_fwd_gather(
        _ptr(x), _ptr(x_rows), x_div, x_phys, _ptr(b), _ptr(offsets), M, K, F, E, dtype, _ptr(h),
        _ptr(act), _stream(stream, x)))


def moe_grouped_gemm_bwd_gather(a, a_rows, a_div, a_phys, b, dc, offsets, M, K, N, E, dtype, da,
                                da_add, db, ws=None, ws_bytes=0, stream=None):
    _check(_lib.moe_grouped_gemm_bwd_gather(
        _ptr(a), _ptr(a_rows), a_div, a_phys, _ptr(b), _ptr(dc), _ptr(offsets), M, K, N, E, dtype,
        _ptr(da), _ptr(da_add), _ptr(db), _ptr(ws), ws_bytes, _stream(stream, dc)))


def moe_act_fwd(h, M, F, dtype, a, stream=None):
    _check(_lib.moe_act_fwd(_ptr(h), M, F, dtype, _ptr(a), _stream(stream, h)))


def moe_act_bwd(h, da, M, F, dtype, dh, stream=None):
    _check(_lib.moe_act_bwd(_ptr(h), _ptr(da), M, F, dtype, _ptr(dh), _stream(stream, h)))


def moe_gather_scale(w, src, n, out, stream=None):
    _check(_lib.moe_gather_scale(_ptr(w), _ptr(src), n, _ptr(out), _stream(stream, out)))


def moe_grouped_gemm_bwd_scaled_gather(a_scaled, b, dy, dc_rows, dc_div, dc_phys, row_scale,
                                       offsets, M, K, N, E, dtype, da, db, ws=None, ws_bytes=0,
                                       stream=None):
    _check(_lib.moe_grouped_gemm_bwd_scaled_gather(
        _ptr(a_scaled), _ptr(b), _ptr(dy), _ptr(dc_rows), dc_div, dc_phys, _ptr(row_scale),
        _ptr(offsets), M, K, N, E, dtype, _ptr(da), _ptr(db), _ptr(ws), ws_bytes,
        _stream(stream, dy)))


def moe_act_bwd_scaled(h, da, row_scale, M, F, dtype, dh, a_scaled, stream=None):
    _check(_lib.moe_act_bwd_scaled(_ptr(h), _ptr(da), _ptr(row_scale), M, F, dtype, _ptr(dh),
                                   _ptr(a_scaled), _stream(stream, h)))

"""Thin Python binding of ``libawq_mi355x.so`` (ctypes).

Argument marshalling only: every step of the path runs in the HIP library.
Torch supplies device memory and the current stream.  Importing this module
loads the library and fails loudly if it has not been built; there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "AwqError",
    "AwqNonFinite",
    "lib_path",
    "load",
    "version",
    "act_stats",
    "weight_stats",
    "search_workspace_size",
    "search_workspace_min_size",
    "search_layer",
    "SearchResult",
    "clip_workspace_size",
    "clip_search",
    "ClipResult",
    "pack",
    "w4a16_gemm",
    "w4a16_workspace_size",
    "w4a16_gemm_noalloc",
    "AWQ_F32",
    "AWQ_BF16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libawq_mi355x.so"

AWQ_F32 = 0
AWQ_BF16 = 1
AWQ_F16 = 2                     # stored steps only
AWQ_SEARCH_ZERO_POINT = 1       # awq_search_layer_flags
AWQ_SEARCH_FP16_STEPS = 2
AWQ_SEARCH_MATRIX_BF16 = 4      # loss contraction on bf16 matrix cores (with correction rows)
AWQ_SEARCH_MATRIX_FP16 = 8      # loss contraction on fp16 matrix cores

_STATUS = {
    0: "AWQ_OK",
    -1: "AWQ_ERR_ARG",
    -2: "AWQ_ERR_SHAPE",
    -3: "AWQ_ERR_DTYPE",
    -4: "AWQ_ERR_WORKSPACE",
    -5: "AWQ_ERR_NONFINITE",
    -6: "AWQ_ERR_HIP",
}


class AwqError(RuntimeError):
    """A C-ABI call returned a negative awq_status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class AwqNonFinite(AwqError):
    """The search met a NaN or Inf (best == -1)."""


def lib_path() -> str:
    return os.path.join(_PKG, _LIBNAME)


_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_uint = ctypes.c_uint
_sz = ctypes.c_size_t

SIGNATURES = {
    "awq_last_error": (ctypes.c_char_p, []),
    "awq_version": (ctypes.c_char_p, []),
    "awq_act_stats": (_int, [_vp, _int, _i64, _i64, _vp, _vp]),
    "awq_act_stats_ex": (_int, [_vp, _int, _i64, _i64, _int, _vp, _vp]),
    "awq_weight_stats": (_int, [_vp, _int, _i64, _i64, _vp, _vp]),
    "awq_search_workspace_size": (_sz, [_i64, _i64, _i64, _int, _int, _int, _int]),
    "awq_search_workspace_min_size": (_sz, [_i64, _i64, _i64, _int, _int, _int, _int]),
    "awq_search_status": (_int, [_vp, _vp, _vp]),
    "awq_search_layer": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _int, _int, _int,
                                _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_search_layer_ex": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _int, _int, _int,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _int]),
    "awq_search_layer_wscale": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _vp, _int, _int, _int,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_clip_workspace_size": (_sz, [_i64, _i64, _int]),
    "awq_clip_search": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _int, _int, _int,
                               _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_search_layer_zp": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _vp, _int, _int, _int,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_search_layer_flags": (_int, [_vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _vp, _int, _int, _int,
                                      _uint, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_pack": (_int, [_vp, _i64, _i64, _int, _vp, _vp]),
    "awq_pack_ex": (_int, [_vp, _i64, _i64, _int, _int, _vp, _vp]),
    "awq_w4a16_gemm_zp": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _int, _vp, _vp, _int, _vp, _sz, _vp]),
    "awq_w4a16_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "awq_w4a16_gemm": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _int, _vp, _vp, _int, _vp, _sz, _vp]),
    "awq_w4a16_workspace_size_ex": (_sz, [_i64, _i64, _i64, _int, _int]),
    "awq_w4a16_noalloc_scratch_bytes": (_sz, []),
    "awq_w4a16_gemm_noalloc": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _int, _vp, _vp, _int, _vp]),
    "awq_w4a16_gemm_ex": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _int, _vp, _int, _vp, _vp, _int, _vp, _sz,
                                 _vp]),
}


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it is missing: no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first with "
            "`python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m weight_only_quantization_awq_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def version() -> str:
    return load().awq_version().decode()


def _check(status: int):
    if status != 0:
        msg = load().awq_last_error().decode(errors="replace")
        raise AwqError(status, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return AWQ_F32
    if t == torch.bfloat16:
        return AWQ_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# ---------------------------------------------------------------------------

_STATS = {"mean": 0, "max": 1}


def act_stats(X: torch.Tensor, statistic: str = "mean") -> torch.Tensor:
    """a_j = mean_n |X[n, j]| (or max_n with statistic="max") as float32 [D_in]."""
    lib = load()
    if statistic not in _STATS:
        raise ValueError("statistic must be 'mean' or 'max'")
    N, D_in = X.shape
    a = torch.empty(D_in, dtype=torch.float32, device=X.device)
    _check(lib.awq_act_stats_ex(_dev(X, "X"), _dtype_code(X.dtype), N, D_in, _STATS[statistic], _dev(a, "a"),
                                _stream(X.device)))
    return a


def weight_stats(W: torch.Tensor) -> torch.Tensor:
    """b_j = mean_o |W[j, o]| as float32 [D_in] (W is [D_in, D_out])."""
    lib = load()
    D_in, D_out = W.shape
    b = torch.empty(D_in, dtype=torch.float32, device=W.device)
    _check(lib.awq_weight_stats(_dev(W, "W"), _dtype_code(W.dtype), D_in, D_out, _dev(b, "b"), _stream(W.device)))
    return b


def search_workspace_size(N: int, D_in: int, D_out: int, x_dtype: torch.dtype, bits: int = 4,
                          group: int = 128, n_alpha: int = 21) -> int:
    lib = load()
    n = lib.awq_search_workspace_size(N, D_in, D_out, _dtype_code(x_dtype), bits, group, n_alpha)
    if n == 0:
        raise AwqError(-2, lib.awq_last_error().decode(errors="replace"))
    return int(n)


def search_workspace_min_size(N: int, D_in: int, D_out: int, x_dtype: torch.dtype, bits: int = 4,
                              group: int = 128, n_alpha: int = 21) -> int:
    """The smallest workspace the search accepts (it then runs in column chunks)."""
    lib = load()
    n = lib.awq_search_workspace_min_size(N, D_in, D_out, _dtype_code(x_dtype), bits, group, n_alpha)
    if n == 0:
        raise AwqError(-2, lib.awq_last_error().decode(errors="replace"))
    return int(n)


@dataclass
class SearchResult:
    losses: torch.Tensor   # float64 [n_alpha]
    best: torch.Tensor     # int32 [1] (device)
    s_best: torch.Tensor   # float32 [D_in]
    scales: torch.Tensor   # float32 [D_in/group, D_out]
    codes: torch.Tensor | None  # int8 [D_in, D_out] (uint8 zero-point codes with zero_point=True)
    zeros: torch.Tensor | None = None  # uint8 [D_in/group, D_out] (zero_point=True)

    def best_index(self) -> int:
        """alpha* index, through awq_search_status (waits for the current stream)."""
        lib = load()
        out = ctypes.c_int32(-1)
        st = lib.awq_search_status(_dev(self.best, "best"), _stream(self.best.device), ctypes.byref(out))
        if st == -5:
            raise AwqNonFinite(st, lib.awq_last_error().decode(errors="replace"))
        _check(st)
        return int(out.value)


def default_alphas(n: int = 21) -> np.ndarray:
    return (np.arange(n, dtype=np.float64) / max(n - 1, 1)).astype(np.float32)


SEARCH_EVENTS = 5


def search_layer(X: torch.Tensor, W: torch.Tensor, alphas=None, bits: int = 4, group: int = 128,
                 a: torch.Tensor | None = None, want_codes: bool = True,
                 workspace: torch.Tensor | None = None, events=None,
                 b: torch.Tensor | None = None, zero_point: bool = False,
                 f16_steps: bool = False, matrix: str | None = None) -> SearchResult:
    """Run the alpha grid search for one layer (asynchronous on the current stream).

    ``workspace``: a caller buffer of at least :func:`search_workspace_min_size`
    bytes (below :func:`search_workspace_size` the search runs in column
    chunks, with identical results); None allocates the one-pass size.

    ``events``: optional list of 5 ``torch.cuda.Event(enable_timing=True)``
    recorded at the phase boundaries (see awq_search_layer_ex).
    ``b``: a weight statistic (e.g. :func:`weight_stats`) selects the
    candidates s = a^alpha / b^(1-alpha) (awq_search_layer_wscale; no events).
    ``zero_point``: asymmetric codes in [0, 2^bits - 1] with zero points
    (awq_search_layer_zp; no events).
    ``f16_steps``: steps rounded to and returned in FP16 (``scales`` is
    float16), with either code kind (awq_search_layer_flags; no events).
    ``matrix``: "bf16" or "fp16" picks the loss contraction's matrix cores on
    layers that may take the bf16 path, instead of the size rule
    (awq_search_layer_flags; no events).
    """
    lib = load()
    N, D_in = X.shape
    D_in2, D_out = W.shape
    if D_in2 != D_in:
        raise ValueError("X and W disagree on D_in")
    dev = X.device
    if alphas is None:
        alphas = default_alphas(21)
    al = np.ascontiguousarray(np.asarray(alphas, dtype=np.float32))
    if a is None:
        a = act_stats(X)
    if workspace is None:
        workspace = torch.empty(search_workspace_size(N, D_in, D_out, X.dtype, bits, group, al.size),
                                dtype=torch.uint8, device=dev)
    losses = torch.empty(al.size, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(D_in, dtype=torch.float32, device=dev)
    scales = torch.empty(D_in // group, D_out, dtype=torch.float32, device=dev)
    codes = torch.empty(D_in, D_out, dtype=torch.int8, device=dev) if want_codes else None
    ev_arr, n_ev = None, 0
    if events is not None:
        if len(events) != SEARCH_EVENTS:
            raise ValueError(f"events must hold {SEARCH_EVENTS} torch.cuda.Event objects")
        st = torch.cuda.current_stream(dev)
        for e in events:            # materialise the underlying hipEvent_t handles
            if not e.cuda_event:
                e.record(st)
        ev_arr = (ctypes.c_void_p * SEARCH_EVENTS)(*[e.cuda_event for e in events])
        n_ev = SEARCH_EVENTS
    if matrix not in (None, "bf16", "fp16"):
        raise ValueError(f"matrix must be None, 'bf16' or 'fp16' (got {matrix!r})")
    if f16_steps or matrix is not None:
        if events is not None:
            raise ValueError("phase events are not available with FP16 steps or a chosen matrix format")
        flags = ((AWQ_SEARCH_FP16_STEPS if f16_steps else 0) | (AWQ_SEARCH_ZERO_POINT if zero_point else 0)
                 | {None: 0, "bf16": AWQ_SEARCH_MATRIX_BF16, "fp16": AWQ_SEARCH_MATRIX_FP16}[matrix])
        if f16_steps:
            scales = torch.empty(D_in // group, D_out, dtype=torch.float16, device=dev)
        zeros = torch.empty(D_in // group, D_out, dtype=torch.uint8, device=dev) if zero_point else None
        if zero_point and codes is not None:
            codes = codes.view(torch.uint8)
        _check(lib.awq_search_layer_flags(
            _dev(X, "X"), _dtype_code(X.dtype), N, D_in, _dev(W, "W"), _dtype_code(W.dtype), D_out,
            _dev(a, "a"), _dev(b, "b") if b is not None else None, al.ctypes.data, al.size, bits, group, flags,
            _dev(losses, "losses"), _dev(best, "best"), _dev(s_best, "s_best"), _dev(scales, "scales"),
            _dev(zeros, "zeros") if zeros is not None else None, _dev(codes, "codes") if codes is not None else None,
            _dev(workspace, "workspace"), workspace.numel(), _stream(dev)))
        return SearchResult(losses, best, s_best, scales, codes, zeros)
    if zero_point:
        if events is not None:
            raise ValueError("phase events are not available with zero-point codes")
        zeros = torch.empty(D_in // group, D_out, dtype=torch.uint8, device=dev)
        codes = codes.view(torch.uint8) if codes is not None else None
        _check(lib.awq_search_layer_zp(
            _dev(X, "X"), _dtype_code(X.dtype), N, D_in, _dev(W, "W"), _dtype_code(W.dtype), D_out,
            _dev(a, "a"), _dev(b, "b") if b is not None else None, al.ctypes.data, al.size, bits, group,
            _dev(losses, "losses"), _dev(best, "best"), _dev(s_best, "s_best"), _dev(scales, "scales"),
            _dev(zeros, "zeros"), _dev(codes, "codes") if codes is not None else None,
            _dev(workspace, "workspace"), workspace.numel(), _stream(dev)))
        return SearchResult(losses, best, s_best, scales, codes, zeros)
    if b is not None:
        if events is not None:
            raise ValueError("phase events are not available with a weight statistic")
        _check(lib.awq_search_layer_wscale(
            _dev(X, "X"), _dtype_code(X.dtype), N, D_in, _dev(W, "W"), _dtype_code(W.dtype), D_out,
            _dev(a, "a"), _dev(b, "b"), al.ctypes.data, al.size, bits, group,
            _dev(losses, "losses"), _dev(best, "best"), _dev(s_best, "s_best"), _dev(scales, "scales"),
            _dev(codes, "codes") if codes is not None else None,
            _dev(workspace, "workspace"), workspace.numel(), _stream(dev)))
        return SearchResult(losses, best, s_best, scales, codes)
    _check(lib.awq_search_layer_ex(
        _dev(X, "X"), _dtype_code(X.dtype), N, D_in, _dev(W, "W"), _dtype_code(W.dtype), D_out,
        _dev(a, "a"), al.ctypes.data, al.size, bits, group,
        _dev(losses, "losses"), _dev(best, "best"), _dev(s_best, "s_best"), _dev(scales, "scales"),
        _dev(codes, "codes") if codes is not None else None,
        _dev(workspace, "workspace"), workspace.numel(), _stream(dev),
        ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None, n_ev))
    return SearchResult(losses, best, s_best, scales, codes)


def clip_workspace_size(N: int, D_in: int, group: int = 128) -> int:
    lib = load()
    n = lib.awq_clip_workspace_size(N, D_in, group)
    if n == 0:
        raise AwqError(-1, lib.awq_last_error().decode(errors="replace"))
    return int(n)


@dataclass
class ClipResult:
    ratio_idx: torch.Tensor          # int32 [D_in/group, D_out]
    scales: torch.Tensor             # float32 [D_in/group, D_out]
    codes: torch.Tensor | None       # int8 [D_in, D_out]
    errors: torch.Tensor | None      # float32 [n_ratio, D_in/group, D_out]


def default_clip_ratios(n: int = 11, lowest: float = 0.5) -> np.ndarray:
    """1, ..., lowest in n equal steps (1 = no clipping)."""
    return np.linspace(1.0, lowest, n).astype(np.float32)


def clip_search(X: torch.Tensor, W: torch.Tensor, s: torch.Tensor, ratios=None, bits: int = 4,
                group: int = 128, want_codes: bool = True, want_errors: bool = False,
                workspace: torch.Tensor | None = None) -> ClipResult:
    """Per-group weight-clipping search with fixed scales s (asynchronous on the current stream)."""
    lib = load()
    N, D_in = X.shape
    D_in2, D_out = W.shape
    if D_in2 != D_in:
        raise ValueError("X and W disagree on D_in")
    dev = X.device
    r = np.ascontiguousarray(np.asarray(default_clip_ratios() if ratios is None else ratios, dtype=np.float32))
    need = clip_workspace_size(N, D_in, group)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    G = D_in // group
    ratio_idx = torch.empty(G, D_out, dtype=torch.int32, device=dev)
    scales = torch.empty(G, D_out, dtype=torch.float32, device=dev)
    codes = torch.empty(D_in, D_out, dtype=torch.int8, device=dev) if want_codes else None
    errors = torch.empty(r.size, G, D_out, dtype=torch.float32, device=dev) if want_errors else None
    _check(lib.awq_clip_search(
        _dev(X, "X"), _dtype_code(X.dtype), N, D_in, _dev(W, "W"), _dtype_code(W.dtype), D_out,
        _dev(s, "s"), r.ctypes.data, r.size, bits, group,
        _dev(ratio_idx, "ratio_idx"), _dev(scales, "scales"),
        _dev(codes, "codes") if codes is not None else None,
        _dev(errors, "errors") if errors is not None else None,
        _dev(workspace, "workspace"), workspace.numel(), _stream(dev)))
    return ClipResult(ratio_idx, scales, codes, errors)


def pack(codes: torch.Tensor, bits: int = 4) -> torch.Tensor:
    """Codes [D_in, D_out] -> uint32 words [D_in/8, D_out] (stored as int32).

    int8 codes are signed (nibble = q + 8); uint8 codes are the zero-point
    codes of ``search_layer(..., zero_point=True)`` (nibble = q).
    """
    lib = load()
    if codes.dtype not in (torch.int8, torch.uint8):
        raise TypeError("codes must be int8 (signed) or uint8 (zero-point codes)")
    D_in, D_out = codes.shape
    packed = torch.empty(D_in // 8, D_out, dtype=torch.int32, device=codes.device)
    _check(lib.awq_pack_ex(_dev(codes, "codes"), D_in, D_out, bits, 1 if codes.dtype == torch.uint8 else 0,
                           _dev(packed, "packed"), _stream(codes.device)))
    return packed


def w4a16_workspace_size(M: int, D_in: int, D_out: int, has_inv_s: bool) -> int:
    return int(load().awq_w4a16_workspace_size(M, D_in, D_out, 1 if has_inv_s else 0))


def w4a16_gemm(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, group: int = 128,
               inv_s: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               zeros: torch.Tensor | None = None) -> torch.Tensor:
    """Y = (X·diag(inv_s))·Dequant(packed, scales[, zeros]); X bf16 [M, D_in].

    ``scales`` float32, or float16 (FP16 steps: awq_w4a16_gemm_ex).
    """
    lib = load()
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    M, D_in = X.shape
    D_out = packed.shape[1]
    if packed.shape[0] * 8 != D_in:
        raise ValueError("packed rows must be D_in/8")
    if out is None:
        out = torch.empty(M, D_out, dtype=out_dtype, device=X.device)
    if scales.dtype == torch.float16:
        need = int(lib.awq_w4a16_workspace_size_ex(M, D_in, D_out, group, AWQ_F16))
        if need == 0:
            raise AwqError(-1, lib.awq_last_error().decode(errors="replace"))
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        _check(lib.awq_w4a16_gemm_ex(
            _dev(X, "X"), M, D_in, D_out, _dev(packed, "packed"), _dev(scales, "scales"), AWQ_F16,
            _dev(zeros, "zeros") if zeros is not None else None, group,
            _dev(inv_s, "inv_s") if inv_s is not None else None, _dev(out, "Y"), _dtype_code(out.dtype),
            _dev(workspace, "workspace"), workspace.numel(), _stream(X.device)))
        return out
    need = w4a16_workspace_size(M, D_in, D_out, inv_s is not None)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    if zeros is not None:
        _check(lib.awq_w4a16_gemm_zp(
            _dev(X, "X"), M, D_in, D_out, _dev(packed, "packed"), _dev(scales, "scales"), _dev(zeros, "zeros"),
            group, _dev(inv_s, "inv_s") if inv_s is not None else None,
            _dev(out, "Y"), _dtype_code(out.dtype),
            _dev(workspace, "workspace") if need else None, workspace.numel() if need else 0,
            _stream(X.device)))
        return out
    _check(lib.awq_w4a16_gemm(
        _dev(X, "X"), M, D_in, D_out, _dev(packed, "packed"), _dev(scales, "scales"), group,
        _dev(inv_s, "inv_s") if inv_s is not None else None,
        _dev(out, "Y"), _dtype_code(out.dtype),
        _dev(workspace, "workspace") if need else None, workspace.numel() if need else 0,
        _stream(X.device)))
    return out


def w4a16_gemm_noalloc(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, group: int = 128,
                       inv_s: torch.Tensor | None = None, out: torch.Tensor | None = None,
                       out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """awq_w4a16_gemm_noalloc: the W4A16 product on the library's static scratch
    (no workspace; float32 steps, signed codes).  Pass ``out`` to allocate
    nothing at all; calls that overlap on one GPU race on the scratch."""
    lib = load()
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    M, D_in = X.shape
    D_out = packed.shape[1]
    if out is None:
        out = torch.empty(M, D_out, dtype=out_dtype, device=X.device)
    _check(lib.awq_w4a16_gemm_noalloc(
        _dev(X, "X"), M, D_in, D_out, _dev(packed, "packed"), _dev(scales, "scales"), group,
        _dev(inv_s, "inv_s") if inv_s is not None else None, _dev(out, "Y"), _dtype_code(out.dtype),
        _stream(X.device)))
    return out


# Load at import time: a missing library is an error, never a silent fallback.
load()

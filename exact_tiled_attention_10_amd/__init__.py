"""Exact tiled attention (FlashAttention forward and backward) on MI355X.

A thin ctypes binding over ``libfa.so``, the C ABI declared in
``include/fa.h``.  Every step of the computation runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with torch
and passes raw device pointers and the current HIP stream.  There is no CPU
fallback: if the library is missing, every call raises.

Low-level entry points carry the C names (``fa_fwd``, ``fa_fwd_gqa``,
``fa_fwd_kv``, ``fa_fwd_kv_workspace_size``, ``fa_fwd_f32``, ``fa_bwd``,
``fa_bwd_gqa``, ``fa_bwd_kv``, ``fa_bwd_workspace_size``, ``fa_bwd_kv_workspace_size``,
``fa_status_string``) and take
preallocated tensors;
``forward``/``backward``/``attention`` allocate, and take key / value tensors
with fewer heads than the queries (grouped-query attention) when the dtype is
bf16.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "FAError", "library_path", "load_library",
    "fa_fwd", "fa_fwd_gqa", "fa_fwd_kv", "fa_fwd_kv_workspace_size", "fa_fwd_fp8",
    "fa_fwd_f32",
    "fa_bwd", "fa_bwd_gqa", "fa_bwd_kv", "fa_bwd_workspace_size", "fa_bwd_kv_workspace_size",
    "fa_status_string",
    "fa_bwd_preprocess", "fa_bwd_main", "fa_bwd_finalize", "fa_bwd_noalloc",
    "FA_STATIC_SCRATCH_BYTES",
    "forward", "backward", "attention",
    "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_HEADDIM", "FA_ERR_ALIGN",
    "FA_ERR_ALIAS", "FA_ERR_SCALE", "FA_ERR_HIP", "FA_ERR_WORKSPACE", "FA_ERR_SCRATCH",
    "FA_MAX_N",
]

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_ALIGN = 4
FA_ERR_ALIAS = 5
FA_ERR_SCALE = 6
FA_ERR_HIP = 7
FA_ERR_WORKSPACE = 8
FA_ERR_SCRATCH = 9
FA_MAX_N = 1 << 22
FA_STATIC_SCRATCH_BYTES = 64 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FAError(RuntimeError):
    """A nonzero status returned by libfa.so."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({fa_status_string(status)})")


def library_path() -> str:
    """The in-tree libfa.so, or the library named by the FA_LIBRARY
    environment variable (e.g. the host-only sanitizer build of the C ABI)."""
    return os.environ.get("FA_LIBRARY") or os.path.join(_PKG, "libfa.so")


def load_library():
    """Load libfa.so (built in-tree by ``build.py``); raise if it is absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_tiled_attention_10_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_gqa.restype = i
    lib.fa_fwd_kv_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_kv_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_kv.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, i, i, f,
                              vp]
    lib.fa_fwd_kv.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, f, f, f, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd_f32.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_kv_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_kv_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                           i, i, i, i, i, f, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                               i, i, i, i, i, i, f, vp]
    lib.fa_bwd_gqa.restype = i
    lib.fa_bwd_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                              i, i, i, i, i, i, i, f, vp]
    lib.fa_bwd_kv.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, vp]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_main.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                i, i, i, i, i, f, vp]
    lib.fa_bwd_main.restype = i
    lib.fa_bwd_finalize.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, f,
                                    vp]
    lib.fa_bwd_finalize.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() or None


def _stream_handle(device: torch.device, stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _dims(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError(f"expected a [B, H, N, d] tensor, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device} != {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _default_scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _raise(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


# ---------------------------------------------------------------------------
# low-level entry points (preallocated outputs), same names as the C ABI
# ---------------------------------------------------------------------------

def fa_fwd(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """bf16 forward into preallocated ``o`` [B,H,N,d] bf16 and ``lse`` [B,H,N] f32."""
    B, H, N, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, N), torch.float32, q.device)
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                               int(bool(causal)), float(scale),
                               _stream_handle(q.device, stream))
    _raise(st, "fa_fwd")


def _kv_heads(q, k) -> int:
    """Key / value head count of ``k`` against ``q`` [B, H, N, d]."""
    B, H, N, d = _dims(q)
    kd = _dims(k)
    if kd[0] != B or kd[2:] != (N, d):
        raise ValueError(f"k: shape {kd} does not match q {(B, H, N, d)} in B, N or d")
    Hkv = kd[1]
    if Hkv < 1 or Hkv > H or H % Hkv:
        raise ValueError(f"query heads {H} are not a multiple of key/value heads {Hkv}")
    return Hkv


def fa_fwd_gqa(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """bf16 forward with grouped-query attention: q, o [B,H,N,d]; k, v [B,Hkv,N,d]."""
    B, H, N, d = _dims(q)
    Hkv = _kv_heads(q, k) if H else k.shape[1]
    for t, nm in ((q, "q"), (o, "o")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, q.device)
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, nm, (B, Hkv, N, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, N), torch.float32, q.device)
    st = load_library().fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv,
                                   N, d, int(bool(causal)), float(scale),
                                   _stream_handle(q.device, stream))
    _raise(st, "fa_fwd_gqa")


def fa_fwd_kv_workspace_size(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load_library().fa_fwd_kv_workspace_size(B, H, Hkv, Nq, Nk, d))


def fa_fwd_kv(q, k, v, o, lse, workspace, causal: bool, scale: float, stream=None) -> None:
    """bf16 forward of Nq queries against Nk keys (bottom-right causal):
    q, o [B,H,Nq,d]; k, v [B,Hkv,Nk,d]; lse [B,H,Nq]; ``workspace`` a uint8
    device tensor of at least ``fa_fwd_kv_workspace_size`` bytes (or None when
    that is 0)."""
    B, H, Nq, d = _dims(q)
    kd = _dims(k)
    Hkv, Nk = kd[1], kd[2]
    if kd[0] != B or kd[3] != d:
        raise ValueError(f"k: shape {kd} does not match q {(B, H, Nq, d)} in B or d")
    if H and (Hkv < 1 or Hkv > H or H % Hkv):
        raise ValueError(f"query heads {H} are not a multiple of key/value heads {Hkv}")
    for t, nm in ((q, "q"), (o, "o")):
        _check(t, nm, (B, H, Nq, d), torch.bfloat16, q.device)
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, nm, (B, Hkv, Nk, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, Nq), torch.float32, q.device)
    nbytes = 0 if workspace is None else _ws_bytes(workspace, q.device)
    st = load_library().fa_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _ptr(workspace), nbytes, B, H, Hkv, Nq, Nk, d,
                                  int(bool(causal)), float(scale),
                                  _stream_handle(q.device, stream))
    _raise(st, "fa_fwd_kv")


def fa_fwd_fp8(q8, k8, v8, o, lse, q_scale: float, k_scale: float, v_scale: float,
               causal: bool, scale: float, stream=None) -> None:
    """Forward on e4m3 inputs: ``q8``, ``k8``, ``v8`` [B,H,N,128] uint8 byte
    codes (or torch.float8_e4m3fn) standing for q_scale * q8 etc.; ``o``
    [B,H,N,128] bf16 and ``lse`` [B,H,N] f32 outputs."""
    B, H, N, d = _dims(q8)
    for t, nm in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{nm}: dtype {t.dtype} is not an e4m3 byte tensor")
        _check(t, nm, (B, H, N, d), t.dtype, q8.device)
    _check(o, "o", (B, H, N, d), torch.bfloat16, q8.device)
    _check(lse, "lse", (B, H, N), torch.float32, q8.device)
    st = load_library().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse),
                                   float(q_scale), float(k_scale), float(v_scale), B, H, N, d,
                                   int(bool(causal)), float(scale),
                                   _stream_handle(q8.device, stream))
    _raise(st, "fa_fwd_fp8")


def fa_fwd_f32(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """fp32 forward into preallocated ``o`` [B,H,N,d] f32 and ``lse`` [B,H,N] f32."""
    B, H, N, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, nm, (B, H, N, d), torch.float32, q.device)
    _check(lse, "lse", (B, H, N), torch.float32, q.device)
    st = load_library().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                   int(bool(causal)), float(scale),
                                   _stream_handle(q.device, stream))
    _raise(st, "fa_fwd_f32")


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d))


def fa_bwd_kv_workspace_size(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load_library().fa_bwd_kv_workspace_size(B, H, Hkv, Nq, Nk, d))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
           stream=None) -> None:
    """bf16 backward into preallocated ``dq``, ``dk``, ``dv``; ``workspace`` is a
    uint8 device tensor of at least ``fa_bwd_workspace_size`` bytes."""
    B, H, N, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"),
                  (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, N), torch.float32, q.device)
    nbytes = _ws_bytes(workspace, q.device)
    st = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                               B, H, N, d, int(bool(causal)), float(scale),
                               _stream_handle(q.device, stream))
    _raise(st, "fa_bwd")


def fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
               stream=None) -> None:
    """bf16 backward with grouped-query attention: q, o, dout, dq [B,H,N,d];
    k, v, dk, dv [B,Hkv,N,d]; dk and dv sum over the query heads of a group."""
    B, H, N, d = _dims(q)
    Hkv = _kv_heads(q, k) if H else k.shape[1]
    for t, nm in ((q, "q"), (o, "o"), (dout, "dout"), (dq, "dq")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, q.device)
    for t, nm in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, Hkv, N, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, N), torch.float32, q.device)
    nbytes = _ws_bytes(workspace, q.device)
    st = load_library().fa_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                                   B, H, Hkv, N, d, int(bool(causal)), float(scale),
                                   _stream_handle(q.device, stream))
    _raise(st, "fa_bwd_gqa")


def fa_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool, scale: float,
              stream=None) -> None:
    """bf16 backward of ``fa_fwd_kv``: q, o, dout, dq [B,H,Nq,d]; k, v, dk, dv
    [B,Hkv,Nk,d]; ``workspace`` of at least ``fa_bwd_workspace_size(B, H, Nq, d)``."""
    B, H, Nq, d = _dims(q)
    kd = _dims(k)
    Hkv, Nk = kd[1], kd[2]
    if kd[0] != B or kd[3] != d:
        raise ValueError(f"k: shape {kd} does not match q {(B, H, Nq, d)} in B or d")
    if H and (Hkv < 1 or Hkv > H or H % Hkv):
        raise ValueError(f"query heads {H} are not a multiple of key/value heads {Hkv}")
    for t, nm in ((q, "q"), (o, "o"), (dout, "dout"), (dq, "dq")):
        _check(t, nm, (B, H, Nq, d), torch.bfloat16, q.device)
    for t, nm in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, Hkv, Nk, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, Nq), torch.float32, q.device)
    nbytes = _ws_bytes(workspace, q.device)
    st = load_library().fa_bwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                                  B, H, Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                  _stream_handle(q.device, stream))
    _raise(st, "fa_bwd_kv")


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool, scale: float,
                   stream=None) -> None:
    """bf16 backward into preallocated ``dq``, ``dk``, ``dv`` with no workspace
    argument: the library's static per-GPU scratch (FA_STATIC_SCRATCH_BYTES)
    stands in for it, so the call allocates nothing.  Calls that overlap on
    one GPU race on that buffer."""
    B, H, N, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"),
                  (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, q.device)
    _check(lse, "lse", (B, H, N), torch.float32, q.device)
    st = load_library().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                       _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                       int(bool(causal)), float(scale),
                                       _stream_handle(q.device, stream))
    _raise(st, "fa_bwd_noalloc")


def _ws_bytes(workspace, device):
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on q's device")
    return workspace.numel() * workspace.element_size()


def fa_bwd_preprocess(o, dout, lse, workspace, stream=None) -> None:
    """Backward stage 1: lse*log2(e), D = rowsum(dO * O) (and at d = 64 a
    zeroed dQ accumulator)."""
    B, H, N, d = _dims(o)
    for t, nm in ((o, "o"), (dout, "dout")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, o.device)
    _check(lse, "lse", (B, H, N), torch.float32, o.device)
    st = load_library().fa_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(lse), _ptr(workspace),
                                          _ws_bytes(workspace, o.device), B, H, N, d,
                                          _stream_handle(o.device, stream))
    _raise(st, "fa_bwd_preprocess")


def fa_bwd_main(q, k, v, dout, dk, dv, workspace, causal: bool, scale: float,
                stream=None) -> None:
    """Backward stage 2: the key-tile kernel (dK, dV; at d = 64 also the dQ
    accumulation)."""
    B, H, N, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, (B, H, N, d), torch.bfloat16, q.device)
    st = load_library().fa_bwd_main(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                    _ptr(dk), _ptr(dv), _ptr(workspace),
                                    _ws_bytes(workspace, q.device), B, H, N, d,
                                    int(bool(causal)), float(scale),
                                    _stream_handle(q.device, stream))
    _raise(st, "fa_bwd_main")


def fa_bwd_finalize(dq, workspace, q=None, k=None, v=None, dout=None, causal: bool = False,
                    scale: float = 1.0, stream=None) -> None:
    """Backward stage 3: dQ.  d = 64: dQ = bf16(accumulator) (q, k, v, dout
    unused); d = 128, 256: the query-tile dQ kernel, which needs q, k, v,
    dout, causal and scale as given to the other stages."""
    B, H, N, d = _dims(dq)
    _check(dq, "dq", (B, H, N, d), torch.bfloat16, dq.device)
    if d != 64:
        for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
            if t is None:
                raise ValueError(f"{nm} is needed by the d = {d} dQ stage")
            _check(t, nm, (B, H, N, d), torch.bfloat16, dq.device)
    st = load_library().fa_bwd_finalize(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                                        _ptr(workspace), _ws_bytes(workspace, dq.device),
                                        B, H, N, d, int(bool(causal)), float(scale),
                                        _stream_handle(dq.device, stream))
    _raise(st, "fa_bwd_finalize")


# ---------------------------------------------------------------------------
# allocating wrappers
# ---------------------------------------------------------------------------

def forward(q, k, v, causal: bool = False, scale: Optional[float] = None,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O, lse = exact attention of [B,H,N,d] bf16 or fp32 tensors on the GPU.

    bf16 ``k`` and ``v`` may have fewer heads than ``q`` (grouped-query
    attention, H a multiple of their head count) and another length than the
    queries (the queries are then the last positions: bottom-right causal)."""
    B, H, N, d = _dims(q)
    s = _default_scale(d, scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if q.dtype != torch.float32 and k.dim() == 4 and k.shape[2] != N:
        nb = fa_fwd_kv_workspace_size(B, H, k.shape[1], N, k.shape[2], d)
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
        fa_fwd_kv(q, k, v, o, lse, ws, causal, s, stream)
    elif q.dtype == torch.float32:
        fa_fwd_f32(q, k, v, o, lse, causal, s, stream)
    elif k.dim() == 4 and k.shape[1] != H:
        fa_fwd_gqa(q, k, v, o, lse, causal, s, stream)
    else:
        fa_fwd(q, k, v, o, lse, causal, s, stream)
    return o, lse


def backward(q, k, v, o, lse, do, causal: bool = False, scale: Optional[float] = None,
             stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV for bf16 tensors, recomputing P from ``lse``."""
    B, H, N, d = _dims(q)
    s = _default_scale(d, scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty(max(1, fa_bwd_kv_workspace_size(B, H, k.shape[1], N, k.shape[2], d)),
                     dtype=torch.uint8, device=q.device)
    if k.dim() == 4 and k.shape[2] != N:
        fa_bwd_kv(q, k, v, o, do, lse, dq, dk, dv, ws, causal, s, stream)
    elif k.dim() == 4 and k.shape[1] != H:
        fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, causal, s, stream)
    else:
        fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal, s, stream)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = forward(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.causal, ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """Differentiable exact attention (bf16): O = softmax(scale Q K^T) V."""
    return _Attention.apply(q, k, v, causal, scale)

"""Python binding for libqgemv (include/qgemv.h): argument marshalling only.

Every computation runs in libqgemv.so (HIP kernels for gfx950, and the C++
host packer). This module only converts Python arguments into pointers and
sizes, picks the current torch stream, and turns error codes into
exceptions. There is no fallback: if the library is not built, importing
anything that needs it raises.

PyTorch is used for device memory and streams only; torch is imported before
the library is loaded so that both share torch's HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

FORMATS = {"int4": 1, "int5": 2, "int8": 3, "nvfp4": 4, "mxfp4": 5, "mxfp8": 6}
STATUS = {0: "OK", -1: "EINVAL", -2: "EFORMAT", -3: "EALIGN", -4: "ERANGE", -5: "EWORKSPACE",
          -6: "EHIP", -7: "EUNSUPPORTED"}
# QGEMV_LIB names another build of the same library (the host-sanitizer test
# loads an address/undefined-behaviour instrumented host build this way)
LIB_PATH = os.environ.get("QGEMV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemv.so")

_lib = None


class Fusion(ctypes.Structure):
    """qgemv_fusion (include/qgemv.h): RMSNorm prologue, bf16 output, flags
    and the split-remainder workspace."""
    _fields_ = [("norm_src", ctypes.c_void_p), ("norm_gamma", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("out_bf16", ctypes.c_void_p), ("flags", ctypes.c_int), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


BATCH_INVARIANT = 1


class QgemvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({strerror(status) if _lib else status})")


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def load(require_torch: bool = True):
    """Load libqgemv.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if require_torch:
        import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_weight_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "qgemv_strerror": (ctypes.c_char_p, [I32]),
        "qgemv_version": (I32, []),
        "qgemv_packed_bytes": (I32, [I32, I64, I64, PSZ, PSZ]),
        "qgemv_expert_stride": (I32, [I32, I64, I64, PSZ, PSZ]),
        "qgemv_pack": (I32, [I32, P, I64, I64, P, P]),
        "qgemv_pack_codes": (I32, [I32, P, P, P, ctypes.c_float, I64, I64, P, P]),
        "qgemv": (I32, [I32, P, P, P, P, P, I64, I64, I32, P]),
        "qgemv_swiglu": (I32, [I32, P, P, P, P, I64, I64, I32, P]),
        "qgemv_ex": (I32, [I32, P, P, P, P, P, I64, I64, I32, ctypes.POINTER(Fusion), P]),
        "qgemv_swiglu_ex": (I32, [I32, P, P, P, P, I64, I64, I32, ctypes.POINTER(Fusion), P]),
        "qgemv_split_workspace_bytes": (I32, [PSZ]),
        "qgemv_moe_workspace_bytes": (I32, [I32, I64, I64, I32, I32, PSZ]),
        "qgemv_moe": (I32, [I32, P, P, P, P, I32, I64, I64, P, P, P, I32, P, P, I32, P, SZ, P]),
        "qgemv_moe_noalloc": (I32, [I32, P, P, P, P, I32, I64, I64, P, P, P, I32, P, P, I32, P]),
        "qgemv_moe_noalloc_max_bytes": (I32, [PSZ]),
        "qgemv_moe_index": (I32, [P, I32, I32, I32, P, P, P, P, P, P]),
        "qgemv_moe_index_by": (I32, [I32, P, I32, I32, I32, P, P, P, P, P, P]),
        "qgemv_moe_route": (I32, [P, I32, I32, I32, P, P, P]),
        "qgemv_moe_fused_workspace_bytes": (I32, [I32, I64, I64, I32, I32, PSZ]),
        "qgemv_moe_fused": (I32, [I32, P, P, P, P, I32, I64, I64, P, P, I32, P, P, I32, P, P, P, SZ, P]),
        "qgemv_dequant": (I32, [I32, P, P, I64, I64, P, P]),
        "qgemv_probe_read": (I32, [P, SZ, P, P]),
        "qgemv_act_quant": (I32, [P, I32, I64, P, P, P]),
        "qgemv_mx": (I32, [I32, P, P, P, P, P, P, I64, I64, I32, P]),
        "qgemv_mx_swiglu": (I32, [I32, P, P, P, P, P, I64, I64, I32, P]),
        "qgemv_mx_swiglu_quant": (I32, [I32, P, P, P, P, P, P, P, I64, I64, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def symbols() -> list[str]:
    """Names of the entry points the binding declares (the C ABI)."""
    return ["qgemv_strerror", "qgemv_version", "qgemv_packed_bytes", "qgemv_expert_stride", "qgemv_pack",
            "qgemv_pack_codes", "qgemv", "qgemv_swiglu", "qgemv_ex", "qgemv_swiglu_ex", "qgemv_split_workspace_bytes",
            "qgemv_moe_workspace_bytes", "qgemv_moe", "qgemv_moe_noalloc", "qgemv_moe_noalloc_max_bytes",
            "qgemv_moe_index", "qgemv_moe_index_by", "qgemv_moe_route", "qgemv_moe_fused_workspace_bytes", "qgemv_moe_fused",
            "qgemv_dequant", "qgemv_probe_read", "qgemv_act_quant", "qgemv_mx", "qgemv_mx_swiglu",
            "qgemv_mx_swiglu_quant"]


def strerror(status: int) -> str:
    return load(False).qgemv_strerror(int(status)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise QgemvError(rc, what)


def _ptr(t):
    """Device or host pointer of a torch tensor / numpy array / int / None."""
    if t is None:
        return None
    dp = getattr(t, "data_ptr", None)   # torch tensors (the common case) first
    if dp is not None:
        return dp()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    if isinstance(t, int):
        return t
    raise TypeError(f"expected a torch tensor, numpy array, int or None, got {type(t).__name__}")


_raw_stream = None


def _stream(stream):
    """HIP stream handle: an int as given, a torch stream's handle, or (None)
    torch's current stream on the current device."""
    global _raw_stream
    if stream is None:
        if _raw_stream is None:
            import torch
            get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            _raw_stream = ((lambda: get(torch.cuda.current_device())) if get is not None
                           else (lambda: torch.cuda.current_stream().cuda_stream))
        return _raw_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ host ---

def packed_bytes(fmt, M: int, K: int) -> tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load(False).qgemv_packed_bytes(_fmt(fmt), M, K, ctypes.byref(a), ctypes.byref(b)), "qgemv_packed_bytes")
    return a.value, b.value


def expert_stride(fmt, M: int, K: int) -> tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load(False).qgemv_expert_stride(_fmt(fmt), M, K, ctypes.byref(a), ctypes.byref(b)), "qgemv_expert_stride")
    return a.value, b.value


def pack(fmt, W: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise and pack a host fp32 [M][K] matrix -> (wq, ws) uint8 arrays."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, K = W.shape
    nq, ns = packed_bytes(fmt, M, K)
    wq = np.empty(nq, np.uint8)
    ws = np.empty(ns, np.uint8)
    _check(load(False).qgemv_pack(_fmt(fmt), _ptr(W), M, K, _ptr(wq), _ptr(ws)), "qgemv_pack")
    return wq, ws


def pack_codes(fmt, codes: np.ndarray, scales: np.ndarray, mins: np.ndarray | None = None,
               tensor_scale: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    f = _fmt(fmt)
    codes = np.ascontiguousarray(codes, dtype=np.int8 if f == 3 else np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8 if f in (4, 5, 6) else np.uint16)
    mins = None if mins is None else np.ascontiguousarray(mins, dtype=np.uint16)
    M, K = codes.shape
    nq, ns = packed_bytes(f, M, K)
    wq = np.empty(nq, np.uint8)
    ws = np.empty(ns, np.uint8)
    _check(load(False).qgemv_pack_codes(f, _ptr(codes), _ptr(scales), _ptr(mins), float(tensor_scale), M, K,
                                        _ptr(wq), _ptr(ws)), "qgemv_pack_codes")
    return wq, ws


# ---------------------------------------------------------------- device ---

def qgemv(fmt, wq, ws, x, y, M: int, K: int, N: int, residual=None, stream=None) -> None:
    _check(load().qgemv(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(x), _ptr(residual), _ptr(y), M, K, N,
                        _stream(stream)), "qgemv")


def qgemv_swiglu(fmt, wq, ws, x, h, I: int, K: int, N: int, stream=None) -> None:
    _check(load().qgemv_swiglu(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(x), _ptr(h), I, K, N, _stream(stream)),
           "qgemv_swiglu")


_fusion_cache: dict = {}


def _fusion(norm_src, norm_gamma, norm_eps, out_bf16, batch_invariant=False, workspace=None):
    """A qgemv_fusion for these arguments (None when all are defaults). The
    struct is only read during the call; equal argument sets share one
    cached object."""
    if norm_src is None and out_bf16 is None and not batch_invariant and workspace is None:
        return None
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    key = (_ptr(norm_src), _ptr(norm_gamma), float(norm_eps), _ptr(out_bf16),
           BATCH_INVARIANT if batch_invariant else 0, _ptr(workspace), wbytes)
    ref = _fusion_cache.get(key)
    if ref is None:
        if len(_fusion_cache) >= 256:
            _fusion_cache.clear()
        ref = _fusion_cache[key] = ctypes.byref(Fusion(*key))
    return ref


def split_workspace_bytes() -> int:
    """Bytes of the split-remainder workspace on the current device."""
    b = ctypes.c_size_t(0)
    _check(load().qgemv_split_workspace_bytes(ctypes.byref(b)), "qgemv_split_workspace_bytes")
    return b.value


def split_workspace(device):
    """A zero-filled split-remainder workspace (uint8 tensor) for qgemv_ex /
    qgemv_swiglu_ex on `device`. Calls that may overlap in time need their
    own; word 0 (int32) turns nonzero if a wait ever timed out."""
    import torch
    with torch.cuda.device(device):
        n = split_workspace_bytes()
    return torch.zeros(n, dtype=torch.uint8, device=device)


def check_split_workspace(workspace) -> None:
    """Synchronise and raise if a wait of a call that used `workspace` (from
    split_workspace) ever timed out: that call's results, and the workspace
    itself, are then invalid until it is zeroed again."""
    import torch
    torch.cuda.synchronize(workspace.device)
    if int(workspace[:4].view(torch.int32).item()) != 0:
        raise RuntimeError("split-remainder wait timed out: results invalid; zero the workspace before reuse")


def check_moe_fused_workspace(workspace) -> None:
    """As check_split_workspace, for a qgemv_moe_fused workspace (byte 12)."""
    import torch
    torch.cuda.synchronize(workspace.device)
    if int(workspace[12:16].view(torch.int32).item()) != 0:
        raise RuntimeError("qgemv_moe_fused dependency wait timed out: results invalid; clear bytes 12-15")


def qgemv_ex(fmt, wq, ws, x, y, M: int, K: int, N: int, residual=None, norm_src=None, norm_gamma=None,
             norm_eps: float = 1e-6, out_bf16=None, batch_invariant=False, workspace=None, stream=None) -> None:
    """qgemv with the optional RMSNorm prologue (norm_src, norm_gamma,
    norm_eps; x may be None then), bf16 output copy (out_bf16; y may be None
    then), batch-invariant summation order and split-remainder workspace
    (a tensor from split_workspace)."""
    _check(load().qgemv_ex(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(x), _ptr(residual), _ptr(y), M, K, N,
                           _fusion(norm_src, norm_gamma, norm_eps, out_bf16, batch_invariant, workspace),
                           _stream(stream)), "qgemv_ex")


def qgemv_swiglu_ex(fmt, wq, ws, x, h, I: int, K: int, N: int, norm_src=None, norm_gamma=None,
                    norm_eps: float = 1e-6, out_bf16=None, batch_invariant=False, workspace=None,
                    stream=None) -> None:
    _check(load().qgemv_swiglu_ex(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(x), _ptr(h), I, K, N,
                                  _fusion(norm_src, norm_gamma, norm_eps, out_bf16, batch_invariant, workspace),
                                  _stream(stream)), "qgemv_swiglu_ex")


def moe_workspace_bytes(E: int, H: int, I: int, N: int, top_k: int) -> int:
    b = ctypes.c_size_t()
    _check(load(False).qgemv_moe_workspace_bytes(E, H, I, N, top_k, ctypes.byref(b)), "qgemv_moe_workspace_bytes")
    return b.value


def qgemv_moe(fmt, wq_gu, ws_gu, wq_dn, ws_dn, E: int, H: int, I: int, x, ids, gates, top_k: int, y, N: int,
              workspace, workspace_bytes: int, residual=None, stream=None) -> None:
    _check(load().qgemv_moe(_fmt(fmt), _ptr(wq_gu), _ptr(ws_gu), _ptr(wq_dn), _ptr(ws_dn), E, H, I, _ptr(x),
                            _ptr(ids), _ptr(gates), top_k, _ptr(residual), _ptr(y), N, _ptr(workspace),
                            workspace_bytes, _stream(stream)), "qgemv_moe")


def qgemv_moe_index(ids, N: int, top_k: int, E: int, counts, offsets, pairs, active, meta, stream=None) -> None:
    _check(load().qgemv_moe_index(_ptr(ids), N, top_k, E, _ptr(counts), _ptr(offsets), _ptr(pairs), _ptr(active),
                                  _ptr(meta), _stream(stream)), "qgemv_moe_index")


def qgemv_moe_noalloc(fmt, wq_gu, ws_gu, wq_dn, ws_dn, E: int, H: int, I: int, x, ids, gates, top_k: int, y, N: int,
                      residual=None, stream=None) -> None:
    """qgemv_moe with its scratch in the library's static per-GPU array (no
    workspace argument; nothing is allocated)."""
    _check(load().qgemv_moe_noalloc(_fmt(fmt), _ptr(wq_gu), _ptr(ws_gu), _ptr(wq_dn), _ptr(ws_dn), E, H, I, _ptr(x),
                                    _ptr(ids), _ptr(gates), top_k, _ptr(residual), _ptr(y), N, _stream(stream)),
           "qgemv_moe_noalloc")


def moe_noalloc_max_bytes() -> int:
    b = ctypes.c_size_t()
    _check(load(False).qgemv_moe_noalloc_max_bytes(ctypes.byref(b)), "qgemv_moe_noalloc_max_bytes")
    return b.value


def qgemv_moe_index_by(routine: int, ids, N: int, top_k: int, E: int, counts, offsets, pairs, active, meta,
                       stream=None) -> None:
    """The routing index as one MoE path computes it: routine 0 = qgemv_moe's
    per-slot routing, 1 = the single launch of qgemv_moe_fused."""
    _check(load().qgemv_moe_index_by(int(routine), _ptr(ids), N, top_k, E, _ptr(counts), _ptr(offsets), _ptr(pairs),
                                     _ptr(active), _ptr(meta), _stream(stream)), "qgemv_moe_index_by")


def qgemv_moe_route(logits, N: int, E: int, top_k: int, ids, gates, stream=None) -> None:
    _check(load().qgemv_moe_route(_ptr(logits), N, E, top_k, _ptr(ids), _ptr(gates), _stream(stream)),
           "qgemv_moe_route")


def moe_fused_workspace_bytes(E: int, H: int, I: int, N: int, top_k: int) -> int:
    b = ctypes.c_size_t()
    _check(load(False).qgemv_moe_fused_workspace_bytes(E, H, I, N, top_k, ctypes.byref(b)),
           "qgemv_moe_fused_workspace_bytes")
    return b.value


def qgemv_moe_fused(fmt, wq_gu, ws_gu, wq_dn, ws_dn, E: int, H: int, I: int, x, logits, top_k: int, y, N: int,
                    workspace, workspace_bytes: int, residual=None, ids_out=None, gates_out=None,
                    stream=None) -> None:
    _check(load().qgemv_moe_fused(_fmt(fmt), _ptr(wq_gu), _ptr(ws_gu), _ptr(wq_dn), _ptr(ws_dn), E, H, I, _ptr(x),
                                  _ptr(logits), top_k, _ptr(residual), _ptr(y), N, _ptr(ids_out), _ptr(gates_out),
                                  _ptr(workspace), workspace_bytes, _stream(stream)), "qgemv_moe_fused")


def qgemv_dequant(fmt, wq, ws, M: int, K: int, out, stream=None) -> None:
    _check(load().qgemv_dequant(_fmt(fmt), _ptr(wq), _ptr(ws), M, K, _ptr(out), _stream(stream)), "qgemv_dequant")


def act_quant(x, codes, scales, N: int, K: int, stream=None) -> None:
    """Dynamic MXFP8 quantisation of bf16 activations x [N][K] into codes
    [N][K] (uint8) and E8M0 scales [N][K/32] (uint8), on the device."""
    _check(load().qgemv_act_quant(_ptr(x), N, K, _ptr(codes), _ptr(scales), _stream(stream)), "qgemv_act_quant")


def qgemv_mx(fmt, wq, ws, xq, xs, y, M: int, K: int, N: int, residual=None, stream=None) -> None:
    """MX GEMV: MXFP8 / MXFP4 weights times MXFP8 activations (from
    act_quant) on the block-scaled MFMA; y [N][M] fp32, N <= 32."""
    _check(load().qgemv_mx(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(xq), _ptr(xs), _ptr(residual), _ptr(y), M, K, N,
                           _stream(stream)), "qgemv_mx")


def qgemv_mx_swiglu(fmt, wq, ws, xq, xs, h, I: int, K: int, N: int, stream=None) -> None:
    """qgemv_mx over [2I][K] weights (gate rows, then up rows) with SwiGLU:
    h [N][I] = silu(gate) * up."""
    _check(load().qgemv_mx_swiglu(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(xq), _ptr(xs), _ptr(h), I, K, N,
                                  _stream(stream)), "qgemv_mx_swiglu")


def qgemv_mx_swiglu_quant(fmt, wq, ws, xq, xs, hq, hs, I: int, K: int, N: int, h=None, stream=None) -> None:
    """qgemv_mx_swiglu whose output is bf16(h) quantised to MXFP8 as act_quant
    does: codes hq [N][I] (uint8) and E8M0 scales hs [N][I/32] (uint8); h
    [N][I] fp32, if given, also receives the h that was quantised."""
    _check(load().qgemv_mx_swiglu_quant(_fmt(fmt), _ptr(wq), _ptr(ws), _ptr(xq), _ptr(xs), _ptr(h), _ptr(hq),
                                        _ptr(hs), I, K, N, _stream(stream)), "qgemv_mx_swiglu_quant")


def qgemv_probe_read(buf, nbytes: int, sink, stream=None) -> None:
    _check(load().qgemv_probe_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "qgemv_probe_read")

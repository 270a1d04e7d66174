"""GPTQ layer quantizer for AMD MI355X (gfx950).

Thin Python binding over the C ABI of libgptq.so (include/gptq.h).  Every
stage of the method runs in the library's HIP kernels; this module only
allocates device memory and passes pointers and the current stream.  PyTorch
is used for device memory and streams only.

    H = torch.zeros(d_in, d_in, device="cuda")
    hessian_accumulate(X, H)                       # H += 2 X^T X
    q = quantize_layer(W, H, bits=4, group_size=128, block_size=128,
                       damp=0.01, act_order=False)
    q.qpacked, q.scales, q.zeros, q.perm

The library must have been built (python -m post_weight_quantization_04_amd.build);
the first call into it raises ImportError if libgptq.so is missing (there is
no fallback path).  The seeded input generator (.synth) does not need it.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "GptqError", "lib", "hessian_accumulate", "hessian_workspace_size", "quantize_layer",
    "quantize_layer_workspace_size", "inverse_factor", "packed_words", "num_groups", "QuantizedLayer",
    "LIB_PATH", "F32", "BF16", "profile_enable", "profile_read", "hessian_accumulate_noalloc",
    "hessian_noalloc_max_d_in", "dequant_matmul", "dequant_matmul_workspace_size", "quantize_layers",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq.so")
F32, BF16 = 0, 1
_STATUS = {0: "GPTQ_OK", 1: "GPTQ_EINVAL", 2: "GPTQ_ENOTSPD", 3: "GPTQ_EHIP", 4: "GPTQ_ENOMEM"}


class GptqError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libgptq.so not found at {LIB_PATH}; build it with "
            "`python -m post_weight_quantization_04_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    c = ctypes
    L.gptq_hessian_workspace_size.argtypes = [c.c_int64, c.c_int64, c.c_int]
    L.gptq_hessian_workspace_size.restype = c.c_size_t
    L.gptq_hessian_accumulate.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_void_p,
                                          c.c_void_p, c.c_size_t, c.c_void_p]
    L.gptq_hessian_accumulate.restype = c.c_int
    L.gptq_hessian_accumulate_noalloc.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_void_p,
                                                  c.c_void_p]
    L.gptq_hessian_accumulate_noalloc.restype = c.c_int
    L.gptq_hessian_noalloc_max_d_in.argtypes = [c.c_int]
    L.gptq_hessian_noalloc_max_d_in.restype = c.c_int64
    L.gptq_quantize_layer_workspace_size.argtypes = [c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int]
    L.gptq_quantize_layer_workspace_size.restype = c.c_size_t
    L.gptq_quantize_layer.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_void_p, c.c_int, c.c_int,
                                      c.c_int, c.c_float, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
                                      c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
    L.gptq_quantize_layer.restype = c.c_int
    L.gptq_dequant_matmul_workspace_size.argtypes = [c.c_int64, c.c_int64, c.c_int64, c.c_int, c.c_int]
    L.gptq_dequant_matmul_workspace_size.restype = c.c_size_t
    L.gptq_dequant_matmul.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_void_p, c.c_void_p, c.c_void_p,
                                      c.c_void_p, c.c_int64, c.c_int, c.c_int, c.c_void_p, c.c_int, c.c_void_p,
                                      c.c_size_t, c.c_void_p]
    L.gptq_dequant_matmul.restype = c.c_int
    L.gptq_quantize_layers_workspace_size.argtypes = [c.c_int, c.c_void_p, c.c_int64, c.c_int, c.c_int, c.c_int,
                                                      c.c_int]
    L.gptq_quantize_layers_workspace_size.restype = c.c_size_t
    L.gptq_quantize_layers.argtypes = [c.c_int, c.c_void_p, c.c_int, c.c_void_p, c.c_int64, c.c_void_p, c.c_int,
                                       c.c_int, c.c_int, c.c_float, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p,
                                       c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
    L.gptq_quantize_layers.restype = c.c_int
    L.gptq_inverse_factor.argtypes = [c.c_void_p, c.c_int64, c.c_float, c.c_int, c.c_void_p, c.c_void_p,
                                      c.c_void_p, c.c_size_t, c.c_void_p]
    L.gptq_inverse_factor.restype = c.c_int
    L.gptq_packed_words.argtypes = [c.c_int64, c.c_int]
    L.gptq_packed_words.restype = c.c_int64
    L.gptq_num_groups.argtypes = [c.c_int64, c.c_int]
    L.gptq_num_groups.restype = c.c_int64
    L.gptq_status_string.argtypes = [c.c_int]
    L.gptq_status_string.restype = c.c_char_p
    L.gptq_last_error.argtypes = []
    L.gptq_last_error.restype = c.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = c.c_char_p
    L.gptq_profile_enable.argtypes = [c.c_int]
    L.gptq_profile_enable.restype = None
    L.gptq_profile_read.argtypes = [c.POINTER(_Profile), c.c_int]
    L.gptq_profile_read.restype = c.c_int
    L.gptq_profile_stage_name.argtypes = [c.c_int]
    L.gptq_profile_stage_name.restype = c.c_char_p
    return L


NUM_STAGES = 8


class _Profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * NUM_STAGES), ("launches", ctypes.c_int64 * NUM_STAGES)]


def profile_enable(on=True) -> None:
    """Record hipEvents around stage launches (see gptq_profile_enable): True
    times every stage, False none, an int is the stage bit mask."""
    if isinstance(on, bool):
        mask = (1 << NUM_STAGES) - 1 if on else 0
    else:
        mask = int(on)
    _lib().gptq_profile_enable(mask)


def profile_read(reset: bool = True) -> dict:
    """{stage name: (summed GPU ms, timed launch groups)} since the last reset."""
    p = _Profile()
    _check(_lib().gptq_profile_read(ctypes.byref(p), int(bool(reset))))
    return {_lib().gptq_profile_stage_name(i).decode(): (p.ms[i], int(p.launches[i])) for i in range(NUM_STAGES)}


_LIB = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return _lib()
    raise AttributeError(name)


def _check(status: int) -> None:
    if status != 0:
        raise GptqError(status, _lib().gptq_last_error().decode(errors="replace"))


def _torch():
    import torch  # memory and streams only
    return torch


def _stream_ptr(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _require(t, name, dtype=None, ndim=None, device=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def packed_words(d_in: int, bits: int) -> int:
    return int(_lib().gptq_packed_words(d_in, bits))


def num_groups(d_in: int, group_size: int) -> int:
    return int(_lib().gptq_num_groups(d_in, group_size))


def hessian_workspace_size(n: int, d_in: int, dtype_code: int) -> int:
    return int(_lib().gptq_hessian_workspace_size(n, d_in, dtype_code))


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def hessian_accumulate(X, H, workspace=None, stream=None) -> None:
    """H += 2 X^T X.  X: [n, d_in] float32/bfloat16 (device); H: [d_in, d_in] float32."""
    torch = _torch()
    _require(X, "X", ndim=2)
    _require(H, "H", dtype=torch.float32, ndim=2)
    n, d = X.shape
    if H.shape != (d, d):
        raise ValueError(f"H must be [{d}, {d}]")
    code = _dtype_code(X)
    ws = _workspace(hessian_workspace_size(n, d, code), X.device, workspace)
    _check(_lib().gptq_hessian_accumulate(X.data_ptr() if n else None, code, n, d, H.data_ptr(),
                                       ws.data_ptr() if ws is not None else None,
                                       0 if ws is None else ws.numel(), _stream_ptr(stream)))


def hessian_accumulate_noalloc(X, H, stream=None) -> None:
    """H += 2 X^T X with the library's static scratch instead of a workspace
    (gptq_hessian_accumulate_noalloc: nothing is allocated; calls that overlap
    on one GPU race)."""
    torch = _torch()
    _require(X, "X", ndim=2)
    _require(H, "H", dtype=torch.float32, ndim=2)
    n, d = X.shape
    if H.shape != (d, d):
        raise ValueError(f"H must be [{d}, {d}]")
    _check(_lib().gptq_hessian_accumulate_noalloc(X.data_ptr() if n else None, _dtype_code(X), n, d, H.data_ptr(),
                                                  _stream_ptr(stream)))


def hessian_noalloc_max_d_in(dtype_code: int) -> int:
    return int(_lib().gptq_hessian_noalloc_max_d_in(dtype_code))


def quantize_layer_workspace_size(d_out, d_in, bits, group_size, block_size, act_order) -> int:
    return int(_lib().gptq_quantize_layer_workspace_size(d_out, d_in, bits, group_size, block_size, int(act_order)))


@dataclass
class QuantizedLayer:
    qpacked: "object"   # uint32 words, torch.int32 view [words, d_out]
    scales: "object"    # float32 [groups, d_out]
    zeros: "object"     # float32 [groups, d_out]
    perm: "object"      # int32 [d_in]
    bits: int
    group_size: int     # effective group size
    d_in: int
    act_order: bool = True   # False: perm is the identity (products then skip the gather)


def quantize_layer(W, H, bits: int = 4, group_size: int = 128, block_size: int = 128, damp: float = 0.01,
                   act_order: bool = False, workspace=None, stream=None) -> QuantizedLayer:
    """Quantize one layer.  W: [d_out, d_in] float32/bfloat16; H: [d_in, d_in] float32 (undamped)."""
    torch = _torch()
    _require(W, "W", ndim=2)
    _require(H, "H", dtype=torch.float32, ndim=2)
    d_out, d_in = W.shape
    if H.shape != (d_in, d_in):
        raise ValueError(f"H must be [{d_in}, {d_in}]")
    G = num_groups(d_in, group_size)
    nw = packed_words(d_in, bits)
    if G < 1 or nw < 0:
        raise GptqError(1, "invalid group_size or bits")
    dev = W.device
    q = torch.empty((max(nw, 0), d_out), dtype=torch.int32, device=dev)
    sc = torch.empty((G, d_out), dtype=torch.float32, device=dev)
    zr = torch.empty((G, d_out), dtype=torch.float32, device=dev)
    pm = torch.empty((d_in,), dtype=torch.int32, device=dev)
    need = quantize_layer_workspace_size(d_out, d_in, bits, group_size, block_size, act_order)
    ws = _workspace(need, dev, workspace)
    _check(_lib().gptq_quantize_layer(W.data_ptr(), _dtype_code(W), d_out, d_in, H.data_ptr(), bits, group_size,
                                   block_size, float(damp), int(bool(act_order)), q.data_ptr(), sc.data_ptr(),
                                   zr.data_ptr(), pm.data_ptr(), ws.data_ptr() if ws is not None else None,
                                   0 if ws is None else ws.numel(), _stream_ptr(stream)))
    g_eff = d_in if (group_size == -1 or group_size >= d_in) else group_size
    return QuantizedLayer(q, sc, zr, pm, bits, g_eff, d_in, bool(act_order))


def quantize_layers(Ws, H, bits: int = 4, group_size: int = 128, block_size: int = 128, damp: float = 0.01,
                    act_order: bool = False, workspace=None, stream=None):
    """Quantize several layers that share the input, hence H (gptq_quantize_layers):
    one factorization, then each W [d_out_l, d_in] as quantize_layer would.
    Returns a list of QuantizedLayer sharing one perm."""
    torch = _torch()
    Ws = list(Ws)
    if not Ws:
        raise ValueError("no layers")
    _require(H, "H", dtype=torch.float32, ndim=2)
    d_in = H.shape[0]
    code = None
    for W in Ws:
        _require(W, "W", ndim=2)
        if W.shape[1] != d_in:
            raise ValueError(f"every W must have {d_in} columns")
        c = _dtype_code(W)
        if code is not None and c != code:
            raise TypeError("every W must have the same dtype")
        code = c
    n = len(Ws)
    G = num_groups(d_in, group_size)
    nw = packed_words(d_in, bits)
    if G < 1 or nw < 0:
        raise GptqError(1, "invalid group_size or bits")
    dev = Ws[0].device
    d_outs = (ctypes.c_int64 * n)(*[W.shape[0] for W in Ws])
    outs = [(torch.empty((nw, W.shape[0]), dtype=torch.int32, device=dev),
             torch.empty((G, W.shape[0]), dtype=torch.float32, device=dev),
             torch.empty((G, W.shape[0]), dtype=torch.float32, device=dev)) for W in Ws]
    pm = torch.empty((d_in,), dtype=torch.int32, device=dev)
    ptrs = lambda xs: (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    need = int(_lib().gptq_quantize_layers_workspace_size(n, d_outs, d_in, bits, group_size, block_size,
                                                           int(act_order)))
    ws = _workspace(need, dev, workspace)
    _check(_lib().gptq_quantize_layers(n, ptrs(Ws), code, d_outs, d_in, H.data_ptr(), bits, group_size, block_size,
                                       float(damp), int(bool(act_order)), ptrs([o[0] for o in outs]),
                                       ptrs([o[1] for o in outs]), ptrs([o[2] for o in outs]), pm.data_ptr(),
                                       ws.data_ptr() if ws is not None else None, 0 if ws is None else ws.numel(),
                                       _stream_ptr(stream)))
    g_eff = d_in if (group_size == -1 or group_size >= d_in) else group_size
    return [QuantizedLayer(o[0], o[1], o[2], pm, bits, g_eff, d_in, bool(act_order)) for o in outs]


def dequant_matmul_workspace_size(m, d_out, d_in, bits, group_size) -> int:
    return int(_lib().gptq_dequant_matmul_workspace_size(m, d_out, d_in, bits, group_size))


def dequant_matmul(A, q: "QuantizedLayer", out_dtype=None, workspace=None, stream=None, use_perm=None):
    """Y = A W_hat^T on the packed layer q (gptq_dequant_matmul).  A: [m, d_in]
    bfloat16/float32 activations in the original column order; returns Y
    [m, d_out] in out_dtype (float32 by default, or bfloat16).  A workspace
    passed in must have been zeroed before its first use (calls leave it so).
    use_perm: gather A through q.perm (default: when q was quantized with
    act-order; otherwise perm is the identity and is not passed)."""
    torch = _torch()
    _require(A, "A", ndim=2)
    m, d_in = A.shape
    if d_in != q.d_in:
        raise ValueError(f"A has {d_in} columns, the layer {q.d_in}")
    d_out = q.scales.shape[1]
    out_dtype = out_dtype or torch.float32
    if use_perm is None:
        use_perm = q.act_order
    Y = torch.empty((m, d_out), dtype=out_dtype, device=A.device)
    need = dequant_matmul_workspace_size(m, d_out, d_in, q.bits, q.group_size)
    # zeroed before its first use (completion counters); calls leave it so
    if workspace is not None and workspace.numel() * workspace.element_size() >= need:
        ws = workspace
    else:
        ws = torch.zeros(need, dtype=torch.uint8, device=A.device) if need else None
    _check(_lib().gptq_dequant_matmul(A.data_ptr() if m else None, _dtype_code(A), m, d_in, q.qpacked.data_ptr(),
                                      q.scales.data_ptr(), q.zeros.data_ptr(),
                                      q.perm.data_ptr() if use_perm else None, d_out, q.bits, q.group_size,
                                      Y.data_ptr(), _dtype_code(Y), ws.data_ptr() if ws is not None else None,
                                      0 if ws is None else ws.numel(), _stream_ptr(stream)))
    return Y


def inverse_factor(H, damp: float = 0.01, act_order: bool = False, workspace=None, stream=None):
    """(perm, U) with (H[perm][:, perm] + lambda I)^-1 = U^T U, U upper (stage 2 alone)."""
    torch = _torch()
    _require(H, "H", dtype=torch.float32, ndim=2)
    d = H.shape[0]
    pm = torch.empty((d,), dtype=torch.int32, device=H.device)
    U = torch.empty((d, d), dtype=torch.float32, device=H.device)
    need = quantize_layer_workspace_size(1, d, 4, -1, 1, act_order)
    ws = _workspace(need, H.device, workspace)
    _check(_lib().gptq_inverse_factor(H.data_ptr(), d, float(damp), int(bool(act_order)), pm.data_ptr(),
                                   U.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream)))
    return pm, U

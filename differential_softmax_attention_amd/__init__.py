"""Python binding of libdiffattn: differential softmax attention on MI355X (gfx950).

Argument marshalling only. Every function builds the C-ABI argument list from torch tensors
(device pointer, element strides) and calls the library of the same name; all arithmetic runs in
the library's HIP kernels on the tensors' device, on torch's current stream. Tensors use the
token-major layout [batch, tokens, heads, dim] with a contiguous last dimension.

The library must be built (``python -m differential_softmax_attention_amd.build`` or
``__graft_entry__.build()``); nothing here falls back to another implementation, and calling an
op without the built library raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdiffattn.so")

DIFFATTN_OK = 0
DIFFATTN_ERR_ARG = 1
DIFFATTN_ERR_UNSUPPORTED = 2
DIFFATTN_ERR_WORKSPACE = 3
DIFFATTN_ERR_HIP = 4
_STATUS_NAMES = {1: "ERR_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_WORKSPACE", 4: "ERR_HIP"}

DIFFATTN_F32 = 0
DIFFATTN_BF16 = 1
EPI_NONE = 0
EPI_RMSNORM_SCALE = 1

# Every symbol the header declares (tests check the library exports all of them).
EXPORTED = ("diffattn_last_error", "diffattn_version", "diffattn_lambda_init", "diffattn_lambda",
            "diffattn_fwd", "diffattn_decode_workspace_size", "diffattn_decode", "diffattn_v2_fwd",
            "diffattn_v2_decode_workspace_size", "diffattn_v2_decode", "diffattn_fwd_train",
            "diffattn_bwd_workspace_size", "diffattn_bwd", "diffattn_lambda_bwd", "diffattn_decode_paged",
            "diffattn_v2_decode_paged", "diffattn_v2_fwd_train", "diffattn_v2_bwd_workspace_size", "diffattn_v2_bwd",
            "diffattn_quantize_fp8", "diffattn_fwd_fp8", "diffattn_fwd_lambda", "diffattn_probe_mfma_peak",
            "diffattn_decode_noalloc", "diffattn_quantize_fp8_qk")
DECODE_NOALLOC_MAX_BYTES = 32 << 20


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Tensor(ctypes.Structure):
    """diffattn_tensor: base pointer and batch / token / head strides in elements."""
    _fields_ = [("ptr", ctypes.c_void_p), ("s_batch", ctypes.c_int64), ("s_seq", ctypes.c_int64),
                ("s_head", ctypes.c_int64)]


_lib = None


def lib():
    """Load libdiffattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m differential_softmax_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        T, vp, i, f, sz = Tensor, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.diffattn_last_error.restype = ctypes.c_char_p
        L.diffattn_last_error.argtypes = []
        L.diffattn_version.restype = i
        L.diffattn_version.argtypes = []
        L.diffattn_lambda_init.restype = ctypes.c_double
        L.diffattn_lambda_init.argtypes = [i]
        L.diffattn_lambda.restype = i
        L.diffattn_lambda.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp]
        L.diffattn_fwd.restype = i
        L.diffattn_fwd.argtypes = [i, T, T, T, T, T, i, i, i, i, i, i, vp, f, i, i, vp, f, f, T, vp]
        L.diffattn_decode_workspace_size.restype = sz
        L.diffattn_decode_workspace_size.argtypes = [i, i, i, i]
        L.diffattn_decode.restype = i
        L.diffattn_decode.argtypes = [i, T, T, T, T, T, vp, i, i, i, i, i, vp, f, i, vp, f, f, T, vp,
                                      sz, vp]
        L.diffattn_v2_fwd.restype = i
        L.diffattn_v2_fwd.argtypes = [i, T, T, T, vp, i, i, i, i, i, i, i, f, T, vp]
        L.diffattn_fwd_train.restype = i
        L.diffattn_fwd_train.argtypes = [i, T, T, T, T, T, i, i, i, i, i, i, vp, f, i, i, vp, f, f, T, vp, vp, vp]
        L.diffattn_bwd_workspace_size.restype = sz
        L.diffattn_bwd_workspace_size.argtypes = [i, i, i]
        L.diffattn_bwd.restype = i
        L.diffattn_bwd.argtypes = [i, T, T, T, T, T, T, i, i, i, i, i, i, vp, f, i, i, vp, f, f, vp, vp,
                                   T, T, T, T, T, vp, vp, vp, sz, vp]
        L.diffattn_lambda_bwd.restype = i
        L.diffattn_lambda_bwd.argtypes = [vp, vp, vp, vp, vp, i, i, vp, vp, vp, vp, vp]
        L.diffattn_v2_decode_workspace_size.restype = sz
        L.diffattn_v2_decode_workspace_size.argtypes = [i, i, i, i]
        L.diffattn_v2_decode.restype = i
        L.diffattn_v2_decode.argtypes = [i, T, T, T, vp, vp, i, i, i, i, i, i, f, T, vp, sz, vp]
        i64 = ctypes.c_int64
        L.diffattn_decode_noalloc.restype = i
        L.diffattn_decode_noalloc.argtypes = [i, T, T, T, T, T, vp, i, i, i, i, i, vp, f, i, vp, f, f, T, vp]
        L.diffattn_decode_paged.restype = i
        L.diffattn_decode_paged.argtypes = [i, T, T, T, T, T, vp, i64, i, i, vp, i, i, i, i, i, vp, f, i, vp, f,
                                            f, T, vp, sz, vp]
        L.diffattn_v2_fwd_train.restype = i
        L.diffattn_v2_fwd_train.argtypes = [i, T, T, T, vp, i, i, i, i, i, i, i, f, T, vp, vp, vp]
        L.diffattn_v2_bwd_workspace_size.restype = sz
        L.diffattn_v2_bwd_workspace_size.argtypes = [i, i, i]
        L.diffattn_v2_bwd.restype = i
        L.diffattn_v2_bwd.argtypes = [i, T, T, T, T, vp, i, i, i, i, i, i, i, f, vp, vp, T, T, T, vp, vp, sz, vp]
        L.diffattn_probe_mfma_peak.restype = i
        L.diffattn_probe_mfma_peak.argtypes = [vp, i, i, ctypes.POINTER(ctypes.c_double), vp]
        L.diffattn_fwd_lambda.restype = i
        L.diffattn_fwd_lambda.argtypes = [i, T, T, T, T, T, i, i, i, i, i, i, vp, vp, vp, vp, i, i, vp, i, i, vp, f, f,
                                          T, vp]
        L.diffattn_quantize_fp8.restype = i
        L.diffattn_quantize_fp8.argtypes = [T, i, i, i, i, T, vp, vp, vp]
        L.diffattn_quantize_fp8_qk.restype = i
        L.diffattn_quantize_fp8_qk.argtypes = [T, T, T, T, i, i, i, i, i, T, T, T, T, vp, vp, vp]
        L.diffattn_fwd_fp8.restype = i
        L.diffattn_fwd_fp8.argtypes = [T, T, T, T, vp, vp, vp, vp, T, i, i, i, i, i, i, vp, f, i, i, vp, f, f, T, vp]
        L.diffattn_v2_decode_paged.restype = i
        L.diffattn_v2_decode_paged.argtypes = [i, T, T, T, vp, i64, i, i, vp, vp, i, i, i, i, i, i, f, T, vp, sz,
                                               vp]
        _lib = L
    return _lib


def _check(status: int):
    if status != DIFFATTN_OK:
        raise DiffAttnError(status, lib().diffattn_last_error().decode())


# ---- argument validation (before any pointer is taken or the library is touched) -------------
# The C ABI receives pointers, strides and sizes only, so this is where operand shapes, dtypes and
# devices are checked against each other: a short operand would otherwise become out-of-bounds
# device reads, a short output out-of-bounds writes, and a dtype mismatch garbage.

def _shape(name: str, t, shape, dtype=None, like=None):
    """t has exactly `shape` (entries None are free), `dtype` if given, and like's device."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
        raise ValueError(f"{name}: expected shape {tuple('*' if w is None else w for w in shape)}, "
                         f"got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {like.device}")
    return t


def _flat(name: str, t, n: int, dtype, like, optional=False):
    """t is a contiguous 1-d (or any-shape) buffer of exactly n elements of dtype on like's device."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of {n} elements, got {t.dtype} "
                         f"shape {tuple(t.shape)}{'' if t.is_contiguous() else ' (not contiguous)'}")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {like.device}")
    return t


def _float_dtype(name: str, t):
    if t.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"{name}: unsupported dtype {t.dtype}; use bfloat16 or float32")
    return t.dtype


def _workspace(t, like):
    if t is not None:
        if not isinstance(t, torch.Tensor) or not t.is_contiguous() or t.device != like.device:
            raise ValueError("workspace must be a contiguous tensor on the operands' device")
    return t


def _v1_operands(q1, q2, k1, k2, v, out, norm_w):
    """Shapes of a V1 call: q1, q2 [B, Nq, H, d]; k1, k2 [B, Nk, H, d]; v [B, Nk, H, dv]; out
    [B, Nq, H, dv]; all one float dtype and one device; norm_w fp32 [dv] or None."""
    if not isinstance(q1, torch.Tensor) or q1.dim() != 4:
        raise ValueError(f"q1: expected a 4-d [batch, tokens, heads, d] tensor")
    B, Nq, H, d = q1.shape
    dt = _float_dtype("q1", q1)
    _shape("q2", q2, (B, Nq, H, d), dt, q1)
    _shape("k1", k1, (B, None, H, d), dt, q1)
    Nk = k1.shape[1]
    _shape("k2", k2, (B, Nk, H, d), dt, q1)
    _shape("v", v, (B, Nk, H, None), dt, q1)
    dv = v.shape[3]
    if out is not None:
        _shape("out", out, (B, Nq, H, dv), dt, q1)
    _flat("norm_w", norm_w, dv, torch.float32, q1, optional=True)
    return B, Nq, Nk, H, d, dv


def _v2_operands(q, k, v, out, same_len=True):
    """Shapes of a V2 call: q [B, N, 2h, d]; k, v [B, Nk, h_kv, d] (Nk = N unless same_len is
    False, as for a decode's cache); out [B, N, h, d]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: expected a 4-d [batch, tokens, 2h, d] tensor")
    B, N, H2, d = q.shape
    if H2 % 2:
        raise ValueError("q must hold an even number of heads (2h)")
    dt = _float_dtype("q", q)
    _shape("k", k, (B, N if same_len else None, None, d), dt, q)
    _shape("v", v, (B, k.shape[1], k.shape[2], d), dt, q)
    if out is not None:
        _shape("out", out, (B, N, H2 // 2, d), dt, q)
    return B, N, k.shape[1], H2 // 2, k.shape[2], d


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DIFFATTN_BF16
    if t.dtype == torch.float32:
        return DIFFATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dp(x: torch.Tensor) -> int:
    """Device address of a GPU tensor. Every pointer the library receives is dereferenced on the
    GPU, so a host tensor is refused here rather than handed over."""
    if not x.is_cuda:
        raise ValueError(f"expected a tensor on the GPU, got one on {x.device}")
    return x.data_ptr()


def _t4(x: torch.Tensor) -> Tensor:
    """A [B, N, H, dim] tensor (last dim contiguous) as a diffattn_tensor."""
    if x.dim() != 4:
        raise ValueError(f"expected a 4-d [batch, tokens, heads, dim] tensor, got shape {tuple(x.shape)}")
    if x.stride(3) != 1 and x.shape[3] > 1:
        raise ValueError("the last dimension must be contiguous")
    return Tensor(_dp(x), x.stride(0), x.stride(1), x.stride(2))


def _ptr(x):
    return None if x is None else _dp(x)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def lambda_init(layer: int) -> float:
    """0.8 - 0.6 exp(-0.3 (layer - 1)); NaN for layer < 1."""
    return float(lib().diffattn_lambda_init(int(layer)))


def diffattn_lambda(lq1, lk1, lq2, lk2, layer: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """lambda per row of four fp32 [n, dim] device tensors: exp(lq1.lk1) - exp(lq2.lk2) + lambda_init."""
    vecs = [t if t.dim() == 2 else t.reshape(1, -1) for t in (lq1, lk1, lq2, lk2)]
    n, dim = vecs[0].shape
    for name, t in zip(("lq1", "lk1", "lq2", "lk2"), vecs):
        _flat(name, t, n * dim, torch.float32, vecs[0])
        _shape(name, t, (n, dim))
    _flat("out", out, n, torch.float32, vecs[0], optional=True)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=vecs[0].device)
    _check(lib().diffattn_lambda(*(_dp(v) for v in vecs), n, dim, int(layer), _dp(out),
                                 _stream(out.device)))
    return out


def diffattn_fwd(q1, q2, k1, k2, v, lam: torch.Tensor, causal: bool = True, epilogue: bool = True,
                 lambda_init_value: float = 0.8, norm_w: torch.Tensor | None = None, eps: float = 1e-5,
                 scale: float = 0.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """DIFF V1 forward. q1, q2: [B, Nq, H, d]; k1, k2: [B, Nk, H, d]; v: [B, Nk, H, dv];
    lam: fp32 [H] on the device. Returns [B, Nq, H, dv] in the input dtype."""
    B, Nq, Nk, H, d, dv = _v1_operands(q1, q2, k1, k2, v, out, norm_w)
    _flat("lam", lam, H, torch.float32, q1)
    if out is None:
        out = torch.empty((B, Nq, H, dv), dtype=q1.dtype, device=q1.device)
    _check(lib().diffattn_fwd(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1), _t4(k2), _t4(v), B, H, Nq, Nk,
                              d, dv, _dp(lam), float(lambda_init_value), int(bool(causal)),
                              EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps),
                              float(scale), _t4(out), _stream(q1.device)))
    return out


def diffattn_decode_workspace_size(batch: int, heads: int, cache_len: int, dv: int) -> int:
    return int(lib().diffattn_decode_workspace_size(batch, heads, cache_len, dv))


def _decode_operands(q1, q2, k1c, k2c, vc, lam, cache_lens, norm_w, out):
    """Shapes of a V1 decode call; returns (q1, q2, out) as 4-d views and (B, H, L, d, dv)."""
    if q1.dim() == 3:
        q1, q2 = q1.unsqueeze(1), q2.unsqueeze(1)
    if out is not None and out.dim() == 3:
        out = out.unsqueeze(1)
    _shape("q1", q1, (None, 1, None, None))
    B, _, H, d = q1.shape
    dt = _float_dtype("q1", q1)
    _shape("q2", q2, (B, 1, H, d), dt, q1)
    _shape("k1c", k1c, (B, None, H, d), dt, q1)
    L = k1c.shape[1]
    _shape("k2c", k2c, (B, L, H, d), dt, q1)
    _shape("vc", vc, (B, L, H, None), dt, q1)
    dv = vc.shape[3]
    if out is not None:
        _shape("out", out, (B, 1, H, dv), dt, q1)
    _flat("lam", lam, H, torch.float32, q1)
    _flat("norm_w", norm_w, dv, torch.float32, q1, optional=True)
    _flat("cache_lens", cache_lens, B, torch.int32, q1, optional=True)
    return q1, q2, out, (B, H, L, d, dv)


def diffattn_decode(q1, q2, k1c, k2c, vc, lam: torch.Tensor, cache_lens: torch.Tensor | None = None,
                    epilogue: bool = True, lambda_init_value: float = 0.8,
                    norm_w: torch.Tensor | None = None, eps: float = 1e-5, scale: float = 0.0,
                    workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """DIFF V1 decode. q1, q2: [B, H, d] (or [B, 1, H, d]); caches [B, L, H, d|dv];
    cache_lens: int32 [B] on the device or None. Returns [B, H, dv]."""
    q1, q2, out, (B, H, L, d, dv) = _decode_operands(q1, q2, k1c, k2c, vc, lam, cache_lens, norm_w, out)
    _workspace(workspace, q1)
    if out is None:
        out = torch.empty((B, 1, H, dv), dtype=q1.dtype, device=q1.device)
    need = diffattn_decode_workspace_size(B, H, L, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q1.device)
    _check(lib().diffattn_decode(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1c), _t4(k2c), _t4(vc),
                                 _ptr(cache_lens), B, H, L, d, dv, _dp(lam),
                                 float(lambda_init_value),
                                 EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps),
                                 float(scale), _t4(out), _dp(workspace), workspace.numel(),
                                 _stream(q1.device)))
    return out.squeeze(1)


def diffattn_decode_noalloc(q1, q2, k1c, k2c, vc, lam: torch.Tensor, out: torch.Tensor,
                            cache_lens: torch.Tensor | None = None, epilogue: bool = True,
                            lambda_init_value: float = 0.8, norm_w: torch.Tensor | None = None, eps: float = 1e-5,
                            scale: float = 0.0) -> torch.Tensor:
    """diffattn_decode with the library's own per-GPU scratch instead of a workspace: the library
    allocates nothing, and neither does this binding (out is the caller's). Calls that overlap on
    one GPU race on that scratch. Returns out viewed as [B, H, dv]."""
    if out is None:
        raise ValueError("out is required: diffattn_decode_noalloc allocates nothing")
    q1, q2, out4, (B, H, L, d, dv) = _decode_operands(q1, q2, k1c, k2c, vc, lam, cache_lens, norm_w, out)
    _check(lib().diffattn_decode_noalloc(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1c), _t4(k2c), _t4(vc),
                                         _ptr(cache_lens), B, H, L, d, dv, _dp(lam), float(lambda_init_value),
                                         EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps),
                                         float(scale), _t4(out4), _stream(q1.device)))
    return out4.squeeze(1)


def diffattn_v2_fwd(q, k, v, lam: torch.Tensor, causal: bool = True, scale: float = 0.0,
                    out: torch.Tensor | None = None, lam_logits: bool = False) -> torch.Tensor:
    """DIFF V2 forward. q: [B, N, 2h, d]; k, v: [B, N, h_kv, d]; lam: fp32 [B, N, h] contiguous,
    lambda itself or (lam_logits=True) the projected logits whose sigmoid the kernel takes.
    Returns [B, N, h, d]."""
    B, N, Nk, h, hkv, d = _v2_operands(q, k, v, out)
    _flat("lam", lam, B * N * h, torch.float32, q)
    _shape("lam", lam, (B, N, h))
    if out is None:
        out = torch.empty((B, N, h, d), dtype=q.dtype, device=q.device)
    _check(lib().diffattn_v2_fwd(_dtype_code(q), _t4(q), _t4(k), _t4(v), _dp(lam), int(bool(lam_logits)), B, N,
                                 h, hkv,
                                 d, int(bool(causal)), float(scale), _t4(out), _stream(q.device)))
    return out


def diffattn_fwd_train(q1, q2, k1, k2, v, lam: torch.Tensor, causal: bool = True, epilogue: bool = True,
                       lambda_init_value: float = 0.8, norm_w: torch.Tensor | None = None, eps: float = 1e-5,
                       scale: float = 0.0, out: torch.Tensor | None = None):
    """DIFF V1 training forward. Returns (out, lse [B, H, Nq, 2] fp32, maps [B, Nq, H, 2, dv] fp32)."""
    B, Nq, Nk, H, d, dv = _v1_operands(q1, q2, k1, k2, v, out, norm_w)
    _flat("lam", lam, H, torch.float32, q1)
    if out is None:
        out = torch.empty((B, Nq, H, dv), dtype=q1.dtype, device=q1.device)
    lse = torch.empty((B, H, Nq, 2), dtype=torch.float32, device=q1.device)
    maps = torch.empty((B, Nq, H, 2, dv), dtype=torch.float32, device=q1.device)
    _check(lib().diffattn_fwd_train(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1), _t4(k2), _t4(v), B, H, Nq, Nk, d,
                                    dv, _dp(lam), float(lambda_init_value), int(bool(causal)),
                                    EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps),
                                    float(scale), _t4(out), _dp(lse), _dp(maps), _stream(q1.device)))
    return out, lse, maps


def diffattn_fwd_lambda(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer: int, causal: bool = True,
                        epilogue: bool = True, norm_w: torch.Tensor | None = None, eps: float = 1e-5,
                        scale: float = 0.0, out: torch.Tensor | None = None, lam_out: torch.Tensor | None = None):
    """DIFF V1 forward with lambda from its four fp32 [H, lam_dim] vectors computed in the same pass.
    Returns (out [B, Nq, H, dv], lambda [H] fp32)."""
    B, Nq, Nk, H, d, dv = _v1_operands(q1, q2, k1, k2, v, out, norm_w)
    for name, x in zip(("lq1", "lk1", "lq2", "lk2"), (lq1, lk1, lq2, lk2)):
        if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.numel() != lq1.numel() \
                or x.numel() % H or x.device != q1.device:
            raise ValueError(f"{name}: expected float32 [H, lam_dim] on the operands' device, like lq1")
    vecs = [x.reshape(H, -1).contiguous() for x in (lq1, lk1, lq2, lk2)]
    _flat("lam_out", lam_out, H, torch.float32, q1, optional=True)
    if out is None:
        out = torch.empty((B, Nq, H, dv), dtype=q1.dtype, device=q1.device)
    if lam_out is None:
        lam_out = torch.empty((H,), dtype=torch.float32, device=q1.device)
    _check(lib().diffattn_fwd_lambda(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1), _t4(k2), _t4(v), B, H, Nq, Nk, d,
                                     dv, *(_dp(x) for x in vecs), vecs[0].shape[1], int(layer),
                                     _dp(lam_out), int(bool(causal)),
                                     EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps),
                                     float(scale), _t4(out), _stream(q1.device)))
    return out, lam_out


def diffattn_quantize_fp8(x: torch.Tensor, out: torch.Tensor | None = None):
    """Dynamic absmax fp8 (OCP e4m3) codes of a bf16 [B, N, H, dim] tensor, one scale per (b, h).
    Returns (codes torch.float8_e4m3fn [B, N, H, dim], scales fp32 [B, H], amax fp32 [B, H])."""
    _shape("x", x, (None, None, None, None), torch.bfloat16)
    B, N, H, dim = x.shape
    if out is not None:
        _shape("out", out, (B, N, H, dim), torch.float8_e4m3fn, x)
    if out is None:
        out = torch.empty((B, N, H, dim), dtype=torch.float8_e4m3fn, device=x.device)
    scales = torch.empty((B, H), dtype=torch.float32, device=x.device)
    amax = torch.empty((B, H), dtype=torch.float32, device=x.device)
    _check(lib().diffattn_quantize_fp8(_t4(x), B, N, H, dim, _t4(out), _dp(scales), _dp(amax),
                                       _stream(x.device)))
    return out, scales, amax


def diffattn_quantize_fp8_qk(q1, q2, k1, k2, out=None):
    """The four score operands quantised in one call: q1, q2 bf16 [B, Nq, H, dim], k1, k2 bf16
    [B, Nk, H, dim]. Returns (codes (cq1, cq2, ck1, ck2) float8_e4m3fn, scales fp32 [4, B, H],
    amax fp32 [4, B, H]); scales[i] is the i-th operand's, in the order q1, q2, k1, k2."""
    _shape("q1", q1, (None, None, None, None), torch.bfloat16)
    B, Nq, H, dim = q1.shape
    _shape("q2", q2, (B, Nq, H, dim), torch.bfloat16, q1)
    _shape("k1", k1, (B, None, H, dim), torch.bfloat16, q1)
    Nk = k1.shape[1]
    _shape("k2", k2, (B, Nk, H, dim), torch.bfloat16, q1)
    f8 = torch.float8_e4m3fn
    if out is None:
        out = tuple(torch.empty(t.shape, dtype=f8, device=q1.device) for t in (q1, q2, k1, k2))
    for name, o, x in zip(("oq1", "oq2", "ok1", "ok2"), out, (q1, q2, k1, k2)):
        _shape(name, o, tuple(x.shape), f8, q1)
    scales = torch.empty((4, B, H), dtype=torch.float32, device=q1.device)
    amax = torch.empty((4, B, H), dtype=torch.float32, device=q1.device)
    _check(lib().diffattn_quantize_fp8_qk(_t4(q1), _t4(q2), _t4(k1), _t4(k2), B, Nq, Nk, H, dim,
                                          *(_t4(o) for o in out), _dp(scales), _dp(amax), _stream(q1.device)))
    return out, scales, amax


def diffattn_fwd_fp8(q1, q2, k1, k2, sq1, sq2, sk1, sk2, v, lam: torch.Tensor, causal: bool = True,
                     epilogue: bool = True, lambda_init_value: float = 0.8, norm_w: torch.Tensor | None = None,
                     eps: float = 1e-5, scale: float = 0.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """DIFF V1 forward with fp8 (e4m3) score operands and their [B, H] scales; v bf16 [B, Nk, H, dv].
    Returns bf16 [B, Nq, H, dv]."""
    f8 = torch.float8_e4m3fn
    _shape("q1", q1, (None, None, None, None), f8)
    B, Nq, H, d = q1.shape
    _shape("q2", q2, (B, Nq, H, d), f8, q1)
    _shape("k1", k1, (B, None, H, d), f8, q1)
    Nk = k1.shape[1]
    _shape("k2", k2, (B, Nk, H, d), f8, q1)
    _shape("v", v, (B, Nk, H, None), torch.bfloat16, q1)
    dv = v.shape[3]
    for name, sc in (("sq1", sq1), ("sq2", sq2), ("sk1", sk1), ("sk2", sk2)):
        _flat(name, sc, B * H, torch.float32, q1)
    _flat("lam", lam, H, torch.float32, q1)
    _flat("norm_w", norm_w, dv, torch.float32, q1, optional=True)
    if out is not None:
        _shape("out", out, (B, Nq, H, dv), torch.bfloat16, q1)
    if out is None:
        out = torch.empty((B, Nq, H, dv), dtype=torch.bfloat16, device=v.device)
    _check(lib().diffattn_fwd_fp8(_t4(q1), _t4(q2), _t4(k1), _t4(k2), _dp(sq1), _dp(sq2),
                                  _dp(sk1), _dp(sk2), _t4(v), B, H, Nq, Nk, d, dv, _dp(lam),
                                  float(lambda_init_value), int(bool(causal)),
                                  EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps), float(scale),
                                  _t4(out), _stream(v.device)))
    return out


def diffattn_v2_fwd_train(q, k, v, lam: torch.Tensor, causal: bool = True, scale: float = 0.0,
                          out: torch.Tensor | None = None, lam_logits: bool = False):
    """DIFF V2 training forward. Returns (out [B, N, h, d], lse [B, h, N, 2] fp32,
    maps [B, N, h, 2, d] fp32)."""
    B, N, Nk, h, hkv, d = _v2_operands(q, k, v, out)
    _flat("lam", lam, B * N * h, torch.float32, q)
    _shape("lam", lam, (B, N, h))
    if out is None:
        out = torch.empty((B, N, h, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, h, N, 2), dtype=torch.float32, device=q.device)
    maps = torch.empty((B, N, h, 2, d), dtype=torch.float32, device=q.device)
    _check(lib().diffattn_v2_fwd_train(_dtype_code(q), _t4(q), _t4(k), _t4(v), _dp(lam), int(bool(lam_logits)),
                                       B, N, h, hkv, d, int(bool(causal)), float(scale), _t4(out), _dp(lse),
                                       _dp(maps), _stream(q.device)))
    return out, lse, maps


def diffattn_v2_bwd_workspace_size(batch: int, h: int, seq: int) -> int:
    return int(lib().diffattn_v2_bwd_workspace_size(batch, h, seq))


def diffattn_v2_bwd(q, k, v, dout, lam: torch.Tensor, lse: torch.Tensor, maps: torch.Tensor, causal: bool = True,
                    scale: float = 0.0, lam_logits: bool = False, workspace: torch.Tensor | None = None) -> dict:
    """DIFF V2 backward for L = sum(dout * out). Returns dq, dk, dv (like the inputs) and dlam
    (fp32 [B, N, h]: the gradient with respect to what lam holds, lambda or its logits)."""
    B, N, Nk, h, hkv, d = _v2_operands(q, k, v, None)
    _shape("dout", dout, (B, N, h, d), q.dtype, q)
    _flat("lam", lam, B * N * h, torch.float32, q)
    _flat("lse", lse, B * h * N * 2, torch.float32, q)
    _flat("maps", maps, B * N * h * 2 * d, torch.float32, q)
    _workspace(workspace, q)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
    dlam = torch.empty((B, N, h), dtype=torch.float32, device=q.device)
    need = diffattn_v2_bwd_workspace_size(B, h, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().diffattn_v2_bwd(_dtype_code(q), _t4(q), _t4(k), _t4(v), _t4(dout), _dp(lam),
                                 int(bool(lam_logits)), B, N, h, hkv, d, int(bool(causal)), float(scale),
                                 _dp(lse), _dp(maps), _t4(g["dq"]), _t4(g["dk"]), _t4(g["dv"]),
                                 _dp(dlam), _dp(workspace), workspace.numel(), _stream(q.device)))
    g["dlam"] = dlam
    return g


def diffattn_bwd_workspace_size(batch: int, heads: int, seq_q: int) -> int:
    return int(lib().diffattn_bwd_workspace_size(batch, heads, seq_q))


def diffattn_bwd(q1, q2, k1, k2, v, dout, lam: torch.Tensor, lse: torch.Tensor, maps: torch.Tensor,
                 causal: bool = True, epilogue: bool = True, lambda_init_value: float = 0.8,
                 norm_w: torch.Tensor | None = None, eps: float = 1e-5, scale: float = 0.0,
                 workspace: torch.Tensor | None = None) -> dict:
    """DIFF V1 backward for L = sum(dout * out). Returns dq1, dq2, dk1, dk2, dv (like the inputs),
    dlam [H] fp32 and dnorm_w [dv] fp32 (None without the epilogue)."""
    B, Nq, Nk, H, d, dv = _v1_operands(q1, q2, k1, k2, v, None, norm_w)
    _shape("dout", dout, (B, Nq, H, dv), q1.dtype, q1)
    _flat("lam", lam, H, torch.float32, q1)
    _flat("lse", lse, B * H * Nq * 2, torch.float32, q1)
    _flat("maps", maps, B * Nq * H * 2 * dv, torch.float32, q1)
    _workspace(workspace, q1)
    g = {k: torch.empty_like(x) for k, x in (("dq1", q1), ("dq2", q2), ("dk1", k1), ("dk2", k2), ("dv", v))}
    dlam = torch.empty((H,), dtype=torch.float32, device=q1.device)
    dnw = torch.empty((dv,), dtype=torch.float32, device=q1.device) if epilogue else None
    need = diffattn_bwd_workspace_size(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q1.device)
    _check(lib().diffattn_bwd(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1), _t4(k2), _t4(v), _t4(dout), B, H, Nq,
                              Nk, d, dv, _dp(lam), float(lambda_init_value), int(bool(causal)),
                              EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps), float(scale),
                              _dp(lse), _dp(maps), _t4(g["dq1"]), _t4(g["dq2"]), _t4(g["dk1"]),
                              _t4(g["dk2"]), _t4(g["dv"]), _dp(dlam), _ptr(dnw), _dp(workspace),
                              workspace.numel(), _stream(q1.device)))
    g["dlam"] = dlam
    g["dnorm_w"] = dnw
    return g


def diffattn_lambda_bwd(lq1, lk1, lq2, lk2, dlam) -> dict:
    """Gradients of the lambda re-parameterisation; vectors fp32 [n, dim] (or [dim]) on the device."""
    vecs = [x.reshape(-1, x.shape[-1]).contiguous() for x in (lq1, lk1, lq2, lk2)]
    n, dim = vecs[0].shape
    for name, x in zip(("lq1", "lk1", "lq2", "lk2"), vecs):
        _shape(name, x, (n, dim), torch.float32, vecs[0])
    dl = dlam.reshape(-1).contiguous()
    _flat("dlam", dl, n, torch.float32, vecs[0])
    outs = [torch.empty_like(x) for x in vecs]
    _check(lib().diffattn_lambda_bwd(*(_dp(x) for x in vecs), _dp(dl), n, dim,
                                     *(_dp(x) for x in outs), _stream(vecs[0].device)))
    return dict(dlq1=outs[0], dlk1=outs[1], dlq2=outs[2], dlk2=outs[3])


def diffattn_v2_decode_workspace_size(batch: int, h: int, h_kv: int, cache_len: int) -> int:
    return int(lib().diffattn_v2_decode_workspace_size(batch, h, h_kv, cache_len))


def diffattn_v2_decode(q, kc, vc, lam: torch.Tensor, cache_lens: torch.Tensor | None = None,
                       scale: float = 0.0, workspace: torch.Tensor | None = None,
                       out: torch.Tensor | None = None, lam_logits: bool = False) -> torch.Tensor:
    """DIFF V2 decode. q: [B, 2h, d] (or [B, 1, 2h, d]); caches kc, vc: [B, L, h_kv, d];
    lam: fp32 [B, h] contiguous (lambda, or its logits with lam_logits=True); cache_lens: int32 [B]
    on the device or None. Returns [B, h, d]."""
    if q.dim() == 3:
        q = q.unsqueeze(1)
    if out is not None and out.dim() == 3:
        out = out.unsqueeze(1)
    _shape("q", q, (None, 1, None, None))
    B, N, L, h, hkv, d = _v2_operands(q, kc, vc, out, same_len=False)
    _flat("lam", lam, B * h, torch.float32, q)
    _shape("lam", lam, (B, h))
    _flat("cache_lens", cache_lens, B, torch.int32, q, optional=True)
    _workspace(workspace, q)
    if out is None:
        out = torch.empty((B, 1, h, d), dtype=q.dtype, device=q.device)
    need = diffattn_v2_decode_workspace_size(B, h, hkv, L)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().diffattn_v2_decode(_dtype_code(q), _t4(q), _t4(kc), _t4(vc), _ptr(cache_lens), _dp(lam),
                                    int(bool(lam_logits)), B, h, hkv, L, d, float(scale), _t4(out), _dp(workspace),
                                    workspace.numel(), _stream(q.device)))
    return out.squeeze(1)


def _check_table(block_table, cache_lens, B: int, L: int, page: int, like):
    """block_table: int32 [B, >= ceil(L / page)] with unit column stride on like's device;
    cache_lens: int32 [B] or None."""
    if not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32 or block_table.dim() != 2 \
            or block_table.stride(1) != 1:
        raise ValueError("block_table must be an int32 [batch, pages_per_seq] tensor with unit column stride")
    if block_table.shape[0] != B or block_table.shape[1] * page < L:
        raise ValueError(f"block_table: shape {tuple(block_table.shape)} does not cover {B} sequences of "
                         f"{L} tokens in pages of {page}")
    if block_table.device != like.device:
        raise ValueError(f"block_table is on {block_table.device}, the other operands on {like.device}")
    _flat("cache_lens", cache_lens, B, torch.int32, like, optional=True)


def diffattn_decode_paged(q1, q2, k1_pages, k2_pages, v_pages, block_table: torch.Tensor, lam: torch.Tensor,
                          cache_lens: torch.Tensor | None = None, max_len: int | None = None,
                          epilogue: bool = True, lambda_init_value: float = 0.8,
                          norm_w: torch.Tensor | None = None, eps: float = 1e-5, scale: float = 0.0,
                          workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """DIFF V1 decode against a paged cache. q1, q2: [B, H, d] (or [B, 1, H, d]); page pools
    k1_pages, k2_pages: [P, page_size, H, d], v_pages: [P, page_size, H, dv]; block_table: int32
    [B, pages_per_seq] on the device; cache_lens: int32 [B] on the device or None (every length
    max_len). max_len defaults to pages_per_seq * page_size. Returns [B, H, dv]."""
    if q1.dim() == 3:
        q1, q2 = q1.unsqueeze(1), q2.unsqueeze(1)
    if out is not None and out.dim() == 3:
        out = out.unsqueeze(1)
    _shape("q1", q1, (None, 1, None, None))
    B, _, H, d = q1.shape
    dt = _float_dtype("q1", q1)
    _shape("q2", q2, (B, 1, H, d), dt, q1)
    _shape("k1_pages", k1_pages, (None, None, H, d), dt, q1)
    P, page = k1_pages.shape[0], k1_pages.shape[1]
    _shape("k2_pages", k2_pages, (P, page, H, d), dt, q1)
    _shape("v_pages", v_pages, (P, page, H, None), dt, q1)
    dv = v_pages.shape[3]
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be an int32 [batch, pages_per_seq] tensor")
    L = int(max_len) if max_len is not None else block_table.shape[1] * page
    _check_table(block_table, cache_lens, B, L, page, q1)
    if out is not None:
        _shape("out", out, (B, 1, H, dv), dt, q1)
    _flat("lam", lam, H, torch.float32, q1)
    _flat("norm_w", norm_w, dv, torch.float32, q1, optional=True)
    _workspace(workspace, q1)
    if out is None:
        out = torch.empty((B, 1, H, dv), dtype=q1.dtype, device=q1.device)
    need = diffattn_decode_workspace_size(B, H, L, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q1.device)
    _check(lib().diffattn_decode_paged(_dtype_code(q1), _t4(q1), _t4(q2), _t4(k1_pages), _t4(k2_pages),
                                       _t4(v_pages), _dp(block_table), block_table.stride(0), P, page,
                                       _ptr(cache_lens), B, H, L, d, dv, _dp(lam), float(lambda_init_value),
                                       EPI_RMSNORM_SCALE if epilogue else EPI_NONE, _ptr(norm_w), float(eps),
                                       float(scale), _t4(out), _dp(workspace), workspace.numel(),
                                       _stream(q1.device)))
    return out.squeeze(1)


def diffattn_v2_decode_paged(q, k_pages, v_pages, block_table: torch.Tensor, lam: torch.Tensor,
                             cache_lens: torch.Tensor | None = None, max_len: int | None = None,
                             scale: float = 0.0, workspace: torch.Tensor | None = None,
                             out: torch.Tensor | None = None, lam_logits: bool = False) -> torch.Tensor:
    """DIFF V2 decode against a paged cache. q: [B, 2h, d] (or [B, 1, 2h, d]); page pools
    k_pages, v_pages: [P, page_size, h_kv, d]; block_table, cache_lens, max_len as in
    diffattn_decode_paged; lam: fp32 [B, h] contiguous. Returns [B, h, d]."""
    if q.dim() == 3:
        q = q.unsqueeze(1)
    if out is not None and out.dim() == 3:
        out = out.unsqueeze(1)
    _shape("q", q, (None, 1, None, None))
    B, _, H2, d = q.shape
    if H2 % 2:
        raise ValueError("q must hold an even number of heads (2h)")
    h = H2 // 2
    dt = _float_dtype("q", q)
    _shape("k_pages", k_pages, (None, None, None, d), dt, q)
    P, page, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _shape("v_pages", v_pages, (P, page, hkv, d), dt, q)
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be an int32 [batch, pages_per_seq] tensor")
    L = int(max_len) if max_len is not None else block_table.shape[1] * page
    _check_table(block_table, cache_lens, B, L, page, q)
    _flat("lam", lam, B * h, torch.float32, q)
    _shape("lam", lam, (B, h))
    if out is not None:
        _shape("out", out, (B, 1, h, d), dt, q)
    _workspace(workspace, q)
    if out is None:
        out = torch.empty((B, 1, h, d), dtype=q.dtype, device=q.device)
    need = diffattn_v2_decode_workspace_size(B, h, hkv, L)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().diffattn_v2_decode_paged(_dtype_code(q), _t4(q), _t4(k_pages), _t4(v_pages),
                                          _dp(block_table), block_table.stride(0), P, page,
                                          _ptr(cache_lens), _dp(lam), int(bool(lam_logits)), B, h, hkv, L, d,
                                          float(scale), _t4(out),
                                          _dp(workspace), workspace.numel(), _stream(q.device)))
    return out.squeeze(1)


def diffattn_probe_mfma_peak(blocks: int = 4096, iters: int = 2000, device="cuda") -> tuple:
    """Launch the dense bf16 MFMA rate probe once; returns (output tensor, flop of the launch)."""
    out = torch.empty((blocks * 256,), dtype=torch.float32, device=device)
    flop = ctypes.c_double(0.0)
    _check(lib().diffattn_probe_mfma_peak(_dp(out), int(blocks), int(iters), ctypes.byref(flop),
                                          _stream(out.device)))
    return out, flop.value


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


diffattn_lambda_init = lambda_init

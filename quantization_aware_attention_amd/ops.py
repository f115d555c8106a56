"""ctypes binding of libqat_attn.so (C ABI in include/qat_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch provides device memory and the current stream.
The binding raises when the library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqat_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qat_attn.h")

# status codes and flags (values of include/qat_attn.h)
QAT_OK, QAT_EINVAL, QAT_EUNSUPPORTED, QAT_EWORKSPACE, QAT_EHIP, QAT_ESCRATCH = 0, 1, 2, 3, 4, 5
QAT_NOALLOC_SCRATCH_BYTES = 64 << 20
QAT_P_ABSMAX_MAX_BYTES = 1 << 30
QAT_DTYPE_BF16, QAT_DTYPE_FP16 = 0, 1
QAT_P_QUANT = 1 << 0
QAT_P_E5M2 = 1 << 1
QAT_QKV_QUANT = 1 << 2
QAT_V_FP8_E5M2 = 1 << 3
QAT_SMOOTH_K = 1 << 4
QAT_BWD_PREPARE, QAT_BWD_DELTA, QAT_BWD_DQ, QAT_BWD_DKDV = 1, 2, 4, 8
QAT_BWD_ALL = 15

_DTYPES = {torch.bfloat16: QAT_DTYPE_BF16, torch.float16: QAT_DTYPE_FP16}


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nkv", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class QatError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def header_functions():
    """Names of the functions include/qat_attn.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qat_[a-z0-9_]+)\s*\(", txt)))


def lib():
    """Load libqat_attn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, u32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    dp = ctypes.POINTER(Dims)
    L.qat_attn_fwd.argtypes = [dp, vp, vp, vp, vp, f32, ctypes.c_int, u32, vp, vp, vp, vp, sz, vp]
    L.qat_attn_fwd.restype = ctypes.c_int
    L.qat_attn_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, f32, ctypes.c_int, u32, vp, vp, vp, vp, sz, vp]
    L.qat_attn_bwd.restype = ctypes.c_int
    L.qat_attn_bwd_stages.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, f32, ctypes.c_int, u32, vp, vp, vp, vp, sz,
                                      u32, vp]
    L.qat_attn_bwd_stages.restype = ctypes.c_int
    L.qat_attn_bwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, f32, ctypes.c_int, u32, vp, vp, vp, vp]
    L.qat_attn_bwd_noalloc.restype = ctypes.c_int
    L.qat_attn_workspace_bytes.argtypes = [dp, u32, ctypes.c_int]
    L.qat_attn_workspace_bytes.restype = sz
    L.qat_quant_v_fp8.argtypes = [dp, vp, vp, vp, vp]
    L.qat_quant_v_fp8.restype = ctypes.c_int
    L.qat_fake_quant_rows.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.qat_fake_quant_rows.restype = ctypes.c_int
    L.qat_selftest_exp2_monotone.argtypes = [f32, f32, vp, vp]
    L.qat_selftest_exp2_monotone.restype = ctypes.c_int
    L.qat_selftest_fq_scale.argtypes = [i32, vp, vp]
    L.qat_selftest_fq_scale.restype = ctypes.c_int
    L.qat_attn_p_group.argtypes = []
    L.qat_attn_p_group.restype = ctypes.c_int
    L.qat_attn_merge.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    L.qat_attn_merge.restype = ctypes.c_int
    L.qat_attn_sum.argtypes = [dp, ctypes.c_int, vp, vp, vp]
    L.qat_attn_sum.restype = ctypes.c_int
    L.qat_attn_strerror.argtypes = [ctypes.c_int]
    L.qat_attn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn, status):
    if status != QAT_OK:
        raise QatError(fn, status, lib().qat_attn_strerror(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    """Check a tensor handed to the library: the C ABI sees only raw pointers,
    so a tensor of the wrong shape, dtype or device would become an
    out-of-bounds device access instead of an error."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _on_device(**named):
    """Last check, after every shape and dtype: the library takes device
    pointers to contiguous storage only."""
    for name, t in named.items():
        if t is not None and not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous CUDA tensor")


def _need_inputs(q, k, v, quant_flags, v_scale):
    """q [B,H,Nq,D] (bf16/fp16), k [B,H,Nkv,D] and v (k's shape; uint8 codes
    with QAT_V_FP8_E5M2, then v_scale fp32 [B,H,D]) on one device."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or q.dtype not in _DTYPES:
        raise ValueError("q must be a 4-D bf16 or fp16 tensor [B, H, N, D]")
    B, H, _, D = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be a 4-D tensor [B, H, Nkv, D]")
    kshape = (B, H, k.shape[2], D)
    _need(k, "k", q.dtype, kshape, q.device)
    fp8v = bool(quant_flags & QAT_V_FP8_E5M2)
    _need(v, "v", torch.uint8 if fp8v else q.dtype, kshape, q.device)
    if fp8v:
        if v_scale is None:
            raise ValueError("v_scale is required with QAT_V_FP8_E5M2")
        _need(v_scale, "v_scale", torch.float32, (B, H, D), q.device)
    elif v_scale is not None:
        raise ValueError("v_scale is only used with QAT_V_FP8_E5M2")


def _need_workspace(ws, q):
    if ws is not None:
        _need(ws, "workspace", torch.uint8, device=q.device)
        if ws.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")


def dims_of(q, k):
    B, H, Nq, D = q.shape
    return Dims(B, H, Nq, k.shape[2], D, _DTYPES[q.dtype])


def workspace_bytes(dims: Dims, quant_flags: int, pass_: int) -> int:
    return int(lib().qat_attn_workspace_bytes(ctypes.byref(dims), quant_flags, pass_))


def p_group() -> int:
    return int(lib().qat_attn_p_group())


def attn_fwd(q, k, v, sm_scale, causal=False, quant_flags=QAT_P_QUANT, v_scale=None,
             out=None, workspace=None):
    """Forward: returns (o, o_hp, lse).  With QAT_V_FP8_E5M2, ``v`` is uint8
    e5m2 codes and ``v_scale`` fp32 [B, H, D]."""
    _need_inputs(q, k, v, quant_flags, v_scale)
    _need_workspace(workspace, q)
    dims = dims_of(q, k)
    if out is None:
        o = torch.empty_like(q)
        o_hp = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], device=q.device, dtype=torch.float32)
    else:
        o, o_hp, lse = out
        _need(o, "out[0] (o)", q.dtype, q.shape, q.device)
        _need(o_hp, "out[1] (o_hp)", q.dtype, q.shape, q.device)
        _need(lse, "out[2] (lse)", torch.float32, q.shape[:3], q.device)
    _on_device(q=q, k=k, v=v, v_scale=v_scale, o=o, o_hp=o_hp, lse=lse, workspace=workspace)
    nbytes = workspace_bytes(dims, quant_flags, 0)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, device=q.device, dtype=torch.uint8)
    st = lib().qat_attn_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(v_scale),
                            float(sm_scale), int(bool(causal)), quant_flags, _ptr(o), _ptr(o_hp),
                            _ptr(lse), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                            _stream())
    _check("qat_attn_fwd", st)
    return o, o_hp, lse


def attn_bwd(q, k, v, o_hp, lse, dout, sm_scale, causal=False, quant_flags=QAT_P_QUANT,
             v_scale=None, out=None, workspace=None, stages=QAT_BWD_ALL):
    """Straight-through backward: returns (dq, dk, dv).  ``stages`` selects a
    subset of the backward stages (qat_attn_bwd_stages)."""
    _need_inputs(q, k, v, quant_flags, v_scale)
    _need(o_hp, "o_hp", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, q.shape[:3], q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    _need_workspace(workspace, q)
    dims = dims_of(q, k)
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty(k.shape, device=k.device, dtype=q.dtype)
    else:
        dq, dk, dv = out
        _need(dq, "out[0] (dq)", q.dtype, q.shape, q.device)
        _need(dk, "out[1] (dk)", q.dtype, k.shape, q.device)
        _need(dv, "out[2] (dv)", q.dtype, k.shape, q.device)
    _on_device(q=q, k=k, v=v, v_scale=v_scale, o_hp=o_hp, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv,
               workspace=workspace)
    nbytes = workspace_bytes(dims, quant_flags, 1)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), device=q.device, dtype=torch.uint8)
    st = lib().qat_attn_bwd_stages(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(v_scale), _ptr(o_hp),
                                   _ptr(lse), _ptr(dout), float(sm_scale), int(bool(causal)), quant_flags,
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), stages,
                                   _stream())
    _check("qat_attn_bwd_stages", st)
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o_hp, lse, dout, sm_scale, causal=False, quant_flags=QAT_P_QUANT,
                     v_scale=None, out=None):
    """The backward on the library's static scratch (qat_attn_bwd_noalloc):
    returns (dq, dk, dv); allocates only the outputs when ``out`` is None."""
    _need_inputs(q, k, v, quant_flags, v_scale)
    _need(o_hp, "o_hp", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, q.shape[:3], q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    if out is None:
        dq, dk = torch.empty_like(q), torch.empty_like(k)
        dv = torch.empty(k.shape, device=k.device, dtype=q.dtype)
    else:
        dq, dk, dv = out
        _need(dq, "out[0] (dq)", q.dtype, q.shape, q.device)
        _need(dk, "out[1] (dk)", q.dtype, k.shape, q.device)
        _need(dv, "out[2] (dv)", q.dtype, k.shape, q.device)
    _on_device(q=q, k=k, v=v, v_scale=v_scale, o_hp=o_hp, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv)
    dims = dims_of(q, k)
    st = lib().qat_attn_bwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(v_scale), _ptr(o_hp),
                                    _ptr(lse), _ptr(dout), float(sm_scale), int(bool(causal)), quant_flags,
                                    _ptr(dq), _ptr(dk), _ptr(dv), _stream())
    _check("qat_attn_bwd_noalloc", st)
    return dq, dk, dv


QAT_MERGE_MAX_CHUNKS = 16


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def attn_merge(o_parts, o_hp_parts, lse_parts, out=None):
    """Merge the forward results of KV chunks by their log-sum-exp
    (qat_attn_merge): returns (o, o_hp, lse)."""
    if not (len(o_parts) == len(o_hp_parts) == len(lse_parts)) or not o_parts:
        raise ValueError("o_parts, o_hp_parts and lse_parts must be non-empty lists of equal length")
    q0 = o_parts[0]
    if not isinstance(q0, torch.Tensor) or q0.dim() != 4 or q0.dtype not in _DTYPES:
        raise ValueError("o_parts[0] must be a 4-D bf16 or fp16 tensor [B, H, Nq, D]")
    for i, (o, oh, l) in enumerate(zip(o_parts, o_hp_parts, lse_parts)):
        _need(o, f"o_parts[{i}]", q0.dtype, q0.shape, q0.device)
        _need(oh, f"o_hp_parts[{i}]", q0.dtype, q0.shape, q0.device)
        _need(l, f"lse_parts[{i}]", torch.float32, q0.shape[:3], q0.device)
    o, o_hp, lse = out if out is not None else (torch.empty_like(q0), torch.empty_like(q0),
                                                torch.empty(q0.shape[:3], dtype=torch.float32, device=q0.device))
    _need(o, "out[0] (o)", q0.dtype, q0.shape, q0.device)
    _need(o_hp, "out[1] (o_hp)", q0.dtype, q0.shape, q0.device)
    _need(lse, "out[2] (lse)", torch.float32, q0.shape[:3], q0.device)
    _on_device(**{f"o_parts[{i}]": x for i, x in enumerate(o_parts)},
               **{f"o_hp_parts[{i}]": x for i, x in enumerate(o_hp_parts)},
               **{f"lse_parts[{i}]": x for i, x in enumerate(lse_parts)}, o=o, o_hp=o_hp, lse=lse)
    dims = dims_of(q0, q0)
    _check("qat_attn_merge", lib().qat_attn_merge(ctypes.byref(dims), len(o_parts), _ptr_array(o_parts),
                                                  _ptr_array(o_hp_parts), _ptr_array(lse_parts), _ptr(o), _ptr(o_hp),
                                                  _ptr(lse), _stream()))
    return o, o_hp, lse


def attn_sum(parts, out=None):
    """Sum of [B, H, N, D] tensors in fp32, part order (qat_attn_sum)."""
    if not parts:
        raise ValueError("parts must be a non-empty list")
    p0 = parts[0]
    if not isinstance(p0, torch.Tensor) or p0.dim() != 4 or p0.dtype not in _DTYPES:
        raise ValueError("parts[0] must be a 4-D bf16 or fp16 tensor [B, H, N, D]")
    for i, t in enumerate(parts):
        _need(t, f"parts[{i}]", p0.dtype, p0.shape, p0.device)
    out = torch.empty_like(p0) if out is None else out
    _need(out, "out", p0.dtype, p0.shape, p0.device)
    _on_device(**{f"parts[{i}]": x for i, x in enumerate(parts)}, out=out)
    dims = dims_of(parts[0], parts[0])
    _check("qat_attn_sum", lib().qat_attn_sum(ctypes.byref(dims), len(parts), _ptr_array(parts), _ptr(out),
                                              _stream()))
    return out


def quant_v_fp8(v):
    """Per-(b, h, d) e5m2 quantization of V: returns (codes uint8, v_scale fp32 [B, H, D])."""
    if not isinstance(v, torch.Tensor) or v.dim() != 4 or v.dtype not in _DTYPES:
        raise ValueError("v must be a 4-D bf16 or fp16 tensor [B, H, N, D]")
    _on_device(v=v)
    B, H, N, D = v.shape
    dims = Dims(B, H, 0, N, D, _DTYPES[v.dtype])
    codes = torch.empty(v.shape, device=v.device, dtype=torch.uint8)
    v_scale = torch.empty((B, H, D), device=v.device, dtype=torch.float32)
    _check("qat_quant_v_fp8", lib().qat_quant_v_fp8(ctypes.byref(dims), _ptr(v), _ptr(codes), _ptr(v_scale), _stream()))
    return codes, v_scale


def fake_quant_rows(x, group, fmt):
    """FQ of fp32 rows (fmt 0 = e4m3fn, 1 = e5m2): returns (codes, scales, xhat)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D float32 tensor [rows, cols]")
    _need(x, "x", torch.float32)
    _on_device(x=x)
    rows, cols = x.shape
    ng = -(-cols // group)
    codes = torch.empty((rows, cols), device=x.device, dtype=torch.uint8)
    scales = torch.empty((rows, ng), device=x.device, dtype=torch.float32)
    xhat = torch.empty((rows, cols), device=x.device, dtype=torch.float32)
    _check("qat_fake_quant_rows", lib().qat_fake_quant_rows(_ptr(x), rows, cols, group, fmt, _ptr(codes),
                                                            _ptr(scales), _ptr(xhat), _stream()))
    return codes, scales, xhat


def selftest_fq_scale(fmt: int) -> int:
    """Number of positive finite fp32 absmax values whose quantizer scale pair
    (s, r) on the GPU differs from the IEEE quotients (fmt 0: e4m3, 1: e5m2)."""
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check("qat_selftest_fq_scale", lib().qat_selftest_fq_scale(int(fmt), _ptr(out), _stream()))
    torch.cuda.synchronize()
    return int(out.item())


def selftest_exp2_monotone(lo=float("-inf"), hi=128.0) -> int:
    """Number of adjacent fp32 pairs in [lo, hi] where the GPU's exp2 decreases."""
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check("qat_selftest_exp2_monotone",
           lib().qat_selftest_exp2_monotone(float(lo), float(hi), _ptr(out), _stream()))
    torch.cuda.synchronize()
    return int(out.item())

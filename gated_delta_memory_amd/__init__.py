"""Python binding of libatma, the MI355X (gfx950) hot path of the ATMA global layer.

Thin argument marshalling over the C ABI declared in ``include/atma.h``: every function
here has the name of the C entry point it calls, checks tensor shapes/dtypes/devices,
allocates outputs when the caller passes none, and hands raw device pointers and the
current HIP stream to the library.  All arithmetic runs in the library's HIP kernels;
there is no CPU or PyTorch fallback.  Importing this module fails with a clear error
if the library has not been built (``python -m gated_delta_memory_amd._build``).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # loads the HIP runtime the library shares (same soname, one instance)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libatma.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "atma.h")

ATMA_OK, ATMA_ERR_NULL, ATMA_ERR_SHAPE, ATMA_ERR_UNSUPPORTED, ATMA_ERR_WORKSPACE, ATMA_ERR_LAUNCH = 0, -1, -2, -3, -4, -5
ATMA_F32, ATMA_BF16 = 0, 1
CHUNK = 64


class AtmaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class PolarParams(ctypes.Structure):
    """Mirror of ``atma_polar_params`` (host struct of device pointers)."""
    _fields_ = [("temp_raw", ctypes.c_void_p), ("null_slope_raw", ctypes.c_void_p),
                ("null_bias", ctypes.c_void_p), ("mag_beta", ctypes.c_void_p),
                ("v_null", ctypes.c_void_p), ("eps", ctypes.c_float)]


class PolarParamGrads(ctypes.Structure):
    """Mirror of ``atma_polar_param_grads`` (host struct of device pointers, fp32 outputs)."""
    _fields_ = [("temp_raw", ctypes.c_void_p), ("null_slope_raw", ctypes.c_void_p),
                ("null_bias", ctypes.c_void_p), ("mag_beta", ctypes.c_void_p), ("v_null", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libatma.so is not built at {LIB_PATH}; run `python gated_delta_memory_amd/_build.py` "
                          f"(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER(PolarParams)
    sig = {
        "atma_gdn_fwd": ([vp] * 8 + [i] * 7 + [vp, sz, vp], i),
        "atma_gdn_fwd_workspace_bytes": ([i] * 6, sz),
        "atma_gdn_fwd_workspace_bytes_dtype": ([i] * 7, sz),
        "atma_gdn_fwd_varlen": ([vp] * 6 + [i, i] + [vp] * 3 + [i] * 6 + [vp, sz, vp], i),
        "atma_gdn_decode_step": ([vp] * 7 + [i] * 5 + [vp], i),
        "atma_polar_attn_fwd": ([vp, vp, vp, P, vp, vp, vp] + [i] * 6 + [vp, sz, vp], i),
        "atma_polar_attn_workspace_bytes": ([i] * 4, sz),
        "atma_polar_attn_fwd_varlen": ([vp, vp, vp, vp, i, i, P, vp, vp, vp] + [i] * 5 + [vp], i),
        "atma_polar_attn_decode": ([vp, vp, vp, i, i, P, vp, vp] + [i] * 5 + [vp, sz, vp], i),
        "atma_polar_attn_decode_workspace_bytes": ([i] * 4, sz),
        "atma_polar_attn_decode_noalloc": ([vp, vp, vp, i, i, P, vp, vp] + [i] * 5 + [vp], i),
        "atma_polar_attn_decode_varlen": ([vp, vp, vp, vp, i, i, P, vp, vp] + [i] * 5 + [vp, sz, vp], i),
        "atma_rope": ([vp, vp] + [i] * 5 + [f, i, vp], i),
        "atma_softmax_attn_fwd": ([vp] * 4 + [i] * 5 + [f, i, vp, sz, vp], i),
        "atma_softmax_attn_workspace_bytes": ([i] * 5 + [f], sz),
        "atma_softmax_attn_decode": ([vp] * 3 + [i, i, f, vp] + [i] * 5 + [vp, sz, vp], i),
        "atma_canon": ([vp] * 5 + [i] * 6 + [f, i, vp], i),
        "atma_polar_attn_fwd_train": ([vp, vp, vp, P, vp, vp, vp, vp] + [i] * 6 + [vp], i),
        "atma_polar_attn_bwd": ([vp, vp, vp, P] + [vp] * 7 + [ctypes.POINTER(PolarParamGrads)] + [i] * 6
                                + [vp, sz, vp], i),
        "atma_polar_attn_bwd_workspace_bytes": ([i] * 5, sz),
        "atma_gdn_bwd": ([vp] * 14 + [i] * 7 + [vp, sz, vp], i),
        "atma_gdn_bwd_workspace_bytes": ([i] * 7, sz),
        "atma_status_string": ([i], ctypes.c_char_p),
        "atma_version": ([], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def header_functions() -> list[str]:
    """Names of every function declared in include/atma.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\**\s+\**(atma_[a-z0-9_]+)\s*\(", text, re.M)))


def _check(fn: str, status: int) -> None:
    if status != ATMA_OK:
        raise AtmaError(fn, status, lib.atma_status_string(status).decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATMA_BF16
    if t.dtype == torch.float32:
        return ATMA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


def _expect(t, name, shape, dtype=None, optional=False):
    """Checks that tensor ``t`` (a buffer the library will read or write) has exactly ``shape``
    and, when given, ``dtype``; None passes only when ``optional``.  Every buffer handed to the
    C ABI goes through here or an equivalent check, so no kernel can run past a buffer's end."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------------------------
# gated-delta memory
# ------------------------------------------------------------------------------------
def atma_gdn_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk=CHUNK, dtype=None) -> int:
    """Workspace bytes of atma_gdn_fwd: for either dtype when ``dtype`` is None, else for that one."""
    if dtype is None:
        return int(lib.atma_gdn_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk))
    return int(lib.atma_gdn_fwd_workspace_bytes_dtype(B, T, H, Dk, Dv, chunk,
                                                      ATMA_BF16 if dtype == torch.bfloat16 else ATMA_F32))


def atma_gdn_fwd(q, k, v, alpha, beta, init_state=None, *, o=None, final_state=None, workspace=None,
                 want_final=True, stream=None):
    """Chunked gated-delta forward.  q, k [B,T,H,Dk], v [B,T,H,Dv] (bf16 or fp32), alpha, beta
    [B,T,H] fp32, init_state [B,H,Dv,Dk] fp32 or None.  Returns (o, final_state or None)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or alpha.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    _f32(alpha, "alpha"), _f32(beta, "beta")
    _expect(init_state, "init_state", (B, H, Dv, Dk), torch.float32, optional=True)
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=q.dtype, device=q.device)
    if final_state is None and want_final:
        final_state = torch.empty(B, H, Dv, Dk, dtype=torch.float32, device=q.device)
    _expect(o, "o", (B, T, H, Dv), q.dtype)
    _expect(final_state, "final_state", (B, H, Dv, Dk), torch.float32, optional=True)
    need = atma_gdn_fwd_workspace_bytes(B, T, H, Dk, Dv, CHUNK, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, alpha, beta, init_state, o, final_state, workspace)
    st = lib.atma_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(init_state), _ptr(o),
                          _ptr(final_state), B, T, H, Dk, Dv, CHUNK, _dtype_code(q), _ptr(workspace),
                          _nbytes(workspace), _stream(stream))
    _check("atma_gdn_fwd", st)
    return o, final_state


def atma_gdn_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, max_seqlen, init_state=None, *, o=None, final_state=None,
                        workspace=None, want_final=True, stream=None):
    """Packed chunked gated-delta forward.  q, k [total,H,Dk], v [total,H,Dv] bf16, alpha, beta
    [total,H] fp32, cu_seqlens int32 [nseq+1] on the device, init_state [nseq,H,Dv,Dk] fp32 or
    None.  Returns (o [total,H,Dv], final_state [nseq,H,Dv,Dk] or None)."""
    total, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != (total, H) or alpha.shape != (total, H) or beta.shape != (total, H):
        raise ValueError("inconsistent packed shapes")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be an int32 vector of nseq + 1 offsets")
    nseq = cu_seqlens.numel() - 1
    _f32(alpha, "alpha"), _f32(beta, "beta")
    _expect(init_state, "init_state", (nseq, H, Dv, Dk), torch.float32, optional=True)
    if o is None:
        o = torch.empty(total, H, Dv, dtype=q.dtype, device=q.device)
    if final_state is None and want_final:
        final_state = torch.empty(nseq, H, Dv, Dk, dtype=torch.float32, device=q.device)
    _expect(o, "o", (total, H, Dv), q.dtype)
    _expect(final_state, "final_state", (nseq, H, Dv, Dk), torch.float32, optional=True)
    need = atma_gdn_fwd_workspace_bytes(nseq, max_seqlen, H, Dk, Dv, CHUNK, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, alpha, beta, cu_seqlens, init_state, o, final_state, workspace)
    st = lib.atma_gdn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_seqlens), nseq,
                                 int(max_seqlen), _ptr(init_state), _ptr(o), _ptr(final_state), total, H, Dk, Dv,
                                 CHUNK, _dtype_code(q), _ptr(workspace), _nbytes(workspace),
                                 _stream(stream))
    _check("atma_gdn_fwd_varlen", st)
    return o, final_state


def atma_gdn_decode_step(q, k, v, alpha, beta, state, *, o=None, stream=None):
    """One recurrent step: q, k [B,H,Dk], v [B,H,Dv], alpha, beta [B,H] fp32, state [B,H,Dv,Dk]
    fp32 (updated in place).  Returns o [B,H,Dv]."""
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    _expect(k, "k", (B, H, Dk), q.dtype)
    _expect(v, "v", (B, H, Dv), q.dtype)
    _expect(alpha, "alpha", (B, H), torch.float32)
    _expect(beta, "beta", (B, H), torch.float32)
    _expect(state, "state", (B, H, Dv, Dk), torch.float32)
    if o is None:
        o = torch.empty(B, H, Dv, dtype=q.dtype, device=q.device)
    _expect(o, "o", (B, H, Dv), q.dtype)
    _dev(q, k, v, alpha, beta, state, o)
    st = lib.atma_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o),
                                  B, H, Dk, Dv, _dtype_code(q), _stream(stream))
    _check("atma_gdn_decode_step", st)
    return o


def atma_gdn_bwd(q, k, v, alpha, beta, do, *, init_state=None, dS_final=None, want_dinit=False, workspace=None,
                 stream=None):
    """Gradients of the chunked memory prefill for upstream ``do`` [B,T,H,Dv] (and ``dS_final``
    [B,H,Dv,Dk] fp32 on the final state).  Returns dict dq, dk, dv (input dtype), dalpha, dbeta
    [B,T,H] fp32 and dinit [B,H,Dv,Dk] fp32 (None unless ``want_dinit``)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, T, H, Dv) or do.shape != v.shape:
        raise ValueError("inconsistent shapes")
    if alpha.shape != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("alpha / beta must be [B, T, H]")
    if k.dtype != q.dtype or v.dtype != q.dtype or do.dtype != q.dtype:
        raise TypeError("q, k, v and do must share a dtype")
    _f32(alpha, "alpha"), _f32(beta, "beta")
    _expect(init_state, "init_state", (B, H, Dv, Dk), torch.float32, optional=True)
    _expect(dS_final, "dS_final", (B, H, Dv, Dk), torch.float32, optional=True)
    dt = _dtype_code(q)
    f = dict(dtype=torch.float32, device=q.device)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dalpha": torch.empty(B, T, H, **f), "dbeta": torch.empty(B, T, H, **f),
           "dinit": torch.empty(B, H, Dv, Dk, **f) if want_dinit else None}
    if workspace is None:
        workspace = torch.empty(lib.atma_gdn_bwd_workspace_bytes(B, T, H, Dk, Dv, 64, dt), dtype=torch.uint8,
                                device=q.device)
    _dev(q, k, v, alpha, beta, do, init_state, dS_final, workspace, *[x for x in out.values() if x is not None])
    st = lib.atma_gdn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(init_state), _ptr(do),
                          _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
                          _ptr(out["dbeta"]), _ptr(out["dinit"]), B, T, H, Dk, Dv, 64, dt, _ptr(workspace),
                          _nbytes(workspace), _stream(stream))
    _check("atma_gdn_bwd", st)
    return out


# ------------------------------------------------------------------------------------
# Polar attention# ------------------------------------------------------------------------------------
# Polar attention
# ------------------------------------------------------------------------------------
def polar_params_struct(params: dict, Hq: int, D: int) -> PolarParams:
    """Pack a dict of per-head fp32 device tensors (temp_raw, null_slope_raw, null_bias,
    mag_beta [Hq]; v_null [Hq, D]; eps float) into the C struct."""
    names = ("temp_raw", "null_slope_raw", "null_bias", "mag_beta", "v_null")
    for name in names:
        _expect(params[name], name, (Hq, D) if name == "v_null" else (Hq,), torch.float32)
    _dev(*(params[name] for name in names))
    return PolarParams(params["temp_raw"].data_ptr(), params["null_slope_raw"].data_ptr(),
                       params["null_bias"].data_ptr(), params["mag_beta"].data_ptr(),
                       params["v_null"].data_ptr(), float(params.get("eps", 1e-12)))


def atma_polar_attn_fwd(q, k, v, params, *, o=None, mu_out=None, meff_out=None, want_mu=False, stream=None):
    """Causal Polar attention.  q [B,T,Hq,D], k, v [B,T,Hkv,D] bf16.  Returns (o, mu, meff)
    (mu / meff are [B,Hq,T] fp32 when requested or passed in, else None)."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _expect(k, "k", (B, T, Hkv, D), q.dtype)
    _expect(v, "v", (B, T, Hkv, D), q.dtype)
    if o is None:
        o = torch.empty_like(q)
    if want_mu and mu_out is None:
        mu_out = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    if want_mu and meff_out is None:
        meff_out = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    _expect(o, "o", (B, T, Hq, D), q.dtype)
    _expect(mu_out, "mu_out", (B, Hq, T), torch.float32, optional=True)
    _expect(meff_out, "meff_out", (B, Hq, T), torch.float32, optional=True)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k, v, o, mu_out, meff_out)
    st = lib.atma_polar_attn_fwd(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(p), _ptr(o), _ptr(mu_out),
                                 _ptr(meff_out), B, T, Hq, Hkv, D, _dtype_code(q), None, 0, _stream(stream))
    _check("atma_polar_attn_fwd", st)
    return o, mu_out, meff_out


def atma_polar_attn_fwd_train(q, k, v, params, *, stream=None):
    """Training forward of causal Polar attention.  q [B,T,Hq,D], k, v [B,T,Hkv,D] bf16.
    Returns (o, mu [B,Hq,T], stats [B,Hq,T,4], dir [B,T,Hq,D]) -- the last three are what
    ``atma_polar_attn_bwd`` reads."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _expect(k, "k", (B, T, Hkv, D), q.dtype)
    _expect(v, "v", (B, T, Hkv, D), q.dtype)
    o = torch.empty_like(q)
    mu = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    stats = torch.empty(B, Hq, T, 4, dtype=torch.float32, device=q.device)
    dirn = torch.empty(B, T, Hq, D, dtype=torch.float32, device=q.device)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k, v)
    st = lib.atma_polar_attn_fwd_train(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(p), _ptr(o), _ptr(mu), _ptr(stats),
                                       _ptr(dirn), B, T, Hq, Hkv, D, _dtype_code(q), _stream(stream))
    _check("atma_polar_attn_fwd_train", st)
    return o, mu, stats, dirn


def atma_polar_attn_bwd(q, k, v, params, mu, stats, dirn, do, *, out=None, workspace=None, stream=None):
    """Gradients of causal Polar attention for upstream ``do`` [B,T,Hq,D] bf16, from the training
    forward's (mu, stats, dir).  Returns dict dq, dk, dv (bf16, shaped as q, k, v) and d_temp_raw,
    d_null_slope_raw, d_null_bias, d_mag_beta [Hq], d_v_null [Hq, D] (fp32).  ``out`` may supply
    that dict's tensors."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _expect(k, "k", (B, T, Hkv, D), q.dtype)
    _expect(v, "v", (B, T, Hkv, D), q.dtype)
    _expect(do, "do", (B, T, Hq, D), q.dtype)
    _expect(mu, "mu", (B, Hq, T), torch.float32)
    _expect(stats, "stats", (B, Hq, T, 4), torch.float32)
    _expect(dirn, "dir", (B, T, Hq, D), torch.float32)
    if out is None:
        f = dict(dtype=torch.float32, device=q.device)
        out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
               "d_temp_raw": torch.empty(Hq, **f), "d_null_slope_raw": torch.empty(Hq, **f),
               "d_null_bias": torch.empty(Hq, **f), "d_mag_beta": torch.empty(Hq, **f),
               "d_v_null": torch.empty(Hq, D, **f)}
    f32 = torch.float32
    for n, shape, dt in (("dq", (B, T, Hq, D), q.dtype), ("dk", (B, T, Hkv, D), q.dtype),
                         ("dv", (B, T, Hkv, D), q.dtype), ("d_temp_raw", (Hq,), f32), ("d_null_slope_raw", (Hq,), f32),
                         ("d_null_bias", (Hq,), f32), ("d_mag_beta", (Hq,), f32), ("d_v_null", (Hq, D), f32)):
        _expect(out.get(n), "out[" + n + "]", shape, dt)
    if workspace is None:
        workspace = torch.empty(lib.atma_polar_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D), dtype=torch.uint8,
                                device=q.device)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k, v, mu, stats, dirn, do, workspace, *out.values())
    g = PolarParamGrads(out["d_temp_raw"].data_ptr(), out["d_null_slope_raw"].data_ptr(),
                        out["d_null_bias"].data_ptr(), out["d_mag_beta"].data_ptr(), out["d_v_null"].data_ptr())
    st = lib.atma_polar_attn_bwd(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(p), _ptr(mu), _ptr(stats), _ptr(dirn),
                                 _ptr(do), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), ctypes.byref(g), B, T,
                                 Hq, Hkv, D, _dtype_code(q), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("atma_polar_attn_bwd", st)
    return out


def atma_polar_attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, params, *, o=None, want_mu=False, stream=None):
    """Packed causal Polar prefill.  q [total,Hq,D], k/v [total,Hkv,D] bf16; cu_seqlens int32
    [nseq+1] on the device.  Returns (o [total,Hq,D], mu [Hq,total] or None, meff [Hq,total] or None)."""
    total, Hq, D = q.shape
    Hkv = k.shape[1]
    _expect(k, "k", (total, Hkv, D), q.dtype)
    _expect(v, "v", (total, Hkv, D), q.dtype)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be an int32 vector of nseq + 1 offsets")
    nseq = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty_like(q)
    _expect(o, "o", (total, Hq, D), q.dtype)
    mu = meff = None
    if want_mu:
        mu = torch.empty(Hq, total, dtype=torch.float32, device=q.device)
        meff = torch.empty(Hq, total, dtype=torch.float32, device=q.device)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k, v, cu_seqlens, o, mu, meff)
    st = lib.atma_polar_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), nseq, int(max_seqlen),
                                        ctypes.byref(p), _ptr(o), _ptr(mu), _ptr(meff), total, Hq, Hkv, D,
                                        _dtype_code(q), _stream(stream))
    _check("atma_polar_attn_fwd_varlen", st)
    return o, mu, meff


def atma_polar_attn_decode_workspace_bytes(B, Hq, cache_len, D=64) -> int:
    return int(lib.atma_polar_attn_decode_workspace_bytes(B, Hq, cache_len, D))


def atma_polar_attn_decode(q, k_cache, v_cache, cache_len, params, *, o=None, mu_out=None, want_mu=False,
                           workspace=None, stream=None):
    """Decode one token.  q [B,Hq,D]; caches [B,Lmax,Hkv,D] bf16 holding cache_len valid slots
    (the new token already written at slot cache_len-1).  Returns (o [B,Hq,D], mu [B,Hq] or None)."""
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, Lmax, Hkv, D), q.dtype)
    _expect(v_cache, "v_cache", (B, Lmax, Hkv, D), q.dtype)
    if o is None:
        o = torch.empty_like(q)
    if want_mu and mu_out is None:
        mu_out = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    _expect(o, "o", (B, Hq, D), q.dtype)
    _expect(mu_out, "mu_out", (B, Hq), torch.float32, optional=True)
    need = atma_polar_attn_decode_workspace_bytes(B, Hq, cache_len, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k_cache, v_cache, o, mu_out, workspace)
    st = lib.atma_polar_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(cache_len), Lmax, ctypes.byref(p),
                                    _ptr(o), _ptr(mu_out), B, Hq, Hkv, D, _dtype_code(q), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream))
    _check("atma_polar_attn_decode", st)
    return o, mu_out


def atma_polar_attn_decode_noalloc(q, k_cache, v_cache, cache_len, params, *, o, mu_out=None, stream=None):
    """Decode one token like atma_polar_attn_decode, with no workspace and no allocation: the
    caller passes o [B,Hq,D] (and optionally mu_out [B,Hq] fp32); the split records live in the
    library's fixed 16 MiB per-device array.  Returns (o, mu_out)."""
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, Lmax, Hkv, D), q.dtype)
    _expect(v_cache, "v_cache", (B, Lmax, Hkv, D), q.dtype)
    _expect(o, "o", (B, Hq, D), q.dtype)
    _expect(mu_out, "mu_out", (B, Hq), torch.float32, optional=True)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k_cache, v_cache, o, mu_out)
    st = lib.atma_polar_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(cache_len), Lmax,
                                            ctypes.byref(p), _ptr(o), _ptr(mu_out), B, Hq, Hkv, D, _dtype_code(q),
                                            _stream(stream))
    _check("atma_polar_attn_decode_noalloc", st)
    return o, mu_out


def atma_polar_attn_decode_varlen(q, k_cache, v_cache, cache_lens, max_cache_len, params, *, o=None, mu_out=None,
                                  want_mu=False, workspace=None, stream=None):
    """Decode one token for sequences of different cache lengths.  q [B,Hq,D]; caches
    [B,Lmax,Hkv,D] bf16; cache_lens int32 [B] on the device (1 <= cache_lens[b] <= max_cache_len).
    Returns (o [B,Hq,D], mu [B,Hq] or None)."""
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, Lmax, Hkv, D), q.dtype)
    _expect(v_cache, "v_cache", (B, Lmax, Hkv, D), q.dtype)
    _expect(cache_lens, "cache_lens", (B,), torch.int32)
    if o is None:
        o = torch.empty_like(q)
    if want_mu and mu_out is None:
        mu_out = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    _expect(o, "o", (B, Hq, D), q.dtype)
    _expect(mu_out, "mu_out", (B, Hq), torch.float32, optional=True)
    need = atma_polar_attn_decode_workspace_bytes(B, Hq, max_cache_len, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    p = polar_params_struct(params, Hq, D)
    _dev(q, k_cache, v_cache, cache_lens, o, mu_out, workspace)
    st = lib.atma_polar_attn_decode_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens),
                                           int(max_cache_len), Lmax, ctypes.byref(p), _ptr(o), _ptr(mu_out), B, Hq,
                                           Hkv, D, _dtype_code(q), _ptr(workspace),
                                           _nbytes(workspace), _stream(stream))
    _check("atma_polar_attn_decode_varlen", st)
    return o, mu_out


def atma_rope(x, theta=10000.0, pos0=0, *, out=None, stream=None):
    """Rotary embedding of x [B,T,H,D] bf16 (row t at position pos0 + t).  Returns the rotated copy."""
    B, T, H, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    _expect(out, "out", (B, T, H, D), x.dtype)
    _dev(x, out)
    st = lib.atma_rope(_ptr(x), _ptr(out), B, T, H, D, int(pos0), float(theta), _dtype_code(x), _stream(stream))
    _check("atma_rope", st)
    return out


def atma_softmax_attn_fwd(q, k, v, rope_theta=0.0, *, o=None, workspace=None, stream=None):
    """NoPE (rope_theta=0) or RoPE causal softmax attention.  q [B,T,Hq,D], k/v [B,T,Hkv,D] bf16."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _expect(k, "k", (B, T, Hkv, D), q.dtype)
    _expect(v, "v", (B, T, Hkv, D), q.dtype)
    if o is None:
        o = torch.empty_like(q)
    _expect(o, "o", (B, T, Hq, D), q.dtype)
    need = int(lib.atma_softmax_attn_workspace_bytes(B, T, Hq, Hkv, D, float(rope_theta)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(q, k, v, o, workspace)
    wsb = 0 if workspace is None else _nbytes(workspace)
    st = lib.atma_softmax_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, Hq, Hkv, D, float(rope_theta),
                                   _dtype_code(q), _ptr(workspace), wsb, _stream(stream))
    _check("atma_softmax_attn_fwd", st)
    return o


def atma_softmax_attn_decode(q, k_cache, v_cache, cache_len, rope_theta=0.0, *, o=None, workspace=None, stream=None):
    """Decode row of the NoPE / RoPE core; for RoPE the cache holds rotated keys (atma_rope)."""
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, "k_cache", (B, Lmax, Hkv, D), q.dtype)
    _expect(v_cache, "v_cache", (B, Lmax, Hkv, D), q.dtype)
    if o is None:
        o = torch.empty_like(q)
    _expect(o, "o", (B, Hq, D), q.dtype)
    need = atma_polar_attn_decode_workspace_bytes(B, Hq, cache_len, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k_cache, v_cache, o, workspace)
    st = lib.atma_softmax_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(cache_len), Lmax, float(rope_theta),
                                      _ptr(o), B, Hq, Hkv, D, _dtype_code(q), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream))
    _check("atma_softmax_attn_decode", st)
    return o


def atma_canon(x, w, state=None, *, residual=False, heads=0, eps=1e-6, update_state=True, y=None, stream=None):
    """Canon prologue: x [B,T,C] bf16, w [K,C] fp32, state [B,K-1,C] bf16 or None (updated in
    place with the last K-1 inputs when ``update_state``).  Returns y [B,T,C]."""
    B, T, C = x.shape
    K = w.shape[0]
    _expect(w, "w", (K, C), torch.float32)
    _expect(state, "state", (B, K - 1, C), x.dtype, optional=True)
    if y is None:
        y = torch.empty_like(x)
    _expect(y, "y", (B, T, C), x.dtype)
    _dev(x, w, state, y)
    st = lib.atma_canon(_ptr(x), _ptr(w), _ptr(state), _ptr(state) if update_state else None, _ptr(y), B, T, C, K,
                        int(bool(residual)), int(heads), float(eps), _dtype_code(x), _stream(stream))
    _check("atma_canon", st)
    return y


def atma_polar_attn_workspace_bytes(B, T, Hq, D=64) -> int:
    return int(lib.atma_polar_attn_workspace_bytes(B, T, Hq, D))


def atma_status_string(status: int) -> str:
    return lib.atma_status_string(int(status)).decode()


def atma_version() -> int:
    return int(lib.atma_version())

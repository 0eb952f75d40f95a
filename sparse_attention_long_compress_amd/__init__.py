"""MI355X (gfx950) Native Sparse Attention: thin Python binding of libnsa.so.

Every function here only marshals arguments (torch device tensors -> raw
pointers, sizes, the current HIP stream) and calls the C ABI declared in
``include/nsa.h``; all computation runs in the library's HIP kernels.  PyTorch
provides device memory and streams only.  If the library is not built, every
call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsa.so")

NSA_BF16, NSA_FP32 = 0, 1
SKIP_CMP_OUT, SKIP_SEL, SKIP_WIN, INDICES_IN = 1, 2, 4, 8

EXPORTED = (
    "nsa_abi_version", "nsa_status_string", "nsa_check_params", "nsa_forward_kernel",
    "nsa_workspace_size",
    "nsa_pool", "nsa_compress_select", "nsa_forward", "nsa_forward_profile", "nsa_select_bwd",
    "nsa_forward_train", "nsa_backward", "nsa_select_bwd_single", "nsa_decode",
    "nsa_forward_noalloc",
)
NOALLOC_SCRATCH_BYTES = 32 << 20


class NsaError(RuntimeError):
    pass


class NsaSaved(ctypes.Structure):
    """nsa_saved_t: the forward tensors the full backward reads."""
    _fields_ = [
        ("indices", ctypes.c_void_p), ("lse_sel", ctypes.c_void_p), ("lse_win", ctypes.c_void_p),
        ("lse_cmp", ctypes.c_void_p), ("o_sel", ctypes.c_void_p), ("o_win", ctypes.c_void_p),
        ("o_cmp", ctypes.c_void_p),
    ]


class NsaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("window", ctypes.c_int32), ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
    ]


_lib = None


def lib():
    """Load libnsa.so (raises NsaError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NsaError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_attention_long_compress_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(NsaParams)
        vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        L.nsa_abi_version.restype = ctypes.c_int
        L.nsa_status_string.argtypes = [ctypes.c_int]
        L.nsa_status_string.restype = ctypes.c_char_p
        L.nsa_check_params.argtypes = [P]
        L.nsa_check_params.restype = ctypes.c_int
        L.nsa_forward_kernel.argtypes = [P]
        L.nsa_forward_kernel.restype = ctypes.c_char_p
        L.nsa_workspace_size.argtypes = [P, ctypes.c_int]
        L.nsa_workspace_size.restype = ctypes.c_size_t
        L.nsa_pool.argtypes = [vp, vp, P, vp, vp, vp]
        L.nsa_pool.restype = ctypes.c_int
        L.nsa_compress_select.argtypes = [vp, vp, vp, P, vp, i32p, vp, ctypes.c_size_t, vp]
        L.nsa_compress_select.restype = ctypes.c_int
        L.nsa_forward.argtypes = [vp, vp, vp, vp, P, vp, i32p, f32p, vp, vp, ctypes.c_size_t, vp]
        L.nsa_forward.restype = ctypes.c_int
        L.nsa_forward_profile.argtypes = [vp, vp, vp, vp, P, vp, i32p, f32p, vp, vp,
                                          ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_void_p)]
        L.nsa_forward_profile.restype = ctypes.c_int
        L.nsa_forward_noalloc.argtypes = [vp, vp, vp, vp, P, vp, i32p, f32p, vp, vp]
        L.nsa_forward_noalloc.restype = ctypes.c_int
        L.nsa_select_bwd.argtypes = [vp, vp, vp, vp, i32p, f32p, vp, vp, P, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
        L.nsa_select_bwd.restype = ctypes.c_int
        L.nsa_select_bwd_single.argtypes = L.nsa_select_bwd.argtypes
        L.nsa_select_bwd_single.restype = ctypes.c_int
        S = ctypes.POINTER(NsaSaved)
        L.nsa_forward_train.argtypes = [vp, vp, vp, vp, P, vp, S, vp, ctypes.c_size_t, vp]
        L.nsa_forward_train.restype = ctypes.c_int
        L.nsa_backward.argtypes = [vp, vp, vp, vp, S, vp, P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.nsa_decode.restype = ctypes.c_int
        L.nsa_decode.argtypes = [vp, vp, vp, vp, vp, i32p, vp, P, vp, i32p, vp]
        L.nsa_backward.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().nsa_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise NsaError(f"{what}: {status_string(code)} ({code})")


def make_params(B, T, Hq, Hkv, D, *, top_k, window, dtype, scale=None, flags=0, block=64):
    return NsaParams(B, T, Hq, Hkv, D, block, top_k, window,
                     float(scale) if scale else 0.0, dtype, flags)


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return NSA_BF16
    if t.dtype == torch.float32:
        return NSA_FP32
    raise NsaError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise NsaError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def params_for(q, k, *, top_k, window, scale=None, flags=0):
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    return make_params(B, T, Hq, Hkv, D, top_k=top_k, window=window, dtype=_dtype_code(q),
                       scale=scale, flags=flags)


def forward_kernel(p: NsaParams) -> str:
    """Name of the selection/window/combine kernel nsa_forward runs for p
    (nsa_forward_kernel)."""
    name = lib().nsa_forward_kernel(ctypes.byref(p))
    if name is None:
        _check(lib().nsa_check_params(ctypes.byref(p)), "nsa_forward_kernel")
    return name.decode()


def workspace_size(p: NsaParams, backward=False) -> int:
    """backward: False (forward), True (selection backward), "full" (nsa_backward)
    or "single" (nsa_select_bwd_single)."""
    mode = {"full": 2, "single": 3}.get(backward, 1 if backward else 0)
    return int(lib().nsa_workspace_size(ctypes.byref(p), mode))


def alloc_workspace(p: NsaParams, device, backward=False):
    torch = _torch()
    n = workspace_size(p, backward)
    if n == 0:
        _check(lib().nsa_check_params(ctypes.byref(p)), "nsa_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def pool(k, v, *, stream=None):
    """Mean-pooled keys/values [B, T/64, Hkv, D] (nsa_pool)."""
    torch = _torch()
    B, T, Hkv, D = k.shape
    p = make_params(B, T, Hkv, Hkv, D, top_k=2, window=1, dtype=_dtype_code(k))
    kc = torch.empty((B, T // 64, Hkv, D), dtype=k.dtype, device=k.device)
    vc = torch.empty_like(kc)
    _check(lib().nsa_pool(_ptr(k), _ptr(v), ctypes.byref(p), _ptr(kc), _ptr(vc), _stream(stream)),
           "nsa_pool")
    return kc, vc


def compress_select(q, k, v, *, top_k, scale=None, workspace=None, stream=None):
    """(o_cmp [B,T,Hq,D], indices [B,Hkv,T,top_k]) from nsa_compress_select."""
    torch = _torch()
    p = params_for(q, k, top_k=top_k, window=1, scale=scale)
    ws = workspace if workspace is not None else alloc_workspace(p, q.device)
    o_cmp = torch.empty_like(q)
    idx = torch.empty((q.shape[0], k.shape[2], q.shape[1], top_k), dtype=torch.int32,
                      device=q.device)
    _check(lib().nsa_compress_select(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(p), _ptr(o_cmp),
                                     _ptr(idx), _ptr(ws), ws.numel(), _stream(stream)),
           "nsa_compress_select")
    return o_cmp, idx


def forward(q, k, v, gates, *, top_k, window, scale=None, flags=0, indices=None,
            want_indices=False, want_lse=False, want_o_sel=False, out=None, workspace=None,
            stream=None, events=None):
    """NSA forward (nsa_forward).  Returns a dict with 'out' and, when asked for,
    'indices', 'lse_sel', 'o_sel'.  With ``indices`` given, the INDICES_IN flag
    is set and that table replaces the top-k step.  ``events``: four raw
    hipEvent_t handles (ints or None) recorded around the three kernels
    (nsa_forward_profile)."""
    torch = _torch()
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if indices is not None:
        flags |= INDICES_IN
    p = params_for(q, k, top_k=top_k, window=window, scale=scale, flags=flags)
    ws = workspace if workspace is not None else alloc_workspace(p, q.device)
    res = {"out": out if out is not None else torch.empty_like(q)}
    idx = indices
    if idx is None and want_indices:
        idx = torch.empty((B, Hkv, T, top_k), dtype=torch.int32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if want_lse else None
    o_sel = torch.empty_like(q) if want_o_sel else None
    if events is None:
        _check(lib().nsa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), ctypes.byref(p),
                                 _ptr(res["out"]), _ptr(idx), _ptr(lse), _ptr(o_sel), _ptr(ws),
                                 ws.numel(), _stream(stream)), "nsa_forward")
    else:
        ev = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e) if e else None for e in events])
        _check(lib().nsa_forward_profile(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), ctypes.byref(p),
                                         _ptr(res["out"]), _ptr(idx), _ptr(lse), _ptr(o_sel),
                                         _ptr(ws), ws.numel(), _stream(stream), ev),
               "nsa_forward_profile")
    if idx is not None:
        res["indices"] = idx
    if lse is not None:
        res["lse_sel"] = lse
    if o_sel is not None:
        res["o_sel"] = o_sel
    return res


def forward_noalloc(q, k, v, gates, *, top_k, window, scale=None, flags=0, indices=None,
                    out, indices_out=None, lse_sel=None, o_sel=None, stream=None):
    """NSA forward without a workspace (nsa_forward_noalloc: the library's fixed
    per-GPU scratch array).  Every output tensor is the caller's: ``out`` and,
    as wanted, ``indices_out`` [B,Hkv,T,top_k] int32, ``lse_sel`` [B,Hq,T]
    fp32, ``o_sel``; ``indices`` given sets INDICES_IN.  Allocates nothing."""
    if indices is not None:
        flags |= INDICES_IN
        indices_out = indices
    p = params_for(q, k, top_k=top_k, window=window, scale=scale, flags=flags)
    _check(lib().nsa_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), ctypes.byref(p),
                                     _ptr(out), _ptr(indices_out), _ptr(lse_sel), _ptr(o_sel),
                                     _stream(stream)), "nsa_forward_noalloc")
    return out


def select_bwd(q, k, v, gates, indices, lse_sel, o_sel, dout, *, top_k, scale=None,
               workspace=None, stream=None, out=None):
    """(dq, dk, dv) of the selection branch (nsa_select_bwd); `out` may pass
    preallocated (dq, dk, dv)."""
    torch = _torch()
    p = params_for(q, k, top_k=top_k, window=1, scale=scale)
    ws = workspace if workspace is not None else alloc_workspace(p, q.device, backward=True)
    if out is not None:
        dq, dk, dv = out
    else:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
    _check(lib().nsa_select_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), _ptr(indices),
                                _ptr(lse_sel), _ptr(o_sel), _ptr(dout), ctypes.byref(p), _ptr(dq),
                                _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(stream)),
           "nsa_select_bwd")
    return dq, dk, dv


SAVED = ("indices", "lse_sel", "lse_win", "lse_cmp", "o_sel", "o_win", "o_cmp")


def _saved_struct(saved):
    return NsaSaved(*[_ptr(saved[n]) for n in SAVED])


def forward_train(q, k, v, gates, *, top_k, window, scale=None, indices=None, out=None,
                  workspace=None, stream=None):
    """NSA forward that also returns every tensor the full backward needs
    (nsa_forward_train): a dict with 'out' and the keys of SAVED."""
    torch = _torch()
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    flags = INDICES_IN if indices is not None else 0
    p = params_for(q, k, top_k=top_k, window=window, scale=scale, flags=flags)
    ws = workspace if workspace is not None else alloc_workspace(p, q.device)
    res = {"out": out if out is not None else torch.empty_like(q)}
    res["indices"] = indices if indices is not None else torch.empty(
        (B, Hkv, T, top_k), dtype=torch.int32, device=q.device)
    for n in ("lse_sel", "lse_win", "lse_cmp"):
        res[n] = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    for n in ("o_sel", "o_win", "o_cmp"):
        res[n] = torch.empty_like(q)
    sv = _saved_struct(res)
    _check(lib().nsa_forward_train(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), ctypes.byref(p),
                                   _ptr(res["out"]), ctypes.byref(sv), _ptr(ws), ws.numel(),
                                   _stream(stream)), "nsa_forward_train")
    return res


def backward(q, k, v, gates, saved, dout, *, top_k, window, scale=None, workspace=None,
             stream=None, out=None):
    """(dq, dk, dv, dgates) of the whole NSA output (nsa_backward); ``saved`` is
    the dict forward_train returned; ``out`` may pass preallocated tensors."""
    torch = _torch()
    p = params_for(q, k, top_k=top_k, window=window, scale=scale)
    ws = workspace if workspace is not None else alloc_workspace(p, q.device, backward="full")
    if out is not None:
        dq, dk, dv, dg = out
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dg = torch.empty_like(gates)
    sv = _saved_struct(saved)
    _check(lib().nsa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), ctypes.byref(sv), _ptr(dout),
                              ctypes.byref(p), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ws),
                              ws.numel(), _stream(stream)), "nsa_backward")
    return dq, dk, dv, dg


def select_bwd_single(q, k, v, gates, indices, lse_sel, o_sel, dout, *, top_k, scale=None,
                      workspace=None, stream=None, out=None):
    """(dq, dk, dv) of the selection branch in one query-stationary pass with
    fp32 atomics (nsa_select_bwd_single; bf16 only, not bitwise reproducible)."""
    torch = _torch()
    p = params_for(q, k, top_k=top_k, window=1, scale=scale)
    ws = workspace if workspace is not None else alloc_workspace(p, q.device, backward="single")
    if out is not None:
        dq, dk, dv = out
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib().nsa_select_bwd_single(_ptr(q), _ptr(k), _ptr(v), _ptr(gates), _ptr(indices),
                                       _ptr(lse_sel), _ptr(o_sel), _ptr(dout), ctypes.byref(p),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                                       _stream(stream)), "nsa_select_bwd_single")
    return dq, dk, dv


def decode(q, k_cache, v_cache, k_cmp, v_cmp, seq_lens, gates, *, top_k, window, scale=None,
           flags=0, want_indices=False, out=None, stream=None):
    """One decode step (nsa_decode): q [B, Hq, D]; caches [B, Lmax, Hkv, D];
    pooled caches [B, Lmax/64, Hkv, D]; seq_lens int32 [B] on the device; gates
    [B, Hq, 3].  Returns {'out': [B, Hq, D]} (+ 'indices' [B, Hkv, top_k])."""
    torch = _torch()
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    p = make_params(B, Lmax, Hq, Hkv, D, top_k=top_k, window=window, dtype=_dtype_code(q),
                    scale=scale, flags=flags)
    res = {"out": out if out is not None else torch.empty_like(q)}
    idx = None
    if want_indices:
        idx = torch.empty((B, Hkv, top_k), dtype=torch.int32, device=q.device)
        res["indices"] = idx
    if seq_lens.dtype != torch.int32:
        raise NsaError("seq_lens must be int32")
    _check(lib().nsa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cmp), _ptr(v_cmp),
                            _ptr(seq_lens), _ptr(gates), ctypes.byref(p), _ptr(res["out"]),
                            _ptr(idx), _stream(stream)), "nsa_decode")
    return res

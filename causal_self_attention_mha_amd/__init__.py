"""Fused causal multi-head self-attention for AMD MI355X (gfx950).

A thin Python binding (ctypes) over the C-ABI library libna_attn.so built from
csrc/ (see include/na_attn.h for the entry points).  This module only
marshals arguments: it checks dtypes, shapes, devices and contiguity, allocates
outputs with torch.empty on the tensors' device, and passes raw device pointers
plus torch's current HIP stream.  Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback, and every entry
point raises if the library is not built or no GPU is present.

Functions (names match the C entry points):
  attn_fwd(q, k, v)                       -> (o, lse)
  attn_bwd(q, k, v, o, dout, lse)         -> (dq, dk, dv)
                                          (return_delta=True: (dq, dk, dv, delta))
  attn_decode(q, k_cache, v_cache, seqlens) -> (o, lse)
  attn_decode_noalloc(q, k_cache, v_cache, seqlens) -> (o, lse)
                                          (no workspace: the library's fixed scratch)
  attn_decode_append(q, k_new, v_new, k_cache, v_cache, seqlens) -> (o, lse)
                                          (appends the new token's key/value rows first)
  attn_prefill(q, k_new, v_new, k_cache, v_cache, cache_lens) -> (o, lse)
                                          (appends k_new, v_new to the caches in place)
  qk_norm_rope_fwd(q, k, cos, sin)        -> (q_out, k_out)   (the prologue: RMS
                                          norm + rotary embedding of q and k)
  qk_norm_rope_bwd(q, k, dq_rot, dk_rot, cos, sin) -> (dq, dk)
  value_gate_fwd(v, ve, gate)             -> v + 3 sigmoid(gate) ve
  value_gate_bwd(ve, gate, dv_out)        -> (dve, dgate)   (dv is dv_out)
The attention calls take window=W (an int >= 0) for sliding-window attention
(key j visible to query i iff i - W <= j <= i), which calls the *_window entry
point; window=None is plain causal attention.  The prologue folds into
attn_prefill and attn_decode_append (rope=(cos, sin), value_gate=(ve, gate)),
into attn_fwd (rope=(cos, sin): q, k raw; returns o, lse and the rotated
q_rot, k_rot) and into attn_bwd (rope=(q_raw, k_raw, cos, sin): dq, dk of the
raw heads).  k and v (and the decode caches) may
have fewer heads than q (grouped-query attention, H a multiple of H_kv; the
*_gqa entry points); dk and dv then have the key/value heads' shape.
bf16 tensors use the bf16 kernels, float32 tensors the fp32 kernels
(forward and backward only).  Layouts: q, k, v, o, dout (B, T, H, 128);
lse, delta (B, H, T) float32; decode q/o (B, H, 128), caches (B, T_cap, H, 128),
seqlens int32 [B] on the device.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["attn_fwd", "attn_bwd", "attn_decode", "attn_decode_noalloc", "attn_decode_append",
           "attn_prefill",
           "qk_norm_rope_fwd",
           "qk_norm_rope_bwd", "value_gate_fwd", "value_gate_bwd", "decode_workspace_bytes",
           "bwd_workspace_bytes",
           "load_library",
           "library_path", "NAError", "HEAD_DIM"]

HEAD_DIM = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_STATUS = {0: "NA_OK", 1: "NA_ERR_INVALID_ARG", 2: "NA_ERR_UNSUPPORTED", 3: "NA_ERR_HIP"}


class NAError(RuntimeError):
    """A library call returned a non-zero na_status."""

    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}: {msg}")
        self.status = status


def library_path() -> str:
    """The in-tree libna_attn.so, or the build named by NA_ATTN_LIBRARY (the
    C-ABI tests use it to load the host-sanitized twin)."""
    return os.environ.get("NA_ATTN_LIBRARY") or os.path.join(_HERE, "lib", "libna_attn.so")


def load_library():
    """Load libna_attn.so (once).  torch is imported first so that the library
    binds to the HIP runtime torch already uses (one runtime per process)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (HIP runtime first; see docstring)
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m causal_self_attention_mha_amd.build` "
            "(hipcc, gfx950).  There is no fallback path.")
    lib = ctypes.CDLL(path)
    vp, i, f32p, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.na_attn_fwd.argtypes = [vp, vp, vp, vp, f32p, i, i, i, i, vp]
    lib.na_attn_bwd.argtypes = [vp, vp, vp, vp, vp, f32p, vp, vp, vp, f32p, vp, sz, i, i, i, i,
                                vp]
    lib.na_attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.na_attn_bwd_workspace_bytes.restype = sz
    lib.na_attn_decode.argtypes = [vp, vp, vp, vp, vp, f32p, i, i, i, i, vp, sz, vp]
    lib.na_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, f32p, i, i, i, i, vp]
    lib.na_attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.na_attn_decode_workspace_bytes.restype = sz
    lib.na_attn_fwd_f32.argtypes = [vp, vp, vp, vp, f32p, i, i, i, i, vp]
    lib.na_attn_bwd_f32.argtypes = [vp, vp, vp, vp, vp, f32p, vp, vp, vp, f32p, i, i, i, i, vp]
    lib.na_attn_bwd_timed.argtypes = lib.na_attn_bwd.argtypes + [vp]  # + events
    lib.na_attn_decode_timed.argtypes = lib.na_attn_decode.argtypes + [vp]
    lib.na_attn_fwd_window.argtypes = [vp, vp, vp, vp, f32p, i, i, i, i, i, vp]
    lib.na_attn_bwd_window.argtypes = lib.na_attn_bwd.argtypes[:-1] + [i, vp, vp]
    lib.na_attn_decode_window.argtypes = [vp, vp, vp, vp, vp, f32p, i, i, i, i, i, vp, sz, vp, vp]
    lib.na_attn_fwd_gqa.argtypes = [vp, vp, vp, vp, f32p, i, i, i, i, i, i, vp]
    lib.na_attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, f32p, vp, vp, vp, f32p, vp, sz, i, i, i,
                                    i, i, i, vp, vp]
    lib.na_attn_decode_gqa.argtypes = [vp, vp, vp, vp, vp, f32p, i, i, i, i, i, i, vp, sz, vp,
                                       vp]
    lib.na_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32p, i, i, i, i, i, i, i, vp]
    lib.na_qk_norm_rope_fwd.argtypes = [vp, vp, vp, vp, f32p, f32p, vp, i, i, i, i, i, i,
                                        ctypes.c_float, vp]
    lib.na_attn_prefill_rope.argtypes = [vp, vp, vp, vp, vp, vp, f32p, f32p, i, ctypes.c_float,
                                         vp, vp, vp, f32p, i, i, i, i, i, i, i, vp]
    lib.na_attn_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, f32p, f32p, i, ctypes.c_float,
                                          vp, vp, vp, f32p, i, i, i, i, i, i, vp, sz, vp]
    lib.na_attn_bwd_rope.argtypes = [vp, vp, vp, vp, vp, f32p, vp, vp, f32p, f32p, i,
                                     ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, f32p, vp, sz, i,
                                     i, i, i, i, i, vp]
    lib.na_attn_fwd_rope.argtypes = [vp, vp, vp, f32p, f32p, i, ctypes.c_float, vp, vp, vp,
                                     f32p, i, i, i, i, i, i, vp]
    lib.na_value_gate_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    lib.na_value_gate_bwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp]
    lib.na_qk_norm_rope_bwd.argtypes = [vp, vp, vp, vp, vp, vp, f32p, f32p, vp, i, i, i, i, i,
                                        i, ctypes.c_float, vp]
    for fn in ("na_attn_fwd", "na_attn_bwd", "na_attn_decode", "na_attn_fwd_f32",
               "na_attn_bwd_f32", "na_attn_bwd_timed", "na_attn_decode_timed",
               "na_attn_fwd_window", "na_attn_bwd_window", "na_attn_decode_window",
               "na_attn_fwd_gqa", "na_attn_bwd_gqa", "na_attn_decode_gqa", "na_attn_prefill",
               "na_qk_norm_rope_fwd", "na_qk_norm_rope_bwd", "na_value_gate_fwd",
               "na_value_gate_bwd", "na_attn_prefill_rope", "na_attn_decode_append",
               "na_attn_bwd_rope", "na_attn_decode_noalloc", "na_attn_fwd_rope"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.na_status_string.argtypes = [ctypes.c_int]
    lib.na_status_string.restype = ctypes.c_char_p
    lib.na_last_error.argtypes = []
    lib.na_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(lib, fn, status):
    if status != 0:
        raise NAError(fn, status, lib.na_last_error().decode())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_train(names, tensors, dtype=None, kv_heads=None):
    """Same dtype, device, contiguity and (B, T, H, 128) shape as the first
    tensor; tensors named in kv_heads may instead have H_kv heads."""
    import torch
    ref = tensors[0]
    _require(ref.is_cuda, f"{names[0]} must be a GPU tensor (no CPU path)")
    _require(ref.dim() == 4 and ref.shape[-1] == HEAD_DIM,
             f"{names[0]} must be (B, T, H, {HEAD_DIM}), got {tuple(ref.shape)}")
    dtype = dtype or ref.dtype
    _require(dtype in (torch.bfloat16, torch.float32), f"unsupported dtype {dtype}")
    for n, t in zip(names, tensors):
        _require(t.dtype == dtype, f"{n} has dtype {t.dtype}, expected {dtype}")
        want = tuple(ref.shape)
        if kv_heads is not None and n in kv_heads:
            want = want[:2] + (kv_heads[n],) + want[3:]
        _require(tuple(t.shape) == want, f"{n} has shape {tuple(t.shape)}, expected {want}")
        _require(t.device == ref.device, f"{n} is on {t.device}, expected {ref.device}")
        _require(t.is_contiguous(), f"{n} must be contiguous")
    return dtype


def _check_buf(name, t, dtype, shape, device):
    """A caller-supplied output or scratch tensor: exact dtype, shape and
    device, contiguous.  Anything else would hand the kernels a host pointer
    or a buffer of the wrong size."""
    _require(t.device == device, f"{name} is on {t.device}, expected {device}")
    _require(t.dtype == dtype, f"{name} has dtype {t.dtype}, expected {dtype}")
    _require(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, "
             f"expected {tuple(shape)}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def _check_workspace(t, need, device):
    """A caller-supplied byte workspace: contiguous, on the device, at least
    `need` bytes.  Returns its size in bytes."""
    _require(t.device == device, f"workspace is on {t.device}, expected {device}")
    _require(t.is_contiguous(), "workspace must be contiguous")
    nbytes = t.numel() * t.element_size()
    _require(nbytes >= need, f"workspace has {nbytes} bytes, needs {need}")
    return nbytes


def _window(window):
    if window is None:
        return None
    _require(int(window) == window and window >= 0, f"window must be an int >= 0, got {window}")
    return int(window)


def _kv_heads(q, k):
    _require(k.dim() == 4, f"k must be (B, T, H_kv, {HEAD_DIM}), got {tuple(k.shape)}")
    H, Hk = q.shape[2], k.shape[2]
    _require(Hk >= 1 and H % Hk == 0, f"q has {H} heads, not a multiple of k's {Hk}")
    return Hk


def attn_fwd(q, k, v, o=None, lse=None, window=None, rope=None, eps=1e-6, q_rot=None,
             k_rot=None):
    """Causal attention forward.  Returns (o, lse): o like q, lse float32 (B, H, T).

    rope=(cos, sin), float32 (T_tab >= T, 64) tables: q and k are the raw
    query and key heads, normalised and rotated inside the call
    (na_attn_fwd_rope: the keys by the prologue kernel, the queries as the
    forward loads them); returns (o, lse, q_rot, k_rot), the rotated heads
    being the q and k that attn_bwd takes (with rope=(q, k, cos, sin))."""
    import torch
    lib = load_library()
    Hk = _kv_heads(q, k)
    dtype = _check_train(("q", "k", "v"), (q, k, v), kv_heads={"k": Hk, "v": Hk})
    B, T, H, D = q.shape
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_train(("q", "o"), (q, o), dtype)
    _check_buf("lse", lse, torch.float32, (B, H, T), q.device)
    window = _window(window)
    if rope is not None:
        cos, sin = rope
        _require(dtype == torch.bfloat16, "rope: bf16 tensors only")
        _check_prologue(q, k, cos, sin, None)
        q_rot = torch.empty_like(q) if q_rot is None else q_rot
        k_rot = torch.empty_like(k) if k_rot is None else k_rot
        _check_buf("q_rot", q_rot, torch.bfloat16, q.shape, q.device)
        _check_buf("k_rot", k_rot, torch.bfloat16, k.shape, q.device)
        _check(lib, "na_attn_fwd_rope",
               lib.na_attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(cos), _ptr(sin),
                                    cos.shape[0], float(eps), _ptr(q_rot), _ptr(k_rot), _ptr(o),
                                    _ptr(lse), B, T, H, Hk, D,
                                    -1 if window is None else window, _stream(q)))
        return o, lse, q_rot, k_rot
    if Hk != H or window is not None:
        _require(dtype == torch.bfloat16, "window / grouped heads: bf16 tensors only")
        w = -1 if window is None else window
        if Hk != H:
            _check(lib, "na_attn_fwd_gqa",
                   lib.na_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, H,
                                       Hk, D, w, _stream(q)))
        else:
            _check(lib, "na_attn_fwd_window",
                   lib.na_attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T,
                                          H, D, w, _stream(q)))
        return o, lse
    fn = "na_attn_fwd" if dtype == torch.bfloat16 else "na_attn_fwd_f32"
    _check(lib, fn, getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, H, D,
                                     _stream(q)))
    return o, lse


def bwd_workspace_bytes(B, T, H, D=HEAD_DIM):
    return int(load_library().na_attn_bwd_workspace_bytes(B, T, H, D))


def attn_bwd(q, k, v, o, dout, lse, dq=None, dk=None, dv=None, delta=None, workspace=None,
             recompute_dq=False, window=None, rope=None, eps=1e-6, return_delta=False,
             value_gate=None):
    """Causal attention backward.  Returns (dq, dk, dv), or (dq, dk, dv, delta)
    with return_delta=True (delta = rowsum(dout * o), the preprocess's (B, H, T)
    fp32 output, allocated here unless given).

    bf16: by default a dS workspace is allocated (or `workspace` is used) so
    that dq is a GEMM over the stored dS; recompute_dq=True passes no
    workspace and the dq pass recomputes S and dP (with or without a
    window).  fp32 has one path.
    rope=(q_raw, k_raw, cos, sin): q and k are the outputs of
    qk_norm_rope_fwd(q_raw, k_raw, cos, sin); dq and dk are returned as the
    gradients of q_raw and k_raw, the prologue's backward done in the same
    kernels (na_attn_bwd_rope).
    value_gate=(ve, gate) (with rope): v is value_gate_fwd(v_in, ve, gate); the
    kernel that writes dv also writes the gate's gradients, and (dve, dgate)
    follow dv in the result (dv is the gradient of v_in as well)."""
    import torch
    lib = load_library()
    Hk = _kv_heads(q, k)
    kvh = {"k": Hk, "v": Hk}
    dtype = _check_train(("q", "k", "v", "o", "dout"), (q, k, v, o, dout), kv_heads=kvh)
    B, T, H, D = q.shape
    _check_buf("lse", lse, torch.float32, (B, H, T), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if delta is None else delta
    _check_train(("q", "dq", "dk", "dv"), (q, dq, dk, dv), dtype,
                 kv_heads={"dk": Hk, "dv": Hk})
    _check_buf("delta", delta, torch.float32, (B, H, T), q.device)
    window = _window(window)
    _require((window is None and Hk == H) or dtype == torch.bfloat16,
             "window / grouped heads: bf16 tensors only")
    if dtype == torch.bfloat16:
        ws_bytes = 0
        if not recompute_dq:
            ws_bytes = bwd_workspace_bytes(B, T, H, D)
            if workspace is None:
                workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            else:
                ws_bytes = _check_workspace(workspace, ws_bytes, q.device)
        else:
            workspace = None
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                _ptr(dv), _ptr(delta), _ptr(workspace), ws_bytes)
        w = -1 if window is None else window
        _require(value_gate is None or rope is not None, "value_gate folds in with rope only")
        if rope is not None:
            q_raw, k_raw, cos, sin = rope
            _require(workspace is not None, "rope needs the dS workspace (recompute_dq=False)")
            ve = gate = dve = dgate = None
            if value_gate is not None:
                ve, gate = value_gate
                _check_value_gate(("v", "ve"), (v, ve), gate)
                dve, dgate = torch.empty_like(ve), torch.empty_like(gate)
            _check_train(("q", "q_raw", "k_raw"), (q, q_raw, k_raw), dtype, kv_heads={"k_raw": Hk})
            for n, t in (("cos", cos), ("sin", sin)):
                _require(t.dtype == torch.float32 and t.device == q.device and t.is_contiguous()
                         and t.dim() == 2 and t.shape[1] == D // 2 and t.shape == cos.shape
                         and t.shape[0] >= T, f"{n} must be contiguous float32 (T_tab >= T, 64)")
            _check(lib, "na_attn_bwd_rope",
                   lib.na_attn_bwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                        _ptr(q_raw), _ptr(k_raw), _ptr(cos), _ptr(sin),
                                        cos.shape[0], float(eps), _ptr(ve), _ptr(gate), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(dve), _ptr(dgate), _ptr(delta),
                                        _ptr(workspace), ws_bytes, B, T, H, Hk, D, w, _stream(q)))
            if value_gate is not None:
                out = (dq, dk, dv, dve, dgate)
                return out + (delta,) if return_delta else out
        elif Hk != H:
            _check(lib, "na_attn_bwd_gqa",
                   lib.na_attn_bwd_gqa(*args, B, T, H, Hk, D, w, _stream(q), None))
        elif window is not None:
            _check(lib, "na_attn_bwd_window",
                   lib.na_attn_bwd_window(*args, B, T, H, D, w, _stream(q), None))
        else:
            _check(lib, "na_attn_bwd", lib.na_attn_bwd(*args, B, T, H, D, _stream(q)))
    else:
        _check(lib, "na_attn_bwd_f32",
               lib.na_attn_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), B, T, H, D,
                                   _stream(q)))
    return (dq, dk, dv, delta) if return_delta else (dq, dk, dv)


def decode_workspace_bytes(B, H, T_cap, D=HEAD_DIM):
    return int(load_library().na_attn_decode_workspace_bytes(B, H, D, T_cap))


def attn_decode(q, k_cache, v_cache, seqlens, o=None, lse=None, workspace=None,
                want_lse=True, window=None):
    """Single-token decode over a padded cache.  Returns (o, lse)."""
    import torch
    lib = load_library()
    _require(q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[-1] == HEAD_DIM,
             "q must be a bf16 GPU tensor (B, H, 128)")
    B, H, D = q.shape
    _require(k_cache.dim() == 4 and k_cache.shape[0] == B and k_cache.shape[3] == D
             and k_cache.shape[2] >= 1 and H % k_cache.shape[2] == 0,
             "k_cache must be (B, T_cap, H_kv, 128) with H a multiple of H_kv")
    T_cap, Hk = k_cache.shape[1], k_cache.shape[2]
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == torch.bfloat16 and t.device == q.device and t.is_contiguous(),
                 f"{n} must be contiguous bf16 on {q.device}")
    _require(v_cache.shape == k_cache.shape, "v_cache must match k_cache")
    _require(seqlens.dtype == torch.int32 and seqlens.shape == (B,) and seqlens.device == q.device
             and seqlens.is_contiguous(), "seqlens must be int32 [B] on the GPU")
    o = torch.empty_like(q) if o is None else o
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_buf("o", o, torch.bfloat16, (B, H, D), q.device)
    if lse is not None:
        _check_buf("lse", lse, torch.float32, (B, H), q.device)
    need = decode_workspace_bytes(B, H, T_cap, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    window = _window(window)
    ws_bytes = _check_workspace(workspace, need, q.device)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse))
    w = -1 if window is None else window
    if Hk != H:
        _check(lib, "na_attn_decode_gqa",
               lib.na_attn_decode_gqa(*args, B, H, Hk, D, T_cap, w, _ptr(workspace), ws_bytes,
                                      _stream(q), None))
    elif window is not None:
        _check(lib, "na_attn_decode_window",
               lib.na_attn_decode_window(*args, B, H, D, T_cap, w, _ptr(workspace), ws_bytes,
                                         _stream(q), None))
    else:
        _check(lib, "na_attn_decode",
               lib.na_attn_decode(*args, B, H, D, T_cap, _ptr(workspace), ws_bytes, _stream(q)))
    return o, lse


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, o=None, lse=None, want_lse=True):
    """attn_decode through na_attn_decode_noalloc: no workspace, the split-KV
    partials go to the library's fixed 16 MiB per-device scratch (sizes that
    need more raise NAError).  Calls on one device share that scratch, so
    calls that may overlap on different streams race.  Returns (o, lse)."""
    import torch
    lib = load_library()
    _require(q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[-1] == HEAD_DIM,
             "q must be a bf16 GPU tensor (B, H, 128)")
    B, H, D = q.shape
    _require(k_cache.dim() == 4 and tuple(k_cache.shape[2:]) == (H, D) and k_cache.shape[0] == B,
             "k_cache must be (B, T_cap, H, 128)")
    T_cap = k_cache.shape[1]
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t.dtype == torch.bfloat16 and t.device == q.device and t.is_contiguous(),
                 f"{n} must be contiguous bf16 on {q.device}")
    _require(v_cache.shape == k_cache.shape, "v_cache must match k_cache")
    _require(seqlens.dtype == torch.int32 and seqlens.shape == (B,) and seqlens.device == q.device
             and seqlens.is_contiguous(), "seqlens must be int32 [B] on the GPU")
    o = torch.empty_like(q) if o is None else o
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_buf("o", o, torch.bfloat16, (B, H, D), q.device)
    if lse is not None:
        _check_buf("lse", lse, torch.float32, (B, H), q.device)
    _check(lib, "na_attn_decode_noalloc",
           lib.na_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens),
                                      _ptr(o), _ptr(lse), B, H, D, T_cap, _stream(q)))
    return o, lse


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, seqlens, o=None, lse=None,
                       workspace=None, want_lse=True, window=None, rope=None, eps=1e-6,
                       value_gate=None):
    """Decode step with the append: writes k_new, v_new (B, H_kv, 128) at row
    seqlens[b] of the caches (in place; seqlens is not updated), then the
    query attends over rows 0 .. seqlens[b].  rope=(cos, sin) float32
    (T_tab >= T_cap, 64): q and k_new are raw heads, normalised and rotated
    at that position; value_gate=(ve, gate): the appended value row is
    v_new + 3 sigmoid(gate) ve.  Returns (o, lse)."""
    import torch
    lib = load_library()
    _require(q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[-1] == HEAD_DIM,
             "q must be a bf16 GPU tensor (B, H, 128)")
    B, H, D = q.shape
    _require(k_cache.dim() == 4 and k_cache.shape[0] == B and k_cache.shape[3] == D
             and k_cache.shape[2] >= 1 and H % k_cache.shape[2] == 0,
             "k_cache must be (B, T_cap, H_kv, 128) with H a multiple of H_kv")
    T_cap, Hk = k_cache.shape[1], k_cache.shape[2]
    for n, t, shape in (("q", q, q.shape), ("k_new", k_new, (B, Hk, D)),
                        ("v_new", v_new, (B, Hk, D)), ("k_cache", k_cache, k_cache.shape),
                        ("v_cache", v_cache, k_cache.shape)):
        _require(t.dtype == torch.bfloat16 and t.device == q.device and t.is_contiguous()
                 and tuple(t.shape) == tuple(shape), f"{n} must be contiguous bf16 {tuple(shape)}")
    _require(seqlens.dtype == torch.int32 and seqlens.shape == (B,) and seqlens.device == q.device
             and seqlens.is_contiguous(), "seqlens must be int32 [B] on the GPU")
    cos = sin = ve = gate = None
    if rope is not None:
        cos, sin = rope
        for n, t in (("cos", cos), ("sin", sin)):
            _require(t.dtype == torch.float32 and t.device == q.device and t.is_contiguous()
                     and t.dim() == 2 and t.shape[1] == D // 2 and t.shape == cos.shape
                     and t.shape[0] >= T_cap, f"{n} must be contiguous float32 (T_tab >= T_cap, 64)")
    if value_gate is not None:
        ve, gate = value_gate
        _require(ve.dtype == torch.bfloat16 and tuple(ve.shape) == (B, Hk, D)
                 and ve.is_contiguous() and ve.device == q.device, "ve must be bf16 (B, H_kv, 128)")
        _require(gate.dtype == torch.bfloat16 and tuple(gate.shape) == (B, Hk)
                 and gate.is_contiguous() and gate.device == q.device, "gate must be bf16 (B, H_kv)")
    o = torch.empty_like(q) if o is None else o
    if want_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_buf("o", o, torch.bfloat16, (B, H, D), q.device)
    if lse is not None:
        _check_buf("lse", lse, torch.float32, (B, H), q.device)
    need = decode_workspace_bytes(B, H, T_cap, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    window = _window(window)
    _check(lib, "na_attn_decode_append",
           lib.na_attn_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(seqlens), _ptr(cos), _ptr(sin),
                                     0 if cos is None else cos.shape[0], float(eps), _ptr(ve),
                                     _ptr(gate), _ptr(o), _ptr(lse), B, H, Hk, D, T_cap,
                                     -1 if window is None else window, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(q)))
    return o, lse


def attn_prefill(q, k_new, v_new, k_cache, v_cache, cache_lens, o=None, lse=None,
                 want_lse=True, window=None, rope=None, eps=1e-6, value_gate=None):
    """Prefill a chunk over a KV cache: appends k_new, v_new at rows
    cache_lens[b] .. of the caches (in place), then the chunk's queries attend
    bottom-right causally over the cache.  Returns (o, lse); cache_lens is not
    updated.  rope=(cos, sin), float32 (T_tab >= T_cap, 64) tables: q and
    k_new are raw heads, RMS-normalised and rotated at their cache positions
    inside the call (na_attn_prefill_rope); with it, value_gate=(ve, gate)
    (bf16 (B, T_q, H_kv, 128) and (B, T_q, H_kv)) appends
    v_new + 3 sigmoid(gate) ve instead of v_new."""
    import torch
    lib = load_library()
    _require(q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 4 and q.shape[-1] == HEAD_DIM,
             "q must be a bf16 GPU tensor (B, T_q, H, 128)")
    B, T_q, H, D = q.shape
    _require(k_new.dim() == 4 and k_new.shape[:2] == (B, T_q) and k_new.shape[3] == D,
             "k_new must be (B, T_q, H_kv, 128)")
    Hk = k_new.shape[2]
    _require(Hk >= 1 and H % Hk == 0, f"q has {H} heads, not a multiple of k_new's {Hk}")
    _require(k_cache.dim() == 4 and k_cache.shape[0] == B and k_cache.shape[2:] == (Hk, D)
             and k_cache.shape[1] >= T_q, "k_cache must be (B, T_cap >= T_q, H_kv, 128)")
    for n, t, shape in (("q", q, q.shape), ("k_new", k_new, k_new.shape),
                        ("v_new", v_new, k_new.shape), ("k_cache", k_cache, k_cache.shape),
                        ("v_cache", v_cache, k_cache.shape)):
        _require(t.dtype == torch.bfloat16 and t.device == q.device and t.is_contiguous()
                 and t.shape == shape, f"{n} must be contiguous bf16 {tuple(shape)} on {q.device}")
    _require(cache_lens.dtype == torch.int32 and cache_lens.shape == (B,)
             and cache_lens.device == q.device and cache_lens.is_contiguous(),
             "cache_lens must be int32 [B] on the GPU")
    T_cap = k_cache.shape[1]
    o = torch.empty_like(q) if o is None else o
    if want_lse and lse is None:
        lse = torch.empty((B, H, T_q), dtype=torch.float32, device=q.device)
    _check_buf("o", o, torch.bfloat16, (B, T_q, H, D), q.device)
    if lse is not None:
        _check_buf("lse", lse, torch.float32, (B, H, T_q), q.device)
    window = _window(window)
    w = -1 if window is None else window
    _require(value_gate is None or rope is not None, "value_gate is taken with rope only")
    if rope is not None:
        cos, sin = rope
        for n, t in (("cos", cos), ("sin", sin)):
            _require(t.dtype == torch.float32 and t.device == q.device and t.is_contiguous()
                     and t.dim() == 2 and t.shape[1] == D // 2 and t.shape == cos.shape
                     and t.shape[0] >= T_cap, f"{n} must be contiguous float32 (T_tab >= T_cap, 64)")
        ve = gate = None
        if value_gate is not None:
            ve, gate = value_gate
            _require(ve.dtype == torch.bfloat16 and ve.shape == k_new.shape and ve.is_contiguous()
                     and ve.device == q.device, "ve must be contiguous bf16 like k_new")
            _require(gate.dtype == torch.bfloat16 and tuple(gate.shape) == tuple(k_new.shape[:3])
                     and gate.is_contiguous() and gate.device == q.device,
                     "gate must be contiguous bf16 (B, T_q, H_kv)")
        _check(lib, "na_attn_prefill_rope",
               lib.na_attn_prefill_rope(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(cache_lens), _ptr(cos), _ptr(sin),
                                        cos.shape[0], float(eps), _ptr(ve), _ptr(gate), _ptr(o),
                                        _ptr(lse), B, T_q, H, Hk, D, T_cap, w, _stream(q)))
        return o, lse
    _check(lib, "na_attn_prefill",
           lib.na_attn_prefill(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                               _ptr(cache_lens), _ptr(o), _ptr(lse), B, T_q, H, Hk, D, T_cap,
                               w, _stream(q)))
    return o, lse


def _check_prologue(q, k, cos, sin, pos_offset, extra=()):
    import torch
    _require(q.is_cuda and q.dtype == torch.bfloat16 and q.dim() == 4 and q.shape[-1] == HEAD_DIM,
             "q must be a bf16 GPU tensor (B, T, H, 128)")
    B, T, H, D = q.shape
    _require(k.dim() == 4 and k.shape[:2] == (B, T) and k.shape[3] == D,
             "k must be (B, T, H_kv, 128)")
    for n, t, shape in (("q", q, q.shape), ("k", k, k.shape)) + tuple(extra):
        _require(t.dtype == torch.bfloat16 and t.device == q.device and t.is_contiguous()
                 and t.shape == shape, f"{n} must be contiguous bf16 {tuple(shape)} on {q.device}")
    _require(cos.dim() == 2 and cos.shape[1] == D // 2 and cos.shape[0] >= T,
             "cos must be (T_tab >= T, 64)")
    for n, t in (("cos", cos), ("sin", sin)):
        _require(t.dtype == torch.float32 and t.device == q.device and t.is_contiguous()
                 and t.shape == cos.shape, f"{n} must be contiguous float32 {tuple(cos.shape)}")
    if pos_offset is not None:
        _require(pos_offset.dtype == torch.int32 and pos_offset.shape == (B,)
                 and pos_offset.device == q.device and pos_offset.is_contiguous(),
                 "pos_offset must be int32 [B] on the GPU")
    return B, T, H, k.shape[2], D, cos.shape[0]


def qk_norm_rope_fwd(q, k, cos, sin, pos_offset=None, eps=1e-6, q_out=None, k_out=None):
    """RMS-normalise each head row of q and k, then rotate the pairs (i, i + 64)
    by the angles whose cos/sin tables (T_tab, 64) float32 are given, at
    positions t + pos_offset[b] (pos_offset int32 [B], clamped on the device
    to [0, T_tab - T]; None for positions t).  Returns (q_out, k_out)."""
    import torch
    lib = load_library()
    B, T, H, Hk, D, T_tab = _check_prologue(q, k, cos, sin, pos_offset)
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _check_buf("q_out", q_out, torch.bfloat16, q.shape, q.device)
    _check_buf("k_out", k_out, torch.bfloat16, k.shape, q.device)
    _check(lib, "na_qk_norm_rope_fwd",
           lib.na_qk_norm_rope_fwd(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(cos), _ptr(sin),
                                   _ptr(pos_offset), B, T, H, Hk, D, T_tab, float(eps),
                                   _stream(q)))
    return q_out, k_out


def qk_norm_rope_bwd(q, k, dq_rot, dk_rot, cos, sin, pos_offset=None, eps=1e-6, dq=None,
                     dk=None):
    """Gradients of q and k through qk_norm_rope_fwd, given the gradients
    dq_rot, dk_rot of its outputs.  Returns (dq, dk)."""
    import torch
    lib = load_library()
    B, T, H, Hk, D, T_tab = _check_prologue(
        q, k, cos, sin, pos_offset, (("dq_rot", dq_rot, q.shape), ("dk_rot", dk_rot, k.shape)))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    _check_buf("dq", dq, torch.bfloat16, q.shape, q.device)
    _check_buf("dk", dk, torch.bfloat16, k.shape, q.device)
    _check(lib, "na_qk_norm_rope_bwd",
           lib.na_qk_norm_rope_bwd(_ptr(q), _ptr(k), _ptr(dq_rot), _ptr(dk_rot), _ptr(dq), _ptr(dk),
                                   _ptr(cos), _ptr(sin), _ptr(pos_offset), B, T, H, Hk, D, T_tab,
                                   float(eps), _stream(q)))
    return dq, dk


def _check_value_gate(names, rows, gate):
    import torch
    ref = rows[0]
    _require(ref.is_cuda and ref.dtype == torch.bfloat16 and ref.dim() == 4
             and ref.shape[-1] == HEAD_DIM, f"{names[0]} must be a bf16 GPU tensor "
             "(B, T, H_kv, 128)")
    for n, t in zip(names, rows):
        _require(t.dtype == torch.bfloat16 and t.device == ref.device and t.is_contiguous()
                 and t.shape == ref.shape, f"{n} must be contiguous bf16 {tuple(ref.shape)}")
    _require(gate.dtype == torch.bfloat16 and gate.device == ref.device and gate.is_contiguous()
             and tuple(gate.shape) == tuple(ref.shape[:3]),
             f"gate must be contiguous bf16 {tuple(ref.shape[:3])}")
    return tuple(ref.shape)


def value_gate_fwd(v, ve, gate, v_out=None):
    """v + 3 sigmoid(gate) ve for v, ve (B, T, H_kv, 128) bf16 and gate
    logits (B, T, H_kv) bf16."""
    import torch
    lib = load_library()
    B, T, Hk, D = _check_value_gate(("v", "ve"), (v, ve), gate)
    v_out = torch.empty_like(v) if v_out is None else v_out
    _check_buf("v_out", v_out, torch.bfloat16, v.shape, v.device)
    _check(lib, "na_value_gate_fwd",
           lib.na_value_gate_fwd(_ptr(v), _ptr(ve), _ptr(gate), _ptr(v_out), B, T, Hk, D,
                                 _stream(v)))
    return v_out


def value_gate_bwd(ve, gate, dv_out, dve=None, dgate=None):
    """Gradients through value_gate_fwd given dv_out: returns (dve, dgate); the
    gradient of v is dv_out itself."""
    import torch
    lib = load_library()
    B, T, Hk, D = _check_value_gate(("ve", "dv_out"), (ve, dv_out), gate)
    dve = torch.empty_like(ve) if dve is None else dve
    dgate = torch.empty_like(gate) if dgate is None else dgate
    _check_buf("dve", dve, torch.bfloat16, ve.shape, ve.device)
    _check_buf("dgate", dgate, torch.bfloat16, gate.shape, ve.device)
    _check(lib, "na_value_gate_bwd",
           lib.na_value_gate_bwd(_ptr(ve), _ptr(gate), _ptr(dv_out), _ptr(dve), _ptr(dgate), B, T,
                                 Hk, D, _stream(ve)))
    return dve, dgate

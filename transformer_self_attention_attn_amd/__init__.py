"""Python binding of libmiattn (argument marshalling only).

Every step of attention runs in the HIP kernels of libmiattn.so; this module
only turns torch tensors into device pointers, sizes and the current HIP
stream, and raises on a non-OK status.  There is no fallback: if the library
is not built, importing the binding's entry points raises.

Entry points with the C names (raw pointers as Python ints):
    attn_fwd, attn_fwd_f32, attn_fwd_masked, attn_fwd_masked_f32,
    attn_bwd, attn_fp8_quantize, attn_fwd_fp8,
    attn_last_error, attn_release
Convenience wrappers on torch tensors:
    attn(q, k, v, causal=False, window=0, seqlens=None, scale=None,
         window_right=0, sinks=0), attn_backward, fp8_quantize, attn_fp8
"""

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmiattn.so")

MIATTN_OK = 0
MIATTN_ERR_INVALID = -1
MIATTN_ERR_UNSUPPORTED = -2
MIATTN_ERR_HIP = -3
MIATTN_ERR_NOMEM = -4

EXPORTS = ("attn_fwd", "attn_fwd_f32", "attn_fwd_masked",
           "attn_fwd_masked_f32", "attn_bwd",
           "attn_fp8_quantize", "attn_fwd_fp8", "attn_last_error",
           "attn_release")

_lib = None


class MiattnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"miattn status {status}: {msg}")
        self.status = status


def load():
    """Load libmiattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp, vp]
    lib.attn_fwd.argtypes = sig
    lib.attn_fwd.restype = ci
    lib.attn_fwd_f32.argtypes = sig
    lib.attn_fwd_f32.restype = ci
    msig = sig[:14] + [ci, ci] + sig[14:]
    lib.attn_fwd_masked.argtypes = msig
    lib.attn_fwd_masked.restype = ci
    lib.attn_fwd_masked_f32.argtypes = msig
    lib.attn_fwd_masked_f32.restype = ci
    lib.attn_bwd.argtypes = [vp] * 9 + [ci] * 6 + [cf] + [ci] * 4 + [vp, vp]
    lib.attn_bwd.restype = ci
    lib.attn_fp8_quantize.argtypes = [vp] * 3 + [ci] * 6 + [vp, vp, ci] + \
        [vp] * 7
    lib.attn_fp8_quantize.restype = ci
    lib.attn_fwd_fp8.argtypes = [vp] * 8 + [ci] * 6 + [cf] + [ci] * 5 + \
        [vp, vp]
    lib.attn_fwd_fp8.restype = ci
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_release.argtypes = []
    lib.attn_release.restype = None
    _lib = lib
    return lib


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
             seqlens, stream):
    """Direct call of the C entry point; pointers are ints (0 = NULL)."""
    return load().attn_fwd(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nk, d,
                           scale, int(causal), window, seqlens or None,
                           stream or None)


def attn_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                 window, seqlens, stream):
    return load().attn_fwd_f32(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nk,
                               d, scale, int(causal), window, seqlens or None,
                               stream or None)


def attn_fwd_masked(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                    window_left, window_right, sinks, seqlens, stream):
    return load().attn_fwd_masked(q, k, v, o, lse or None, B, Hq, Hkv, Nq,
                                  Nk, d, scale, int(causal), window_left,
                                  window_right, sinks, seqlens or None,
                                  stream or None)


def attn_fwd_masked_f32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                        causal, window_left, window_right, sinks, seqlens,
                        stream):
    return load().attn_fwd_masked_f32(q, k, v, o, lse or None, B, Hq, Hkv,
                                      Nq, Nk, d, scale, int(causal),
                                      window_left, window_right, sinks,
                                      seqlens or None, stream or None)


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
             causal, window_left, window_right, sinks, seqlens, stream):
    return load().attn_bwd(q, k, v, o, dout, lse or None, dq, dk, dv, B, Hq,
                           Hkv, Nq, Nk, d, scale, int(causal), window_left,
                           window_right, sinks, seqlens or None,
                           stream or None)


def attn_fp8_quantize(q, k, v, B, Hq, Hkv, Nq, Nk, d, seqlens, signs,
                      per_tensor, q8, sq, k8, sk, v8t, sv, stream):
    return load().attn_fp8_quantize(q, k, v, B, Hq, Hkv, Nq, Nk, d,
                                    seqlens or None, signs or None,
                                    int(per_tensor), q8, sq, k8, sk, v8t,
                                    sv, stream or None)


def attn_fwd_fp8(q8, sq, k8, sk, v8t, sv, o, lse, B, Hq, Hkv, Nq, Nk, d,
                 scale, rotated, causal, window_left, window_right, sinks,
                 seqlens, stream):
    return load().attn_fwd_fp8(q8, sq, k8, sk, v8t, sv, o, lse or None, B,
                               Hq, Hkv, Nq, Nk, d, scale, int(rotated),
                               int(causal), window_left, window_right, sinks,
                               seqlens or None, stream or None)


def attn_last_error():
    return load().attn_last_error().decode()


def attn_release():
    load().attn_release()


def _need(t, name, dtype, shape, device):
    """Raises ValueError unless tensor `t` has this dtype and shape, is
    contiguous and lives on `device`: the kernels read or write exactly that
    many elements at that address."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got "
                         f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _seqlens_ptr(seqlens, B, device):
    """Device address of an int32 [B] valid-length tensor (0 for None)."""
    import torch
    if seqlens is None:
        return 0
    _need(seqlens, "seqlens", torch.int32, (B,), device)
    return seqlens.data_ptr()


def _check_qkv(q, k, v, dtypes, require_gpu=True):
    """(B, Hq, Hkv, Nq, Nk, d) of q [B,Hq,Nq,d] and k, v [B,Hkv,Nk,d], after
    checking that they share one dtype out of `dtypes`, are contiguous 4-d
    tensors on one device (a GPU unless require_gpu is False) and agree in
    B and d."""
    if q.dtype not in dtypes:
        raise TypeError(f"q must be one of {dtypes}, got {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    if require_gpu and not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or \
            k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k "
                         f"{tuple(k.shape)}, v {tuple(v.shape)}")
    return B, Hq, Hkv, Nq, Nk, d


def check_attn_args(q, k, v, out=None, lse=None, seqlens=None,
                    require_gpu=True):
    """The checks `attn` makes before any launch: q, k, v as in _check_qkv
    (bfloat16 or float32), `out` like q, `lse` float32 [B, Hq, Nq] and
    `seqlens` int32 [B], all contiguous on q's device (None: not given).
    Returns (B, Hq, Hkv, Nq, Nk, d)."""
    import torch
    shp = _check_qkv(q, k, v, (torch.bfloat16, torch.float32), require_gpu)
    B, Hq, Hkv, Nq, Nk, d = shp
    if out is not None:
        _need(out, "out", q.dtype, q.shape, q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, Nq), q.device)
    _seqlens_ptr(seqlens, B, q.device)
    return shp


def check_backward_args(q, k, v, o, lse, dout, seqlens=None,
                        require_gpu=True):
    """The checks `attn_backward` makes before any launch: q, k, v, o, dout
    bfloat16 (o and dout like q), lse float32 [B, Hq, Nq], seqlens int32
    [B], all contiguous on q's device."""
    import torch
    shp = _check_qkv(q, k, v, (torch.bfloat16,), require_gpu)
    B, Hq, Hkv, Nq, Nk, d = shp
    _need(o, "o", torch.bfloat16, q.shape, q.device)
    _need(dout, "dout", torch.bfloat16, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, Hq, Nq), q.device)
    _seqlens_ptr(seqlens, B, q.device)
    return shp


def fp8_buffer_shapes(B, Hq, Hkv, Nq, Nk, d):
    """Shapes of the quantized buffers (see attn_fp8_quantize); Nk is padded
    to whole 64-key tiles."""
    nkp = (Nk + 63) // 64 * 64
    return dict(q8=(B, Hq, Nq, d), sq=(B, Hq, (Nq + 63) // 64),
                k8=(B, Hkv, nkp, d), sk=(B, Hkv, nkp // 64),
                v8t=(B, Hkv, nkp // 64, d, 64), sv=(B, Hkv, nkp // 64))


def check_fp8_state(z, out=None, lse=None, seqlens=None):
    """The checks `attn_fp8` makes before any launch: every buffer of `z`
    (what fp8_quantize returned) has the shape its recorded problem needs
    and its dtype (codes uint8, scales float32), all on one device; out is
    bfloat16 [B, Hq, Nq, d], lse float32 [B, Hq, Nq], seqlens int32 [B].
    Returns (B, Hq, Hkv, Nq, Nk, d)."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = z["shape"]
    dev = z["q8"].device
    for name, shp in fp8_buffer_shapes(B, Hq, Hkv, Nq, Nk, d).items():
        dt = torch.float32 if name.startswith("s") else torch.uint8
        _need(z[name], name, dt, shp, dev)
    if out is not None:
        _need(out, "out", torch.bfloat16, (B, Hq, Nq, d), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, Nq), dev)
    _seqlens_ptr(seqlens, B, dev)
    return B, Hq, Hkv, Nq, Nk, d


def attn(q, k, v, *, causal=False, window=0, seqlens=None, scale=None,
         out=None, lse=None, stream=None, window_right=0, sinks=0):
    """Attention on torch device tensors.

    q: [B, Hq, Nq, d], k/v: [B, Hkv, Nk, d], all bfloat16 or all float32,
    contiguous, on the same GPU.  seqlens: int32 device tensor [B] or None.
    out (like q) and lse (float32 [B, Hq, Nq]) may be given; they are
    checked like the inputs.  Returns (o, lse).  The default scale is
    1/sqrt(d).  window_right or sinks > 0, or a window without the causal
    mask, select the masked entry points (window is then the left limit of
    the neighbourhood).
    """
    import torch
    B, Hq, Hkv, Nq, Nk, d = check_attn_args(q, k, v, out, lse, seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    sl = _seqlens_ptr(seqlens, B, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    bf = q.dtype == torch.bfloat16
    if window_right or sinks or (window and not causal):
        fn = attn_fwd_masked if bf else attn_fwd_masked_f32
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale), causal,
                int(window), int(window_right), int(sinks), sl, stream)
    else:
        fn = attn_fwd if bf else attn_fwd_f32
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale), causal,
                int(window), sl, stream)
    if rc != MIATTN_OK:
        raise MiattnError(rc, attn_last_error())
    return out, lse


def attn_backward(q, k, v, o, lse, dout, *, causal=False, window=0,
                  seqlens=None, scale=None, window_right=0, sinks=0,
                  stream=None):
    """Gradients (dq, dk, dv) of attention on bfloat16 GPU tensors.

    q, k, v, seqlens and the mask arguments as for `attn`; o and lse are what
    `attn` returned for them, dout the gradient of the loss with respect to
    o.  Returns new tensors dq like q, dk and dv like k.
    """
    import torch
    B, Hq, Hkv, Nq, Nk, d = check_backward_args(q, k, v, o, lse, dout,
                                                seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    sl = _seqlens_ptr(seqlens, B, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    rc = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                  dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                  dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                  float(scale), causal, int(window), int(window_right),
                  int(sinks), sl, stream)
    if rc != MIATTN_OK:
        raise MiattnError(rc, attn_last_error())
    return dq, dk, dv


def fp8_quantize(q, k, v, *, seqlens=None, signs=None, per_tensor=False,
                 stream=None):
    """E4M3 codes and block scales of bfloat16 GPU tensors q, k, v (see
    attn_fp8_quantize in include/miattn.h).  signs: int8 GPU tensor of d
    entries +-1 (rotate Q and K) or None.  Returns a dict with q8, sq, k8,
    sk, v8t, sv, `rotated` and the problem's `shape`."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _check_qkv(q, k, v, (torch.bfloat16,))
    dev = q.device
    sgn = 0
    if signs is not None:
        _need(signs, "signs", torch.int8, (d,), dev)
        sgn = signs.data_ptr()
    sl = _seqlens_ptr(seqlens, B, dev)
    out = {name: torch.empty(shp, dtype=torch.float32 if name[0] == "s"
                             else torch.uint8, device=dev)
           for name, shp in fp8_buffer_shapes(B, Hq, Hkv, Nq, Nk,
                                              d).items()}
    out["rotated"] = signs is not None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = attn_fp8_quantize(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq,
                           Hkv, Nq, Nk, d, sl, sgn, per_tensor,
                           out["q8"].data_ptr(), out["sq"].data_ptr(),
                           out["k8"].data_ptr(), out["sk"].data_ptr(),
                           out["v8t"].data_ptr(), out["sv"].data_ptr(),
                           stream)
    if rc != MIATTN_OK:
        raise MiattnError(rc, attn_last_error())
    out["shape"] = (B, Hq, Hkv, Nq, Nk, d)
    return out


def attn_fp8(z, *, causal=False, window=0, seqlens=None, scale=None,
             window_right=0, sinks=0, out=None, lse=None, stream=None):
    """Attention on the output of fp8_quantize; returns (o bf16, lse).
    seqlens must be the valid lengths the codes were quantized with."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = check_fp8_state(z, out, lse, seqlens)
    dev = z["q8"].device
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    sl = _seqlens_ptr(seqlens, B, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = attn_fwd_fp8(z["q8"].data_ptr(), z["sq"].data_ptr(),
                      z["k8"].data_ptr(), z["sk"].data_ptr(),
                      z["v8t"].data_ptr(), z["sv"].data_ptr(),
                      out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                      float(scale), z["rotated"], causal, int(window),
                      int(window_right), int(sinks), sl, stream)
    if rc != MIATTN_OK:
        raise MiattnError(rc, attn_last_error())
    return out, lse

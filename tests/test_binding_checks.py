"""The Python binding's argument checks: every tensor a kernel reads or
writes is checked for dtype, shape, contiguity and device before any launch.
The checks are plain functions, exercised here with CPU tensors (no GPU)."""

import pytest
import torch

import transformer_self_attention_attn_amd as mi


def qkv(B=2, Hq=4, Hkv=2, Nq=5, Nk=7, d=64, dtype=torch.bfloat16):
    return (torch.zeros(B, Hq, Nq, d, dtype=dtype),
            torch.zeros(B, Hkv, Nk, d, dtype=dtype),
            torch.zeros(B, Hkv, Nk, d, dtype=dtype))


def test_attn_args_accepts_consistent_tensors():
    q, k, v = qkv()
    out = torch.empty_like(q)
    lse = torch.empty(2, 4, 5)
    sl = torch.tensor([3, 7], dtype=torch.int32)
    assert mi.check_attn_args(q, k, v, out, lse, sl, require_gpu=False) == \
        (2, 4, 2, 5, 7, 64)


@pytest.mark.parametrize("bad", [
    "out_dtype", "out_short", "out_noncontig", "lse_dtype", "lse_short",
    "v_shape", "k_batch", "k_dim", "dtype_mix", "seqlens_dtype",
    "seqlens_len", "q_3d", "q_fp16"])
def test_attn_args_rejects(bad):
    q, k, v = qkv()
    out, lse, sl = None, None, None
    if bad == "out_dtype":
        out = torch.empty(q.shape, dtype=torch.float32)
    elif bad == "out_short":
        out = torch.empty(2, 4, 4, 64, dtype=torch.bfloat16)
    elif bad == "out_noncontig":
        out = torch.empty(2, 4, 64, 5, dtype=torch.bfloat16).transpose(2, 3)
    elif bad == "lse_dtype":
        lse = torch.empty(2, 4, 5, dtype=torch.float64)
    elif bad == "lse_short":
        lse = torch.empty(2, 4, 4)
    elif bad == "v_shape":
        v = torch.zeros(2, 2, 6, 64, dtype=torch.bfloat16)
    elif bad == "k_batch":
        k = torch.zeros(3, 2, 7, 64, dtype=torch.bfloat16)
        v = k.clone()
    elif bad == "k_dim":
        k = torch.zeros(2, 2, 7, 128, dtype=torch.bfloat16)
        v = k.clone()
    elif bad == "dtype_mix":
        v = v.float()
    elif bad == "seqlens_dtype":
        sl = torch.tensor([3, 7], dtype=torch.int64)
    elif bad == "seqlens_len":
        sl = torch.tensor([3], dtype=torch.int32)
    elif bad == "q_3d":
        q = q[0]
    elif bad == "q_fp16":
        q, k, v = qkv(dtype=torch.float16)
    with pytest.raises((ValueError, TypeError)):
        mi.check_attn_args(q, k, v, out, lse, sl, require_gpu=False)


def test_attn_args_require_a_gpu():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="GPU"):
        mi.check_attn_args(q, k, v)
    with pytest.raises(ValueError, match="GPU"):
        mi.attn(q, k, v)


@pytest.mark.parametrize("bad", ["o_shape", "dout_dtype", "lse_shape",
                                 "q_fp32", "seqlens_len"])
def test_backward_args_rejects(bad):
    q, k, v = qkv()
    o, dout = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(2, 4, 5)
    sl = None
    if bad == "o_shape":
        o = torch.empty(2, 4, 6, 64, dtype=torch.bfloat16)
    elif bad == "dout_dtype":
        dout = dout.float()
    elif bad == "lse_shape":
        lse = torch.empty(2, 4)
    elif bad == "q_fp32":
        q, k, v = qkv(dtype=torch.float32)
    elif bad == "seqlens_len":
        sl = torch.zeros(5, dtype=torch.int32)
    with pytest.raises((ValueError, TypeError)):
        mi.check_backward_args(q, k, v, o, lse, dout, sl, require_gpu=False)
    q, k, v = qkv()
    assert mi.check_backward_args(
        q, k, v, torch.empty_like(q), torch.empty(2, 4, 5),
        torch.empty_like(q), None, require_gpu=False) == (2, 4, 2, 5, 7, 64)


def fp8_state(B=2, Hq=4, Hkv=2, Nq=70, Nk=130, d=64):
    z = {name: torch.zeros(shp, dtype=torch.float32 if name[0] == "s"
                           else torch.uint8)
         for name, shp in mi.fp8_buffer_shapes(B, Hq, Hkv, Nq, Nk,
                                               d).items()}
    z["rotated"] = False
    z["shape"] = (B, Hq, Hkv, Nq, Nk, d)
    return z


def test_fp8_buffer_shapes_pad_keys_to_tiles():
    shp = mi.fp8_buffer_shapes(2, 4, 2, 70, 130, 64)
    assert shp["k8"] == (2, 2, 192, 64)
    assert shp["v8t"] == (2, 2, 3, 64, 64)
    assert shp["sq"] == (2, 4, 2) and shp["sk"] == (2, 2, 3)


@pytest.mark.parametrize("bad", ["k8_short", "sv_dtype", "v8t_layout",
                                 "out_shape", "lse_dtype", "seqlens_len",
                                 "seqlens_dtype"])
def test_fp8_state_rejects(bad):
    z = fp8_state()
    out = lse = sl = None
    if bad == "k8_short":
        z["k8"] = torch.zeros(2, 2, 130, 64, dtype=torch.uint8)
    elif bad == "sv_dtype":
        z["sv"] = z["sv"].double()
    elif bad == "v8t_layout":
        z["v8t"] = torch.zeros(2, 2, 3, 64 * 64, dtype=torch.uint8)
    elif bad == "out_shape":
        out = torch.empty(2, 4, 70, 128, dtype=torch.bfloat16)
    elif bad == "lse_dtype":
        lse = torch.empty(2, 4, 70, dtype=torch.bfloat16)
    elif bad == "seqlens_len":
        sl = torch.zeros(3, dtype=torch.int32)
    elif bad == "seqlens_dtype":
        sl = torch.zeros(2, dtype=torch.int16)
    with pytest.raises((ValueError, TypeError)):
        mi.check_fp8_state(z, out, lse, sl)
    assert mi.check_fp8_state(fp8_state()) == (2, 4, 2, 70, 130, 64)


def test_fp8_quantize_rejects_mismatched_v():
    q, k, _ = qkv()
    v = torch.zeros(2, 2, 6, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mi.fp8_quantize(q, k, v)

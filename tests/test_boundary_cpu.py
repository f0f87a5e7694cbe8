"""CPU-only: the C-ABI library loads, exports what include/miattn.h declares,
and rejects bad arguments on the host before any HIP call."""

import os
import re

import pytest

import transformer_self_attention_attn_amd as mi

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "miattn.h")

# fake, 16-byte aligned device addresses: validation must reject the call
# before anything dereferences them
P = 0x10000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(mi.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = mi.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def good(**over):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=4, Hkv=2, Nq=64, Nk=64, d=64,
             scale=0.125, causal=1, window=0, seqlens=0, stream=0)
    a.update(over)
    return a


def call(fn, a):
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
              a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
              a["window"], a["seqlens"], a["stream"])


BAD = [
    (dict(q=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(v=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(o=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(B=0), mi.MIATTN_ERR_INVALID, "positive"),
    (dict(Hq=-1), mi.MIATTN_ERR_INVALID, "positive"),
    (dict(Nk=0), mi.MIATTN_ERR_INVALID, "positive"),
    (dict(d=0), mi.MIATTN_ERR_INVALID, "positive"),
    (dict(Hq=6, Hkv=4), mi.MIATTN_ERR_INVALID, "multiple"),
    (dict(Nq=65), mi.MIATTN_ERR_INVALID, "exceeds"),
    (dict(window=-1), mi.MIATTN_ERR_INVALID, "negative"),
    (dict(scale=float("nan")), mi.MIATTN_ERR_INVALID, "finite"),
    (dict(scale=float("inf")), mi.MIATTN_ERR_INVALID, "finite"),
    (dict(q=P + 2), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(lse=P + 4), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(d=96), mi.MIATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(d=256), mi.MIATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(window=8, causal=0), mi.MIATTN_ERR_UNSUPPORTED, "causal"),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 12, Nk=1 << 12),
     mi.MIATTN_ERR_INVALID, "too large"),
]


@pytest.mark.parametrize("fn_name", ["attn_fwd", "attn_fwd_f32"])
@pytest.mark.parametrize("over,code,msg", BAD,
                         ids=[str(b[0]) for b in BAD])
def test_rejected_on_host(fn_name, over, code, msg):
    fn = getattr(mi, fn_name)
    rc = call(fn, good(**over))
    assert rc == code
    err = mi.attn_last_error()
    assert fn_name in err and msg in err, err


def call_masked(fn, a):
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
              a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
              a["window"], a.get("window_right", 0), a.get("sinks", 0),
              a["seqlens"], a["stream"])


# the masked entry points take every check above except the one-sided
# window rule (a window without the causal mask is allowed there), plus
# non-negative right limits and sink counts
BAD_MASKED = [b for b in BAD if b[2] != "causal"] + [
    (dict(window_right=-1), mi.MIATTN_ERR_INVALID, "negative"),
    (dict(sinks=-3), mi.MIATTN_ERR_INVALID, "negative"),
    (dict(sinks=-1, causal=0, window=8), mi.MIATTN_ERR_INVALID, "negative"),
]


@pytest.mark.parametrize("fn_name", ["attn_fwd_masked",
                                     "attn_fwd_masked_f32"])
@pytest.mark.parametrize("over,code,msg", BAD_MASKED,
                         ids=[str(b[0]) for b in BAD_MASKED])
def test_masked_rejected_on_host(fn_name, over, code, msg):
    fn = getattr(mi, fn_name)
    rc = call_masked(fn, good(**over))
    assert rc == code
    err = mi.attn_last_error()
    assert fn_name in err and msg in err, err


def call_bwd(a):
    return mi.attn_bwd(a["q"], a["k"], a["v"], a["o"], a.get("dout", P),
                       a["lse"], a.get("dq", P), a.get("dk", P),
                       a.get("dv", P), a["B"], a["Hq"], a["Hkv"], a["Nq"],
                       a["Nk"], a["d"], a["scale"], a["causal"], a["window"],
                       a.get("window_right", 0), a.get("sinks", 0),
                       a["seqlens"], a["stream"])


# the backward entry point takes the masked entry points' checks, and needs
# dout, lse, dq, dk and dv as well
BAD_BWD = BAD_MASKED + [
    (dict(dout=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(lse=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(dq=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(dv=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(dk=P + 8), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(dout=P + 2), mi.MIATTN_ERR_INVALID, "aligned"),
]


@pytest.mark.parametrize("over,code,msg", BAD_BWD,
                         ids=[str(b[0]) for b in BAD_BWD])
def test_backward_rejected_on_host(over, code, msg):
    rc = call_bwd(good(**over))
    assert rc == code
    err = mi.attn_last_error()
    assert "attn_bwd" in err and msg in err, err


def test_lse_may_be_null_and_still_validated():
    rc = call(mi.attn_fwd, good(lse=0, d=80))
    assert rc == mi.MIATTN_ERR_UNSUPPORTED


def test_torch_wrapper_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mi.attn(q, q, q)
    with pytest.raises(TypeError):
        mi.attn(q, q, q.float())


def call_quant(a):
    return mi.attn_fp8_quantize(
        a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
        a["d"], a["seqlens"], a.get("signs", 0), a.get("per_tensor", 0),
        a.get("q8", P), a.get("sq", P), a.get("k8", P), a.get("sk", P),
        a.get("v8t", P), a.get("sv", P), a["stream"])


# the quantizer takes the shape checks of the forward (no scale or mask
# arguments), non-null outputs, 16-byte aligned codes and 4-byte aligned
# scales, and the one-resource limit on a sequence's bytes
BAD_QUANT = [b for b in BAD if b[2] not in ("causal", "finite")
             and "lse" not in b[0] and "o" not in b[0]
             and "window" not in b[0]] + [
    (dict(q8=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(sk=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(v8t=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(k8=P + 8), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(sq=P + 2), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(B=1, Hq=1, Hkv=1, Nq=64, Nk=1 << 23, d=128),
     mi.MIATTN_ERR_UNSUPPORTED, "2^31"),
]


@pytest.mark.parametrize("over,code,msg", BAD_QUANT,
                         ids=[str(b[0]) for b in BAD_QUANT])
def test_fp8_quantize_rejected_on_host(over, code, msg):
    rc = call_quant(good(**over))
    assert rc == code
    err = mi.attn_last_error()
    assert "attn_fp8_quantize" in err and msg in err, err


def call_fwd8(a):
    return mi.attn_fwd_fp8(
        a.get("q8", P), a.get("sq", P), a.get("k8", P), a.get("sk", P),
        a.get("v8t", P), a.get("sv", P), a["o"], a["lse"], a["B"], a["Hq"],
        a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a.get("rotated", 0),
        a["causal"], a["window"], a.get("window_right", 0),
        a.get("sinks", 0), a["seqlens"], a["stream"])


# the FP8 forward takes the masked entry points' checks (its code buffers
# stand where q, k, v stand there), non-null 4-byte aligned scales and the
# one-resource limit
BAD_FWD8 = [b for b in BAD_MASKED
            if not any(key in b[0] for key in ("q", "v"))] + [
    (dict(q8=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(v8t=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(k8=P + 4), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(sq=0), mi.MIATTN_ERR_INVALID, "non-null"),
    (dict(sv=P + 1), mi.MIATTN_ERR_INVALID, "aligned"),
    (dict(B=1, Hq=1, Hkv=1, Nq=64, Nk=1 << 23, d=128),
     mi.MIATTN_ERR_UNSUPPORTED, "2^31"),
]


@pytest.mark.parametrize("over,code,msg", BAD_FWD8,
                         ids=[str(b[0]) for b in BAD_FWD8])
def test_fwd_fp8_rejected_on_host(over, code, msg):
    rc = call_fwd8(good(**over))
    assert rc == code
    err = mi.attn_last_error()
    assert "attn_fwd_fp8" in err and msg in err, err


@pytest.mark.parametrize("Nq,Nk,d", [(1 << 23, 1 << 23, 128),
                                     (64, (1 << 24) - 63, 64)])
def test_backward_rejects_sequences_past_one_resource(Nq, Nk, d):
    """The backward kernels address a whole sequence through one buffer
    resource (32-bit byte range): 2^31 bytes or more is refused."""
    rc = call_bwd(good(B=1, Hq=1, Hkv=1, Nq=Nq, Nk=Nk, d=d))
    assert rc == mi.MIATTN_ERR_UNSUPPORTED
    assert "2^31" in mi.attn_last_error()


@pytest.mark.parametrize("fn_name", ["attn_fwd", "attn_fwd_masked"])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_sequence_of_2gib_rejected_on_host(fn_name, d):
    """The prefill kernel addresses a head's query rows with 32-bit byte
    offsets: Nq rows of d bf16 must span less than 2^31 bytes."""
    fn = getattr(mi, fn_name)
    n = (1 << 31) // (2 * d)  # exactly 2^31 bytes of query rows
    a = good(B=1, Hq=1, Hkv=1, Nq=n, Nk=n, d=d)
    rc = call(fn, a) if fn_name == "attn_fwd" else call_masked(fn, a)
    assert rc == mi.MIATTN_ERR_UNSUPPORTED
    err = mi.attn_last_error()
    assert fn_name in err and "2^31" in err, err

"""GPU parity of the FP8 path (attn_fp8_quantize, attn_fwd_fp8, through the
C ABI) against the FP8 reference (`oracle.fp8`).

  * Quantization is byte work: every E4M3 code and every block scale must
    equal the reference's bit for bit (the reference takes each rounding
    decision in float32, as the kernel does).
  * The forward kernel is compared with the exact (fp64) attention of the
    dequantized operands.  Besides fp32 accumulation it rounds each
    probability, times 256 and its tile's V-scale ratio, to E4M3 before the
    second product: a relative error uniform in +-2^-4, rms 2^-4/sqrt(3)
    = 3.6%.  An output row is a weighted mean of V rows whose own size
    shrinks with the same averaging that shrinks this error, so the
    relative error of o stays near that rms.  Bar: sum|o - ref| / sum|ref|
    <= 5e-2 and max|o - ref| <= 0.1 max|ref|; lse (formed from the
    unrounded probabilities, fp32 throughout) within 1e-3 + 1e-5 |lse|.
  * The page's accuracy comparison: RMSE against the exact attention of the
    bf16 inputs, block quantization with incoherent processing against one
    scale per tensor, on inputs with a few large shared channels in Q and K.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_self_attention_attn_amd as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

W = synth.Workload
TOL = dict(rel_l1=5e-2, max_rel=0.1, lse=1e-3, lse_rel=1e-5)


def gpu_quant(w, x, signs, per_tensor):
    q, k, v, sl = gu.to_dev(x)
    sg = None if signs is None else torch.from_numpy(signs).to(gu.DEV)
    z = mi.fp8_quantize(q, k, v, seqlens=sl, signs=sg, per_tensor=per_tensor)
    torch.cuda.synchronize()
    return z, sl


def ref_quant(w, x, signs, per_tensor):
    sl = x["seqlens"]
    if sl is None:
        sl = np.full(w.B, w.Nk)
    return oracle.fp8.quantize_all(x["q32"], x["k32"], x["v32"], sl,
                                   signs=None if signs is None else
                                   signs.astype(np.float64),
                                   per_tensor=per_tensor)


def natural_v(v8t, nk):
    """[B][H][T][d][64] -> [B][H][T*64][d], first nk rows."""
    b, h, t, d, _ = v8t.shape
    return v8t.permute(0, 1, 2, 4, 3).reshape(b, h, t * 64, d)[:, :, :nk]


FP8_CASES = [
    # (workload, rotated, per_tensor)
    (W("fp8-gqa-d128-causal-padded", 2, 4, 2, 300, 300, 128, "bf16", True,
       len_lo=1, len_hi=300), True, False),
    (W("fp8-mha-d128-noncausal", 2, 2, 2, 200, 200, 128, "bf16", False),
     False, False),
    (W("fp8-d64-causal", 2, 4, 4, 257, 257, 64, "bf16", True), True, False),
    (W("fp8-per-tensor-d128", 2, 4, 2, 260, 260, 128, "bf16", True,
       len_lo=100, len_hi=260), False, True),
    (W("fp8-chunk-d128", 2, 4, 2, 70, 333, 128, "bf16", True, len_lo=80,
       len_hi=333), True, False),
    (W("fp8-window-sinks-d64", 2, 4, 2, 400, 400, 64, "bf16", True,
       window=65, sinks=4, len_lo=100, len_hi=400), True, False),
    (W("fp8-two-sided-d128", 1, 4, 1, 300, 300, 128, "bf16", False,
       window=40, window_right=70), True, False),
    # wholly allowed tiles in a window run apart from the sink tiles
    (W("fp8-wide-win-sinks-d128", 2, 4, 2, 1100, 1100, 128, "bf16", True,
       window=400, sinks=70, len_lo=600, len_hi=1100), True, False),
    (W("fp8-outliers-d128", 2, 4, 2, 256, 256, 128, "bf16", True,
       outlier_channels=4, outlier_mag=20.0), True, False),
]


@pytest.mark.parametrize("w,rot,pt", FP8_CASES, ids=lambda c: getattr(
    c, "name", str(c)))
def test_fp8_quantize_bit_exact(w, rot, pt):
    gu.say(f"[gpu] fp8 quantize {w.name} rotated={rot} per_tensor={pt}")
    x = synth.make_inputs(w, 51)
    signs = synth.make_signs(w.d, 51) if rot else None
    z, _ = gpu_quant(w, x, signs, pt)
    ref = ref_quant(w, x, signs, pt)
    q8 = z["q8"].cpu().numpy()
    assert np.array_equal(q8, ref["q"][0]), "q codes"
    assert np.array_equal(z["sq"].cpu().numpy(), ref["q"][1]), "q scales"
    k8 = z["k8"].cpu().numpy()
    assert np.array_equal(k8[:, :, :w.Nk], ref["k"][0]), "k codes"
    assert np.all(k8[:, :, w.Nk:] == 0)
    assert np.array_equal(z["sk"].cpu().numpy(), ref["k"][1]), "k scales"
    v8 = natural_v(z["v8t"], w.Nk).cpu().numpy()
    assert np.array_equal(v8, ref["v"][0]), "v codes"
    assert np.array_equal(z["sv"].cpu().numpy(), ref["v"][1]), "v scales"


def compare_o(name, o, lse, ro, rl):
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    live = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), ~live), f"{name}: empty rows"
    assert np.all(go[~live] == 0)
    err = np.abs(go[live] - ro[live])
    mag = np.abs(ro[live]).max()
    rel = err.sum() / np.abs(ro[live]).sum()
    lerr = (np.abs(gl[live] - rl[live]) /
            (TOL["lse"] + TOL["lse_rel"] * np.abs(rl[live]))).max()
    gu.say(f"  {name}: rel_l1={rel:.3e} max_abs={err.max():.3e} "
           f"max|ref|={mag:.3e} lse_err/bound={lerr:.3e}")
    assert rel <= TOL["rel_l1"], f"{name}: rel_l1 {rel}"
    assert err.max() <= TOL["max_rel"] * mag, f"{name}: max_abs {err.max()}"
    assert lerr <= 1.0, f"{name}: lse error {lerr} of its bound"


@pytest.mark.parametrize("w,rot,pt", FP8_CASES, ids=lambda c: getattr(
    c, "name", str(c)))
def test_fp8_forward_matches_oracle(w, rot, pt):
    gu.say(f"[gpu] fp8 forward {w.name} rotated={rot} per_tensor={pt}")
    x = synth.make_inputs(w, 52)
    signs = synth.make_signs(w.d, 52) if rot else None
    z, sl = gpu_quant(w, x, signs, pt)
    kw = dict(causal=w.causal, window=w.window, window_right=w.window_right,
              sinks=w.sinks)
    o, lse = mi.attn_fp8(z, seqlens=sl, scale=w.scale, **kw)
    torch.cuda.synchronize()
    ref = ref_quant(w, x, signs, pt)
    ro, rl = oracle.fp8.attention_quantized(
        ref["q"], ref["k"], ref["v"], scale=w.scale, rotated=rot,
        seqlens=x["seqlens"], **kw)
    compare_o(w.name, o, lse, ro, rl)


def test_fp8_rmse_block_rotated_vs_per_tensor():
    """The page's comparison, on the GPU path: RMSE of FP8 attention against
    the exact attention of the bf16 inputs, with block scales and the
    rotation against one scale per tensor and no rotation."""
    w = W("fp8-rmse-outliers", 2, 4, 2, 1024, 1024, 128, "bf16", True,
          outlier_channels=4, outlier_mag=20.0)
    x = synth.make_inputs(w, 53)
    signs = synth.make_signs(w.d, 53)
    exact, lse = oracle.attention(x["q32"], x["k32"], x["v32"],
                                  scale=w.scale, causal=True)
    live = np.isfinite(lse)
    res = {}
    for name, sg, pt in (("block+rotation", signs, False),
                         ("per-tensor", None, True)):
        z, sl = gpu_quant(w, x, sg, pt)
        o, _ = mi.attn_fp8(z, seqlens=sl, scale=w.scale, causal=True)
        torch.cuda.synchronize()
        res[name] = oracle.fp8.rmse(o.float().cpu().numpy(), exact, live)
    ratio = res["per-tensor"] / res["block+rotation"]
    gu.say(f"  rmse block+rotation={res['block+rotation']:.4e} "
           f"per-tensor={res['per-tensor']:.4e} ratio={ratio:.2f}")
    assert ratio > 1.5, res


@pytest.mark.parametrize("scale", [0.0, -0.07], ids=["scale0", "negscale"])
def test_fp8_scale_edge(scale):
    """scale 0: every allowed key weighs the same; a negative scale takes
    the Q codes' sign flip inside the kernel."""
    w = W("fp8-scale-edge-d128", 2, 4, 2, 200, 200, 128, "bf16", True,
          len_lo=30, len_hi=200)
    gu.say(f"[gpu] fp8 forward {w.name} scale={scale}")
    x = synth.make_inputs(w, 54)
    signs = synth.make_signs(w.d, 54)
    z, sl = gpu_quant(w, x, signs, False)
    o, lse = mi.attn_fp8(z, seqlens=sl, scale=scale, causal=True)
    torch.cuda.synchronize()
    ref = ref_quant(w, x, signs, False)
    ro, rl = oracle.fp8.attention_quantized(
        ref["q"], ref["k"], ref["v"], scale=scale, rotated=True, causal=True,
        seqlens=x["seqlens"])
    compare_o(f"{w.name} scale={scale}", o, lse, ro, rl)


def test_fp8_nan_padding_is_never_read():
    """NaN in every padded row of Q, K and V changes no code, no scale and
    no output."""
    w = W("fp8-nan-pad-d64", 3, 4, 2, 300, 300, 64, "bf16", True, len_lo=1,
          len_hi=300)
    gu.say(f"[gpu] fp8 {w.name}")
    signs = synth.make_signs(w.d, 55)
    xs = synth.make_inputs(w, 55)
    xn = synth.make_inputs(w, 55, pad_fill="nan")
    za, sl = gpu_quant(w, xs, signs, False)
    zb, _ = gpu_quant(w, xn, signs, False)
    for key in ("q8", "sq", "k8", "sk", "v8t", "sv"):
        assert torch.equal(za[key], zb[key]), key
    oa, la = mi.attn_fp8(za, seqlens=sl, scale=w.scale, causal=True)
    ob, lb = mi.attn_fp8(zb, seqlens=sl, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.all(torch.isfinite(ob))


def test_fp8_full_size_gqa_causal_prefill():
    """gqa-causal-prefill at full size: every code and scale against the
    reference, and sampled output rows against the exact attention of the
    dequantized operands."""
    w = synth.by_name("gqa-causal-prefill")
    gu.say(f"[gpu] fp8 {w.name} (full size)")
    x = synth.make_inputs(w, 3)
    signs = synth.make_signs(w.d, 3)
    z, sl = gpu_quant(w, x, signs, False)
    ref = ref_quant(w, x, signs, False)
    assert np.array_equal(z["q8"].cpu().numpy(), ref["q"][0])
    assert np.array_equal(z["sq"].cpu().numpy(), ref["q"][1])
    assert np.array_equal(z["k8"].cpu().numpy(), ref["k"][0])
    assert np.array_equal(z["sk"].cpu().numpy(), ref["k"][1])
    assert np.array_equal(natural_v(z["v8t"], w.Nk).cpu().numpy(),
                          ref["v"][0])
    assert np.array_equal(z["sv"].cpu().numpy(), ref["v"][1])
    o, lse = mi.attn_fp8(z, seqlens=sl, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1003)
    picks = gu.sample_rows(w, None, rng)
    qd = oracle.fp8.dequantize(*ref["q"])
    kd = oracle.fp8.dequantize(*ref["k"])
    vd = oracle.fp8.dequantize(*ref["v"])
    ro, rl = oracle.attention_rows(qd, kd, vd, picks, scale=w.scale / w.d,
                                   causal=True)
    idx = tuple(np.array(picks).T)
    compare_o(f"{w.name} sampled", o[idx], lse[idx], ro, rl)
    # the lightest query blocks are handed out at run time: over launches in
    # a row into NaN-filled outputs every row is written, bitwise the same
    for _ in range(3):
        o2 = torch.full_like(o, float("nan"))
        l2 = torch.full_like(lse, float("nan"))
        mi.attn_fp8(z, seqlens=sl, scale=w.scale, causal=True, out=o2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(l2, lse)

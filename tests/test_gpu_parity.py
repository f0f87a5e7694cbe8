"""GPU parity: libmiattn (through its C ABI) against the fp64 oracle.

Reduced sizes compare every row and span several query blocks and 64-key
tiles with ragged tails.  The five workloads run at full size with three
seeds each: every row of the fp32 case, the padded GPT-2-shaped prefill, the
grouped-query prefill and the decode step; four whole (batch, head) slices
and sampled rows of the others for the 16384-token sliding window.  Edge cases:
empty sequences, one valid key, window of one, N below one tile, GQA groups
of 1, 2, 4, 7 and 16, negative and zero scale, NaN in the padding.
"""

import math

import numpy as np
import pytest
import torch

import synth
import transformer_self_attention_attn_amd as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

W = synth.Workload

PREFILL_CASES = [
    W("mha-d64-nocausal-ragged", 2, 4, 4, 300, 300, 64, "bf16", False),
    W("mha-d128-nocausal-ragged", 2, 4, 4, 300, 300, 128, "bf16", False),
    W("gqa3-d64-causal-padded", 3, 6, 2, 333, 333, 64, "bf16", True,
      len_lo=1, len_hi=333),
    W("mqa7-d128-causal", 2, 7, 1, 257, 257, 128, "bf16", True),
    W("gqa2-d64-window64", 2, 4, 2, 700, 700, 64, "bf16", True, window=64),
    W("d128-window1-self-only", 1, 2, 2, 130, 130, 128, "bf16", True,
      window=1),
    W("d64-window1024-long", 1, 2, 2, 2000, 2000, 64, "bf16", True,
      window=1024),
    W("d128-below-one-tile-padded", 3, 2, 1, 17, 17, 128, "bf16", True,
      len_lo=0, len_hi=17),
    W("d64-exact-tile", 1, 1, 1, 128, 128, 64, "bf16", True),
    W("gqa4-d128-window100-padded", 2, 8, 2, 515, 515, 128, "bf16", True,
      window=100, len_lo=60, len_hi=515),
    W("amp3-d128-causal", 1, 2, 1, 200, 200, 128, "bf16", True, amp=3.0),
    # longer d=64 rows: dead rows, lengths from 1 key, a ragged last tile
    W("d64-long-causal-padded", 3, 4, 2, 777, 777, 64, "bf16", True,
      len_lo=1, len_hi=777),
    W("d64-long-nocausal", 2, 2, 1, 1000, 1000, 64, "bf16", False),
]


@pytest.mark.parametrize("w", PREFILL_CASES, ids=lambda w: w.name)
def test_prefill_small(w):
    for seed in (11, 12):
        gu.check_full(w.name, w, seed)


DECODE_CASES = [
    W("decode-gqa4-d128-padded", 6, 8, 2, 1, 3000, 128, "bf16", True,
      len_lo=0, len_hi=3000),
    W("decode-mha-d64-full", 2, 4, 4, 1, 1100, 64, "bf16", True),
    W("decode-window100", 4, 8, 2, 1, 2100, 128, "bf16", True, window=100,
      len_lo=1, len_hi=2100),
    W("decode-gqa7-d64", 3, 14, 2, 1, 777, 64, "bf16", True, len_lo=1,
      len_hi=777),
    W("decode-mqa16-d128", 2, 16, 1, 1, 1025, 128, "bf16", True,
      len_lo=500, len_hi=1025),
    W("decode-nocausal", 2, 8, 2, 1, 600, 128, "bf16", False, len_lo=1,
      len_hi=600),
    W("decode-one-key", 2, 4, 1, 1, 1, 64, "bf16", True),
    # more query heads per K/V head than one wavefront's 16 MFMA columns:
    # 32 -> two chunks of 16, 24 -> two of 12, 17 (prime) -> 17 of one
    W("decode-mqa32-d64", 2, 32, 1, 1, 900, 64, "bf16", True, len_lo=1,
      len_hi=900),
    W("decode-g24-d128", 2, 48, 2, 1, 700, 128, "bf16", True, len_lo=300,
      len_hi=700),
    W("decode-g17-d128", 1, 17, 1, 1, 600, 128, "bf16", True),
    # split sizes: small problems take 128-key splits; 160 (batch, K/V
    # head) groups over 2048 keys take 256 (the full-size configurations
    # cover 512 and 1024)
    W("decode-chunk256", 20, 32, 8, 1, 2048, 128, "bf16", True, len_lo=1,
      len_hi=2048),
]


@pytest.mark.parametrize("w", DECODE_CASES, ids=lambda w: w.name)
def test_decode_small(w):
    for seed in (21, 22):
        gu.check_full(w.name, w, seed)


def test_decode_chunk_boundaries():
    """Valid lengths on and around split boundaries (multiples of 128 keys:
    the split size is a power of two from 128 up)."""
    w = W("decode-boundaries", 8, 4, 1, 1, 2048, 128, "bf16", True,
          len_lo=1, len_hi=2048)
    x = synth.make_inputs(w, 31)
    x["seqlens"] = np.array([1, 511, 512, 513, 1024, 1025, 2047, 2048],
                            dtype=np.int32)
    q, k, v, sl = gu.to_dev(x)
    o, lse = gu.run_gpu(w, x, dev_inputs=(q, k, v, sl))
    go, gl = gu.host(o, lse)
    import oracle
    ro, rl = oracle.attention(x["q32"], x["k32"], x["v32"], scale=w.scale,
                              causal=True, seqlens=x["seqlens"])
    gu.compare(w.name, "bf16", go, gl, ro, rl)


FP32_CASES = [
    W("fp32-gqa-causal-padded-d128", 2, 4, 2, 150, 150, 128, "fp32", True,
      len_lo=1, len_hi=150),
    W("fp32-window-d64", 1, 2, 1, 200, 200, 64, "fp32", True, window=17),
    W("fp32-decode-d64", 3, 4, 2, 1, 300, 64, "fp32", True, len_lo=0,
      len_hi=300),
]


@pytest.mark.parametrize("w", FP32_CASES, ids=lambda w: w.name)
def test_fp32_small(w):
    gu.check_full(w.name, w, 41)


def test_scale_zero_and_negative():
    w = W("scale-edge", 2, 4, 2, 190, 190, 128, "bf16", True, len_lo=50,
          len_hi=190)
    gu.check_full("scale-zero", w, 51, scale=0.0)
    gu.check_full("scale-negative", w, 52, scale=-0.2)
    wn = W("scale-negative-nocausal", 1, 2, 2, 150, 150, 64, "bf16", False)
    gu.check_full(wn.name, wn, 53, scale=-0.3)
    wd = W("decode-scale-zero", 2, 4, 2, 1, 700, 128, "bf16", True,
           len_lo=1, len_hi=700)
    gu.check_full(wd.name, wd, 54, scale=0.0)


# ---- the five workloads at full size ----------------------------------------

def test_config_fp32_single_head():
    w = synth.by_name("fp32-single-head")
    for seed in (1, 101, 201):
        gu.check_full(w.name, w, seed)


# every row of the full-size workloads the oracle finishes in seconds, three
# seeds each (k, 100 + k, 200 + k for workload k; the first is the bench's)
@pytest.mark.parametrize("name,seed", [
    (name, base + off)
    for name, base in (("gpt2-small-causal-padded", 2),
                       ("gqa-causal-prefill", 3), ("decode-gqa", 5))
    for off in (0, 100, 200)])
def test_config_full_size_all_rows(name, seed):
    w = synth.by_name(name)
    gu.check_full(name, w, seed)


@pytest.mark.parametrize("seed,slices", [
    (4, [(0, 0), (0, 15), (1, 7), (1, 15)]),
    (104, [(0, 3), (1, 12)]),
    (204, [(1, 0), (0, 9)])])
def test_sliding_window_causal_whole_slices(seed, slices):
    """sliding-window-causal at full size (B=2 H=16 N=16384 d=64, window
    1024): whole (batch, head) slices, every query row, against the oracle's
    dense masked rows (16384 keys each); sampled rows of the other slices
    are checked by test_config_full_size_sampled."""
    w = synth.by_name("sliding-window-causal")
    gu.check_whole_slices(w.name, w, seed, slices)


# ---- Nq new rows against a longer key sequence (1 < Nq < Nk) ---------------

CHUNK_SMALL = [
    # chunk against a padded cache; some caches shorter than the chunk
    W("chunk-causal-d128", 3, 4, 2, 70, 300, 128, "bf16", True, len_lo=20,
      len_hi=300),
    W("chunk-causal-d64", 2, 6, 3, 33, 200, 64, "bf16", True, len_lo=1,
      len_hi=200),
    W("chunk-window-d128", 2, 4, 1, 130, 520, 128, "bf16", True, window=100,
      len_lo=200, len_hi=520),
    W("chunk-full-d64", 2, 4, 4, 257, 700, 64, "bf16", True),
    W("cross-d128", 2, 8, 2, 90, 333, 128, "bf16", False, len_lo=1,
      len_hi=333),
    W("cross-d64-full", 1, 4, 2, 129, 300, 64, "bf16", False),
    W("chunk-fp32", 2, 4, 2, 20, 150, 64, "fp32", True, len_lo=5,
      len_hi=150),
    W("cross-fp32", 2, 2, 1, 40, 90, 128, "fp32", False, len_lo=1,
      len_hi=90),
    # short chunks (query heads x rows of a K/V head within 16 columns) take
    # the split-K matrix-core decode kernel; taller ones the prefill
    W("chunk4-gqa4-d128-padded", 3, 8, 2, 4, 700, 128, "bf16", True,
      len_lo=1, len_hi=700),
    W("chunk16-mha-d64", 2, 4, 4, 16, 500, 64, "bf16", True),
    W("chunk32-mha-d64-short", 3, 3, 3, 32, 1024, 64, "bf16", True,
      len_lo=1, len_hi=1024),
    W("chunk5-gqa7-d128-cross", 2, 14, 2, 5, 600, 128, "bf16", False,
      len_lo=1, len_hi=600),
    W("chunk3-win-sinks-d64", 2, 4, 2, 3, 900, 64, "bf16", True, window=50,
      sinks=4, len_lo=1, len_hi=900),
    W("chunk8-two-sided-d128", 2, 2, 2, 8, 300, 128, "bf16", False,
      window=20, window_right=10, len_lo=30, len_hi=300),
    W("chunk64-mha-d128", 2, 2, 2, 64, 777, 128, "bf16", True, len_lo=1,
      len_hi=777),
    W("chunk65-mha-d128", 2, 2, 2, 65, 777, 128, "bf16", True, len_lo=1,
      len_hi=777),
]


@pytest.mark.parametrize("w", CHUNK_SMALL, ids=lambda w: w.name)
def test_chunk_and_cross_small(w):
    gu.check_full(w.name, w, 71)


@pytest.mark.parametrize("name,seed", [
    ("decode-chunk4-gqa", 22),
    ("chunk32-gpt2-causal", 16),
    ("chunked-prefill-gqa", 17),
    ("cross-attention-padded", 18),
])
def test_chunk_and_cross_full_size_sampled(name, seed):
    w = synth.by_name(name)
    gu.check_sampled(name, w, seed)


# ---- two-sided local windows and sink keys (attn_fwd_masked*) --------------

MASK_SMALL = [
    # window on both sides, no causal mask, padded; tiles cut by both limits
    W("two-sided-d128", 2, 4, 2, 300, 300, 128, "bf16", False, window=40,
      window_right=70, len_lo=100, len_hi=300),
    W("two-sided-d64-wide", 2, 6, 3, 333, 333, 64, "bf16", False,
      window=130, window_right=129),
    # right limit only: row i sees keys j < i + window_right
    W("right-only-d64", 1, 4, 1, 200, 200, 64, "bf16", False,
      window_right=65),
    # left limit only without the causal mask: keys j > i - window, all later
    W("left-only-noncausal-d128", 2, 2, 2, 260, 260, 128, "bf16", False,
      window=64),
    # causal window plus sinks: sink tiles and window tiles apart, adjacent
    # and overlapping
    W("causal-win-sinks-d64", 2, 6, 3, 600, 600, 64, "bf16", True, window=65,
      sinks=4, len_lo=1, len_hi=600),
    W("causal-win-sinks-tile-d128", 2, 4, 2, 520, 520, 128, "bf16", True,
      window=100, sinks=65, len_lo=200, len_hi=520),
    W("causal-self-only-sinks-d128", 1, 4, 4, 300, 300, 128, "bf16", True,
      window=1, sinks=130),
    # a window wide enough for wholly allowed tiles, apart from the sink
    # tiles: the steps of the window run without per-step tests
    W("causal-wide-win-sinks-d128", 2, 4, 2, 1100, 1100, 128, "bf16", True,
      window=400, sinks=70, len_lo=600, len_hi=1100),
    W("two-sided-wide-sinks-d128", 2, 4, 2, 700, 700, 128, "bf16", False,
      window=300, window_right=260, sinks=9),
    W("sinks-past-window-d64", 2, 4, 2, 400, 400, 64, "bf16", True,
      window=50, sinks=200),
    # two-sided window with sinks, no causal mask
    W("two-sided-sinks-d64", 2, 4, 2, 450, 450, 64, "bf16", False, window=33,
      window_right=31, sinks=7, len_lo=40, len_hi=450),
    # chunk against a cache with window and sinks
    W("chunk-win-sinks-d128", 2, 4, 2, 70, 600, 128, "bf16", True,
      window=100, sinks=10, len_lo=20, len_hi=600),
    W("cross-two-sided-d64", 2, 4, 2, 150, 400, 64, "bf16", False, window=60,
      window_right=20, sinks=3, len_lo=10, len_hi=400),
    # decode: sinks in the first split, the window in the last, the middle
    # splits dead
    W("decode-win-sinks-d128", 4, 8, 2, 1, 1300, 128, "bf16", True,
      window=300, sinks=5, len_lo=1, len_hi=1300),
    W("decode-win-sinks-d64", 3, 12, 3, 1, 2000, 64, "bf16", True,
      window=17, sinks=600, len_lo=1, len_hi=2000),
    # fp32 path
    W("fp32-two-sided-sinks", 2, 4, 2, 150, 150, 64, "fp32", False, window=20,
      window_right=30, sinks=3, len_lo=5, len_hi=150),
    W("fp32-causal-win-sinks", 1, 2, 1, 200, 200, 128, "fp32", True,
      window=64, sinks=65),
    W("fp32-decode-win-sinks", 2, 4, 1, 1, 500, 128, "fp32", True,
      window=100, sinks=7, len_lo=1, len_hi=500),
]


@pytest.mark.parametrize("w", MASK_SMALL, ids=lambda w: w.name)
def test_masks_small(w):
    gu.check_full(w.name, w, 81)


@pytest.mark.parametrize("name,seed", [
    ("local-window-bidirectional", 19),
    ("sliding-window-sinks", 20),
    ("decode-window-sinks", 21),
])
def test_masks_full_size_sampled(name, seed):
    w = synth.by_name(name)
    gu.check_sampled(name, w, seed)


@pytest.mark.parametrize("name,seed", [
    ("sliding-window-causal", 4),
    ("sliding-window-causal", 104),
    ("sliding-window-causal", 204),
])
def test_config_full_size_sampled(name, seed):
    w = synth.by_name(name)
    gu.check_sampled(name, w, seed)


# ---- robustness and invariants ----------------------------------------------

@pytest.mark.parametrize("w", [
    W("nan-pad-prefill", 3, 4, 2, 300, 300, 128, "bf16", True, len_lo=1,
      len_hi=300),
    W("nan-pad-decode", 4, 8, 2, 1, 1300, 128, "bf16", True, len_lo=1,
      len_hi=1300),
    W("nan-pad-fp32", 2, 2, 1, 100, 100, 64, "fp32", True, len_lo=1,
      len_hi=100),
], ids=lambda w: w.name)
def test_nan_padding_is_never_read(w):
    gu.say(f"[gpu] {w.name}")
    a = synth.make_inputs(w, 61, pad_fill="draw")
    b = synth.make_inputs(w, 61, pad_fill="nan")
    oa, la = gu.run_gpu(w, a)
    ob, lb = gu.run_gpu(w, b)
    assert torch.isfinite(ob.float()).all()
    assert torch.equal(oa, ob)
    assert torch.equal(la, lb)


def test_tail_queue_every_launch():
    """A causal launch of several rounds of the chip's workgroup slots takes
    each XCD's lightest query blocks from a run-time queue whose counters the
    launch zeroes again as it ends.  Over launches in a row, with the outputs
    filled with NaN before each, every row is written every time and the
    results are bitwise the same."""
    w = synth.by_name("gqa-causal-prefill")
    gu.say(f"[gpu] tail queue {w.name}")
    q, k, v, sl = gu.to_dev(synth.make_inputs(w, 3))
    ref = None
    for _ in range(4):
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32,
                         device=q.device)
        mi.attn(q, k, v, causal=True, seqlens=sl, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        if ref is None:
            ref = (o, lse)
        else:
            assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])


def test_deterministic_bitwise():
    for w in (W("det-prefill", 2, 8, 2, 520, 520, 128, "bf16", True),
              W("det-decode", 4, 8, 2, 1, 2000, 128, "bf16", True, len_lo=1,
                len_hi=2000)):
        x = synth.make_inputs(w, 71)
        dev = gu.to_dev(x)
        o1, l1 = gu.run_gpu(w, x, dev_inputs=dev)
        o2, l2 = gu.run_gpu(w, x, dev_inputs=dev)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_equals_repeated_mha_bitwise():
    w = W("gqa", 2, 6, 2, 300, 300, 128, "bf16", True, len_lo=100,
          len_hi=300)
    x = synth.make_inputs(w, 81)
    q, k, v, sl = gu.to_dev(x)
    og, lg = gu.run_gpu(w, x, dev_inputs=(q, k, v, sl))
    kr = k.repeat_interleave(3, dim=1).contiguous()
    vr = v.repeat_interleave(3, dim=1).contiguous()
    wm = w.with_(Hkv=6)
    om, lm = gu.run_gpu(wm, x, dev_inputs=(q, kr, vr, sl))
    assert torch.equal(og, om) and torch.equal(lg, lm)


def test_window_n_equals_causal_bitwise():
    w = W("win", 2, 4, 2, 333, 333, 64, "bf16", True)
    x = synth.make_inputs(w, 91)
    dev = gu.to_dev(x)
    oc, lc = gu.run_gpu(w, x, dev_inputs=dev)
    for win in (333, 5000):
        ow, lw = gu.run_gpu(w, x, dev_inputs=dev, window=win)
        assert torch.equal(oc, ow) and torch.equal(lc, lw)


def test_v_ones_gives_ones():
    w = W("vones", 2, 4, 2, 260, 260, 128, "bf16", True, len_lo=1,
          len_hi=260, amp=2.0)
    x = synth.make_inputs(w, 95)
    q, k, v, sl = gu.to_dev(x)
    v1 = torch.ones_like(v)
    o, lse = gu.run_gpu(w, x, dev_inputs=(q, k, v1, sl))
    live = torch.isfinite(lse)
    assert (o.float()[live] - 1).abs().max().item() <= 8e-3
    assert (o.float()[~live] == 0).all()


@pytest.mark.parametrize("d,N,pos", [
    (64, 256, [40, 100, 200, 255]),
    (128, 256, [40, 100, 200, 255]),
    # 1024 keys at d=64: the key early and late in long rows
    (64, 1024, [40, 300, 700, 1000]),
], ids=["d64", "d128", "d64-long"])
def test_dominant_key_anywhere_in_a_tile(d, N, pos):
    """One key dominates every query's scores by about 200 (log2 units), far
    past the lazy-rescale threshold and past what fp32 can hold as an
    unshifted weight, so the running maximum must see it wherever it sits.
    Batch b puts it at key pos[b]: the first 64-key tile and later ones, both
    32-key halves of a tile.  The output must be that key's V row and lse its
    score (the oracle's exact values)."""
    import oracle
    B, H = 4, 2
    g = torch.Generator().manual_seed(7)
    u = torch.ones(d) / math.sqrt(d)
    amp = math.sqrt(140.0 * math.sqrt(d))  # dominant score amp^2 / sqrt(d)
    q = 0.1 * torch.randn(B, H, N, d, generator=g) + amp * u
    k = 0.1 * torch.randn(B, H, N, d, generator=g)
    for b, j in enumerate(pos):
        k[b, :, j] = amp * u
    v = torch.randn(B, H, N, d, generator=g)
    qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
    scale = 1.0 / math.sqrt(d)
    o, lse = gu.mi.attn(qb.to(gu.DEV), kb.to(gu.DEV), vb.to(gu.DEV),
                        causal=False, scale=scale)
    torch.cuda.synchronize()
    go, gl = gu.host(o, lse)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    ro, rl = oracle.attention(f64(qb), f64(kb), f64(vb), scale=scale)
    # the dominant scores really are far above the rest
    s_dom = (f64(qb)[0, 0, 0] @ f64(kb)[0, 0, pos[0]]) * scale
    assert s_dom * 1.4426950408889634 > 150
    gu.compare(f"dominant-key-d{d}", "bf16", go, gl, ro, rl)
    for b, j in enumerate(pos):
        assert np.abs(go[b] - f64(vb)[b, :, j][:, None, :]).max() <= 2e-2

"""Seeded input generation.

Recipe: numpy Generator(PCG64(seed)); draw, in this order,
  1. the per-sequence valid lengths (only for padded workloads), integers
     uniform in [len_lo, len_hi] inclusive;
  2. Q, then K, then V as float32 standard normals of the full buffer shape,
     each multiplied by the workload's amplitude;
then cast to the storage dtype (bf16: round to nearest even, done by torch).
The fp32 copies returned for the oracle hold exactly the values the GPU sees.
With outlier_channels > 0, that many channels (distinct, drawn next) of
both Q and K are multiplied by outlier_mag, a few large channels shared by
queries and keys.
The output gradient dO of the backward pass comes from its own stream,
Generator(PCG64([seed, 1])): float32 standard normals of the query shape,
cast the same way.
Optionally the padded region (keys at or beyond the valid length, query rows
beyond the live rows) is overwritten with NaN to prove outputs never read it.
Inputs too large to draw on the host (sequences of millions of rows) come
from `device_normal`: torch's Philox generator on the device, seeded with
the given seed, float32 standard normals cast to the storage dtype; only the
rows a check needs are copied back.
"""

import numpy as np
import torch


def _draw(rng, shape, amp):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if amp != 1.0:
        x *= np.float32(amp)
    return x


def make_inputs(w, seed, pad_fill="draw"):
    """Returns a dict:
        q, k, v        torch CPU tensors in the storage dtype, contiguous
        q32, k32, v32  numpy float32 arrays with the same values
        seqlens        numpy int32 [B] or None
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = None
    if w.padded:
        seqlens = rng.integers(w.len_lo, w.len_hi, size=w.B,
                               endpoint=True).astype(np.int32)
    qs = (w.B, w.Hq, w.Nq, w.d)
    ks = (w.B, w.Hkv, w.Nk, w.d)
    arrs = [_draw(rng, qs, w.amp), _draw(rng, ks, w.amp),
            _draw(rng, ks, w.amp)]
    if w.outlier_channels:
        ch = rng.choice(w.d, size=w.outlier_channels, replace=False)
        arrs[0][..., ch] *= np.float32(w.outlier_mag)
        arrs[1][..., ch] *= np.float32(w.outlier_mag)
    if pad_fill == "nan":
        lens = seqlens if seqlens is not None else np.full(w.B, w.Nk)
        for b in range(w.B):
            vl = int(lens[b])
            arrs[1][b, :, vl:] = np.nan
            arrs[2][b, :, vl:] = np.nan
            if w.Nq == w.Nk:
                arrs[0][b, :, vl:] = np.nan
    elif pad_fill != "draw":
        raise ValueError(pad_fill)
    out = {"seqlens": seqlens}
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    for name, a in zip(("q", "k", "v"), arrs):
        t = torch.from_numpy(a).to(tdt).contiguous()
        out[name] = t
        out[name + "32"] = a if tdt == torch.float32 else \
            t.to(torch.float32).numpy()
    return out


def make_dout(w, seed, pad_fill="draw"):
    """dO for the backward pass: (torch CPU tensor in the storage dtype,
    numpy float32 copy with the same values).  pad_fill="nan" writes NaN into
    the rows of dead queries (Nq == Nk, rows at or beyond the valid length,
    lengths from make_inputs with the same seed)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    a = _draw(rng, (w.B, w.Hq, w.Nq, w.d), 1.0)
    if pad_fill == "nan" and w.Nq == w.Nk and w.padded:
        lens = make_inputs(w, seed)["seqlens"]
        for b in range(w.B):
            a[b, :, int(lens[b]):] = np.nan
    elif pad_fill not in ("draw", "nan"):
        raise ValueError(pad_fill)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    t = torch.from_numpy(a).to(tdt).contiguous()
    return t, (a if tdt == torch.float32 else t.to(torch.float32).numpy())


def make_signs(d, seed):
    """The random diagonal of the FP8 path's incoherent processing: d
    entries +1 / -1 (int8), from Generator(PCG64([seed, 2]))."""
    rng = np.random.Generator(np.random.PCG64([seed, 2]))
    return rng.choice(np.array([-1, 1], dtype=np.int8), size=d)


def device_normal(shape, seed, device, dtype=torch.bfloat16):
    """float32 standard normals of `shape` drawn on `device` from
    torch.Generator(device).manual_seed(seed), cast to `dtype` (round to
    nearest even) one slice of the leading dimension at a time, so that the
    float32 draw of only one slice is held at once."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        out[i] = torch.randn(shape[1:], generator=g, device=device,
                             dtype=torch.float32).to(dtype)
    return out

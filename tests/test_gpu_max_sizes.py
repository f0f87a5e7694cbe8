"""GPU parity at the largest sizes the library accepts, on rows the oracle
computes one by one.

* Prefill: a head's query rows one tile short of the 2^31-byte limit of the
  prefill kernel's 32-bit query addressing (Nq = Nk = 8388544 rows at
  d = 128, two query heads on one K/V head), causal with a 64-key window, so
  that the launch stays short while its blocks, tiles and offsets span the
  whole range.
* Decode: a cache of 68157440 keys (17 GB per K or V tensor), more than
  65535 splits of 1024 keys, so the split size doubles to 2048; a window of
  2048 keys plus 4 sink keys keeps the oracle's work small, and the two
  sequences' valid lengths differ, so the window sits near the end of a
  17 GB buffer in one and inside it in the other.

Inputs are drawn on the device (synth.device_normal); the keys a sampled row
sees are copied back and the oracle attends over exactly those keys.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_self_attention_attn_amd as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _rows_host(t, b, h, lo, hi):
    return t[b, h, lo:hi].float().cpu().numpy()[None, None]


def test_prefill_query_rows_at_the_2gib_limit():
    d, n, g = 128, (1 << 31) // (2 * 128) - 64, 2
    window = 64
    gu.say(f"[gpu] prefill max size: B=1 Hq={g} Hkv=1 Nq=Nk={n} d={d} "
           f"causal window={window}")
    q = synth.device_normal((1, g, n, d), 71, gu.DEV)
    k = synth.device_normal((1, 1, n, d), 72, gu.DEV)
    v = synth.device_normal((1, 1, n, d), 73, gu.DEV)
    o, lse = mi.attn(q, k, v, causal=True, window=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(74)
    rows = sorted({0, 1, 63, 64, 127, 128, n // 2, n - 129, n - 128, n - 65,
                   n - 64, n - 2, n - 1,
                   *map(int, rng.integers(0, n, size=40))})
    scale = 1.0 / np.sqrt(d)
    for h in range(g):
        for i in rows:
            lo = max(0, i - window + 1)
            # the row's keys, lo .. i: as one query at the end of a chunk of
            # i + 1 - lo keys it sees every one of them under the causal mask
            ro, rl = oracle.attention(_rows_host(q, 0, h, i, i + 1),
                                      _rows_host(k, 0, 0, lo, i + 1),
                                      _rows_host(v, 0, 0, lo, i + 1),
                                      scale=scale, causal=True)
            go = o[0, h, i].float().cpu().numpy().astype(np.float64)
            gl = lse[0, h, i:i + 1].cpu().numpy().astype(np.float64)
            gu.compare(f"prefill-max h={h} row={i}", "bf16", go[None],
                       gl, ro[0, 0], rl[0, 0])
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_decode_cache_beyond_65535_splits():
    d, g, nk = 128, 4, 65 << 20
    window, sinks = 2048, 4
    lens = np.array([nk, nk - 12345], dtype=np.int32)
    gu.say(f"[gpu] decode max size: B=2 Hq={g} Hkv=1 Nk={nk} d={d} "
           f"window={window} sinks={sinks} lens={lens.tolist()}")
    q = synth.device_normal((2, g, 1, d), 81, gu.DEV)
    k = synth.device_normal((2, 1, nk, d), 82, gu.DEV)
    v = synth.device_normal((2, 1, nk, d), 83, gu.DEV)
    sl = torch.from_numpy(lens).to(gu.DEV)
    o, lse = mi.attn(q, k, v, causal=True, window=window, sinks=sinks,
                     seqlens=sl)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    for b in range(2):
        L = int(lens[b])
        # the keys row 0 (position L - 1) sees: sinks 0 .. 3 and the window
        # L - 2048 .. L - 1 (disjoint here); as one query at the end of a
        # chunk of those keys it sees every one of them
        kk = np.concatenate([_rows_host(k, b, 0, 0, sinks),
                             _rows_host(k, b, 0, L - window, L)], axis=2)
        vv = np.concatenate([_rows_host(v, b, 0, 0, sinks),
                             _rows_host(v, b, 0, L - window, L)], axis=2)
        for h in range(g):
            ro, rl = oracle.attention(_rows_host(q, b, h, 0, 1), kk, vv,
                                      scale=scale, causal=True)
            go = o[b, h, 0].float().cpu().numpy().astype(np.float64)
            gl = lse[b, h, 0:1].cpu().numpy().astype(np.float64)
            gu.compare(f"decode-max b={b} h={h}", "bf16", go[None], gl,
                       ro[0, 0], rl[0, 0])
    del q, k, v, o, lse
    torch.cuda.empty_cache()

"""The hot path inside a captured HIP graph: the headline prefill (long
enough that its light causal blocks come from the run-time ticket queue),
the decode step (split partials in the library's workspace) and the fp32
case, captured once and replayed several times.  Between the replays the
program runs the same calls eagerly (which advances the host's ring of
ticket-counter sets) and synchronises; every replay must equal the eager
result bit for bit (the kernels are deterministic).  The eager calls come
first, so the workspace already has its size when the graph is captured
(growing it frees and allocates memory, which a capture cannot hold).
"""

import pytest
import torch

import synth
import transformer_self_attention_attn_amd as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _calls(inputs, outs):
    for (q, k, v, sl, causal), (o, lse) in zip(inputs, outs):
        mi.attn(q, k, v, causal=causal, seqlens=sl, out=o, lse=lse)


def test_graph_replays_match_eager():
    specs = [(synth.by_name("gqa-causal-prefill"), 3),
             (synth.by_name("decode-gqa"), 5),
             (synth.by_name("fp32-single-head"), 1)]
    inputs = []
    for w, seed in specs:
        x = synth.make_inputs(w, seed)
        q, k, v, sl = gu.to_dev(x)
        inputs.append((q, k, v, sl, w.causal))
    gu.say("[gpu] graph: " + ", ".join(w.name for w, _ in specs))

    def fresh():
        return [(torch.empty_like(q),
                 torch.empty(q.shape[:3], dtype=torch.float32,
                             device=q.device))
                for q, _, _, _, _ in inputs]

    ref = fresh()
    _calls(inputs, ref)
    torch.cuda.synchronize()

    got = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _calls(inputs, got)
    torch.cuda.synchronize()

    eager = fresh()
    for rep in range(4):
        for o, lse in got:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for (w, _), (o, lse), (ro, rl) in zip(specs, got, ref):
            assert torch.equal(o, ro), f"replay {rep}: {w.name} o differs"
            assert torch.equal(lse.nan_to_num(0.0), rl.nan_to_num(0.0)) and \
                torch.equal(lse.isnan(), rl.isnan()), \
                f"replay {rep}: {w.name} lse differs"
        # the program's own eager work between replays
        _calls(inputs, eager)
        torch.cuda.synchronize()
        for (w, _), (o, lse), (ro, rl) in zip(specs, eager, ref):
            assert torch.equal(o, ro), f"eager {rep}: {w.name} o differs"
        gu.say(f"  replay {rep}: bitwise equal to the eager calls")


def test_graph_backward_and_fp8_match_eager():
    """The backward pass (workspace, three launches) and the FP8 path
    (quantizer, then the forward on the codes with its run-time tail) of
    the headline prefill, captured and replayed the same way; the tensors
    a call allocates during the capture come from the graph's own pool and
    each replay rewrites them."""
    w = synth.by_name("gqa-causal-prefill")
    x = synth.make_inputs(w, 3)
    q, k, v, _ = gu.to_dev(x)
    dout = synth.make_dout(w, 3)[0].to(gu.DEV)
    signs = torch.from_numpy(synth.make_signs(w.d, 3)).to(gu.DEV)
    gu.say("[gpu] graph: backward and FP8 on gqa-causal-prefill")
    o, lse = mi.attn(q, k, v, causal=True)

    def calls():
        grads = mi.attn_backward(q, k, v, o, lse, dout, causal=True)
        z = mi.fp8_quantize(q, k, v, signs=signs)
        o8, l8 = mi.attn_fp8(z, causal=True)
        return grads + (o8, l8)

    ref = calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = calls()
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "o8", "lse8")
    for rep in range(3):
        for t in got:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(names, got, ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs"
        again = calls()
        torch.cuda.synchronize()
        for name, t, r in zip(names, again, ref):
            assert torch.equal(t, r), f"eager {rep}: {name} differs"
        gu.say(f"  replay {rep}: bitwise equal to the eager calls")

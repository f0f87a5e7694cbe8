"""Workload shapes: one fp32 correctness case, three bf16 prefill cases and
one bf16 decode step, then three shapes with 1 < Nq < Nk (new rows against a
cache, cross-attention) and three local-window variants (a window on both
sides, a window plus sink keys).

They stand in for the pages' workloads (GPT-2 / BERT / long-context models);
no dataset or trained weight is used: Q, K and V are i.i.d. normal draws of
the stated shape, and valid lengths are uniform draws (right padding).
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str            # "fp32" or "bf16"
    causal: bool
    window: int = 0       # 0 = no window (the left limit: pos - j < window)
    window_right: int = 0  # 0 = no right limit (j - pos < window_right)
    sinks: int = 0        # keys j < sinks are always kept (within causal/valid)
    len_lo: int = 0       # valid lengths drawn uniformly from [len_lo, len_hi]
    len_hi: int = 0       # (both 0: every sequence is full length)
    amp: float = 1.0      # Q, K, V = amp * N(0, 1)
    outlier_channels: int = 0  # channels of Q and K scaled by outlier_mag
    outlier_mag: float = 1.0

    @property
    def padded(self):
        return self.len_hi > 0

    @property
    def scale(self):
        return 1.0 / (self.d ** 0.5)

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = (
    # single head, fp32, no mask: the small correctness case
    Workload("fp32-single-head", B=1, Hq=1, Hkv=1, Nq=128, Nk=128, d=64,
             dtype="fp32", causal=False),
    # GPT-2-small-shaped causal MHA with right padding
    Workload("gpt2-small-causal-padded", B=16, Hq=12, Hkv=12, Nq=1024,
             Nk=1024, d=64, dtype="bf16", causal=True, len_lo=512,
             len_hi=1024),
    # grouped-query causal prefill, 7 query heads per K/V head
    Workload("gqa-causal-prefill", B=4, Hq=28, Hkv=4, Nq=4096, Nk=4096,
             d=128, dtype="bf16", causal=True, amp=0.5),
    # sliding-window causal attention: self plus the previous 1023 keys
    Workload("sliding-window-causal", B=2, Hq=16, Hkv=16, Nq=16384,
             Nk=16384, d=64, dtype="bf16", causal=True, window=1024),
    # one decode step against a padded KV cache
    Workload("decode-gqa", B=64, Hq=32, Hkv=8, Nq=1, Nk=8192, d=128,
             dtype="bf16", causal=True, len_lo=2048, len_hi=8192),
    # speculative decoding: 4 draft tokens checked against decode-gqa's
    # caches in one call (G * Nq = 16 query columns per K/V head)
    Workload("decode-chunk4-gqa", B=64, Hq=32, Hkv=8, Nq=4, Nk=8192, d=128,
             dtype="bf16", causal=True, len_lo=2048, len_hi=8192),
    # -- Nq new rows against a longer key sequence (1 < Nq < Nk) --
    # 32 new tokens after a prompt (the generation setting of the SpAtten
    # review: 992 prompt tokens, 32 generated), GPT-2-small heads, padded cache
    Workload("chunk32-gpt2-causal", B=16, Hq=12, Hkv=12, Nq=32, Nk=1024,
             d=64, dtype="bf16", causal=True, len_lo=512, len_hi=1024),
    # the last 1024-token chunk of an 8192-token prompt, GQA heads
    Workload("chunked-prefill-gqa", B=4, Hq=28, Hkv=4, Nq=1024, Nk=8192,
             d=128, dtype="bf16", causal=True, amp=0.5),
    # encoder-decoder (cross) attention: 1024 decoder queries against padded
    # encoder outputs of up to 2048 tokens, no causal mask
    Workload("cross-attention-padded", B=16, Hq=12, Hkv=12, Nq=1024,
             Nk=2048, d=64, dtype="bf16", causal=False, len_lo=1024,
             len_hi=2048),
    # -- local windows --
    # Longformer-style encoder self-attention: each token sees the 256
    # tokens on either side and itself (no causal mask), 4096-token inputs
    Workload("local-window-bidirectional", B=4, Hq=12, Hkv=12, Nq=4096,
             Nk=4096, d=64, dtype="bf16", causal=False, window=257,
             window_right=257),
    # the sliding-window shape above with the first 4 keys kept as sinks
    Workload("sliding-window-sinks", B=2, Hq=16, Hkv=16, Nq=16384,
             Nk=16384, d=64, dtype="bf16", causal=True, window=1024,
             sinks=4),
    # one decode step over a padded cache that keeps a 2048-key window plus
    # 4 sink keys (the decode-gqa heads, twice the cache length)
    Workload("decode-window-sinks", B=32, Hq=32, Hkv=8, Nq=1, Nk=16384,
             d=128, dtype="bf16", causal=True, window=2048, sinks=4,
             len_lo=4096, len_hi=16384),
)


def by_name(name):
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)

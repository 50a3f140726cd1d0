"""Shapes of the synthetic workloads.

The pages train BERT-Large (1-bit LAMB page, experiments paragraph; 1-bit
Adam article, section 5 table) and GPT-3 1.3B (1-bit Adam article, section 5
table).  No weights or datasets are used: only the parameter shapes are taken,
so that the fused flat momentum buffers have the real sizes and the real
per-tensor segment structure.

BERT-Large is laid out with fused QKV weights, which gives exactly the 302
tensors the 1-bit LAMB page counts when it motivates one fused 1D buffer
(layer-scaling paragraph).  Its first 295 tensors (embeddings, 24 encoder
layers, pooler) are the 335,141,888-element BertModel buffer used by the
1-bit Adam workload.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

Tensor = Tuple[str, int]


def _prod(*dims: int) -> int:
    out = 1
    for d in dims:
        out *= d
    return out


def bert_large_tensors(with_heads: bool = True) -> List[Tensor]:
    """BERT-Large parameter tensors (hidden 1024, FFN 4096, 24 layers,
    vocab 30522, 512 positions, 2 token types), QKV fused per layer."""
    h, f, vocab = 1024, 4096, 30522
    t: List[Tensor] = [
        ("emb.word", _prod(vocab, h)),
        ("emb.pos", _prod(512, h)),
        ("emb.type", _prod(2, h)),
        ("emb.ln.g", h),
        ("emb.ln.b", h),
    ]
    for layer in range(24):
        p = f"l{layer}."
        t += [
            (p + "qkv.w", _prod(3 * h, h)),
            (p + "qkv.b", 3 * h),
            (p + "o.w", _prod(h, h)),
            (p + "o.b", h),
            (p + "ln1.g", h),
            (p + "ln1.b", h),
            (p + "ffn1.w", _prod(f, h)),
            (p + "ffn1.b", f),
            (p + "ffn2.w", _prod(h, f)),
            (p + "ffn2.b", h),
            (p + "ln2.g", h),
            (p + "ln2.b", h),
        ]
    t += [("pooler.w", _prod(h, h)), ("pooler.b", h)]
    if with_heads:
        t += [
            ("mlm.w", _prod(h, h)),
            ("mlm.b", h),
            ("mlm.ln.g", h),
            ("mlm.ln.b", h),
            ("mlm.decoder.b", vocab),
            ("nsp.w", _prod(2, h)),
            ("nsp.b", 2),
        ]
    return t


def gpt13b_tensors() -> List[Tensor]:
    """GPT-style 1.3B tensors: d=2048, FFN 8192, 24 layers, vocab 50257
    embedding (tied output), fused QKV, final LayerNorm.  The workload names
    no position embedding, so none is included."""
    d, f, vocab = 2048, 8192, 50257
    t: List[Tensor] = [("emb.word", _prod(vocab, d))]
    for layer in range(24):
        p = f"l{layer}."
        t += [
            (p + "qkv.w", _prod(3 * d, d)),
            (p + "qkv.b", 3 * d),
            (p + "o.w", _prod(d, d)),
            (p + "o.b", d),
            (p + "ln1.g", d),
            (p + "ln1.b", d),
            (p + "ffn1.w", _prod(f, d)),
            (p + "ffn1.b", f),
            (p + "ffn2.w", _prod(d, f)),
            (p + "ffn2.b", d),
            (p + "ln2.g", d),
            (p + "ln2.b", d),
        ]
    t += [("lnf.g", d), ("lnf.b", d)]
    return t


def segment_offsets(sizes: List[int]) -> List[int]:
    """Prefix offsets [0, s0, s0+s1, ..., total] of consecutive segments."""
    off = [0]
    for s in sizes:
        off.append(off[-1] + s)
    return off


def _pad_to(x: int, m: int) -> int:
    return ((x + m - 1) // m) * m


@dataclass
class Workload:
    """One synthetic workload: buffer sizes, worker count and the knobs the
    pages fix for it.  ``segments`` are the per-tensor element counts (their
    sum is ``N``; a trailing zero-momentum pad segment is included when the
    buffer had to be padded to a multiple of 64*n)."""

    name: str
    kind: str  # "adam", "lamb" or "int8"
    N: int
    n: int
    steps: int
    segments: List[int] = field(default_factory=list)
    seg_names: List[str] = field(default_factory=list)
    pad: int = 0
    clip: float = 0.0  # <= 0 disables the clamp
    reset_interval: int = 0  # 0 disables the periodic error reset
    t0: int = 1
    lr: float = 6e-5
    eps: float = 1e-6
    beta1: float = 0.9
    beta2: float = 0.999
    r_threshold: float = 0.1
    r_min: float = 0.5
    r_max: float = 4.0
    block: int = 256
    sigma_mode: str = ""
    seed: int = 0

    @property
    def L(self) -> int:
        return self.N // self.n if self.n else 0


def _c1() -> Workload:
    return Workload(
        name="adam_2^20_x4", kind="adam", N=1 << 20, n=4, steps=10,
        segments=[1 << 20], seg_names=["flat"], sigma_mode="const1e-3", seed=1,
    )


def _c2() -> Workload:
    tensors = bert_large_tensors(with_heads=False)
    N = sum(s for _, s in tensors)
    assert N == 335_141_888
    # sigma is drawn per 2^20-element segment (320 segments, the last short)
    segs = []
    left = N
    while left > 0:
        segs.append(min(1 << 20, left))
        left -= segs[-1]
    return Workload(
        name="bert_large_335M_x8", kind="adam", N=N, n=8, steps=20,
        segments=segs, seg_names=[f"seg{i}" for i in range(len(segs))],
        sigma_mode="loguniform_1e-5_1e-2", seed=2,
    )


def _c3() -> Workload:
    tensors = bert_large_tensors(with_heads=True)
    raw = sum(s for _, s in tensors)
    assert len(tensors) == 302 and raw == 336_226_108
    n = 16
    N = _pad_to(raw, 64 * n)
    segs = [s for _, s in tensors]
    names = [nm for nm, _ in tensors]
    if N > raw:
        segs.append(N - raw)
        names.append("pad")
    return Workload(
        name="bert_large_lamb_302t_x16", kind="lamb", N=N, n=n, steps=20,
        segments=segs, seg_names=names, pad=N - raw,
        sigma_mode="loguniform_1e-6_1e-1", seed=3,
    )


def _c4() -> Workload:
    return Workload(
        name="int8_sr_2^30", kind="int8", N=1 << 30, n=1, steps=10,
        segments=[1 << 30], seg_names=["flat"], block=256,
        sigma_mode="laplace_1e-3_outliers", seed=4,
    )


def _c5() -> Workload:
    tensors = gpt13b_tensors()
    N = sum(s for _, s in tensors)
    assert len(tensors) == 291 and N == 1_311_528_960
    n = 16
    assert N % (64 * n) == 0
    return Workload(
        name="gpt_1.3B_x16", kind="adam", N=N, n=n, steps=5,
        segments=[s for _, s in tensors], seg_names=[nm for nm, _ in tensors],
        clip=2.0, reset_interval=2000, sigma_mode="loguniform_1e-5_1e-2", seed=5,
    )


WORKLOADS = {
    "adam_2^20_x4": _c1,
    "bert_large_335M_x8": _c2,
    "bert_large_lamb_302t_x16": _c3,
    "int8_sr_2^30": _c4,
    "gpt_1.3B_x16": _c5,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]()


def scaled_lamb(n: int, target_elems: int, seed: int = 3) -> Workload:
    """A small LAMB workload with the BERT-Large segment *structure* (the same
    mix of tiny bias/LayerNorm vectors and large matrices) scaled down so the
    oracle finishes in seconds: every tensor keeps at least its vector size
    class but matrices are shrunk by a common factor."""
    tensors = bert_large_tensors(with_heads=True)
    total = sum(s for _, s in tensors)
    factor = max(1, total // target_elems)
    segs = []
    for _, s in tensors:
        if s >= 1 << 20:
            segs.append(max(64, s // factor))
        else:
            segs.append(s)
    raw = sum(segs)
    N = _pad_to(raw, 64 * n)
    names = [nm for nm, _ in tensors]
    if N > raw:
        segs.append(N - raw)
        names.append("pad")
    return Workload(
        name=f"lamb_scaled_{N}_x{n}", kind="lamb", N=N, n=n, steps=4,
        segments=segs, seg_names=names, pad=N - raw,
        sigma_mode="loguniform_1e-6_1e-1", seed=seed,
    )

"""Workload descriptions: parameter-tensor lists, worker counts and value recipes.

The 1-bit Adam review (nubint.ai, "1-bit Adam: Communication Efficient
Large-Scale Training with Adam's Convergence Speed", Main results) reports
training BERT-Large, BERT (SQuAD) and ResNet models; the QSDP review
(abstract) names GPT models up to 1.3B parameters.  None of those datasets or
weights is used: an optimizer step depends only on tensor shapes and value
statistics, so each workload below is a list of parameter shapes plus the
distributions its synthetic values are drawn from.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Tuple

Shape = Tuple[int, ...]


def _numel(shape: Shape) -> int:
    return int(math.prod(shape))


def _bert_layers(hidden: int, ffn: int, layers: int) -> List[Tuple[str, Shape]]:
    out: List[Tuple[str, Shape]] = []
    for i in range(layers):
        p = f"layer{i}."
        out += [
            (p + "attn.q.weight", (hidden, hidden)), (p + "attn.q.bias", (hidden,)),
            (p + "attn.k.weight", (hidden, hidden)), (p + "attn.k.bias", (hidden,)),
            (p + "attn.v.weight", (hidden, hidden)), (p + "attn.v.bias", (hidden,)),
            (p + "attn.out.weight", (hidden, hidden)), (p + "attn.out.bias", (hidden,)),
            (p + "ln1.gamma", (hidden,)), (p + "ln1.beta", (hidden,)),
            (p + "ffn.w1", (ffn, hidden)), (p + "ffn.b1", (ffn,)),
            (p + "ffn.w2", (hidden, ffn)), (p + "ffn.b2", (hidden,)),
            (p + "ln2.gamma", (hidden,)), (p + "ln2.beta", (hidden,)),
        ]
    return out


def bert_large() -> List[Tuple[str, Shape]]:
    """24 layers, hidden 1024, FFN 4096, Q/K/V kept separate, plus a 30522x1024
    token embedding and a 512x1024 position embedding: 386 tensors."""
    return _bert_layers(1024, 4096, 24) + [
        ("embed.token", (30522, 1024)), ("embed.position", (512, 1024))]


def bert_base() -> List[Tuple[str, Shape]]:
    """12 layers, hidden 768, FFN 3072, plus a 30522x768 embedding: 193 tensors."""
    return _bert_layers(768, 3072, 12) + [("embed.token", (30522, 768))]


def gpt_1p3b() -> List[Tuple[str, Shape]]:
    """24 layers, d 2048, FFN 8192, fused QKV, a tied 50257x2048 embedding
    counted once and a final LayerNorm: 291 tensors."""
    d, f = 2048, 8192
    out: List[Tuple[str, Shape]] = []
    for i in range(24):
        p = f"h{i}."
        out += [
            (p + "ln1.gamma", (d,)), (p + "ln1.beta", (d,)),
            (p + "attn.qkv.weight", (3 * d, d)), (p + "attn.qkv.bias", (3 * d,)),
            (p + "attn.out.weight", (d, d)), (p + "attn.out.bias", (d,)),
            (p + "ln2.gamma", (d,)), (p + "ln2.beta", (d,)),
            (p + "mlp.w1", (f, d)), (p + "mlp.b1", (f,)),
            (p + "mlp.w2", (d, f)), (p + "mlp.b2", (d,)),
        ]
    out += [("wte", (50257, d)), ("ln_f.gamma", (d,)), ("ln_f.beta", (d,))]
    return out


def resnet50() -> List[Tuple[str, Shape]]:
    """53 bias-free convolutions each followed by BatchNorm gamma/beta, and a
    1000x2048 classifier with bias: 161 tensors, 25,557,032 elements."""
    out: List[Tuple[str, Shape]] = [
        ("stem.conv", (64, 3, 7, 7)), ("stem.bn.gamma", (64,)), ("stem.bn.beta", (64,))]

    def conv_bn(name: str, shape: Shape) -> None:
        out.append((name + ".conv", shape))
        out.append((name + ".bn.gamma", (shape[0],)))
        out.append((name + ".bn.beta", (shape[0],)))

    in_ch = 64
    for s, (width, blocks) in enumerate([(64, 3), (128, 4), (256, 6), (512, 3)]):
        for b in range(blocks):
            p = f"stage{s}.block{b}."
            conv_bn(p + "reduce", (width, in_ch, 1, 1))
            conv_bn(p + "spatial", (width, width, 3, 3))
            conv_bn(p + "expand", (4 * width, width, 1, 1))
            if b == 0:
                conv_bn(p + "downsample", (4 * width, in_ch, 1, 1))
            in_ch = 4 * width
    out += [("fc.weight", (1000, 2048)), ("fc.bias", (1000,))]
    return out


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    ``g_sigma`` is the standard deviation of the per-worker gradients;
    ``g_shared`` the fraction of gradient variance shared by all workers
    (0 for independent draws); ``v_kind`` selects the frozen-variance recipe:
    ``"sq_normal"`` gives v = |N(0, v_a)|^2 + v_b, ``"lognormal"`` gives
    v = exp(N(v_a, v_b)).
    """
    name: str
    tensors: Tuple[Tuple[str, Shape], ...]
    workers: int
    grad_dtype: str            # "f32" or "bf16"
    steps: int
    g_sigma: float
    v_kind: str
    v_a: float
    v_b: float
    g_shared: float = 0.0
    p_sigma: float = 0.02
    beta1: float = 0.9
    lr: float = 1e-4
    eps: float = 1e-8
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def numel(self) -> List[int]:
        return [_numel(s) for _, s in self.tensors]

    @property
    def num_tensors(self) -> int:
        return len(self.tensors)


def tensor_list(name: str) -> List[Tuple[str, Shape]]:
    return list(WORKLOADS[name].tensors)


def padded_layout(numel: List[int]) -> Tuple[List[int], int]:
    """Flat layout shared by every flat buffer: tensor t starts at element
    ``off[t]``, a multiple of 64 (one 64-bit sign word), and the padded length
    is ``N = off[T]``.  Returns (off[0..T], N)."""
    off = [0]
    for n in numel:
        off.append(off[-1] + (n + 63) // 64 * 64)
    return off, off[-1]


WORKLOADS = {
    "single_tensor_2p20": Workload(
        name="single_tensor_2p20", tensors=(("w", (1 << 20,)),), workers=4,
        grad_dtype="f32", steps=10, g_sigma=1e-3, v_kind="sq_normal", v_a=1e-3, v_b=1e-12),
    "bert_large": Workload(
        name="bert_large", tensors=tuple(bert_large()), workers=8, grad_dtype="f32",
        steps=20, g_sigma=1e-3, v_kind="lognormal", v_a=-14.0, v_b=2.0),
    "bert_base_w64": Workload(
        name="bert_base_w64", tensors=tuple(bert_base()), workers=64, grad_dtype="f32",
        steps=10, g_sigma=1e-3, v_kind="lognormal", v_a=-14.0, v_b=2.0, g_shared=0.7),
    "gpt_1p3b_bf16": Workload(
        name="gpt_1p3b_bf16", tensors=tuple(gpt_1p3b()), workers=8, grad_dtype="bf16",
        steps=5, g_sigma=5e-4, v_kind="lognormal", v_a=-15.0, v_b=2.0),
    "resnet50_w32": Workload(
        name="resnet50_w32", tensors=tuple(resnet50()), workers=32, grad_dtype="f32",
        steps=20, g_sigma=1e-2, v_kind="sq_normal", v_a=1e-2, v_b=1e-12),
}

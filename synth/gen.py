"""Seeded generator for qwen3_5-MoE-shaped routed-expert layers (canonical layout).

Canonical layout (the MLX-style affine layout the pages' loaders read):
  * a quantised matrix W[rows, cols] is `codes` (uint32) of shape
    [rows, cols*bits/32]: each row is an LSB-first bitstream, element i of the
    row holding stream bits [bits*i, bits*i+bits), stream bit t being bit
    (t mod 32) of word t//32;
  * `scales` / `biases` are uint16 bit patterns (bf16 or fp16) of shape
    [rows, cols/group]; symmetric tensors have no biases and store the code
    offset-binary (nibble u = q + 8);
  * a dense row (the bf16 shared-expert gate of the W4A16 export) stores its
    bf16 bit patterns in `codes` as uint16 [rows, cols].
Stacked routed experts carry a leading expert axis.

Only random draws and dtype rounding happen here. Codes are drawn as random
32-bit words, which makes every code uniform for any width (3-bit included).

Distributions (per workload; see the recipe table in the design notes):
  * scale ~ U(0.002, 0.02), rounded to the scale dtype;
  * 4-bit affine: bias = -8*scale + N(0, 1e-3) (standard deviation 1e-3);
  * 3-bit affine: bias = -4*scale exactly;
  * 8-bit affine: bias = -128*scale + N(0, 1e-3);
  * 2-, 5- and 6-bit affine: bias = -c*scale + N(0, 1e-3), c = 2, 16, 32;
  * router and gate row: scale and noise multiplied by a closed-form factor
    so the fp32 logits of x ~ N(0,1) have unit variance
    (factor = 1/sqrt(H * E[w^2]), with E[w^2] = E[s^2]*E[(q-c)^2] + noise^2);
  * x ~ N(0,1) in bf16 (fp16 for the W4A16 workload);
  * Zipf-skewed routing: per-expert logit bias -1.1*ln(rank), rank a seeded
    permutation of 1..E.
Every tensor is drawn from numpy.random.default_rng([cfg, layer, kind, index])
so any one expert can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

AFFINE, SYMMETRIC, DENSE, MXFP4 = 0, 1, 2, 3
BF16, FP16, E8M0 = 0, 1, 2

KIND = dict(router=0, gate_row=1, gate=2, up=3, down=4, sh_gate=5, sh_up=6,
            sh_down=7, x=8, zipf=9)


@dataclass(frozen=True)
class QFormat:
    bits: int          # 2..8 (16 for DENSE)
    group: int         # 32, 64 or 128 (0 for DENSE)
    mode: int          # AFFINE, SYMMETRIC, DENSE, MXFP4
    scale_dtype: int   # BF16, FP16 (value dtype for DENSE) or E8M0 (uint8 exponents)


Q4G64 = QFormat(4, 64, AFFINE, BF16)
Q3G64 = QFormat(3, 64, AFFINE, BF16)
Q8G64 = QFormat(8, 64, AFFINE, BF16)
Q2G64 = QFormat(2, 64, AFFINE, BF16)
Q5G64 = QFormat(5, 64, AFFINE, BF16)
Q6G64 = QFormat(6, 64, AFFINE, BF16)
S4G128 = QFormat(4, 128, SYMMETRIC, FP16)
MX4G32 = QFormat(4, 32, MXFP4, E8M0)
DENSE_BF16 = QFormat(16, 0, DENSE, BF16)


def words_per_row(fmt: QFormat, cols: int) -> int:
    assert fmt.mode != DENSE
    assert (cols * fmt.bits) % 32 == 0
    return cols * fmt.bits // 32


@dataclass
class QTensor:
    fmt: QFormat
    rows: int
    cols: int
    codes: np.ndarray
    scales: Optional[np.ndarray] = None
    biases: Optional[np.ndarray] = None


@dataclass(frozen=True)
class ConfigSpec:
    cfg_id: int
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    act: int
    router: QFormat
    gate_row: QFormat
    routed: QFormat
    shared: QFormat
    rows: Tuple[int, ...]
    layers: int
    bias: str = "none"          # "none" | "zipf"
    zipf_s: float = 1.1


@dataclass
class Layer:
    spec: ConfigSpec
    layer: int
    router: QTensor
    gate_row: QTensor
    gate: QTensor
    up: QTensor
    down: QTensor
    sh_gate: QTensor
    sh_up: QTensor
    sh_down: QTensor
    logit_bias: Optional[np.ndarray] = None


_H, _E, _K, _I = 2048, 256, 8, 512
CONFIGS = {
    0: ConfigSpec(0, "decode-1row-q4g64", _H, _E, _K, _I, _I, BF16,
                  Q4G64, Q4G64, Q4G64, Q4G64, rows=(1,), layers=1),
    1: ConfigSpec(1, "decode-8rows-40layers-q4g64", _H, _E, _K, _I, _I, BF16,
                  Q4G64, Q4G64, Q4G64, Q4G64, rows=(8,), layers=40),
    2: ConfigSpec(2, "decode-mixed-q3g64-routed", _H, _E, _K, _I, _I, BF16,
                  Q8G64, Q8G64, Q3G64, Q4G64, rows=(1, 8), layers=40),
    3: ConfigSpec(3, "prefill-512rows-q4g64", _H, _E, _K, _I, _I, BF16,
                  Q4G64, Q4G64, Q4G64, Q4G64, rows=(512,), layers=1),
    4: ConfigSpec(4, "prefill-2048rows-w4a16-zipf", _H, _E, _K, _I, _I, FP16,
                  S4G128, DENSE_BF16, S4G128, S4G128, rows=(2048,), layers=1,
                  bias="zipf"),
}


def make_tiny_config(base: ConfigSpec, cfg_id: int = 100, hidden=256, n_experts=16,
                     top_k=4, inter=128, shared_inter=128) -> ConfigSpec:
    """Same formats as `base`, at small shapes (CPU tests)."""
    return replace(base, cfg_id=cfg_id, name=base.name + "-tiny", hidden=hidden,
                   n_experts=n_experts, top_k=top_k, inter=inter,
                   shared_inter=shared_inter)


# ---------------------------------------------------------------- rounding
def f32_to_bf16_bits(v) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); uint16 bits."""
    f = np.asarray(v, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _bf16_bits_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_fp16_bits(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _to_bits(vals: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(vals) if dtype == BF16 else f64_to_fp16_bits(vals)


def _from_bits(bits: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == BF16:
        return _bf16_bits_to_f64(bits)
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# ------------------------------------------------------------- distributions
_ES2 = (0.002 ** 2 + 0.002 * 0.02 + 0.02 ** 2) / 3.0   # E[s^2], s ~ U(0.002, 0.02)


def _code_offset(fmt: QFormat) -> int:
    return {2: 2, 3: 4, 4: 8, 5: 16, 6: 32, 8: 128}[fmt.bits]


def _noise_std(fmt: QFormat) -> float:
    if fmt.mode != AFFINE or fmt.bits == 3:
        return 0.0
    return 1e-3


def _unit_logit_factor(fmt: QFormat, hidden: int) -> float:
    """Multiplier for scale and noise giving logits of unit variance for x ~ N(0,1)."""
    if fmt.mode == DENSE:
        return 1.0
    n = 1 << fmt.bits
    c = _code_offset(fmt)
    # E[(q-c)^2] for q uniform on 0..n-1 (symmetric: q-c is the signed code)
    m2 = (n * n - 1) / 12.0 + ((n - 1) / 2.0 - c) ** 2
    ew2 = _ES2 * m2 + _noise_std(fmt) ** 2
    return 1.0 / np.sqrt(hidden * ew2)


def _draw_qtensor(rng: np.random.Generator, fmt: QFormat, rows: int, cols: int,
                  mult: float = 1.0) -> QTensor:
    if fmt.mode == DENSE:
        vals = rng.standard_normal((rows, cols)) / np.sqrt(cols)
        return QTensor(fmt, rows, cols, _to_bits(vals, fmt.scale_dtype))
    wpr = words_per_row(fmt, cols)
    codes = rng.integers(0, 1 << 32, size=(rows, wpr), dtype=np.uint32)
    ng = cols // fmt.group
    if fmt.mode == MXFP4:
        # every 4-bit code equally likely; block scales 2^-9 .. 2^-6 uniformly
        # (weights of rms ~0.03, the order of the affine draws' ~0.06)
        return QTensor(fmt, rows, cols, codes,
                       rng.integers(127 - 9, 127 - 5, size=(rows, ng)).astype(np.uint8), None)
    s_bits = _to_bits(rng.uniform(0.002, 0.02, size=(rows, ng)) * mult, fmt.scale_dtype)
    if fmt.mode == SYMMETRIC:
        return QTensor(fmt, rows, cols, codes, s_bits, None)
    s = _from_bits(s_bits, fmt.scale_dtype)
    b = -_code_offset(fmt) * s
    sd = _noise_std(fmt)
    if sd > 0:
        b = b + rng.normal(0.0, sd * mult, size=(rows, ng))
    return QTensor(fmt, rows, cols, codes, s_bits, _to_bits(b, fmt.scale_dtype))


def _rng(spec: ConfigSpec, layer: int, kind: str, index: int) -> np.random.Generator:
    return np.random.default_rng([spec.cfg_id, layer, KIND[kind], index])


def _stack(ts):
    t0 = ts[0]
    return QTensor(t0.fmt, t0.rows, t0.cols,
                   np.stack([t.codes for t in ts]),
                   None if t0.scales is None else np.stack([t.scales for t in ts]),
                   None if t0.biases is None else np.stack([t.biases for t in ts]))


def make_expert(spec: ConfigSpec, layer: int, e: int):
    """(gate [I,H], up [I,H], down [H,I]) of routed expert e; e == E is the shared expert."""
    H = spec.hidden
    if e == spec.n_experts:
        fmt, I = spec.shared, spec.shared_inter
        kinds = ("sh_gate", "sh_up", "sh_down")
        e_idx = 0
    else:
        fmt, I = spec.routed, spec.inter
        kinds = ("gate", "up", "down")
        e_idx = e
    g = _draw_qtensor(_rng(spec, layer, kinds[0], e_idx), fmt, I, H)
    u = _draw_qtensor(_rng(spec, layer, kinds[1], e_idx), fmt, I, H)
    d = _draw_qtensor(_rng(spec, layer, kinds[2], e_idx), fmt, H, I)
    return g, u, d


def make_logit_bias(spec: ConfigSpec, layer: int) -> Optional[np.ndarray]:
    if spec.bias == "none":
        return None
    ranks = _rng(spec, layer, "zipf", 0).permutation(spec.n_experts) + 1
    return (-spec.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)


def make_layer(spec: ConfigSpec, layer: int = 0) -> Layer:
    H, E = spec.hidden, spec.n_experts
    router = _draw_qtensor(_rng(spec, layer, "router", 0), spec.router, E, H,
                           _unit_logit_factor(spec.router, H))
    gate_row = _draw_qtensor(_rng(spec, layer, "gate_row", 0), spec.gate_row, 1, H,
                             _unit_logit_factor(spec.gate_row, H))
    experts = [make_expert(spec, layer, e) for e in range(E)]
    sg, su, sd = make_expert(spec, layer, E)
    return Layer(spec, layer, router, gate_row,
                 _stack([x[0] for x in experts]), _stack([x[1] for x in experts]),
                 _stack([x[2] for x in experts]), sg, su, sd,
                 make_logit_bias(spec, layer))


def make_x(spec: ConfigSpec, layer: int, rows: int, rep: int = 0) -> np.ndarray:
    """Activations [rows, H] as uint16 bits (bf16, or fp16 for FP16 activations)."""
    v = _rng(spec, layer, "x", rep).standard_normal((rows, spec.hidden))
    return _to_bits(v, spec.act)

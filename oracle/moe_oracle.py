"""FP64 CPU oracle of the routed-expert FFN with low-bit affine expert weights.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or call this module. The product (the HIP library
and its Python binding) never does, and shares no code with it.

It evaluates the plain definition in float64: it reads the canonical
(MLX-style) layout produced by `synth`, unpacks codes with numpy's bit
routines, dequantises, and runs the layer with numpy matmuls. No blocking,
fusion or reordering beyond those library steps.

Sources (page title, then section):
  * "qwen3_5_moe on native CUDA with 3-bit routed experts ... #803", Activity,
    the "Progress on the 4-bit gate" comment: fp32 logits over the experts and
    the shared expert's gate row; top-k by logit, ties to the lower id; weights
    exp(l - l_top) over the k; the shared expert as one more slot weighted by
    sigmoid(gate); the slots' fma sum; SwiGLU epilogue (gate and up).
  * same page, "What I want to run": MLX affine, groups of 64; routed experts
    3-bit, other weights 4-bit, routers and the shared gate 8-bit.
  * "Sage-A1.5 (qwen3_5 MoE 35B-A3B) on the XPU backend ... #1329", Proposal:
    MLX 4-bit affine 4/64 export; 256 experts, top-8.
  * "Sage-1.5-W4A16" model card, Model details and Recipe: int4 symmetric
    weights, group 128, 16-bit compute, no activation quantisation; the
    shared-expert gate kept in BF16.
  * same card, Performance, the decode speed table: a reference checkpoint
    whose experts are MXFP4. The pages name the format and do not define it;
    `dequant` takes the public OCP Microscaling (MX) v1.0 definition: blocks
    of 32 FP4 E2M1 elements sharing one E8M0 scale (parity of real MXFP4
    checkpoints against this layout is unpinned).
Readings where the pages are silent (each listed in the design notes):
  * the weights are divided by their sum over the k picks (renormalised softmax);
  * the affine dequantisation is w = scale*q + bias per group, the symmetric
    one w = scale*(u - 8) for the stored nibble u;
  * MXFP4: element i of a row is stream nibble i (low nibble first, as for
    every other width), w = e2m1(nibble) * 2^(e - 127) for its block's
    exponent byte e, e = 255 giving NaN; no bias term;
  * SwiGLU is h = silu(gate.x) * (up.x), silu(z) = z*sigmoid(z);
  * the shared gate is one row of H weights with no bias: sigma(row.x);
  * NaN orders above +inf above every finite value, then the lower id;
  * the pick is decided on the fp32-rounded logits (the pages' precision);
    weights, gate and outputs are evaluated from the float64 logits.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Optional, Tuple

import numpy as np

AFFINE, SYMMETRIC, DENSE, MXFP4 = 0, 1, 2, 3
BF16, FP16, E8M0 = 0, 1, 2


# ------------------------------------------------------------------ numbers
def half_bits_to_f64(bits, dtype: int) -> np.ndarray:
    """Exact conversion of bf16 / fp16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == FP16:
        return b.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown 16-bit dtype {dtype}")


def unpack_codes(words: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """Codes of one packed matrix [rows, words] -> int64 [rows, cols].

    Each row is an LSB-first bitstream: element i holds stream bits
    [bits*i, bits*i + bits) and stream bit t is bit (t mod 32) of word t//32.
    """
    w = np.ascontiguousarray(words, dtype="<u4")
    rows = w.shape[0]
    stream = np.unpackbits(w.view(np.uint8).reshape(rows, -1), axis=1,
                           bitorder="little")
    stream = stream[:, : cols * bits].reshape(rows, cols, bits)
    return np.packbits(stream, axis=2, bitorder="little")[:, :, 0].astype(np.int64)


def e2m1_to_f64(code) -> np.ndarray:
    """FP4 E2M1 elements (OCP MX v1.0) -> float64.

    Bit 3 is the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa:
    exponent 0 is subnormal (0 or 0.5), otherwise 2^(E-1) * (1 + m/2). The
    eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    ex, m = (c >> 1) & 3, (c & 1).astype(np.float64)
    mag = np.where(ex == 0, 0.5 * m, np.exp2(ex - 1.0) * (1.0 + 0.5 * m))
    return sign * mag


def e8m0_to_f64(e) -> np.ndarray:
    """E8M0 scale bytes (OCP MX v1.0) -> float64: 2^(e - 127), 0xFF is NaN."""
    v = np.asarray(e, dtype=np.int64)
    return np.where(v == 255, np.nan, np.exp2(v - 127.0))


def dequant(fmt, codes, scales, biases, cols: int) -> np.ndarray:
    """Dense float64 matrix [rows, cols] of one quantised matrix."""
    if fmt.mode == DENSE:
        return half_bits_to_f64(codes, fmt.scale_dtype).reshape(-1, cols)
    if fmt.mode == MXFP4:
        if fmt.bits != 4 or fmt.group != 32 or fmt.scale_dtype != E8M0:
            raise ValueError("MXFP4 is 4-bit E2M1 in blocks of 32 with E8M0 scales")
        q = unpack_codes(codes, 4, cols)
        return e2m1_to_f64(q) * e8m0_to_f64(scales)[:, np.arange(cols) // 32]
    q = unpack_codes(codes, fmt.bits, cols).astype(np.float64)
    gidx = np.arange(cols) // fmt.group
    s = half_bits_to_f64(scales, fmt.scale_dtype)[:, gidx]
    if fmt.mode == AFFINE:
        b = half_bits_to_f64(biases, fmt.scale_dtype)[:, gidx]
        return s * q + b
    if fmt.mode == SYMMETRIC:
        return s * (q - 8.0)
    raise ValueError(f"unknown mode {fmt.mode}")


def dequant_qtensor(t, index: Optional[int] = None) -> np.ndarray:
    """Dequantise a synth.QTensor (one matrix of a stacked tensor if index is given)."""
    if index is None:
        return dequant(t.fmt, t.codes, t.scales, t.biases, t.cols)
    return dequant(t.fmt, t.codes[index],
                   None if t.scales is None else t.scales[index],
                   None if t.biases is None else t.biases[index], t.cols)


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


# ------------------------------------------------------------------ routing
def topk_ids(logits32: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert ids per row: NaN first, then larger value, then lower id.

    logits32 [R, E] are float32 values; -0.0 and +0.0 compare equal.
    """
    R, E = logits32.shape
    nan = np.isnan(logits32)
    val = np.where(nan, 0.0, logits32.astype(np.float64))
    val = val + 0.0                    # -0.0 -> +0.0, so signed zeros tie
    ids = np.broadcast_to(np.arange(E), (R, E))
    order = np.lexsort((ids, -val, ~nan), axis=1)
    return order[:, :k].astype(np.int32)


def softmax_over_picks(l_sel: np.ndarray) -> np.ndarray:
    """exp(l - l_top) over the k picks, divided by their sum (rows of l_sel)."""
    with np.errstate(invalid="ignore"):
        m = np.max(l_sel, axis=1, keepdims=True)
        e = np.exp(l_sel - m)
        return e / e.sum(axis=1, keepdims=True)


@dataclass
class Routing:
    ids: np.ndarray          # int32 [R, k]
    p: np.ndarray            # float64 [R, k]
    sigma: np.ndarray        # float64 [R]
    logits: np.ndarray       # float64 [R, E] (bias included)
    gate_logit: np.ndarray   # float64 [R]
    gap: np.ndarray          # float64 [R]: k-th minus (k+1)-th sorted logit


def route(x: np.ndarray, Wr: np.ndarray, wg: np.ndarray, k: int,
          logit_bias: Optional[np.ndarray] = None,
          ids: Optional[np.ndarray] = None) -> Routing:
    """Router of the layer: logits, picks, renormalised weights, shared gate.

    x [R, H] float64; Wr [E, H]; wg [H]. With `ids` given, the picks are taken
    as input (used where the GPU's picks differ on a near-tie).
    """
    with np.errstate(invalid="ignore"):
        logits = x @ Wr.T
        if logit_bias is not None:
            logits = logits + np.asarray(logit_bias, np.float32).astype(np.float64)
        c = x @ wg
    if ids is None:
        ids = topk_ids(logits.astype(np.float32), k)
    ids = np.asarray(ids, dtype=np.int32)
    l_sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    p = softmax_over_picks(l_sel)
    E = logits.shape[1]
    if k < E:
        srt = -np.sort(-np.where(np.isnan(logits), np.inf, logits), axis=1)
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(logits.shape[0], np.inf)
    return Routing(ids, p, sigmoid(c), logits, c, gap)


# ------------------------------------------------------------------ experts
def swiglu_expert(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray):
    """One expert MLP on rows x [n, H]: g, u, h = silu(g)*u, e = Wd h."""
    with np.errstate(invalid="ignore"):
        g = x @ Wg.T
        u = x @ Wu.T
        h = silu(g) * u
        e = h @ Wd.T
    return g, u, h, e


class DenseExperts:
    """Dequantised (float64) router and experts of one synth.Layer, cached per expert."""

    def __init__(self, layer, provider: Optional[Callable] = None, cache: bool = True):
        self.layer = layer
        self.spec = layer.spec
        self._provider = provider
        self._cache: Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
        self._use_cache = cache
        self._router = None

    def router(self):
        if self._router is None:
            L = self.layer
            self._router = (dequant_qtensor(L.router), dequant_qtensor(L.gate_row)[0])
        return self._router

    def expert(self, e: int):
        if e in self._cache:
            return self._cache[e]
        E = self.spec.n_experts
        if self._provider is not None:
            g, u, d = self._provider(e)
            mats = (dequant_qtensor(g), dequant_qtensor(u), dequant_qtensor(d))
        elif e == E:
            L = self.layer
            mats = (dequant_qtensor(L.sh_gate), dequant_qtensor(L.sh_up),
                    dequant_qtensor(L.sh_down))
        else:
            L = self.layer
            mats = (dequant_qtensor(L.gate, e), dequant_qtensor(L.up, e),
                    dequant_qtensor(L.down, e))
        if self._use_cache:
            self._cache[e] = mats
        return mats


@dataclass
class LayerOut:
    y: np.ndarray            # [R, H]
    routing: Routing
    g: np.ndarray            # [R, k+1, I] (slot k: shared expert)
    u: np.ndarray
    h: np.ndarray
    e: np.ndarray            # [R, k+1, H] unweighted slot outputs


def act_to_f64(x_bits: np.ndarray, act_dtype: int) -> np.ndarray:
    return half_bits_to_f64(x_bits, act_dtype)


def _combine(p: np.ndarray, sigma: np.ndarray, e: np.ndarray) -> np.ndarray:
    """y = sum_j p_j e_j + sigma * shared, slots in pick order, shared last."""
    k = p.shape[1]
    y = np.zeros((e.shape[0], e.shape[2]))
    with np.errstate(invalid="ignore"):
        for j in range(k):
            y = y + p[:, j:j + 1] * e[:, j, :]
        y = y + sigma[:, None] * e[:, k, :]
    return y


def moe_forward(layer, x_bits: np.ndarray, dense: Optional[DenseExperts] = None,
                ids: Optional[np.ndarray] = None, form: str = "per_row") -> LayerOut:
    """The MoE FFN of one layer on rows x_bits [R, H] (activation bit patterns).

    form="per_row": each row runs its k experts and the shared expert alone.
    form="expert_major": each expert runs once on all rows that picked it.
    Both evaluate the same definition; they differ only in float64 rounding.
    """
    spec = layer.spec
    dense = dense or DenseExperts(layer)
    x = act_to_f64(x_bits, spec.act)
    R, H = x.shape
    k, E = spec.top_k, spec.n_experts
    Wr, wg = dense.router()
    rt = route(x, Wr, wg, k, layer.logit_bias, ids)
    I = spec.inter
    Is = spec.shared_inter
    Imax = max(I, Is)
    g = np.zeros((R, k + 1, Imax))
    u = np.zeros_like(g)
    h = np.zeros_like(g)
    e = np.zeros((R, k + 1, H))
    if form == "per_row":
        for r in range(R):
            for j in range(k + 1):
                eid = E if j == k else int(rt.ids[r, j])
                Wg, Wu, Wd = dense.expert(eid)
                gg, uu, hh, ee = swiglu_expert(x[r:r + 1], Wg, Wu, Wd)
                n = gg.shape[1]
                g[r, j, :n], u[r, j, :n], h[r, j, :n], e[r, j] = gg[0], uu[0], hh[0], ee[0]
    elif form == "expert_major":
        slots = {}
        for r in range(R):
            for j in range(k):
                slots.setdefault(int(rt.ids[r, j]), []).append((r, j))
        slots[E] = [(r, k) for r in range(R)]
        for eid in sorted(slots):
            rows = np.array([rj[0] for rj in slots[eid]])
            cols = np.array([rj[1] for rj in slots[eid]])
            Wg, Wu, Wd = dense.expert(eid)
            gg, uu, hh, ee = swiglu_expert(x[rows], Wg, Wu, Wd)
            n = gg.shape[1]
            g[rows, cols, :n], u[rows, cols, :n], h[rows, cols, :n] = gg, uu, hh
            e[rows, cols] = ee
    else:
        raise ValueError(form)
    y = _combine(rt.p, rt.sigma, e)
    return LayerOut(y, rt, g, u, h, e)


def row_error(y: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per-row max|y - y_ref| / max|y_ref| (the pass criterion is <= 2e-3)."""
    d = np.max(np.abs(y.astype(np.float64) - y_ref), axis=-1)
    m = np.max(np.abs(y_ref), axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(m > 0, d / np.where(m > 0, m, 1.0), d)


def class_errors(a: np.ndarray, ref: np.ndarray) -> dict:
    """Worst-column and aggregate error of one projection class.

    worst_col: max over columns of max|a - ref| / max|ref| within that column;
    aggregate: ||a - ref||_F / ||ref||_F.
    """
    a = np.asarray(a, np.float64).reshape(-1, ref.shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    ok = np.isfinite(r).all(axis=1)
    a, r = a[ok], r[ok]
    if r.size == 0:
        return dict(worst_col=0.0, aggregate=0.0, max_abs=0.0)
    d = np.abs(a - r)
    cm = np.max(np.abs(r), axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        wc = np.max(np.where(cm > 0, np.max(d, axis=0) / np.where(cm > 0, cm, 1), 0))
        agg = np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-300)
    return dict(worst_col=float(wc), aggregate=float(agg), max_abs=float(d.max()))

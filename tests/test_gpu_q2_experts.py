"""GPU parity of 2-bit affine experts (g64, bf16 scale and bias) on the
decode path, against the FP64 oracle.

2-bit codes are the narrowest of the MLX affine widths (2 to 8 bits) the
pages' loader reads, and the proposal there adds affine experts at widths
other than 4 beside the 4-bit form ("qwen3_5_moe on native CUDA with 3-bit
routed experts #803", What exists on native; Proposal and questions). The
decode kernels read them as pairs 1 + q/16, the 4-bit pair value, so the
control is the pages' own kind: the same codes widened to 4-bit words give
the same bytes. moe_forward_windows serves prompt rows exactly (the grouped
GEMMs' parity at this width is in test_gpu_grouped_widths.py). Layers: the full-size decode layer with 2-bit
routed and shared experts (bf16 and fp16 activations), a mixed one (2-bit
routed, 4-bit shared) and a small one (H=512, E=64, k=4).
"""
import copy
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth import to_abi
from synth.gen import FP16, Q2G64, Q4G64, QTensor

from gpu_common import binding, build_layer, check_parity, log, run_gpu, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu

FULL_Q2 = replace(synth.CONFIGS[1], cfg_id=307, name="decode-8rows-q2g64-experts", routed=Q2G64, shared=Q2G64)
FULL_Q2_FP16 = replace(FULL_Q2, cfg_id=308, name="decode-8rows-q2g64-experts-fp16", act=FP16)
MIXED_Q2 = replace(FULL_Q2, cfg_id=309, name="decode-8rows-q2-routed-q4-shared", shared=Q4G64)
SMALL_Q2 = synth.make_tiny_config(FULL_Q2, cfg_id=310, hidden=512, n_experts=64, top_k=4, inter=256,
                                  shared_inter=256)

_cache = {}


def layer_of(spec):
    if spec.cfg_id not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        Lh, dev = build_layer(spec, 0)
        _cache[spec.cfg_id] = (Lh, dev, O.DenseExperts(Lh))
    return _cache[spec.cfg_id]


@pytest.mark.parametrize("spec,rows", [(FULL_Q2, 8), (FULL_Q2_FP16, 8), (MIXED_Q2, 8), (SMALL_Q2, 1),
                                       (SMALL_Q2, 16)],
                         ids=["full-bf16", "full-fp16", "mixed", "small-r1", "small-r16"])
def test_q2_experts_decode_parity(spec, rows):
    log(f"case q2 decode {spec.name} rows={rows}")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=7)
    check_parity(Lh, xb, run_gpu(dev, Lh, xb), dense, name=f"q2-{spec.cfg_id}-r{rows}", strict_y=1e-4)


@pytest.mark.parametrize("spec", [FULL_Q2, SMALL_Q2], ids=["full", "small"])
def test_q2_experts_batch_equals_solo_bit_for_bit(spec):
    rows = 8 if spec.hidden == 2048 else 16
    log(f"case q2 batch invariance {spec.name} rows={rows}")
    Lh, dev, _ = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=9)
    batch = run_gpu(dev, Lh, xb, taps=False)
    for r in (0, rows // 2, rows - 1):
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        for key in ("ids", "p", "sg", "y"):
            u, v = solo[key][0], batch[key][r]
            if u.dtype == np.float32:
                u, v = u.view(np.uint32), v.view(np.uint32)
            assert np.array_equal(u, v), f"row {r} {key} differs"


def _widen_q2_to_q4(t):
    """The same codes as 4-bit words (8 codes per word), scales and biases kept."""
    E = t.codes.shape[0]
    out = np.empty((E, t.rows, t.cols // 8), np.uint32)
    for e in range(E):
        q = O.unpack_codes(t.codes[e], 2, t.cols).astype(np.uint32).reshape(t.rows, -1, 8)
        w = np.zeros(q.shape[:2], np.uint32)
        for i in range(8):
            w |= q[:, :, i] << np.uint32(4 * i)
        out[e] = w
    return QTensor(Q4G64, t.rows, t.cols, out, t.scales, t.biases)


@pytest.mark.parametrize("act16", [0, 1], ids=["bf16", "fp16"])
def test_q2_equals_widened_4bit_bit_for_bit(act16):
    """2-bit codes rewritten as 4-bit words (routed and shared) give the same
    picks, h, per-slot outputs and y, bit for bit."""
    B = binding()
    spec2 = replace(SMALL_Q2, cfg_id=311 + act16, act=FP16 if act16 else SMALL_Q2.act)
    Lh2, dev2 = build_layer(spec2, 0)
    spec4 = replace(spec2, routed=Q4G64, shared=Q4G64)
    Lh4 = copy.copy(Lh2)
    Lh4.spec = spec4
    for name in ("gate", "up", "down"):
        setattr(Lh4, name, _widen_q2_to_q4(getattr(Lh2, name)))
    for name in ("sh_gate", "sh_up", "sh_down"):
        t = getattr(Lh2, name)
        w = _widen_q2_to_q4(QTensor(t.fmt, t.rows, t.cols, t.codes[None], t.scales[None],
                                    t.biases[None]))
        setattr(Lh4, name, QTensor(Q4G64, t.rows, t.cols, w.codes[0], t.scales, t.biases))
    dev4 = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec4)), to_abi.tensors(Lh4))
    xb = synth.make_x(spec2, 0, 8, rep=2)
    a = run_gpu(dev2, Lh2, xb)
    b = run_gpu(dev4, Lh4, xb)
    assert np.array_equal(a["ids"], b["ids"])
    for key in ("y", "h", "e"):
        assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), key
    check_parity(Lh2, xb, a, name=f"q2-widened-{act16}", strict_y=1e-4)


def test_q2_experts_windows_served():
    B = binding()
    torch = torch_mod()
    Lh, dev, dense = layer_of(FULL_Q2)
    xb = synth.make_x(FULL_Q2, 0, 20, rep=3)
    x = to_dev_x(xb)
    ids, p, sg, y = B.forward_windows(dev, x)
    torch.cuda.synchronize()
    g = dict(ids=ids.cpu().numpy(), p=p.cpu().numpy(), sg=sg.cpu().numpy(), y=y.cpu().numpy())
    check_parity(Lh, xb, g, dense, name="q2-windows-r20", strict_y=1e-4)
    solo = run_gpu(dev, Lh, xb[17:18], taps=False)
    assert np.array_equal(solo["y"][0].view(np.uint32), g["y"][17].view(np.uint32))

"""GPU parity of 8-bit affine experts (g64, bf16 scale and bias) on the
decode path, against the FP64 oracle.

8-bit codes are among the MLX affine widths (2 to 8 bits) the pages' loader
reads, and the proposal there adds affine experts at widths other than 4
beside the 4-bit form ("qwen3_5_moe on native CUDA with 3-bit routed experts
#803", the issue's "Affine experts at other widths" proposal). The decode kernels
read them (with bf16 activations as low and high nibble pairs, with fp16
ones as one pair set), and moe_forward_windows serves prompt rows exactly
(the grouped GEMMs' parity at this width is in test_gpu_grouped_widths.py).
Layers: the full-size decode
layer with 8-bit routed and shared experts (bf16 and fp16 activations), a
mixed one (8-bit routed, 4-bit shared) and a small one (H=512, E=64, k=4).
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth.gen import FP16, Q4G64, Q8G64

from gpu_common import binding, build_layer, check_parity, log, run_gpu, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu

FULL_Q8 = replace(synth.CONFIGS[1], cfg_id=303, name="decode-8rows-q8g64-experts", routed=Q8G64, shared=Q8G64)
FULL_Q8_FP16 = replace(FULL_Q8, cfg_id=304, name="decode-8rows-q8g64-experts-fp16", act=FP16)
MIXED_Q8 = replace(FULL_Q8, cfg_id=305, name="decode-8rows-q8-routed-q4-shared", shared=Q4G64)
SMALL_Q8 = synth.make_tiny_config(FULL_Q8, cfg_id=306, hidden=512, n_experts=64, top_k=4, inter=256,
                                  shared_inter=256)

_cache = {}


def layer_of(spec):
    if spec.cfg_id not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        Lh, dev = build_layer(spec, 0)
        _cache[spec.cfg_id] = (Lh, dev, O.DenseExperts(Lh))
    return _cache[spec.cfg_id]


@pytest.mark.parametrize("spec,rows", [(FULL_Q8, 8), (FULL_Q8_FP16, 8), (MIXED_Q8, 8), (SMALL_Q8, 1),
                                       (SMALL_Q8, 5), (SMALL_Q8, 16)],
                         ids=["full-bf16", "full-fp16", "mixed", "small-r1", "small-r5", "small-r16"])
def test_q8_experts_decode_parity(spec, rows):
    log(f"case q8 decode {spec.name} rows={rows}")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=7)
    check_parity(Lh, xb, run_gpu(dev, Lh, xb), dense, name=f"q8-{spec.cfg_id}-r{rows}", strict_y=1e-4)


@pytest.mark.parametrize("spec", [FULL_Q8, FULL_Q8_FP16, SMALL_Q8], ids=["full-bf16", "full-fp16", "small"])
def test_q8_experts_batch_equals_solo_bit_for_bit(spec):
    rows = 8 if spec.hidden == 2048 else 16
    log(f"case q8 batch invariance {spec.name} rows={rows}")
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


def test_q8_experts_windows_served():
    B = binding()
    torch = torch_mod()
    Lh, dev, dense = layer_of(FULL_Q8)
    xb = synth.make_x(FULL_Q8, 0, 20, rep=3)
    x = to_dev_x(xb)
    ids, p, sg, y = B.forward_windows(dev, x)
    torch.cuda.synchronize()
    g = dict(ids=ids.cpu().numpy(), p=p.cpu().numpy(), sg=sg.cpu().numpy(), y=y.cpu().numpy())
    check_parity(Lh, xb, g, dense, name="q8-windows-r20", strict_y=1e-4)
    solo = run_gpu(dev, Lh, xb[17:18], taps=False)
    assert np.array_equal(solo["y"][0].view(np.uint32), g["y"][17].view(np.uint32))

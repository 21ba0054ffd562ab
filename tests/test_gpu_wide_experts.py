"""GPU parity of 5- and 6-bit affine experts (g64, bf16 scale and bias) on
the decode path, against the FP64 oracle.

5 and 6 bits are among the MLX affine widths (2 to 8 bits) the pages' loader
reads, and the proposal there adds affine experts at widths other than 4
("qwen3_5_moe on native CUDA with 3-bit routed experts #803", What exists on
native; Proposal and questions). The decode kernels read them as pairs
1 + q/32 and 1 + q/64 (exact in fp16 and in bf16); a lane's 16-bit pair
halves hold whole fields for most pairs and the rest in the spare bits (see
the kernel layout notes). Layers: full-size decode layers with 5-bit and
6-bit routed and shared experts (bf16 and fp16 activations), 6-bit routed
beside a 4-bit shared expert, and small ones (H=512, E=64, k=4). Prompt rows
through moe_forward_windows here; the grouped GEMMs' parity at these widths is
in test_gpu_grouped_widths.py.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth.gen import FP16, Q4G64, Q5G64, Q6G64

from gpu_common import binding, build_layer, check_parity, log, run_gpu, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu

FULL_Q5 = replace(synth.CONFIGS[1], cfg_id=320, name="decode-8rows-q5g64-experts", routed=Q5G64, shared=Q5G64)
FULL_Q6 = replace(synth.CONFIGS[1], cfg_id=321, name="decode-8rows-q6g64-experts", routed=Q6G64, shared=Q6G64)
FULL_Q5_FP16 = replace(FULL_Q5, cfg_id=322, name="decode-8rows-q5g64-experts-fp16", act=FP16)
FULL_Q6_FP16 = replace(FULL_Q6, cfg_id=323, name="decode-8rows-q6g64-experts-fp16", act=FP16)
MIXED_Q6 = replace(FULL_Q6, cfg_id=324, name="decode-8rows-q6-routed-q4-shared", shared=Q4G64)
SMALL_Q5 = synth.make_tiny_config(FULL_Q5, cfg_id=325, hidden=512, n_experts=64, top_k=4, inter=256,
                                  shared_inter=256)
SMALL_Q6 = synth.make_tiny_config(FULL_Q6, cfg_id=326, hidden=512, n_experts=64, top_k=4, inter=256,
                                  shared_inter=256)

_cache = {}


def layer_of(spec):
    if spec.cfg_id not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        Lh, dev = build_layer(spec, 0)
        _cache[spec.cfg_id] = (Lh, dev, O.DenseExperts(Lh))
    return _cache[spec.cfg_id]


CASES = [(FULL_Q5, 8), (FULL_Q5_FP16, 8), (FULL_Q6, 8), (FULL_Q6_FP16, 8), (MIXED_Q6, 8),
         (SMALL_Q5, 1), (SMALL_Q5, 16), (SMALL_Q6, 1), (SMALL_Q6, 16)]


@pytest.mark.parametrize("spec,rows", CASES, ids=[f"{s.cfg_id}-r{r}" for s, r in CASES])
def test_wide_experts_decode_parity(spec, rows):
    log(f"case wide decode {spec.name} rows={rows}")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=7)
    check_parity(Lh, xb, run_gpu(dev, Lh, xb), dense, name=f"wide-{spec.cfg_id}-r{rows}", strict_y=1e-4)


@pytest.mark.parametrize("spec", [FULL_Q5, FULL_Q6_FP16, SMALL_Q6], ids=["q5", "q6-fp16", "q6-small"])
def test_wide_experts_batch_equals_solo_bit_for_bit(spec):
    rows = 8 if spec.hidden == 2048 else 16
    log(f"case wide batch invariance {spec.name} rows={rows}")
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


@pytest.mark.parametrize("spec", [FULL_Q5, MIXED_Q6], ids=["q5", "q6-mixed"])
def test_wide_experts_windows_served(spec):
    B = binding()
    torch = torch_mod()
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, 20, rep=3)
    x = to_dev_x(xb)
    ids, p, sg, y = B.forward_windows(dev, x)
    torch.cuda.synchronize()
    g = dict(ids=ids.cpu().numpy(), p=p.cpu().numpy(), sg=sg.cpu().numpy(), y=y.cpu().numpy())
    check_parity(Lh, xb, g, dense, name=f"wide-windows-{spec.cfg_id}", strict_y=1e-4)
    solo = run_gpu(dev, Lh, xb[17:18], taps=False)
    assert np.array_equal(solo["y"][0].view(np.uint32), g["y"][17].view(np.uint32))

"""GPU parity of prompt chunks with 2-, 5-, 6- and 8-bit affine experts
(g64, bf16 scale and bias) through the grouped GEMMs, at the 512-row chunk
shape (hidden 2048, 256 experts, top-8, intermediate 512).

The pages' loader reads MLX affine experts at 2 to 8 bits, and each width is
to be checked on decode and on prompt rows separately ("qwen3_5_moe on native
CUDA with 3-bit routed experts #803", What exists on native; Proposal and
questions, 2). The grouped GEMMs read these widths through their generic B
layout (the chunk block copied to LDS as packed, each lane unpacking its
row's whole chunk into pairs 1 + q/M). Per case:
  * prompt rows: the chunk through the grouped path; decode rows: the same
    chunk through moe_forward_windows (the decode kernels, 16-row windows);
  * ids identical between the two (weights within fp32 rounding: the two
    routers add the logits in other orders), every row's y within the 2e-3
    row error of the other form;
  * 24 rows sampled across the chunk, of each form, against the fp64
    oracle (per-row form), with per-class errors for the grouped form
    (taps) reported, prompt and decode rows under their own names.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth.gen import Q2G64, Q4G64, Q5G64, Q6G64, Q8G64

from gpu_common import binding, build_layer, check_parity, log, run_gpu, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu

C3 = synth.CONFIGS[3]
CASES = [
    replace(C3, cfg_id=330, name="prefill-512rows-q2g64-experts", routed=Q2G64, shared=Q2G64),
    replace(C3, cfg_id=331, name="prefill-512rows-q5g64-experts", routed=Q5G64, shared=Q5G64),
    replace(C3, cfg_id=332, name="prefill-512rows-q6g64-experts", routed=Q6G64, shared=Q6G64),
    replace(C3, cfg_id=333, name="prefill-512rows-q8g64-experts", routed=Q8G64, shared=Q8G64),
    replace(C3, cfg_id=334, name="prefill-512rows-q6-routed-q4-shared", routed=Q6G64, shared=Q4G64),
]
SAMPLE = np.unique(np.linspace(0, 511, 24).astype(int))


@pytest.mark.parametrize("spec", CASES, ids=[s.name for s in CASES])
def test_grouped_width_parity_prompt_and_decode(spec):
    log(f"case grouped width {spec.name}")
    B = binding()
    torch = torch_mod()
    Lh, dev = build_layer(spec, 0)
    xb = synth.make_x(spec, 0, spec.rows[0], rep=11)
    g = run_gpu(dev, Lh, xb, grouped=True)
    ids, p, sg, y = B.forward_windows(dev, to_dev_x(xb))
    torch.cuda.synchronize()
    d = dict(ids=ids.cpu().numpy(), p=p.cpu().numpy(), sg=sg.cpu().numpy(), y=y.cpu().numpy())
    # the chunk router (MFMA logits over 32-row blocks) and the decode router
    # add the logits in other orders: same picks here, weights within fp32
    # rounding of each other
    assert np.array_equal(g["ids"], d["ids"])
    assert np.allclose(g["p"], d["p"], rtol=1e-5, atol=1e-7)
    assert np.allclose(g["sg"], d["sg"], rtol=1e-5, atol=1e-7)
    err = O.row_error(g["y"], d["y"].astype(np.float64))
    log(f"{spec.name}: prompt vs decode rows, worst row error {err.max():.3e}")
    assert err.max() <= 2e-3
    dense = O.DenseExperts(Lh, cache=True)
    sub = lambda src: {k_: v[SAMPLE] for k_, v in src.items()}
    check_parity(Lh, xb[SAMPLE], sub(g), dense, name=f"grouped-{spec.cfg_id}-prompt-rows")
    check_parity(Lh, xb[SAMPLE], sub(d), dense, name=f"grouped-{spec.cfg_id}-decode-rows", strict_y=1e-4)


def test_grouped_refuses_unread_pairs():
    """An 8-bit routed format with a 2-bit shared expert is read by the
    decode kernels but not by the grouped GEMMs: refused by name."""
    B = binding()
    spec = synth.make_tiny_config(replace(C3, routed=Q8G64, shared=Q2G64), cfg_id=335, hidden=512,
                                  n_experts=64, top_k=4, inter=256, shared_inter=256)
    Lh, dev = build_layer(spec, 0)
    x = to_dev_x(synth.make_x(spec, 0, 8, rep=1))
    ids, p, sg = B.route(dev, x)
    with pytest.raises(B.MoeError, match="not read by the grouped GEMMs"):
        B.experts(dev, x, ids, p, sg, True)

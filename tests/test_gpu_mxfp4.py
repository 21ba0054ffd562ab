"""GPU parity of MXFP4 experts on the decode path, the 16-row windows and the
exact chunk form, against the FP64 oracle.

The pages name an MXFP4-expert checkpoint as the reference beside the W4A16
export ("Sage-1.5-W4A16" model card, Performance, decode speed table) and do
not define the format; the oracle and the kernels take the public OCP
Microscaling v1.0 definition (FP4 E2M1 elements, one E8M0 exponent byte per
32). The decode kernels turn each byte of codes into an exact fp16 / bf16
pair with gfx950's FP4 conversion and multiply each group's dot by
2^(e - 127) in fp32. Layers: full-size decode layers with MXFP4 routed and
shared experts (bf16 and fp16 activations), MXFP4 routed beside a 4-bit
affine shared expert, small layers (H=512, E=64, k=4), a shared expert of
2048 (64 groups per row), and a layer with NaN (e = 255) and 2^-127 (e = 0)
block scales. The grouped GEMMs refuse MXFP4 by name.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth import to_abi
from synth.gen import FP16, MX4G32, Q4G64

from gpu_common import binding, build_layer, check_parity, log, run_gpu, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu

FULL_MX = replace(synth.CONFIGS[1], cfg_id=330, name="decode-8rows-mxfp4-experts", routed=MX4G32,
                  shared=MX4G32)
FULL_MX_FP16 = replace(FULL_MX, cfg_id=331, name="decode-8rows-mxfp4-experts-fp16", act=FP16)
MIXED_MX = replace(FULL_MX, cfg_id=332, name="decode-8rows-mxfp4-routed-q4-shared", shared=Q4G64)
SMALL_MX = synth.make_tiny_config(FULL_MX, cfg_id=333, hidden=512, n_experts=64, top_k=4, inter=256,
                                  shared_inter=256)
WIDE_SHARED_MX = replace(SMALL_MX, cfg_id=334, name="small-mxfp4-shared-2048", shared_inter=2048)

_cache = {}


def layer_of(spec):
    if spec.cfg_id not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        Lh, dev = build_layer(spec, 0)
        _cache[spec.cfg_id] = (Lh, dev, O.DenseExperts(Lh))
    return _cache[spec.cfg_id]


def _np(t):
    return t.cpu().numpy()


def _windows(dev, xb):
    B = binding()
    ids, p, sg, y = B.forward_windows(dev, to_dev_x(xb))
    torch_mod().cuda.synchronize()
    return dict(ids=_np(ids), p=_np(p), sg=_np(sg), y=_np(y))


def _exact(dev, xb):
    B = binding()
    ids, p, sg, y = B.forward_exact(dev, to_dev_x(xb))
    torch_mod().cuda.synchronize()
    return dict(ids=_np(ids), p=_np(p), sg=_np(sg), y=_np(y))


def _bits_equal(a, b, what):
    for key in ("ids", "p", "sg", "y"):
        u, v = a[key], b[key]
        if u.dtype == np.float32:
            u, v = u.view(np.uint32), v.view(np.uint32)
        assert np.array_equal(u, v), f"{what}: {key} differs"


CASES = [(FULL_MX, 8), (FULL_MX_FP16, 8), (MIXED_MX, 8), (SMALL_MX, 1), (SMALL_MX, 16),
         (WIDE_SHARED_MX, 4)]


@pytest.mark.parametrize("spec,rows", CASES, ids=[f"{s.cfg_id}-r{r}" for s, r in CASES])
def test_mxfp4_decode_parity(spec, rows):
    log(f"case mxfp4 decode {spec.name} rows={rows}")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=7)
    check_parity(Lh, xb, run_gpu(dev, Lh, xb), dense, name=f"mxfp4-{spec.cfg_id}-r{rows}", strict_y=1e-4)


def test_mxfp4_batch_equals_solo_bit_for_bit():
    log("case mxfp4 batch invariance")
    Lh, dev, _ = layer_of(FULL_MX)
    xb = synth.make_x(FULL_MX, 0, 8, rep=9)
    batch = run_gpu(dev, Lh, xb, taps=False)
    for r in (0, 4, 7):
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        _bits_equal({k: v[0:1] for k, v in solo.items()}, {k: v[r:r + 1] for k, v in batch.items()},
                    f"row {r}")


@pytest.mark.parametrize("spec,rows", [(SMALL_MX, 40), (FULL_MX, 64), (MIXED_MX, 24)],
                         ids=["small-40", "full-64", "mixed-24"])
def test_mxfp4_exact_equals_windows_and_oracle(spec, rows):
    """The exact chunk form equals the 16-row windows bit for bit, and both
    match the oracle."""
    log(f"case mxfp4 exact/windows {spec.name} rows={rows}")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=5)
    w = _windows(dev, xb)
    ex = _exact(dev, xb)
    _bits_equal(ex, w, f"{spec.name} exact vs windows")
    sample = np.unique([0, 1, rows // 3, rows // 2, rows - 2, rows - 1])
    check_parity(Lh, xb[sample], {k: v[sample] for k, v in ex.items()}, dense,
                 name=f"mxfp4-exact-{spec.cfg_id}-r{rows}", strict_y=1e-4)
    solo = run_gpu(dev, Lh, xb[rows - 1:rows], taps=False)
    assert np.array_equal(solo["y"][0].view(np.uint32), ex["y"][rows - 1].view(np.uint32))


def test_mxfp4_exact_refuses_more_than_32_shared_groups():
    B = binding()
    Lh, dev, _ = layer_of(WIDE_SHARED_MX)
    with pytest.raises(B.MoeError, match="MOE_EUNSUPPORTED.*32 groups"):
        B.forward_exact(dev, to_dev_x(synth.make_x(WIDE_SHARED_MX, 0, 4)))


def test_mxfp4_grouped_refused_by_name():
    B = binding()
    torch = torch_mod()
    Lh, dev, _ = layer_of(SMALL_MX)
    x = to_dev_x(synth.make_x(SMALL_MX, 0, 32))
    ids, p, sg = B.route(dev, x)
    torch.cuda.synchronize()
    with pytest.raises(B.MoeError, match="MOE_EUNSUPPORTED.*mxfp4"):
        B.experts(dev, x, ids, p, sg, True)


def test_mxfp4_nan_and_subnormal_block_scales():
    """e = 255 in one gate block of an expert some rows pick makes exactly
    those rows NaN; e = 0 (2^-127) on a whole up projection of another
    expert leaves its rows finite and close to the oracle."""
    spec = replace(SMALL_MX, cfg_id=335, name="small-mxfp4-edge-scales")
    B = binding()
    Lh = synth.make_layer(spec, 0)
    rows = 16
    xb = synth.make_x(spec, 0, rows, rep=11)
    ids0 = O.moe_forward(Lh, xb).routing.ids
    e_nan = int(ids0[0, 0])
    e_tiny = next(int(e) for e in ids0[1:].ravel() if int(e) != e_nan and not np.any(ids0[0] == e))
    Lh.gate.scales[e_nan, 5, 2] = 255
    Lh.up.scales[e_tiny] = 0
    dev = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec)), to_abi.tensors(Lh))
    log(f"case mxfp4 edge scales nan={e_nan} tiny={e_tiny}")
    dense = O.DenseExperts(Lh)
    g = run_gpu(dev, Lh, xb)
    nan_rows = np.any(g["ids"] == e_nan, axis=1)
    assert nan_rows[0] and not nan_rows.all()
    assert np.array_equal(np.isnan(g["y"]).all(axis=1), nan_rows)
    assert not np.isnan(g["y"][~nan_rows]).any()
    check_parity(Lh, xb, g, dense, name="mxfp4-edge-scales", strict_y=1e-4)
    ex = _exact(dev, xb)
    _bits_equal(ex, _windows(dev, xb), "edge scales exact vs windows")

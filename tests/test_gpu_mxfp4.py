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
block scales. Prompt chunks through the grouped GEMMs (512-row chunk shape,
and a small Zipf layer with fp16 activations beside a 4-bit shared expert):
the FP4 converter scales each byte by its block scale into an fp16 operand,
exact for block exponents 104..140 and 255; a layer with any other exponent
is refused by name (the packer's MOE_LAYER_MX_FP16 flag).
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

FULL_MX = replace(synth.CONFIGS[1], cfg_id=360, name="decode-8rows-mxfp4-experts", routed=MX4G32,
                  shared=MX4G32)
FULL_MX_FP16 = replace(FULL_MX, cfg_id=361, name="decode-8rows-mxfp4-experts-fp16", act=FP16)
MIXED_MX = replace(FULL_MX, cfg_id=362, name="decode-8rows-mxfp4-routed-q4-shared", shared=Q4G64)
SMALL_MX = synth.make_tiny_config(FULL_MX, cfg_id=363, hidden=512, n_experts=64, top_k=4, inter=256,
                                  shared_inter=256)
WIDE_SHARED_MX = replace(SMALL_MX, cfg_id=364, name="small-mxfp4-shared-2048", shared_inter=2048)

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


PROMPT_MX = replace(synth.CONFIGS[3], cfg_id=366, name="prefill-512rows-mxfp4-experts", routed=MX4G32,
                    shared=MX4G32)
SMALL_ZIPF_MX = replace(synth.make_tiny_config(synth.CONFIGS[4], cfg_id=367, hidden=512, n_experts=64, top_k=8,
                                               inter=256, shared_inter=256),
                        name="small-zipf-fp16-mxfp4-routed-q4-shared", routed=MX4G32, shared=Q4G64)
SAMPLE = np.unique(np.linspace(0, 511, 24).astype(int))


@pytest.mark.parametrize("spec", [PROMPT_MX, SMALL_ZIPF_MX], ids=["512rows", "small-zipf-fp16"])
def test_mxfp4_grouped_prompt_and_decode(spec):
    """Prompt rows through the grouped GEMMs against the same rows through
    the decode kernels (16-row windows) and against the oracle."""
    log(f"case mxfp4 grouped {spec.name}")
    B = binding()
    torch = torch_mod()
    Lh, dev, dense = layer_of(spec)
    rows = spec.rows[0] if spec.hidden == 2048 else 200
    xb = synth.make_x(spec, 0, rows, rep=11)
    g = run_gpu(dev, Lh, xb, grouped=True)
    bias = torch.from_numpy(Lh.logit_bias).cuda() if Lh.logit_bias is not None else None
    ids, p, sg, y = B.forward_windows(dev, to_dev_x(xb), bias)
    torch.cuda.synchronize()
    d = dict(ids=ids.cpu().numpy(), p=p.cpu().numpy(), sg=sg.cpu().numpy(), y=y.cpu().numpy())
    # the chunk router and the decode router add the logits in other orders
    same = np.all(g["ids"] == d["ids"], axis=1)
    assert same.mean() > 0.97, f"{(~same).sum()} rows pick differently"
    err = O.row_error(g["y"][same], d["y"][same].astype(np.float64))
    log(f"{spec.name}: prompt vs decode rows, worst row error {err.max():.3e}")
    assert err.max() <= 2e-3
    sample = SAMPLE if rows == 512 else np.arange(rows)
    sub = lambda src: {k_: v[sample] for k_, v in src.items()}
    check_parity(Lh, xb[sample], sub(g), dense, name=f"mxfp4-grouped-{spec.cfg_id}-prompt-rows")
    check_parity(Lh, xb[sample], sub(d), dense, name=f"mxfp4-grouped-{spec.cfg_id}-decode-rows", strict_y=1e-4)


def test_mxfp4_grouped_nan_block_scale():
    """e = 255 (NaN) is within what the grouped GEMMs read: exactly the rows
    that pick the expert come out NaN, the rest match the oracle."""
    spec = replace(SMALL_MX, cfg_id=368, name="small-mxfp4-nan-scale")
    B = binding()
    Lh = synth.make_layer(spec, 0)
    rows = 48
    xb = synth.make_x(spec, 0, rows, rep=13)
    e_nan = int(O.moe_forward(Lh, xb).routing.ids[0, 1])
    Lh.down.scales[e_nan, 7, 3] = 255
    dev = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec)), to_abi.tensors(Lh))
    assert dev.c.flags & 1
    log(f"case mxfp4 grouped nan scale e={e_nan}")
    g = run_gpu(dev, Lh, xb, grouped=True)
    nan_rows = np.any(g["ids"] == e_nan, axis=1)
    assert nan_rows[0] and not nan_rows.all()
    assert np.array_equal(np.isnan(g["y"]).any(axis=1), nan_rows)
    check_parity(Lh, xb, g, O.DenseExperts(Lh), name="mxfp4-grouped-nan-scale")


@pytest.mark.parametrize("e_bad", [103, 141])
def test_mxfp4_grouped_refuses_exponents_outside_fp16(e_bad):
    """One block exponent outside 104..140 and the grouped call refuses the
    layer by name; the exact form reads it."""
    spec = replace(SMALL_MX, cfg_id=369, name="small-mxfp4-wide-exponent")
    B = binding()
    torch = torch_mod()
    Lh = synth.make_layer(spec, 0)
    # in the down projection: its outputs stay fp32 (h, carried in fp16 by
    # both forms, would overflow past 65504 with 2^14-scaled up weights)
    Lh.sh_down.scales[3, 5] = e_bad
    dev = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec)), to_abi.tensors(Lh))
    assert not dev.c.flags & 1
    xb = synth.make_x(spec, 0, 32)
    x = to_dev_x(xb)
    ids, p, sg = B.route(dev, x)
    torch.cuda.synchronize()
    with pytest.raises(B.MoeError, match="MOE_EUNSUPPORTED.*not exact"):
        B.experts(dev, x, ids, p, sg, True)
    ex = _exact(dev, xb)
    check_parity(Lh, xb, ex, O.DenseExperts(Lh), name=f"mxfp4-exact-exponent-{e_bad}", strict_y=1e-4)


def test_mxfp4_nan_and_subnormal_block_scales():
    """e = 255 in one gate block of an expert some rows pick makes exactly
    those rows NaN; e = 0 (2^-127) on a whole up projection of another
    expert leaves its rows finite and close to the oracle."""
    spec = replace(SMALL_MX, cfg_id=365, name="small-mxfp4-edge-scales")
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

"""GPU tests of the exact chunk form (moe_forward_exact): prompt rows with
the decode step's bits at chunk cost.

The pages ask that a prompt wider than 16 rows take the same sum as one row
before wide prompts are accepted ("Native server: --backend xpu for Nemotron
on Intel Arc", maintainer comment). moe_forward_exact runs the decode
router's per-row arithmetic for all rows, sorts the rows into expert blocks
of at most 16 and runs the decode kernels' per-row gate/up and down +
combine arithmetic on them. Checked here, bit for bit (fp32 words):
  * every row equals moe_forward_windows (the decode kernels in 16-row
    windows, itself equal to one-row steps) and sampled rows equal their
    one-row decode steps (route + decode experts on that row alone);
  * the result does not depend on how the chunk is cut into calls (the
    512-row chunk cut at 300, the 2048-row chunk cut at 1000 and at 37);
  * sampled rows against the fp64 oracle, per class through the taps.
Shapes: the 512-row 4-bit chunk, the 2048-row W4A16 Zipf chunk, the mixed
3-bit layer, an 8-bit layer and small layers (H=512) with 1, 17 and 40 rows.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth.gen import MX4G32, Q2G64, Q3G64, Q5G64, Q6G64, Q8G64, S4G128

from gpu_common import binding, build_layer, check_parity, log, run_gpu, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu

SMALL = synth.make_tiny_config(synth.CONFIGS[3], cfg_id=350, hidden=512, n_experts=64, top_k=8, inter=256,
                               shared_inter=256)
SMALL_ZIPF = replace(synth.make_tiny_config(synth.CONFIGS[4], cfg_id=351, hidden=512, n_experts=64, top_k=8,
                                            inter=256, shared_inter=256), bias="zipf")
MIXED3 = replace(synth.CONFIGS[2], cfg_id=352, name="exact-mixed-3bit", rows=(64,))
Q8 = replace(synth.CONFIGS[3], cfg_id=353, name="exact-512rows-q8g64-experts", routed=Q8G64, shared=Q8G64)
# intermediate 1024: four 256-wide K blocks per down matrix, two per wave of
# a wave pair, so each pass of two slots reloads its weights
WIDE_I = synth.make_tiny_config(synth.CONFIGS[3], cfg_id=354, hidden=512, n_experts=64, top_k=8, inter=1024,
                                shared_inter=1024)

_cache = {}


def layer_of(spec):
    if spec.cfg_id not in _cache:
        if len(_cache) > 1:
            _cache.clear()
        _cache[spec.cfg_id] = build_layer(spec, 0)
    return _cache[spec.cfg_id]


def _np(t):
    return t.cpu().numpy()


def _bias(Lh):
    torch = torch_mod()
    return torch.from_numpy(Lh.logit_bias).cuda() if Lh.logit_bias is not None else None


def exact(Lh, dev, xb, cuts=()):
    """moe_forward_exact over the chunk, cut into calls at `cuts`."""
    B = binding()
    torch = torch_mod()
    x = to_dev_x(xb)
    bias = _bias(Lh)
    bounds = [0, *cuts, xb.shape[0]]
    outs = [B.forward_exact(dev, x[a:b], bias) for a, b in zip(bounds[:-1], bounds[1:])]
    torch.cuda.synchronize()
    return {k_: np.concatenate([_np(o[i]) for o in outs]) for i, k_ in enumerate(("ids", "p", "sg", "y"))}


def windows(Lh, dev, xb):
    B = binding()
    torch = torch_mod()
    ids, p, sg, y = B.forward_windows(dev, to_dev_x(xb), _bias(Lh))
    torch.cuda.synchronize()
    return dict(ids=_np(ids), p=_np(p), sg=_np(sg), y=_np(y))


def assert_bits_equal(a, b, what):
    for key in ("ids", "p", "sg", "y"):
        u, v = a[key], b[key]
        if u.dtype == np.float32:
            u, v = u.view(np.uint32), v.view(np.uint32)
        bad = np.where(~np.all(u.reshape(len(u), -1) == v.reshape(len(v), -1), axis=1))[0]
        assert bad.size == 0, f"{what}: {key} differs on rows {bad[:8]}"


@pytest.mark.parametrize("spec,rows", [(SMALL, 1), (SMALL, 17), (SMALL, 40), (SMALL_ZIPF, 40), (MIXED3, 64)],
                         ids=["small-r1", "small-r17", "small-r40", "small-zipf-r40", "mixed3-r64"])
def test_exact_equals_windows_and_one_row_steps(spec, rows):
    log(f"case exact {spec.name} rows={rows}")
    Lh, dev = layer_of(spec)
    xb = synth.make_x(spec, 0, rows, rep=21)
    e = exact(Lh, dev, xb)
    assert_bits_equal(e, windows(Lh, dev, xb), f"{spec.name} exact vs windows")
    for r in sorted({0, rows // 2, rows - 1}):
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        assert_bits_equal({k_: e[k_][r:r + 1] for k_ in e}, solo, f"{spec.name} row {r} vs its one-row step")


@pytest.mark.parametrize("cfg,cuts", [(3, (300,)), (4, (1000,)), (4, (37, 1500))],
                         ids=["c3-cut300", "c4-cut1000", "c4-cut37-1500"])
def test_exact_is_cut_invariant_at_chunk_size(cfg, cuts):
    spec = synth.CONFIGS[cfg]
    log(f"case exact cut {spec.name} cuts={cuts}")
    Lh, dev = layer_of(spec)
    xb = synth.make_x(spec, 0, spec.rows[0], rep=5)
    whole = exact(Lh, dev, xb)
    assert_bits_equal(whole, exact(Lh, dev, xb, cuts), f"{spec.name} whole vs cut at {cuts}")
    if cuts == (300,) or cuts == (1000,):
        assert_bits_equal(whole, windows(Lh, dev, xb), f"{spec.name} exact vs windows")
    # sampled rows against the oracle, per class through the taps
    B = binding()
    torch = torch_mod()
    sel = np.unique(np.linspace(0, xb.shape[0] - 1, 12).astype(int))
    R, E, k, H = len(sel), spec.n_experts, spec.top_k, spec.hidden
    Imax = max(spec.inter, spec.shared_inter)
    f = dict(device="cuda", dtype=torch.float32)
    tp = dict(logits=torch.full((R, E + 1), float("nan"), **f), gu=torch.full((R, k + 1, 2, Imax), float("nan"), **f),
              h=torch.full((R, k + 1, Imax), float("nan"), **f), e=torch.full((R, k + 1, H), float("nan"), **f))
    ids, p, sg, y = B.forward_exact(dev, to_dev_x(xb[sel]), _bias(Lh), taps=tp)
    torch.cuda.synchronize()
    g = dict(ids=_np(ids), p=_np(p), sg=_np(sg), y=_np(y), **{k_: _np(v) for k_, v in tp.items()})
    assert_bits_equal(g, {k_: whole[k_][sel] for k_ in whole}, f"{spec.name} sampled rows alone vs in the chunk")
    check_parity(Lh, xb[sel], g, name=f"exact-c{cfg}-sampled", strict_y=1e-4)


def test_exact_8bit_experts_equal_windows():
    Lh, dev = layer_of(Q8)
    xb = synth.make_x(Q8, 0, 96, rep=2)
    assert_bits_equal(exact(Lh, dev, xb, (50,)), windows(Lh, dev, xb), "8-bit exact (cut at 50) vs windows")


def test_exact_wide_intermediate_equals_windows():
    """Down matrices of more K blocks than a wave pair holds at once: every
    pass of two slots of an expert block uses its own weights, so a block of
    many slots (40 rows, top-8 of 64 experts) equals the windows bit for bit
    (not only its first two slots)."""
    Lh, dev = layer_of(WIDE_I)
    xb = synth.make_x(WIDE_I, 0, 40, rep=23)
    assert_bits_equal(exact(Lh, dev, xb), windows(Lh, dev, xb), "inter-1024 exact vs windows")


@pytest.mark.parametrize("fmt,cid", [(Q3G64, 370), (Q8G64, 371), (Q2G64, 372), (Q5G64, 373), (Q6G64, 374),
                                     (S4G128, 375), (MX4G32, 376)],
                         ids=["q3", "q8", "q2", "q5", "q6", "s4g128", "mxfp4"])
def test_exact_wide_intermediate_formats_equal_windows(fmt, cid):
    """The same at intermediate 1024 for every other expert format (routed
    and shared of one format), each with its own exact-form kernels."""
    spec = replace(WIDE_I, cfg_id=cid, name=f"exact-inter1024-{cid}", routed=fmt, shared=fmt)
    log(f"case exact inter-1024 {spec.name}")
    Lh, dev = layer_of(spec)
    xb = synth.make_x(spec, 0, 40, rep=24)
    assert_bits_equal(exact(Lh, dev, xb), windows(Lh, dev, xb), f"{spec.name} exact vs windows")


def test_exact_refuses_a_short_workspace():
    B = binding()
    torch = torch_mod()
    Lh, dev = layer_of(SMALL)
    x = to_dev_x(synth.make_x(SMALL, 0, 40, rep=1))
    ws = B.new_workspace(dev, 20, B.MOE_WS_EXACT)
    with pytest.raises(B.MoeError, match="MOE_ENOSPACE.*MOE_WS_EXACT"):
        B.forward_exact(dev, x, ws=ws)
    torch.cuda.synchronize()

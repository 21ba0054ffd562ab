"""GPU parity of the grouped (prompt-chunk) path against the FP64 oracle.

Runs moe_route + moe_experts_grouped through the C ABI on an MI355X. The
grouped GEMMs dequantise to fp16 and sum in another order than the per-row
form, so outputs are judged by the tolerance (2e-3 of max|y| per row), not
bits; ids must still equal the oracle's except on near-tie rows.

Cases: the 512-row 4-bit chunk and the 2048-row W4A16 chunk with
Zipf-skewed routing (every row: ids, weights, gate/up, h, e and y against the
oracle's expert-major form, which dequantises each expert once), the
mixed-width layer (3-bit routed experts), and small layers (H=512, E=64)
whose row counts give empty experts, single-row tiles, large tiles with
ragged tails and a shared expert wider than the routed ones.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth

from gpu_common import build_layer, check_parity, log, run_gpu

pytestmark = pytest.mark.gpu

SMALL = synth.make_tiny_config(synth.CONFIGS[3], cfg_id=310, hidden=512, n_experts=64,
                               top_k=4, inter=256, shared_inter=256)
# W4A16 formats, Zipf-skewed routing (hot experts take 128-row tiles), shared
# expert twice as wide as the routed ones
SMALL_ZIPF = replace(synth.make_tiny_config(synth.CONFIGS[4], cfg_id=311, hidden=512,
                                            n_experts=64, top_k=8, inter=256,
                                            shared_inter=512), bias="zipf")

_cache = {}


def layer_of(spec, layer=0):
    key = (spec.cfg_id, spec.name, layer)
    if key not in _cache:
        if len(_cache) > 2:
            _cache.clear()
        Lh, dev = build_layer(spec, layer)
        _cache[key] = (Lh, dev, O.DenseExperts(Lh))
    return _cache[key]


def expert_rows(ids, E):
    return np.bincount(ids.reshape(-1), minlength=E)


@pytest.mark.parametrize("rows", [1, 7, 33, 130, 300])
def test_grouped_small_ragged(rows):
    log(f"case grouped small rows={rows}")
    Lh, dev, dense = layer_of(SMALL)
    xb = synth.make_x(SMALL, 0, rows, rep=20 + rows)
    g = run_gpu(dev, Lh, xb, grouped=True)
    check_parity(Lh, xb, g, dense, name=f"grouped-small-r{rows}")


@pytest.mark.parametrize("rows", [5, 96, 250])
def test_grouped_small_zipf_w4a16(rows):
    log(f"case grouped small zipf rows={rows}")
    Lh, dev, dense = layer_of(SMALL_ZIPF)
    xb = synth.make_x(SMALL_ZIPF, 0, rows, rep=40 + rows)
    g = run_gpu(dev, Lh, xb, grouped=True)
    rep, _ = check_parity(Lh, xb, g, dense, name=f"grouped-small-zipf-r{rows}")
    if rows == 250:
        # the skew puts at least one routed expert on the 128-row tiles
        assert expert_rows(g["ids"], SMALL_ZIPF.n_experts).max() >= 96


def test_grouped_chunk_512_rows_q4():
    spec = synth.CONFIGS[3]
    log("case grouped c3 rows=512")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, 512, rep=0)
    g = run_gpu(dev, Lh, xb, grouped=True)
    assert np.all(np.isfinite(g["y"]))
    check_parity(Lh, xb, g, dense, name="grouped-c3-r512", form="expert_major")


def test_grouped_chunk_2048_rows_w4a16_zipf():
    spec = synth.CONFIGS[4]
    log("case grouped c4 rows=2048")
    Lh, dev, dense = layer_of(spec)
    xb = synth.make_x(spec, 0, 2048, rep=0)
    g = run_gpu(dev, Lh, xb, grouped=True)
    assert np.all(np.isfinite(g["y"]))
    cnt = expert_rows(g["ids"], spec.n_experts)
    log(f"c4 rows per expert: max {cnt.max()} empty {(cnt == 0).sum()}")
    assert cnt.max() >= 128
    check_parity(Lh, xb, g, dense, name="grouped-c4-r2048", form="expert_major")


def test_grouped_mixed_3bit_routed():
    spec = synth.CONFIGS[2]
    log("case grouped c2 rows=64")
    Lh, dev, dense = layer_of(spec, 5)
    xb = synth.make_x(spec, 5, 64, rep=7)
    g = run_gpu(dev, Lh, xb, grouped=True)
    check_parity(Lh, xb, g, dense, name="grouped-c2-r64", form="expert_major")


@pytest.mark.parametrize("spec", [synth.CONFIGS[1], SMALL_ZIPF], ids=["c1", "small-zipf"])
def test_grouped_agrees_with_decode(spec):
    """Same routing bits; outputs of the two forms within the tolerance."""
    log(f"case grouped-vs-decode {spec.name}")
    Lh, dev, _ = layer_of(spec)
    xb = synth.make_x(spec, 0, 16 if spec.hidden == 512 else 8, rep=13)
    a = run_gpu(dev, Lh, xb, grouped=False, taps=False)
    b = run_gpu(dev, Lh, xb, grouped=True, taps=False)
    for key in ("ids", "p", "sg"):
        assert np.array_equal(a[key], b[key]), key
    err = O.row_error(b["y"], a["y"].astype(np.float64))
    assert err.max() <= 2e-3, err.max()


def test_grouped_is_deterministic():
    Lh, dev, _ = layer_of(SMALL_ZIPF)
    xb = synth.make_x(SMALL_ZIPF, 0, 250, rep=6)
    a = run_gpu(dev, Lh, xb, grouped=True, taps=False)
    b = run_gpu(dev, Lh, xb, grouped=True, taps=False)
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))


def test_grouped_nan_and_zero_rows():
    Lh, dev, dense = layer_of(SMALL)
    xb = synth.make_x(SMALL, 0, 40, rep=9)
    xb[3, 17] = 0x7FC0       # NaN in row 3
    xb[5, :] = 0             # all-zero row 5
    g = run_gpu(dev, Lh, xb, grouped=True)
    assert np.all(np.isnan(g["y"][3]))
    assert np.all(g["y"][5] == 0.0)
    check_parity(Lh, xb, g, dense, name="grouped-small-nan-zero")


def test_grouped_skips_out_of_range_ids_on_a_dirty_workspace():
    """Slots whose id is outside [0, E) add nothing (as in the decode form),
    also when the workspace holds an earlier call's slot outputs."""
    from gpu_common import binding, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    Lh, dev, _ = layer_of(SMALL)
    rows = 24
    x = to_dev_x(synth.make_x(SMALL, 0, rows, rep=91))
    ws = B.new_workspace(dev, rows, True)
    ids, p, sg = B.route(dev, x, ws=ws)
    B.experts(dev, x, ids, p, sg, True, ws=ws)        # leaves slot outputs behind
    bad = ids.clone()
    bad[::3, 1] = -1
    bad[1::4, 2] = SMALL.n_experts
    yg = B.experts(dev, x, bad, p, sg, True, ws=ws)
    parts = [B.experts(dev, x[i:i + 8], bad[i:i + 8], p[i:i + 8], sg[i:i + 8], False,
                       ws=B.new_workspace(dev, 8, False)) for i in range(0, rows, 8)]
    torch.cuda.synchronize()
    yd = torch.cat(parts).cpu().numpy().astype(np.float64)
    err = O.row_error(yg.cpu().numpy(), yd)
    assert err.max() <= 2e-3, err.max()

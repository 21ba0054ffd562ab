"""GPU parity at the largest layer shape the library accepts: hidden 4096,
routed and shared intermediate 2048, top-8, 4-bit affine g64 experts and
router with a bf16 gate row, 16 decode rows (the decode path's most).

What the shape reaches that the workload shapes (hidden 2048, intermediate
512) do not:
  * 16 K slices of 256 against the 8 waves of a gate/up workgroup, so every
    wave runs a second slice in place;
  * the decode gate/up LDS at its largest: 16 rows of 4096 activations,
    their chunk sums and the slice partials (152 KiB of the CU's 160);
  * 8 K blocks per down slot (4 per wave pair) and 64 output tiles per row;
  * 16 column blocks of 256 in the grouped gate/up GEMM and K = 4096 in its
    ring;
  * the exact form's 8-row passes (hidden above 3072).
The layer has 64 experts (13.5 MB each, 880 MB in all): the expert count
is not a shape limit of these kernels, and 256 experts of this size would
take 3.5 GB of host arrays to draw and pack.

The oracle (fp64, 200 MB per dequantised expert, held only while the
decode and grouped tests use it) runs on three sampled rows: every row's
outputs are independent of the other rows of its batch (checked bit for
bit at this shape below), so a sampled row's reference is the oracle on
that row alone. The 16 rows of every form are also compared with each
other bit for bit where the forms promise it."""
import pytest

import oracle.moe_oracle as O
import synth

from gpu_common import (assert_rows_bits_equal, binding, build_layer, check_parity, log, run_gpu,
                        to_dev_x, torch_mod)

pytestmark = pytest.mark.gpu

MAX = synth.make_tiny_config(synth.CONFIGS[1], cfg_id=395, hidden=4096, n_experts=64, top_k=8,
                             inter=2048, shared_inter=2048)
ROWS = 16
SAMPLE = [0, 7, 15]

_state = {}


def _layer():
    if "layer" not in _state:
        log(f"[max-shape] drawing and packing {MAX.name}: H={MAX.hidden} I={MAX.inter} E={MAX.n_experts}")
        Lh, dev = build_layer(MAX, 0)
        xb = synth.make_x(MAX, 0, ROWS, rep=91)
        _state["layer"] = (Lh, dev, xb)
    return _state["layer"]


def _oracle_dense():
    """The sampled rows' experts, dequantised once for the decode and
    grouped tests (about 27 experts, 5.4 GB of fp64)."""
    if "dense" not in _state:
        Lh, _, _ = _layer()
        _state["dense"] = O.DenseExperts(Lh)
    return _state["dense"]


def _bias(Lh):
    torch = torch_mod()
    return torch.from_numpy(Lh.logit_bias).cuda() if Lh.logit_bias is not None else None


def _rows(g, sel):
    return {k_: v[sel] for k_, v in g.items()}


def test_max_shape_decode_parity_and_batch_invariance():
    Lh, dev, xb = _layer()
    log(f"case max-shape decode rows={ROWS}")
    g = run_gpu(dev, Lh, xb)
    for r in SAMPLE:
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        assert_rows_bits_equal(_rows(g, [r]), solo, f"max-shape row {r} batch vs solo")
    log(f"[max-shape] oracle on rows {SAMPLE}")
    check_parity(Lh, xb[SAMPLE], _rows(g, SAMPLE), _oracle_dense(), name="decode-max-shape-r16",
                 form="expert_major")


def test_max_shape_grouped_parity():
    Lh, dev, xb = _layer()
    log(f"case max-shape grouped rows={ROWS}")
    g = run_gpu(dev, Lh, xb, grouped=True)
    log(f"[max-shape] oracle on rows {SAMPLE}")
    try:
        check_parity(Lh, xb[SAMPLE], _rows(g, SAMPLE), _oracle_dense(), name="grouped-max-shape-r16",
                     form="expert_major")
    finally:
        _state.pop("dense", None)


def test_max_shape_exact_equals_windows_and_decode():
    """moe_forward_exact (8-row passes at this hidden size) equals the
    16-row decode windows bit for bit on a ragged 40-row chunk, and its first
    16 rows equal the plain decode step of those rows."""
    Lh, dev, _ = _layer()
    B = binding()
    torch = torch_mod()
    xb = synth.make_x(MAX, 0, 40, rep=92)
    log("case max-shape exact vs windows rows=40")
    x = to_dev_x(xb)
    e = [t.cpu().numpy() for t in B.forward_exact(dev, x, _bias(Lh))]
    w = [t.cpu().numpy() for t in B.forward_windows(dev, x, _bias(Lh))]
    torch.cuda.synchronize()
    keys = ("ids", "p", "sg", "y")
    ed, wd = dict(zip(keys, e)), dict(zip(keys, w))
    assert_rows_bits_equal(ed, wd, "max-shape exact vs windows")
    d = run_gpu(dev, Lh, xb[:ROWS], taps=False)
    assert_rows_bits_equal(_rows(ed, slice(0, ROWS)), d, "max-shape exact vs decode")
    _state.clear()

"""GPU parity on a layer whose every dimension is off the workload shapes'
powers of two, within what the library accepts: hidden 1280, routed
intermediate 768, shared intermediate 256, top-6 of 64 experts.

What it reaches that the other tests do not:
  * 5 K slices of 256: a decode gate/up workgroup of 5 waves, the router's
    5 slice waves, and prompt-chunk logits with 3 of the 8 waves idle;
  * 20 output tiles of 64 per row in the decode down (not a multiple of the
    8 XCDs, so tiles map to workgroups without the XCD grouping) and 5 column
    blocks in the grouped down GEMM;
  * 3 K blocks per routed down matrix, split unevenly over a slot's two
    waves (two and one), in the decode and exact down;
  * routed and shared experts of different widths in every form (the
    shared gate/up's last column blocks skipped in the grouped GEMM);
  * 6 picks per row (slot counts not a power of two).
Every form is checked against the oracle (decode, grouped) or bit for bit
against the form it promises to equal (batch = solo, exact = windows =
decode). The same checks run at top-1 and top-3, and at the smallest
accepted shape (hidden and intermediates 256)."""
import pytest

import synth

from gpu_common import (assert_rows_bits_equal, binding, build_layer, check_parity, log, run_gpu,
                        to_dev_x, torch_mod)

pytestmark = pytest.mark.gpu

ODD = synth.make_tiny_config(synth.CONFIGS[1], cfg_id=396, hidden=1280, n_experts=64, top_k=6,
                             inter=768, shared_inter=256)

_state = {}


def _layer():
    if "layer" not in _state:
        log(f"[odd-shape] drawing and packing {ODD.name}: H={ODD.hidden} I={ODD.inter} "
            f"Is={ODD.shared_inter} k={ODD.top_k}")
        _state["layer"] = build_layer(ODD, 0)
    return _state["layer"]


def _bias(Lh):
    torch = torch_mod()
    return torch.from_numpy(Lh.logit_bias).cuda() if Lh.logit_bias is not None else None


@pytest.mark.parametrize("rows", [1, 7, 16])
def test_odd_shape_decode_parity(rows):
    Lh, dev = _layer()
    log(f"case odd-shape decode rows={rows}")
    xb = synth.make_x(ODD, 0, rows, rep=101 + rows)
    g = run_gpu(dev, Lh, xb)
    check_parity(Lh, xb, g, name=f"decode-odd-shape-r{rows}")
    if rows > 1:
        for r in (0, rows - 1):
            solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
            assert_rows_bits_equal({k_: v[r:r + 1] for k_, v in g.items()}, solo,
                                   f"odd-shape row {r} batch vs solo")


@pytest.mark.parametrize("rows", [33, 200])
def test_odd_shape_grouped_parity(rows):
    Lh, dev = _layer()
    log(f"case odd-shape grouped rows={rows}")
    xb = synth.make_x(ODD, 0, rows, rep=121 + rows)
    check_parity(Lh, xb, run_gpu(dev, Lh, xb, grouped=True), name=f"grouped-odd-shape-r{rows}",
                 form="expert_major")


def test_odd_shape_exact_equals_windows_and_decode():
    Lh, dev = _layer()
    B = binding()
    torch = torch_mod()
    xb = synth.make_x(ODD, 0, 45, rep=131)
    log("case odd-shape exact vs windows rows=45")
    x = to_dev_x(xb)
    keys = ("ids", "p", "sg", "y")
    e = dict(zip(keys, [t.cpu().numpy() for t in B.forward_exact(dev, x, _bias(Lh))]))
    w = dict(zip(keys, [t.cpu().numpy() for t in B.forward_windows(dev, x, _bias(Lh))]))
    torch.cuda.synchronize()
    assert_rows_bits_equal(e, w, "odd-shape exact vs windows")
    d = run_gpu(dev, Lh, xb[:16], taps=False)
    assert_rows_bits_equal({k_: v[:16] for k_, v in e.items()}, d, "odd-shape exact vs decode")
    _state.clear()


# top-1 and top-3 on 128 experts (two router tiles, so picks are handed from
# tile to tile): one or three slots per row, a down workgroup of two or six
# waves, a shared intermediate wider than the routed one
SMALL_K = {k: synth.make_tiny_config(synth.CONFIGS[1], cfg_id=396 + k, hidden=768, n_experts=128, top_k=k,
                                     inter=256, shared_inter=512) for k in (1, 3)}


@pytest.mark.parametrize("k", [1, 3])
def test_small_top_k_every_form(k):
    spec = SMALL_K[k]
    log(f"case top-{k} {spec.name}")
    Lh, dev = build_layer(spec, 0)
    B = binding()
    torch = torch_mod()
    xd = synth.make_x(spec, 0, 16, rep=141 + k)
    g = run_gpu(dev, Lh, xd)
    check_parity(Lh, xd, g, name=f"decode-top{k}-r16")
    solo = run_gpu(dev, Lh, xd[5:6], taps=False)
    assert_rows_bits_equal({k_: v[5:6] for k_, v in g.items()}, solo, f"top-{k} row 5 batch vs solo")
    xg = synth.make_x(spec, 0, 150, rep=151 + k)
    check_parity(Lh, xg, run_gpu(dev, Lh, xg, grouped=True), name=f"grouped-top{k}-r150",
                 form="expert_major")
    xe = synth.make_x(spec, 0, 37, rep=161 + k)
    x = to_dev_x(xe)
    keys = ("ids", "p", "sg", "y")
    e = dict(zip(keys, [t.cpu().numpy() for t in B.forward_exact(dev, x, _bias(Lh))]))
    w = dict(zip(keys, [t.cpu().numpy() for t in B.forward_windows(dev, x, _bias(Lh))]))
    torch.cuda.synchronize()
    assert_rows_bits_equal(e, w, f"top-{k} exact vs windows")


# the smallest shape accepted: one K slice (a decode gate/up workgroup of one
# wave, a one-slice router), 4 down tiles per row, one column block in the
# grouped down GEMM
MIN = synth.make_tiny_config(synth.CONFIGS[1], cfg_id=390, hidden=256, n_experts=64, top_k=8,
                             inter=256, shared_inter=256)


@pytest.mark.parametrize("rows", [1, 16])
def test_smallest_shape_every_form(rows):
    log(f"case smallest shape rows={rows}")
    Lh, dev = build_layer(MIN, 0)
    B = binding()
    torch = torch_mod()
    xd = synth.make_x(MIN, 0, rows, rep=171 + rows)
    g = run_gpu(dev, Lh, xd)
    check_parity(Lh, xd, g, name=f"decode-smallest-r{rows}")
    xg = synth.make_x(MIN, 0, 10 * rows, rep=181 + rows)
    check_parity(Lh, xg, run_gpu(dev, Lh, xg, grouped=True), name=f"grouped-smallest-r{10 * rows}",
                 form="expert_major")
    xe = synth.make_x(MIN, 0, 2 * rows + 3, rep=191 + rows)
    x = to_dev_x(xe)
    keys = ("ids", "p", "sg", "y")
    e = dict(zip(keys, [t.cpu().numpy() for t in B.forward_exact(dev, x, _bias(Lh))]))
    w = dict(zip(keys, [t.cpu().numpy() for t in B.forward_windows(dev, x, _bias(Lh))]))
    torch.cuda.synchronize()
    assert_rows_bits_equal(e, w, "smallest exact vs windows")

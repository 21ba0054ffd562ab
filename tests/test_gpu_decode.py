"""GPU parity of the router and the decode path against the FP64 oracle.

Runs through the C ABI (libmoe.so) on an MI355X. Inputs are the seeded
synthetic layers of the decode workloads: 4-bit g64 (1 and 8 rows), the
mixed-width layer (3-bit routed, 4-bit shared, 8-bit router and gate) and
the W4A16 formats, plus a small layer (H=512, E=64, k=4, I=256) for the
edge cases (16 rows, NaN and all-zero rows).
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth.gen import Q4G64, QTensor

from gpu_common import build_layer, check_parity, log, run_gpu

pytestmark = pytest.mark.gpu

SMALL = synth.make_tiny_config(synth.CONFIGS[0], cfg_id=300, hidden=512, n_experts=64,
                               top_k=4, inter=256, shared_inter=256)
SMALL_MIXED = synth.make_tiny_config(synth.CONFIGS[2], cfg_id=301, hidden=512, n_experts=64,
                                     top_k=8, inter=256, shared_inter=256)

_cache = {}


def layer_of(spec, layer=0):
    key = (spec.cfg_id, spec.name, layer)
    if key not in _cache:
        if len(_cache) > 3:
            _cache.clear()
        Lh, dev = build_layer(spec, layer)
        _cache[key] = (Lh, dev, O.DenseExperts(Lh))
    return _cache[key]


@pytest.mark.parametrize("cfg,rows,layer", [(0, 1, 0), (1, 8, 0), (1, 8, 39), (2, 1, 0),
                                            (2, 8, 17), (4, 8, 0)])
def test_decode_parity_workloads(cfg, rows, layer):
    spec = synth.CONFIGS[cfg]
    log(f"case decode cfg={cfg} rows={rows} layer={layer}")
    Lh, dev, dense = layer_of(spec, layer)
    xb = synth.make_x(spec, layer, rows, rep=3)
    g = run_gpu(dev, Lh, xb)
    rep, _ = check_parity(Lh, xb, g, dense, name=f"decode-c{cfg}-r{rows}-l{layer}", strict_y=1e-4)
    # the fp32 decode path reaches the fp64 reference closely on every class
    assert rep["logits"]["worst_col"] < 1e-4


@pytest.mark.parametrize("rows", [1, 5, 16])
def test_decode_parity_small_ragged_and_max_rows(rows):
    log(f"case decode small rows={rows}")
    Lh, dev, dense = layer_of(SMALL)
    xb = synth.make_x(SMALL, 0, rows, rep=rows)
    check_parity(Lh, xb, run_gpu(dev, Lh, xb), dense, name=f"decode-small-r{rows}", strict_y=1e-4)


@pytest.mark.parametrize("spec", [synth.CONFIGS[1], synth.CONFIGS[2], SMALL], ids=["c1", "c2", "small"])
def test_batch_equals_solo_bit_for_bit(spec):
    """A row's outputs are bit-identical alone or inside a batch of rows."""
    rows = 8 if spec.hidden == 2048 else 16
    log(f"case batch-invariance {spec.name} rows={rows}")
    Lh, dev, _ = layer_of(spec, 0)
    xb = synth.make_x(spec, 0, rows, rep=11)
    batch = run_gpu(dev, Lh, xb, taps=False)
    for r in range(rows):
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        for key in ("ids", "p", "sg", "y"):
            assert np.array_equal(solo[key][0].view(np.uint32) if solo[key].dtype == np.float32
                                  else solo[key][0],
                                  batch[key][r].view(np.uint32) if batch[key].dtype == np.float32
                                  else batch[key][r]), f"row {r} {key} differs"


def test_decode_is_deterministic():
    spec = synth.CONFIGS[1]
    Lh, dev, _ = layer_of(spec, 0)
    xb = synth.make_x(spec, 0, 8, rep=5)
    a = run_gpu(dev, Lh, xb, taps=False)
    b = run_gpu(dev, Lh, xb, taps=False)
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))


def _widen_to_q4(t):
    E = t.codes.shape[0]
    out = np.empty((E, t.rows, t.cols // 8), np.uint32)
    for e in range(E):
        q = O.unpack_codes(t.codes[e], 3, t.cols).astype(np.uint32).reshape(t.rows, -1, 8)
        w = np.zeros(q.shape[:2], np.uint32)
        for i in range(8):
            w |= q[:, :, i] << np.uint32(4 * i)
        out[e] = w
    return QTensor(Q4G64, t.rows, t.cols, out, t.scales, t.biases)


def test_3bit_equals_widened_4bit_bit_for_bit():
    """The pages' control: 3-bit codes rewritten as 4-bit words give the same bytes."""
    import copy
    from dataclasses import replace

    from gpu_common import binding
    from synth import to_abi
    B = binding()
    spec3 = SMALL_MIXED
    Lh3, dev3, _ = layer_of(spec3)
    spec4 = replace(spec3, routed=Q4G64)
    Lh4 = copy.copy(Lh3)
    Lh4.spec = spec4
    Lh4.gate, Lh4.up, Lh4.down = _widen_to_q4(Lh3.gate), _widen_to_q4(Lh3.up), _widen_to_q4(Lh3.down)
    dev4 = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec4)), to_abi.tensors(Lh4))
    xb = synth.make_x(spec3, 0, 8, rep=2)
    a = run_gpu(dev3, Lh3, xb)
    b = run_gpu(dev4, Lh4, xb)
    assert np.array_equal(a["ids"], b["ids"])
    for key in ("y", "h", "e"):
        assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), key
    check_parity(Lh3, xb, a, name="decode-small-mixed-3bit", strict_y=1e-4)


def test_nan_and_zero_rows():
    Lh, dev, dense = layer_of(SMALL)
    xb = synth.make_x(SMALL, 0, 4, rep=9)
    xb[1, 100] = 0x7FC0      # NaN in row 1
    xb[2, :] = 0             # all-zero row 2
    g = run_gpu(dev, Lh, xb)
    k = SMALL.top_k
    assert list(g["ids"][1]) == list(range(k)) and np.all(np.isnan(g["p"][1]))
    assert np.isnan(g["sg"][1]) and np.all(np.isnan(g["y"][1]))
    assert list(g["ids"][2]) == list(range(k)) and np.all(g["p"][2] == 1.0 / k)
    assert g["sg"][2] == 0.5 and np.all(g["y"][2] == 0.0)
    check_parity(Lh, xb, g, dense, name="decode-small-nan-zero")


def test_workspace_reused_across_row_counts_bit_for_bit():
    """One workspace, zero-filled once, serves calls of different row counts
    and both forms in turn (the decode router's hand-off words must be empty
    at the start of every call); each call gives the bytes a fresh workspace
    gives."""
    from gpu_common import binding, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    spec = synth.CONFIGS[1]
    Lh, dev, _ = layer_of(spec, 0)
    ws = B.new_workspace(dev, 64, True)      # sized for the largest call below
    calls = [(8, False), (1, False), (16, False), (64, True), (3, False), (32, True), (8, False), (1, False)]
    for i, (rows, grouped) in enumerate(calls):
        log(f"case workspace reuse call {i} rows={rows} grouped={grouped}")
        x = to_dev_x(synth.make_x(spec, 0, rows, rep=20 + i))
        ids, p, sg = B.route(dev, x, ws=ws)
        y = B.experts(dev, x, ids, p, sg, grouped, ws=ws)
        ids2, p2, sg2 = B.route(dev, x)
        y2 = B.experts(dev, x, ids2, p2, sg2, grouped)
        torch.cuda.synchronize()
        for name, u, v in (("ids", ids, ids2), ("p", p, p2), ("sg", sg, sg2), ("y", y, y2)):
            assert torch.equal(u.view(torch.int32), v.view(torch.int32)), f"call {i} rows {rows}: {name}"


def test_decode_16_row_window_at_full_size():
    """16 decode rows (the widest window) through a full-size layer: parity,
    and every row bit-identical to its one-row step. At this size the
    activations go to LDS by direct loads rather than through registers."""
    spec = synth.CONFIGS[1]
    Lh, dev, dense = layer_of(spec, 0)
    rows = 16
    log(f"case decode window rows={rows} full size")
    xb = synth.make_x(spec, 0, rows, rep=31)
    batch = run_gpu(dev, Lh, xb)
    check_parity(Lh, xb, batch, dense, name="decode-c1-r16", strict_y=1e-4)
    for r in (0, 7, 15):
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        for key in ("ids", "p", "sg", "y"):
            a_, b_ = solo[key][0], batch[key][r]
            if a_.dtype == np.float32:
                a_, b_ = a_.view(np.uint32), b_.view(np.uint32)
            assert np.array_equal(a_, b_), f"row {r} {key} differs"


def test_router_hand_off_repeated_calls():
    """Many back-to-back router calls on one workspace, two inputs in turn
    (no host sync between calls): every call's picks, weights and gates equal
    the first call's for the same input, bit for bit (a stale or torn
    hand-off word between tile workgroups would show as a changed pick)."""
    from gpu_common import binding, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    spec = synth.CONFIGS[1]
    Lh, dev, _ = layer_of(spec, 0)
    ws = B.new_workspace(dev, 8, False)
    xs = [to_dev_x(synth.make_x(spec, 0, 8, rep=40 + i)) for i in range(2)]
    ref = [B.route(dev, x, ws=ws) for x in xs]
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in r) for r in ref]
    outs = []
    for it in range(200):
        outs.append(B.route(dev, xs[it % 2], ws=ws))
    torch.cuda.synchronize()
    for it, o in enumerate(outs):
        for name, u, v in zip(("ids", "p", "sg"), o, ref[it % 2]):
            assert torch.equal(u.view(torch.int32), v.view(torch.int32)), f"call {it}: {name}"


def test_forward_windows_same_bits_however_cut():
    """moe_forward_windows over 40 prompt rows: one call (windows 16 + 16 + 8)
    and another cut (7 rows, then 33) give the same bits, each row equals its
    one-row decode step, and the rows pass parity against the oracle."""
    from gpu_common import binding, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    spec = synth.CONFIGS[1]
    Lh, dev, dense = layer_of(spec, 0)
    rows = 40
    log(f"case forward_windows rows={rows}")
    xb = synth.make_x(spec, 0, rows, rep=50)
    x = to_dev_x(xb)
    a = B.forward_windows(dev, x)
    b1 = B.forward_windows(dev, x[:7].contiguous())
    b2 = B.forward_windows(dev, x[7:].contiguous())
    torch.cuda.synchronize()
    g = {name: t.cpu().numpy() for name, t in zip(("ids", "p", "sg", "y"), a)}
    for i, name in enumerate(("ids", "p", "sg", "y")):
        cut = torch.cat([b1[i], b2[i]])
        assert torch.equal(a[i].view(torch.int32), cut.view(torch.int32)), f"{name} depends on the cut"
    for r in (0, 6, 7, 15, 16, 39):
        solo = run_gpu(dev, Lh, xb[r:r + 1], taps=False)
        for key in ("ids", "p", "sg", "y"):
            u, v = solo[key][0], g[key][r]
            if u.dtype == np.float32:
                u, v = u.view(np.uint32), v.view(np.uint32)
            assert np.array_equal(u, v), f"row {r} {key} differs from its one-row step"
    check_parity(Lh, xb, g, dense, name="forward-windows-c1-r40", strict_y=1e-4)


def _pick_biases(E, k, seed=7):
    """Logit-bias vectors that drive the top-k search through its hard cases;
    with x = 0 every logit equals its bias exactly."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    out = {}
    b = np.zeros(E, f32)                       # ties at the k-th place, across tiles
    b[[200, 17, 90, E - 1, 1]] = 3.0
    b[[250, 66, 130, 5, 199, 64]] = 2.0
    out["boundary-ties"] = b
    one = f32(1.0)                             # keys one unit in the last place apart
    steps = rng.integers(0, 12, E)
    b = np.array([np.nextafter(one, f32(2.0)) if s == 0 else one for s in steps], f32)
    for e in range(E):
        for _ in range(int(steps[e])):
            b[e] = np.nextafter(b[e], f32(2.0))
    out["last-bit"] = b
    b = -rng.uniform(1.0, 10.0, E).astype(f32) # negatives with both zeros on top
    b[[3, 100, 180]] = -0.0
    b[[40, 222]] = 0.0
    b[[9, 150]] = -np.float32(1e-38)           # denormal-sized just below zero
    out["signed-zeros"] = b
    b = rng.standard_normal(E).astype(f32)     # NaN above +inf above finite
    b[[130, 7]] = np.nan
    b[64] = np.inf
    b[rng.choice(E, 40, replace=False)] = -np.inf
    b[[130, 7]] = np.nan
    b[64] = np.inf
    out["nan-inf"] = b
    b = np.full(E, -np.inf, f32)               # fewer finite values than k
    b[[33, 190, 77]] = [0.5, -2.0, 0.5]
    out["mostly-minus-inf"] = b
    b = np.full(E, 0.5, f32)                   # one above a flat rest
    b[201] = 0.75
    out["flat-but-one"] = b
    out["normal"] = rng.standard_normal(E).astype(f32)
    return out


@pytest.mark.parametrize("cfg,rows", [(1, 3), (1, 40), (2, 3), (2, 40), (4, 3), (4, 40)])
def test_pick_order_from_crafted_logits(cfg, rows):
    """x = 0 makes every logit its logit bias, so crafted biases test the
    pick itself: ids equal the oracle's (value desc, id asc, NaN first,
    -0 == +0) bit for bit, p agrees within 1e-6 (NaN where the oracle's is),
    and the gate is sigmoid(0) = 1/2. 3 rows take the one-launch decode
    router, 40 rows the prompt-chunk logits kernel and the per-row pick;
    routers: 4-bit affine, 8-bit affine, int4-symmetric g128 with fp16
    activations and a bf16 gate row."""
    from gpu_common import binding, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    spec = synth.CONFIGS[cfg]
    Lh, dev, _ = layer_of(spec, 0)
    E, k, H = spec.n_experts, spec.top_k, spec.hidden
    x = to_dev_x(np.zeros((rows, H), np.uint16))
    for name, bias in _pick_biases(E, k).items():
        log(f"[pick] cfg {cfg} rows {rows} {name}")
        ids, p, sg = B.route(dev, x, logit_bias=torch.from_numpy(bias).cuda())
        torch.cuda.synchronize()
        ids, p, sg = ids.cpu().numpy(), p.cpu().numpy(), sg.cpu().numpy()
        ref = O.route(np.zeros((rows, H)), np.zeros((E, H)), np.zeros(H), k, logit_bias=bias)
        assert (ids == ref.ids).all(), f"{name}: ids {ids[0]} vs {ref.ids[0]}"
        nan = np.isnan(ref.p)
        assert (np.isnan(p) == nan).all(), f"{name}: NaN pattern of p"
        assert np.allclose(p[~nan], ref.p[~nan], rtol=1e-6, atol=1e-7), f"{name}: p {p[0]} vs {ref.p[0]}"
        assert (sg == 0.5).all(), f"{name}: gate"


def test_tree_window_rows_equal_one_row_steps():
    """A verify window shaped like a draft tree: 16 rows drawn from 6
    distinct inputs, some repeated (sibling branches that carry the same
    hidden state), so units serve up to several copies of a row in one pass.
    Every row equals its one-row step bit for bit, and equal inputs give
    equal bits."""
    spec = synth.CONFIGS[1]
    Lh, dev, _ = layer_of(spec, 3)
    base = synth.make_x(spec, 3, 6, rep=61)
    tree = [0, 1, 1, 2, 3, 3, 3, 4, 1, 5, 5, 0, 2, 4, 4, 3]
    xb = base[tree]
    g = run_gpu(dev, Lh, xb, taps=False)
    for r, src in enumerate(tree):
        solo = run_gpu(dev, Lh, base[src:src + 1], taps=False)
        for key in ("ids", "p", "sg", "y"):
            u, v = solo[key][0], g[key][r]
            if u.dtype == np.float32:
                u, v = u.view(np.uint32), v.view(np.uint32)
            assert np.array_equal(u, v), f"row {r} (input {src}) {key} differs"


def test_router_wait_bound_reports_rows_not_handed_off():
    """The decode router's failure path, forced from the host: with the
    test hook ending the hand-off wait at once, every row is reported as not
    handed off (ids -1, NaN weights and gate) instead of being picked from
    missing entries, and the failure is counted. The count is sticky: the
    next call on that workspace also reports failed rows (so do the windows
    of moe_forward_windows after it), until moe_route_failures clears it.
    Then, with no clearing of the workspace in between, the next call equals
    a call on a fresh workspace bit for bit: the late tiles' words of the
    failed call carry its epoch and are not taken for the new call's."""
    from gpu_common import binding, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    spec = synth.CONFIGS[1]
    Lh, dev, _ = layer_of(spec, 0)
    x = to_dev_x(synth.make_x(spec, 0, 8, rep=71))
    x2 = to_dev_x(synth.make_x(spec, 0, 16, rep=72))
    ref = B.route(dev, x, ws=B.new_workspace(dev, 8, False))
    ws = B.new_workspace(dev, 16, False)
    assert B.route_failures(ws) == 0
    ids, p, sg = B.route(dev, x, ws=ws, taps={"route_wait_limit": -1})
    torch.cuda.synchronize()
    assert (ids.cpu() == -1).all()
    assert torch.isnan(p.cpu()).all() and torch.isnan(sg.cpu()).all()
    # sticky: a normal call after the failure still reports failed rows,
    # and so does every window of a windowed prompt on that workspace
    ids2, p2, _ = B.route(dev, x, ws=ws)
    _, _, _, yw = B.forward_windows(dev, x2, ws=ws)
    torch.cuda.synchronize()
    assert (ids2.cpu() == -1).all() and torch.isnan(p2.cpu()).all()
    assert torch.isnan(yw.cpu()).all()
    # 8 rows of the failed call, 8 of the next one, 16 of the windows
    assert B.route_failures(ws, clear=True) == 32
    assert B.route_failures(ws) == 0
    # no zero-fill: the failed call's hand-off words are stale for this call
    for _ in range(3):
        again = B.route(dev, x, ws=ws)
        torch.cuda.synchronize()
        for name, u, v in zip(("ids", "p", "sg"), again, ref):
            assert torch.equal(u.view(torch.int32), v.view(torch.int32)), name
    assert B.route_failures(ws) == 0


@pytest.mark.parametrize("rows", [32, 33])
def test_route_at_the_one_launch_limit(rows):
    """32 rows are the most the one-launch decode router takes (128 tile
    workgroups that hand picks to one another, all resident at once); 33 go
    to the logits kernel and the per-row pick. At full size both give the
    oracle's ids (except near-tie rows), weights within 1e-5 and the gate
    within 1e-6."""
    from gpu_common import binding, check_ids, to_dev_x, torch_mod
    B = binding()
    torch = torch_mod()
    spec = synth.CONFIGS[1]
    Lh, dev, dense = layer_of(spec, 5)
    xb = synth.make_x(spec, 5, rows, rep=81)
    ids, p, sg = B.route(dev, to_dev_x(xb), ws=B.new_workspace(dev, rows, rows > 16))
    torch.cuda.synchronize()
    ids, p, sg = ids.cpu().numpy(), p.cpu().numpy(), sg.cpu().numpy()
    Wr, wg = dense.router()
    ref = O.route(O.act_to_f64(xb, spec.act), Wr, wg, spec.top_k)
    same, near, counts = check_ids(ref, ids, spec.top_k, f"route-r{rows}")
    assert np.allclose(p[same], ref.p[same], rtol=0, atol=1e-5)
    assert np.allclose(sg, ref.sigma, rtol=0, atol=1e-6)
    log(f"[route] rows {rows}: {counts}")

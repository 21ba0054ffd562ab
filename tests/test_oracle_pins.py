"""Pins of the FP64 oracle against what the pages and mathematics fix (CPU only).

Each test checks the oracle against something other than itself: hand-worked
words and values (tests/golden), a bit-by-bit pure-Python unpacker, exact
integer arithmetic, brute force over all experts, and invariants.
"""
import math
from dataclasses import replace
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth.gen import (MX4G32, Q2G64, Q3G64, Q4G64, Q5G64, Q6G64, Q8G64, S4G128, QFormat,
                       QTensor)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks(name):
    cases, cur = {}, None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = cases.setdefault(line[1:-1], {})
            continue
        k, *v = line.split()
        cur[k] = v
    return cases


# ------------------------------------------------------------ hand-worked words
@pytest.mark.parametrize("case", list(_blocks("dequant_words.txt")))
def test_hand_worked_dequant(case):
    c = _blocks("dequant_words.txt")[case]
    bits, group, cols = int(c["bits"][0]), int(c["group"][0]), int(c["cols"][0])
    mode = {"affine": O.AFFINE, "symmetric": O.SYMMETRIC}[c["mode"][0]]
    sd = O.FP16 if "scale_fp16" in c else O.BF16
    fmt = QFormat(bits, group, mode, sd)
    nw = cols * bits // 32
    words = np.zeros((1, nw), np.uint32)
    for i, w in enumerate(c["words"]):
        words[0, i] = int(w, 16)
    ng = cols // group
    s = np.full((1, ng), int((c.get("scale_bf16") or c["scale_fp16"])[0], 16), np.uint16)
    b = None
    if mode == O.AFFINE:
        b = np.full((1, ng), int(c["bias_bf16"][0], 16), np.uint16)
    q = O.unpack_codes(words, bits, cols)[0]
    qh = [int(v) for v in c["q_head"]]
    if mode == O.SYMMETRIC:
        assert list(q[: len(qh)]) == qh      # stored nibbles (offset binary)
    else:
        assert list(q[: len(qh)]) == qh
    W = O.dequant(fmt, words, s, b, cols)[0]
    wh = [float(v) for v in c["w_head"]]
    assert np.array_equal(W[: len(wh)], np.array(wh))
    x = np.zeros(cols)
    x[: int(c["ones_prefix"][0])] = 1.0
    assert float(W @ x) == float(c["dot"][0])


@pytest.mark.parametrize("case", list(_blocks("mxfp4_words.txt")))
def test_hand_worked_mxfp4(case):
    """E2M1 elements and E8M0 block scales against hand-worked values."""
    c = _blocks("mxfp4_words.txt")[case]
    cols = int(c["cols"][0])
    words = np.zeros((1, cols // 8), np.uint32)
    for i, w in enumerate(c["words"]):
        words[0, i] = int(w, 16)
    s = np.array([[int(v, 16) for v in c["scales"]]], np.uint8)
    W = O.dequant(MX4G32, words, s, None, cols)[0]
    for item in c["w_at"]:
        i, v = item.split(":")
        got, want = W[int(i)], float(v)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want)
    x = np.zeros(cols)
    x[: int(c["ones_prefix"][0])] = 1.0
    dot, want = float(W @ x), float(c["dot"][0])
    assert (math.isnan(dot) and math.isnan(want)) or dot == want


def test_e8m0_matches_torch_dtype():
    """Every E8M0 byte against torch's float8_e8m0fnu conversion (a library
    implementation of the same OCP type)."""
    torch = pytest.importorskip("torch")
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.e8m0_to_f64(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_mxfp4_row_is_blockwise_scaled_codes():
    """A random MXFP4 row equals its codes' values times its block scales:
    scaling one block's exponent by +1 doubles exactly that block."""
    rng = np.random.default_rng(11)
    cols = 256
    words = rng.integers(0, 1 << 32, size=(1, cols // 8), dtype=np.uint32)
    s = rng.integers(100, 150, size=(1, cols // 32)).astype(np.uint8)
    W = O.dequant(MX4G32, words, s, None, cols)[0]
    s2 = s.copy()
    s2[0, 3] += 1
    W2 = O.dequant(MX4G32, words, s2, None, cols)[0]
    blk = np.arange(cols) // 32
    assert np.array_equal(W2[blk == 3], 2.0 * W[blk == 3])
    assert np.array_equal(W2[blk != 3], W[blk != 3])
    # magnitudes come from the 8-value set times the block scale
    mags = np.abs(W) / np.exp2(s[0, blk].astype(np.float64) - 127.0)
    assert set(np.unique(mags)) <= {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}


def _py_unpack(words_row, bits, cols):
    """Element i = stream bits [bits*i, bits*i+bits); stream bit t = bit t%32 of word t//32."""
    out = []
    for i in range(cols):
        v = 0
        for j in range(bits):
            t = bits * i + j
            v |= ((int(words_row[t // 32]) >> (t % 32)) & 1) << j
        out.append(v)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_unpack_matches_bit_by_bit_definition(bits):
    rng = np.random.default_rng(7 + bits)
    cols = 256
    words = rng.integers(0, 1 << 32, size=(5, cols * bits // 32), dtype=np.uint32)
    q = O.unpack_codes(words, bits, cols)
    for r in range(words.shape[0]):
        assert list(q[r]) == _py_unpack(words[r], bits, cols)


def test_bf16_fp16_exact_conversion():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = smallest bf16 subnormal 2^-133
    v = O.half_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F80], np.uint16), O.BF16)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133 and v[3] == np.inf
    # fp16: 0x3C00 = 1, 0x0001 = 2^-24, 0x7BFF = 65504
    v = O.half_bits_to_f64(np.array([0x3C00, 0x0001, 0x7BFF], np.uint16), O.FP16)
    assert list(v) == [1.0, 2.0 ** -24, 65504.0]


# ------------------------------------------------------------ exact integer case
@pytest.mark.parametrize("fmt", [Q4G64, Q3G64, Q8G64, Q2G64, Q5G64, Q6G64, S4G128])
def test_integer_exact_projection(fmt):
    """s = 2^-k per group (k varies), b = -c*s: every projection is a dyadic rational."""
    rng = np.random.default_rng(11)
    rows, cols = 6, 256
    words = rng.integers(0, 1 << 32, size=(rows, cols * fmt.bits // 32), dtype=np.uint32)
    ng = cols // fmt.group
    kexp = rng.integers(3, 9, size=(rows, ng))
    off = {2: 2, 3: 4, 4: 8, 5: 16, 6: 32, 8: 128}[fmt.bits]
    # bf16 / fp16 bits of 2^-k and -off * 2^-k
    if fmt.scale_dtype == O.BF16:
        s_bits = ((127 - kexp) << 7).astype(np.uint16)
        lo = int(math.log2(off))
        b_bits = (0x8000 | ((127 - kexp + lo) << 7)).astype(np.uint16)
    else:
        s_bits = ((15 - kexp) << 10).astype(np.uint16)
        b_bits = None
    if fmt.mode == O.SYMMETRIC:
        b_bits = None
    x_int = rng.integers(-4, 5, size=cols)
    W = O.dequant(fmt, words, s_bits, b_bits, cols)
    got = W @ x_int.astype(np.float64)
    for r in range(rows):
        q = _py_unpack(words[r], fmt.bits, cols)
        acc = Fraction(0)
        for i in range(cols):
            k = int(kexp[r, i // fmt.group])
            acc += Fraction(q[i] - off, 2 ** k) * int(x_int[i])
        assert Fraction(got[r]) == acc


def test_mxfp4_exact_projection():
    """Scales 2^(e-127) for random e and small integer activations: every
    projection is a dyadic rational, checked against exact sums of the
    hand-worked E2M1 values (tests/golden/mxfp4_words.txt, all 16 codes)."""
    table = {}
    for item in _blocks("mxfp4_words.txt")["e2m1_table"]["w_at"][:16]:
        i, v = item.split(":")
        table[int(i)] = Fraction(float(v))
    rng = np.random.default_rng(12)
    rows, cols = 5, 256
    words = rng.integers(0, 1 << 32, size=(rows, cols // 8), dtype=np.uint32)
    e = rng.integers(117, 137, size=(rows, cols // 32)).astype(np.uint8)
    x_int = rng.integers(-4, 5, size=cols)
    got = O.dequant(MX4G32, words, e, None, cols) @ x_int.astype(np.float64)
    for r in range(rows):
        q = _py_unpack(words[r], 4, cols)
        acc = Fraction(0)
        for i in range(cols):
            acc += table[q[i]] * Fraction(2) ** (int(e[r, i // 32]) - 127) * int(x_int[i])
        assert Fraction(got[r]) == acc


# ------------------------------------------------------------ routing
def _hand_routing():
    c = {}
    for line in open(os.path.join(GOLDEN, "routing_hand.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, *v = line.split()
            c[k] = v
    return c


def test_hand_routing_example():
    c = _hand_routing()
    lg = np.array([float(v) for v in c["logits"]])
    E, k = lg.size, int(c["k"][0])
    x = lg[None, :]
    rt = O.route(x, np.eye(E), np.zeros(E), k)
    assert list(rt.ids[0]) == [int(v) for v in c["ids"]]
    assert np.allclose(rt.p[0], [float(v) for v in c["p"]], rtol=0, atol=5e-9)
    assert rt.sigma[0] == float(c["sigma"][0])
    # the near-tie measure: the k-th minus the (k+1)-th sorted logit
    assert rt.gap[0] == float(c["gap"][0])


def _cmp_key(v, e):
    # NaN first, then larger value, then lower id (a direct comparator form)
    if math.isnan(v):
        return (0, 0.0, e)
    return (1, -v, e)


def test_topk_against_comparator_sort_with_ties_and_nan():
    rng = np.random.default_rng(3)
    R, E, k = 200, 64, 8
    l = rng.integers(-3, 4, size=(R, E)).astype(np.float32)       # many exact ties
    l[5, 10] = np.nan
    l[6, :] = np.nan
    l[7, 3] = np.inf
    l[8, :] = 0.0
    l[8, 5] = -0.0
    ids = O.topk_ids(l, k)
    for r in range(R):
        ref = sorted(range(E), key=lambda e: _cmp_key(float(l[r, e]) + 0.0, e))[:k]
        assert list(ids[r]) == ref


def test_flat_row_closed_form():
    spec = synth.make_tiny_config(synth.CONFIGS[0], cfg_id=101)
    L = synth.make_layer(spec, 0)
    x = np.zeros((1, spec.hidden), np.uint16)
    out = O.moe_forward(L, x)
    assert list(out.routing.ids[0]) == list(range(spec.top_k))
    assert np.all(out.routing.p == 1.0 / spec.top_k)
    assert out.routing.sigma[0] == 0.5
    assert np.all(out.y == 0.0)


def test_nan_row():
    spec = synth.make_tiny_config(synth.CONFIGS[0], cfg_id=102)
    L = synth.make_layer(spec, 0)
    x = synth.make_x(spec, 0, 2)
    x[1, 17] = 0x7FC0            # bf16 quiet NaN
    out = O.moe_forward(L, x)
    assert list(out.routing.ids[1]) == list(range(spec.top_k))
    assert np.all(np.isnan(out.routing.p[1])) and np.isnan(out.routing.sigma[1])
    assert np.all(np.isnan(out.y[1]))
    assert np.all(np.isfinite(out.y[0]))


# ------------------------------------------------------------ experts
def test_swiglu_hand_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "swiglu_hand.txt"))
            if l.strip() and not l.startswith("#")]
    g = np.array([float(r[0]) for r in rows])
    u = np.array([float(r[1]) for r in rows])
    h = np.array([float(r[2]) for r in rows])
    assert np.allclose(O.silu(g) * u, h, rtol=0, atol=5e-9)


def test_expert_against_python_loops_gate_up_distinct():
    """A tiny expert evaluated with pure-Python loops and math.exp."""
    rng = np.random.default_rng(5)
    H, I = 12, 5
    Wg, Wu, Wd = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    x = rng.normal(size=H)
    g, u, h, e = O.swiglu_expert(x[None], Wg, Wu, Wd)
    for i in range(I):
        gi = sum(Wg[i, j] * x[j] for j in range(H))
        ui = sum(Wu[i, j] * x[j] for j in range(H))
        hi = gi / (1 + math.exp(-gi)) * ui
        assert abs(h[0, i] - hi) < 1e-12
    for o in range(H):
        hh = [sum(Wg[i, j] * x[j] for j in range(H)) for i in range(I)]
        uu = [sum(Wu[i, j] * x[j] for j in range(H)) for i in range(I)]
        eo = sum(Wd[o, i] * (hh[i] / (1 + math.exp(-hh[i])) * uu[i]) for i in range(I))
        assert abs(e[0, o] - eo) < 1e-11


def _tiny(base_id, cfg_id, **kw):
    return synth.make_tiny_config(synth.CONFIGS[base_id], cfg_id=cfg_id, **kw)


@pytest.mark.parametrize("base", [0, 2, 4, "mx"])
def test_brute_force_all_experts(base):
    """Dense evaluation of every expert for every row, combined by a dense
    routing-weight matrix that is zero off the picks."""
    if base == "mx":
        spec = replace(_tiny(2, 116), routed=MX4G32, shared=MX4G32)
    else:
        spec = _tiny(base, 110 + base)
    L = synth.make_layer(spec, 0)
    R = 9
    xb = synth.make_x(spec, 0, R)
    out = O.moe_forward(L, xb)
    dense = O.DenseExperts(L)
    x = O.act_to_f64(xb, spec.act)
    Wr, wg = dense.router()
    E, k = spec.n_experts, spec.top_k
    Pm = np.zeros((R, E))
    for r in range(R):
        for j in range(k):
            Pm[r, out.routing.ids[r, j]] = out.routing.p[r, j]
    ysum = np.zeros((R, spec.hidden))
    for e in range(E):
        Wg, Wu, Wd = dense.expert(e)
        ysum += Pm[:, e:e + 1] * (((x @ Wg.T) * O.sigmoid(x @ Wg.T) * (x @ Wu.T)) @ Wd.T)
    Wg, Wu, Wd = dense.expert(E)
    ysum += O.sigmoid(x @ wg)[:, None] * (((x @ Wg.T) * O.sigmoid(x @ Wg.T) * (x @ Wu.T)) @ Wd.T)
    assert np.max(np.abs(out.y - ysum)) <= 1e-12 * np.max(np.abs(ysum))


def test_invariants_and_forms_agree():
    spec = _tiny(0, 120)
    L = synth.make_layer(spec, 0)
    xb = synth.make_x(spec, 0, 33)
    a = O.moe_forward(L, xb, form="per_row")
    b = O.moe_forward(L, xb, form="expert_major")
    assert np.array_equal(a.routing.ids, b.routing.ids)
    assert np.max(np.abs(a.y - b.y)) <= 1e-12 * np.max(np.abs(a.y))
    p = a.routing.p
    assert np.allclose(p.sum(1), 1.0, atol=1e-12, rtol=0)
    assert np.all(np.diff(p, axis=1) <= 1e-15)                # non-increasing
    assert np.all((a.routing.sigma > 0) & (a.routing.sigma < 1))


def test_grouped_equals_per_token_rows():
    """A batch of rows gives each row the same result as running it alone."""
    spec = _tiny(0, 121)
    L = synth.make_layer(spec, 0)
    xb = synth.make_x(spec, 0, 7)
    dense = O.DenseExperts(L)
    batch = O.moe_forward(L, xb, dense, form="expert_major")
    for r in range(7):
        solo = O.moe_forward(L, xb[r:r + 1], dense)
        assert np.array_equal(solo.routing.ids[0], batch.routing.ids[r])
        assert np.max(np.abs(solo.y[0] - batch.y[r])) <= 1e-12 * np.max(np.abs(solo.y[0]))


def test_relabelling_experts_permutes_ids_only():
    spec = _tiny(0, 122)
    L = synth.make_layer(spec, 0)
    xb = synth.make_x(spec, 0, 5)
    out = O.moe_forward(L, xb)
    assert np.all(out.routing.gap > 1e-9)
    perm = np.random.default_rng(1).permutation(spec.n_experts)   # new id n holds old perm[n]
    import copy
    L2 = copy.copy(L)

    def pq(t):
        return QTensor(t.fmt, t.rows, t.cols, t.codes[perm],
                       None if t.scales is None else t.scales[perm],
                       None if t.biases is None else t.biases[perm])
    L2.router, L2.gate, L2.up, L2.down = pq(L.router), pq(L.gate), pq(L.up), pq(L.down)
    out2 = O.moe_forward(L2, xb)
    inv = np.argsort(perm)
    assert np.array_equal(out2.routing.ids, inv[out.routing.ids])
    assert np.max(np.abs(out2.y - out.y)) <= 1e-12 * np.max(np.abs(out.y))


def test_k1_single_pick_is_one_dense_mlp():
    spec = _tiny(0, 123, top_k=1)
    L = synth.make_layer(spec, 0)
    xb = synth.make_x(spec, 0, 3)
    out = O.moe_forward(L, xb)
    assert np.all(out.routing.p == 1.0)
    dense = O.DenseExperts(L)
    x = O.act_to_f64(xb, spec.act)
    for r in range(3):
        e = int(out.routing.ids[r, 0])
        y1 = O.swiglu_expert(x[r:r + 1], *dense.expert(e))[3][0]
        ys = O.swiglu_expert(x[r:r + 1], *dense.expert(spec.n_experts))[3][0]
        ref = y1 + out.routing.sigma[r] * ys
        assert np.max(np.abs(out.y[r] - ref)) <= 1e-12 * np.max(np.abs(ref))


# ------------------------------------------------------------ format identities
def _pack_lsb(q: np.ndarray, bits: int) -> np.ndarray:
    """Test-side LSB-first packer (independent of the library's packer)."""
    rows, cols = q.shape
    out = np.zeros((rows, cols * bits // 32), np.uint32)
    for r in range(rows):
        acc = 0
        for i in range(cols):
            acc |= int(q[r, i]) << (bits * i)
        for w in range(out.shape[1]):
            out[r, w] = (acc >> (32 * w)) & 0xFFFFFFFF
    return out


def test_3bit_widened_to_4bit_is_identical():
    """The pages' control: 3-bit codes rewritten as 4-bit words give the same layer."""
    spec3 = _tiny(2, 130)
    L3 = synth.make_layer(spec3, 0)
    import copy
    L4 = copy.copy(L3)

    def widen(t):
        E = t.codes.shape[0]
        c4 = np.stack([_pack_lsb(O.unpack_codes(t.codes[e], 3, t.cols), 4) for e in range(E)])
        return QTensor(Q4G64, t.rows, t.cols, c4, t.scales, t.biases)
    L4.gate, L4.up, L4.down = widen(L3.gate), widen(L3.up), widen(L3.down)
    xb = synth.make_x(spec3, 0, 6)
    a, b = O.moe_forward(L3, xb), O.moe_forward(L4, xb)
    assert np.array_equal(a.y, b.y) and np.array_equal(a.routing.ids, b.routing.ids)


def test_symmetric_equals_affine_with_bias_minus_8s():
    rng = np.random.default_rng(9)
    rows, cols = 8, 512
    words = rng.integers(0, 1 << 32, size=(rows, cols // 8), dtype=np.uint32)
    s = synth.f64_to_fp16_bits(rng.uniform(0.002, 0.02, size=(rows, cols // 128)))
    Wsym = O.dequant(S4G128, words, s, None, cols)
    b = synth.f64_to_fp16_bits(-8.0 * O.half_bits_to_f64(s, O.FP16))
    Waff = O.dequant(QFormat(4, 128, O.AFFINE, O.FP16), words, s, b, cols)
    assert np.array_equal(Wsym, Waff)
    # group 128 equals group 64 with each scale duplicated
    W64 = O.dequant(QFormat(4, 64, O.SYMMETRIC, O.FP16), words, np.repeat(s, 2, axis=1), None, cols)
    assert np.array_equal(Wsym, W64)


def test_zipf_skew_and_uniform_occupancy():
    """Workload structure: Zipf bias makes the hottest expert > 10x the mean."""
    spec = _tiny(4, 140, n_experts=64, hidden=256, inter=64, shared_inter=64)
    L = synth.make_layer(spec, 0)
    xb = synth.make_x(spec, 0, 512)
    dense = O.DenseExperts(L)
    x = O.act_to_f64(xb, spec.act)
    Wr, wg = dense.router()
    rt = O.route(x, Wr, wg, spec.top_k, L.logit_bias)
    cnt = np.bincount(rt.ids.ravel(), minlength=spec.n_experts)
    assert cnt.max() > 10 * cnt.mean()


def test_router_logits_are_unit_scale():
    spec = synth.CONFIGS[0]
    rng_layer = synth.make_layer(synth.make_tiny_config(spec, cfg_id=150, hidden=2048,
                                                        n_experts=64, inter=64,
                                                        shared_inter=64), 0)
    xb = synth.make_x(rng_layer.spec, 0, 64)
    x = O.act_to_f64(xb, O.BF16)
    Wr = O.dequant_qtensor(rng_layer.router)
    l = x @ Wr.T
    assert 0.8 < l.std() < 1.25


def test_gate_goes_through_silu_not_up():
    """Gate weights all -1 and x = 1: g = -H, silu(g) ~ 0, so routed slots vanish.
    With gate and up swapped the slots would be large."""
    import copy
    spec = _tiny(0, 160)
    L = copy.copy(synth.make_layer(spec, 0))
    t = L.gate
    codes = np.zeros_like(t.codes)
    biases = np.full_like(t.biases, 0xBF80)          # bf16 -1.0: w = s*0 + (-1)
    L.gate = QTensor(t.fmt, t.rows, t.cols, codes, t.scales, biases)
    xb = np.full((2, spec.hidden), 0x3F80, np.uint16)  # x = 1
    out = O.moe_forward(L, xb)
    assert np.max(np.abs(out.h[:, : spec.top_k, :])) < 1e-30
    ys = out.routing.sigma[:, None] * out.e[:, spec.top_k, :]
    assert np.max(np.abs(out.y - ys)) <= 1e-12 * np.max(np.abs(ys))


def test_logit_bias_is_added():
    E, k = 8, 2
    x = np.zeros((1, E))
    bias = np.zeros(E, np.float32)
    bias[5] = 10.0
    bias[2] = 3.0
    rt = O.route(x, np.eye(E), np.zeros(E), k, bias)
    assert list(rt.ids[0]) == [5, 2]
    assert np.allclose(rt.p[0], [1 / (1 + math.exp(-7)), math.exp(-7) / (1 + math.exp(-7))])


# ------------------------------------------------------------ parity metrics
def _metric_blocks():
    """[name] blocks of tests/golden/error_metrics_hand.txt; matrices as rows
    separated by '|'."""
    out = {}
    for name, kv in _blocks("error_metrics_hand.txt").items():
        d = {}
        for key, v in kv.items():
            if "|" in v:
                rows, cur = [], []
                for t in v:
                    if t == "|":
                        rows.append(cur)
                        cur = []
                    else:
                        cur.append(float(t))
                rows.append(cur)
                d[key] = np.array(rows)
            else:
                d[key] = np.array([float(t) for t in v])
        out[name] = d
    return out


def test_row_error_hand_worked():
    """Each row is normalised by its own max|ref| (not the batch's)."""
    c = _metric_blocks()["row_error"]
    err = O.row_error(c["got"], c["ref"])
    assert np.array_equal(err, c["err"])


def test_class_errors_hand_worked():
    """Worst column (per-column normalisation) and the Frobenius aggregate,
    rows with a non-finite reference left out."""
    c = _metric_blocks()["class_errors"]
    rep = O.class_errors(c["got"], c["ref"])
    assert rep["worst_col"] == float(c["worst_col"][0])
    assert abs(rep["aggregate"] - float(c["aggregate"][0])) <= 1e-9
    assert rep["max_abs"] == float(c["max_abs"][0])


def test_dense_row_is_bf16():
    """A DENSE row holds bf16 bit patterns (hand-worked values)."""
    c = {}
    for line in open(os.path.join(GOLDEN, "dense_row_hand.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, *v = line.split()
            c[k] = v
    bits = np.array([[int(b, 16) for b in c["bits"]]], np.uint16)
    W = O.dequant(synth.gen.DENSE_BF16, bits, None, None, bits.shape[1])
    assert list(W[0]) == [float(v) for v in c["values"]]


def test_gap_is_kth_minus_next():
    """gap = (k-th) - (k+1)-th sorted logit, for several k on one row."""
    lg = np.array([[5.0, -1.0, 3.0, 3.0, 0.5, 2.0]])
    for k, want in ((1, 2.0), (2, 0.0), (3, 1.0), (4, 1.5), (5, 1.5)):
        rt = O.route(lg, np.eye(6), np.zeros(6), k)
        assert rt.gap[0] == want, (k, rt.gap[0])

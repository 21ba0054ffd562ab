"""Host-side checks of the C ABI (no GPU needed): exports, refusals, pack layout.

The packed layout is decoded here by a test-side reader written from the
layout description in include/moe.h, and compared with the oracle's unpack
of the canonical input.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle.moe_oracle as O
import synth
from synth import to_abi
from synth.gen import MX4G32, Q2G64, Q3G64, Q4G64, Q5G64, Q6G64, S4G128
from dataclasses import replace

qr = pytest.importorskip("quantized_routed_expert_fp32_amd")
B = qr.binding
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return B.lib()


def test_exports_every_declared_symbol():
    L = _lib()
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", hdr, re.M))
    assert declared, "no declarations parsed"
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(L, name)


def _desc(spec):
    return B.layer_desc(*to_abi.desc_args(spec))


def test_pack_size_matches_layout_arithmetic():
    _lib()
    spec = synth.CONFIGS[1]
    n = B.pack_size(_desc(spec))
    # one 4-bit g64 expert: gate+up codes 1 MiB, scales 128 KiB; down 512 KiB + 64 KiB
    expert = 1024 * 2048 // 2 + 1024 * 32 * 4 + 2048 * 512 // 2 + 2048 * 8 * 4
    assert expert == 1769472
    a256 = lambda v: (v + 255) // 256 * 256        # every section starts 256-byte aligned
    router = a256(256 * 2048 // 2) + a256(256 * 32 * 4)
    gate_row = a256(2048 // 2) + a256(32 * 4)
    assert n == router + gate_row + 257 * expert


@pytest.mark.parametrize("cls,fmt", [
    ("routed", (7, 64, 0, 0)), ("routed", (5, 128, 0, 0)), ("router", (3, 64, 0, 0)),
    ("router", (6, 64, 0, 0)),
    ("router", (2, 64, 0, 0)), ("gate_row", (2, 64, 0, 0)),
    ("shared", (4, 32, 0, 0)), ("routed", (4, 128, 1, 0)), ("gate_row", (16, 0, 2, 1)),
])
def test_unsupported_formats_refused_by_name(cls, fmt):
    _lib()
    spec = synth.CONFIGS[0]
    args = list(to_abi.desc_args(spec))
    idx = {"router": 6, "gate_row": 7, "routed": 8, "shared": 9}[cls]
    args[idx] = fmt
    with pytest.raises(B.MoeError) as ei:
        B.pack_size(B.layer_desc(*args))
    msg = str(ei.value)
    assert "MOE_EUNSUPPORTED" in msg
    assert {"router": "router", "gate_row": "gate row", "routed": "routed experts",
            "shared": "shared expert"}[cls] in msg


@pytest.mark.parametrize("routed,shared,ok", [(Q5G64, Q5G64, True), (Q6G64, Q4G64, True),
                                               (Q5G64, Q3G64, False), (Q4G64, Q6G64, False),
                                               (Q5G64, Q6G64, False)])
def test_wide_expert_pairings(routed, shared, ok):
    """5/6-bit experts pair with a shared expert of the same width or 4-bit
    affine; other pairings are refused by name before anything is built."""
    _lib()
    spec = replace(synth.CONFIGS[0], routed=routed, shared=shared)
    d = B.layer_desc(*to_abi.desc_args(spec))
    if ok:
        assert B.pack_size(d) > 0
    else:
        with pytest.raises(B.MoeError, match="MOE_EUNSUPPORTED.*5- and 6-bit experts pair"):
            B.pack_size(d)


@pytest.mark.parametrize("routed,shared,ok", [(MX4G32, MX4G32, True), (MX4G32, Q4G64, True),
                                               (Q4G64, MX4G32, False), (MX4G32, S4G128, False),
                                               (MX4G32, Q3G64, False)])
def test_mxfp4_expert_pairings(routed, shared, ok):
    """MXFP4 routed experts pair with an MXFP4 or 4-bit affine shared expert;
    other pairings are refused by name before anything is built."""
    _lib()
    spec = replace(synth.CONFIGS[0], routed=routed, shared=shared)
    d = B.layer_desc(*to_abi.desc_args(spec))
    if ok:
        assert B.pack_size(d) > 0
    else:
        with pytest.raises(B.MoeError, match="MOE_EUNSUPPORTED.*MXFP4 routed experts pair"):
            B.pack_size(d)


@pytest.mark.parametrize("cls", ["router", "gate_row"])
def test_mxfp4_router_and_gate_row_refused(cls):
    _lib()
    args = list(to_abi.desc_args(synth.CONFIGS[0]))
    args[{"router": 6, "gate_row": 7}[cls]] = (4, 32, 3, 2)
    with pytest.raises(B.MoeError, match="MOE_EUNSUPPORTED.*mxfp4"):
        B.pack_size(B.layer_desc(*args))


@pytest.mark.parametrize("field,val", [("hidden", 300), ("n_experts", 100), ("top_k", 9),
                                       ("inter", 384)])
def test_unsupported_shapes_refused(field, val):
    _lib()
    d = _desc(synth.CONFIGS[0])
    setattr(d, field, val)
    with pytest.raises(B.MoeError, match=field):
        B.pack_size(d)


def test_workspace_limits():
    _lib()
    d = _desc(synth.CONFIGS[1])
    assert B.workspace_size(d, 8, False) > 0
    with pytest.raises(B.MoeError, match="decode"):
        B.workspace_size(d, 17, False)
    assert B.workspace_size(d, 2048, True) > B.workspace_size(d, 512, True)


# ------------------------------------------------------------ layout reader
def _read_chunk_codes(lane_words, bits, mx=False):
    """32 codes of one lane's chunk, from the pair arrangement in include/moe.h
    and the kernel header: pair p holds codes 2p (low half) and 2p+1 (high half);
    MXFP4 pair p is byte p (code 2p in its low nibble)."""
    q = np.zeros(32, np.int64)
    w = [int(v) for v in lane_words]
    for p in range(16):
        for hi in (0, 1):
            i = 2 * p + hi
            if mx:
                q[i] = (w[p // 4] >> (8 * (p % 4) + 4 * hi)) & 0xF
            elif bits == 4:
                q[i] = (w[p // 4] >> (16 * hi + 4 * (p % 4))) & 0xF
            elif bits == 2:
                q[i] = (w[p // 8] >> (16 * hi + 2 * (p % 8))) & 3
            elif bits == 5:
                if p < 15:
                    q[i] = (w[p // 3] >> (16 * hi + 5 * (p % 3))) & 31
                else:
                    q[i] = sum(((w[b] >> (31 if hi else 15)) & 1) << b for b in range(5))
            elif bits == 6:
                if p < 12:
                    q[i] = (w[p // 2] >> (16 * hi + 6 * (p % 2))) & 63
                else:
                    m = p - 12
                    q[i] = ((w[m] >> (16 * hi + 12)) & 15) | (((w[4 + m // 2] >> (16 * hi + 12 + 2 * (m % 2))) & 3) << 4)
            elif bits == 8:
                q[i] = (w[p // 2] >> (16 * hi + 8 * (p % 2))) & 0xFF
            else:
                if p < 15:
                    q[i] = (w[p // 5] >> (16 * hi + 3 * (p % 5))) & 7
                else:
                    q[i] = sum(((w[b] >> (31 if hi else 15)) & 1) << b for b in range(3))
    return q


def _read_matrix(buf, codes_off, scales_off, bits, group, affine, O_rows, K, rowmap, mx=False):
    cb = 4 * bits
    nch, nkb, gpb = K // 32, K // 256, 256 // group
    scb = 4 if affine else 1 if mx else 2
    q = np.zeros((O_rows, K), np.int64)
    s = np.zeros((O_rows, K // group), np.uint16)
    b = np.zeros((O_rows, K // group), np.uint16)
    for t in range(O_rows // 64):
        for lane in range(64):
            row = rowmap(t, lane)
            for c in range(nch):
                blk = codes_off + (t * nch + c) * 64 * cb
                if bits == 8:
                    raw = np.concatenate([buf[blk + lane * 16: blk + lane * 16 + 16],
                                          buf[blk + 1024 + lane * 16: blk + 1024 + lane * 16 + 16]])
                else:
                    raw = buf[blk + lane * cb: blk + lane * cb + cb]
                q[row, 32 * c: 32 * c + 32] = _read_chunk_codes(raw.view("<u4"), bits, mx)
            for kb in range(nkb):
                sb = scales_off + ((t * nkb + kb) * 64 + lane) * gpb * scb
                ent = buf[sb: sb + gpb * scb].view("<u4" if affine else "<u1" if mx else "<u2")
                for gi in range(gpb):
                    g = kb * gpb + gi
                    if affine:
                        s[row, g] = ent[gi] & 0xFFFF
                        b[row, g] = ent[gi] >> 16
                    else:
                        s[row, g] = ent[gi]
    return q, s, b


@pytest.mark.parametrize("base", [0, 2, 4, "q2", "q5", "q6", "mx"])
def test_packed_layout_decodes_to_canonical(base):
    _lib()
    if base in ("q2", "q5", "q6", "mx"):     # routed and shared experts of that format
        f = {"q2": Q2G64, "q5": Q5G64, "q6": Q6G64, "mx": MX4G32}[base]
        src = replace(synth.CONFIGS[0], routed=f, shared=f)
        cfg_id = 210 + f.bits + (10 if base == "mx" else 0)
    else:
        src, cfg_id = synth.CONFIGS[base], 200 + base
    spec = synth.make_tiny_config(src, cfg_id=cfg_id, hidden=512,
                                  n_experts=64, top_k=4, inter=256, shared_inter=256)
    Lh = synth.make_layer(spec, 0)
    buf, lc = B.pack_layer_host(_desc(spec), to_abi.tensors(Lh))
    H, I = spec.hidden, spec.inter
    f = spec.routed
    aff, mx = f.mode == O.AFFINE, f.mode == O.MXFP4
    for e in (0, 37, 63):
        blk = lc.experts_off + e * lc.expert_stride
        q, s, b = _read_matrix(buf, blk + lc.gu.codes, blk + lc.gu.scales, f.bits, f.group, aff,
                               2 * I, H, lambda t, l: 64 * t + l, mx)
        # tile t, lane l < 32 -> gate row 32t+l ; lane >= 32 -> up row 32t+l-32
        perm = np.array([32 * (r // 64) + (r % 64) % 32 + (I if r % 64 >= 32 else 0)
                         for r in range(2 * I)])
        canon_q = np.concatenate([O.unpack_codes(Lh.gate.codes[e], f.bits, H),
                                  O.unpack_codes(Lh.up.codes[e], f.bits, H)])
        assert np.array_equal(q, canon_q[perm])
        canon_s = np.concatenate([Lh.gate.scales[e], Lh.up.scales[e]])
        assert np.array_equal(s, canon_s[perm])
        if aff:
            assert np.array_equal(b, np.concatenate([Lh.gate.biases[e], Lh.up.biases[e]])[perm])
        q, s, b = _read_matrix(buf, blk + lc.dn.codes, blk + lc.dn.scales, f.bits, f.group, aff,
                               H, I, lambda t, l: 64 * t + l, mx)
        assert np.array_equal(q, O.unpack_codes(Lh.down.codes[e], f.bits, I))
        assert np.array_equal(s, Lh.down.scales[e])
    fr = spec.router
    q, s, b = _read_matrix(buf, lc.router_off, lc.router_scale_off, fr.bits, fr.group,
                           fr.mode == O.AFFINE, spec.n_experts, H, lambda t, l: 64 * t + l)
    assert np.array_equal(q, O.unpack_codes(Lh.router.codes, fr.bits, H))


def test_packing_is_deterministic():
    _lib()
    spec = synth.make_tiny_config(synth.CONFIGS[2], cfg_id=210, hidden=512, n_experts=64,
                                  top_k=4, inter=256, shared_inter=256)
    Lh = synth.make_layer(spec, 0)
    a, _ = B.pack_layer_host(_desc(spec), to_abi.tensors(Lh))
    b, _ = B.pack_layer_host(_desc(spec), to_abi.tensors(Lh))
    assert np.array_equal(a, b)


def test_null_source_refused():
    _lib()
    spec = synth.make_tiny_config(synth.CONFIGS[0], cfg_id=211, hidden=512, n_experts=64,
                                  top_k=4, inter=256, shared_inter=256)
    Lh = synth.make_layer(spec, 0)
    t = to_abi.tensors(Lh)
    t["down"] = (t["down"][0], None, t["down"][2])
    with pytest.raises(B.MoeError, match="down"):
        B.pack_layer_host(_desc(spec), t)


@pytest.mark.parametrize("patch,flag", [(None, 1), (104, 1), (140, 1), (255, 1), (103, 0), (141, 0), (0, 0)])
def test_mxfp4_fp16_flag(patch, flag):
    """The packer marks an MXFP4 layer MOE_LAYER_MX_FP16 exactly when every
    block exponent of its experts lies in 104..140 or is 255 (one exponent of
    the shared down projection is patched)."""
    _lib()
    spec = synth.make_tiny_config(replace(synth.CONFIGS[0], routed=MX4G32, shared=MX4G32), cfg_id=230,
                                  hidden=512, n_experts=64, top_k=4, inter=256, shared_inter=256)
    Lh = synth.make_layer(spec, 0)
    if patch is not None:
        Lh.sh_down.scales[17, 2] = patch
    _, lc = B.pack_layer_host(_desc(spec), to_abi.tensors(Lh))
    assert lc.flags == flag


def test_fp16_flag_clear_without_mxfp4():
    _lib()
    spec = synth.make_tiny_config(synth.CONFIGS[0], cfg_id=231, hidden=512, n_experts=64, top_k=4,
                                  inter=256, shared_inter=256)
    _, lc = B.pack_layer_host(_desc(spec), to_abi.tensors(synth.make_layer(spec, 0)))
    assert lc.flags == 0

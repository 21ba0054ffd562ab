"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the FP64 oracle on the same seeded inputs.

Pass criteria (the method's contract):
  * expert ids: the same set per row, except on near-tie rows, where the
    oracle's k-th and (k+1)-th logits are within 1e-5 (counted and
    reported); the order inside a row may differ only between picks whose
    oracle logits are within 1e-5 of each other. Where the GPU's ids differ
    from the oracle's in any way, y, p and sigma are compared with the
    oracle run on the GPU's ids;
  * y per row: max|y - y_ref| <= 2e-3 * max|y_ref|;
  * per projection class the worst-column and aggregate errors are reported.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

import oracle.moe_oracle as O
import synth
from synth import to_abi

TOL_Y = 2e-3
NEAR_TIE = 1e-5


def torch_mod():
    import torch
    return torch


def binding():
    import quantized_routed_expert_fp32_amd as qr
    return qr.binding


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build_layer(spec, layer=0):
    B = binding()
    Lh = synth.make_layer(spec, layer)
    dev = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec)), to_abi.tensors(Lh))
    return Lh, dev


def to_dev_x(xb):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()


def run_gpu(dev, Lh, xb, grouped=False, taps=True, stream=None):
    torch = torch_mod()
    B = binding()
    spec = Lh.spec
    R, E, k, H = xb.shape[0], spec.n_experts, spec.top_k, spec.hidden
    Imax = max(spec.inter, spec.shared_inter)
    x = to_dev_x(xb)
    bias = torch.from_numpy(Lh.logit_bias).cuda() if Lh.logit_bias is not None else None
    tp = None
    if taps:
        f = dict(device="cuda", dtype=torch.float32)
        tp = dict(logits=torch.full((R, E + 1), float("nan"), **f),
                  gu=torch.full((R, k + 1, 2, Imax), float("nan"), **f),
                  h=torch.full((R, k + 1, Imax), float("nan"), **f),
                  e=torch.full((R, k + 1, H), float("nan"), **f))
    ids, p, sg = B.route(dev, x, bias, taps=tp, stream=stream)
    y = B.experts(dev, x, ids, p, sg, grouped, taps=tp, stream=stream)
    torch.cuda.synchronize()
    out = dict(ids=ids.cpu().numpy(), p=p.cpu().numpy(), sg=sg.cpu().numpy(), y=y.cpu().numpy())
    if taps:
        for kk, v in tp.items():
            out[kk] = v.cpu().numpy()
    return out


def assert_rows_bits_equal(a, b, what, keys=("ids", "p", "sg", "y")):
    """Asserts that two forms' outputs are bit-identical row by row."""
    for key in keys:
        u, v = a[key], b[key]
        if u.dtype == np.float32:
            u, v = u.view(np.uint32), v.view(np.uint32)
        bad = np.where(~np.all(u.reshape(len(u), -1) == v.reshape(len(v), -1), axis=1))[0]
        assert bad.size == 0, f"{what}: {key} differs on rows {bad[:8]}"


def near_tie_rows(routing, k):
    """Rows whose oracle k-th and (k+1)-th logits are within NEAR_TIE: the
    only rows whose pick set may differ from the oracle's."""
    with np.errstate(invalid="ignore"):
        return np.isfinite(routing.gap) & (routing.gap < NEAR_TIE)


def check_ids(routing, gids, k, name=""):
    """Asserts the id rule; returns (same, near, counts): `same` marks rows
    whose ids equal the oracle's slot for slot."""
    ref = routing.ids
    near = near_tie_rows(routing, k)
    same = np.all(gids == ref, axis=1)
    same_set = np.all(np.sort(gids, axis=1) == np.sort(ref, axis=1), axis=1)
    bad_set = ~same_set & ~near
    assert not bad_set.any(), f"{name}: pick sets differ on rows {np.where(bad_set)[0][:10]} " \
                              f"(gaps {routing.gap[bad_set][:5]})"
    # same set, other order: each moved pick's oracle logit within NEAR_TIE
    # of the logit the oracle has in that slot
    reorder = same_set & ~same
    for r in np.where(reorder)[0]:
        lg = routing.logits[r]
        for j in np.where(gids[r] != ref[r])[0]:
            d = abs(lg[gids[r, j]] - lg[ref[r, j]])
            assert d < NEAR_TIE, f"{name}: row {r} slot {j} order differs with logit gap {d:.3e}"
    counts = dict(near_tie_rows=int(near.sum()), set_differs_on_ties=int((~same_set).sum()),
                  order_differs_within_ties=int(reorder.sum()))
    return same, near, counts


def check_parity(Lh, xb, g, dense=None, name="", tol_y=TOL_Y, strict_y=None, report=True,
                 form="per_row"):
    """Asserts the contract; returns the per-class error report.
    form: the oracle's evaluation form ("expert_major" for large chunks)."""
    spec = Lh.spec
    k = spec.top_k
    dense = dense or O.DenseExperts(Lh)
    ref = O.moe_forward(Lh, xb, dense, form=form)
    same, near, counts = check_ids(ref.routing, g["ids"], k, name)
    forced = ref
    if (~same).any():
        forced = O.moe_forward(Lh, xb, dense, ids=g["ids"], form=form)
    ref_y = np.where(same[:, None], ref.y, forced.y)
    finite = np.all(np.isfinite(ref_y), axis=1)
    err = O.row_error(g["y"][finite], ref_y[finite]) if finite.any() else np.zeros(0)
    worst = float(err.max()) if err.size else 0.0
    rep = dict(name=name, rows=int(xb.shape[0]), **counts, worst_row_err=worst)
    # routing weights, gate, logits
    rp = np.where(same[:, None], ref.routing.p, forced.routing.p)
    with np.errstate(invalid="ignore"):
        rep["p_max_rel"] = float(np.nanmax(np.abs(g["p"] - rp) / np.maximum(np.abs(rp), 1e-30)))
        rep["sigma_max_abs"] = float(np.nanmax(np.abs(g["sg"] - ref.routing.sigma)))
    if "logits" in g:
        lg = np.concatenate([ref.routing.logits, ref.routing.gate_logit[:, None]], axis=1)
        rep["logits"] = O.class_errors(g["logits"][finite], lg[finite])
    if "gu" in g:
        rows = finite
        I, Is = spec.inter, spec.shared_inter
        fg, fu, fh, fe = (np.where(same[:, None, None], a, b) for a, b in
                          ((ref.g, forced.g), (ref.u, forced.u), (ref.h, forced.h), (ref.e, forced.e)))
        if rows.any():
            rep["gate"] = O.class_errors(g["gu"][rows, :k, 0, :I], fg[rows, :k, :I])
            rep["up"] = O.class_errors(g["gu"][rows, :k, 1, :I], fu[rows, :k, :I])
            rep["h"] = O.class_errors(g["h"][rows, :k, :I], fh[rows, :k, :I])
            rep["down"] = O.class_errors(g["e"][rows, :k, :], fe[rows, :k, :])
            rep["shared_h"] = O.class_errors(g["h"][rows, k, :Is], fh[rows, k, :Is])
            rep["shared_down"] = O.class_errors(g["e"][rows, k, :], fe[rows, k, :])
    rep["y"] = O.class_errors(g["y"][finite], ref_y[finite])
    if report:
        log("PARITY " + json.dumps(rep))
        path = os.environ.get("MOE_PARITY_LOG")
        if path:
            with open(path, "a") as f:
                f.write(json.dumps(rep) + "\n")
    assert worst <= tol_y, f"{name}: worst row error {worst:.3e} > {tol_y}"
    if strict_y is not None:
        assert worst <= strict_y, f"{name}: worst row error {worst:.3e} > {strict_y}"
    # NaN-ness agrees
    assert np.array_equal(np.isnan(g["y"]).any(axis=1), ~finite)
    return rep, ref

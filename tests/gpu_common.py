"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the FP64 oracle on the same seeded inputs.

Pass criteria (the method's contract):
  * expert ids equal, in pick order, except on near-tie rows: rows where two
    of the oracle's top k+1 sorted logits are within 1e-5 (counted and
    reported; their y is compared with the oracle run on the GPU's ids);
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


def near_tie_rows(routing, k):
    srt = -np.sort(-np.where(np.isnan(routing.logits), np.inf, routing.logits), axis=1)
    top = srt[:, : k + 1]
    with np.errstate(invalid="ignore"):
        gaps = np.abs(np.diff(top, axis=1))
    return np.any(gaps < NEAR_TIE, axis=1) & np.all(np.isfinite(top), axis=1)


def check_parity(Lh, xb, g, dense=None, name="", tol_y=TOL_Y, strict_y=None, report=True):
    """Asserts the contract; returns the per-class error report."""
    spec = Lh.spec
    k = spec.top_k
    dense = dense or O.DenseExperts(Lh)
    ref = O.moe_forward(Lh, xb, dense)
    near = near_tie_rows(ref.routing, k)
    same = np.all(g["ids"] == ref.routing.ids, axis=1)
    bad = ~same & ~near
    assert not bad.any(), f"{name}: ids differ on non-tie rows {np.where(bad)[0][:10]}"
    forced = ref
    if (~same).any():
        forced = O.moe_forward(Lh, xb, dense, ids=g["ids"])
    ref_y = np.where(same[:, None], ref.y, forced.y)
    finite = np.all(np.isfinite(ref_y), axis=1)
    err = O.row_error(g["y"][finite], ref_y[finite]) if finite.any() else np.zeros(0)
    worst = float(err.max()) if err.size else 0.0
    rep = dict(name=name, rows=int(xb.shape[0]), near_tie_rows=int(near.sum()),
               id_mismatch_on_ties=int((~same).sum()), worst_row_err=worst)
    # routing weights, gate, logits
    rp = np.where(same[:, None], ref.routing.p, forced.routing.p)
    with np.errstate(invalid="ignore"):
        rep["p_max_rel"] = float(np.nanmax(np.abs(g["p"] - rp) / np.maximum(np.abs(rp), 1e-30)))
        rep["sigma_max_abs"] = float(np.nanmax(np.abs(g["sg"] - ref.routing.sigma)))
    if "logits" in g:
        lg = np.concatenate([ref.routing.logits, ref.routing.gate_logit[:, None]], axis=1)
        rep["logits"] = O.class_errors(g["logits"][finite], lg[finite])
    if "gu" in g:
        rows = same & finite
        I, Is = spec.inter, spec.shared_inter
        if rows.any():
            rep["gate"] = O.class_errors(g["gu"][rows, :k, 0, :I], ref.g[rows, :k, :I])
            rep["up"] = O.class_errors(g["gu"][rows, :k, 1, :I], ref.u[rows, :k, :I])
            rep["h"] = O.class_errors(g["h"][rows, :k, :I], ref.h[rows, :k, :I])
            rep["down"] = O.class_errors(g["e"][rows, :k, :], ref.e[rows, :k, :])
            rep["shared_h"] = O.class_errors(g["h"][rows, k, :Is], ref.h[rows, k, :Is])
            rep["shared_down"] = O.class_errors(g["e"][rows, k, :], ref.e[rows, k, :])
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

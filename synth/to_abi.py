"""Plain-data view of a synth.Layer for the C ABI (formats as tuples, arrays as-is)."""
from __future__ import annotations


def fmt_tuple(f):
    return (f.bits, f.group, f.mode, f.scale_dtype)


def desc_args(spec):
    """Arguments of binding.layer_desc for a ConfigSpec."""
    return (spec.hidden, spec.n_experts, spec.top_k, spec.inter, spec.shared_inter, spec.act,
            fmt_tuple(spec.router), fmt_tuple(spec.gate_row), fmt_tuple(spec.routed),
            fmt_tuple(spec.shared))


def tensors(layer):
    """name -> (codes, scales, biases) in the canonical layout."""
    out = {}
    for n in ("router", "gate_row", "gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        t = getattr(layer, n)
        out[n] = (t.codes, t.scales, t.biases)
    return out

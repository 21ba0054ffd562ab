"""GPU test of moe_forward_windows_noalloc (the entry point that allocates
nothing: its workspace is a fixed device array inside the library).

Through the C ABI it must give the same bits as moe_forward_windows with a
caller's workspace, on two calls in a row (the second with fewer rows, so it
runs on the array as the first call left it; a 4-bit affine and an MXFP4
layer), and refuse a layer whose
windows need more than the array holds, before anything is enqueued.
"""
import ctypes as C
from dataclasses import replace

import numpy as np
import pytest

import synth
from synth import to_abi
from synth.gen import MX4G32

from gpu_common import binding, log, to_dev_x, torch_mod

pytestmark = pytest.mark.gpu


def _bits(t):
    a = t.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


SPECS = [synth.CONFIGS[1],
         replace(synth.CONFIGS[1], cfg_id=380, name="decode-mxfp4-experts", routed=MX4G32, shared=MX4G32)]


@pytest.mark.parametrize("spec", SPECS, ids=["q4g64", "mxfp4"])
def test_noalloc_equals_workspace_form_on_two_calls(spec):
    B = binding()
    torch = torch_mod()
    Lh = synth.make_layer(spec, 2)
    dev = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec)), to_abi.tensors(Lh))
    for n, rows in enumerate((27, 5)):
        log(f"case noalloc call {n}: rows={rows}")
        x = to_dev_x(synth.make_x(spec, 2, rows, rep=40 + n))
        got = B.forward_windows_noalloc(dev, x)
        want = B.forward_windows(dev, x, ws=B.new_workspace(dev, min(rows, 16), False))
        torch.cuda.synchronize()
        for name, u, v in zip(("ids", "p", "shared_gate", "y"), got, want):
            assert np.array_equal(_bits(u), _bits(v)), f"call {n}: {name} differs"
        assert np.all(np.isfinite(got[3].cpu().numpy()))


def test_noalloc_refuses_layers_above_its_array():
    """hidden 1024, 64 experts, top-8, intermediate 2048: a 16-row window
    needs 2 x 589,824 bytes of fp16 h parts, above the 512 KiB array."""
    B = binding()
    L = B.lib()
    q4 = (4, 64, 0, 0)
    desc = B.layer_desc(1024, 64, 8, 2048, 2048, 0, q4, q4, q4, q4)
    need = B.workspace_size(desc, 16, False)
    assert need > 512 * 1024
    layer = B.LayerC()
    layer.d = desc                       # refused on the size check, before the layer is read
    torch = torch_mod()
    x = torch.zeros((16, 1024), dtype=torch.int16, device="cuda")
    out = torch.zeros((16, 8), dtype=torch.int32, device="cuda")
    st = L.moe_forward_windows_noalloc(C.byref(layer), C.c_void_p(x.data_ptr()), 16, None,
                                       C.c_void_p(out.data_ptr()), C.c_void_p(out.data_ptr()),
                                       C.c_void_p(out.data_ptr()), C.c_void_p(out.data_ptr()), None)
    assert st == -4, st
    msg = L.moe_last_error().decode()
    assert "524288" in msg and str(need) in msg, msg

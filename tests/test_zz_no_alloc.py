"""The no-allocation decode entry point (the library's own per-device
workspace) against the workspace-taking one, through the C ABI: identical
outputs and routing, on two calls in a row, the second with fewer rows."""

import numpy as np
import pytest
import torch

from mxfp4_moe_decode_amd import binding, synth
from tests import helpers

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,rows", [("tiny", (4, 1)), ("decode16", (16, 5))])
def test_noalloc_decode_equals_workspace_decode(name, rows):
    cfg = synth.workload(name)
    gl = helpers.gpu_layer(cfg)
    ws = binding.decode_workspace(gl)
    lib = binding.load()
    for i, T in enumerate(rows):
        x = _dev(synth.activations(cfg, T=T, index=40 + i))
        r = _dev(synth.activations(cfg, T=T, index=50 + i))
        print(f"[noalloc] {name} call {i} T={T}", flush=True)
        y_ref, ids_ref, w_ref = binding.fused_moe_mxfp4_decode(gl, x, residual=r, workspace=ws, return_routing=True)
        y = torch.empty_like(x)
        ids = torch.empty(T, cfg["k"], dtype=torch.int32, device="cuda")
        w = torch.empty(T, cfg["k"], dtype=torch.float32, device="cuda")
        st = lib.fused_moe_mxfp4_decode_noalloc(gl.c, binding._ptr(x), T, binding._ptr(r), binding._ptr(y),
                                                binding._ptr(ids), binding._ptr(w), binding._stream())
        assert st == 0, st
        torch.cuda.synchronize()
        assert np.array_equal(_host(y), _host(y_ref))
        assert np.array_equal(ids.cpu().numpy(), ids_ref.cpu().numpy())
        assert np.array_equal(w.cpu().numpy(), w_ref.cpu().numpy())
        assert not np.any((_host(y) & 0x7f80) == 0x7f80)


def test_noalloc_rejects_invalid_rows():
    cfg = synth.workload("tiny")
    gl = helpers.gpu_layer(cfg)
    x = _dev(synth.activations(cfg, T=17))
    y = torch.empty_like(x)
    st = binding.load().fused_moe_mxfp4_decode_noalloc(gl.c, binding._ptr(x), 17, None, binding._ptr(y), None, None,
                                                       binding._stream())
    assert st == -2

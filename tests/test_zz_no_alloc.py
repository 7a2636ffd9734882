"""gdr_chunk_fwd_static -- the chunkwise forward with the library's static
scratch instead of a caller workspace (no device allocation) -- called
through the C ABI and checked against gdr_chunk_fwd on the same inputs: two
calls in a row on one GPU, the second on a smaller problem, each bit-identical
to the workspace call (so within any parity bar)."""
import ctypes

import numpy as np
import pytest
import torch

from channel_wise_gated_amd import gdr
from channel_wise_gated_amd.inputs import WORKLOADS, make_inputs_device

pytestmark = pytest.mark.gpu
TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def _rel(a, b):
    a, b = a.double().cpu().numpy(), b.double().cpu().numpy()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _static_call(x, chunk):
    """gdr_chunk_fwd_static through ctypes; outputs allocated beforehand."""
    lib = gdr.load()
    B, H, T, dk = x["q"].shape
    desc = gdr.make_desc(B, H, T, dk, dk, chunk, gdr._dtype_code(x["q"]), gdr.GDR_F32)
    o = torch.full((B, H, T, dk), float("nan"), device="cuda")
    sT = torch.full((B, H, dk, dk), float("nan"), device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    rc = lib.gdr_chunk_fwd_static(ctypes.byref(desc), p(x["q"]), p(x["k"]), p(x["v"]), p(x["log_alpha"]),
                                  p(x["b"]), p(x["w"]), p(x["gamma"]), p(x["z"]), p(x["S0"]), p(o), p(sT), stream)
    assert rc == gdr.GDR_OK, gdr.gdr_status_string(rc)
    torch.cuda.synchronize()
    return o, sT


@pytest.mark.parametrize("first,second", [
    # the long-context shape at 8192 tokens (more chunks than the static
    # scratch holds at once: several segments), then a small ragged batch
    (("stress", dict(T=8192), 128), ("gdn2", dict(B=2, H=3, T=333), 64)),
])
def test_static_forward_matches_the_workspace_forward(first, second):
    for name, sizes, chunk in (first, second):
        wl = WORKLOADS[name].with_sizes(**sizes)
        print(f"static forward: {name} {sizes} chunk {chunk}", flush=True)
        x = make_inputs_device(wl, "cuda", seed=77)
        o_ref, s_ref = gdr.gdr_chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                         gamma=x["gamma"], z=x["z"], S0=x["S0"], chunk=chunk)
        torch.cuda.synchronize()
        o, sT = _static_call(x, chunk)
        tol = TOL[x["q"].dtype]
        assert _rel(o, o_ref) <= tol and _rel(sT, s_ref) <= tol
        assert torch.equal(o, o_ref) and torch.equal(sT, s_ref)

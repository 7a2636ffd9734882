"""The Python binding rejects malformed tensor arguments before anything is
launched: a wrong shape, dtype, layout or device raises ValueError.  These run
on the CPU: shapes and dtypes are checked before the device, so CPU tensors of
the wrong shape fail on the shape, and well-formed CPU tensors fail on the
device (a host pointer is never handed to a kernel)."""
import os

import pytest
import torch

from channel_wise_gated_amd import gdr

pytestmark = pytest.mark.skipif(not os.path.exists(gdr.LIB_PATH), reason="libgdr.so not built")

B, H, T, D = 2, 3, 70, 64
bf, f32 = torch.bfloat16, torch.float32


def good():
    r = lambda *s, dt=bf: torch.zeros(*s, dtype=dt)
    return dict(q=r(B, H, T, D), k=r(B, H, T, D), v=r(B, H, T, D), log_alpha=r(B, H, T, D, dt=f32),
                b=r(B, H, T, D), w=r(B, H, T, D), gamma=r(H, D, dt=f32), z=r(B, H, T, D),
                S0=r(B, H, D, D, dt=f32))


def fwd(x, **kw):
    return gdr.gdr_chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], gamma=x["gamma"],
                             z=x["z"], S0=x["S0"], **kw)


BAD_FWD = {
    "k shape": dict(k=torch.zeros(B, H, T, D - 1, dtype=bf)),
    "v dtype": dict(v=torch.zeros(B, H, T, D, dtype=f32)),
    "b dtype (fp32 b with bf16 q)": dict(b=torch.zeros(B, H, T, D, dtype=f32)),
    "w rank": dict(w=torch.zeros(B, H, dtype=bf)),
    "log_alpha bf16": dict(log_alpha=torch.zeros(B, H, T, D, dtype=bf)),
    "log_alpha short": dict(log_alpha=torch.zeros(B, H, T - 1, D, dtype=f32)),
    "per-token b short": dict(b=torch.zeros(B, H, T - 1, dtype=bf)),
    "gamma shape": dict(gamma=torch.zeros(H + 1, D, dtype=f32)),
    "z dtype": dict(z=torch.zeros(B, H, T, D, dtype=f32)),
    "S0 short": dict(S0=torch.zeros(B, H, D, D - 8, dtype=f32)),
    "S0 bf16": dict(S0=torch.zeros(B, H, D, D, dtype=bf)),
    "q strided": dict(q=torch.zeros(B, H, D, T, dtype=bf).transpose(2, 3)),
    "q fp16": dict(q=torch.zeros(B, H, T, D, dtype=torch.float16)),
}


@pytest.mark.parametrize("case", sorted(BAD_FWD))
def test_forward_rejects_malformed_inputs(case):
    x = good()
    x.update(BAD_FWD[case])
    with pytest.raises(ValueError) as e:
        fwd(x)
    assert "GPU device" not in str(e.value)   # caught by the argument's own check


@pytest.mark.parametrize("out", ["o shape", "o dtype", "S_T shape", "workspace dtype", "workspace small"])
def test_forward_rejects_malformed_outputs(out):
    kw, msg = {"o shape": (dict(o=torch.zeros(B, H, T - 1, D)), "shape"),
               "o dtype": (dict(o=torch.zeros(B, H, T, D, dtype=bf)), "dtype"),
               "S_T shape": (dict(S_T=torch.zeros(B, H, D, D + 1)), "shape"),
               "workspace dtype": (dict(workspace=torch.zeros(1 << 20, dtype=f32)), "uint8"),
               "workspace small": (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "needed")}[out]
    with pytest.raises(ValueError, match=msg):
        fwd(good(), **kw)


def test_well_formed_host_tensors_fail_on_the_device():
    with pytest.raises(ValueError, match="GPU device"):
        fwd(good())


def test_gated_rejects_malformed_gate_and_outputs():
    x = good()
    call = lambda **kw: gdr.gdr_chunk_fwd_gated(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                                kw.pop("g", torch.zeros(B, H, T, D, dtype=bf)), **kw)
    with pytest.raises(ValueError):
        call(g=torch.zeros(B, H, T, D, dtype=f32))
    with pytest.raises(ValueError):
        call(norm_weight=torch.zeros(H, D + 1))
    with pytest.raises(ValueError):
        call(y=torch.zeros(B, H, T, D))          # head-major instead of token-major
    with pytest.raises(ValueError):
        call(o=torch.zeros(B, H, T, D, dtype=bf))


def test_backward_rejects_malformed_inputs():
    x = good()
    dO = torch.zeros(B, H, T, D)
    call = lambda **kw: gdr.gdr_chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                          kw.pop("dO", dO), gamma=x["gamma"], z=x["z"], S0=x["S0"], **kw)
    with pytest.raises(ValueError):
        call(dO=torch.zeros(B, H, T, D + 1))
    with pytest.raises(ValueError):
        call(dO=torch.zeros(B, H, T, D, dtype=torch.float16))
    with pytest.raises(ValueError):
        call(dS_T=torch.zeros(B, H, D, D, dtype=bf))
    with pytest.raises(ValueError, match="GPU device"):
        call()


def test_backward_rejects_a_host_or_strided_cu_seqlens():
    x = {k: (v[:1] if v.dim() == 4 else v) for k, v in good().items()}
    x["S0"] = torch.zeros(2, H, D, D)
    dO = torch.zeros(1, H, T, D)
    call = lambda cu: gdr.gdr_chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO,
                                        gamma=x["gamma"], z=x["z"], S0=x["S0"], cu_seqlens=cu)
    with pytest.raises(ValueError, match="contiguous"):
        call(torch.tensor([0, 0, 30, 0, 70], dtype=torch.int32)[::2])
    with pytest.raises(ValueError):
        call(torch.tensor([0, 30, 70], dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU device"):
        call(torch.tensor([0, 30, 70], dtype=torch.int32))   # a host tensor never reaches a kernel


def test_varlen_forward_rejects_malformed_inputs():
    x = {k: (v[:1] if v.dim() == 4 else v) for k, v in good().items()}
    cu = torch.tensor([0, 30, 70], dtype=torch.int32)
    call = lambda **kw: gdr.gdr_chunk_fwd_varlen(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                                 kw.pop("cu", cu), gamma=x["gamma"], **kw)
    with pytest.raises(ValueError):
        call(S0=torch.zeros(3, H, D, D))          # two sequences, three states
    with pytest.raises(ValueError):
        call(cu=torch.tensor([0, 70], dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU device"):
        call()


def test_decode_rejects_malformed_inputs():
    r = lambda *s, dt=bf: torch.zeros(*s, dtype=dt)
    S = r(B, H, D, D, dt=f32)
    args = dict(q=r(B, H, D), k=r(B, H, D), v=r(B, H, D), log_alpha=r(B, H, D, dt=f32), b=r(B, H, D),
                w=r(B, H, D))
    call = lambda S, **kw: gdr.gdr_decode_step(S, **{**args, **kw})
    with pytest.raises(ValueError):
        call(r(B, H, D, D))                        # bf16 state
    with pytest.raises(ValueError):
        call(S[:, :, :-1])                         # short state
    with pytest.raises(ValueError):
        call(S, log_alpha=r(B, H, D))              # bf16 log-decay
    with pytest.raises(ValueError):
        call(S, b=r(B, H, D, dt=f32))              # fp32 gate with bf16 inputs
    with pytest.raises(ValueError):
        call(S, o=r(B, H, D + 1, dt=f32))
    with pytest.raises(ValueError, match="GPU device"):
        call(S)


def test_output_gate_backward_and_projection_reject_malformed_inputs():
    o = torch.zeros(B, H, T, D)
    g = torch.zeros(B, H, T, D, dtype=bf)
    with pytest.raises(ValueError):
        gdr.gdr_output_gate_bwd(o, g, torch.zeros(B, H, T, D, dtype=bf))   # dy head-major
    with pytest.raises(ValueError):
        gdr.gdr_output_gate_bwd(o.to(bf), g, torch.zeros(B, T, H, D, dtype=bf))
    ranks = (32, 32, 32, 32, 32)
    x = torch.zeros(1, 8, 64, dtype=bf)
    with pytest.raises(ValueError):
        gdr.gdr_gate_proj(x, torch.zeros(160, 32, dtype=bf), torch.zeros(5 * H * D * 32, dtype=bf), None, ranks, H, D)
    with pytest.raises(ValueError):
        gdr.gdr_gate_proj(x, torch.zeros(160, 64, dtype=bf), torch.zeros(5 * H * D * 32 - 8, dtype=bf), None, ranks,
                          H, D)

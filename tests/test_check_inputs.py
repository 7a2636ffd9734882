"""The opt-in precondition check (gdr_check_inputs): per input tensor, the
count of elements that are NaN or +-inf, and for log alpha also > 0 or < -30.
The expected counts are the plain definition evaluated with numpy on the
host copies of the same tensors (no part of the recurrence is involved).
The host-side tests run without a GPU: validation returns before any launch,
and the binding rejects host tensors."""
import ctypes
import os

import numpy as np
import pytest
import torch

from channel_wise_gated_amd import gdr

pytestmark = pytest.mark.skipif(not os.path.exists(gdr.LIB_PATH), reason="libgdr.so not built")

DEV = "cuda"


def _raw(desc, **over):
    """gdr_check_inputs through ctypes with fake (never dereferenced) device
    addresses; only validation outcomes are asserted."""
    p = dict(q=16, k=32, v=48, la=64, b=80, w=96, gamma=None, z=None, counts=128)
    p.update(over)
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    d = None if desc is None else ctypes.byref(desc)
    return gdr.load().gdr_check_inputs(d, c(p["q"]), c(p["k"]), c(p["v"]), c(p["la"]), c(p["b"]), c(p["w"]),
                                       c(p["gamma"]), c(p["z"]), c(p["counts"]), None)


def test_check_rejects_before_launch():
    d = gdr.make_desc(B=2, H=3, T=100, dk=64, dv=64)
    assert _raw(None) == gdr.GDR_ERR_INVALID_ARG
    assert _raw(d, counts=None) == gdr.GDR_ERR_INVALID_ARG
    assert _raw(d, counts=132) == gdr.GDR_ERR_INVALID_ARG          # counters not 8-byte aligned
    assert _raw(d, q=None) == gdr.GDR_ERR_INVALID_ARG
    assert _raw(d, k=40) == gdr.GDR_ERR_INVALID_ARG                # misaligned input
    assert _raw(d, la=None) == gdr.GDR_ERR_INVALID_ARG             # per-channel alpha needs a pointer
    assert _raw(d, z=24) == gdr.GDR_ERR_INVALID_ARG
    assert _raw(gdr.make_desc(B=0, H=3, T=100, dk=64, dv=64), gamma=40) == gdr.GDR_ERR_INVALID_ARG
    assert _raw(gdr.make_desc(B=2, H=3, T=100, dk=80, dv=80)) == gdr.GDR_ERR_UNSUPPORTED
    assert _raw(gdr.make_desc(B=2, H=3, T=100, dk=64, dv=64, alpha_mode=gdr.ZEROS)) == gdr.GDR_ERR_INVALID_ARG


def test_check_binding_rejects_host_and_malformed_tensors():
    B, H, T, D = 1, 2, 40, 64
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)
    args = (z(B, H, T, D), z(B, H, T, D), z(B, H, T, D), z(B, H, T, D, dt=torch.float32), z(B, H, T, D),
            z(B, H, T, D))
    with pytest.raises(ValueError, match="GPU device"):
        gdr.gdr_check_inputs(*args)
    with pytest.raises(ValueError):
        gdr.gdr_check_inputs(*args, counts=torch.zeros(8, dtype=torch.int32))
    with pytest.raises(ValueError):
        gdr.gdr_check_inputs(args[0], args[1], args[2], z(B, H, T, D), args[4], args[5])  # bf16 log alpha


def _bad(x, log_alpha=False):
    a = x.float().cpu().numpy()
    bad = ~np.isfinite(a)
    if log_alpha:
        with np.errstate(invalid="ignore"):
            bad |= (a > 0) | (a < -30)
    return int(bad.sum())


def _plant(t, n, values, gen):
    """Write `values` (cycled) at n distinct random positions of t."""
    flat = t.view(-1)
    idx = torch.randperm(flat.numel(), generator=gen)[:n]
    vals = torch.tensor([values[i % len(values)] for i in range(n)], dtype=torch.float32).to(t.dtype)
    flat[idx.to(flat.device)] = vals.to(flat.device)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("gates", ["channel", "token"])
def test_check_counts_planted_violations(dtype, gates):
    """Counts match the definition on ragged sizes (T = 77: per-token gates
    end in a partial 16-byte group), for both input dtypes and gate shapes;
    the boundary values 0, -0 and -30 of log alpha are valid."""
    gen = torch.Generator().manual_seed(5)
    B, H, T, D = 2, 3, 77, 64
    rn = lambda *s, dt=dtype: torch.randn(*s, generator=gen).to(dt).to(DEV)
    q, k, v, z = rn(B, H, T, D), rn(B, H, T, D), rn(B, H, T, D), rn(B, H, T, D)
    gs = (B, H, T, D) if gates == "channel" else (B, H, T)
    la = (-torch.rand(*gs, generator=gen) * 5).to(DEV)
    b, w = rn(*gs), rn(*gs)
    gamma = rn(H, D, dt=torch.float32)
    inf, nan = float("inf"), float("nan")
    _plant(q, 5, [nan], gen)
    _plant(k, 3, [inf, -inf], gen)
    _plant(v, 2, [-inf], gen)
    _plant(la, 9, [0.5, -31.0, nan, inf, -inf, 0.0, -0.0, -30.0, 1e-30], gen)
    _plant(b, 2, [nan], gen)
    _plant(w, 1, [inf], gen)
    _plant(z, 3, [nan, -inf], gen)
    _plant(gamma, 1, [inf], gen)
    counts = gdr.gdr_check_inputs(q, k, v, la, b, w, gamma=gamma, z=z)
    torch.cuda.synchronize()
    want = [_bad(q), _bad(k), _bad(v), _bad(la, True), _bad(b), _bad(w), _bad(z), _bad(gamma)]
    assert want[3] == 6  # 0.5, -31, nan, inf, -inf, 1e-30 (0, -0 and -30 are valid)
    assert counts.cpu().tolist() == want, dict(zip(gdr.CHECK_NAMES, zip(counts.cpu().tolist(), want)))


@pytest.mark.gpu
def test_check_counts_zero_on_clean_inputs_and_unread_gates():
    """A clean batch counts nothing; gates in a constant mode, a missing z or
    gamma, are not read (their counters stay 0), and the counters are
    cleared on every call (a counts tensor is reused)."""
    from channel_wise_gated_amd.inputs import WORKLOADS, make_inputs_device
    x = make_inputs_device(WORKLOADS["gdn2"], DEV, seed=3)
    counts = torch.full((8,), 77, dtype=torch.int64, device=DEV)
    gdr.gdr_check_inputs(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], gamma=x["gamma"], z=x["z"],
                         counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8
    q = x["q"].clone()
    q.view(-1)[123] = float("nan")
    gdr.gdr_check_inputs(q, x["k"], x["v"], 0, 1, 1, counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [1, 0, 0, 0, 0, 0, 0, 0]

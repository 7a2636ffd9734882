"""Seeded generator properties and the oracle regression fixture."""
import os

import numpy as np
import torch

from channel_wise_gated_amd.inputs import WORKLOADS, key_participation_ratio, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "oracle_tiny_regression.txt")


def test_generator_is_seeded_and_in_range():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=128)
    a = make_inputs(wl)
    b = make_inputs(wl)
    for key in ("q", "k", "v", "log_alpha", "b", "w", "z", "gamma", "S0"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.bfloat16 and a["log_alpha"].dtype == torch.float32
    assert float(a["log_alpha"].max()) <= 0.0
    assert 0.0 < float(a["b"].min()) and float(a["b"].max()) <= 2.0
    assert 0.0 < float(a["w"].min()) and float(a["w"].max()) <= 1.0
    # a different step gives different tokens, the static gain stays
    c = make_inputs(wl, step=1)
    assert not torch.equal(a["q"], c["q"]) and torch.equal(a["gamma"], c["gamma"])


def test_kda_gates_are_per_token():
    wl = WORKLOADS["kda"].with_sizes(B=1, H=2, T=64)
    x = make_inputs(wl)
    assert x["b"].shape == (1, 2, 64) and x["b"] is x["w"]
    assert x["gamma"] is None and x["z"] is None and x["S0"] is None


def test_stress_decay_rows_and_sparse_keys(oracle_mod):
    wl = WORKLOADS["stress"].with_sizes(T=256, H=2)
    x = make_inputs(wl)
    one_minus = -np.expm1(x["log_alpha"].double().numpy())
    slow = one_minus < 1.5e-3
    # a fixed half of the channels of every head is slow at every token
    assert np.all(slow.sum(-1) == 64)
    assert np.all(slow == slow[:, :, :1, :])
    assert one_minus[slow].min() >= 1e-4 * 0.99 and one_minus[~slow].max() <= 0.5
    kk = x["k"].double().numpy()[0, 0]
    kn = np.stack([oracle_mod.prepass(kk[t], kk[t])[1] for t in range(kk.shape[0])])
    pr = key_participation_ratio(kn)
    assert 3.0 < pr < 20.0, pr   # keys concentrate on a few channels


def test_oracle_regression_fixture(oracle_mod):
    from tests.golden.make_golden import compute
    o, sT = compute()
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#"):
                continue
            kind, idx, val = line.split()
            val = float(val)
            if kind == "o_norm":
                got = np.linalg.norm(o)
            elif kind == "S_T_norm":
                got = np.linalg.norm(sT)
            else:
                ix = tuple(int(i) for i in idx.split(","))
                got = (o if kind == "o" else sT)[ix]
            assert abs(got - val) <= 1e-12 * max(1.0, abs(val)), (kind, idx, got, val)

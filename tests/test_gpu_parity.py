"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (element-wise relative L2 over the whole tensor, outputs and final states
both compared): <= 2e-3 for bf16 inputs, <= 1e-5 for fp32 inputs.  Small cases
run the oracle on everything; the workloads at their full sizes run the GPU on
everything, in the launch configuration the benchmark times, and the oracle on
sampled (batch, head) streams.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from channel_wise_gated_amd import gdr
from channel_wise_gated_amd.inputs import WORKLOADS, make_inputs, make_inputs_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tol_for(x):
    return TOL_BF16 if x["q"].dtype == torch.bfloat16 else TOL_F32


def dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def gpu_chunk(x, chunk, **kw):
    d = dev(x)
    o, sT = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                              gamma=d["gamma"], z=d["z"], S0=d["S0"], chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), sT.cpu().numpy()


def oracle_run(x, **kw):
    return oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                          gamma=x["gamma"], z=x["z"], S0=x["S0"], **kw)


def sample_streams(x, pairs):
    """Inputs of the chosen (b, h) streams as a [1, n, ...] problem."""
    out = {}
    for key, val in x.items():
        if not isinstance(val, torch.Tensor):
            out[key] = val
        elif key == "gamma":
            out[key] = torch.stack([val[h] for _, h in pairs])
        else:
            out[key] = torch.stack([val[b, h] for b, h in pairs])[None]
    return out


def check(name, got, ref, tol):
    e = rel(got, ref)
    print(f"{name}: rel L2 {e:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(got)), name
    assert e <= tol, (name, e)
    return e


# ----------------------------------------------------------------------------
# chunkwise forward, small sizes: oracle on everything
# ----------------------------------------------------------------------------

def test_chunk_tiny_fp32_config():
    wl = WORKLOADS["tiny"]
    x = make_inputs(wl)
    o, sT = gpu_chunk(x, wl.chunk)
    ro, rs = oracle_run(x)
    check("tiny o", o, ro, TOL_F32)
    check("tiny S_T", sT, rs, TOL_F32)


@pytest.mark.parametrize("name,chunk,T", [
    ("kda", 64, 512), ("gdn2", 64, 512), ("gdn2", 128, 512), ("stress", 64, 1024),
    ("stress", 128, 1024), ("tiny", 64, 192)])
def test_chunk_small_cases(name, chunk, T):
    wl = WORKLOADS[name].with_sizes(B=2 if name != "tiny" else 1, H=3, T=T)
    x = make_inputs(wl)
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    check(f"{name} C{chunk} o", o, ro, tol_for(x))
    check(f"{name} C{chunk} S_T", sT, rs, tol_for(x))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,chunk", [(64, 64), (64, 128), (128, 64)])
def test_chunk_dims_and_dtypes(dtype, d, chunk):
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=256, dk=d, dv=d, dtype=dtype)
    x = make_inputs(wl)
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    check(f"{dtype} d{d} C{chunk} o", o, ro, tol_for(x))
    check(f"{dtype} d{d} C{chunk} S_T", sT, rs, tol_for(x))


# ----------------------------------------------------------------------------
# ragged sequence lengths: T not a multiple of the chunk (short last chunk)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,chunk,T", [
    ("gdn2", 64, 1), ("gdn2", 64, 37), ("gdn2", 128, 100), ("gdn2", 128, 129),
    ("kda", 64, 203), ("stress", 128, 333), ("tiny", 64, 70)])
def test_chunk_ragged_tail(name, chunk, T):
    wl = WORKLOADS[name].with_sizes(B=2, H=2, T=T)
    x = make_inputs(wl)
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    check(f"{name} T{T} C{chunk} o", o, ro, tol_for(x))
    check(f"{name} T{T} C{chunk} S_T", sT, rs, tol_for(x))


def test_ragged_tail_leaves_neighbours_untouched():
    """The padding rows of a short last chunk are never stored: o is written
    exactly over [B,H,T] (a guard region around it keeps its fill value)."""
    wl = WORKLOADS["gdn2"].with_sizes(B=2, H=2, T=77)
    x = dev(make_inputs(wl))
    B, H, T, dv = 2, 2, 77, wl.dv
    big = torch.full((B * H * T * dv + 4096,), 12345.0, device=DEV)
    o = big[2048:2048 + B * H * T * dv].view(B, H, T, dv)
    call = gdr.ChunkCall(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["gamma"],
                         x["z"], x["S0"], chunk=64, o=o)
    call()
    torch.cuda.synchronize()
    assert bool((big[:2048] == 12345.0).all()) and bool((big[-2048:] == 12345.0).all())
    ro, _ = oracle_run({k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()})
    check("guarded o", o.cpu().numpy(), ro, TOL_BF16)


def test_prefill_then_decode_handoff():
    """A chunkwise prefill of a ragged length followed by decode steps from
    its final state equals the recurrence over the whole sequence."""
    wl = WORKLOADS["gdn2"].with_sizes(B=2, H=2, T=150)
    x = make_inputs(wl)
    Tp = 141
    pre = {k: (v[:, :, :Tp].contiguous() if isinstance(v, torch.Tensor) and k not in ("gamma", "S0")
               else v) for k, v in x.items()}
    o_pre, S = gpu_chunk(pre, 64)
    S = torch.from_numpy(S).to(DEV)
    outs = [o_pre]
    for tt in range(Tp, wl.T):
        xt = {k: (v[:, :, tt] if isinstance(v, torch.Tensor) and k not in ("gamma", "S0") else v)
              for k, v in x.items()}
        outs.append(gpu_decode(S, xt).float().cpu().numpy()[:, :, None])
    torch.cuda.synchronize()
    ro, rs = oracle_run(x)
    check("prefill+decode o", np.concatenate(outs, axis=2), ro, TOL_BF16)
    check("prefill+decode S", S.cpu().numpy(), rs, TOL_BF16)


# ----------------------------------------------------------------------------
# packed batches of sequences of different lengths
# ----------------------------------------------------------------------------

def packed_inputs(name, lens, seed_shift=0, **sizes):
    """A [1,H,T,d] packed batch (T = sum of lens), per-sequence S0 [N,H,dk,dv]
    and the int32 offsets."""
    T = int(sum(lens))
    wl = WORKLOADS[name].with_sizes(B=1, H=2, T=T, seed=WORKLOADS[name].seed + seed_shift, **sizes)
    x = make_inputs(wl)
    N = len(lens)
    S0 = None
    if wl.s0:
        S0 = (0.02 * torch.from_numpy(np.random.default_rng(7 + seed_shift).standard_normal(
            (N, wl.H, wl.dk, wl.dv)))).float()
    x["S0"] = S0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, cu


def oracle_packed(x, cu):
    """The oracle run per sequence on the slices of the packed batch."""
    outs, states = [], []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        xs = {key: (val[:, :, a:b].contiguous() if isinstance(val, torch.Tensor) and key not in ("gamma", "S0")
                    else val) for key, val in x.items()}
        xs["S0"] = None if x["S0"] is None else x["S0"][n:n + 1]
        ro, rs = oracle_run(xs)
        outs.append(ro)
        states.append(rs[0])
    return np.concatenate(outs, axis=2), np.stack(states)


def gpu_packed(x, cu, chunk):
    d = dev(x)
    cut = torch.from_numpy(cu).to(DEV)
    o, sT = gdr.gdr_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cut,
                                     gamma=d["gamma"], z=d["z"], S0=d["S0"], chunk=chunk)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), sT.cpu().numpy()


@pytest.mark.parametrize("name,chunk", [("gdn2", 64), ("gdn2", 128), ("kda", 64), ("stress", 128),
                                        ("tiny", 64), ("gdn", 128)])
def test_varlen_mixed_lengths(name, chunk):
    lens = [0, 1, 63, 64, 65, 200, 0, 129, 17]
    x, cu = packed_inputs(name, lens)
    o, sT = gpu_packed(x, cu, chunk)
    ro, rs = oracle_packed(x, cu)
    check(f"varlen {name} C{chunk} o", o, ro, tol_for(x))
    if x["S0"] is None:
        rs = np.where(np.array(lens)[:, None, None, None] > 0, rs, 0.0)
    check(f"varlen {name} C{chunk} S_T", sT, rs, tol_for(x))
    empty = [n for n, L in enumerate(lens) if L == 0]
    s0 = np.zeros_like(sT) if x["S0"] is None else x["S0"].numpy()
    for n in empty:  # an empty sequence hands its S0 through unchanged
        assert np.array_equal(sT[n], s0[n])


def test_varlen_equal_lengths_match_the_batched_call():
    """N equal lengths packed give bit-identical results to a [N,H,T,d] call."""
    N, L = 3, 150
    wl = WORKLOADS["gdn2"].with_sizes(B=N, H=2, T=L)
    x = make_inputs(wl)
    ob, sb = gpu_chunk(x, 64)
    packed = {key: (val.permute(1, 0, 2, *range(3, val.dim())).reshape(1, wl.H, N * L, *val.shape[3:]).contiguous()
                    if isinstance(val, torch.Tensor) and key not in ("gamma", "S0") else val)
              for key, val in x.items()}
    cu = (np.arange(N + 1) * L).astype(np.int32)
    op, sp = gpu_packed(packed, cu, 64)
    op = op.reshape(wl.H, N, L, wl.dv).transpose(1, 0, 2, 3)
    assert np.array_equal(op, ob)
    assert np.array_equal(sp, sb)


@pytest.mark.parametrize("chunk", [128, 64])
def test_segmented_call_matches_the_phase_calls(chunk):
    """The whole call runs a long uniform batch in segments of chunks (here
    16 streams x 79 or 157 chunks: three or more segments), handing the fp32
    state from one segment to the next; the separate intra / scan calls do not
    segment.  Both must give bit-identical outputs and final states."""
    wl = WORKLOADS["stress"].with_sizes(T=10000)
    xd = make_inputs_device(wl, DEV, seed=21)
    args = (xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"], xd["gamma"], xd["z"], xd["S0"])
    whole = gdr.ChunkCall(*args, chunk=chunk)
    phased = gdr.ChunkCall(*args, chunk=chunk)
    o1, s1 = whole()
    phased.intra()
    o2, s2 = phased.scan()
    torch.cuda.synchronize()
    print(f"segmented C{chunk}: max |diff| o {float((o1 - o2).abs().max()):.3e} "
          f"S_T {float((s1 - s2).abs().max()):.3e}", flush=True)
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)


def test_long_call_d64_matches_the_phase_calls_and_the_oracle():
    """The long whole call at d = 64, chunk 64 (16 streams x 256 chunks, run
    in segments): bit-identical to the phase calls, and within the bar of the
    oracle on two sampled streams."""
    wl = WORKLOADS["stress"].with_sizes(T=16384, dk=64, dv=64)
    xd = make_inputs_device(wl, DEV, seed=23)
    args = (xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"], xd["gamma"], xd["z"], xd["S0"])
    whole = gdr.ChunkCall(*args, chunk=64)
    phased = gdr.ChunkCall(*args, chunk=64)
    o1, s1 = whole()
    phased.intra()
    o2, s2 = phased.scan()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    bi = torch.tensor([0, 0], device=DEV)
    hi = torch.tensor([3, 14], device=DEV)
    xs = {key: (None if val is None else (val[hi].cpu() if key == "gamma" else val[bi, hi][None].cpu()))
          for key, val in xd.items()}
    ro, rs = oracle_run(xs)
    check("long d64 o sampled", o1[bi, hi][None].float().cpu().numpy(), ro, TOL_BF16)
    check("long d64 S_T sampled", s1[bi, hi][None].cpu().numpy(), rs, TOL_BF16)


# ----------------------------------------------------------------------------
# the workloads at full size: GPU on everything, oracle on sampled streams
# ----------------------------------------------------------------------------

FULL_RAGGED = [("stress", 128, 32768 - 45, [(0, 2), (0, 13)])]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,chunk,T,pairs", FULL_RAGGED)
def test_chunk_full_size_ragged_sampled(name, chunk, T, pairs):
    """The long-context workload with a length that is not a multiple of the
    chunk, in the benchmark's launch configuration, sampled streams."""
    wl = WORKLOADS[name].with_sizes(T=T)
    print(f"full-size ragged {name} B{wl.B} H{wl.H} T{wl.T} C{chunk}", flush=True)
    xd = make_inputs_device(wl, DEV, seed=13)
    o, sT = gdr.gdr_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"],
                              gamma=xd["gamma"], z=xd["z"], S0=xd["S0"], chunk=chunk)
    torch.cuda.synchronize()
    bi = torch.tensor([b for b, _ in pairs], device=DEV)
    hi = torch.tensor([h for _, h in pairs], device=DEV)
    xs = {key: (None if val is None else (val[hi].cpu() if key == "gamma" else val[bi, hi][None].cpu()))
          for key, val in xd.items()}
    ro, rs = oracle_run(xs)
    check(f"{name} T{T} C{chunk} o sampled", o[bi, hi][None].float().cpu().numpy(), ro, TOL_BF16)
    check(f"{name} T{T} C{chunk} S_T sampled", sT[bi, hi][None].cpu().numpy(), rs, TOL_BF16)


FULL = [("kda", 64, [(0, 0), (1, 7), (2, 11), (3, 15)]),
        ("gdn2", 64, [(0, 3), (1, 12)]),
        ("stress", 64, [(0, 0), (0, 9)]),
        ("stress", 128, [(0, 5), (0, 14)]),
        ("gdn", 128, [(0, 1), (0, 10)])]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,chunk,pairs", FULL)
def test_chunk_full_size_sampled(name, chunk, pairs):
    """Full-size workload on the GPU (inputs drawn on the device with the same
    recipe), sampled (batch, head) streams through the oracle."""
    wl = WORKLOADS[name]
    print(f"full-size {name} B{wl.B} H{wl.H} T{wl.T} C{chunk}", flush=True)
    xd = make_inputs_device(wl, DEV, seed=11)
    o, sT = gdr.gdr_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"],
                              gamma=xd["gamma"], z=xd["z"], S0=xd["S0"], chunk=chunk)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(sT).all())
    bi = torch.tensor([b for b, _ in pairs], device=DEV)
    hi = torch.tensor([h for _, h in pairs], device=DEV)
    xs = {}
    for key, val in xd.items():
        if val is None:
            xs[key] = None
        elif key == "gamma":
            xs[key] = val[hi].cpu()
        else:
            xs[key] = val[bi, hi][None].cpu()
    ro, rs = oracle_run(xs)
    check(f"{name} C{chunk} o sampled", o[bi, hi][None].float().cpu().numpy(), ro, TOL_BF16)
    check(f"{name} C{chunk} S_T sampled", sT[bi, hi][None].cpu().numpy(), rs, TOL_BF16)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def decode_inputs(wl, step):
    x = make_inputs(wl, step=step)
    sq = {}
    for key in ("q", "k", "v", "log_alpha", "z"):
        sq[key] = None if x[key] is None else x[key][:, :, 0]
    for key in ("b", "w"):
        val = x[key]
        sq[key] = val[:, :, 0] if val.dim() == 4 else val[:, :, 0]
    sq["gamma"] = x["gamma"]
    sq["S0"] = x["S0"]
    return sq


def gpu_decode(S, x, **kw):
    d = dev(x)
    return gdr.gdr_decode_step(S, d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                               gamma=d["gamma"], z=d["z"], **kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gates", ["gdn2", "kda"])
def test_decode_small_many_steps(d, dtype, gates):
    wl = WORKLOADS["decode"].with_sizes(B=3, H=2, dk=d, dv=d, dtype=dtype, gates=gates)
    x0 = decode_inputs(wl, 0)
    S = x0["S0"].clone().to(DEV)
    Sref = x0["S0"].double().numpy()
    outs, refs = [], []
    for step in range(12):
        x = decode_inputs(wl, step)
        o = gpu_decode(S, x)
        ro, Sref = oracle.decode_step(Sref, x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                      gamma=x["gamma"], z=x["z"])
        outs.append(o.float().cpu().numpy())
        refs.append(ro)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    check(f"decode d{d} {dtype} {gates} o", np.stack(outs), np.stack(refs), tol)
    check(f"decode d{d} {dtype} {gates} S", S.cpu().numpy(), Sref, tol)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_scalar_decay(d):
    """Decode with one decay and one beta per token (Gated DeltaNet)."""
    wl = WORKLOADS["decode"].with_sizes(B=3, H=2, dk=d, dv=d, alpha="scalar", gates="kda")
    x0 = decode_inputs(wl, 0)
    assert x0["log_alpha"].dim() == 2
    S = x0["S0"].clone().to(DEV)
    Sref = x0["S0"].double().numpy()
    outs, refs = [], []
    for step in range(12):
        x = decode_inputs(wl, step)
        o = gpu_decode(S, x)
        ro, Sref = oracle.decode_step(Sref, x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                      gamma=x["gamma"], z=x["z"])
        outs.append(o.float().cpu().numpy())
        refs.append(ro)
    torch.cuda.synchronize()
    check(f"decode scalar decay d{d} o", np.stack(outs), np.stack(refs), TOL_BF16)
    check(f"decode scalar decay d{d} S", S.cpu().numpy(), Sref, TOL_BF16)


@pytest.mark.timeout(600)
def test_decode_full_config_1024_steps():
    """256 sequences x 16 heads, 1024 consecutive steps, one launch per step
    (inputs of all steps drawn on the device up front); the oracle follows 24
    sampled streams through all steps."""
    wl = WORKLOADS["decode"]
    pairs = [(b, h) for b in (0, 37, 101, 200, 255, 128) for h in (0, 5, 10, 15)]
    bi = torch.tensor([p[0] for p in pairs], device=DEV)
    hi = torch.tensor([p[1] for p in pairs], device=DEV)
    xd = make_inputs_device(wl, DEV, seed=5, steps=wl.steps)
    S = xd["S0"].clone()
    Sref = xd["S0"][bi, hi][None].double().cpu().numpy()
    gam = xd["gamma"][hi].cpu()
    host = {k: xd[k][:, bi, hi].cpu() for k in ("q", "k", "v", "log_alpha", "b", "w", "z")}
    outs = []
    checkpoints = {}
    for step in range(wl.steps):
        o = gdr.gdr_decode_step(S, xd["q"][step], xd["k"][step], xd["v"][step],
                                xd["log_alpha"][step], xd["b"][step], xd["w"][step],
                                gamma=xd["gamma"], z=xd["z"][step])
        outs.append(o[bi, hi])
        if step in (0, 511, wl.steps - 1):
            checkpoints[step] = S[bi, hi].clone()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(S).all())
    got = torch.stack(outs).float().cpu().numpy()
    num = den = 0.0
    for step in range(wl.steps):
        xs = {k: v[step][None] for k, v in host.items()}
        ro, Sref = oracle.decode_step(Sref, xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["b"],
                                      xs["w"], gamma=gam, z=xs["z"])
        num += float(np.sum((got[step] - ro[0]) ** 2))
        den += float(np.sum(ro[0] ** 2))
        if step in checkpoints:
            check(f"decode S after step {step + 1}", checkpoints[step].cpu().numpy(), Sref[0], TOL_BF16)
        if step % 256 == 0:
            print(f"decode oracle step {step}", flush=True)
    e = (num / den) ** 0.5
    print(f"decode 1024 steps o rel L2 {e:.3e}", flush=True)
    assert e <= TOL_BF16


def test_decode_equals_chunk():
    """Running the decode step T times equals one chunkwise call."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=128)
    x = make_inputs(wl)
    o_chunk, s_chunk = gpu_chunk(x, 64)
    S = x["S0"].clone().to(DEV)
    outs = []
    for t in range(wl.T):
        xt = {k: (v[:, :, t] if isinstance(v, torch.Tensor) and k not in ("gamma", "S0") else v)
              for k, v in x.items()}
        outs.append(gpu_decode(S, xt).float().cpu().numpy())
    torch.cuda.synchronize()
    o_dec = np.stack(outs, axis=2)
    ro, rs = oracle_run(x)
    check("decode-as-prefill o", o_dec, ro, TOL_BF16)
    check("chunk o", o_chunk, ro, TOL_BF16)
    check("decode-as-prefill S", S.cpu().numpy(), rs, TOL_BF16)
    check("decode vs chunk S", S.cpu().numpy(), s_chunk, 2 * TOL_BF16)


# ----------------------------------------------------------------------------
# edge cases and degenerate gates
# ----------------------------------------------------------------------------

def test_zero_length_sequence_copies_state():
    wl = WORKLOADS["gdn2"].with_sizes(B=2, H=3, T=64)
    x = dev(make_inputs(wl))
    q = x["q"][:, :, :0].contiguous()
    o, sT = gdr.gdr_chunk_fwd(q, q, q, x["log_alpha"][:, :, :0].contiguous(),
                              x["b"][:, :, :0].contiguous(), x["w"][:, :, :0].contiguous(),
                              gamma=x["gamma"], z=q, S0=x["S0"])
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(sT, x["S0"])
    _, sT0 = gdr.gdr_chunk_fwd(q, q, q, x["log_alpha"][:, :, :0].contiguous(),
                               x["b"][:, :, :0].contiguous(), x["w"][:, :, :0].contiguous())
    torch.cuda.synchronize()
    assert torch.count_nonzero(sT0).item() == 0


@pytest.mark.parametrize("chunk", [64, 128])
def test_alpha_zero_and_extreme_decay_runs(chunk):
    """log alpha = -30 (alpha ~ 0: memory cleared) at single tokens, and long
    runs of it that force the exact-exponential path of diagonal blocks."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=256)
    x = make_inputs(wl)
    la = x["log_alpha"].clone()
    la[:, 0, 37] = -30.0
    la[:, 1, 100:140] = -30.0      # a run wider than a 16-token block
    la[:, 1, 200:203, :64] = -30.0
    x["log_alpha"] = la
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    check(f"alpha->0 C{chunk} o", o, ro, TOL_BF16)
    check(f"alpha->0 C{chunk} S_T", sT, rs, TOL_BF16)


# ----------------------------------------------------------------------------
# the fused output gate: y = RMSNorm(o) * weight * sigmoid(g), token-major
# ----------------------------------------------------------------------------

def gated_case(wl, seed=3):
    x = make_inputs(wl)
    r = np.random.default_rng(seed)
    g = torch.from_numpy(r.standard_normal((wl.B, wl.H, wl.T, wl.dv))).to(x["v"].dtype)
    nw = torch.from_numpy(1.0 + 0.2 * r.standard_normal((wl.H, wl.dv))).float()
    return x, g, nw


@pytest.mark.parametrize("name,chunk,T,d", [("gdn2", 64, 256, 128), ("stress", 128, 300, 128),
                                            ("gdn2", 64, 77, 64), ("tiny", 64, 256, 64), ("gdn", 128, 129, 128)])
def test_gated_output(name, chunk, T, d):
    """The gated whole call against the oracle's recurrence followed by the
    oracle's output gate."""
    wl = WORKLOADS[name].with_sizes(B=2, H=2, T=T, dk=d, dv=d)
    x, g, nw = gated_case(wl)
    dd = dev(x)
    y, sT = gdr.gdr_chunk_fwd_gated(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["b"], dd["w"], g.to(DEV),
                                    gamma=dd["gamma"], z=dd["z"], S0=dd["S0"], norm_weight=nw.to(DEV),
                                    eps=1e-6, chunk=chunk)
    torch.cuda.synchronize()
    ro, rs = oracle_run(x)
    ry = oracle.output_gate(ro, g, norm_weight=nw, eps=1e-6)
    tol = tol_for(x)
    check(f"gated {name} C{chunk} T{T} d{d} y", y.cpu().numpy(), ry, tol)
    check(f"gated {name} C{chunk} T{T} d{d} S_T", sT.cpu().numpy(), rs, tol)


def test_gated_output_fp32_inputs_d128():
    """fp32 inputs at d = 128 (three bf16 planes per operand) through the
    gated whole call, against the oracle's recurrence and output gate."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=130, dtype="f32")
    x, g, nw = gated_case(wl, seed=5)
    dd = dev(x)
    y, sT = gdr.gdr_chunk_fwd_gated(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["b"], dd["w"], g.to(DEV),
                                    gamma=dd["gamma"], z=dd["z"], S0=dd["S0"], norm_weight=nw.to(DEV),
                                    eps=1e-6, chunk=64)
    torch.cuda.synchronize()
    ro, rs = oracle_run(x)
    ry = oracle.output_gate(ro, g, norm_weight=nw, eps=1e-6)
    check("gated f32 d128 y", y.cpu().numpy(), ry, TOL_F32)
    check("gated f32 d128 S_T", sT.cpu().numpy(), rs, TOL_F32)


def test_gated_output_bf16_and_segmented():
    """bf16 y against the oracle's y rounded to bf16; and at a length that runs
    in segments, the gated call equals the output gate applied (in fp64) to
    the ungated call's o, and its final state equals the ungated one."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=256)
    x, g, nw = gated_case(wl, seed=4)
    dd = dev(x)
    y, _ = gdr.gdr_chunk_fwd_gated(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["b"], dd["w"], g.to(DEV),
                                   gamma=dd["gamma"], z=dd["z"], S0=dd["S0"], norm_weight=nw.to(DEV),
                                   chunk=64, out_dtype=torch.bfloat16)
    ro, _ = oracle_run(x)
    ry = torch.from_numpy(oracle.output_gate(ro, g, norm_weight=nw)).to(torch.bfloat16).double().numpy()
    check("gated bf16 y (vs oracle rounded to bf16)", y.float().cpu().numpy(), ry, TOL_BF16)
    wl = WORKLOADS["stress"].with_sizes(T=10000)
    xd = make_inputs_device(wl, DEV, seed=31)
    gd = torch.randn((wl.B, wl.H, wl.T, wl.dv), device=DEV).to(torch.bfloat16)
    args = (xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"])
    o, s1 = gdr.gdr_chunk_fwd(*args, gamma=xd["gamma"], z=xd["z"], S0=xd["S0"], chunk=128)
    y, s2 = gdr.gdr_chunk_fwd_gated(*args, gd, gamma=xd["gamma"], z=xd["z"], S0=xd["S0"], chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    ry = oracle.output_gate(o.cpu(), gd.cpu(), eps=1e-6)
    check("gated segmented y vs gate(o)", y.cpu().numpy(), ry, 1e-5)


# ----------------------------------------------------------------------------
# scalar decay (one log alpha per token: Gated DeltaNet, DeltaNet) -- bf16
# inputs take the scalar-decay intra-chunk kernel
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("chunk,d,T,gates,gain", [
    (64, 128, 300, "kda", False), (128, 128, 300, "kda", False), (64, 64, 257, "gdn2", True),
    (128, 64, 129, "gdn2", True), (128, 128, 200, "gdn2", True), (64, 128, 64, "kda", True)])
def test_scalar_decay(chunk, d, T, gates, gain):
    """Per-token decay with per-token beta (b = w) or per-channel b, w, with
    and without the read-out gain, ragged lengths included."""
    wl = WORKLOADS["gdn"].with_sizes(B=2, H=2, T=T, dk=d, dv=d, gates=gates, gain=gain)
    x = make_inputs(wl)
    assert x["log_alpha"].dim() == 3
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    check(f"scalar decay C{chunk} d{d} T{T} {gates} o", o, ro, TOL_BF16)
    check(f"scalar decay C{chunk} d{d} T{T} {gates} S_T", sT, rs, TOL_BF16)


@pytest.mark.parametrize("chunk", [64, 128])
def test_scalar_decay_matches_the_per_channel_kernel(chunk):
    """The same decay given per token (scalar-decay kernel) and replicated over
    the channels (general kernel): both against the oracle, and against each
    other far inside the tolerance."""
    wl = WORKLOADS["gdn"].with_sizes(B=1, H=3, T=320)
    x = make_inputs(wl)
    o1, s1 = gpu_chunk(x, chunk)
    y = dict(x)
    y["log_alpha"] = x["log_alpha"][..., None].expand(*x["log_alpha"].shape, wl.dk).contiguous()
    o2, s2 = gpu_chunk(y, chunk)
    ro, rs = oracle_run(x)
    check(f"scalar kernel C{chunk} o", o1, ro, TOL_BF16)
    check(f"per-channel kernel C{chunk} o", o2, ro, TOL_BF16)
    check(f"scalar vs per-channel C{chunk} o", o1, o2, 1e-4)
    check(f"scalar vs per-channel C{chunk} S_T", s1, s2, 1e-4)


@pytest.mark.parametrize("chunk", [64, 128])
def test_scalar_decay_extreme_runs(chunk):
    """Per-token log alpha = -30 at single tokens and over runs wider than a
    block (the exact-exponential path of diagonal blocks), and alpha = 1."""
    wl = WORKLOADS["gdn"].with_sizes(B=1, H=2, T=256)
    x = make_inputs(wl)
    la = x["log_alpha"].clone()
    la[:, 0, 37] = -30.0
    la[:, 1, 100:140] = -30.0
    la[:, 0, 150:256] = 0.0
    x["log_alpha"] = la
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    check(f"scalar alpha->0 C{chunk} o", o, ro, TOL_BF16)
    check(f"scalar alpha->0 C{chunk} S_T", sT, rs, TOL_BF16)


def adversarial_inputs(wl, start, n, bval=1.99):
    """One key repeated over n tokens with erase strength bval near 2 and no
    decay there: the chunk's unit-lower-triangular system becomes badly
    conditioned (the regime the Muir notes' section 2.4 stability discussion
    probes adversarially)."""
    x = make_inputs(wl)
    k = x["k"].clone()
    k[:, :, start:start + n] = k[:, :, start:start + 1]
    b = x["b"].clone()
    b[:, :, start:start + n] = bval
    la = x["log_alpha"].clone()
    la[:, :, start:start + n] = 0.0
    x.update(k=k, b=b, log_alpha=la)
    return x


def chunk_system_cond(x, bi, hi, t0, C):
    """cond_2(I + L) of the chunk starting at token t0 (fp64, from the
    oracle's pre-pass and the decayed Gram of the chunk algebra)."""
    kn = np.stack([oracle.prepass(x["q"][bi, hi, t], x["k"][bi, hi, t])[1] for t in range(t0, t0 + C)])
    b = x["b"][bi, hi, t0:t0 + C].double().numpy()
    lam = np.cumsum(x["log_alpha"][bi, hi, t0:t0 + C].double().numpy(), axis=0)
    Tm = np.eye(C)
    for t in range(C):
        for s_ in range(t):
            Tm[t, s_] += np.sum(b[t] * kn[t] * np.exp(lam[t] - lam[s_]) * kn[s_])
    return float(np.linalg.cond(Tm))


@pytest.mark.parametrize("chunk,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32")])  # fp32 mode: C = 64
def test_ill_conditioned_chunk_system(chunk, dtype):
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=256, dtype=dtype)
    x = adversarial_inputs(wl, chunk, chunk)
    cond = chunk_system_cond(x, 0, 0, chunk, chunk)
    assert cond > 1e3, cond
    o, sT = gpu_chunk(x, chunk)
    ro, rs = oracle_run(x)
    print(f"cond(I+L) = {cond:.3e}", flush=True)
    # each mode's own bar, whatever the conditioning
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    check(f"ill-conditioned C{chunk} {dtype} o", o, ro, tol)
    check(f"ill-conditioned C{chunk} {dtype} S_T", sT, rs, tol)


def test_gate_modes_and_options():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=128)
    x = make_inputs(wl)
    cases = {
        "linear-attention (b=0, alpha=1, w=1)": dict(log_alpha=0, b=0, w=1),
        "per-token alpha and gates": dict(log_alpha=x["log_alpha"][..., 0].contiguous(),
                                          b=x["b"][..., 0].contiguous(), w=x["w"][..., 0].contiguous()),
        "DeltaNet (alpha=1, b=w=1)": dict(log_alpha=0, b=1, w=1),
    }
    for label, over in cases.items():
        y = dict(x)
        y.update(over)
        o, sT = gpu_chunk(y, 64)
        ro, rs = oracle_run(y)
        check(label + " o", o, ro, TOL_BF16)
        check(label + " S_T", sT, rs, TOL_BF16)
    # no pre-pass normalisation, a query scale and a bf16 output
    y = dict(x)
    kn = torch.nn.functional.normalize(x["k"].float(), dim=-1).to(torch.bfloat16)
    y["k"] = kn
    d = dev(y)
    o, sT = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                              gamma=d["gamma"], z=d["z"], S0=d["S0"], normalize_qk=False,
                              scale=0.125, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rs = oracle_run(y, normalize_qk=False, scale=0.125)
    # a bf16 o against the oracle's o rounded to bf16 (the rounding of the
    # stored output is not the path's error); the state stays fp32
    ro16 = torch.from_numpy(ro).to(torch.bfloat16).double().numpy()
    check("raw qk, scale, bf16 o (vs oracle rounded to bf16)", o.float().cpu().numpy(), ro16, TOL_BF16)
    check("raw qk, scale S_T", sT.cpu().numpy(), rs, TOL_BF16)


def test_zero_keys_and_state_aliasing():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=128)
    x = make_inputs(wl)
    k = x["k"].clone()
    k[:, :, 10] = 0.0          # SiLU(0) = 0: unit-norm floor gives a zero key
    k[:, :, 77:80] = 0.0
    x["k"] = k
    ro, rs = oracle_run(x)
    d = dev(x)
    S = d["S0"].clone()
    o, sT = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                              gamma=d["gamma"], z=d["z"], S0=S, S_T=S)   # S_T aliases S0
    torch.cuda.synchronize()
    assert sT.data_ptr() == S.data_ptr()
    check("zero keys o", o.cpu().numpy(), ro, TOL_BF16)
    check("zero keys, aliased S", S.cpu().numpy(), rs, TOL_BF16)


def test_nan_stays_in_its_stream_and_runs_are_deterministic():
    wl = WORKLOADS["gdn2"].with_sizes(B=2, H=3, T=256)
    x = make_inputs(wl)
    o1, s1 = gpu_chunk(x, 64)
    o2, s2 = gpu_chunk(x, 64)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    v = x["v"].clone()
    v[1, 2, 70, 5] = float("nan")
    x["v"] = v
    o3, s3 = gpu_chunk(x, 64)
    assert np.isnan(o3[1, 2]).any()
    mask = np.ones(o3.shape[:2], dtype=bool)
    mask[1, 2] = False
    assert np.array_equal(o3[mask], o1[mask]) and np.array_equal(s3[mask], s1[mask])


def test_whole_call_and_decode_replay_from_a_hip_graph():
    """The whole chunkwise call (long enough to run in segments) and a decode
    step captured in one HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager results bit for bit."""
    wl = WORKLOADS["stress"].with_sizes(T=10000)
    xd = make_inputs_device(wl, DEV, seed=23)
    call = gdr.ChunkCall(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"], xd["gamma"],
                         xd["z"], xd["S0"], chunk=128)
    dwl = WORKLOADS["decode"].with_sizes(B=4, H=2)
    xdec = dev(decode_inputs(dwl, 0))
    S_init = xdec["S0"].clone()
    S_graph = S_init.clone()
    o_eager, s_eager = [t.clone() for t in call()]
    S_e = S_init.clone()
    od_eager = gpu_decode(S_e, xdec).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
        gpu_decode(S_graph.clone(), xdec)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        o_g, s_g = call()
        od_g = gpu_decode(S_graph, xdec)
    for rep in range(3):
        call.o.zero_()
        S_graph.copy_(S_init)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_eager), rep
        assert torch.equal(s_g, s_eager), rep
        assert torch.equal(od_g, od_eager), rep
        assert torch.equal(S_graph, S_e), rep
        _ = (xd["q"].float() * 2).sum()  # eager work between replays
    print("graph replays match the eager results", flush=True)


# ----------------------------------------------------------------------------
# the five-gate low-rank projection (x -> log alpha, b, g, w, z)
# ----------------------------------------------------------------------------

def gate_weights(dm, H, d, ranks, seed, bias=True):
    r = np.random.default_rng(seed)
    R = sum(ranks)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    wd = bf(r.standard_normal((R, dm)) / np.sqrt(dm))
    wu = {n: bf(r.standard_normal((H * d, rk)) / np.sqrt(rk)) for n, rk in zip(gdr.GATE_ORDER, ranks)}
    bs = torch.from_numpy(0.5 * r.standard_normal((5, H * d))).float() if bias else None
    return wd, wu, bs


@pytest.mark.parametrize("B,T,dm,H,d,ranks,bias", [
    (2, 300, 256, 2, 128, (64, 64, 128, 128, 128), True),
    (1, 77, 512, 4, 64, (32, 64, 32, 96, 128), False),
    (1, 1, 64, 1, 128, (32, 32, 32, 32, 32), True)])
def test_gate_proj(B, T, dm, H, d, ranks, bias):
    r = np.random.default_rng(7)
    x = torch.from_numpy(r.standard_normal((B, T, dm))).to(torch.bfloat16)
    wd, wu, bs = gate_weights(dm, H, d, ranks, 8, bias)
    out = gdr.gdr_gate_proj(x.to(DEV), wd.to(DEV), {n: t.to(DEV) for n, t in wu.items()},
                            None if bs is None else bs.to(DEV), ranks, H, d)
    torch.cuda.synchronize()
    ref = oracle.gate_proj(x, wd, wu, np.zeros((5, H * d)) if bs is None else bs, ranks, H, d)
    for n in gdr.GATE_ORDER:
        got = out[n].float().cpu().numpy()
        want = ref[n] if n == "f" else torch.from_numpy(ref[n]).to(torch.bfloat16).double().numpy()
        check(f"gate proj B{B} T{T} dm{dm} H{H} d{d} {n}", got, want, TOL_BF16)


def test_gate_proj_skips_unwanted_gates_and_fp32_outputs():
    ranks = (64, 64, 128, 128, 128)
    r = np.random.default_rng(9)
    x = torch.from_numpy(r.standard_normal((1, 130, 256))).to(torch.bfloat16)
    wd, wu, bs = gate_weights(256, 2, 128, ranks, 10)
    out = gdr.gdr_gate_proj(x.to(DEV), wd.to(DEV), {n: t.to(DEV) for n, t in wu.items()}, bs.to(DEV), ranks,
                            2, 128, out_dtype=torch.float32, gates=("f", "w"))
    torch.cuda.synchronize()
    assert set(out) == {"f", "w"}
    ref = oracle.gate_proj(x, wd, wu, bs, ranks, 2, 128)
    check("gate proj fp32 f", out["f"].cpu().numpy(), ref["f"], TOL_F32 * 10)
    check("gate proj fp32 w", out["w"].cpu().numpy(), ref["w"], TOL_F32 * 10)


def test_layer_pipeline_projection_recurrence_output_gate():
    """x -> gate projection -> chunkwise recurrence -> gated output, against
    the oracle's three steps on the same inputs (the GPU gates, stored bf16,
    are what both recurrences consume)."""
    B, T, H, d = 1, 200, 2, 128
    dm, ranks = 256, (64, 64, 128, 128, 128)
    r = np.random.default_rng(11)
    x = torch.from_numpy(r.standard_normal((B, T, dm))).to(torch.bfloat16)
    wd, wu, bs = gate_weights(dm, H, d, ranks, 12)
    gates = gdr.gdr_gate_proj(x.to(DEV), wd.to(DEV), {n: t.to(DEV) for n, t in wu.items()}, bs.to(DEV),
                              ranks, H, d)
    wl = WORKLOADS["gdn2"].with_sizes(B=B, H=H, T=T)
    xin = make_inputs(wl)
    gamma = xin["gamma"]
    q, k, v = (xin[n].to(DEV) for n in ("q", "k", "v"))
    nw = torch.from_numpy(1.0 + 0.1 * r.standard_normal((H, d))).float()
    y, sT = gdr.gdr_chunk_fwd_gated(q, k, v, gates["f"], gates["b"], gates["w"], gates["g"], gamma=gamma.to(DEV),
                                    z=gates["q"], norm_weight=nw.to(DEV), chunk=64)
    torch.cuda.synchronize()
    gc = {n: t.cpu() for n, t in gates.items()}
    ro, rs = oracle.forward(xin["q"], xin["k"], xin["v"], gc["f"], gc["b"], gc["w"], gamma=gamma, z=gc["q"])
    ry = oracle.output_gate(ro, gc["g"], norm_weight=nw)
    check("layer pipeline y", y.cpu().numpy(), ry, TOL_BF16)
    check("layer pipeline S_T", sT.cpu().numpy(), rs, TOL_BF16)


# ----------------------------------------------------------------------------
# backward: every gradient against the oracle's reverse-mode backward
# ----------------------------------------------------------------------------

def bwd_compare(x, tag, seed=5, do_bf16=False, with_dst=True, tol=None, **kw):
    r = np.random.default_rng(seed)
    B, H, T, dk = x["q"].shape
    dv = x["v"].shape[-1]
    dO = torch.from_numpy(r.standard_normal((B, H, T, dv))).float()
    if do_bf16:
        dO = dO.to(torch.bfloat16)
    dST = torch.from_numpy(0.1 * r.standard_normal((B, H, dk, dv))).float() if with_dst else None
    d = dev(x)
    g = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO.to(DEV),
                          gamma=d["gamma"], z=d["z"], S0=d["S0"], dS_T=None if dST is None else dST.to(DEV), **kw)
    torch.cuda.synchronize()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO,
                          gamma=x["gamma"], z=x["z"], S0=x["S0"], dS_T=dST, **kw)
    tol = tol if tol is not None else tol_for(x)
    for key in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dgamma", "dz", "dS0"):
        if ref[key] is None:
            assert g[key] is None, key
            continue
        check(f"bwd {tag} {key}", g[key].cpu().numpy(), ref[key], tol)


@pytest.mark.parametrize("name,B,H,T,d", [
    ("gdn2", 1, 2, 200, 128), ("kda", 2, 2, 130, 128), ("tiny", 1, 1, 256, 64), ("gdn", 1, 2, 192, 128),
    ("stress", 1, 2, 150, 128), ("gdn2", 2, 1, 64, 64)])
def test_backward_small_cases(name, B, H, T, d):
    wl = WORKLOADS[name].with_sizes(B=B, H=H, T=T, dk=d, dv=d)
    bwd_compare(make_inputs(wl), f"{name} B{B} H{H} T{T} d{d}")


@pytest.mark.parametrize("chunk,dtype,d", [(64, "bf16", 128), (128, "bf16", 128), (64, "f32", 64)])
def test_forward_is_bit_reproducible(chunk, dtype, d):
    """Two calls on the same inputs give bit-identical o and S_T: no result
    depends on the order in which workgroups or waves finish."""
    x = make_inputs(WORKLOADS["gdn2"].with_sizes(B=2, H=2, T=700, dk=d, dv=d, dtype=dtype))
    print(f"forward reproducibility: C{chunk} {dtype} d{d}", flush=True)
    runs = [gpu_chunk(x, chunk) for _ in range(2)]
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("name,T,d,dtype,do_bf16,packed", [
    ("gdn2", 200, 128, "bf16", False, False), ("gdn2", 100, 64, "f32", False, False),
    ("kda", 130, 128, "bf16", True, False), ("gdn2", 0, 128, "bf16", False, True)])
def test_backward_workspace_contents_do_not_matter(name, T, d, dtype, do_bf16, packed):
    """The backward's workspace arrays share memory where their lifetimes do
    not overlap, so every value a kernel reads must have been written earlier
    in the same call: a workspace filled with NaN gives gradients bit-identical
    to a zero-filled one (which also needs every reduction in the backward to
    run in a fixed order)."""
    r = np.random.default_rng(29)
    if packed:
        x, cu = packed_inputs(name, [0, 65, 1, 130, 17], seed_shift=5)
        cuj = torch.from_numpy(cu).to(DEV)
        nseq = len(cu) - 1
    else:
        x, cuj, nseq = make_inputs(WORKLOADS[name].with_sizes(B=1, H=2, T=T, dk=d, dv=d, dtype=dtype)), None, None
    B, H, TT, dk = x["q"].shape
    dv = x["v"].shape[-1]
    dO = torch.from_numpy(r.standard_normal((B, H, TT, dv))).float()
    if do_bf16:
        dO = dO.to(torch.bfloat16)
    nS = nseq if packed else B
    dST = torch.from_numpy(0.1 * r.standard_normal((nS, H, dk, dv))).float().to(DEV)
    dd = dev(x)
    lib = gdr.load()
    amode, _ = gdr._log_alpha_arg(dd["log_alpha"], (B, H, TT, dk))
    bmode, _ = gdr._gate_arg(dd["b"], "b", (B, H, TT, dk), (dd["q"].dtype,))
    wmode, _ = gdr._gate_arg(dd["w"], "w", (B, H, TT, dv), (dd["q"].dtype,))
    desc = gdr.make_desc(B, H, TT, dk, dv, 64, gdr._dtype_code(dd["q"]),
                         gdr.GDR_BF16 if do_bf16 else gdr.GDR_F32, 1, 1.0, amode, bmode, wmode)
    n = ctypes.c_size_t(0)
    if packed:
        assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(desc), nseq, ctypes.byref(n)) == gdr.GDR_OK
    else:
        assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)) == gdr.GDR_OK
    print(f"workspace poisoning: {name} T{TT} d{d} {dtype} dO bf16 {do_bf16} packed {packed}, {n.value} B", flush=True)
    outs = []
    for fill in (0, 0xFF):  # all-ones bytes are NaN in fp32 and in bf16
        ws = torch.full((n.value,), fill, dtype=torch.uint8, device=DEV)
        g = gdr.gdr_chunk_bwd(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["b"], dd["w"], dO.to(DEV),
                              gamma=dd["gamma"], z=dd["z"], S0=dd["S0"], dS_T=dST, workspace=ws,
                              cu_seqlens=cuj)
        torch.cuda.synchronize()
        outs.append(g)
    for key, val in outs[0].items():
        if val is None:
            continue
        assert bool(torch.isfinite(val).all()), key
        assert torch.equal(val, outs[1][key]), key


def test_backward_fp32_inputs_and_bf16_upstream():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=100, dtype="f32")
    bwd_compare(make_inputs(wl), "f32 inputs")
    wl2 = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=100)
    bwd_compare(make_inputs(wl2), "bf16 dO", do_bf16=True)


def test_backward_options_and_edges():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=70)
    x = make_inputs(wl)
    bwd_compare(x, "no dS_T", with_dst=False)
    bwd_compare({**x, "S0": None, "gamma": None, "z": None}, "no S0, no gain")
    # without the pre-pass the keys must have unit norm for a bounded state
    y = dict(x)
    y["k"] = torch.nn.functional.normalize(x["k"].float(), dim=-1).to(x["k"].dtype)
    bwd_compare(y, "no normalisation, scale", normalize_qk=False, scale=0.5)
    bwd_compare(make_inputs(WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=1)), "T1")
    bwd_compare({**x, "log_alpha": 0.0, "w": 1.0}, "constant decay and write gates")
    bwd_compare({**x, "b": 0.0}, "no erase")


def test_backward_outputs_left_out_are_not_written_and_change_nothing():
    """Null gradient pointers: the rest is bit-identical to the full call."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=150)
    d = dev(make_inputs(wl))
    r = np.random.default_rng(9)
    dO = torch.from_numpy(r.standard_normal((1, 2, 150, 128))).float().to(DEV)
    dST = torch.from_numpy(0.1 * r.standard_normal((1, 2, 128, 128))).float().to(DEV)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO)
    kw = dict(gamma=d["gamma"], z=d["z"], S0=d["S0"], dS_T=dST)
    full = gdr.gdr_chunk_bwd(*args, **kw)
    for keep in (("dq", "dS0"), ("dlog_alpha", "dgamma"), ("dk", "dv", "db", "dw", "dz"), ()):
        part = gdr.gdr_chunk_bwd(*args, **kw, outputs=keep)
        torch.cuda.synchronize()
        for name in gdr.BWD_OUTPUTS:
            if name in keep:
                assert torch.equal(part[name], full[name]), (keep, name)
            else:
                assert part[name] is None


def test_backward_extreme_and_steep_decays():
    """log alpha = -30 at single tokens and over runs wider than a 16-token
    block (the pair-by-pair path of the Gram kernels), and a block whose decay
    range is just under that path's threshold (pivot factors near e^50)."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=256)
    x = make_inputs(wl)
    la = x["log_alpha"].clone()
    la[:, 0, 37] = -30.0
    la[:, 0, 160:176] = -3.3
    la[:, 1, 100:140] = -30.0
    la[:, 1, 200:203, :64] = -30.0
    x["log_alpha"] = la
    bwd_compare(x, "extreme decays")


def test_backward_empty_sequence_passes_the_state_gradient():
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=0)
    x = dev(make_inputs(wl))
    dST = torch.randn(1, 2, 128, 128, device=DEV)
    g = gdr.gdr_chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                          torch.empty(1, 2, 0, 128, device=DEV), gamma=x["gamma"], z=x["z"], S0=x["S0"], dS_T=dST)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dST)
    assert torch.count_nonzero(g["dgamma"]) == 0



@pytest.mark.timeout(600)
def test_backward_full_size_sampled():
    """The long-context shape (B1 H16 T32768 d128, bf16) on the GPU as one
    call; two sampled heads' gradients through the oracle."""
    wl = WORKLOADS["stress"]
    print(f"full-size backward B{wl.B} H{wl.H} T{wl.T}", flush=True)
    xd = make_inputs_device(wl, DEV, seed=11)
    g0 = torch.Generator(device=DEV).manual_seed(23)
    dO = torch.randn(wl.B, wl.H, wl.T, wl.dv, device=DEV, generator=g0)
    dST = 0.1 * torch.randn(wl.B, wl.H, wl.dk, wl.dv, device=DEV, generator=g0)
    g = gdr.gdr_chunk_bwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"], dO,
                          gamma=xd["gamma"], z=xd["z"], S0=xd["S0"], dS_T=dST)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dlog_alpha", "dz", "dS0"):
        assert bool(torch.isfinite(g[key]).all()), key
    for h in (3, 14):
        xs = {}
        for key, val in xd.items():
            if val is None:
                xs[key] = None
            elif key == "gamma":
                xs[key] = val[h:h + 1].cpu()
            else:
                xs[key] = val[:, h:h + 1].cpu()
        ref = oracle.backward(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["b"], xs["w"],
                              dO[:, h:h + 1].cpu(), gamma=xs["gamma"], z=xs["z"], S0=xs["S0"],
                              dS_T=dST[:, h:h + 1].cpu())
        for key in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dz", "dS0", "dgamma"):
            if ref[key] is None:
                continue
            got = g[key][h:h + 1] if key == "dgamma" else g[key][:, h:h + 1]
            check(f"bwd full T{wl.T} head {h} {key}", got.cpu().numpy(), ref[key], TOL_BF16)


@pytest.mark.timeout(900)
def test_long_sequences_forward_and_backward():
    """One sequence of half a million tokens (B1 H2 T524288, chunk 128): the
    whole forward on the GPU, one head's outputs and final state through the
    oracle; then the backward at T131072 the same way (64-bit offsets, chains
    of 4096 and 2048 chunks)."""
    wl = WORKLOADS["stress"].with_sizes(H=2, T=1 << 19)
    print(f"long forward T{wl.T}", flush=True)
    xd = make_inputs_device(wl, DEV, seed=31)
    o, sT = gdr.gdr_chunk_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"],
                              gamma=xd["gamma"], z=xd["z"], S0=xd["S0"], chunk=128)
    torch.cuda.synchronize()
    h = 1
    xs = {k: (None if v is None else (v[h:h + 1].cpu() if k == "gamma" else v[:, h:h + 1].cpu()))
          for k, v in xd.items()}
    ro, rs = oracle_run(xs)
    check(f"long T{wl.T} o", o[:, h:h + 1].cpu().numpy(), ro, TOL_BF16)
    check(f"long T{wl.T} S_T", sT[:, h:h + 1].cpu().numpy(), rs, TOL_BF16)
    del o, sT, xd, xs, ro, rs
    torch.cuda.empty_cache()
    wb = WORKLOADS["stress"].with_sizes(H=2, T=1 << 17)
    print(f"long backward T{wb.T}", flush=True)
    xd = make_inputs_device(wb, DEV, seed=37)
    gen = torch.Generator(device=DEV).manual_seed(41)
    dO = torch.randn(1, 2, wb.T, wb.dv, device=DEV, generator=gen)
    g = gdr.gdr_chunk_bwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["b"], xd["w"], dO,
                          gamma=xd["gamma"], z=xd["z"], S0=xd["S0"])
    torch.cuda.synchronize()
    xs = {k: (None if v is None else (v[h:h + 1].cpu() if k == "gamma" else v[:, h:h + 1].cpu()))
          for k, v in xd.items()}
    ref = oracle.backward(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["b"], xs["w"], dO[:, h:h + 1].cpu(),
                          gamma=xs["gamma"], z=xs["z"], S0=xs["S0"])
    for key in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dz", "dS0", "dgamma"):
        got = g[key][h:h + 1] if key == "dgamma" else g[key][:, h:h + 1]
        check(f"long bwd T{wb.T} {key}", got.cpu().numpy(), ref[key], TOL_BF16)


def test_backward_nan_stays_in_its_stream():
    """A NaN in one stream's keys poisons that stream's gradients only (and
    dgamma of its head); the other streams' gradients equal the clean run's
    bit for bit."""
    wl = WORKLOADS["gdn2"].with_sizes(B=2, H=2, T=100)
    x = make_inputs(wl)
    r = np.random.default_rng(13)
    dO = torch.from_numpy(r.standard_normal((2, 2, 100, 128))).float().to(DEV)
    d = dev(x)
    run = lambda k: gdr.gdr_chunk_bwd(d["q"], k, d["v"], d["log_alpha"], d["b"], d["w"], dO,
                                      gamma=d["gamma"], z=d["z"], S0=d["S0"])
    clean = run(d["k"])
    kbad = d["k"].clone()
    kbad[1, 0, 37, 5] = float("nan")
    bad = run(kbad)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dz", "dS0"):
        assert not bool(torch.isfinite(bad[key][1, 0]).all()), key
        for bi, hi in ((0, 0), (0, 1), (1, 1)):
            assert torch.equal(bad[key][bi, hi], clean[key][bi, hi]), (key, bi, hi)
    assert torch.equal(bad["dgamma"][1], clean["dgamma"][1])


@pytest.mark.parametrize("name", ["gdn2", "kda", "tiny", "gdn"])
def test_backward_varlen_mixed_lengths(name):
    """Packed batch backward (lengths 0, 1, 63, 64, 65, 200, 0, 129, 17): each
    sequence's gradients against the oracle's backward on its slice; dS0 per
    sequence; dgamma summed over the sequences."""
    lens = [0, 1, 63, 64, 65, 200, 0, 129, 17]
    x, cu = packed_inputs(name, lens, seed_shift=3)
    N, H, T = len(lens), x["q"].shape[1], x["q"].shape[2]
    dk, dv = x["q"].shape[-1], x["v"].shape[-1]
    r = np.random.default_rng(19)
    dO = torch.from_numpy(r.standard_normal((1, H, T, dv))).float()
    dST = torch.from_numpy(0.1 * r.standard_normal((N, H, dk, dv))).float()
    d = dev(x)
    g = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO.to(DEV),
                          gamma=d["gamma"], z=d["z"], S0=d["S0"], dS_T=dST.to(DEV),
                          cu_seqlens=torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    tol = tol_for(x)
    per_tok = {key: [] for key in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dz")}
    dS0, dgam = [], 0.0
    for n in range(N):
        a0, b0 = int(cu[n]), int(cu[n + 1])
        xs = {key: (val[:, :, a0:b0].contiguous() if isinstance(val, torch.Tensor) and key not in ("gamma", "S0")
                    else val) for key, val in x.items()}
        s0 = None if x["S0"] is None else x["S0"][n:n + 1]
        ref = oracle.backward(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["b"], xs["w"],
                              dO[:, :, a0:b0].contiguous(), gamma=xs["gamma"], z=xs["z"], S0=s0,
                              dS_T=dST[n:n + 1])
        for key in per_tok:
            if ref[key] is not None:
                per_tok[key].append(ref[key])
        dS0.append(ref["dS0"][0])
        if ref["dgamma"] is not None:
            dgam = dgam + ref["dgamma"]
    for key, parts in per_tok.items():
        if not parts:
            assert g[key] is None, key
            continue
        check(f"bwd varlen {name} {key}", g[key].cpu().numpy(), np.concatenate(parts, axis=2), tol)
    check(f"bwd varlen {name} dS0", g["dS0"].cpu().numpy(), np.stack(dS0), tol)
    if x["gamma"] is not None:
        check(f"bwd varlen {name} dgamma", g["dgamma"].cpu().numpy(), dgam, tol)


@pytest.mark.parametrize("d,gdt,ydt,weight", [(128, torch.bfloat16, torch.float32, True),
                                              (128, torch.float32, torch.bfloat16, False),
                                              (64, torch.bfloat16, torch.bfloat16, True)])
def test_output_gate_backward(d, gdt, ydt, weight):
    """The output gate's backward against the oracle's (ragged T, two batches)."""
    r = np.random.default_rng(71)
    B, H, T = 2, 3, 150
    o = torch.from_numpy(r.standard_normal((B, H, T, d))).float()
    g = torch.from_numpy(r.standard_normal((B, H, T, d))).to(gdt)
    dy = torch.from_numpy(r.standard_normal((B, T, H, d))).to(ydt)
    nw = torch.from_numpy(1.0 + 0.1 * r.standard_normal((H, d))).float() if weight else None
    got = gdr.gdr_output_gate_bwd(o.to(DEV), g.to(DEV), dy.to(DEV), None if nw is None else nw.to(DEV), eps=1e-5)
    torch.cuda.synchronize()
    do, dg, dw = oracle.output_gate_backward(o, g.float(), dy.float(), norm_weight=nw, eps=1e-5)
    check(f"out gate bwd d{d} d_o", got["d_o"].cpu().numpy(), do, TOL_F32)
    check(f"out gate bwd d{d} dg", got["dg"].cpu().numpy(), dg, TOL_F32)
    if weight:
        check(f"out gate bwd d{d} d_norm_weight", got["d_norm_weight"].cpu().numpy(), dw, TOL_F32)
    else:
        assert got["d_norm_weight"] is None


def test_gated_forward_keeps_o_and_layer_backward_chain():
    """The gated forward also writes o (bit-identical to the plain forward's);
    then the layer's backward: the output gate's backward on that o, and the
    recurrence's backward with its d_o, against the oracle's two steps."""
    wl = WORKLOADS["gdn2"].with_sizes(B=1, H=2, T=150)
    x = make_inputs(wl)
    r = np.random.default_rng(83)
    g = torch.from_numpy(r.standard_normal((1, 2, 150, 128))).to(torch.bfloat16)
    nw = torch.from_numpy(1.0 + 0.1 * r.standard_normal((2, 128))).float()
    dy = torch.from_numpy(r.standard_normal((1, 150, 2, 128))).float()
    d = dev(x)
    o_keep = torch.empty(1, 2, 150, 128, device=DEV)
    y, sT = gdr.gdr_chunk_fwd_gated(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], g.to(DEV),
                                    gamma=d["gamma"], z=d["z"], S0=d["S0"], norm_weight=nw.to(DEV), eps=1e-6,
                                    chunk=64, o=o_keep)
    o_plain, _ = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                                   gamma=d["gamma"], z=d["z"], S0=d["S0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o_keep, o_plain)
    og = gdr.gdr_output_gate_bwd(o_keep, g.to(DEV), dy.to(DEV), nw.to(DEV), eps=1e-6)
    gb = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], og["d_o"],
                           gamma=d["gamma"], z=d["z"], S0=d["S0"])
    torch.cuda.synchronize()
    ro, _ = oracle_run(x)
    do_ref, dg_ref, dw_ref = oracle.output_gate_backward(ro, g.float(), dy, norm_weight=nw, eps=1e-6)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], torch.from_numpy(do_ref),
                          gamma=x["gamma"], z=x["z"], S0=x["S0"])
    check("layer bwd dg", og["dg"].cpu().numpy(), dg_ref, TOL_BF16)
    check("layer bwd d_norm_weight", og["d_norm_weight"].cpu().numpy(), dw_ref, TOL_BF16)
    for key in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dz", "dgamma", "dS0"):
        check(f"layer bwd {key}", gb[key].cpu().numpy(), ref[key], TOL_BF16)


def test_backward_varlen_all_sequences_empty():
    """A packed batch whose sequences are all empty (T = 0): dS0 = dS_T per
    sequence, dgamma = 0, nothing else touched."""
    x, cu = packed_inputs("gdn2", [0, 0, 0])
    d = dev(x)
    dST = torch.randn(3, 2, 128, 128, device=DEV)
    g = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                          torch.empty(1, 2, 0, 128, device=DEV), gamma=d["gamma"], z=d["z"], S0=d["S0"],
                          dS_T=dST, cu_seqlens=torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dST)
    assert torch.count_nonzero(g["dgamma"]) == 0

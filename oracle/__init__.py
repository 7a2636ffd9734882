"""fp64 CPU oracle of the channel-wise gated delta rule -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never serves the product path and it
shares no code with the HIP kernels; the only thing both sides share is the
seeded input generator (``channel_wise_gated_amd.inputs``), which holds none of
the method's arithmetic.

The arithmetic lives in ``gdr_oracle.c`` (plain C, double precision, a token
loop per (batch, head) stream, forward and its reverse-mode backward).  This wrapper only broadcasts gate arguments to
full per-channel fp64 arrays and marshals pointers.  The method it follows is
stated in the C file's header: Muir reading notes (arXiv:2611.08376) section 2.1
for the GDN-2 update and the read-out gain; the "Kimi3 = GPT2 x 22580" blog,
section 3 "DeltaNet", for the SiLU + L2 pre-pass.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.gdr_oracle_forward.restype = ctypes.c_int
    lib.gdr_oracle_forward.argtypes = [
        ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        ctypes.c_double, ctypes.c_int, _dp, _dp, _dp, ctypes.c_int]
    lib.gdr_oracle_prepass.restype = None
    lib.gdr_oracle_prepass.argtypes = [
        ctypes.c_int, _dp, _dp, _dp, _dp, ctypes.c_double, ctypes.c_int, _dp, _dp]
    lib.gdr_oracle_backward.restype = ctypes.c_int
    lib.gdr_oracle_backward.argtypes = [
        ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        ctypes.c_double, ctypes.c_int, _dp, _dp, _dp,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.gdr_oracle_max_threads.restype = ctypes.c_int
    lib.gdr_oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _f64(x):
    """Exact upcast of a numpy array / torch tensor to a C-contiguous fp64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (any dtype, CPU)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _gate(g, shape, name):
    """Broadcast a gate argument to a full per-channel array of ``shape``.

    ``g`` may be a scalar (0 or 1 for the constant gate modes), a per-token
    array [B, H, T] (broadcast over channels) or a full [B, H, T, d] array.
    """
    if np.isscalar(g):
        return np.full(shape, float(g), dtype=np.float64)
    a = _f64(g)
    if a.shape == tuple(shape[:3]):
        a = a[..., None]
    if a.shape[:3] != tuple(shape[:3]) or a.shape[3] not in (1, shape[3]):
        raise ValueError(f"gate {name}: shape {a.shape} does not fit {shape}")
    return np.ascontiguousarray(np.broadcast_to(a, shape))


def default_threads(n_streams: int) -> int:
    """min(#independent streams, cores this process may run on)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(int(n_streams), cores))


def forward(q, k, v, log_alpha, b, w, gamma=None, z=None, S0=None,
            scale=1.0, normalize_qk=True, threads=None):
    """Token recurrence in fp64.

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; log_alpha: [B, H, T, dk],
    [B, H, T] or a scalar; b: like log_alpha over dk; w: over dv;
    gamma: [H, dk] or None (= 1); z: [B, H, T, dk] or None (2 sigma(z) = 1);
    S0: [B, H, dk, dv] or None (= 0).

    Returns (o [B, H, T, dv], S_T [B, H, dk, dv]) as fp64 numpy arrays.
    """
    lib = _load()
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k, v shapes disagree")
    la = _gate(log_alpha, (B, H, T, dk), "log_alpha")
    bb = _gate(b, (B, H, T, dk), "b")
    ww = _gate(w, (B, H, T, dv), "w")
    g = None
    if gamma is not None:
        g = _f64(gamma)
        if g.shape != (H, dk):
            raise ValueError("gamma must be [H, dk]")
        g = np.ascontiguousarray(np.broadcast_to(g[None], (B, H, dk)))
    zz = _f64(z)
    if zz is not None and zz.shape != (B, H, T, dk):
        raise ValueError("z must be [B, H, T, dk]")
    s0 = _f64(S0)
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("S0 must be [B, H, dk, dv]")
    o = np.empty((B, H, T, dv), dtype=np.float64)
    sT = np.empty((B, H, dk, dv), dtype=np.float64)
    n = B * H
    if threads is None:
        threads = default_threads(n)
    rc = lib.gdr_oracle_forward(n, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                                _ptr(bb), _ptr(ww), _ptr(g), _ptr(zz),
                                float(scale), int(bool(normalize_qk)), _ptr(s0),
                                _ptr(o), _ptr(sT), int(threads))
    if rc != 0:
        raise MemoryError("oracle could not allocate its per-stream scratch")
    return o, sT


def _gate_grad(g, full, name):
    """Reduce a per-channel gradient ``full`` [B, H, T, d] to the shape of the
    gate argument ``g``: per-token gates sum over the channels, constant
    (scalar) gates have no gradient (None)."""
    if np.isscalar(g):
        return None
    shape = np.shape(g)
    if len(shape) == 3:
        return full.sum(axis=-1)
    return full


def backward(q, k, v, log_alpha, b, w, dO, gamma=None, z=None, S0=None, dS_T=None,
             scale=1.0, normalize_qk=True, threads=None):
    """Reverse-mode derivatives of ``forward`` in fp64 for the loss
    <dO, o> + <dS_T, S_T> (dS_T None = 0).

    Arguments as ``forward``, plus dO [B, H, T, dv] and dS_T [B, H, dk, dv].
    Returns a dict with dq, dk, dv [like q, k, v]; dlog_alpha, db, dw shaped
    like their gate argument (per-token gates summed over the channels; None
    for a constant gate); dgamma [H, dk] (summed over batch and tokens; None
    without gamma); dz [B, H, T, dk] (None without z); dS0 [B, H, dk, dv].
    """
    lib = _load()
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = qf.shape
    dv = vf.shape[3]
    la = _gate(log_alpha, (B, H, T, dk), "log_alpha")
    bb = _gate(b, (B, H, T, dk), "b")
    ww = _gate(w, (B, H, T, dv), "w")
    g = None
    if gamma is not None:
        g = _f64(gamma)
        if g.shape != (H, dk):
            raise ValueError("gamma must be [H, dk]")
        g = np.ascontiguousarray(np.broadcast_to(g[None], (B, H, dk)))
    zz = _f64(z)
    s0 = _f64(S0)
    do = _f64(dO)
    if do.shape != (B, H, T, dv):
        raise ValueError("dO must be [B, H, T, dv]")
    dst = _f64(dS_T)
    out = {n: np.empty((B, H, T, dk)) for n in ("dq", "dk", "dlog_alpha", "db", "dz")}
    out["dv"] = np.empty((B, H, T, dv))
    out["dw"] = np.empty((B, H, T, dv))
    out["dgamma"] = np.empty((B, H, dk))
    out["dS0"] = np.empty((B, H, dk, dv))
    n = B * H
    if threads is None:
        threads = default_threads(n)
    rc = lib.gdr_oracle_backward(n, T, dk, dv, _ptr(qf), _ptr(kf), _ptr(vf), _ptr(la), _ptr(bb), _ptr(ww),
                                 _ptr(g), _ptr(zz), float(scale), int(bool(normalize_qk)), _ptr(s0),
                                 _ptr(do), _ptr(dst), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["dlog_alpha"]), _ptr(out["db"]), _ptr(out["dw"]),
                                 _ptr(out["dgamma"]), _ptr(out["dz"]), _ptr(out["dS0"]), int(threads))
    if rc != 0:
        raise MemoryError("oracle could not allocate its per-stream scratch")
    out["dlog_alpha"] = _gate_grad(log_alpha, out["dlog_alpha"], "log_alpha")
    out["db"] = _gate_grad(b, out["db"], "b")
    out["dw"] = _gate_grad(w, out["dw"], "w")
    out["dgamma"] = out["dgamma"].sum(axis=0) if gamma is not None else None
    if z is None:
        out["dz"] = None
    return out


def prepass(q, k, gamma=None, z=None, scale=1.0, normalize_qk=True):
    """Pre-pass of a single token: returns (q_tilde [dk], k_unit [dk]) in fp64."""
    lib = _load()
    q = _f64(q).reshape(-1)
    k = _f64(k).reshape(-1)
    dk = q.shape[0]
    g = None if gamma is None else _f64(gamma).reshape(-1)
    zz = None if z is None else _f64(z).reshape(-1)
    qt = np.empty(dk)
    kn = np.empty(dk)
    lib.gdr_oracle_prepass(dk, _ptr(q), _ptr(k), _ptr(g), _ptr(zz), float(scale),
                           int(bool(normalize_qk)), _ptr(qt), _ptr(kn))
    return qt, kn


def decode_step(S, q, k, v, log_alpha, b, w, gamma=None, z=None, scale=1.0,
                normalize_qk=True, threads=None):
    """One decode step = the recurrence over a single token, state carried.

    S: [B, H, dk, dv]; per-token tensors [B, H, d] (or [B, H, 1, d]).
    Returns (o [B, H, dv], S_new [B, H, dk, dv]).
    """
    def t1(x):
        if x is None or np.isscalar(x):
            return x
        a = _f64(x)
        return a if a.ndim == 4 else a[:, :, None, :]
    def g1(x):
        if x is None or np.isscalar(x):
            return x
        a = _f64(x)
        if a.ndim == 2:       # per-token scalar gate [B, H]
            return a[:, :, None]
        return a if a.ndim == 4 else a[:, :, None, :]
    o, sT = forward(t1(q), t1(k), t1(v), g1(log_alpha), g1(b), g1(w), gamma=gamma,
                    z=t1(z), S0=S, scale=scale, normalize_qk=normalize_qk,
                    threads=threads)
    return o[:, :, 0, :], sT


def max_threads() -> int:
    return _load().gdr_oracle_max_threads()


def output_gate(o, g, norm_weight=None, eps=1e-6):
    """The layer's output gate after the recurrence (Muir reading notes,
    section 2.1: a per-head RMSNorm of o, after which the output gate g_t
    modulates every channel).  The pages give neither the gate's activation
    nor the norm's epsilon; this follows the library's reading: a sigmoid gate
    and eps added to the mean square.

    o, g: [B,H,T,dv]; norm_weight: [H,dv] or None (= 1).  Returns
    y [B,T,H,dv] (token-major) in fp64.
    """
    o = _f64(o)
    g = _f64(g)
    mean_sq = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(mean_sq + eps)
    if norm_weight is not None:
        y = y * _f64(norm_weight)[None, :, None, :]
    y = y / (1.0 + np.exp(-g))
    return np.ascontiguousarray(y.transpose(0, 2, 1, 3))


def output_gate_backward(o, g, dy, norm_weight=None, eps=1e-6):
    """Reverse mode of output_gate: for the loss <dy, y>, the gradients of o,
    g and norm_weight.  With r = (mean_c o_c^2 + eps)^(-1/2), n = o r,
    s = sigmoid(g) and u = dy * weight * s (the gradient reaching n):
      dg = dy * n * weight * s * (1 - s)
      d weight[h, c] = sum over batch and tokens of dy * n * s
      do = r * (u - n * sum_c(u_c n_c) / dv)      (through the row norm)
    dy: [B,T,H,dv] (token-major, as y).  Returns (do, dg, d_norm_weight or
    None) in fp64, do and dg as [B,H,T,dv].
    """
    o = _f64(o)
    g = _f64(g)
    dy = np.ascontiguousarray(_f64(dy).transpose(0, 2, 1, 3))
    dv = o.shape[-1]
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    n = o * r
    s = 1.0 / (1.0 + np.exp(-g))
    wgt = np.ones(o.shape[1:2] + (1, dv)) if norm_weight is None else _f64(norm_weight)[:, None, :]
    dg = dy * n * wgt * s * (1.0 - s)
    dw = None if norm_weight is None else np.sum(dy * n * s, axis=(0, 2))
    u = dy * wgt * s
    do = r * (u - n * np.sum(u * n, axis=-1, keepdims=True) / dv)
    return do, dg, dw


GATE_ORDER = ("f", "b", "g", "w", "q")


def gate_proj(x, w_down, w_up, bias, ranks, H, d):
    """The five gates from one shared low-rank projection (Muir reading notes,
    section 2.3: a shared down-projection, then a per-gate up-projection and
    channel bias give each gate's logits; ranks (r_f, r_b, r_g, r_w, r_q)).
    The pages print neither the formula nor the activations; this follows the
    library's reading, with the ranges section 2.1 states:
      decay  alpha = sigmoid(l_f)   -> returned as log alpha = log sigmoid(l_f)
      erase  b = 2 sigmoid(l_b)     in (0, 2)
      output gate logits l_g        (the gated output applies a sigmoid)
      write  w = sigmoid(l_w)       in (0, 1)
      query gain logits z = l_q     (the read-out applies 2 sigmoid(z))

    x: [B,T,dm]; w_down: [R,dm] with R = sum(ranks) (rows in gate order
    f, b, g, w, q); w_up: dict gate -> [H*d, r_gate]; bias: [5, H*d] in gate
    order.  Weights are nn.Linear-style [out, in].  Returns a dict gate ->
    [B,H,T,d] fp64 (log alpha for "f").
    """
    x = _f64(x)
    wd = _f64(w_down)
    bias = _f64(bias)
    B, T, _ = x.shape
    h = x @ wd.T                       # [B,T,R]
    out = {}
    r0 = 0
    for gi, name in enumerate(GATE_ORDER):
        r = int(ranks[gi])
        logits = h[..., r0:r0 + r] @ _f64(w_up[name]).T + bias[gi]   # [B,T,H*d]
        r0 += r
        if name == "f":
            val = -np.logaddexp(0.0, -logits)        # log sigmoid
        elif name == "b":
            val = 2.0 / (1.0 + np.exp(-logits))
        elif name == "w":
            val = 1.0 / (1.0 + np.exp(-logits))
        else:                                        # g, q: logits
            val = logits
        out[name] = np.ascontiguousarray(val.reshape(B, T, H, d).transpose(0, 2, 1, 3))
    return out

"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own loop.  Each check uses a different
formulation of the same quantity, so that a dropped term, a wrong sign, a wrong
index or a transposed operand in the oracle fails at least one of them:

* pre-pass against library routines (torch SiLU / F.normalize in fp64);
* DeltaNet: the blog's sequential prefill (Kimi3 = GPT2 x 22580, hubwiz
  translation, section 4 "DeltaNet", the sequential delta-rule loop) and its
  UT-transform chunk algorithm (same section, chunk_delta_rule_forward);
* linear attention (same blog, section 4, sequential / chunked linear
  attention) as the closed form o_t = sum_{s<=t} (q_t . k_s) v_s;
* gated linear attention (b = 0) as an O(T^2) sum with explicit decay products;
* Gated DeltaNet / KDA in the blog's column convention
  S_t = S_{t-1} Diag(alpha)(I - beta k k^T) + beta v k^T, o_t = S_t q_t
  (section 4, the reparameterised DeltaNet, with the decay of section 5
  "Gated Delta Net" and the per-channel decay of section 6 "KDA");
* general GDN-2: brute-force products of the dense transition matrices; the
  whole-sequence and chunked triangular systems T Z = [V_hat, K_hat decayed]
  of the Muir reading notes (arXiv:2611.08376) section 2.4; exact recall for
  b = 1 (blog section 3, unit-norm read-back); alpha = 0 clears the memory
  (blog section 5); linearity in (v, S0); split/resume; gain only touching the
  read-out (Muir notes section 2.1); the write/erase sensitivity identity of
  Prop. 3.1 (Muir notes section 2.2); the erase-key eigen-relation.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

RTOL = 1e-12


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def softplus(x):
    return np.logaddexp(0.0, x)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def problem(seed, B=1, H=2, T=24, dk=8, dv=6, decay=0.3, s0=True, gain=True):
    r = np.random.default_rng(seed)
    p = dict(
        q=r.standard_normal((B, H, T, dk)),
        k=r.standard_normal((B, H, T, dk)),
        v=r.standard_normal((B, H, T, dv)),
        log_alpha=-decay * softplus(r.standard_normal((B, H, T, dk))),
        b=2.0 * sigmoid(r.standard_normal((B, H, T, dk))),
        w=sigmoid(r.standard_normal((B, H, T, dv))),
        gamma=(1.0 + 0.2 * r.standard_normal((H, dk))) if gain else None,
        z=r.standard_normal((B, H, T, dk)) if gain else None,
        S0=(0.3 * r.standard_normal((B, H, dk, dv))) if s0 else None,
    )
    return p


def lib_prepass(q, k, gamma=None, z=None, scale=1.0):
    """SiLU + L2 and the read-out gain with torch library routines, fp64."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    qh = F.normalize(F.silu(qt), dim=-1, eps=1e-12)
    kn = F.normalize(F.silu(kt), dim=-1, eps=1e-12)
    if z is not None:
        qh = qh * 2.0 * torch.sigmoid(torch.from_numpy(np.asarray(z, dtype=np.float64)))
    if gamma is not None:
        g = torch.from_numpy(np.asarray(gamma, dtype=np.float64))
        qh = qh * g[None, :, None, :]
    return (scale * qh).numpy(), kn.numpy()


def features(p, scale=1.0):
    qt, kn = lib_prepass(p["q"], p["k"], p["gamma"], p["z"], scale)
    kh = p["b"] * kn if np.ndim(p["b"]) == 4 else p["b"][..., None] * kn
    vh = p["w"] * p["v"] if np.ndim(p["w"]) == 4 else p["w"][..., None] * p["v"]
    return qt, kn, kh, vh


def run(oracle_mod, p, **kw):
    return oracle_mod.forward(p["q"], p["k"], p["v"], p["log_alpha"], p["b"], p["w"],
                              gamma=p["gamma"], z=p["z"], S0=p["S0"], **kw)


# ----------------------------------------------------------------------------
# pre-pass
# ----------------------------------------------------------------------------

def test_prepass_matches_library_routines(oracle_mod):
    r = np.random.default_rng(11)
    for dk in (4, 64, 128):
        q, k, z = r.standard_normal((3, dk))
        gamma = 1.0 + 0.1 * r.standard_normal(dk)
        qt, kn = oracle_mod.prepass(q, k, gamma=gamma, z=z, scale=0.7)
        qt_ref, kn_ref = lib_prepass(q[None, None, None], k[None, None, None],
                                     gamma[None], z[None, None, None], 0.7)
        assert rel(qt, qt_ref.reshape(-1)) < RTOL
        assert rel(kn, kn_ref.reshape(-1)) < RTOL
        assert abs(np.linalg.norm(kn) - 1.0) < 1e-14


def test_prepass_zero_key_and_no_normalise(oracle_mod):
    dk = 16
    qt, kn = oracle_mod.prepass(np.zeros(dk), np.zeros(dk))
    assert np.all(kn == 0.0) and np.all(qt == 0.0)  # SiLU(0) = 0 and the 1e-12 floor
    r = np.random.default_rng(3)
    q, k = r.standard_normal((2, dk))
    qt, kn = oracle_mod.prepass(q, k, normalize_qk=False, scale=2.0)
    assert rel(qt, 2.0 * q) < RTOL and rel(kn, k) < RTOL


# ----------------------------------------------------------------------------
# DeltaNet (alpha = 1, b = w = beta, no gain)
# ----------------------------------------------------------------------------

def deltanet_problem(seed, B=2, H=2, T=32, d=8):
    r = np.random.default_rng(seed)
    return dict(q=r.standard_normal((B, H, T, d)), k=r.standard_normal((B, H, T, d)),
                v=r.standard_normal((B, H, T, d)),
                beta=sigmoid(r.standard_normal((B, H, T))),
                S0=0.3 * r.standard_normal((B, H, d, d)))


def test_deltanet_sequential_prefill(oracle_mod):
    p = deltanet_problem(0)
    qn, kn = lib_prepass(p["q"], p["k"])
    # sequential delta-rule prefill, batched over (b, h), row convention
    S = torch.from_numpy(p["S0"].copy())
    q_, k_, v_ = (torch.from_numpy(x) for x in (qn, kn, p["v"]))
    beta = torch.from_numpy(p["beta"])
    outs = []
    for i in range(q_.shape[2]):
        ki = k_[:, :, i:i + 1]
        v_old = ki @ S
        u = beta[:, :, i, None, None] * (v_[:, :, i:i + 1] - v_old)
        S = S + ki.transpose(-1, -2) @ u
        outs.append(q_[:, :, i:i + 1] @ S)
    o_ref = torch.cat(outs, dim=2).numpy()
    o, sT = oracle_mod.forward(p["q"], p["k"], p["v"], 0.0, p["beta"], p["beta"], S0=p["S0"])
    assert rel(o, o_ref) < RTOL
    assert rel(sT, S.numpy()) < RTOL


@pytest.mark.parametrize("C", [1, 4, 8, 32])
def test_deltanet_ut_transform_chunks(oracle_mod, C):
    """UT/WY chunk form: (I + tril(K_b K^T, -1))^-1 applied to K_b and V_b."""
    p = deltanet_problem(1)
    qn, kn = lib_prepass(p["q"], p["k"])
    B, H, T, d = qn.shape
    o_ref = np.empty_like(p["v"])
    s_ref = np.empty_like(p["S0"])
    for bb in range(B):
        for hh in range(H):
            S = p["S0"][bb, hh].copy()
            for c0 in range(0, T, C):
                sl = slice(c0, c0 + C)
                Q, K, V = qn[bb, hh, sl], kn[bb, hh, sl], p["v"][bb, hh, sl]
                be = p["beta"][bb, hh, sl][:, None]
                Kb, Vb = K * be, V * be
                Tinv = np.linalg.inv(np.eye(len(K)) + np.tril(Kb @ K.T, -1))
                W, U = Tinv @ Kb, Tinv @ Vb
                u = U - W @ S
                o_ref[bb, hh, sl] = Q @ S + np.tril(Q @ K.T) @ u
                S = S + K.T @ u
            s_ref[bb, hh] = S
    o, sT = oracle_mod.forward(p["q"], p["k"], p["v"], 0.0, p["beta"], p["beta"], S0=p["S0"])
    assert rel(o, o_ref) < 1e-11
    assert rel(sT, s_ref) < 1e-11


# ----------------------------------------------------------------------------
# linear attention (b = 0, alpha = 1, w = 1) and gated linear attention (b = 0)
# ----------------------------------------------------------------------------

def test_linear_attention_closed_form(oracle_mod):
    p = problem(2, gain=False)
    qt, kn, _, _ = features(p)
    scores = np.einsum("bhtj,bhsj->bhts", qt, kn)
    o_ref = np.einsum("bhts,bhsv->bhtv", np.tril(scores), p["v"])
    o_ref += np.einsum("bhtj,bhjv->bhtv", qt, p["S0"])
    s_ref = p["S0"] + np.einsum("bhtj,bhtv->bhjv", kn, p["v"])
    o, sT = oracle_mod.forward(p["q"], p["k"], p["v"], 0.0, 0.0, 1.0, S0=p["S0"])
    assert rel(o, o_ref) < RTOL
    assert rel(sT, s_ref) < RTOL


def test_gated_linear_attention_explicit_products(oracle_mod):
    p = problem(3, T=20)
    qt, kn, _, vh = features(p)
    alpha = np.exp(p["log_alpha"])
    B, H, T, dk = qt.shape
    o_ref = np.zeros_like(vh)
    for bb in range(B):
        for hh in range(H):
            a = alpha[bb, hh]
            for t in range(T):
                head = np.prod(a[: t + 1], axis=0)          # prod_{r<=t} alpha_r
                S = head[:, None] * p["S0"][bb, hh]
                for s in range(t + 1):
                    dec = np.prod(a[s + 1: t + 1], axis=0)  # prod_{r=s+1..t}
                    S = S + dec[:, None] * np.outer(kn[bb, hh, s], vh[bb, hh, s])
                o_ref[bb, hh, t] = qt[bb, hh, t] @ S
    o, _ = oracle_mod.forward(p["q"], p["k"], p["v"], p["log_alpha"], 0.0, p["w"],
                              gamma=p["gamma"], z=p["z"], S0=p["S0"])
    assert rel(o, o_ref) < RTOL


# ----------------------------------------------------------------------------
# Gated DeltaNet (scalar alpha) and KDA (per-channel alpha), b = w = beta,
# in the blog's column convention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("per_channel", [False, True])
def test_gdn_kda_column_convention(oracle_mod, per_channel):
    r = np.random.default_rng(4 + per_channel)
    B, H, T, d = 1, 3, 28, 8
    q, k, v = r.standard_normal((3, B, H, T, d))
    beta = sigmoid(r.standard_normal((B, H, T)))
    if per_channel:
        la = -0.4 * softplus(r.standard_normal((B, H, T, d)))
    else:
        la = -0.4 * softplus(r.standard_normal((B, H, T)))
    S0 = 0.3 * r.standard_normal((B, H, d, d))
    qn, kn = lib_prepass(q, k)
    o_ref = np.empty_like(v)
    s_ref = np.empty_like(S0)
    for bb in range(B):
        for hh in range(H):
            Sc = S0[bb, hh].T.copy()           # column convention: [dv, dk]
            for t in range(T):
                kt = kn[bb, hh, t][:, None]
                a = np.exp(la[bb, hh, t]) * np.ones(d)
                be = beta[bb, hh, t]
                Sc = Sc @ np.diag(a) @ (np.eye(d) - be * kt @ kt.T) + be * v[bb, hh, t][:, None] @ kt.T
                o_ref[bb, hh, t] = Sc @ qn[bb, hh, t]
            s_ref[bb, hh] = Sc.T
    o, sT = oracle_mod.forward(q, k, v, la, beta, beta, S0=S0)
    assert rel(o, o_ref) < RTOL
    assert rel(sT, s_ref) < RTOL


# ----------------------------------------------------------------------------
# general GDN-2
# ----------------------------------------------------------------------------

def brute_force(qt, kn, kh, vh, alpha, S0):
    """S_t = (M_t...M_1) S0 + sum_s (M_t...M_{s+1}) k_s^T v_hat_s,
    M_t = (I - k_t^T k_hat_t) Diag(alpha_t), all products formed explicitly."""
    T, dk = kn.shape
    I = np.eye(dk)
    M = [(I - np.outer(kn[t], kh[t])) @ np.diag(alpha[t]) for t in range(T)]
    o = np.empty((T, vh.shape[1]))
    S = None
    for t in range(T):
        P = I.copy()
        for r_ in range(t, -1, -1):
            P = P @ M[r_]
        S = P @ S0
        for s in range(t + 1):
            P = I.copy()
            for r_ in range(t, s, -1):
                P = P @ M[r_]
            S = S + P @ np.outer(kn[s], vh[s])
        o[t] = qt[t] @ S
    return o, S


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_bruteforce_transition_products(oracle_mod, seed):
    p = problem(seed, B=1, H=2, T=12, dk=6, dv=5, decay=0.5)
    qt, kn, kh, vh = features(p)
    alpha = np.exp(p["log_alpha"])
    o, sT = run(oracle_mod, p)
    for hh in range(2):
        o_ref, s_ref = brute_force(qt[0, hh], kn[0, hh], kh[0, hh], vh[0, hh], alpha[0, hh],
                                   p["S0"][0, hh])
        assert rel(o[0, hh], o_ref) < RTOL
        assert rel(sT[0, hh], s_ref) < RTOL


def chunk_system(qt, kn, kh, vh, la, S0, C):
    """Chunkwise form: per chunk solve (I + L) [U_bar, Y] = [V_hat, K_hat e^Lam]
    with L[t,s] = (k_hat_t . pi_ts) . k_s (s < t), pi_ts = exp(Lam_t - Lam_s);
    then U = U_bar - Y S, O = (Q e^Lam) S + A U, S <- e^Lam_C S + (K e^{Lam_C-Lam})^T U."""
    T, dk = kn.shape
    S = S0.copy()
    O = np.empty((T, vh.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        n = sl.stop - sl.start
        Lam = np.cumsum(la[sl], axis=0)
        diff = Lam[:, None, :] - Lam[None, :, :]
        causal = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
        pi = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
        L = np.tril(np.einsum("tj,tsj,sj->ts", kh[sl], pi, kn[sl]), -1)
        A = np.tril(np.einsum("tj,tsj,sj->ts", qt[sl], pi, kn[sl]))
        Tm = np.eye(n) + L
        Ubar = np.linalg.solve(Tm, vh[sl])
        Y = np.linalg.solve(Tm, kh[sl] * np.exp(Lam))
        U = Ubar - Y @ S
        O[sl] = (qt[sl] * np.exp(Lam)) @ S + A @ U
        S = np.exp(Lam[-1])[:, None] * S + (kn[sl] * np.exp(Lam[-1] - Lam)).T @ U
    return O, S


@pytest.mark.parametrize("C", [1, 3, 8, 16, 48])
def test_triangular_chunk_system(oracle_mod, C):
    p = problem(8, B=1, H=2, T=48, dk=8, dv=6)
    qt, kn, kh, vh = features(p)
    o, sT = run(oracle_mod, p)
    for hh in range(2):
        o_ref, s_ref = chunk_system(qt[0, hh], kn[0, hh], kh[0, hh], vh[0, hh],
                                    p["log_alpha"][0, hh], p["S0"][0, hh], C)
        assert rel(o[0, hh], o_ref) < 1e-11
        assert rel(sT[0, hh], s_ref) < 1e-11


def test_exact_recall_unit_erase(oracle_mod):
    """With b_t = 1 the key written at t reads back exactly v_hat_t: k_t S_t = v_hat_t."""
    p = problem(9, T=10)
    p["b"] = np.ones_like(p["b"])
    qt, kn, kh, vh = features(p)
    for T in (1, 5, 10):
        sub = {key: (val[:, :, :T] if (val is not None and np.ndim(val) == 4 and key not in ("S0",))
                     else val) for key, val in p.items()}
        _, sT = run(oracle_mod, sub)
        read = np.einsum("bhj,bhjv->bhv", kn[:, :, T - 1], sT)
        assert rel(read, vh[:, :, T - 1]) < 1e-13


def test_alpha_zero_clears_memory(oracle_mod):
    p = problem(10, T=16)
    t0 = 9
    p["log_alpha"][:, :, t0, :] = -1000.0   # exp underflows to exactly 0 in fp64
    qt, kn, kh, vh = features(p)
    sub = {key: (val[:, :, : t0 + 1] if (val is not None and np.ndim(val) == 4 and key != "S0")
                 else val) for key, val in p.items()}
    _, s_t0 = run(oracle_mod, sub)
    assert rel(s_t0, np.einsum("bhj,bhv->bhjv", kn[:, :, t0], vh[:, :, t0])) < 1e-14
    # and nothing before t0 influences what follows
    q2 = dict(p)
    q2["v"] = p["v"].copy()
    q2["v"][:, :, :t0] += 5.0
    q2["S0"] = p["S0"] * -3.0
    o1, s1 = run(oracle_mod, p)
    o2, s2 = run(oracle_mod, q2)
    assert rel(o2[:, :, t0:], o1[:, :, t0:]) < 1e-13
    assert rel(s2, s1) < 1e-13


def test_joint_linearity_in_values_and_state(oracle_mod):
    p1 = problem(12)
    p2 = problem(13)
    p2.update({key: p1[key] for key in ("q", "k", "log_alpha", "b", "w", "gamma", "z")})
    a, c = 0.7, -1.9
    pm = dict(p1)
    pm["v"] = a * p1["v"] + c * p2["v"]
    pm["S0"] = a * p1["S0"] + c * p2["S0"]
    o1, s1 = run(oracle_mod, p1)
    o2, s2 = run(oracle_mod, p2)
    om, sm = run(oracle_mod, pm)
    assert rel(om, a * o1 + c * o2) < 1e-12
    assert rel(sm, a * s1 + c * s2) < 1e-12


def test_split_resume(oracle_mod):
    p = problem(14, T=40)
    o, sT = run(oracle_mod, p)
    cut = 17
    first = {key: (val[:, :, :cut] if (val is not None and np.ndim(val) == 4 and key != "S0") else val)
             for key, val in p.items()}
    second = {key: (val[:, :, cut:] if (val is not None and np.ndim(val) == 4 and key != "S0") else val)
              for key, val in p.items()}
    o1, s1 = run(oracle_mod, first)
    second["S0"] = s1
    o2, s2 = run(oracle_mod, second)
    assert rel(np.concatenate([o1, o2], axis=2), o) < 1e-13
    assert rel(s2, sT) < 1e-13


def test_gain_touches_only_the_readout(oracle_mod):
    p = problem(15)
    o, sT = run(oracle_mod, p)
    p_nogain = dict(p, gamma=None, z=None)
    o0, s0 = run(oracle_mod, p_nogain)
    assert rel(sT, s0) < 1e-15 or np.array_equal(sT, s0)
    # o is linear in gamma for fixed z
    g1 = p["gamma"]
    g2 = np.random.default_rng(16).standard_normal(g1.shape)
    oa, _ = run(oracle_mod, dict(p, gamma=g1))
    ob, _ = run(oracle_mod, dict(p, gamma=g2))
    oc, _ = run(oracle_mod, dict(p, gamma=g1 + g2))
    assert rel(oc, oa + ob) < 1e-12
    # gamma = 1 and z = 0 give exactly the un-gained read-out
    B, H, T, dk = p["q"].shape
    o1, _ = run(oracle_mod, dict(p, gamma=np.ones((H, dk)), z=np.zeros((B, H, T, dk))))
    assert rel(o1, o0) < 1e-15


def test_erase_write_sensitivity_identity(oracle_mod):
    """Prop. 3.1 (Muir notes section 2.2): for isotropic unit-variance
    perturbations, E|dS|^2 from the erase gate equals sum_j k_j^2 |S_hat_j|^2 and
    from the write gate equals |k|^2 |v|^2, independent of the key's sparsity."""
    r = np.random.default_rng(17)
    dk, dv = 8, 6
    q, k = r.standard_normal((2, 1, 1, 1, dk))
    v = r.standard_normal((1, 1, 1, dv))
    la = -0.3 * softplus(r.standard_normal((1, 1, 1, dk)))
    b = 2.0 * sigmoid(r.standard_normal((1, 1, 1, dk)))
    w = sigmoid(r.standard_normal((1, 1, 1, dv)))
    S0 = r.standard_normal((1, 1, dk, dv))
    _, kn = lib_prepass(q, k)
    kn = kn[0, 0, 0]
    S_hat = np.exp(la[0, 0, 0])[:, None] * S0[0, 0]

    def S_of(bb, ww):
        return oracle_mod.forward(q, k, v, la, bb, ww, S0=S0)[1][0, 0]

    base = S_of(b, w)
    erase = 0.0
    for j in range(dk):
        e = np.zeros_like(b)
        e[..., j] = 1.0
        erase += np.sum((S_of(b + e, w) - base) ** 2)  # S is affine in b: exact difference
    write = 0.0
    for j in range(dv):
        e = np.zeros_like(w)
        e[..., j] = 1.0
        write += np.sum((S_of(b, w + e) - base) ** 2)
    assert abs(erase - np.sum(kn ** 2 * np.sum(S_hat ** 2, axis=1))) < 1e-12 * max(1.0, erase)
    assert abs(write - np.sum(kn ** 2) * np.sum(v ** 2)) < 1e-12 * max(1.0, write)


def test_erase_key_eigen_relation(oracle_mod):
    """(I - k^T k_hat) k^T = (1 - k_hat . k) k^T: a state along k only rescales."""
    r = np.random.default_rng(18)
    dk, dv = 8, 5
    q, k = r.standard_normal((2, 1, 1, 1, dk))
    v = r.standard_normal((1, 1, 1, dv))
    b = 2.0 * sigmoid(r.standard_normal((1, 1, 1, dk)))
    x = r.standard_normal(dv)
    _, kn = lib_prepass(q, k)
    kn = kn[0, 0, 0]
    S0 = np.outer(kn, x)[None, None]
    _, sT = oracle_mod.forward(q, k, v, 0.0, b, 0.0, S0=S0)
    assert rel(sT[0, 0], (1.0 - (b[0, 0, 0] * kn) @ kn) * np.outer(kn, x)) < 1e-13


# ----------------------------------------------------------------------------
# the pins fail on plausible mistakes (mistakes planted in a numpy copy)
# ----------------------------------------------------------------------------

def token_loop(qt, kn, kh, vh, alpha, S0, variant):
    S = S0.copy()
    o = np.empty((len(kn), vh.shape[1]))
    for t in range(len(kn)):
        if variant == "write_before_decay":
            S = S + np.outer(kn[t], vh[t] - kh[t] @ S)
            S = alpha[t][:, None] * S
        else:
            Sh = alpha[t][:, None] * S
            if variant == "erase_along_khat":     # the other reading of the update
                S = Sh - np.outer(kh[t], kn[t] @ Sh) + np.outer(kn[t], vh[t])
            elif variant == "read_before_write":
                o[t] = qt[t] @ Sh
                S = Sh + np.outer(kn[t], vh[t] - kh[t] @ Sh)
                continue
            else:
                S = Sh + np.outer(kn[t], vh[t] - kh[t] @ Sh)
        o[t] = qt[t] @ S
    return o, S


@pytest.mark.parametrize("variant", ["erase_along_khat", "write_before_decay", "read_before_write"])
def test_pins_reject_planted_mistakes(variant):
    p = problem(19, B=1, H=1, T=16, dk=6, dv=5, decay=0.5)
    qt, kn, kh, vh = features(p)
    args = (qt[0, 0], kn[0, 0], kh[0, 0], vh[0, 0])
    la = p["log_alpha"][0, 0]
    good_o, good_s = token_loop(*args, np.exp(la), p["S0"][0, 0], "correct")
    bad_o, bad_s = token_loop(*args, np.exp(la), p["S0"][0, 0], variant)
    ref_o, ref_s = chunk_system(*args, la, p["S0"][0, 0], 4)
    assert rel(good_o, ref_o) < 1e-11 and rel(good_s, ref_s) < 1e-11
    assert rel(bad_o, ref_o) > 1e-3


# ----------------------------------------------------------------------------
# the layer's output gate (Muir notes section 2.1: per-head RMSNorm of o, then
# the output gate modulates every channel; sigmoid and eps are the readings)
# ----------------------------------------------------------------------------

def test_output_gate_unit_rms_and_scale_invariance(oracle_mod):
    """With the gate saturated open (sigmoid -> 1), no weight and eps = 0 the
    output has unit RMS over the channels of each (token, head), and scaling
    o by a positive constant changes nothing."""
    r = np.random.default_rng(5)
    o = r.standard_normal((2, 3, 7, 16))
    g = np.full_like(o, 60.0)
    y = oracle_mod.output_gate(o, g, eps=0.0)
    assert y.shape == (2, 7, 3, 16)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(oracle_mod.output_gate(3.7 * o, g, eps=0.0), y, rtol=1e-12)


def test_output_gate_hand_example_and_layout(oracle_mod):
    """o = (1, -1, 1, -1) has mean square 1, so with g = 0 (sigmoid = 1/2)
    and a weight of 2 for head 1 only, y = o / 2 for head 0 and o for head 1;
    the (head, token) axes come out transposed."""
    o = np.zeros((1, 2, 3, 4))
    o[0, 0, 2] = [1.0, -1.0, 1.0, -1.0]
    o[0, 1, 1] = [1.0, -1.0, 1.0, -1.0]
    o[0, 0, 0] = o[0, 0, 1] = o[0, 1, 0] = o[0, 1, 2] = [2.0, 2.0, 2.0, 2.0]
    wgt = np.ones((2, 4))
    wgt[1] = 2.0
    y = oracle_mod.output_gate(o, np.zeros_like(o), norm_weight=wgt, eps=0.0)
    np.testing.assert_allclose(y[0, 2, 0], [0.5, -0.5, 0.5, -0.5], rtol=1e-15)
    np.testing.assert_allclose(y[0, 1, 1], [1.0, -1.0, 1.0, -1.0], rtol=1e-15)
    np.testing.assert_allclose(y[0, 0, 0], [0.5, 0.5, 0.5, 0.5], rtol=1e-15)
    np.testing.assert_allclose(y[0, 0, 1], [1.0, 1.0, 1.0, 1.0], rtol=1e-15)


def test_output_gate_zero_input_and_gate_values(oracle_mod):
    """o = 0 with eps > 0 gives 0 (no division by zero); the gate factor at
    logit x is 1 / (1 + e^-x): x = ln 3 gives 3/4."""
    y0 = oracle_mod.output_gate(np.zeros((1, 1, 2, 8)), np.zeros((1, 1, 2, 8)), eps=1e-6)
    assert np.all(y0 == 0.0)
    o = np.ones((1, 1, 1, 8))
    y = oracle_mod.output_gate(o, np.full_like(o, np.log(3.0)), eps=0.0)
    np.testing.assert_allclose(y, 0.75, rtol=1e-14)


# ----------------------------------------------------------------------------
# the five-gate low-rank projection (Muir notes section 2.3; activations and
# layouts are the library's reading, ranges from section 2.1)
# ----------------------------------------------------------------------------

def _gate_problem(seed, B=2, T=5, dm=12, H=2, d=3, ranks=(2, 2, 3, 3, 3)):
    r = np.random.default_rng(seed)
    R = sum(ranks)
    x = r.standard_normal((B, T, dm))
    wd = r.standard_normal((R, dm)) / np.sqrt(dm)
    wu = {n: r.standard_normal((H * d, rk)) / np.sqrt(rk) for n, rk in zip(("f", "b", "g", "w", "q"), ranks)}
    bias = 0.3 * r.standard_normal((5, H * d))
    return x, wd, wu, bias, ranks, H, d


def _logits(out):
    """Undo each gate's activation (a different formulation from the oracle's)."""
    return {"f": np.log(np.expm1(-out["f"])) * -1.0,        # log alpha = -softplus(-l)
            "b": np.log(out["b"] / (2.0 - out["b"])),
            "w": np.log(out["w"] / (1.0 - out["w"])),
            "g": out["g"], "q": out["q"]}


def test_gate_proj_zero_weights_give_the_bias(oracle_mod):
    x, wd, wu, bias, ranks, H, d = _gate_problem(1)
    out = oracle_mod.gate_proj(x, np.zeros_like(wd), wu, bias, ranks, H, d)
    bh = bias.reshape(5, H, d)
    np.testing.assert_allclose(out["b"][1, 1, 3], 2.0 / (1.0 + np.exp(-bh[1, 1])), rtol=1e-14)
    np.testing.assert_allclose(out["w"][0, 0, 4], 1.0 / (1.0 + np.exp(-bh[3, 0])), rtol=1e-14)
    np.testing.assert_allclose(out["f"][1, 0, 0], np.log(1.0 / (1.0 + np.exp(-bh[0, 0]))), rtol=1e-13)
    np.testing.assert_allclose(out["g"][0, 1, 2], bh[2, 1], rtol=1e-15)
    np.testing.assert_allclose(out["q"][1, 1, 1], bh[4, 1], rtol=1e-15)
    assert np.all(out["f"] < 0) and np.all((out["b"] > 0) & (out["b"] < 2)) and np.all((out["w"] > 0) & (out["w"] < 1))


def test_gate_proj_linear_low_rank_and_separate(oracle_mod):
    """The logits minus the bias are linear in x, of rank at most r_gate over
    the tokens, and each gate depends only on its own rows of the down-projection
    and its own up-projection."""
    x, wd, wu, bias, ranks, H, d = _gate_problem(2, B=1, T=20)
    x2 = np.random.default_rng(9).standard_normal(x.shape)
    l1 = _logits(oracle_mod.gate_proj(x, wd, wu, bias, ranks, H, d))
    l2 = _logits(oracle_mod.gate_proj(x2, wd, wu, bias, ranks, H, d))
    l12 = _logits(oracle_mod.gate_proj(x + x2, wd, wu, bias, ranks, H, d))
    bh = bias.reshape(5, 1, H, 1, d)
    for gi, n in enumerate(("f", "b", "g", "w", "q")):
        lin = l1[n] + l2[n] - bh[gi]
        np.testing.assert_allclose(l12[n], lin, rtol=1e-9, atol=1e-9)
        tok_by_chan = (l1[n] - bh[gi])[0].transpose(1, 0, 2).reshape(x.shape[1], H * d)
        assert np.linalg.matrix_rank(tok_by_chan, tol=1e-9) <= ranks[gi]
    # perturb the up-projection of the write gate and the down-projection rows of
    # the erase gate: only those gates move
    wu2 = dict(wu)
    wu2["w"] = wu["w"] + 0.5
    wd2 = wd.copy()
    wd2[ranks[0]:ranks[0] + ranks[1]] += 0.5
    base = oracle_mod.gate_proj(x, wd, wu, bias, ranks, H, d)
    pert = oracle_mod.gate_proj(x, wd2, wu2, bias, ranks, H, d)
    for n in ("f", "g", "q"):
        np.testing.assert_array_equal(base[n], pert[n])
    assert not np.allclose(base["w"], pert["w"]) and not np.allclose(base["b"], pert["b"])


def test_gate_proj_layout(oracle_mod):
    """Output channel j = h * d + c of token (b, t) lands at [b, h, t, c]:
    an up-projection that copies one rank column to a single output channel."""
    x, wd, wu, bias, ranks, H, d = _gate_problem(3)
    wq = np.zeros_like(wu["q"])
    wq[1 * d + 2, 0] = 1.0                      # head 1, channel 2 <- first q rank
    wu2 = dict(wu)
    wu2["q"] = wq
    out = oracle_mod.gate_proj(x, wd, wu2, np.zeros_like(bias), ranks, H, d)
    rq0 = sum(ranks[:4])
    expect = x @ wd[rq0]                        # [B,T]
    np.testing.assert_allclose(out["q"][:, 1, :, 2], expect, rtol=1e-13)
    mask = np.ones((H, d), dtype=bool)
    mask[1, 2] = False
    assert np.all(out["q"].transpose(0, 2, 1, 3)[:, :, mask] == 0.0)


# ----------------------------------------------------------------------------
# backward (reverse-mode derivatives of the same recurrence for the loss
# <dO, o> + <dS_T, S_T>): pinned to the forward oracle by central differences,
# to itself across a split sequence, and to a closed form
# ----------------------------------------------------------------------------

def _bwd_problem(seed, B=1, H=2, T=9, d=4, per_token=False, gain=True):
    r = np.random.default_rng(seed)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    gshape = (B, H, T) if per_token else (B, H, T, d)
    p = dict(q=r.standard_normal((B, H, T, d)), k=r.standard_normal((B, H, T, d)),
             v=r.standard_normal((B, H, T, d)), log_alpha=-0.3 * r.random(gshape),
             b=2.0 * sig(r.standard_normal(gshape)), w=sig(r.standard_normal(gshape)),
             S0=r.standard_normal((B, H, d, d)))
    if gain:
        p["gamma"] = 1.0 + 0.1 * r.standard_normal((H, d))
        p["z"] = r.standard_normal((B, H, T, d))
    dO = r.standard_normal((B, H, T, d))
    dST = r.standard_normal((B, H, d, d))
    return p, dO, dST


def _loss(oracle_mod, p, dO, dST, **kw):
    o, sT = oracle_mod.forward(**p, **kw)
    return float((o * dO).sum() + (sT * dST).sum())


def _fd_check(oracle_mod, p, dO, dST, grads, names, n_samples, seed, **kw):
    r = np.random.default_rng(seed)
    key = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "b": "db", "w": "dw",
           "z": "dz", "S0": "dS0", "gamma": "dgamma"}
    h = 1e-6
    for name in names:
        arr = p[name]
        flat = [tuple(ix) for ix in np.ndindex(arr.shape)]
        picks = flat if len(flat) <= n_samples else [flat[i] for i in r.choice(len(flat), n_samples, replace=False)]
        for ix in picks:
            ap, am = arr.copy(), arr.copy()
            ap[ix] += h
            am[ix] -= h
            num = (_loss(oracle_mod, {**p, name: ap}, dO, dST, **kw) -
                   _loss(oracle_mod, {**p, name: am}, dO, dST, **kw)) / (2 * h)
            got = grads[key[name]][ix]
            assert abs(got - num) <= 1e-6 * (1.0 + abs(num)), (name, ix, got, num)


ALL_INPUTS = ("q", "k", "v", "log_alpha", "b", "w", "z", "S0", "gamma")


def test_backward_matches_central_differences(oracle_mod):
    p, dO, dST = _bwd_problem(21)
    g = oracle_mod.backward(**p, dO=dO, dS_T=dST)
    _fd_check(oracle_mod, p, dO, dST, g, ALL_INPUTS, 24, 1)


def test_backward_per_token_gates_scale_and_no_normalisation(oracle_mod):
    p, dO, dST = _bwd_problem(22, per_token=True)
    g = oracle_mod.backward(**p, dO=dO, dS_T=dST)
    assert g["db"].shape == (1, 2, 9) and g["dlog_alpha"].shape == (1, 2, 9)
    _fd_check(oracle_mod, p, dO, dST, g, ("log_alpha", "b", "w", "q", "k"), 18, 2)
    p2, dO2, dST2 = _bwd_problem(23, gain=False)
    g2 = oracle_mod.backward(**p2, dO=dO2, dS_T=dST2, scale=0.7, normalize_qk=False)
    assert g2["dz"] is None and g2["dgamma"] is None
    _fd_check(oracle_mod, p2, dO2, dST2, g2, ("q", "k", "v", "log_alpha", "S0"), 18, 3,
              scale=0.7, normalize_qk=False)


def test_backward_constant_gates_have_no_gradient(oracle_mod):
    p, dO, dST = _bwd_problem(24, gain=False)
    p.update(log_alpha=0.0, b=0.0, w=1.0)
    g = oracle_mod.backward(**p, dO=dO, dS_T=dST)
    assert g["dlog_alpha"] is None and g["db"] is None and g["dw"] is None
    _fd_check(oracle_mod, p, dO, dST, g, ("q", "k", "v", "S0"), 12, 4)


def test_backward_split_resume_across_checkpoints(oracle_mod):
    """Gradients of a 150-token sequence (three checkpoint segments) equal the
    backward of its last 61 tokens, from the state the first 89 leave, whose
    dS0 is then fed as dS_T to the backward of the first 89."""
    p, dO, dST = _bwd_problem(25, T=150, d=6)
    full = oracle_mod.backward(**p, dO=dO, dS_T=dST)
    cut = 89
    head = {n: (a[:, :, :cut] if n not in ("S0", "gamma") else a) for n, a in p.items()}
    tail = {n: (a[:, :, cut:] if n not in ("S0", "gamma") else a) for n, a in p.items()}
    _, s_cut = oracle_mod.forward(**head)
    tail["S0"] = s_cut
    gt = oracle_mod.backward(**tail, dO=dO[:, :, cut:], dS_T=dST)
    gh = oracle_mod.backward(**head, dO=dO[:, :, :cut], dS_T=gt["dS0"])
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dz"):
        np.testing.assert_allclose(np.concatenate([gh[n], gt[n]], axis=2), full[n], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(gh["dS0"], full["dS0"], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(gh["dgamma"] + gt["dgamma"], full["dgamma"], rtol=1e-9, atol=1e-11)


def test_backward_linear_attention_closed_form(oracle_mod):
    """b = 0, alpha = w = 1, no normalisation: o_t = sum_{s<=t} (q_t . k_s) v_s,
    so dv_s = sum_{t>=s} (q_t . k_s) dO_t and dq_t = sum_{s<=t} (dO_t . v_s) k_s."""
    r = np.random.default_rng(26)
    B, H, T, d = 1, 1, 12, 5
    q, k, v = (r.standard_normal((B, H, T, d)) for _ in range(3))
    dO = r.standard_normal((B, H, T, d))
    g = oracle_mod.backward(q, k, v, 0.0, 0.0, 1.0, dO, normalize_qk=False)
    qk = q[0, 0] @ k[0, 0].T                      # [t, s]
    mask = np.tril(np.ones((T, T)))
    np.testing.assert_allclose(g["dv"][0, 0], (qk * mask).T @ dO[0, 0], rtol=1e-12)
    np.testing.assert_allclose(g["dq"][0, 0], ((dO[0, 0] @ v[0, 0].T) * mask) @ k[0, 0], rtol=1e-12)


def test_output_gate_backward_matches_central_differences(oracle_mod):
    """Every gradient of the output gate's backward against central differences
    of output_gate (the forward), with and without a norm weight."""
    r = np.random.default_rng(61)
    B, H, T, dv = 2, 2, 3, 6
    o = r.standard_normal((B, H, T, dv))
    g = r.standard_normal((B, H, T, dv))
    wgt = 1.0 + 0.3 * r.standard_normal((H, dv))
    dy = r.standard_normal((B, T, H, dv))
    eps = 1e-3
    for w_ in (wgt, None):
        do, dg, dw = oracle_mod.output_gate_backward(o, g, dy, norm_weight=w_, eps=eps)
        loss = lambda o_, g_, w2: float(np.sum(dy * oracle_mod.output_gate(o_, g_, norm_weight=w2, eps=eps)))
        h = 1e-6
        for name, x, grad in (("o", o, do), ("g", g, dg)) + ((("w", wgt, dw),) if w_ is not None else ()):
            for idx in [(0, 1, 2, 3), (1, 0, 0, 5), (1, 1, 1, 0)] if x.ndim == 4 else [(0, 2), (1, 5)]:
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"o": (xp, g, w_), "g": (o, xp, w_), "w": (o, g, xp)}[name]
                args_m = {"o": (xm, g, w_), "g": (o, xm, w_), "w": (o, g, xm)}[name]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])

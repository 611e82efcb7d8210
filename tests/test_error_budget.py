"""Where the bf16 matrix paths' error comes from (CPU, no GPU).

A model of the chunked form the two-pass path evaluates, written here in
fp64 torch, with each place the kernels round to bf16 (or hold fp32)
switchable on its own:

  operands  K e^g, K e^-g, Q e^g, K e^{G-g} as matrix operands
  A         the off-diagonal blocks of -Diag(beta) Kg Kn^T
  inverse   the doubling product of the 16x16 diagonal inverses,
            (I - N)(I + N^2)(I + N^4)(I + N^8), and the block forward
            substitution of the off-diagonal blocks of (I + A)^{-1}
  T         T Diag(beta) as the operand of W and U
  P         P = lower(Qg Kn^T)
  W, U      W = T Kg and U = T V as stored operands
  S0 copy   the bf16 copy of the fp32 start state in E = U - W S0 and Qg S0
  E copy    E as the operand of the state update and of P E
  state     the fp32 state between chunks
  output    o in bf16 (round to nearest even)

With every site off the model is the chunked algebra in exact arithmetic
and must equal the fp64 token-loop oracle to ~1e-12 (so the chunked form
itself is pinned against the recurrence).  Each site alone, then all of
them, give the error budget against the bar of the bf16 parity tests
(max-relative 2e-2), at the workloads' gates and at stronger ones (-1 per
token, inside the factored range), and for the blocked form the matrix
paths take beyond that range (per-token gates of -3, channels alternating
0 and -4.5).  The chunk, block and rounding layout
follow the kernels' (C = 64, 16-row blocks); the order of fp32
accumulations inside a product is not modelled (fp64 instead), so the
model bounds the rounding of stored values, which dominates.
"""
import math

import numpy as np
import pytest
import torch

import kda_inputs as gen
import oracle
from kda_testutil import report

C, BLK = 64, 16
SITES = ["operands", "A", "inverse", "T", "P", "W, U", "S0 copy", "E copy", "state", "output"]


def rb(x, on):
    """bf16 round to nearest even when `on`, else unchanged (fp64)."""
    return x.to(torch.bfloat16).to(torch.float64) if on else x


def rf(x, on):
    return x.to(torch.float32).to(torch.float64) if on else x


def diag_inverse(N, on):
    """(I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) for a strictly lower
    16x16 N, with the kernels' bf16 operands when `on`."""
    eye = torch.eye(BLK, dtype=torch.float64)
    Nb = rb(N, on)
    M2 = Nb @ Nb
    M4 = rb(M2, on) @ rb(M2, on)
    M8 = rb(M4, on) @ rb(M4, on)
    Z1 = rb(eye + M8, on) @ rb(eye - N, on)
    Z2 = rb(eye + M4, on) @ rb(Z1, on)
    Z3 = rb(eye + M2, on) @ rb(Z2, on)
    return rb(Z3, on)


def blocked_products(q, k, g, on):
    """B = [k_r . (k_s e^{g_r - g_s})] and Pq = [q_r . (k_s e^{g_r - g_s})] for
    s in the row blocks up to r's, by the blocked form: the decay between r
    (block I) and s splits at rho_I, the cumulative gate before block I, into
    X_I = K_I e^{g - rho_I} (Q_I for Pq) and Y^(I) = K e^{rho_I - g} over the
    rows of blocks 0..I, each rounded to bf16 when `on` (the kernels'
    operands).  Entries with s in a later block stay zero."""
    L = q.shape[0]
    B = torch.zeros((L, L), dtype=torch.float64)
    Pq = torch.zeros((L, L), dtype=torch.float64)
    for I in range((L + BLK - 1) // BLK):
        r0, r1 = BLK * I, min(BLK * (I + 1), L)
        rho = g[r0 - 1] if I > 0 else torch.zeros_like(g[0])
        X = rb(k[r0:r1] * torch.exp(g[r0:r1] - rho), on)
        QX = rb(q[r0:r1] * torch.exp(g[r0:r1] - rho), on)
        Y = rb(k[:r1] * torch.exp(rho - g[:r1]), on)
        B[r0:r1, :r1] = X @ Y.T
        Pq[r0:r1, :r1] = QX @ Y.T
    return B, Pq


def chunk_model(q, k, v, la, beta, S, scale, s, form="factored"):
    """One chunk (rows of one head) through the chunked form; s: the set of
    sites that round; form: how B and P are formed ("factored": Kg Kn^T and
    Qg Kn^T; "blocked": blocked_products).  Returns (o, S_next)."""
    L = q.shape[0]
    g = torch.cumsum(la, 0)                                  # [L, dk] natural units
    G = g[-1]
    Kg = rb(k * torch.exp(g), "operands" in s)
    Kn = rb(k * torch.exp(-g), "operands" in s)
    Qg = rb(q * torch.exp(g), "operands" in s)
    Kd = rb(k * torch.exp(G - g), "operands" in s)
    if form == "blocked":
        B, Pq = blocked_products(q, k, g, "operands" in s)
    else:
        B, Pq = Kg @ Kn.T, Qg @ Kn.T
    A = torch.tril(beta[:, None] * B, -1)                    # (I + A) E = Diag(beta)(V - Kg S0)
    # T = (I + A)^{-1}: diagonal blocks by the doubling product, the rest
    # by block forward substitution with the kernels' roundings
    nb = (L + BLK - 1) // BLK
    Lp = nb * BLK
    Ap = torch.zeros((Lp, Lp), dtype=torch.float64)
    Ap[:L, :L] = A
    An = rb(-Ap, "A" in s)                                   # stored -A blocks
    inv_on = "inverse" in s
    dinv = [diag_inverse(Ap[BLK * I:BLK * (I + 1), BLK * I:BLK * (I + 1)], inv_on)
            for I in range(nb)]
    T = torch.zeros((Lp, Lp), dtype=torch.float64)
    for J in range(nb):
        col = {J: dinv[J]}
        for I in range(J + 1, nb):
            z = torch.zeros((BLK, BLK), dtype=torch.float64)
            for K2 in range(J, I):
                z = z + An[BLK * I:BLK * (I + 1), BLK * K2:BLK * (K2 + 1)] @ rb(col[K2], inv_on)
            col[I] = dinv[I] @ rb(z, inv_on)
        for I in range(J, nb):
            T[BLK * I:BLK * (I + 1), BLK * J:BLK * (J + 1)] = col[I]
    T = T[:L, :L]
    Tb = rb(T * beta[None, :], "T" in s)                     # T Diag(beta)
    W = rb(Tb @ Kg, "W, U" in s)
    U = rb(Tb @ v, "W, U" in s)
    P = rb(torch.tril(Pq), "P" in s)
    S0 = rb(S, "S0 copy" in s)
    E = U - W @ S0
    Eb = rb(E, "E copy" in s)
    o = scale * (Qg @ S0 + P @ Eb)
    S_next = rf(torch.exp(G)[:, None] * S + Kd.T @ Eb, "state" in s)
    return rb(o, "output" in s), S_next


def model_prefill(inp, scale, sites, form="factored"):
    """All sequences and heads of a packed batch through the chunk model."""
    f = lambda t: t.to(torch.float64)
    q, k, v, la, beta = (f(inp[x]) for x in ("q", "k", "v", "log_alpha", "beta"))
    cu = inp["cu_seqlens"].tolist()
    T, H, dk = q.shape
    dv = v.shape[2]
    o = torch.zeros((T, H, dv), dtype=torch.float64)
    hT = torch.zeros((len(cu) - 1, H, dk, dv), dtype=torch.float64)
    for n in range(len(cu) - 1):
        for h in range(H):
            S = torch.zeros((dk, dv), dtype=torch.float64) if inp["h0"] is None \
                else inp["h0"][n, h].to(torch.float64)
            for c0 in range(cu[n], cu[n + 1], C):
                c1 = min(c0 + C, cu[n + 1])
                o[c0:c1, h], S = chunk_model(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h],
                                             la[c0:c1, h], beta[c0:c1, h], S, scale, sites, form)
            hT[n, h] = S
    return o.numpy(), hT.numpy()


def rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def inputs(case):
    inp = gen.prefill_inputs([1024, 300], 2, 128, 128, "bf16",
                             "softplus" if case == "softplus" else "uniform",
                             state_std=0.02, seed=97, device="cpu")
    if case == "decay_1":
        inp["log_alpha"].fill_(-1.0)
    return inp


@pytest.mark.parametrize("case", ["softplus", "uniform", "decay_1"])
def test_error_budget(case):
    inp = inputs(case)
    scale = 1.0 / math.sqrt(128)
    h = lambda t: t.to(torch.float32).numpy()
    o_ref, h_ref = oracle.prefill(h(inp["q"]), h(inp["k"]), h(inp["v"]), h(inp["log_alpha"]),
                                  h(inp["beta"]), h0=h(inp["h0"]),
                                  cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                                  scale=scale)
    # exact arithmetic: the chunked form is the recurrence
    o0, h0_ = model_prefill(inp, scale, set())
    assert rel(o0, o_ref) < 1e-10 and rel(h0_, h_ref) < 1e-10, (rel(o0, o_ref), rel(h0_, h_ref))
    budget = {}
    for site in SITES:
        o1, h1 = model_prefill(inp, scale, {site})
        budget[site] = (rel(o1, o_ref), rel(h1, h_ref))
    o_all, h_all = model_prefill(inp, scale, set(SITES))
    for site, (eo, eh) in budget.items():
        report("budget %s: %s alone" % (case, site), o=eo, hT=eh)
    report("budget %s: every site" % case, o=rel(o_all, o_ref), hT=rel(h_all, h_ref))
    # the whole model stays well inside the bf16 bar, and no single site
    # exceeds the total by much (roundings do not cancel systematically)
    assert rel(o_all, o_ref) <= 1e-2 and rel(h_all, h_ref) <= 1e-2
    assert max(e for e, _ in budget.values()) <= 1.5 * rel(o_all, o_ref) + 1e-4


def strong_inputs(case):
    inp = gen.prefill_inputs([300, 129], 2, 128, 128, "bf16", "uniform", state_std=0.02,
                             seed=98, device="cpu")
    la = inp["log_alpha"]
    if case == "decay_3":
        la.fill_(-3.0)
    else:                        # channels alternating 0 and -4.5: 16-row blocks sum to -72
        la[..., 0::2] = 0.0
        la[..., 1::2] = -4.5
    return inp


@pytest.mark.parametrize("case", ["decay_3", "channels_0_4.5"])
def test_blocked_form_error_budget(case):
    """The blocked form the matrix paths take for chunks beyond the factored
    range (every 16-row block's gate sum still inside it).  In exact
    arithmetic it is the recurrence (pins the per-block factorisation); with
    every bf16 rounding site on it stays well inside the bf16 bar, where the
    factored form's bf16 operands overflow (e^{-g} past bf16's range)."""
    inp = strong_inputs(case)
    scale = 1.0 / math.sqrt(128)
    h = lambda t: t.to(torch.float32).numpy()
    o_ref, h_ref = oracle.prefill(h(inp["q"]), h(inp["k"]), h(inp["v"]), h(inp["log_alpha"]),
                                  h(inp["beta"]), h0=h(inp["h0"]),
                                  cu_seqlens=inp["cu_seqlens"].numpy().astype(np.int64),
                                  scale=scale)
    o0, h0_ = model_prefill(inp, scale, set(), "blocked")
    assert rel(o0, o_ref) < 1e-10 and rel(h0_, h_ref) < 1e-10, (rel(o0, o_ref), rel(h0_, h_ref))
    o1, h1 = model_prefill(inp, scale, set(SITES), "blocked")
    report("budget %s: blocked form, every site" % case, o=rel(o1, o_ref), hT=rel(h1, h_ref))
    assert rel(o1, o_ref) <= 1e-2 and rel(h1, h_ref) <= 1e-2
    of, _ = model_prefill(inp, scale, {"operands"}, "factored")
    assert not np.isfinite(of).all()

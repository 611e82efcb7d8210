"""Pins for the fp64 oracle: each test ties it to something other than itself.

The definition being pinned is the per-token KDA recurrence of "Kimi Delta
Attention: la atencion lineal detras de Kimi K2 y Qwen3", section "Cómo
funciona Kimi Delta Attention paso a paso":
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale * S_t^T q_t,           alpha_t = exp(log_alpha_t).

Pins used (none re-types the oracle's step list):
  * brute force: explicit d_k x d_k transition matrices multiplied out as
    products (no recurrence), plus the diagonal-plus-low-rank form of the
    transition ("Cos'è Kimi Delta Attention (KDA)?", section "Gating per
    canale: cosa rende KDA diverso");
  * the two named ancestors: alpha = 1 is DeltaNet, alpha constant across
    channels is Gated DeltaNet (both pages' lineage tables);
  * closed forms: beta = 0 gives pure channel-wise decay; beta = 1 with a
    unit key reads back exactly the value just written (the "erase, then
    write" reading of the delta rule, "Cos'è Kimi Delta Attention (KDA)?",
    section "La regola delta come memoria associativa"); basis keys give a
    per-row formula;
  * linearity in (v, h0) and in the output scale; the norm bound that unit
    keys give (first page, notes on key normalisation);
  * a hand-derived three-token example (tests/golden/worked_example_d2.json);
  * mutation checks: plausible mistakes planted in a copy of the oracle's C
    source must each fail at least one of the pins above.
"""
import json
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(x):
    """Round to float32 and come back: the exact values the oracle will see."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def rand_case(rng, T, H, dk, dv, unit_keys=True, beta_range=(0.0, 1.0),
              la_range=(-0.3, 0.0)):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = rng.uniform(la_range[0], la_range[1], (T, H, dk))
    beta = rng.uniform(beta_range[0], beta_range[1], (T, H))
    return f32(q), f32(k), f32(v), f32(la), f32(beta)


def transition(k, la, beta):
    """M = (I - beta k k^T) Diag(alpha), built as an explicit matrix."""
    dk = k.shape[0]
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(la))


def brute_force_one_head(q, k, v, la, beta, S0, scale):
    """S_t = M_t...M_1 S0 + sum_{s<=t} M_t...M_{s+1} beta_s k_s v_s^T,
    every product formed explicitly (quadratic in T, no recurrence)."""
    T, dk = k.shape
    Ms = [transition(k[s], la[s], beta[s]) for s in range(T)]
    o = np.zeros((T, v.shape[1]))
    S_t = None
    for t in range(T):
        def prod(a, b):  # M_b ... M_a (b >= a), identity when empty
            P = np.eye(dk)
            for s in range(a, b + 1):
                P = Ms[s] @ P
            return P
        S_t = prod(0, t) @ S0
        for s in range(t + 1):
            S_t = S_t + prod(s + 1, t) @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = scale * S_t.T @ q[t]
    return o, S_t


# --------------------------------------------------------------------------
# brute force and transition structure
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,dk,dv,seed", [(1, 3, 2, 0), (7, 4, 3, 1),
                                          (16, 8, 5, 2), (12, 6, 8, 3)])
def test_brute_force_unrolled_product(T, dk, dv, seed):
    rng = np.random.default_rng(seed)
    H = 2
    q, k, v, la, beta = rand_case(rng, T, H, dk, dv, unit_keys=(seed % 2 == 0))
    h0 = rng.standard_normal((1, H, dk, dv)) * 0.5
    scale = 0.37
    o, hT = oracle.prefill(q, k, v, la, beta, h0=h0, scale=scale)
    for h in range(H):
        ob, Sb = brute_force_one_head(q[:, h], k[:, h], v[:, h], la[:, h],
                                      beta[:, h], h0[0, h], scale)
        assert np.max(np.abs(o[:, h] - ob)) <= 1e-12 * max(1.0, np.max(np.abs(ob)))
        assert np.max(np.abs(hT[0, h] - Sb)) <= 1e-12 * max(1.0, np.max(np.abs(Sb)))


def test_transition_is_diagonal_plus_rank_one():
    """(I - b k k^T) Diag(a) = Diag(a) - b k (a*k)^T: pins the brute force's
    matrix construction to the diagonal-plus-low-rank reading."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        dk = int(rng.integers(1, 9))
        k = rng.standard_normal(dk)
        la = rng.uniform(-1, 0, dk)
        b = rng.uniform(0, 1)
        a = np.exp(la)
        dplr = np.diag(a) - b * np.outer(k, a * k)
        assert np.max(np.abs(transition(k, la, b) - dplr)) < 1e-14


# --------------------------------------------------------------------------
# named special cases
# --------------------------------------------------------------------------
def test_alpha_one_is_deltanet():
    """log alpha = 0 everywhere: plain delta rule S = (I - b k k^T) S + b k v^T."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 40, 3, 8, 6
    q, k, v, la, beta = rand_case(rng, T, H, dk, dv)
    la[:] = 0.0
    o, hT = oracle.prefill(q, k, v, la, beta, scale=1.0)
    # the DeltaNet layout (no gate at all) is the same computation
    o2, hT2 = oracle.prefill(q, k, v, None, beta, scale=1.0)
    assert np.array_equal(o, o2) and np.array_equal(hT, hT2)
    for h in range(H):
        S = np.zeros((dk, dv))
        for t in range(T):
            kk = k[t, h]
            S = S - beta[t, h] * np.outer(kk, kk @ S) + beta[t, h] * np.outer(kk, v[t, h])
            np.testing.assert_allclose(o[t, h], S.T @ q[t, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(hT[0, h], S, rtol=0, atol=1e-13)


def test_scalar_gate_is_gated_deltanet():
    """alpha_t = a_t * 1 on every channel: S = a_t (I - b k k^T) S + b k v^T."""
    rng = np.random.default_rng(12)
    T, H, dk, dv = 40, 2, 8, 4
    q, k, v, la, beta = rand_case(rng, T, H, dk, dv)
    scalar = f32(rng.uniform(-0.2, 0.0, (T, H)))
    la = np.repeat(scalar[:, :, None], dk, axis=2)
    h0 = rng.standard_normal((1, H, dk, dv))
    o, hT = oracle.prefill(q, k, v, la, beta, h0=h0, scale=0.5)
    # the Gated DeltaNet layout ([T, H], one gate per head) is the same computation
    o2, hT2 = oracle.prefill(q, k, v, scalar, beta, h0=h0, scale=0.5)
    assert np.array_equal(o, o2) and np.array_equal(hT, hT2)
    for h in range(H):
        S = h0[0, h].copy()
        for t in range(T):
            kk = k[t, h]
            a = np.exp(scalar[t, h])
            S = a * (S - beta[t, h] * np.outer(kk, kk @ S)) + beta[t, h] * np.outer(kk, v[t, h])
            np.testing.assert_allclose(o[t, h], 0.5 * S.T @ q[t, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(hT[0, h], S, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_beta_zero_is_pure_channel_decay():
    rng = np.random.default_rng(13)
    T, H, dk, dv = 30, 2, 6, 5
    q, k, v, la, beta = rand_case(rng, T, H, dk, dv)
    beta[:] = 0.0
    h0 = rng.standard_normal((1, H, dk, dv))
    o, hT = oracle.prefill(q, k, v, la, beta, h0=h0, scale=0.25)
    g = np.cumsum(la, axis=0)                       # [T, H, dk]
    for h in range(H):
        for t in range(T):
            S_t = np.exp(g[t, h])[:, None] * h0[0, h]
            np.testing.assert_allclose(o[t, h], 0.25 * S_t.T @ q[t, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(hT[0, h], np.exp(g[-1, h])[:, None] * h0[0, h],
                                   rtol=0, atol=1e-13)


def exact_unit_keys(rng, T, H, dk):
    """Keys of exactly unit norm in float32: four entries of +-1/2."""
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            idx = rng.choice(dk, 4, replace=False)
            k[t, h, idx] = rng.choice([-0.5, 0.5], 4)
    return k


def test_beta_one_unit_key_reads_back_value():
    """beta = 1, |k| = 1: the corrected state maps k_t to v_t exactly; with
    q_t = k_t the output is scale * v_t."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 50, 2, 16, 8
    _, _, v, la, beta = rand_case(rng, T, H, dk, dv)
    k = exact_unit_keys(rng, T, H, dk)
    beta[:] = 1.0
    h0 = rng.standard_normal((1, H, dk, dv))
    o, _ = oracle.prefill(k, k, v, la, beta, h0=h0, scale=0.125)
    np.testing.assert_allclose(o, 0.125 * v, rtol=0, atol=1e-13)


def test_basis_keys_row_formula():
    """k_t = e_{i_t}: channel i_t's row becomes (1-b) a S[i] + b v; every
    other row only decays.  Pins the decay axis, the decay-before-predict
    order and the sign of the correction."""
    rng = np.random.default_rng(15)
    T, H, dk, dv = 60, 2, 5, 3
    _, _, v, la, beta = rand_case(rng, T, H, dk, dv)
    q = f32(rng.standard_normal((T, H, dk)))
    idx = rng.integers(0, dk, (T, H))
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            k[t, h, idx[t, h]] = 1.0
    h0 = rng.standard_normal((1, H, dk, dv))
    o, hT = oracle.prefill(q, k, v, la, beta, h0=h0, scale=1.0)
    for h in range(H):
        rows = [h0[0, h, c].copy() for c in range(dk)]
        for t in range(T):
            a = np.exp(la[t, h])
            rows = [a[c] * rows[c] for c in range(dk)]
            i = idx[t, h]
            rows[i] = (1 - beta[t, h]) * rows[i] + beta[t, h] * v[t, h]
            expect_o = sum(q[t, h, c] * rows[c] for c in range(dk))
            np.testing.assert_allclose(o[t, h], expect_o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(hT[0, h], np.stack(rows), rtol=0, atol=1e-13)


def test_worked_example_golden():
    with open(os.path.join(HERE, "golden", "worked_example_d2.json")) as f:
        ex = json.load(f)
    T = len(ex["beta"])
    q = np.array(ex["q"], dtype=np.float64).reshape(T, 1, 2)
    k = np.array(ex["k"], dtype=np.float64).reshape(T, 1, 2)
    v = np.array(ex["v"], dtype=np.float64).reshape(T, 1, 2)
    la = np.log(np.array(ex["alpha"], dtype=np.float64)).reshape(T, 1, 2)
    beta = np.array(ex["beta"], dtype=np.float64).reshape(T, 1)
    o, hT = oracle.prefill(q, k, v, la, beta, scale=ex["scale"])
    tol = ex["tolerance"]
    np.testing.assert_allclose(o[:, 0], np.array(ex["expected_o"]), rtol=0, atol=tol)
    np.testing.assert_allclose(hT[0, 0], np.array(ex["expected_hT"]), rtol=0, atol=tol)


# --------------------------------------------------------------------------
# structural properties
# --------------------------------------------------------------------------
def test_linear_in_values_and_initial_state():
    """(o, hT) is jointly linear in (v, h0) for fixed q, k, alpha, beta.
    Values are multiples of 1/256, so the mixed values stay exact in float32."""
    rng = np.random.default_rng(16)
    T, H, dk, dv = 25, 2, 6, 4
    q, k, _, la, beta = rand_case(rng, T, H, dk, dv)
    v1 = np.round(rng.standard_normal((T, H, dv)) * 256) / 256
    v2 = np.round(rng.standard_normal((T, H, dv)) * 256) / 256
    h1 = rng.standard_normal((1, H, dk, dv))
    h2 = rng.standard_normal((1, H, dk, dv))
    a, b = 0.75, -1.25
    o1, s1 = oracle.prefill(q, k, v1, la, beta, h0=h1)
    o2, s2 = oracle.prefill(q, k, v2, la, beta, h0=h2)
    vmix = a * v1 + b * v2
    assert np.array_equal(f32(vmix), vmix)
    o3, s3 = oracle.prefill(q, k, vmix, la, beta, h0=a * h1 + b * h2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + b * s2, rtol=0, atol=1e-12)
    o0, s0 = oracle.prefill(q, k, np.zeros_like(v1), la, beta, h0=np.zeros_like(h1))
    assert not o0.any() and not s0.any()


def test_output_scale_is_linear_and_state_independent():
    rng = np.random.default_rng(17)
    q, k, v, la, beta = rand_case(rng, 20, 2, 6, 6)
    o1, s1 = oracle.prefill(q, k, v, la, beta, scale=1.0)
    o2, s2 = oracle.prefill(q, k, v, la, beta, scale=0.3)
    np.testing.assert_allclose(o2, 0.3 * o1, rtol=1e-14, atol=1e-15)
    assert np.array_equal(s1, s2)


def test_unit_key_norm_bound():
    """Unit keys, beta in [0,1], alpha in (0,1]: ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    rng = np.random.default_rng(18)
    T, dk, dv = 80, 8, 8
    q, k, v, la, beta = rand_case(rng, T, 1, dk, dv)
    h0 = rng.standard_normal((1, 1, dk, dv)) * 3
    prev = np.linalg.norm(h0)
    for t in range(T):
        cu = np.array([0, t + 1])
        _, hT = oracle.prefill(q[:t + 1], k[:t + 1], v[:t + 1], la[:t + 1],
                               beta[:t + 1], h0=h0, cu_seqlens=cu)
        cur = np.linalg.norm(hT)
        assert cur <= prev + beta[t, 0] * np.linalg.norm(v[t, 0]) + 1e-12
        prev = cur


def test_varlen_equals_separate_sequences_and_empty_ones():
    rng = np.random.default_rng(19)
    lens = [5, 0, 9, 1, 0, 14]
    T = sum(lens)
    H, dk, dv = 2, 4, 3
    q, k, v, la, beta = rand_case(rng, T, H, dk, dv)
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, hT = oracle.prefill(q, k, v, la, beta, h0=h0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        on, hn = oracle.prefill(q[a:b], k[a:b], v[a:b], la[a:b], beta[a:b],
                                h0=h0[n:n + 1], cu_seqlens=[0, L])
        assert np.array_equal(o[a:b], on)
        assert np.array_equal(hT[n], hn[0])
        if L == 0:
            assert np.array_equal(hT[n], h0[n])


def test_decode_step_equals_one_token_prefill():
    rng = np.random.default_rng(20)
    N, H, dk, dv = 3, 2, 6, 5
    q, k, v, la, beta = rand_case(rng, N, H, dk, dv)
    S = rng.standard_normal((N, H, dk, dv))
    o, S1 = oracle.decode_step(q, k, v, la, beta, S, scale=0.7)
    cu = np.arange(N + 1)
    o2, S2 = oracle.prefill(q, k, v, la, beta, h0=S, cu_seqlens=cu, scale=0.7)
    assert np.array_equal(o, o2)
    assert np.array_equal(S1, S2)
    # gate layouts: a per-head gate and no gate, against their expanded forms
    g = f32(rng.uniform(-0.3, 0.0, (N, H)))
    oh, Sh = oracle.decode_step(q, k, v, g, beta, S, scale=0.7)
    oe, Se = oracle.decode_step(q, k, v, np.repeat(g[:, :, None], dk, axis=2), beta, S, scale=0.7)
    assert np.array_equal(oh, oe) and np.array_equal(Sh, Se)
    on, Sn = oracle.decode_step(q, k, v, None, beta, S, scale=0.7)
    oz, Sz = oracle.decode_step(q, k, v, np.zeros_like(la), beta, S, scale=0.7)
    assert np.array_equal(on, oz) and np.array_equal(Sn, Sz)


def _chained_decode(q, k, v, la, beta, S, lengths, scale):
    """Several decode tokens per sequence, one decode_step call per token
    and per sequence (no re-indexing of a packed batch): the plain meaning of
    applying a sequence's first lengths[n] tokens in order."""
    N, m, H = q.shape[:3]
    dv = v.shape[-1]
    o = np.full((N, m, H, dv), np.nan)
    S_out = np.array(S, dtype=np.float64, copy=True)
    for n in range(N):
        L = m if lengths is None else min(max(int(lengths[n]), 0), m)
        Sn = S_out[n:n + 1]
        for t in range(L):
            g = None if la is None else la[n:n + 1, t]
            o[n, t], Sn = oracle.decode_step(q[n:n + 1, t], k[n:n + 1, t], v[n:n + 1, t], g,
                                             beta[n:n + 1, t], Sn, scale=scale)
        S_out[n:n + 1] = Sn
    return o, S_out


def _decode_multi_matches_chain(mod, gate, lengths, seed):
    rng = np.random.default_rng(seed)
    N, m, H, dk, dv = 6, 4, 2, 5, 3
    q, k, v, la, beta = rand_case(rng, N * m, H, dk, dv)
    shp = lambda x: x.reshape((N, m) + x.shape[1:])
    q, k, v, la, beta = shp(q), shp(k), shp(v), shp(la), shp(beta)
    if gate == "head":
        la = f32(rng.uniform(-0.4, 0.0, (N, m, H)))
    elif gate == "none":
        la = None
    S = rng.standard_normal((N, H, dk, dv))
    o, S1 = mod.decode_multi(q, k, v, la, beta, S, lengths=lengths, scale=0.6)
    oc, Sc = _chained_decode(q, k, v, la, beta, S, lengths, 0.6)
    same_nan = np.array_equal(np.isnan(o), np.isnan(oc))
    return (same_nan and np.array_equal(np.nan_to_num(o), np.nan_to_num(oc))
            and np.array_equal(S1, Sc))


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("lengths", [None, [-2, 0, 1, 3, 4, 9], [4, 4, 0, 2, 1, 3]])
def test_decode_multi_equals_chained_decode_steps(gate, lengths):
    """decode_multi re-indexes [N, m, H, .] tokens into a packed prefill;
    it must equal one decode_step per token and sequence: all m tokens
    without lengths, the first clamp(lengths[n], 0, m) otherwise, NaN in the
    rows of tokens not applied, the state untouched for a sequence that
    applies none ("Kimi Linear acaba de superar a la atención completa en sus
    propios términos", section "Qué observar tras el lanzamiento de Kimi
    Linear": verifying and committing draft tokens must give the tokens'
    own recurrence)."""
    assert _decode_multi_matches_chain(oracle, gate, lengths, seed=31)


# planted mistakes in the re-indexing wrapper (oracle/__init__.py)
WRAPPER_MUTANTS = {
    "clamp one short": ("np.clip(np.asarray(lengths, dtype=np.int64), 0, m)",
                        "np.clip(np.asarray(lengths, dtype=np.int64), 0, m - 1)", 1),
    "tokens taken sequence-minor": ("take = np.concatenate([n * m + np.arange(lens[n]) for n in range(N)])",
                                    "take = np.concatenate([np.arange(lens[n]) * N + n for n in range(N)])", 1),
    "outputs scattered to the first rows": ("o[take] = o_t", "o[:len(take)] = o_t", 1),
    "head gate read as the first channel of a per-channel gate":
        ("if la is not None and la.shape[-1] == 1 and np.asarray(log_alpha).ndim == 3:",
         "if False:", 1),
}


def test_decode_multi_planted_mistakes_are_caught(tmp_path):
    """Each planted mistake in decode_multi's re-indexing fails the chained
    comparison above for at least one gate layout and length vector."""
    import importlib.util
    here = os.path.dirname(oracle.__file__)
    src = open(oracle.__file__).read()
    for name, (old, new, count) in WRAPPER_MUTANTS.items():
        assert src.count(old) == count, "mutation anchor not found: " + name
        d = tmp_path / re.sub(r"\W+", "_", name)
        d.mkdir()
        (d / "__init__.py").write_text(src.replace(old, new))
        for f in ("libkda_oracle.so",):
            os.symlink(os.path.join(here, f), d / f)
        spec = importlib.util.spec_from_file_location("dm_mutant_" + d.name, str(d / "__init__.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        caught = False
        for gate in ("channel", "head", "none"):
            for lengths in ([-2, 0, 1, 3, 4, 9], [4, 4, 0, 2, 1, 3]):
                try:
                    ok = _decode_multi_matches_chain(mod, gate, lengths, seed=31)
                except Exception:
                    ok = False
                caught |= not ok
        assert caught, "planted mistake not caught: " + name


# --------------------------------------------------------------------------
# mutation checks: planted mistakes must be caught by the pins above
# --------------------------------------------------------------------------
MUTANTS = {
    "error sign flipped": ("w[j] = beta * ((double)v[j] - u[j]);",
                           "w[j] = beta * ((double)v[j] + u[j]);", 1),
    "beta dropped": ("w[j] = beta * (", "w[j] = 1.0 * (", 1),
    "decay exponent sign": ("const double ac = exp((double)log_alpha[c]);",
                            "const double ac = exp(-(double)log_alpha[c]);", 2),
    "predict with the query": ("u[j] += (ac * row[j]) * kc;",
                               "u[j] += (ac * row[j]) * (double)q[c];", 1),
    "predict from the undecayed state": ("u[j] += (ac * row[j]) * kc;",
                                         "u[j] += row[j] * kc;", 1),
    "correction term dropped": ("const double s = ac * row[j] + kc * w[j];",
                                "const double s = ac * row[j] + 0.0 * kc * w[j];", 1),
    "read before the update": ("row[j] = s;\n            o[j] += s * qc;",
                               "o[j] += row[j] * qc;\n            row[j] = s;", 1),
    "scale dropped": ("o[j] *= scale;", "o[j] *= 1.0;", 1),
    "initial state ignored": ("if (J->h0) memcpy", "if (0) memcpy", 1),
    "last token dropped": ("t < J->cu_seqlens[n + 1]; ++t", "t + 1 < J->cu_seqlens[n + 1]; ++t", 1),
    "decay indexed by value channel": ("const double s = ac * row[j] + kc * w[j];",
                                       "const double s = exp((double)log_alpha[j]) * row[j] + kc * w[j];", 1),
}


def _pins_pass(mod):
    """Run a compact version of the pins against oracle module ``mod``;
    return False as soon as one fails."""
    rng = np.random.default_rng(7)
    T, H, dk, dv = 9, 2, 6, 4          # dk > dv keeps the planted index bug in bounds
    q, k, v, la, beta = rand_case(rng, T, H, dk, dv)
    h0 = rng.standard_normal((1, H, dk, dv))
    o, hT = mod.prefill(q, k, v, la, beta, h0=h0, scale=0.37)
    for h in range(H):
        ob, Sb = brute_force_one_head(q[:, h], k[:, h], v[:, h], la[:, h],
                                      beta[:, h], h0[0, h], 0.37)
        if np.max(np.abs(o[:, h] - ob)) > 1e-10 or np.max(np.abs(hT[0, h] - Sb)) > 1e-10:
            return False
    return True


def test_planted_mistakes_are_caught(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")).read()
    assert _pins_pass(oracle)
    for name, (old, new, count) in MUTANTS.items():
        assert src.count(old) == count, "mutation anchor not found: " + name
        mutated = src.replace(old, new)
        d = tmp_path / re.sub(r"\W+", "_", name)
        d.mkdir()
        (d / "kda_oracle.c").write_text(mutated)
        # a throwaway copy of the oracle package pointing at the mutant
        init = open(oracle.__file__).read()
        (d / "__init__.py").write_text(init)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                        str(d / "kda_oracle.c"), "-o", str(d / "libkda_oracle.so"),
                        "-lm"], check=True)
        import importlib.util
        spec = importlib.util.spec_from_file_location("mutant_" + d.name,
                                                      str(d / "__init__.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        assert not _pins_pass(mod), "planted mistake not caught: " + name


# --------------------------------------------------------------------------
# the fused input front-end's activations
# --------------------------------------------------------------------------
def test_front_end_closed_forms():
    """softplus(0) = ln 2 and sigmoid(0) = 1/2; softplus(x) - softplus(-x) = x
    and sigmoid(y) + sigmoid(-y) = 1 (both follow from e^x / (1 + e^x) =
    1 - 1 / (1 + e^x)); softplus equals log(1 + e^x) where that form is
    exact enough; the normalised rows have unit norm and do not change when
    q, k are scaled."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((50, 3, 4)) * 4
    z = np.zeros((1, 1, 2))
    _, _, la0, b0 = oracle.front_end(z, z, gate_pre=z, beta_pre=z[..., 0], gate_scale=1.0,
                                     l2norm=False)
    assert np.allclose(la0, -np.log(2.0), rtol=0, atol=1e-15)
    assert np.allclose(b0, 0.5, rtol=0, atol=1e-15)
    q = rng.standard_normal((50, 3, 8))
    _, _, lp, bp = oracle.front_end(q, q, gate_pre=x, beta_pre=x[..., 0], gate_scale=0.3)
    _, _, lm, bm = oracle.front_end(q, q, gate_pre=-x, beta_pre=-x[..., 0], gate_scale=0.3)
    assert np.allclose(lp - lm, -0.3 * x, rtol=0, atol=1e-12)
    assert np.allclose(bp + bm, 1.0, rtol=0, atol=1e-14)
    small = np.abs(x) < 20
    assert np.allclose(lp[small], -0.3 * np.log(1.0 + np.exp(x[small])), rtol=1e-12, atol=1e-14)
    qn, kn, _, _ = oracle.front_end(q, 2.5 * q)
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(qn, kn, atol=1e-15)
    qs, _, _, _ = oracle.front_end(7.0 * q, q)
    assert np.allclose(qs, qn, atol=1e-15)


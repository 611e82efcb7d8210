"""Pins for the gradient oracle (oracle.backward): each ties it to something
other than its own derivation.

The gradients are those of L = <o, dO> + <hT, dhT> for the per-token KDA
recurrence of "Kimi Delta Attention: la atencion lineal detras de Kimi K2 y
Qwen3", section "Cómo funciona Kimi Delta Attention paso a paso".

  * finite differences of the (already pinned) forward oracle: central
    differences along random directions, for every input (q, k, v,
    log_alpha, beta, h0) on ragged packed batches with all three gate
    layouts;
  * closed forms of a one-token sequence from a zero state, worked out by
    hand from S_1 = beta k v^T, o = scale beta (k.q) v, plus the transposed
    one-token transition for dh0 from a non-zero state;
  * mutation checks: plausible mistakes planted in a copy of the gradient
    oracle's C source must each fail the finite-difference pin.
"""
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle


def f32(x):
    return np.asarray(x, dtype=np.float32)


def case(rng, lens, H, dk, dv, gate="channel"):
    T = int(sum(lens))
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    if gate == "channel":
        la = f32(-rng.uniform(0.01, 0.3, (T, H, dk)))
    elif gate == "head":
        la = f32(-rng.uniform(0.01, 0.3, (T, H)))
    else:
        la = None
    beta = rng.uniform(0.0, 1.0, (T, H))
    N = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(q=f32(q), k=f32(k), v=f32(v), la=la, beta=f32(beta),
                h0=rng.standard_normal((N, H, dk, dv)), cu=cu,
                do=rng.standard_normal((T, H, dv)), dhT=rng.standard_normal((N, H, dk, dv)))


def loss(mod, c, **over):
    x = dict(c)
    x.update(over)
    o, hT = mod.prefill(x["q"], x["k"], x["v"], x["la"], x["beta"], h0=x["h0"],
                        cu_seqlens=x["cu"], scale=0.4)
    return float((o * c["do"]).sum() + (hT * c["dhT"]).sum())


GRAD = {"q": "dq", "k": "dk", "v": "dv", "la": "dlog_alpha", "beta": "dbeta", "h0": "dh0"}


def fd_errors(mod, c, rng, eps=1e-3):
    """Relative mismatch of <grad, delta> against central differences of the
    forward oracle, per input.  Inputs the oracle reads as float32 are
    perturbed in float32, and the perturbation actually represented is the
    one used."""
    g = mod.backward(c["q"], c["k"], c["v"], c["la"], c["beta"], c["do"], h0=c["h0"],
                     dhT=c["dhT"], cu_seqlens=c["cu"], scale=0.4)
    errs = {}
    for name, gname in GRAD.items():
        if c[name] is None:
            assert g[gname] is None
            continue
        x = np.asarray(c[name], dtype=np.float64)
        d = rng.standard_normal(x.shape)
        if name == "h0":
            xp, xm = x + eps * d, x - eps * d
        else:
            xp, xm = f32(x + eps * d), f32(x - eps * d)
        fd = (loss(mod, c, **{name: xp}) - loss(mod, c, **{name: xm})) / 2.0
        an = float((g[gname] * (np.asarray(xp, np.float64) - np.asarray(xm, np.float64)) / 2.0).sum())
        errs[name] = abs(fd - an) / max(abs(an), 1e-12)
    return errs


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
def test_finite_differences(gate):
    rng = np.random.default_rng(11)
    c = case(rng, [70, 0, 1, 150], 2, 8, 6, gate)
    for name, e in fd_errors(oracle, c, rng).items():
        assert e < 1e-4, (name, e)


def test_finite_differences_square_head():
    rng = np.random.default_rng(12)
    c = case(rng, [129], 1, 16, 16)
    for name, e in fd_errors(oracle, c, rng).items():
        assert e < 1e-4, (name, e)


def test_one_token_closed_form():
    """One token from a zero state: S_1 = beta k v^T, o = scale beta (k.q) v,
    so with L = <o, dO> + <S_1, dhT>:
      dq = scale beta (v.dO) k,          dk = scale beta (v.dO) q + beta dhT v,
      dv = scale beta (k.q) dO + beta dhT^T k,
      dbeta = scale (k.q)(v.dO) + k^T dhT v,  dlog_alpha = 0 (nothing decays)."""
    rng = np.random.default_rng(13)
    dk, dv, scale = 5, 3, 0.7
    q, k, v = (f32(rng.standard_normal(n)).astype(np.float64) for n in (dk, dk, dv))
    b = float(f32(0.6))
    la = f32(-rng.uniform(0.01, 0.5, dk))
    dO = rng.standard_normal(dv)
    dhT = rng.standard_normal((dk, dv))
    g = oracle.backward(q[None, None], k[None, None], v[None, None], la[None, None],
                        np.array([[b]]), dO[None, None], dhT=dhT[None, None], scale=scale)
    kq, vdo = k @ q, v @ dO
    assert np.allclose(g["dq"][0, 0], scale * b * vdo * k, atol=1e-13)
    assert np.allclose(g["dk"][0, 0], scale * b * vdo * q + b * dhT @ v, atol=1e-13)
    assert np.allclose(g["dv"][0, 0], scale * b * kq * dO + b * dhT.T @ k, atol=1e-13)
    assert np.isclose(g["dbeta"][0, 0], scale * kq * vdo + k @ dhT @ v, atol=1e-13)
    assert np.allclose(g["dlog_alpha"], 0.0, atol=1e-15)


def test_one_token_dh0_is_transposed_transition():
    """dh0 of one token = M^T (dhT + scale q dO^T), M = (I - beta k k^T)
    Diag(alpha) the token's transition: the adjoint of a linear map."""
    rng = np.random.default_rng(14)
    dk, dv, scale = 6, 4, 0.5
    q, k = (f32(rng.standard_normal(dk)).astype(np.float64) for _ in range(2))
    v = f32(rng.standard_normal(dv)).astype(np.float64)
    la = f32(-rng.uniform(0.01, 0.5, dk)).astype(np.float64)
    b = float(f32(0.3))
    dO, dhT = rng.standard_normal(dv), rng.standard_normal((dk, dv))
    h0 = rng.standard_normal((dk, dv))
    g = oracle.backward(q[None, None], k[None, None], v[None, None], la[None, None],
                        np.array([[b]]), dO[None, None], h0=h0[None, None],
                        dhT=dhT[None, None], scale=scale)
    M = (np.eye(dk) - b * np.outer(k, k)) @ np.diag(np.exp(la))
    assert np.allclose(g["dh0"][0, 0], M.T @ (dhT + scale * np.outer(q, dO)), atol=1e-12)


# --------------------------------------------------------------------------
# mutation checks
# --------------------------------------------------------------------------
MUTANTS = {
    "read adjoint not added": ("L[c * dv + j] += J->scale * (double)q[c] * dO[j];",
                               "L[c * dv + j] += 0.0 * (double)q[c] * dO[j];", 1),
    "dq from the state before the token": ("acc += S[c * dv + j] * dO[j];",
                                           "acc += segS[i * SE + c * dv + j] * dO[j];", 1),
    "dbeta from the error, not the residual": ("db += dw[j] * r[j];", "db += dw[j] * w[j];", 1),
    "predict term of dk dropped": ("dkc += D[c * dv + j] * du;",
                                   "dkc += 0.0 * D[c * dv + j] * du;", 1),
    "state adjoint not decayed": ("L[c * dv + j] = a * dD[c * dv + j];",
                                  "L[c * dv + j] = dD[c * dv + j];", 1),
    "gate gradient from the undecayed state": ("g += dD[c * dv + j] * D[c * dv + j];",
                                               "g += dD[c * dv + j] * segS[i * SE + c * dv + j];", 1),
    "dhT ignored": ("if (J->dhT) memcpy", "if (0) memcpy", 1),
}


def _pins_pass(mod):
    rng = np.random.default_rng(15)
    c = case(rng, [40, 90], 1, 6, 5)
    if any(e > 1e-4 for e in fd_errors(mod, c, rng).values()):
        return False
    return True


def test_planted_mistakes_are_caught(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    here = os.path.dirname(oracle.__file__)
    src = open(os.path.join(here, "kda_oracle_bwd.c")).read()
    assert _pins_pass(oracle)
    import importlib.util
    for name, (old, new, count) in MUTANTS.items():
        assert src.count(old) == count, "mutation anchor not found: " + name
        d = tmp_path / re.sub(r"\W+", "_", name)
        d.mkdir()
        # a throwaway copy of the oracle package: the forward untouched, the
        # gradient source mutated
        shutil.copy(os.path.join(here, "kda_oracle.c"), d / "kda_oracle.c")
        (d / "kda_oracle_bwd.c").write_text(src.replace(old, new))
        (d / "__init__.py").write_text(open(oracle.__file__).read())
        for s, lib in (("kda_oracle.c", "libkda_oracle.so"),
                       ("kda_oracle_bwd.c", "libkda_oracle_bwd.so")):
            subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                            str(d / s), "-o", str(d / lib), "-lm"], check=True)
        spec = importlib.util.spec_from_file_location("bwd_mutant_" + d.name, str(d / "__init__.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        assert not _pins_pass(mod), "planted mistake not caught: " + name

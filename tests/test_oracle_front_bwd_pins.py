"""Pins for the chain rule through the fused input front-end
(oracle.front_end_backward), each against finite differences of functions
already pinned elsewhere:

  * the front-end alone: central differences of oracle.front_end along
    random directions, for raw q and k (rows of several norms), the gate
    pre-activations (per channel and per head) and the beta
    pre-activations; rows below the normalisation floor, where the divisor
    is the constant eps, separately (closed form dx_n / eps, and central
    differences with steps that stay below the floor);
  * the composition with the recurrence: L = <o, dO> + <hT, dhT> for the
    prefill of the front-end's outputs, differentiated numerically along
    random directions of the raw inputs, against front_end_backward applied
    to the gradient oracle's gradients;
  * mutation checks: each plausible mistake planted in a copy of
    front_end_backward fails one of the first two pins.
"""
import inspect

import numpy as np
import pytest

import oracle

EPS = 1e-6


def raw_case(rng, T, H, d, gate="channel"):
    q = rng.standard_normal((T, H, d)) * rng.uniform(0.3, 3.0, (T, H, 1))
    k = rng.standard_normal((T, H, d)) * rng.uniform(0.3, 3.0, (T, H, 1))
    # a few rows below the normalisation floor
    q[0, 0] *= 1e-8
    k[-1, -1] *= 1e-8
    g = rng.standard_normal((T, H, d) if gate == "channel" else (T, H)) * 2.0
    y = rng.standard_normal((T, H)) * 2.0
    return q, k, g, y


def fe_loss(q, k, g, y, w, c, l2norm=True):
    qn, kn, la, b = oracle.front_end(q, k, g, y, gate_scale=c, l2norm=l2norm, eps=EPS)
    return float((qn * w[0]).sum() + (kn * w[1]).sum() + (la * w[2]).sum() + (b * w[3]).sum())


def fe_fd_errors(fn, gate="channel", l2norm=True, seed=21):
    rng = np.random.default_rng(seed)
    T, H, d, c = 7, 2, 6, 0.3
    q, k, g, y = raw_case(rng, T, H, d, gate)
    w = [rng.standard_normal(x.shape) for x in (q, k, g, y)]
    dq, dk, dg, dy = fn(q, k, g, y, w[0], w[1], w[2], w[3], gate_scale=c, l2norm=l2norm, eps=EPS)
    errs = {}
    for name, idx in (("q", 0), ("k", 1), ("gate_pre", 2), ("beta_pre", 3)):
        args = [q, k, g, y]
        x = args[idx]
        h = 1e-6
        dirn = rng.standard_normal(x.shape)
        if name in ("q", "k"):
            # rows below the floor have their own pin (a step this size
            # would cross the floor there)
            dirn[np.linalg.norm(x, axis=-1) <= EPS] = 0.0
        ap, am = list(args), list(args)
        ap[idx], am[idx] = x + h * dirn, x - h * dirn
        fd = (fe_loss(*ap, w, c, l2norm) - fe_loss(*am, w, c, l2norm)) / (2 * h)
        an = float(((dq, dk, dg, dy)[idx] * dirn).sum())
        errs[name] = abs(fd - an) / max(abs(an), 1e-12)
    return errs


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("l2norm", [True, False])
def test_front_end_finite_differences(gate, l2norm):
    for name, e in fe_fd_errors(oracle.front_end_backward, gate, l2norm).items():
        assert e < 1e-5, (name, e)


def sub_floor_error(fn):
    """Below the floor the divisor is the constant eps, so the map is x / eps
    and its gradient dx_n / eps; relative mismatch of fn against central
    differences of front_end with steps that stay below the floor."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((1, 1, 4)) * 1e-8
    dxn = rng.standard_normal((1, 1, 4))
    dq, _, _, _ = fn(x, x, None, None, dxn, dxn, None, None, eps=EPS)
    dirn = rng.standard_normal(x.shape)
    h = 1e-10
    f = lambda x_: float((oracle.front_end(x_, x_, eps=EPS)[0] * dxn).sum())
    fd = (f(x + h * dirn) - f(x - h * dirn)) / (2 * h)
    return abs(fd - float((dq * dirn).sum())) / abs(fd)


def test_sub_floor_row_scales_by_the_floor():
    x = np.full((1, 1, 4), 1e-9)
    dxn = np.array([[[1.0, -2.0, 0.5, 3.0]]])
    dq, _, _, _ = oracle.front_end_backward(x, x, None, None, dxn, dxn, None, None, eps=EPS)
    assert np.allclose(dq, dxn / EPS, rtol=1e-14)
    assert sub_floor_error(oracle.front_end_backward) < 1e-6


def test_composition_with_the_recurrence():
    rng = np.random.default_rng(22)
    lens, H, d, c, scale = [37, 0, 1, 50], 2, 8, 0.2, 0.4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k, g, y = raw_case(rng, T, H, d)
    q[0, 0] /= 1e-8          # keep every row above the floor here
    k[-1, -1] /= 1e-8
    v = rng.standard_normal((T, H, d))
    h0 = rng.standard_normal((len(lens), H, d, d)) * 0.1
    dO = rng.standard_normal((T, H, d))
    dhT = rng.standard_normal((len(lens), H, d, d))

    def loss(q_, k_, g_, y_):
        qn, kn, la, b = oracle.front_end(q_, k_, g_, y_, gate_scale=c)
        o, hT = oracle.prefill(qn, kn, v, la, b, h0=h0, cu_seqlens=cu, scale=scale)
        return float((o * dO).sum() + (hT * dhT).sum())

    qn, kn, la, b = oracle.front_end(q, k, g, y, gate_scale=c)
    grads = oracle.backward(qn, kn, v, la, b, dO, h0=h0, dhT=dhT, cu_seqlens=cu, scale=scale)
    dq, dk, dg, dy = oracle.front_end_backward(q, k, g, y, grads["dq"], grads["dk"],
                                               grads["dlog_alpha"], grads["dbeta"], gate_scale=c)
    # the recurrence oracle reads float32: step sizes well above its rounding
    for idx, an_grad in enumerate((dq, dk, dg, dy)):
        args = [q, k, g, y]
        dirn = rng.standard_normal(args[idx].shape)
        h = 1e-3
        ap, am = list(args), list(args)
        ap[idx], am[idx] = args[idx] + h * dirn, args[idx] - h * dirn
        fd = (loss(*ap) - loss(*am)) / (2 * h)
        an = float((an_grad * dirn).sum())
        assert abs(fd - an) <= 2e-3 * max(abs(an), 1.0), (idx, fd, an)


MUTANTS = {
    "projection dropped": ("(dxn - xn * proj) / n", "dxn / n"),
    "divided by the norm twice": ("(dxn - xn * proj) / n", "(dxn - xn * proj) / (n * n)"),
    "softplus derivative as sigmoid(-g)": ("-gate_scale / (1.0 + np.exp(-g))", "-gate_scale / (1.0 + np.exp(g))"),
    "gate scale sign": ("-gate_scale / (1.0 + np.exp(-g))", "gate_scale / (1.0 + np.exp(-g))"),
    "sigmoid derivative as beta": ("b * (1.0 - b) * np.asarray(dbeta", "b * np.asarray(dbeta"),
    "floor branch not scaled": ("dxn / eps)", "dxn)"),
}


def pins_pass(fn):
    return max(fe_fd_errors(fn).values()) < 1e-5 and sub_floor_error(fn) < 1e-6


def test_planted_mistakes_are_caught():
    src = inspect.getsource(oracle.front_end_backward)
    assert pins_pass(oracle.front_end_backward)
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, "mutation anchor not found: " + name
        ns = {"np": np}
        exec(src.replace(old, new), ns)
        assert not pins_pass(ns["front_end_backward"]), "planted mistake not caught: " + name

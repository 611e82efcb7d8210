"""fp64 CPU oracle for the Kimi Delta Attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
product path (``gated_delta_rule_05_amd``) never imports it, and this package
imports nothing from there.

The arithmetic lives in ``kda_oracle.c``: the per-token recurrence
S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, o_t = scale S_t^T q,
in double precision ("Kimi Delta Attention: la atencion lineal detras de Kimi
K2 y Qwen3", section "Cómo funciona Kimi Delta Attention paso a paso"; the
diagonal-plus-low-rank transition of "Cos'è Kimi Delta Attention (KDA)?",
section "Gating per canale: cosa rende KDA diverso").  This module only builds that file with gcc and
marshals numpy arrays into it.

The gradients live in ``kda_oracle_bwd.c``: the reverse-mode derivative of
the same token loop, step by step in reverse order (``backward`` below).
The fused input front-end's activations (``front_end``) and the chain rule
through them (``front_end_backward``) are numpy, in float64.

Pins (the tests that tie this oracle to something other than itself) live in
``tests/test_oracle_pins.py`` and, for the gradients,
``tests/test_oracle_bwd_pins.py``: a brute-force product of explicit transition
matrices, the DeltaNet and Gated DeltaNet special cases, the beta = 0 closed
form, the beta = 1 read-back, the basis-key closed form, linearity, the
stability bound and a hand-derived worked example; the several-token
decode wrapper is pinned against one decode_step per token and sequence; the
front-end's chain rule is pinned by finite differences in
``tests/test_oracle_front_bwd_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_BWD_SRC = os.path.join(_HERE, "kda_oracle_bwd.c")
_BWD_LIB = os.path.join(_HERE, "libkda_oracle_bwd.so")
_lib = None
_bwd_lib = None


def _gcc(src, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(force: bool = True) -> str:
    """Compile kda_oracle.c (forward) and kda_oracle_bwd.c (gradients) into
    their shared libraries with gcc (host only)."""
    if force or not os.path.exists(_LIB):
        _gcc(_SRC, _LIB)
    if os.path.exists(_BWD_SRC) and (force or not os.path.exists(_BWD_LIB)):
        _gcc(_BWD_SRC, _BWD_LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.kdaref_prefill.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p, i64p,
                                       i64, i64, i64, i64, ctypes.c_double,
                                       f64p, f64p, ctypes.c_int]
        lib.kdaref_prefill.restype = ctypes.c_int
        lib.kdaref_decode_step.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p,
                                           i64, i64, i64, i64, ctypes.c_double,
                                           f64p]
        lib.kdaref_decode_step.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x, shape):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _gate(log_alpha, lead, dk):
    """Per-key-channel log gates [*lead, d_k] from any of the three layouts.

    KDA gives one gate per key channel.  Gated DeltaNet gives one scalar per
    (token, head) that every key channel of the head shares ("Cos'è Kimi
    Delta Attention (KDA)?", section "Gating per canale: cosa rende KDA
    diverso"): that scalar repeated over d_k.  DeltaNet has no decay (the
    delta rule alone, "Kimi Delta Attention: la atencion lineal detras de
    Kimi K2 y Qwen3", section "DeltaNet, Gated DeltaNet y KDA: tabla
    comparativa"): log_alpha None means zeros, alpha = 1."""
    lead = tuple(lead)
    if log_alpha is None:
        return np.zeros(lead + (dk,), dtype=np.float32)
    a = np.asarray(log_alpha, dtype=np.float32)
    if a.shape == lead:
        a = np.repeat(a[..., None], dk, axis=-1)
    return _f32(a, lead + (dk,))


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def prefill(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, scale=None,
            threads: int = 0):
    """Run the token-by-token recurrence over a packed batch.

    q, k: [T, H, d_k]; v: [T, H, d_v]; log_alpha: [T, H, d_k] (KDA),
    [T, H] (Gated DeltaNet) or None (DeltaNet); beta: [T, H];
    h0: [N, H, d_k, d_v] or None (zeros); cu_seqlens: [N+1] or None (one
    sequence of length T).  Inputs are taken as float32 values (bf16 and fp32
    stored values convert exactly).  Returns (o [T, H, d_v], hT [N, H, d_k,
    d_v]) as float64.  ``scale`` defaults to 1/sqrt(d_k).
    """
    q = np.asarray(q)
    T, H, dk = q.shape
    dv = np.asarray(v).shape[2]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    if int(cu[-1]) != T:
        raise ValueError("cu_seqlens[-1] must equal the token count")
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    qa = _f32(q, (T, H, dk))
    ka = _f32(k, (T, H, dk))
    va = _f32(v, (T, H, dv))
    la = _gate(log_alpha, (T, H), dk)
    ba = _f32(beta, (T, H))
    h0a = None
    if h0 is not None:
        h0a = np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
        if h0a.shape != (N, H, dk, dv):
            raise ValueError("h0 must be [N, H, d_k, d_v]")
    o = np.zeros((T, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kdaref_prefill(
        _ptr(qa, ctypes.c_float), _ptr(ka, ctypes.c_float),
        _ptr(va, ctypes.c_float), _ptr(la, ctypes.c_float),
        _ptr(ba, ctypes.c_float), _ptr(h0a, ctypes.c_double),
        _ptr(cu, ctypes.c_int64), N, H, dk, dv, float(scale),
        _ptr(o, ctypes.c_double), _ptr(hT, ctypes.c_double), int(threads))
    if rc != 0:
        raise RuntimeError("kdaref_prefill failed with code %d" % rc)
    return o, hT


def decode_step(q, k, v, log_alpha, beta, S, scale=None):
    """One token per sequence.  q, k: [N, H, d_k]; v: [N, H, d_v];
    log_alpha: [N, H, d_k], [N, H] or None (as in prefill); beta: [N, H];
    S: [N, H, d_k, d_v] (not modified).
    Returns (o [N, H, d_v], S_new [N, H, d_k, d_v]) as float64."""
    q = np.asarray(q)
    N, H, dk = q.shape
    dv = np.asarray(v).shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    qa = _f32(q, (N, H, dk))
    ka = _f32(k, (N, H, dk))
    va = _f32(v, (N, H, dv))
    la = _gate(log_alpha, (N, H), dk)
    ba = _f32(beta, (N, H))
    Sa = np.array(S, dtype=np.float64, copy=True, order="C")
    if Sa.shape != (N, H, dk, dv):
        raise ValueError("S must be [N, H, d_k, d_v]")
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().kdaref_decode_step(
        _ptr(qa, ctypes.c_float), _ptr(ka, ctypes.c_float),
        _ptr(va, ctypes.c_float), _ptr(la, ctypes.c_float),
        _ptr(ba, ctypes.c_float), _ptr(Sa, ctypes.c_double),
        N, H, dk, dv, float(scale), _ptr(o, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("kdaref_decode_step failed with code %d" % rc)
    return o, Sa


def decode_multi(q, k, v, log_alpha, beta, S, lengths=None, scale=None):
    """m tokens per sequence, applied in order to the sequence's state.

    q, k: [N, m, H, d_k]; v: [N, m, H, d_v]; log_alpha: [N, m, H, d_k],
    [N, m, H] or None; beta: [N, m, H]; S: [N, H, d_k, d_v] (not modified);
    lengths: [N] tokens applied per sequence (clamped to [0, m]; None = m).
    Returns (o [N, m, H, d_v] with NaN in the rows of tokens not applied,
    S_new [N, H, d_k, d_v]) as float64.  Tokens applied in order are the
    recurrence itself, so this is prefill() over each sequence's applied
    tokens starting from its state: no arithmetic of its own."""
    q = np.asarray(q)
    N, m, H, dk = q.shape
    dv = np.asarray(v).shape[3]
    lens = np.full(N, m, dtype=np.int64) if lengths is None else \
        np.clip(np.asarray(lengths, dtype=np.int64), 0, m)
    take = np.concatenate([n * m + np.arange(lens[n]) for n in range(N)]).astype(np.int64)
    flat = lambda x, tail: np.asarray(x).reshape((N * m, H) + tail)[take]
    la = None if log_alpha is None else np.asarray(log_alpha).reshape((N * m, H, -1))[take]
    if la is not None and la.shape[-1] == 1 and np.asarray(log_alpha).ndim == 3:
        la = la[..., 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    o_t, S_new = prefill(flat(q, (dk,)), flat(k, (dk,)), flat(v, (dv,)), la,
                         flat(beta, ()), h0=S, cu_seqlens=cu, scale=scale)
    o = np.full((N * m, H, dv), np.nan)
    o[take] = o_t
    return o.reshape(N, m, H, dv), S_new


def _load_bwd():
    global _bwd_lib
    if _bwd_lib is None:
        if not os.path.exists(_BWD_LIB):
            _gcc(_BWD_SRC, _BWD_LIB)
        lib = ctypes.CDLL(_BWD_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.kdaref_backward.argtypes = [f32p, f32p, f32p, f32p, f32p, f64p,
                                        ctypes.POINTER(ctypes.c_int64), i64, i64, i64, i64,
                                        ctypes.c_double, f64p, f64p, f64p, f64p, f64p, f64p,
                                        f64p, f64p, ctypes.c_int]
        lib.kdaref_backward.restype = ctypes.c_int
        _bwd_lib = lib
    return _bwd_lib


def backward(q, k, v, log_alpha, beta, do, h0=None, dhT=None, cu_seqlens=None, scale=None,
             threads: int = 0):
    """Gradients of <o, do> + <hT, dhT> for the prefill over a packed batch.

    Arguments as in prefill(), plus do [T, H, d_v] (the adjoint of o) and
    dhT [N, H, d_k, d_v] or None (zeros: the adjoint of the final states).
    Returns a dict of float64 arrays: dq, dk [T, H, d_k], dv [T, H, d_v],
    dlog_alpha (the layout of log_alpha: [T, H, d_k], [T, H] for one gate
    per head, None without a gate), dbeta [T, H], dh0 [N, H, d_k, d_v].
    A per-head gate reaches every key channel, so its gradient is the sum of
    the per-channel gradients over the channels."""
    q = np.asarray(q)
    T, H, dk = q.shape
    dv = np.asarray(v).shape[2]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    if int(cu[-1]) != T:
        raise ValueError("cu_seqlens[-1] must equal the token count")
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    la = _gate(log_alpha, (T, H), dk)
    d = lambda x, shape: None if x is None else np.ascontiguousarray(
        np.asarray(x, dtype=np.float64).reshape(shape))
    h0a, dOa, dhTa = d(h0, (N, H, dk, dv)), d(do, (T, H, dv)), d(dhT, (N, H, dk, dv))
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dlog_alpha=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)),
               dh0=np.zeros((N, H, dk, dv)))
    rc = _load_bwd().kdaref_backward(
        _ptr(_f32(q, (T, H, dk)), ctypes.c_float), _ptr(_f32(k, (T, H, dk)), ctypes.c_float),
        _ptr(_f32(v, (T, H, dv)), ctypes.c_float), _ptr(la, ctypes.c_float),
        _ptr(_f32(beta, (T, H)), ctypes.c_float), _ptr(h0a, ctypes.c_double),
        _ptr(cu, ctypes.c_int64), N, H, dk, dv, float(scale),
        _ptr(dOa, ctypes.c_double), _ptr(dhTa, ctypes.c_double),
        _ptr(out["dq"], ctypes.c_double), _ptr(out["dk"], ctypes.c_double),
        _ptr(out["dv"], ctypes.c_double), _ptr(out["dlog_alpha"], ctypes.c_double),
        _ptr(out["dbeta"], ctypes.c_double), _ptr(out["dh0"], ctypes.c_double), int(threads))
    if rc != 0:
        raise RuntimeError("kdaref_backward failed with code %d" % rc)
    if log_alpha is None:
        out["dlog_alpha"] = None
    elif np.asarray(log_alpha).shape == (T, H):
        out["dlog_alpha"] = out["dlog_alpha"].sum(axis=-1)
    return out


def front_end(q, k, gate_pre=None, beta_pre=None, gate_scale=1.0, l2norm=True, eps=1e-6):
    """The fused input front-end's activations, in float64.

    q, k divided by max(||x||_2, eps) per (token, head) when l2norm (the
    unit keys the delta rule needs: "Kimi Delta Attention: la atencion
    lineal detras de Kimi K2 y Qwen3", notes on key normalisation);
    log_alpha = -gate_scale * softplus(gate_pre), softplus(x) = log(1 + e^x)
    written as max(x, 0) + log1p(e^-|x|); beta = 1 / (1 + e^-beta_pre).
    Missing pre-activations give None.  Returns (q, k, log_alpha, beta)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if l2norm:
        q = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), eps)
        k = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), eps)
    la = None
    if gate_pre is not None:
        x = np.asarray(gate_pre, dtype=np.float64)
        la = -gate_scale * (np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))
    beta = None
    if beta_pre is not None:
        beta = 1.0 / (1.0 + np.exp(-np.asarray(beta_pre, dtype=np.float64)))
    return q, k, la, beta


def front_end_backward(q, k, gate_pre, beta_pre, dq, dk, dlog_alpha, dbeta, gate_scale=1.0,
                       l2norm=True, eps=1e-6):
    """Gradients through front_end, in float64: given the gradients with
    respect to its outputs (normalised q and k, log_alpha, beta), those with
    respect to its inputs (raw q and k, gate_pre, beta_pre).  By the chain
    rule through each of its three maps:
      x_n = x / n with n = max(||x||_2, eps): where ||x|| > eps the Jacobian
        of x / ||x|| is (I - x_n x_n^T) / ||x||, so dx = (dx_n - x_n (x_n .
        dx_n)) / n; where ||x|| <= eps, n is the constant eps and dx = dx_n / eps;
      log_alpha = -c softplus(g): softplus' = sigmoid, so dg = -c sigmoid(g) dlog_alpha;
      beta = sigmoid(y): sigmoid' = beta (1 - beta), so dy = beta (1 - beta) dbeta.
    Without l2norm dq and dk pass through; a missing gate_pre / beta_pre
    gives None for its gradient.  Returns (dq, dk, dgate_pre, dbeta_pre)."""
    def unit_back(x, dxn):
        x = np.asarray(x, dtype=np.float64)
        dxn = np.asarray(dxn, dtype=np.float64)
        nrm = np.linalg.norm(x, axis=-1, keepdims=True)
        n = np.maximum(nrm, eps)
        xn = x / n
        proj = np.sum(xn * dxn, axis=-1, keepdims=True)
        return np.where(nrm > eps, (dxn - xn * proj) / n, dxn / eps)

    if l2norm:
        dq_raw, dk_raw = unit_back(q, dq), unit_back(k, dk)
    else:
        dq_raw = np.asarray(dq, dtype=np.float64)
        dk_raw = np.asarray(dk, dtype=np.float64)
    dg = None
    if gate_pre is not None:
        g = np.asarray(gate_pre, dtype=np.float64)
        dg = -gate_scale / (1.0 + np.exp(-g)) * np.asarray(dlog_alpha, dtype=np.float64)
    dy = None
    if beta_pre is not None:
        b = 1.0 / (1.0 + np.exp(-np.asarray(beta_pre, dtype=np.float64)))
        dy = b * (1.0 - b) * np.asarray(dbeta, dtype=np.float64)
    return dq_raw, dk_raw, dg, dy

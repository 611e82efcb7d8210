"""GPU parity of the fused input front-end, through the C ABI.

Raw q and k (not normalised), bf16 gate pre-activations x and bf16 beta
pre-activations y go in; the kernels normalise q and k per (token, head),
form log_alpha = -c softplus(x) and beta = sigmoid(y) while staging, and
run the recurrence.  Reference: the oracle's front_end activations (fp64)
fed to the oracle's prefill / decode.  Cases: the two-pass matrix path
(bf16, d = 128) and the vector path (fp32), ragged batches, per-channel
and per-head gates, each part of the front-end on its own; decode at three
head sizes.  Also: a call with only normalisation equals, within the bar,
the plain call on inputs normalised outside.

Bars: max-relative error <= 1e-5 (fp32) or 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
import oracle
from kda_testutil import host, rel_err, report, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
LENS = [300, 64, 1, 129, 0, 77]
C_GATE = 0.05


def raw_inputs(lens, H, d, dtype, seed, gate="channel"):
    T = int(sum(lens))
    dt = gen.torch_dtype(dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    gshape = (T, H, d) if gate == "channel" else (T, H)
    return dict(
        q=gen.normal((T, H, d), seed, gen.Q, DEV, dt, std=3.0),
        k=gen.normal((T, H, d), seed, gen.K, DEV, dt, std=0.5),
        v=gen.normal((T, H, d), seed, gen.V, DEV, dt),
        gate_pre=gen.normal(gshape, seed, gen.LOG_ALPHA, DEV, torch.bfloat16),
        beta_pre=gen.normal((T, H), seed, gen.BETA, DEV, torch.bfloat16),
        h0=gen.normal((len(lens), H, d, d), seed, gen.STATE, DEV, torch.float32, std=0.05),
        cu_seqlens=cu)


def reference(inp, parts):
    norm, use_gate, use_beta = parts
    q, k, la, beta = oracle.front_end(host(inp["q"]), host(inp["k"]),
                                      host(inp["gate_pre"]) if use_gate else None,
                                      host(inp["beta_pre"]) if use_beta else None,
                                      gate_scale=C_GATE, l2norm=norm)
    if not use_gate:
        la = host(inp["log_alpha"])
    if not use_beta:
        beta = host(inp["beta"])
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    return oracle.prefill(q, k, host(inp["v"]), la, beta, h0=host(inp["h0"]), cu_seqlens=cu)


def with_activations_outside(inp, parts, gate):
    """log_alpha and beta for the parts the call does not fuse (computed on
    the host from the oracle, then stored as the kernels expect)."""
    _, _, la, beta = oracle.front_end(host(inp["q"]), host(inp["k"]), host(inp["gate_pre"]),
                                      host(inp["beta_pre"]), gate_scale=C_GATE, l2norm=False)
    inp["log_alpha"] = torch.tensor(la, dtype=torch.float32, device=DEV).contiguous()
    inp["beta"] = torch.tensor(beta, dtype=torch.float32, device=DEV).contiguous()


PARTS = [(True, True, True), (True, False, False), (False, True, False), (False, False, True)]


@pytest.mark.parametrize("parts", PARTS)
@pytest.mark.parametrize("dtype,path,d,gate", [("bf16", "two_pass", 128, "channel"),
                                               ("bf16", "two_pass", 128, "head"),
                                               ("f32", "vector", 64, "channel")])
def test_prefill_front_end(parts, dtype, path, d, gate):
    inp = raw_inputs(LENS, 2, d, dtype, 400, gate)
    with_activations_outside(inp, parts, gate)
    norm, use_gate, use_beta = parts
    if not norm:
        # the delta rule needs unit keys: without the kernel's normalisation
        # the inputs come normalised (in fp32, then stored)
        for x in ("q", "k"):
            t = inp[x].float()
            inp[x] = (t / t.norm(dim=-1, keepdim=True)).to(inp[x].dtype)
    o, hT = kda.prefill(inp["q"], inp["k"], inp["v"], None if use_gate else inp["log_alpha"],
                        None if use_beta else inp["beta"], h0=inp["h0"],
                        cu_seqlens=inp["cu_seqlens"], path=path, gate=gate,
                        l2norm_qk=norm, gate_pre=inp["gate_pre"] if use_gate else None,
                        gate_scale=C_GATE, beta_pre=inp["beta_pre"] if use_beta else None)
    o_ref, h_ref = reference(inp, parts)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("front-end %s %s %s %s" % (dtype, path, gate, parts), o=eo, hT=eh)
    assert eo <= tol_for(dtype) and eh <= tol_for(dtype)


def test_prefill_normalisation_matches_outside():
    """Normalising in the kernel agrees with normalising outside (both within
    the bar of the oracle; not bitwise: outside, the unit rows are rounded
    to bf16 before the products)."""
    inp = raw_inputs([257, 64], 2, 128, "bf16", 410)
    with_activations_outside(inp, None, "channel")
    o1, h1 = kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                         h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path="two_pass",
                         l2norm_qk=True)
    qn = (inp["q"].float() / inp["q"].float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    kn = (inp["k"].float() / inp["k"].float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    o2, h2 = kda.prefill(qn, kn, inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                         cu_seqlens=inp["cu_seqlens"], path="two_pass")
    assert rel_err(host(o1), host(o2)) <= 2e-2 and rel_err(host(h1), host(h2)) <= 2e-2


@pytest.mark.parametrize("dtype,d,gate", [("bf16", 128, "channel"), ("f32", 32, "head"),
                                          ("bf16", 64, "channel")])
def test_decode_front_end(dtype, d, gate):
    N, H = 37, 3
    inp = raw_inputs([1] * N, H, d, dtype, 420, gate)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=421, device=DEV)
    q, k, v = (inp[x].reshape(N, H, d) for x in ("q", "k", "v"))
    gp = inp["gate_pre"].reshape((N, H, d) if gate == "channel" else (N, H))
    bp = inp["beta_pre"].reshape(N, H)
    S1 = S.clone()
    o = kda.decode_step(q, k, v, None, None, S1, gate=gate, l2norm_qk=True, gate_pre=gp,
                        gate_scale=C_GATE, beta_pre=bp)
    qf, kf, la, beta = oracle.front_end(host(q), host(k), host(gp), host(bp), gate_scale=C_GATE)
    o_ref, S_ref = oracle.decode_step(qf, kf, host(v), la, beta, host(S))
    eo, es = rel_err(host(o), o_ref), rel_err(host(S1), S_ref)
    report("front-end decode %s d=%d %s" % (dtype, d, gate), o=eo, S=es)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)

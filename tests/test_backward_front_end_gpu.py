"""GPU parity of the prefill gradients through the fused input front-end
(kda_bwd with options.front), through the C ABI.

Raw q and k, bf16 gate pre-activations and bf16 beta pre-activations go in;
the gradients come out with respect to them.  Reference: the oracle's
front_end activations (fp64), its gradient oracle on them, and its chain
rule through the front-end (oracle.front_end_backward), all on the same
stored inputs.  Cases: each part of the front-end on its own and all
together, per-channel and per-head gates, a ragged packed batch with
empty and one-token sequences, non-zero h0 and dhT; normalisation alone
with no gate; an all-empty batch (dh0 = dhT); per-row power-of-two scales
of q and k, which scale dq and dk by the inverse factor, bit for bit, and
leave the other gradients unchanged.

Bar: max-relative error <= 2e-2 per gradient tensor, the backward's bar.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
import oracle
from kda_testutil import host, rel_err, report

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2
LENS = [300, 64, 1, 129, 0, 77]
C_GATE = 0.05


def case(parts, gate, seed):
    norm, use_gate, use_beta = parts
    H, d = 2, 128
    T, N = sum(LENS), len(LENS)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(LENS)]), dtype=torch.int32, device=DEV)
    q = gen.normal((T, H, d), seed, gen.Q, DEV, torch.bfloat16, std=3.0)
    k = gen.normal((T, H, d), seed, gen.K, DEV, torch.bfloat16, std=0.5)
    if not norm:
        # the delta rule needs unit keys: normalised outside (fp32, then stored)
        q = (q.float() / q.float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        k = (k.float() / k.float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    gshape = (T, H, d) if gate == "channel" else (T, H)
    gp = gen.normal(gshape, seed, gen.LOG_ALPHA, DEV, torch.bfloat16)
    bp = gen.normal((T, H), seed, gen.BETA, DEV, torch.bfloat16)
    # the parts not fused take their activations from the oracle, stored fp32
    _, _, la, b = oracle.front_end(host(q), host(k), host(gp), host(bp), gate_scale=C_GATE,
                                   l2norm=False)
    inp = dict(q=q, k=k, v=gen.normal((T, H, d), seed, gen.V, DEV, torch.bfloat16),
               gp=gp if use_gate else None, bp=bp if use_beta else None,
               la=None if use_gate else torch.tensor(la, dtype=torch.float32, device=DEV),
               beta=None if use_beta else torch.tensor(b, dtype=torch.float32, device=DEV),
               h0=gen.normal((N, H, d, d), seed, gen.STATE, DEV, torch.float32, std=0.05),
               do=gen.normal((T, H, d), seed, gen.DO, DEV, torch.bfloat16),
               dhT=gen.normal((N, H, d, d), seed, gen.DHT, DEV, torch.float32, std=0.1), cu=cu)
    return inp


def reference(inp, parts):
    norm, use_gate, use_beta = parts
    q, k = host(inp["q"]), host(inp["k"])
    gp = host(inp["gp"]) if use_gate else None
    bp = host(inp["bp"]) if use_beta else None
    qn, kn, la, b = oracle.front_end(q, k, gp, bp, gate_scale=C_GATE, l2norm=norm)
    if not use_gate:
        la = host(inp["la"])
    if not use_beta:
        b = host(inp["beta"])
    cu = inp["cu"].cpu().numpy().astype(np.int64)
    g = oracle.backward(qn, kn, host(inp["v"]), la, b, host(inp["do"]), h0=host(inp["h0"]),
                        dhT=host(inp["dhT"]), cu_seqlens=cu)
    dq, dk, dgp, dbp = oracle.front_end_backward(q, k, gp, bp, g["dq"], g["dk"], g["dlog_alpha"],
                                                 g["dbeta"], gate_scale=C_GATE, l2norm=norm)
    return dict(dq=dq, dk=dk, dv=g["dv"], dlog_alpha=dgp if use_gate else g["dlog_alpha"],
                dbeta=dbp if use_beta else g["dbeta"], dh0=g["dh0"])


# (l2norm_qk, gate_pre, beta_pre), gate layout; the head layout matters only
# with gate_pre
CASES = [((True, True, True), "channel"), ((True, False, False), "channel"),
         ((False, True, False), "channel"), ((False, False, True), "channel"),
         ((True, True, True), "head"), ((False, True, False), "head")]


@pytest.mark.parametrize("parts,gate", CASES)
def test_backward_front_end(parts, gate):
    inp = case(parts, gate, 500)
    g = kda.backward(inp["q"], inp["k"], inp["v"], inp["la"], inp["beta"], inp["do"], h0=inp["h0"],
                     dhT=inp["dhT"], cu_seqlens=inp["cu"], gate=gate, l2norm_qk=parts[0],
                     gate_pre=inp["gp"], gate_scale=C_GATE, beta_pre=inp["bp"])
    r = reference(inp, parts)
    errs = {key: rel_err(host(g[key]), r[key]) for key in r}
    report("backward front-end %s %s" % (gate, parts), **errs)
    for key, e in errs.items():
        assert e <= TOL, (key, e)


def test_backward_front_end_no_gate():
    """Normalisation only, with no gate at all (DeltaNet): the chain rule
    through the normalisation alone."""
    parts = (True, False, False)
    inp = case(parts, "channel", 510)
    g = kda.backward(inp["q"], inp["k"], inp["v"], None, inp["beta"], inp["do"], h0=inp["h0"],
                     dhT=inp["dhT"], cu_seqlens=inp["cu"], gate="none", l2norm_qk=True)
    assert g["dlog_alpha"] is None
    q, k = host(inp["q"]), host(inp["k"])
    qn, kn, _, _ = oracle.front_end(q, k)
    cu = inp["cu"].cpu().numpy().astype(np.int64)
    r = oracle.backward(qn, kn, host(inp["v"]), None, host(inp["beta"]), host(inp["do"]),
                        h0=host(inp["h0"]), dhT=host(inp["dhT"]), cu_seqlens=cu)
    dq, dk, _, _ = oracle.front_end_backward(q, k, None, None, r["dq"], r["dk"], None, None)
    errs = {"dq": rel_err(host(g["dq"]), dq), "dk": rel_err(host(g["dk"]), dk),
            "dv": rel_err(host(g["dv"]), r["dv"]), "dbeta": rel_err(host(g["dbeta"]), r["dbeta"]),
            "dh0": rel_err(host(g["dh0"]), r["dh0"])}
    report("backward front-end, no gate", **errs)
    for key, e in errs.items():
        assert e <= TOL, (key, e)


def test_backward_front_end_empty_batch():
    """Sequences with no tokens: nothing to normalise or activate; dh0 = dhT."""
    H, d = 2, 128
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    z = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=DEV)
    dhT = gen.normal((3, H, d, d), 520, gen.DHT, DEV, torch.float32, std=0.1)
    g = kda.backward(z(0, H, d), z(0, H, d), z(0, H, d), None, None, z(0, H, d), dhT=dhT,
                     cu_seqlens=cu, l2norm_qk=True, gate_pre=z(0, H, d), gate_scale=C_GATE,
                     beta_pre=z(0, H))
    assert torch.equal(g["dh0"], dhT)


@pytest.mark.parametrize("parts,gate", [((True, True, True), "channel"),
                                        ((True, True, True), "head")])
def test_backward_front_end_from_saved_chunk_states(parts, gate):
    """A prefill through the front-end that saves its chunk states, then the
    backward through the same front-end from that record: the oracle's
    gradients at the same bar, and close to the backward that recomputes
    the forward pass (the record is bf16 either way)."""
    inp = case(parts, gate, 510)
    T, N, H = inp["q"].shape[0], len(LENS), 2
    rec = torch.empty(kda.chunk_states_bytes(T, N, H), dtype=torch.uint8, device=DEV)
    fe = dict(gate=gate, l2norm_qk=parts[0], gate_pre=inp["gp"], gate_scale=C_GATE,
              beta_pre=inp["bp"])
    kda.prefill(inp["q"], inp["k"], inp["v"], inp["la"], inp["beta"], h0=inp["h0"],
                cu_seqlens=inp["cu"], chunk_states=rec, **fe)
    args = (inp["q"], inp["k"], inp["v"], inp["la"], inp["beta"], inp["do"])
    kw = dict(h0=inp["h0"], dhT=inp["dhT"], cu_seqlens=inp["cu"], **fe)
    g = kda.backward(*args, chunk_states=rec, **kw)
    base = kda.backward(*args, **kw)
    r = reference(inp, parts)
    errs = {key: rel_err(host(g[key]), r[key]) for key in r}
    near = {key: rel_err(host(g[key]), host(base[key]).astype(np.float64)) for key in r}
    report("backward front-end from saved states %s %s" % (gate, parts), **errs)
    report("  against the recomputing backward", **near)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
    for key, e in near.items():
        assert e <= 1e-2, (key, e)


def test_backward_front_end_row_scale_invariance():
    """Normalisation is invariant to a positive factor per (token, head) row,
    so with q and k rows scaled by powers of two (2^-8 .. 2^8) the gradient
    with respect to a raw row scales by the inverse factor and every other
    gradient is unchanged.  A power of two passes exactly through each step
    (the norm, its reciprocal, the projection, the bf16 rounding), so both
    hold bit for bit: dq = 2^-e dq_unscaled and dk likewise, the same bits
    for dv, dlog_alpha, dbeta and dh0."""
    parts, gate = (True, True, True), "channel"
    inp = case(parts, gate, 530)
    T, H = inp["q"].shape[:2]
    rng = np.random.default_rng(531)
    eq = torch.from_numpy(rng.integers(-8, 9, size=(T, H))).to(DEV).double()
    ek = torch.from_numpy(rng.integers(-8, 9, size=(T, H))).to(DEV).double()
    scaled = lambda x, e, s: (x.double() * torch.pow(2.0, s * e)[..., None]).to(x.dtype)
    kw = dict(h0=inp["h0"], dhT=inp["dhT"], cu_seqlens=inp["cu"], gate=gate, l2norm_qk=True,
              gate_pre=inp["gp"], gate_scale=C_GATE, beta_pre=inp["bp"])
    g1 = kda.backward(inp["q"], inp["k"], inp["v"], None, None, inp["do"], **kw)
    g2 = kda.backward(scaled(inp["q"], eq, 1), scaled(inp["k"], ek, 1), inp["v"], None, None,
                      inp["do"], **kw)
    assert torch.equal(g2["dq"], scaled(g1["dq"], eq, -1))
    assert torch.equal(g2["dk"], scaled(g1["dk"], ek, -1))
    for key in ("dv", "dlog_alpha", "dbeta", "dh0"):
        assert torch.equal(g2[key], g1[key]), key

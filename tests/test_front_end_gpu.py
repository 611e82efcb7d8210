"""GPU parity of the fused input front-end, through the C ABI.

Raw q and k (not normalised), bf16 gate pre-activations x and bf16 beta
pre-activations y go in; the kernels normalise q and k per (token, head),
form log_alpha = -c softplus(x) and beta = sigmoid(y) while staging, and
run the recurrence.  Reference: the oracle's front_end activations (fp64)
fed to the oracle's prefill / decode.  Cases: both matrix paths (bf16,
d = 128) and the vector path (fp32), ragged batches, per-channel
and per-head gates, each part of the front-end on its own; decode at three
head sizes.  Also: a call with only normalisation equals, within the bar,
the plain call on inputs normalised outside; and per-row power-of-two
scales of q and k (with some all-zero rows) leave every bit of the
outputs unchanged, on every prefill path and in decode.

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
                                               ("bf16", "matrix", 128, "channel"),
                                               ("bf16", "matrix", 128, "head"),
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


@pytest.mark.parametrize("dtype,path,d,gate", [("bf16", "two_pass", 128, "channel"),
                                               ("bf16", "two_pass", 128, "head"),
                                               ("bf16", "matrix", 128, "channel"),
                                               ("bf16", "matrix", 128, "head"),
                                               ("f32", "vector", 64, "channel")])
@pytest.mark.parametrize("c", [4.0, 12.0])
def test_prefill_front_end_strong_gates(dtype, path, d, gate, c):
    """Gate scales of 4 and 12 (log_alpha = -c softplus(x), about -3 and -9
    per token): every chunk leaves the factored range, its 16-row blocks
    inside it at 4 (the blocked form) and beyond it at 12 (the pairwise
    form; the vector path is pairwise at both), so the front-end's gates
    feed those forms, which recompute them from the pre-activations."""
    inp = raw_inputs(LENS, 2, d, dtype, 420, gate)
    o, hT = kda.prefill(inp["q"], inp["k"], inp["v"], None, None, h0=inp["h0"],
                        cu_seqlens=inp["cu_seqlens"], path=path, gate=gate, l2norm_qk=True,
                        gate_pre=inp["gate_pre"], gate_scale=c, beta_pre=inp["beta_pre"])
    q, k, la, beta = oracle.front_end(host(inp["q"]), host(inp["k"]), host(inp["gate_pre"]),
                                      host(inp["beta_pre"]), gate_scale=c, l2norm=True)
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    o_ref, h_ref = oracle.prefill(q, k, host(inp["v"]), la, beta, h0=host(inp["h0"]),
                                  cu_seqlens=cu)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("front-end, gate scale %g, %s %s %s" % (c, dtype, path, gate), o=eo, hT=eh)
    assert eo <= tol_for(dtype) and eh <= tol_for(dtype)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()


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


@pytest.mark.parametrize("path,tiles", [("matrix", 1), ("two_pass", 8)])
def test_prefill_front_end_with_snapshots(path, tiles):
    """The front-end together with state snapshots (every 64 tokens, up to
    4 per sequence): o and hT equal the front-end call without snapshots,
    and each snapshot equals, bit for bit, the final state of a front-end
    prefill of that prefix alone (the same path and value tiles)."""
    lens = [300, 64, 1, 129, 0, 256]
    H, snap, cap = 2, 64, 4
    inp = raw_inputs(lens, H, 128, "bf16", 430)
    kw = dict(path=path, value_tiles=tiles, l2norm_qk=True, gate_scale=C_GATE)
    N = len(lens)
    snaps = torch.full((N, cap, H, 128, 128), 5.0, dtype=torch.float32, device=DEV)
    o, hT, snaps = kda.prefill(inp["q"], inp["k"], inp["v"], None, None, h0=inp["h0"],
                               cu_seqlens=inp["cu_seqlens"], gate_pre=inp["gate_pre"],
                               beta_pre=inp["beta_pre"], snapshot_tokens=snap, snapshots=snaps,
                               **kw)
    o0, hT0 = kda.prefill(inp["q"], inp["k"], inp["v"], None, None, h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], gate_pre=inp["gate_pre"],
                          beta_pre=inp["beta_pre"], **kw)
    assert torch.equal(o, o0) and torch.equal(hT, hT0)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pairs = [(n, j) for n in range(N) for j in range(cap) if (j + 1) * snap <= lens[n]]
    idx = np.concatenate([np.arange(cu[n], cu[n] + (j + 1) * snap) for n, j in pairs])
    sel = torch.tensor(idx, device=DEV)
    plens = [(j + 1) * snap for _, j in pairs]
    pcu = torch.tensor(np.concatenate([[0], np.cumsum(plens)]), dtype=torch.int32, device=DEV)
    ph0 = inp["h0"][torch.tensor([n for n, _ in pairs], device=DEV)].contiguous()
    sub = {x: inp[x][sel].contiguous() for x in ("q", "k", "v", "gate_pre", "beta_pre")}
    _, phT = kda.prefill(sub["q"], sub["k"], sub["v"], None, None, h0=ph0, cu_seqlens=pcu,
                         gate_pre=sub["gate_pre"], beta_pre=sub["beta_pre"], **kw)
    got = torch.stack([snaps[n, j] for n, j in pairs])
    assert torch.equal(got, phT)


def scaled_rows(x, e):
    """x with row (token, head) multiplied by 2^e[token, head]: exact in bf16
    and fp32 (only the exponent changes)."""
    return (x.double() * torch.pow(2.0, e.double())[..., None]).to(x.dtype)


@pytest.mark.parametrize("dtype,path,d,gate", [("bf16", "two_pass", 128, "channel"),
                                               ("bf16", "matrix", 128, "channel"),
                                               ("bf16", "matrix", 128, "head"),
                                               ("f32", "vector", 64, "channel")])
def test_prefill_normalisation_row_scale_invariance(dtype, path, d, gate):
    """The in-kernel normalisation of q and k is a per-(token, head) row
    operation, so scaling each row of q and of k by its own power of two
    (2^-8 .. 2^8) changes no normalised value: a power-of-two factor passes
    exactly through every step (the squares and their sum, the square root
    at an even power, the reciprocal, the products), so the call on the
    scaled inputs must give the same bits as the call on the originals.  A
    row that picked up another row's norm (inside one reduction, the rows
    differ by up to 2^16) would be far off.  Some rows are all zero (q, k or
    both), which the normalisation keeps at zero (their norm is below the
    1e-6 floor); the unscaled call is also checked against the oracle."""
    inp = raw_inputs(LENS, 2, d, dtype, 440, gate)
    T, H = inp["q"].shape[:2]
    rng = np.random.default_rng(441)
    zq = torch.from_numpy(rng.random((T, H)) < 0.05).to(DEV)
    zk = torch.from_numpy(rng.random((T, H)) < 0.05).to(DEV)
    inp["q"][zq] = 0
    inp["k"][zk] = 0
    eq = torch.from_numpy(rng.integers(-8, 9, size=(T, H))).to(DEV)
    ek = torch.from_numpy(rng.integers(-8, 9, size=(T, H))).to(DEV)
    kw = dict(h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path, gate=gate, l2norm_qk=True,
              gate_pre=inp["gate_pre"], gate_scale=C_GATE, beta_pre=inp["beta_pre"])
    o1, h1 = kda.prefill(inp["q"], inp["k"], inp["v"], None, None, **kw)
    o2, h2 = kda.prefill(scaled_rows(inp["q"], eq), scaled_rows(inp["k"], ek), inp["v"], None,
                         None, **kw)
    o_ref, h_ref = reference(inp, (True, True, True))
    eo, eh = rel_err(host(o1), o_ref), rel_err(host(h1), h_ref)
    so, sh = rel_err(host(o2), host(o1)), rel_err(host(h2), host(h1))
    report("front-end row scales %s %s %s" % (dtype, path, gate), o=eo, hT=eh, o_scaled=so,
           hT_scaled=sh)
    assert eo <= tol_for(dtype) and eh <= tol_for(dtype)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_normalisation_row_scale_invariance(dtype, d):
    """Decode's normalisation is applied after its reductions (they are
    linear in q and k, so a power-of-two row factor passes through them
    exactly): row scales of 2^-8 .. 2^8 on q and k give the same bits, and
    all-zero rows stay zero."""
    N, H = 37, 3
    inp = raw_inputs([1] * N, H, d, dtype, 450)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=451, device=DEV)
    q, k, v = (inp[x].reshape(N, H, d).clone() for x in ("q", "k", "v"))
    q[0, 1] = 0
    k[2, 0] = 0
    q[5, 2] = 0
    k[5, 2] = 0
    rng = np.random.default_rng(452)
    eq = torch.from_numpy(rng.integers(-8, 9, size=(N, H))).to(DEV)
    ek = torch.from_numpy(rng.integers(-8, 9, size=(N, H))).to(DEV)
    gp = inp["gate_pre"].reshape(N, H, d)
    bp = inp["beta_pre"].reshape(N, H)
    kw = dict(gate_pre=gp, gate_scale=C_GATE, beta_pre=bp, l2norm_qk=True)
    S1, S2 = S.clone(), S.clone()
    o1 = kda.decode_step(q, k, v, None, None, S1, **kw)
    o2 = kda.decode_step(scaled_rows(q, eq), scaled_rows(k, ek), v, None, None, S2, **kw)
    qf, kf, la, beta = oracle.front_end(host(q), host(k), host(gp), host(bp), gate_scale=C_GATE)
    o_ref, S_ref = oracle.decode_step(qf, kf, host(v), la, beta, host(S))
    eo, es = rel_err(host(o1), o_ref), rel_err(host(S1), S_ref)
    so, ss = rel_err(host(o2), host(o1)), rel_err(host(S2), host(S1))
    report("front-end decode row scales %s d=%d" % (dtype, d), o=eo, S=es, o_scaled=so,
           S_scaled=ss)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)

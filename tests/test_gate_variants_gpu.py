"""GPU parity of the gate variants and of the decode state pool, through
the C ABI.

Gated DeltaNet takes one scalar gate per (token, head), applied to every key
channel; DeltaNet has no gate (alpha = 1).  For every prefill path and for
decode:
  * parity against the fp64 oracle (which takes the same layouts);
  * bitwise equality with the KDA call whose per-channel gate repeats the
    scalar (or is zero): the kernels broadcast the gate when they load it,
    so nothing else may differ.

Decode with a state pool (state_index): sequences update scattered slots of
a larger pool; out-of-range indices skip their sequence.  Checked against
the oracle on the gathered states and bitwise against the plain call; slots
no sequence owns, and the outputs of skipped sequences, stay untouched.

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

# (dtype, path, d): fp32 vector path, both bf16 matrix paths
PATHS = [("f32", "vector", 64), ("bf16", "matrix", 128), ("bf16", "two_pass", 128)]
LENS = [300, 64, 1, 129, 0, 77]


def inputs(dtype, d, seed):
    inp = gen.prefill_inputs(LENS, 2, d, d, dtype, "softplus", state_std=0.05, seed=seed,
                             device=DEV)
    T = inp["q"].shape[0]
    inp["head_gate"] = gen.gates((T, 2), seed + 1, DEV, "uniform").contiguous()
    return inp


def run(inp, path, la, gate):
    return kda.prefill(inp["q"], inp["k"], inp["v"], la, inp["beta"], h0=inp["h0"],
                       cu_seqlens=inp["cu_seqlens"], path=path, gate=gate)


def oracle_run(inp, la):
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    return oracle.prefill(host(inp["q"]), host(inp["k"]), host(inp["v"]), la,
                          host(inp["beta"]), h0=host(inp["h0"]), cu_seqlens=cu)


@pytest.mark.parametrize("dtype,path,d", PATHS)
def test_gated_deltanet_prefill(dtype, path, d):
    inp = inputs(dtype, d, 90)
    g = inp["head_gate"]
    o, hT = run(inp, path, g, "head")
    o_ref, h_ref = oracle_run(inp, host(g))
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("gated deltanet %s %s" % (dtype, path), o=eo, hT=eh)
    assert eo <= tol_for(dtype) and eh <= tol_for(dtype)
    # bitwise the KDA call with the scalar repeated over the key channels
    o2, hT2 = run(inp, path, g[:, :, None].expand(-1, -1, d).contiguous(), "channel")
    assert torch.equal(o, o2) and torch.equal(hT, hT2)


@pytest.mark.parametrize("dtype,path,d", PATHS)
def test_deltanet_prefill(dtype, path, d):
    inp = inputs(dtype, d, 91)
    o, hT = run(inp, path, None, "none")
    o_ref, h_ref = oracle_run(inp, None)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("deltanet %s %s" % (dtype, path), o=eo, hT=eh)
    assert eo <= tol_for(dtype) and eh <= tol_for(dtype)
    o2, hT2 = run(inp, path, torch.zeros_like(inp["log_alpha"]), "channel")
    assert torch.equal(o, o2) and torch.equal(hT, hT2)


def decode_case(N, H, d, dtype, seed):
    tok = gen.decode_token_inputs(N, H, d, d, dtype, "uniform", seed=seed, device=DEV)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=seed, device=DEV)
    tok["head_gate"] = gen.gates((N, H), seed + 1, DEV, "uniform").contiguous()
    return tok, S


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 32)])
@pytest.mark.parametrize("gate", ["head", "none"])
def test_decode_gate_variants(dtype, d, gate):
    N, H = 37, 3
    tok, S = decode_case(N, H, d, dtype, 92)
    la = tok["head_gate"] if gate == "head" else None
    S1 = S.clone()
    o = kda.decode_step(tok["q"], tok["k"], tok["v"], la, tok["beta"], S1, gate=gate)
    o_ref, S_ref = oracle.decode_step(host(tok["q"]), host(tok["k"]), host(tok["v"]),
                                      None if la is None else host(la), host(tok["beta"]),
                                      host(S))
    eo, es = rel_err(host(o), o_ref), rel_err(host(S1), S_ref)
    report("decode %s %s d=%d" % (gate, dtype, d), o=eo, S=es)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)
    full = (la[:, :, None].expand(-1, -1, d).contiguous() if la is not None
            else torch.zeros_like(tok["log_alpha"]))
    S2 = S.clone()
    o2 = kda.decode_step(tok["q"], tok["k"], tok["v"], full, tok["beta"], S2)
    assert torch.equal(o, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype,d,gate", [("bf16", 128, "channel"), ("f32", 64, "head"),
                                          ("bf16", 16, "none")])
def test_decode_state_pool(dtype, d, gate):
    N, H, M = 29, 2, 50                       # 29 sequences, a pool of 50 states
    tok, _ = decode_case(N, H, d, dtype, 93)
    la = {"channel": tok["log_alpha"], "head": tok["head_gate"], "none": None}[gate]
    rng = np.random.default_rng(94)
    slots = rng.permutation(M)[:N].astype(np.int32)
    slots[[3, 11]] = [-1, M + 5]                 # two sequences skipped
    index = torch.tensor(slots, device=DEV)
    pool = gen.decode_state(M, H, d, d, std=0.05, seed=95, device=DEV)
    pool0 = pool.clone()
    sentinel = 7.0
    o = torch.full((N, H, d), sentinel, dtype=tok["q"].dtype, device=DEV)
    kda.decode_step(tok["q"], tok["k"], tok["v"], la, tok["beta"], pool, out=o, gate=gate,
                    state_index=index)
    live = [n for n in range(N) if 0 <= slots[n] < M]
    # live sequences: the plain call on the gathered states, bitwise
    sel = torch.tensor(live, device=DEV)
    gathered = pool0[index[sel].long()].clone()
    sub = lambda t: None if t is None else t[sel].contiguous()
    o_plain = kda.decode_step(sub(tok["q"]), sub(tok["k"]), sub(tok["v"]), sub(la),
                              sub(tok["beta"]), gathered, gate=gate)
    assert torch.equal(o[sel], o_plain)
    assert torch.equal(pool[index[sel].long()], gathered)
    # ... and the oracle
    o_ref, S_ref = oracle.decode_step(host(sub(tok["q"])), host(sub(tok["k"])),
                                      host(sub(tok["v"])), host(sub(la)),
                                      host(sub(tok["beta"])), host(pool0[index[sel].long()]))
    eo, es = rel_err(host(o[sel]), o_ref), rel_err(host(pool[index[sel].long()]), S_ref)
    report("decode pool %s %s d=%d" % (gate, dtype, d), o=eo, S=es)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)
    # skipped sequences write nothing; slots no sequence owns stay as they were
    for n in (3, 11):
        assert bool((o[n] == sentinel).all())
    owned = set(int(slots[n]) for n in live)
    free = torch.tensor([m for m in range(M) if m not in owned], device=DEV)
    assert torch.equal(pool[free], pool0[free])


@pytest.mark.parametrize("dtype,path,d", PATHS)
@pytest.mark.parametrize("pattern", ["all", "alternating"])
def test_gated_deltanet_beyond_factored_range(dtype, path, d, pattern):
    """Gated DeltaNet with gates of -3 per token (every 64-token chunk, or
    every other chunk of each sequence, beyond the factored form's range):
    the blocked form on the matrix paths (the pairwise form on the vector
    path), with the scalar gate loaded per (token, head); parity with the
    oracle and bitwise equality with the KDA call on the expanded gate."""
    inp = inputs(dtype, d, 92)
    g = inp["head_gate"]
    if pattern == "all":
        g.fill_(-3.0)
    else:
        cu = inp["cu_seqlens"].cpu().tolist()
        for n in range(len(cu) - 1):
            for c0 in range(cu[n], cu[n + 1], 64):
                g[c0:min(c0 + 64, cu[n + 1])] = -3.0 if ((c0 - cu[n]) // 64) % 2 == 0 else -0.05
    o, hT = run(inp, path, g, "head")
    o_ref, h_ref = oracle_run(inp, host(g))
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("gated deltanet beyond the factored range (%s) %s %s" % (pattern, dtype, path),
           o=eo, hT=eh)
    assert eo <= tol_for(dtype) and eh <= tol_for(dtype)
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()
    o2, hT2 = run(inp, path, g[:, :, None].expand(-1, -1, d).contiguous(), "channel")
    assert torch.equal(o, o2) and torch.equal(hT, hT2)

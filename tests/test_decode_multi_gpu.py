"""GPU parity of the several-token decode (kda_decode_multi), through the
C ABI.

m tokens per sequence applied in order, one pass over the states: the
verify and commit calls of speculative decoding.  Checked against the fp64
oracle (the token recurrence over each sequence's applied tokens), and bit
for bit against m single decode steps, which apply the same arithmetic to
one token at a time.  Also: the states stay untouched without write_state;
a sequence that applies no token keeps its state; rows of tokens not
applied, and skipped sequences of a state pool, are never written.

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
SENTINEL = 7.0


def tokens(N, m, H, d, dtype, seed):
    """N*m decode tokens laid out [N, m, H, .], plus a per-head gate."""
    t = gen.decode_token_inputs(N * m, H, d, d, dtype, "uniform", seed=seed, device=DEV)
    out = {key: x.reshape((N, m) + tuple(x.shape[1:])).contiguous() for key, x in t.items()}
    out["head_gate"] = gen.gates((N, m, H), seed + 1, DEV, "uniform").contiguous()
    return out


def gate_of(tok, gate):
    return {"channel": tok["log_alpha"], "head": tok["head_gate"], "none": None}[gate]


def run(tok, gate, S, **kw):
    return kda.decode_multi(tok["q"], tok["k"], tok["v"], gate_of(tok, gate), tok["beta"], S,
                            gate=gate, **kw)


def oracle_run(tok, gate, S, lengths=None):
    la = gate_of(tok, gate)
    return oracle.decode_multi(host(tok["q"]), host(tok["k"]), host(tok["v"]),
                               None if la is None else host(la), host(tok["beta"]), host(S),
                               lengths=lengths)


CASES = [("bf16", 128, "channel", 4), ("bf16", 64, "head", 7), ("f32", 64, "channel", 3),
         ("f32", 16, "none", 5), ("bf16", 32, "channel", 1)]


@pytest.mark.parametrize("dtype,d,gate,m", CASES)
def test_verify_then_commit(dtype, d, gate, m):
    N, H = 37, 3
    tok = tokens(N, m, H, d, dtype, 200 + m)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=201, device=DEV)
    S0 = S.clone()
    # verify: the outputs of all m tokens, S only read
    o = run(tok, gate, S, write_state=False)
    assert torch.equal(S, S0)
    o_ref, _ = oracle_run(tok, gate, S0)
    eo = rel_err(host(o), o_ref)
    # commit an accepted prefix per sequence (0 .. m tokens), no outputs
    rng = np.random.default_rng(202)
    acc = rng.integers(0, m + 1, N).astype(np.int32)
    acc[0], acc[1] = 0, m
    lengths = torch.tensor(acc, device=DEV)
    assert run(tok, gate, S, outputs=False, lengths=lengths) is None
    _, S_ref = oracle_run(tok, gate, S0, lengths=acc)
    es = rel_err(host(S), S_ref)
    report("decode multi %s d=%d %s m=%d" % (dtype, d, gate, m), o=eo, S=es)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)
    assert torch.equal(S[0], S0[0])              # no token applied: state as it was


@pytest.mark.parametrize("dtype,d,gate,m", CASES)
def test_equals_single_steps(dtype, d, gate, m):
    N, H = 19, 2
    tok = tokens(N, m, H, d, dtype, 210 + m)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=211, device=DEV)
    S1 = S.clone()
    o = run(tok, gate, S)                        # outputs and state together
    la = gate_of(tok, gate)
    for i in range(m):
        oi = kda.decode_step(tok["q"][:, i].contiguous(), tok["k"][:, i].contiguous(),
                             tok["v"][:, i].contiguous(),
                             None if la is None else la[:, i].contiguous(),
                             tok["beta"][:, i].contiguous(), S1, gate=gate)
        assert torch.equal(o[:, i], oi)
    assert torch.equal(S, S1)


def test_unapplied_rows_untouched():
    N, m, H, d = 11, 5, 2, 64
    tok = tokens(N, m, H, d, "bf16", 220)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=221, device=DEV)
    S0 = S.clone()
    acc = np.array([0, 1, 2, 3, 4, 5, 5, 2, 0, 9, -3], dtype=np.int32)   # clamped to [0, m]
    o = torch.full((N, m, H, d), SENTINEL, dtype=torch.bfloat16, device=DEV)
    run(tok, "channel", S, out=o, lengths=torch.tensor(acc, device=DEV))
    o_ref, S_ref = oracle_run(tok, "channel", S0, lengths=acc)
    live = ~np.isnan(o_ref)
    assert rel_err(host(o)[live], o_ref[live]) <= 2e-2
    assert rel_err(host(S), S_ref) <= 2e-2
    assert bool((o.float().cpu().numpy()[~live] == SENTINEL).all())
    for n in np.flatnonzero(np.clip(acc, 0, m) == 0):
        assert torch.equal(S[n], S0[n])


@pytest.mark.parametrize("dtype,d,gate", [("bf16", 128, "channel"), ("f32", 32, "head")])
def test_state_pool(dtype, d, gate):
    N, m, H, M = 23, 3, 2, 40                    # 23 sequences, a pool of 40 states
    tok = tokens(N, m, H, d, dtype, 230)
    rng = np.random.default_rng(231)
    slots = rng.permutation(M)[:N].astype(np.int32)
    slots[[4, 9]] = [-1, M + 2]                  # two sequences skipped
    index = torch.tensor(slots, device=DEV)
    pool = gen.decode_state(M, H, d, d, std=0.05, seed=232, device=DEV)
    pool0 = pool.clone()
    o = torch.full((N, m, H, d), SENTINEL, dtype=tok["q"].dtype, device=DEV)
    run(tok, gate, pool, out=o, state_index=index)
    live = [n for n in range(N) if 0 <= slots[n] < M]
    sel = torch.tensor(live, device=DEV)
    gathered = pool0[index[sel].long()]
    sub = {key: x[sel].contiguous() for key, x in tok.items()}
    o_ref, S_ref = oracle_run(sub, gate, gathered)
    eo, es = rel_err(host(o[sel]), o_ref), rel_err(host(pool[index[sel].long()]), S_ref)
    report("decode multi pool %s d=%d %s" % (dtype, d, gate), o=eo, S=es)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)
    for n in (4, 9):
        assert bool((o[n] == SENTINEL).all())
    owned = set(int(slots[n]) for n in live)
    free = torch.tensor([x for x in range(M) if x not in owned], device=DEV)
    assert torch.equal(pool[free], pool0[free])


# ---------------------------------------------------------------------------
# the fused input front-end, per token
# ---------------------------------------------------------------------------
C_GATE = 0.05


def raw_tokens(N, m, H, d, dtype, gate, seed):
    """Raw q and k, bf16 gate and beta pre-activations, [N, m, H, .]."""
    dt = gen.torch_dtype(dtype)
    gshape = (N, m, H, d) if gate == "channel" else (N, m, H)
    return dict(q=gen.normal((N, m, H, d), seed, gen.Q, DEV, dt, std=3.0),
                k=gen.normal((N, m, H, d), seed, gen.K, DEV, dt, std=0.5),
                v=gen.normal((N, m, H, d), seed, gen.V, DEV, dt),
                gp=gen.normal(gshape, seed, gen.LOG_ALPHA, DEV, torch.bfloat16),
                bp=gen.normal((N, m, H), seed, gen.BETA, DEV, torch.bfloat16))


@pytest.mark.parametrize("dtype,d,gate,m", [("bf16", 128, "channel", 4), ("f32", 64, "head", 3),
                                            ("bf16", 32, "channel", 5)])
def test_front_end_matches_oracle_and_single_steps(dtype, d, gate, m):
    """With every part of the front-end: the outputs and the committed states
    against the oracle's activations fed to its recurrence, and bit for bit
    against m single front-end decode steps."""
    N, H = 29, 3
    t = raw_tokens(N, m, H, d, dtype, gate, 230 + m)
    S = gen.decode_state(N, H, d, d, std=0.05, seed=231, device=DEV)
    S0 = S.clone()
    fe = dict(l2norm_qk=True, gate_pre=t["gp"], gate_scale=C_GATE, beta_pre=t["bp"])
    o = kda.decode_multi(t["q"], t["k"], t["v"], None, None, S, gate=gate, **fe)
    qn, kn, la, b = oracle.front_end(host(t["q"]), host(t["k"]), host(t["gp"]), host(t["bp"]),
                                     gate_scale=C_GATE)
    o_ref, S_ref = oracle.decode_multi(qn, kn, host(t["v"]), la, b, host(S0))
    eo, es = rel_err(host(o), o_ref), rel_err(host(S), S_ref)
    report("decode multi front-end %s d=%d %s m=%d" % (dtype, d, gate, m), o=eo, S=es)
    assert eo <= tol_for(dtype) and es <= tol_for(dtype)
    # m single steps with the same front-end
    S1 = S0.clone()
    for i in range(m):
        oi = kda.decode_step(t["q"][:, i].contiguous(), t["k"][:, i].contiguous(),
                             t["v"][:, i].contiguous(), None, None, S1, gate=gate,
                             l2norm_qk=True, gate_pre=t["gp"][:, i].contiguous(),
                             gate_scale=C_GATE, beta_pre=t["bp"][:, i].contiguous())
        assert torch.equal(oi, o[:, i]), i
    assert torch.equal(S1, S)

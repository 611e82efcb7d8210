"""GPU parity of kda_fwd_prefill on edge cases of the gates and the batch,
for every kernel path, against the fp64 oracle (through the C ABI).

Gates: no decay with beta = 1 (DeltaNet with full writes); beta = 0 (the
state only decays: outputs read the decayed initial state); per-token
gates of -1.2 on every channel, so the summed gate over a 64-token chunk
reaches -76.8, the edge of the factored exponentials' range; a mix of
undecayed and -1.2 channels; and the rest of the gate domain the pages
allow (any alpha in (0, 1], "Kimi Delta Attention: la atencion lineal
detras de Kimi K2 y Qwen3", section "Cómo funciona Kimi Delta Attention
paso a paso"): -3 and -10 per token on every channel, a mix of undecayed
and -10 channels, and per-token gates uniform in [-12, 0].  Beyond the
factored range every path switches, for the chunks concerned, to the
blocked form (each 16-row block's own gate sum still in range: -3 per
token) or the exact pairwise form (the vector path always) and must match
the oracle; further cases alternate such chunks with ordinary ones inside
each sequence (the first chunk included), and cycle through the factored,
blocked and pairwise forms chunk by chunk.

Batch: 200 short sequences (lengths 0..150, empty ones included, non-zero
initial states), through each path; on the two-pass path this also walks
many short blocks of chunks.

Bars: max-relative error <= 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs) on o
and on the final states.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
from kda_testutil import host, oracle_prefill, rel_err, report, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (dtype, path): the fp32 vector path and both bf16 matrix paths
PATHS = [("f32", "vector"), ("bf16", "matrix"), ("bf16", "two_pass")]


def run(inp, path):
    return kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                       h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path)


def check(inp, path, dtype, name):
    o, hT = run(inp, path)
    o_ref, h_ref = oracle_prefill(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("%s %s" % (name, path), o=eo, hT=eh)
    tol = tol_for(dtype)
    assert eo <= tol and eh <= tol
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()


def gate_case(inp, case):
    la = inp["log_alpha"]
    if case == "no_decay_beta1":
        la.zero_()
        inp["beta"].fill_(1.0)
    elif case == "beta0":
        inp["beta"].zero_()
    elif case == "strong_decay":
        la.fill_(-1.2)
    elif case == "mixed":
        la[:, :, 0::2] = 0.0
        la[:, :, 1::2] = -1.2
    elif case == "decay_3":
        la.fill_(-3.0)
    elif case == "decay_10":
        la.fill_(-10.0)
    elif case == "mixed_0_10":
        la[:, :, 0::2] = 0.0
        la[:, :, 1::2] = -10.0
    elif case == "uniform_12":
        g = torch.Generator(device="cpu").manual_seed(83)
        la.copy_(-12.0 * torch.rand(la.shape, generator=g))
    elif case == "alternating":
        # -3 per token in the even 64-token chunks of each sequence (beyond
        # the factored range), -0.1 in the odd ones
        cu = inp["cu_seqlens"].cpu().tolist()
        for n in range(len(cu) - 1):
            for c0 in range(cu[n], cu[n + 1], 64):
                wild = ((c0 - cu[n]) // 64) % 2 == 0
                la[c0:min(c0 + 64, cu[n + 1])] = -3.0 if wild else -0.1
    elif case == "tiers":
        # each 64-token chunk takes one of the forms by (chunk index + sequence)
        # mod 4: 0 factored (-0.1 per token); 1 every 16-row block in range
        # but the chunk not (-3); 2 one block beyond the range (-10 on its
        # rows 16..31, -0.1 elsewhere); 3 channels alternating 0 and -4.5, so
        # 16-row blocks span 72 nats and the within-block factors are large
        cu = inp["cu_seqlens"].cpu().tolist()
        for n in range(len(cu) - 1):
            for c0 in range(cu[n], cu[n + 1], 64):
                c1 = min(c0 + 64, cu[n + 1])
                kind = ((c0 - cu[n]) // 64 + n) % 4
                if kind == 0:
                    la[c0:c1] = -0.1
                elif kind == 1:
                    la[c0:c1] = -3.0
                elif kind == 2:
                    la[c0:c1] = -0.1
                    la[c0 + 16:min(c0 + 32, c1)] = -10.0
                else:
                    la[c0:c1, :, 0::2] = 0.0
                    la[c0:c1, :, 1::2] = -4.5
    return inp


WIDE = ["decay_3", "decay_10", "mixed_0_10", "uniform_12", "alternating", "tiers"]


@pytest.mark.parametrize("dtype,path", PATHS)
@pytest.mark.parametrize("case", WIDE)
def test_whole_gate_domain(dtype, path, case):
    inp = gen.prefill_inputs([300, 64, 1, 129], 2, 128, 128, dtype, "uniform", state_std=0.1,
                             seed=84, device=DEV)
    check(gate_case(inp, case), path, dtype, "gates %s" % case)


@pytest.mark.parametrize("case", ["alternating", "tiers"])
@pytest.mark.parametrize("tiles", [1, 2, 4])
def test_fused_exact_form_every_tile_width(tiles, case):
    """The fused path's strong-gate forms at each value-tile width (its
    producer/consumer split differs with the width), on a batch with enough
    pairs for the automatic tiling to matter: blocked chunks alternating with
    ordinary ones, and chunks cycling through the factored, blocked and
    pairwise forms."""
    inp = gen.prefill_inputs([300, 64, 1, 129, 200], 8, 128, 128, "bf16", "uniform",
                             state_std=0.1, seed=85, device=DEV)
    gate_case(inp, case)
    o, hT = kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                        h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path="matrix",
                        value_tiles=tiles)
    o_ref, h_ref = oracle_prefill(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    report("fused %s gates, %d value tiles" % (case, tiles), o=eo, hT=eh)
    assert eo <= tol_for("bf16") and eh <= tol_for("bf16")
    assert torch.isfinite(o).all() and torch.isfinite(hT).all()


@pytest.mark.parametrize("dtype,path", PATHS)
@pytest.mark.parametrize("case", ["no_decay_beta1", "beta0", "strong_decay", "mixed"])
def test_degenerate_gates(dtype, path, case):
    inp = gen.prefill_inputs([300, 64, 1, 129], 2, 128, 128, dtype, "uniform", state_std=0.1,
                             seed=80, device=DEV)
    check(gate_case(inp, case), path, dtype, "gates %s" % case)


@pytest.mark.parametrize("dtype,path", PATHS)
def test_many_short_sequences(dtype, path):
    rng = np.random.default_rng(81)
    lens = rng.integers(0, 151, 200)
    lens[::17] = 0
    inp = gen.prefill_inputs(lens, 2, 128, 64, dtype, "softplus", state_std=0.05, seed=82,
                             device=DEV)
    check(inp, path, dtype, "200 short sequences")


@pytest.mark.parametrize("N", [300, 2500, 16500])
def test_plan_order_is_longest_first_permutation(N):
    """The device plan (the fused and vector paths' dispatch order, kept in
    the first N int32 of the workspace) must be bit-exactly the ranking by
    length, longest first, ties by sequence index -- a permutation of
    0..N-1 -- and the identity order above 16384 sequences.  Lengths with
    many ties and zeros; N = 2500 spans three of the kernel's 1024-length
    tiles."""
    rng = np.random.default_rng(90 + N)
    lens = rng.integers(0, 5, N) * 3
    lens[::7] = 0
    T = int(lens.sum())
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    z = torch.zeros((T, 1, 128), dtype=torch.bfloat16, device=DEV)
    la = torch.zeros((T, 1, 128), dtype=torch.float32, device=DEV)
    beta = torch.zeros((T, 1), dtype=torch.float32, device=DEV)
    ws = torch.zeros(kda.prefill_workspace_bytes(T, N, 1, 128, 128, path="matrix"),
                     dtype=torch.uint8, device=DEV)
    kda.prefill(z, z, z, la, beta, cu_seqlens=cu, path="matrix", workspace=ws,
                final_state=False)
    torch.cuda.synchronize()
    order = ws[:4 * N].view(torch.int32).cpu().numpy()
    if N > 16384:
        want = np.arange(N)
    else:
        want = np.array(sorted(range(N), key=lambda i: (-int(lens[i]), i)))
    assert np.array_equal(np.sort(order), np.arange(N))       # a permutation
    assert np.array_equal(order, want)

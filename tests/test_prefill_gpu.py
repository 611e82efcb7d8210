"""GPU parity of kda_fwd_prefill against the fp64 oracle (through the C ABI),
plus properties that hold at any size.

Parity: max-relative error of o and of the final states hT against the
oracle on the same seeded inputs, at 1e-5 for fp32 inputs and 2e-2 for bf16
inputs (fp32 state).  Cases span several chunks, ragged tails, empty
sequences, non-zero initial states and every supported head dimension.

Properties (the regression list that serving a chunked recurrent state
calls for -- long-context recall, batching, state across block boundaries):
varlen == separate calls (bitwise), run-to-run determinism (bitwise),
causality (bitwise), split prefill == whole prefill, hT aliasing h0,
empty sequences keep h0, NaN confined to its own sequence.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen
from kda_testutil import host, oracle_prefill, rel_err, rel_err_slices, report, tol_for, TOL_F32

pytestmark = pytest.mark.gpu
DEV = "cuda"
# the two bf16 matrix-core paths: one fused kernel, or a chunk-parallel pass
# plus a serial state-carry pass
MATRIX_PATHS = ["matrix", "two_pass"]


def call(inp, **kw):
    return kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                       h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], **kw)


def parity(inp, name, tol, scale=None, **kw):
    """Whole-tensor and worst (sequence, head) slice errors of o and hT."""
    o, hT = call(inp, scale=scale, **kw)
    o_ref, hT_ref = oracle_prefill(inp, scale=scale)
    cu = inp["cu_seqlens"].cpu().numpy()
    eo = rel_err(host(o), o_ref)
    es = rel_err(host(hT), hT_ref)
    so = rel_err_slices(host(o), o_ref, cu)
    ss = rel_err_slices(host(hT), hT_ref, cu, states=True)
    report(name, o=eo, hT=es, o_worst_slice=so, hT_worst_slice=ss)
    assert eo <= tol, "o max-rel error %.3e > %.1e" % (eo, tol)
    assert es <= tol, "hT max-rel error %.3e > %.1e" % (es, tol)
    assert so <= tol, "o worst (sequence, head) error %.3e > %.1e" % (so, tol)
    assert ss <= tol, "hT worst (sequence, head) error %.3e > %.1e" % (ss, tol)
    return eo, es


def test_tiny_f32_workload():
    """1 x 64 tokens, H=2, d=16, fp32, zero initial state."""
    w = gen.WORKLOADS["tiny_f32"]
    inp = gen.workload_prefill_inputs(w, seed=0, device=DEV)
    parity(inp, "tiny_f32", TOL_F32)


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (128, 16), (32, 64), (64, 32),
                                   (128, 128), (64, 128)])
def test_f32_shapes_ragged(dk, dv):
    inp = gen.prefill_inputs([1, 33, 70, 0, 100, 64], 2, dk, dv, "f32", "uniform",
                             state_std=0.1, seed=dk + dv, device=DEV)
    parity(inp, "f32 dk=%d dv=%d ragged" % (dk, dv), TOL_F32)


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (128, 32), (128, 16), (64, 64),
                                   (32, 128), (16, 16)])
def test_bf16_shapes_ragged(dk, dv):
    inp = gen.prefill_inputs([1, 31, 64, 65, 200, 0, 129, 300], 3, dk, dv, "bf16",
                             "softplus", state_std=0.02, seed=7 * dk + dv, device=DEV)
    parity(inp, "bf16 dk=%d dv=%d ragged" % (dk, dv), tol_for("bf16"))


@pytest.mark.parametrize("path", MATRIX_PATHS)
@pytest.mark.parametrize("dv", [128, 64, 32, 16])
def test_matrix_paths_ragged(path, dv):
    """Both matrix paths, every d_v, ragged and empty sequences, h0 != 0."""
    inp = gen.prefill_inputs([1, 31, 64, 65, 200, 0, 129, 300], 3, 128, dv, "bf16",
                             "softplus", state_std=0.02, seed=300 + dv, device=DEV)
    parity(inp, "%s dv=%d ragged" % (path, dv), tol_for("bf16"), path=path)


@pytest.mark.parametrize("path,tiles", [("matrix", 1), ("matrix", 2), ("matrix", 4), ("matrix", 8),
                                        ("two_pass", 4), ("two_pass", 8)])
def test_matrix_path_every_tile_width(path, tiles):
    """Each value-tile width of both matrix paths (128 and 64 (fused only), 32, 16 columns)."""
    inp = gen.prefill_inputs([200, 64, 1, 129], 3, 128, 128, "bf16", "softplus",
                             state_std=0.02, seed=40 + tiles, device=DEV)
    o, hT = call(inp, path=path, value_tiles=tiles)
    o_ref, hT_ref = oracle_prefill(inp)
    eo, es = rel_err(host(o), o_ref), rel_err(host(hT), hT_ref)
    report("%s path, %d value tiles" % (path, tiles), o=eo, hT=es)
    assert eo <= tol_for("bf16") and es <= tol_for("bf16")


@pytest.mark.parametrize("blocks", [1, 2, 5])
def test_two_pass_block_size_invariance_bitwise(blocks):
    """The two-pass path carries the state between blocks of chunks in fp32,
    so the block size cannot change a single bit of o or hT -- also when hT
    is not requested and the state crosses blocks through the workspace."""
    inp = gen.prefill_inputs([700, 3, 0, 450], 2, 128, 128, "bf16", "softplus",
                             state_std=0.02, seed=60, device=DEV)
    o1, h1 = call(inp, path="two_pass")
    o2, h2 = call(inp, path="two_pass", block_chunks=blocks)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o3, none = call(inp, path="two_pass", block_chunks=blocks, final_state=False)
    assert none is None and torch.equal(o1, o3)


@pytest.mark.parametrize("blocks", [0, 1, 3])
def test_two_pass_max_seqlen_bitwise(blocks):
    """max_seqlen (the longest sequence, given by the caller) only bounds the
    two-pass block loop: the same bits as the loop over total_T."""
    lens = [700, 3, 0, 450, 64]
    inp = gen.prefill_inputs(lens, 2, 128, 128, "bf16", "softplus", state_std=0.02,
                             seed=62, device=DEV)
    o1, h1 = call(inp, path="two_pass", block_chunks=blocks)
    o2, h2 = call(inp, path="two_pass", block_chunks=blocks, max_seqlen=max(lens))
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o3, h3 = call(inp, path="two_pass", block_chunks=blocks, max_seqlen=sum(lens) + 5)
    assert torch.equal(o1, o3) and torch.equal(h1, h3)


def test_two_pass_max_seqlen_too_small_flags_the_cut_sequence():
    """A sequence longer than max_seqlen (a broken caller promise) gets a NaN
    final state; the shorter sequences are untouched, and so are the cut
    sequence's outputs up to max_seqlen."""
    lens = [300, 64, 129, 0]
    inp = gen.prefill_inputs(lens, 2, 128, 128, "bf16", "softplus", state_std=0.02,
                             seed=63, device=DEV)
    o1, h1 = call(inp, path="two_pass")
    o2, h2 = call(inp, path="two_pass", max_seqlen=192, block_chunks=1)
    assert torch.isnan(h2[0]).all()
    assert torch.equal(h1[1:], h2[1:])
    cu = inp["cu_seqlens"].cpu().numpy()
    assert torch.equal(o1[:192], o2[:192])
    assert torch.equal(o1[cu[1]:], o2[cu[1]:])


def test_matrix_paths_agree():
    """The fused and the two-pass kernels on the same inputs agree with each
    other to the bf16 bar (same operand rounding, different summation)."""
    inp = gen.prefill_inputs([1000, 77, 1], 2, 128, 128, "bf16", "softplus", state_std=0.02,
                             seed=61, device=DEV)
    o_f, h_f = call(inp, path="matrix")
    o_t, h_t = call(inp, path="two_pass")
    report("fused vs two-pass", o=rel_err(host(o_t), host(o_f)), hT=rel_err(host(h_t), host(h_f)))
    assert rel_err(host(o_t), host(o_f)) <= tol_for("bf16")
    assert rel_err(host(h_t), host(h_f)) <= tol_for("bf16")


def test_chunk_length_invariance():
    """The vector path (chunks of 32, fp32 products) and the matrix path
    (chunks of 64, bf16 products) on the same bf16 inputs agree with each
    other to the bf16 bar: the chunk length is not part of the result."""
    inp = gen.prefill_inputs([300, 77, 1], 2, 128, 128, "bf16", "uniform", state_std=0.02,
                             seed=44, device=DEV)
    o_v, h_v = call(inp, path="vector")
    o_m, h_m = call(inp, path="matrix")
    o_ref, h_ref = oracle_prefill(inp)
    e_vm = rel_err(host(o_m), host(o_v))
    report("vector (C=32) vs matrix (C=64)", o=e_vm, hT=rel_err(host(h_m), host(h_v)),
           o_vec_vs_oracle=rel_err(host(o_v), o_ref))
    assert rel_err(host(o_v), o_ref) <= 5e-3     # vector path: only the bf16 output rounding
    assert e_vm <= tol_for("bf16")
    assert rel_err(host(h_m), host(h_v)) <= tol_for("bf16")


@pytest.mark.parametrize("path", MATRIX_PATHS)
def test_custom_scale(path):
    inp = gen.prefill_inputs([50, 77], 2, 128, 128, "bf16", "uniform", state_std=0.02,
                             seed=9, device=DEV)
    parity(inp, "%s bf16 scale=0.05" % path, tol_for("bf16"), scale=0.05, path=path)


@pytest.mark.parametrize("path", MATRIX_PATHS)
def test_batch4_t4096_workload(path):
    """4 x 4096 tokens, H=16, d=128, bf16, zero initial state (every pair checked)."""
    w = gen.WORKLOADS["batch4_t4096"]
    inp = gen.workload_prefill_inputs(w, seed=1, device=DEV)
    parity(inp, "batch4_t4096 %s" % path, tol_for("bf16"), path=path)


# --------------------------------------------------------------------------
# properties
# --------------------------------------------------------------------------
# (dtype, path) of the property checks: the fp32 vector path and both matrix paths
PROP_CASES = [("f32", "auto"), ("bf16", "matrix"), ("bf16", "two_pass")]


@pytest.mark.parametrize("dtype,path", PROP_CASES)
def test_varlen_equals_separate_calls_bitwise(dtype, path):
    lens = [70, 0, 5, 130, 64]
    inp = gen.prefill_inputs(lens, 2, 128, 64, dtype, "softplus", state_std=0.02, seed=21,
                             device=DEV)
    o, hT = call(inp, path=path)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for n, L in enumerate(lens):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = {kk: inp[kk][a:b] for kk in ("q", "k", "v", "log_alpha", "beta")}
        o_n, h_n = kda.prefill(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"],
                               h0=inp["h0"][n:n + 1].contiguous(), path=path)
        assert torch.equal(o[a:b], o_n)
        assert torch.equal(hT[n:n + 1], h_n)


@pytest.mark.parametrize("dtype,path", PROP_CASES)
def test_repeat_runs_bitwise(dtype, path):
    inp = gen.prefill_inputs([300, 45, 129], 4, 128, 128, dtype, "softplus",
                             state_std=0.02, seed=22, device=DEV)
    o1, h1 = call(inp, path=path)
    o2, h2 = call(inp, path=path)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("dtype,path", PROP_CASES)
def test_causal_prefix_bitwise(dtype, path):
    """Changing tokens after position t leaves every output up to t unchanged."""
    T, t_cut = 200, 90            # cut inside a chunk
    inp = gen.prefill_inputs([T], 2, 128, 128, dtype, "uniform", state_std=0.02, seed=23,
                             device=DEV)
    o1, _ = call(inp, path=path)
    pert = dict(inp)
    for kk in ("q", "k", "v"):
        x = inp[kk].clone()
        x[t_cut + 1:] = x[t_cut + 1:].flip(0)
        pert[kk] = x
    la = inp["log_alpha"].clone()
    la[t_cut + 1:] *= 0.5
    pert["log_alpha"] = la
    o2, _ = call(pert, path=path)
    assert torch.equal(o1[:t_cut + 1], o2[:t_cut + 1])
    assert not torch.equal(o1[t_cut + 1:], o2[t_cut + 1:])


@pytest.mark.parametrize("dtype,path", PROP_CASES)
def test_split_prefill_equals_whole(dtype, path):
    """Prefill of the first part, then of the rest from the carried state,
    equals one prefill of the whole sequence (state across a call boundary
    that falls inside a chunk)."""
    T, cut = 333, 150
    inp = gen.prefill_inputs([T], 3, 128, 128, dtype, "softplus", state_std=0.02, seed=24,
                             device=DEV)
    o_all, h_all = call(inp, path=path)
    first = {kk: inp[kk][:cut] for kk in ("q", "k", "v", "log_alpha", "beta")}
    rest = {kk: inp[kk][cut:] for kk in ("q", "k", "v", "log_alpha", "beta")}
    o1, h1 = kda.prefill(first["q"], first["k"], first["v"], first["log_alpha"],
                         first["beta"], h0=inp["h0"], path=path)
    o2, h2 = kda.prefill(rest["q"], rest["k"], rest["v"], rest["log_alpha"], rest["beta"],
                         h0=h1, path=path)
    tol = tol_for(dtype)
    e_o = rel_err(host(torch.cat([o1, o2])), host(o_all))
    e_h = rel_err(host(h2), host(h_all))
    report("split prefill %s" % dtype, o=e_o, hT=e_h)
    assert e_o <= tol and e_h <= tol


@pytest.mark.parametrize("path", MATRIX_PATHS)
def test_final_state_may_alias_initial_state(path):
    inp = gen.prefill_inputs([100, 7], 2, 128, 128, "bf16", "uniform", state_std=0.02,
                             seed=25, device=DEV)
    o1, h1 = call(inp, path=path)
    h = inp["h0"].clone()
    o2, h2 = kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=h,
                         cu_seqlens=inp["cu_seqlens"], final_state=h, path=path,
                         block_chunks=1)
    assert h2.data_ptr() == h.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(h1, h)


@pytest.mark.parametrize("dk,path", [(64, "auto"), (128, "matrix"), (128, "two_pass")])
def test_empty_sequences_keep_initial_state(dk, path):
    inp = gen.prefill_inputs([0, 10, 0], 2, dk, 64, "bf16", "uniform", state_std=0.5,
                             seed=26, device=DEV)
    _, hT = call(inp, path=path)
    assert torch.equal(hT[0], inp["h0"][0]) and torch.equal(hT[2], inp["h0"][2])
    empty = gen.prefill_inputs([0, 0], 2, dk, 64, "bf16", "uniform", state_std=0.5, seed=27,
                               device=DEV)
    o, hT = call(empty, path=path)
    assert o.shape[0] == 0 and torch.equal(hT, empty["h0"])
    no_h0 = dict(empty, h0=None)
    _, hT = call(no_h0, path=path)
    assert torch.count_nonzero(hT) == 0


@pytest.mark.parametrize("path", MATRIX_PATHS)
def test_no_final_state_requested(path):
    inp = gen.prefill_inputs([90], 2, 128, 128, "bf16", "uniform", seed=28, device=DEV)
    o1, _ = call(inp, path=path)
    o2, h = call(inp, final_state=False, path=path)
    assert h is None and torch.equal(o1, o2)


@pytest.mark.parametrize("path", MATRIX_PATHS)
def test_nan_stays_in_its_sequence(path):
    lens = [100, 100, 100]
    inp = gen.prefill_inputs(lens, 2, 128, 128, "bf16", "uniform", state_std=0.02, seed=29,
                             device=DEV)
    o_ref, h_ref = call(inp, path=path)
    bad = dict(inp)
    v = inp["v"].clone()
    v[150, 1, 3] = float("nan")         # sequence 1, head 1
    bad["v"] = v
    o, hT = call(bad, path=path)
    assert torch.equal(o[:100], o_ref[:100]) and torch.equal(o[200:], o_ref[200:])
    assert torch.equal(hT[0], h_ref[0]) and torch.equal(hT[2], h_ref[2])
    assert torch.equal(o[100:200, 0], o_ref[100:200, 0])     # other head untouched
    assert torch.isnan(hT[1, 1]).any()

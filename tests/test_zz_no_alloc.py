"""The allocation-free prefill (kda_fwd_prefill_noalloc) through the C ABI:
its outputs equal kda_fwd_prefill_ex's on the same inputs, bit for bit,
for each kernel path, over two calls in a row on one GPU -- the second with
a smaller input, so it must not depend on what the first left in the
library's device array.  The second call's first half of tokens has gates
of -3 per token, so its chunks there take the blocked form (the vector
path: the pairwise form).  The
same kernels run on both entry points; only the workspace differs (a
caller buffer vs the static array)."""
import pytest
import torch

import gated_delta_rule_05_amd as kda
import kda_inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (first call's lengths, second call's lengths, heads, dtype, path)
CASES = [
    ([20000, 9000, 0, 4097], [3000, 65], 32, "bf16", "two_pass"),
    ([700] * 40 + [1, 0, 33] * 8, [300, 64, 1] * 43, 4, "bf16", "auto"),   # fused: >= 128 pairs
    ([300, 0, 77, 64], [40, 1], 2, "f32", "auto"),                         # vector path
]


def _inputs(lens, H, dtype, seed):
    dk = 128 if dtype == "bf16" else 64
    return gen.prefill_inputs(lens, H, dk, dk, dtype, "softplus", state_std=0.02, seed=seed,
                              device=DEV)


def _both(inp, path):
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    kw = dict(h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], path=path,
              max_seqlen=max(inp["lengths"]))
    o1, h1 = kda.prefill(*args, **kw)
    o2, h2 = kda.prefill(*args, no_alloc=True, **kw)
    torch.cuda.synchronize()
    return (o1, h1), (o2, h2)


@pytest.mark.parametrize("first,second,H,dtype,path", CASES)
def test_noalloc_prefill_equals_workspace_prefill(first, second, H, dtype, path):
    for i, lens in enumerate((first, second)):
        print("[no_alloc] path=%s dtype=%s H=%d call %d: %d sequences, %d tokens"
              % (path, dtype, H, i, len(lens), sum(lens)), flush=True)
        inp = _inputs(lens, H, dtype, 700 + 10 * i + H)
        if i == 1:
            inp["log_alpha"][: sum(lens) // 2] = -3.0
        (o1, h1), (o2, h2) = _both(inp, path)
        assert torch.equal(o1, o2), "o differs on call %d" % i
        assert torch.equal(h1, h2), "hT differs on call %d" % i
        assert torch.isfinite(o2).all() and torch.isfinite(h2).all()

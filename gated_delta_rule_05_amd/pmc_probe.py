"""Workload driver for rocprofv3 counter runs (HBM traffic per kernel).

Runs, on cuda:0, one long-context prefill of 32 heads (d = 128, bf16) over
``--chunks`` 64-token chunks with the library's default path, one decode
step of 256 x 32 states, and a 512 MiB device-to-device copy whose byte
count calibrates the counters.  Used as

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o <name> --output-format csv -- \\
        python3 -m gated_delta_rule_05_amd.pmc_probe

(and again with WRITE_SIZE); bench.py reads the resulting per-launch
figures from profiles/traffic.json.
"""
import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--chunks", type=int, default=512)
    args = ap.parse_args()
    import torch
    import gated_delta_rule_05_amd as kda
    import kda_inputs as gen

    T, H, d = 64 * args.chunks, 32, 128
    inp = gen.prefill_inputs([T], H, d, d, "bf16", "softplus", state_std=0.0, seed=2, device="cuda")
    kda.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    S = gen.decode_state(256, H, d, d, std=0.02, seed=3, device="cuda")
    t = gen.decode_token_inputs(256, H, d, d, "bf16", "uniform", seed=3, step=0, device="cuda")
    kda.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], S)
    a = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)                       # 512 MiB read + 512 MiB written
    torch.cuda.synchronize()
    print("pmc probe done: T=%d H=%d" % (T, H), flush=True)


if __name__ == "__main__":
    main()

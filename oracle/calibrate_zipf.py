"""Calibrate the Zipf(1.1) logit-prior strength beta (an input-generation parameter).

Routes the seeded token bank of the tiered workload through the oracle's router for a
grid of beta values and reports the share of top-4 selections that land in the 128
highest-prior experts; the workload asks for about 70%.  Calls only the oracle and the
input generators.  Usage:  python -m oracle.calibrate_zipf [n_tokens]
"""
import sys

import numpy as np

import oracle
import synth


def hot_share(beta: float, n_tokens: int = 512, cfg: int = 2) -> float:
    wl = synth.WORKLOADS[cfg]
    router = wl.router(0)
    bias = synth.zipf_logit_bias(wl.seed, wl.E, beta)
    hot = set(synth.hot_set(wl.seed, wl.E).tolist())
    xs = wl.tokens_bank(n_tokens)
    xf = synth.bf16_to_f32(xs) if wl.x_bf16 else xs
    hits = 0
    for t in range(n_tokens):
        logits = oracle.router_logits(router, xf[t].astype(np.float64), bias, wl.router_bf16)
        idx, _, _ = oracle.route(logits, wl.K)
        hits += sum(int(e) in hot for e in idx)
    return hits / (n_tokens * wl.K)


def main():
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 512
    for beta in [0.3, 0.35, 0.4, 0.45, 0.5, 0.6, 1.0]:
        print(f"beta {beta:.2f}: hot share {hot_share(beta, n):.3f}")


if __name__ == "__main__":
    main()

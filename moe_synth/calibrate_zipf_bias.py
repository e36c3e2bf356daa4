"""Writes zipf_bias_e288.npy: a per-expert router-logit bias that makes expert
popularity follow a (capped) Zipf law with exponent s = 1 over 288 experts.

This is input preparation for the load-imbalanced verify workload (64 streams x
4 tokens, as in multi-token-prediction verification).  It is not part of the
layer's arithmetic and nothing on the kernel path reads it except as an input.

Why a calibration is needed: with top-8-of-288 selection on N(0,1) logits, the
naive bias b_r = -ln r is far steeper than Zipf (only ~100 experts are ever
touched), and no expert can be picked by more than every token, so the target
inclusion probability of expert of rank r is taken as pi_r = min(1, c/r) with c
chosen so that sum_r pi_r = 8 (the expected number of experts per token).

Fixed-point iteration on a Monte-Carlo sample of logit rows:
    b <- b + 0.5 * (ln pi'_r - ln pihat_r)
where pihat_r is the measured top-8 inclusion frequency and pi' is pi capped at
0.995 and rescaled to sum 8 (a cap strictly below 1 keeps the log finite).

Run:  python -m moe_synth.calibrate_zipf_bias
"""
import os

import numpy as np

E, K = 288, 8
ROWS, ITERS, SEED = 32768, 60, 12345


def target_inclusion(num_experts: int, top_k: int) -> np.ndarray:
    r = np.arange(1, num_experts + 1, dtype=np.float64)
    lo, hi = 0.0, float(num_experts)
    for _ in range(200):  # bisection for c with sum(min(1, c/r)) = top_k
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c / r).sum() > top_k:
            hi = c
        else:
            lo = c
    return np.minimum(1.0, 0.5 * (lo + hi) / r)


def inclusion_frequency(noise: np.ndarray, bias: np.ndarray, top_k: int) -> np.ndarray:
    scores = noise + bias[None, :]
    top = np.argpartition(-scores, top_k - 1, axis=1)[:, :top_k]
    counts = np.bincount(top.ravel(), minlength=bias.shape[0])
    return counts / noise.shape[0]


def calibrate() -> np.ndarray:
    rng = np.random.default_rng(SEED)
    noise = rng.standard_normal((ROWS, E)).astype(np.float32).astype(np.float64)
    pi = target_inclusion(E, K)
    capped = np.minimum(pi, 0.995)
    capped *= K / capped.sum()
    bias = -0.5 * np.log(np.arange(1, E + 1, dtype=np.float64))
    for _ in range(ITERS):
        freq = np.maximum(inclusion_frequency(noise, bias, K), 0.5 / ROWS)
        bias += 0.5 * (np.log(capped) - np.log(freq))
        bias -= bias.max()
    return bias.astype(np.float32)


if __name__ == "__main__":
    b = calibrate()
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_e288.npy")
    np.save(out, b)
    pi = target_inclusion(E, K)
    rng = np.random.default_rng(SEED + 1)
    check = inclusion_frequency(rng.standard_normal((ROWS, E)), b.astype(np.float64), K)
    print(f"wrote {out}; L1(freq - pi) on a fresh sample = {np.abs(check - pi).sum():.4f}")
    print("bias[:5] =", b[:5], " bias[-1] =", b[-1])

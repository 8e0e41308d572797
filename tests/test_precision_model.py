"""A NumPy model of the attention's operand rounding, re-run on the CPU: why the matrix-core
operands are fp16 rather than bf16 when the I/O is bf16 and the bar is sum|d| / sum|ref| <= 2e-3.

Each scheme computes softmax(Q K^T / sqrt(128)) V on the workloads' N(0,1) inputs (stored bf16,
rotated in fp64) with its roundings applied and is compared with the exact result:
  all_bf16     rotated Q and K, the probabilities P and the output rounded to bf16
  k_bf16       rotated K bf16 (a bf16 cache), Q and P fp16, output bf16
  fp16_ops     Q, K and P fp16, output bf16          (the kernels' scheme)
  exact_out    exact arithmetic, output rounded to bf16 (the floor that bf16 output sets)
The model is not the oracle and not the kernel: it isolates the effect of where values are
rounded.  It pins the ordering that the design relies on: all_bf16 and k_bf16 fail the bar,
fp16_ops passes it, and fp16_ops stays within 10 % of the bf16-output floor.
"""
import math

import numpy as np

import qi_inputs as qin
from oracle import qi_oracle as O


def bf16(x):
    return qin.bf16_bits_to_f64(qin.f32_to_bf16_bits(np.asarray(x, np.float64).astype(np.float32)))


def f16(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def attend(q, k, v, rq, rk, rp):
    """Softmax attention of one head with the given roundings of Q, K and the probabilities."""
    s = rq(q) @ rk(k).T / math.sqrt(128)
    s = s - s.max(axis=1, keepdims=True)
    p = rp(np.exp(s))
    return (p @ v) / p.sum(axis=1, keepdims=True)


def scheme_errors(n_keys=4096, n_q=256, seeds=(1, 2, 3)):
    ident = lambda x: x
    errs = {"all_bf16": [], "k_bf16": [], "fp16_ops": [], "exact_out": []}
    for seed in seeds:
        rng = np.random.default_rng([77, seed])
        pos = np.stack([np.zeros(n_keys, np.int64), np.arange(n_keys) // 64 - 32, np.arange(n_keys) % 64 - 32], 1)
        c, s = O.rope_tables(pos)
        q = O.rotate(bf16(rng.standard_normal((n_q, 1, 128))), c[:n_q], s[:n_q])[:, 0]
        k = O.rotate(bf16(rng.standard_normal((n_keys, 1, 128))), c, s)[:, 0]
        v = bf16(rng.standard_normal((n_keys, 128)))
        ref = attend(q, k, v, ident, ident, ident)
        rel = lambda got: np.abs(got - ref).sum() / np.abs(ref).sum()
        errs["all_bf16"].append(rel(bf16(attend(q, k, v, bf16, bf16, bf16))))
        errs["k_bf16"].append(rel(bf16(attend(q, k, v, f16, bf16, f16))))
        errs["fp16_ops"].append(rel(bf16(attend(q, k, v, f16, f16, f16))))
        errs["exact_out"].append(rel(bf16(ref)))
    return {name: float(np.mean(e)) for name, e in errs.items()}


def test_fp16_operands_meet_the_bar_and_bf16_operands_do_not():
    e = scheme_errors()
    print({k: f"{v:.2e}" for k, v in e.items()})
    assert e["all_bf16"] > 2e-3
    assert e["k_bf16"] > 2e-3
    assert e["fp16_ops"] < 2e-3
    assert e["exact_out"] <= e["fp16_ops"] <= 1.1 * e["exact_out"]

"""Pins of the oracle's LM-head step (logits = h W^T, row log-partition
functions): hand-computed logits of small integer operands, and the closed form
of the partition function when every logit of a row is equal."""
import numpy as np

import oracle


def _bits(x):
    x = np.asarray(x, np.float32)
    assert np.array_equal((x.view(np.uint32) & 0xFFFF), np.zeros_like(x, np.uint32)), "not bf16"
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_small_integer_logits_are_exact():
    h = [[1.0, 2.0, 0.0], [0.0, -1.0, 3.0]]
    w = [[1.0, 0.0, 1.0], [2.0, 1.0, 0.0], [0.5, 0.5, -2.0]]
    logits, lse = oracle.lm_head(_bits(h), _bits(w), [1.0, 0.5])
    assert np.array_equal(logits, [[1.0, 4.0, 1.5], [3.0, -1.0, -6.5]])
    want0 = np.log(np.exp(1.0) + np.exp(4.0) + np.exp(1.5))
    want1 = np.log(np.exp(6.0) + np.exp(-2.0) + np.exp(-13.0))
    assert abs(lse[0] - want0) < 1e-14 and abs(lse[1] - want1) < 1e-14


def test_equal_logits_partition_function():
    """Every vocabulary row equal: all logits of a row equal l, lse = l/T + ln V."""
    rng = np.random.default_rng(0)
    d, V = 64, 1000
    h = rng.standard_normal((5, d)).astype(np.float32)
    hb = _bits((h.view(np.uint32) & 0xFFFF0000).view(np.float32))
    wrow = (rng.standard_normal(d).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    wb = _bits(np.tile(wrow, (V, 1)))
    T = np.array([0.3, 0.7, 1.0, 1.5, 2.0])
    logits, lse = oracle.lm_head(hb, wb, T)
    l = oracle.bf16_bits_to_f64(hb) @ oracle.bf16_bits_to_f64(wb[0])
    assert np.allclose(logits, l[:, None], rtol=0, atol=1e-12)
    assert np.allclose(lse, l / T + np.log(V), rtol=0, atol=1e-10)

"""Pins of the oracle's all-gather + GEMM (oracle.gemm_ag) against what the
pages and the mathematics fix, without the HIP path.

The operation ("FLUX: Fast Software-based Communication Overlap On GPUs
Through Kernel Fusion", TL;DR: the all-gather fused as the GEMM's prologue;
"mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", Section 4) is the
column-parallel linear layer: every rank gathers the activation row slices
and multiplies them by its own column shard of the weight.  Its invariant:
the tp ranks' outputs, side by side, are the unsharded layer's output.
"""
import numpy as np
import torch

import oracle
import synthetic


def _bf16_bits_of(values_f64: np.ndarray) -> np.ndarray:
    # independent rounding: float64 -> float32 (exact for these integers) ->
    # torch's BF16 conversion
    t = torch.from_numpy(values_f64.astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_column_shards_assemble_the_unsharded_product():
    tp, S, K, Nl = 8, 6, 40, 12
    rng = np.random.default_rng(11)
    x_full = rng.integers(-3, 4, size=(tp * S, K)).astype(np.float64)
    w_full = rng.integers(-3, 4, size=(tp * Nl, K)).astype(np.float64)
    xb = _bf16_bits_of(x_full)
    wb = _bf16_bits_of(w_full)
    slices = [xb[d * S:(d + 1) * S] for d in range(tp)]
    ys = []
    for r in range(tp):
        xg, y = oracle.gemm_ag(slices, wb[r * Nl:(r + 1) * Nl])
        assert np.array_equal(xg, xb)  # every rank gathers the same activations
        ys.append(y)
    want = _bf16_bits_of(x_full @ w_full.T)  # |entries| <= 9 * 40: exact in float64 and float32
    assert np.array_equal(np.concatenate(ys, axis=1), want)


def test_gathered_rows_follow_source_rank():
    cfg = synthetic.AG_CONFIGS["ag_tiny"]
    xs, w = synthetic.make_ag_inputs(cfg, "integer")
    xg, y = oracle.gemm_ag(xs, w)
    for d in range(cfg.tp):
        assert np.array_equal(xg[d * cfg.S:(d + 1) * cfg.S], xs[d])
        # each slice's output rows are that slice's product alone
        assert np.array_equal(y[d * cfg.S:(d + 1) * cfg.S], oracle.gemm_ag([xs[d]] * cfg.tp, w)[1][:cfg.S])


def test_normal_inputs_within_summation_bound_of_fp64():
    cfg = synthetic.AG_CONFIGS["ag_tiny"]
    xs, w = synthetic.make_ag_inputs(cfg, "normal")
    _, y = oracle.gemm_ag(xs, w)
    x = np.concatenate([oracle.bf16_to_f32(a).astype(np.float64) for a in xs], axis=0)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    ref = x @ wf.T
    got = oracle.bf16_to_f32(y).astype(np.float64)
    mag = np.maximum(np.abs(got), np.abs(ref))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    bound = ulp + cfg.K * 2.0 ** -24 * (np.abs(x) @ np.abs(wf).T) + 1e-30
    assert np.all(np.abs(got - ref) <= bound)


def test_ag_inputs_are_seeded_and_shaped():
    cfg = synthetic.AG_CONFIGS["ag_qkv"]
    xs, w = synthetic.make_ag_inputs(cfg, "normal", M=64)
    assert len(xs) == 8 and all(x.shape == (8, cfg.K) and x.dtype == np.uint16 for x in xs)
    assert w.shape == (cfg.N, cfg.K)
    xs2, w2 = synthetic.make_ag_inputs(cfg, "normal", M=64)
    assert all(np.array_equal(a, b) for a, b in zip(xs, xs2)) and np.array_equal(w, w2)
    assert not np.array_equal(xs[0], xs[1])

"""Exact-integer pin of the whole layer (router, top-1, gate/up
pre-activations, SwiGLU, fold, down product, shared expert, combine).

On the integer-valued layers of ``integer_layer`` every intermediate is an
exact integer (see that module), so the GPU's outputs are compared bit for
bit with int64 matrix products: logits, top-1 ids (lower id on ties), the
routing weight 1.0, out_assign and shared_out (fp32), and y (bf16 of their
exact sum).  The gate and up pre-activations reach the outputs through
h = bf16(g * u), so any error in them that changes a stored h changes
out_assign exactly.

The CPU test pins the construction itself: the fp64 oracle, fed the stored
inputs (packed codes, scales 1.0), gives the int64 model's values exactly
when h is not rounded.
"""
import numpy as np
import pytest

import integer_layer as IL
import oracle
import workloads as W
from gpu_harness import spec_of

CASES = [
    # (T, E, routed format): 96-row tiles with a 2nd tile per expert, 32-row
    # bodies in the 96-row kernel, the 32- and 16-row kernels, bf16 weights,
    # and b-bit codes on the fp16 gate/up path
    (600, 4, W.I4G32),
    (300, 16, W.I4G32),
    (20, 8, W.I4G32),
    (5, 8, W.I4G32),
    (300, 4, W.BF16),
    (300, 4, "i2g32"),
    (96, 4, "i3g32"),
    (40, 4, "i5g32"),
]


def _id(c):
    return f"{c[2]}_T{c[0]}_E{c[1]}"


CPU_CASES = [(300, 4, W.I4G32), (64, 4, "i3g32"), (64, 4, W.BF16)]


@pytest.mark.parametrize("T,E,fmt", CPU_CASES, ids=[_id(c) for c in CPU_CASES])
def test_integer_model_equals_oracle(T, E, fmt):
    """The int64 model with h unrounded equals the fp64 oracle exactly."""
    cfg, inp, ints = IL.build(_id((T, E, fmt)), T, E, fmt)
    logits, ids, out, shared = IL.reference(ints, cfg.n_shared, round_h=False)
    assert np.array_equal(oracle.router_logits(inp["x"], oracle.BF16, inp["wr"], oracle.BF16,
                                               cfg.d, cfg.E), logits.astype(np.float64))
    w = np.ones((T, 1))
    y, oa, so = oracle.moe_experts(spec_of(cfg), inp, ids[:, None], w)
    assert np.array_equal(oa, out.astype(np.float64))
    assert np.array_equal(so, shared.astype(np.float64))
    assert np.array_equal(y, (out + shared).astype(np.float64))


@pytest.mark.gpu
@pytest.mark.parametrize("T,E,fmt", CASES, ids=[_id(c) for c in CASES])
def test_integer_layer_bit_exact_on_gpu(T, E, fmt):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpu_harness import GpuLayer, check_plan
    cfg, inp, ints = IL.build(_id((T, E, fmt)), T, E, fmt)
    logits, ids, out, shared = IL.reference(ints, cfg.n_shared)
    print(f"[run] integer {_id((T, E, fmt))}", flush=True)
    res = GpuLayer(cfg, inp).run(inp["x"])
    assert np.array_equal(res["logits"], logits.astype(np.float32))
    assert np.array_equal(res["ids"][:, 0], ids)
    assert np.array_equal(res["w"], np.ones((T, 1), np.float32))
    check_plan(cfg, res)
    oa = res["out_assign"][res["inv_perm"][np.arange(T)]]
    bad = oa != out.astype(np.float32)
    assert not bad.any(), f"out_assign: {int(bad.sum())} elements differ, e.g. row {np.argwhere(bad)[0]}"
    assert np.array_equal(res["shared_out"], shared.astype(np.float32))
    y_bits = W.to_bf16_bits((out + shared).astype(np.float32))
    assert np.array_equal(res["y_bits"].view(np.uint16), y_bits)

"""Host checks of the seeded input generator (no method arithmetic here)."""
import numpy as np
import torch

import workloads as W


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
        # exact ties: low 16 bits = 0x8000, both parities of the kept bit
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38, 1e-40, -1e-40,
                  np.inf, -np.inf], np.float32),
    ])
    ours = W.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = W.bf16_round_bits(np.array([np.nan], np.float32))
    assert np.isnan(W.bf16_bits_to_f32(nan))[0]


def test_workload_shapes_and_recipe():
    w = W.WORKLOADS[4]
    assert (w.group, w.bh, w.bkv) == (3, 384, 128)
    x = W.make_inputs(W.WORKLOADS[2])
    assert x.xq.shape == (32, 256, 64) and x.xk.shape == (8, 256, 64)
    assert x.gamma_q.dtype == np.float32 and not np.all(x.gamma_q == 1)
    x1 = W.make_inputs(W.WORKLOADS[1])
    assert np.all(x1.gamma_q == 1) and np.all(x1.gamma_k == 1)
    # seeded: identical on a second draw
    y = W.make_inputs(W.WORKLOADS[2])
    np.testing.assert_array_equal(x.xq, y.xq)
    # bf16 workloads hand out bf16-representable values
    w5 = W.WORKLOADS[5].replace(seq_len=64)
    z = W.make_inputs(w5)
    np.testing.assert_array_equal(W.bf16_round(z.xq), z.xq)


def test_flop_count_matches_the_closed_form():
    w = W.WORKLOADS[5]
    f = w.attn_flops()
    assert f["total"] == 12 * 128 * 32 * 4096 * 4097 // 2
    assert f["fwd"] * 3 == f["total"]

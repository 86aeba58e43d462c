"""The seeded input generators: determinism, bf16 rounding, distributions."""
import numpy as np
import torch

import selscan_inputs as si


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  1e-30, 3e38], np.float32)])
    bits, wide = si.bf16_round_np(x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(wide, t.to(torch.float32).numpy())
    bits2, wide2 = si.bf16_round(x)
    assert np.array_equal(bits, bits2) and np.array_equal(wide, wide2)


def test_generators_are_deterministic():
    a = si.make_fwd_inputs(2, 16, 8, 4, si.BF16, True, seed=5)
    b = si.make_fwd_inputs(2, 16, 8, 4, si.BF16, True, seed=5)
    for f in ("u", "delta", "Bm", "Cm", "z"):
        assert np.array_equal(getattr(a, f).bits, getattr(b, f).bits)
    assert np.array_equal(a.delta_bias, b.delta_bias)
    c = si.make_fwd_inputs(2, 16, 8, 4, si.BF16, True, seed=6)
    assert not np.array_equal(a.u.bits, c.u.bits)
    w = si.WORKLOADS["decode"]
    s1 = si.decode_step_inputs(w, 3, batch=4)
    s2 = si.decode_step_inputs(w, 3, batch=4)
    assert np.array_equal(s1.u.bits, s2.u.bits)


def test_distributions():
    inp = si.make_fwd_inputs(2, 512, 256, 16, si.F32, True, seed=7)
    assert abs(inp.u.value.std() - 1) < 0.02 and abs(inp.u.value.mean()) < 0.02
    assert abs(inp.delta.value.std() - 0.5) < 0.01
    dt = np.log1p(np.exp(inp.delta_bias.astype(np.float64)))      # recovers the drawn dt
    assert dt.min() >= 1e-3 * (1 - 1e-5) and dt.max() <= 0.1 * (1 + 1e-5)
    assert np.array_equal(inp.A[5], -np.arange(1, 17, dtype=np.float32))
    assert np.all(inp.D_skip == 1)


def test_workload_table():
    w = si.WORKLOADS
    assert (w["tiny_f32"].batch, w["tiny_f32"].L, w["tiny_f32"].dim, w["tiny_f32"].N) == \
        (1, 256, 64, 16)
    assert (w["mamba130m_layer"].batch, w["mamba130m_layer"].L, w["mamba130m_layer"].dim) == \
        (8, 2048, 1536)
    assert (w["long_seq"].L, w["long_seq"].dim) == (131072, 2048)
    assert (w["large_layer"].batch, w["large_layer"].dim) == (16, 5120)
    assert (w["decode"].batch, w["decode"].dim, w["decode"].decode_steps) == (256, 5120, 1024)

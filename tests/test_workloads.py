"""Host-side checks of the seeded workload generator (no method arithmetic)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0, 1e-30], np.float32)])
    x = x.astype(np.float32)
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_long_tail_counts():
    c = workloads.long_tail_counts()
    assert c == [1, 1, 2, 7, 17, 39, 85, 178, 369, 771, 1662, 3783, 9467, 16384, 16384, 16384]
    wl = workloads.config("longtail")
    assert wl.T == 65534 and sorted(wl.counts.tolist()) == c
    assert set(wl.ranks.tolist()) <= {8, 16, 32, 64}


def test_configs_shapes():
    wl = workloads.config("llama_up")
    assert (wl.d_in, wl.d_out, wl.n_adapters, wl.T, wl.R) == (4096, 14336, 32, 65536, 960)
    assert wl.ranks.tolist()[:5] == [8, 16, 32, 64, 8]
    assert wl.alphas.tolist()[:4] == [8.0, 16.0, 32.0, 8.0]
    t = workloads.config("tiny")
    assert t.dtype == "f32" and t.T == 128 and t.ranks.tolist() == [4, 8]
    q = workloads.config("qwen_q")
    assert q.T == 16384 and set(q.ranks.tolist()) == {16}


def test_draw_deterministic_and_thread_independent():
    a = workloads.draw(3, 1, (5000, 16), 0.5, "bf16")
    b = workloads.draw(3, 1, (5000, 16), 0.5, "bf16")
    assert np.array_equal(a, b)
    # bf16-representable
    assert np.array_equal(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(a)), a)
    assert abs(float(a.std()) - 0.5) < 0.02

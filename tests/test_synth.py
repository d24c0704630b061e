"""The seeded workload generator: determinism, block regeneration, bf16 rounding."""
import numpy as np
import torch

from sparse_memory_linear_sdm_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 0.0, 65504.0], np.float32)])
    ours = synth.bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_blockwise():
    wl = synth.small("layer1p4b", B=2, T=5000, d_model=32)
    x1, s1 = synth.gen_x(wl, seed=0)
    x2, _ = synth.gen_x(wl, seed=0)
    assert np.array_equal(x1, x2) and s1.dtype == np.uint16
    part, _ = synth.gen_x(wl, seed=0, t0=4000, t1=4500, batches=[1])
    assert np.array_equal(part[0], x1[1, 4000:4500])
    x3, _ = synth.gen_x(wl, seed=1)
    assert not np.array_equal(x1, x3)


def test_long_workload_repeats_every_block_once_later():
    wl = synth.small("long1m", T=8 * 4096, d_model=4)
    x, _ = synth.gen_x(wl, seed=0)
    blocks = x[0].reshape(8, 4096, 4)
    for k in range(4, 8):
        matches = [j for j in range(4) if np.array_equal(blocks[k], blocks[j])]
        assert len(matches) == 1
    assert sorted(j for k in range(4, 8) for j in range(4)
                  if np.array_equal(blocks[k], blocks[j])) == [0, 1, 2, 3]


def test_workload_shapes():
    wl = synth.WORKLOADS["layer1p4b"]
    assert wl.N == 131044 and wl.P == 1706 and wl.slot_bytes_per_token_head() == 98304
    p = synth.gen_params(synth.small("tiny"))
    assert p["w_proj"].shape == (162, 64) and p["w_proj"].dtype == np.float32
    m0 = synth.gen_m0(synth.small("tiny"))
    assert m0.shape == (1, 1024, 16) and abs(m0.std() - 0.02) < 0.002

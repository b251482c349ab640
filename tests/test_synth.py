"""The seeded input generator: published test vector, determinism, slicing,
storage rounding and the statistics each workload asks for. CPU only."""

import numpy as np
import torch

import synth
from synth import workloads


def test_splitmix64_published_vector():
    # SplitMix64 from state 0: first two outputs
    assert synth._mix64_int(synth.GAMMA) == 0xE220A8397B1DCDAF
    assert synth._mix64_int(2 * synth.GAMMA) == 0x6E789E6AA1B965F4
    base = synth.stream_base(0, 0)
    r = synth.raw64(0, 0, np.arange(3, dtype=np.uint64))
    assert [int(x) for x in r] == [synth._mix64_int(base + (i + 1) * synth.GAMMA) for i in range(3)]


def test_deterministic_and_sliceable():
    w = workloads.C2_DECODE_32K
    shape = (1, 2, 1024, 128)
    a = synth.generate(w.recipe("K"), shape)
    b = synth.generate(w.recipe("K"), shape)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(synth.generate_slice(w.recipe("K"), shape, (0, 1), 100, 300), a[0, 1, 100:300])
    c = synth.generate(w.recipe("V"), shape)
    assert not np.array_equal(a, c)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 3
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_normal_statistics():
    z = synth.std_normal(7, 3, np.arange(1 << 21, dtype=np.uint64)).astype(np.float64)
    assert abs(z.mean()) < 3e-3 and abs(z.std() - 1.0) < 3e-3
    assert np.abs(z).max() < 4.33
    # quantiles against Phi^-1
    for p, q in [(0.5, 0.0), (0.8413447, 1.0), (0.9772499, 2.0)]:
        assert abs(np.quantile(z, p) - q) < 1e-2


def test_block_offset_recipe():
    w = workloads.C3_DECODE_128K
    shape = (1, 1, 4096, 128)
    k = synth.bf16_bits_to_f32(synth.generate(w.recipe("K"), shape)).astype(np.float64)
    assert abs(k.std() - np.sqrt(1.25)) < 0.02
    blocks = k.reshape(64, 64, 128)
    # within a block the common offset shows up as a between-block variance of 0.25
    assert abs(blocks.mean(axis=1).var(axis=0).mean() - (0.25 + 1 / 64)) < 0.03


def test_tiny_fp32_scale():
    w = workloads.C1_TINY
    q = synth.generate(w.recipe("Q"), w.shape("Q"))
    assert q.dtype == np.float32
    z = synth.std_normal(w.seed, synth.TAG_Q, np.arange(q.size, dtype=np.uint64))
    np.testing.assert_array_equal(q.ravel(), z * np.float32(workloads.INV_SQRT_128))


def test_workload_geometry():
    c3 = workloads.C3_DECODE_128K
    assert (c3.W, c3.nB, c3.G, c3.n_tiles) == (8191, 2048, 4, 1)
    c5 = workloads.C5_PREFILL
    assert (c5.n_tiles, c5.q_start + c5.Tq) == (64, c5.T)
    assert workloads.C1_TINY.W == 255 and workloads.C2_DECODE_32K.W == 2047


def test_layer_and_lookahead_tags_are_distinct():
    # every (tensor, layer, lookahead distance) of a stack draws its own stream
    w = workloads.C4_OFFLOAD
    tags = []
    for layer in range(4):
        for name in ("Q", "K", "V", "F_self"):
            tags.append(w.recipe(name, layer).tag)
        tags += [w.recipe("F", layer, ahead).tag for ahead in range(1, 10)]
    assert len(tags) == len(set(tags))
    try:
        w.recipe("F", 0, 10)
    except ValueError:
        pass
    else:
        raise AssertionError("a lookahead of 10 layers must be refused")

"""Host side of the seeded input generator (CPU only)."""

import numpy as np

import synth
from synth import workloads as W


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 1234567: the first outputs of the published generator
    s, out = 1234567, []
    for _ in range(5):
        s = (s + synth.GAMMA) & synth.MASK64
        out.append(synth.mix64_int(s))
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_array_and_scalar_mix_agree():
    z = np.array([0, 1, 2 ** 63, 2 ** 64 - 1, 0x123456789ABCDEF], dtype=np.uint64)
    with np.errstate(over="ignore"):
        got = synth._mix64(z)
    assert [int(v) for v in got] == [synth.mix64_int(int(v)) for v in z]


def test_counter_addressable():
    full = synth.tensor(3, 7, 5000, 0.5)
    part = synth.tensor(3, 7, 1000, 0.5, start=2500)
    assert np.array_equal(full[2500:3500], part)
    idx = np.array([4999, 0, 1234])
    assert np.array_equal(synth.values(3, 7, idx, 0.5), full[idx])


def test_moments_and_support():
    v = synth.tensor(0, 1, 1 << 20, 2.0).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 2.0) < 0.01
    assert np.all(np.abs(v) <= 12.0 + 1e-6)
    g = synth.tensor(0, 2, 1 << 16, 0.02, offset=1.0).astype(np.float64)
    assert abs(g.mean() - 1.0) < 1e-3 and abs(g.std() - 0.02) < 1e-3
    a = synth.tensor(0, 3, 1 << 16, 1e-6, mode=synth.MODE_ABS_F32)
    assert np.all(a >= 0)


def test_bf16_mode_truncates():
    f = synth.tensor(5, 9, 4096, 1.0)
    b = synth.tensor(5, 9, 4096, 1.0, mode=synth.MODE_BF16)
    assert np.array_equal(b, (f.view(np.uint32) >> 16).astype(np.uint16))
    wb = synth.bf16_bits_to_f32(b)
    assert np.all(np.abs(wb) <= np.abs(f))


def test_streams_and_seeds_differ():
    a = synth.tensor(0, 1, 256, 1.0)
    assert not np.array_equal(a, synth.tensor(0, 2, 256, 1.0))
    assert not np.array_equal(a, synth.tensor(1, 1, 256, 1.0))


def test_workload_sizes():
    assert W.MINI_OPT_N == 1_722_400_768
    assert W.SHARD_N == 3_670_000_000
    assert W.SHARD.softmax.heads * 4 == W.SHARD.softmax.total_heads == 112

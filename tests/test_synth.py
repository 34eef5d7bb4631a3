"""The seeded input generator: deterministic, random-access, right distributions."""
import numpy as np

import synth
from oracle import bf16_to_f32 as F


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of the published generator
    # (java.util.SplittableRandom / Vigna's splitmix64.c with x = 0).
    def mix(z):
        m = (1 << 64) - 1
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9 & m
        z = (z ^ (z >> 27)) * 0x94D049BB133111EB & m
        return z ^ (z >> 31)
    golden = 0x9E3779B97F4A7C15
    assert mix(golden) == 0xE220A8397B1DCDAF  # first output of splitmix64 from x = 0
    base = mix(mix(0) + 5)
    raw = synth.raw_u64(0, 5, 0, 4)
    for i in range(4):
        assert int(raw[i]) == mix((base + (i + 1) * golden) & ((1 << 64) - 1))


def test_random_access_and_chunking():
    a = synth.normal_bf16(3, 7, 0, 10_000_000)  # chunked across threads
    b = synth.normal_bf16(3, 7, 1234, 1000)
    assert np.array_equal(a[1234:2234], b)
    c = synth.normal_f32(3, 7, 999, 3)
    assert np.array_equal(c, synth.normal_f32(3, 7, 999, 3))


def test_distributions():
    n = 1 << 20
    v = F(synth.normal_bf16(0, 1, 0, n)).astype(np.float64)
    assert abs(v.mean()) < 5 / np.sqrt(n) and abs(v.std() - 1) < 5 / np.sqrt(2 * n) + 2e-3
    w = synth.normal_f32(0, 5, 0, n, std=1 / np.sqrt(5120)).astype(np.float64)
    assert abs(w.std() * np.sqrt(5120) - 1) < 0.01
    u = synth.uniform_f32(0, 6, 0, n, -0.01, 0.01)
    assert u.min() >= -0.01 and u.max() < 0.01 and abs(u.mean()) < 1e-4
    nw = F(synth.uniform_bf16(0, 3, 0, 5120, 0.9, 1.1))
    assert nw.min() >= 0.89 and nw.max() <= 1.11


def test_workload_table():
    wl = synth.WORKLOADS["decode1"]
    assert (wl.d, wl.E, wl.G, wl.kg, wl.k, wl.f, wl.scale) == (5120, 256, 8, 4, 8, 2560, 2.5)
    assert synth.WORKLOADS["tiny"].gs == 4
    b = synth.router_bias(synth.WORKLOADS["skew32k"])
    assert np.all(b[list(synth.HOT16)] == np.float32(0.5))
    assert np.all(np.abs(np.delete(b, list(synth.HOT16))) < 0.01)

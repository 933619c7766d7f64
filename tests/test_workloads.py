"""Host logic of the seeded input generator and workload tables."""
import numpy as np

from workloads import configs, rng, synth


def test_splitmix64_reference_values():
    # SplitMix64 from state 0: the published first outputs of the generator.
    s = rng.Stream(0, "x")
    s.key = np.uint64(0)
    w = s.words(0, 3)
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_deterministic_and_distinct():
    a = synth.normal_f64(0, "a", (1000,))
    assert np.array_equal(a, synth.normal_f64(0, "a", (1000,)))
    assert not np.array_equal(a, synth.normal_f64(0, "b", (1000,)))
    assert not np.array_equal(a, synth.normal_f64(1, "a", (1000,)))
    big = synth.normal_f64(0, "m", (200000,))
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1) < 0.01


def test_outliers_and_distributions():
    x = synth.gelu_with_outliers(0, "o", 64, 4608)
    cols = synth.outlier_columns(0, "o/outcols", 4608)
    assert cols.size == 5 and len(set(cols.tolist())) == 5
    assert synth.outlier_columns(0, "p/outcols", 1152).size == 1
    base = synth.gelu_normal(0, "o", 64, 4608)
    assert np.array_equal(x[:, cols], (base[:, cols].astype(np.float64) * 20).astype(np.float32))
    rest = np.setdiff1d(np.arange(4608), cols)
    assert np.array_equal(x[:, rest], base[:, rest])
    s = synth.silu_normal(0, "s", 16, 64)
    assert s.min() > -0.2785 and s.dtype == np.float32  # SiLU minimum is about -0.2785


def test_bf16_rounding_ties_to_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    b = synth.f32_to_bf16_bits(f)
    back = synth.bf16_bits_to_f32(b)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]


def test_workload_tables():
    wl = configs.WORKLOADS
    assert wl["c1"].M == 256 and wl["c1"].layers[0].K == 512
    assert [l.name for l in wl["c2"].layers] == ["qkv", "proj", "fc1", "fc2"]
    assert wl["c2"].M == 4096 and all(l.cfg for l in wl["c2"].layers)
    assert all(l.hadamard_block == 128 and l.a_bits == 4 for l in wl["c3"].layers)
    c4 = wl["c4"]
    assert c4.M == 18432 and sum(l.a_bits == 8 for l in c4.layers) == 2
    assert c4.layers[0].seg_offsets().tolist() == [0, 3072, 6144, 9216, 12288, 15360, 18432]
    assert len(wl["c5"].layers) == 112
    sch = configs.c5_schedule()
    assert sch.shape == (50, 112) and set(np.unique(sch).tolist()) == {0, 2, 4}
    c6 = wl["c6"]
    assert len(c6.layers) == 112 and c6.steps == 50 and c6.stages == 4
    ws = configs.c6_w_schedule()
    assert ws.shape == (4, 112) and set(np.unique(ws).tolist()) == {0, 2, 4}
    stages = [configs.stage_of(c6, t) for t in range(c6.steps)]
    assert stages == sorted(stages) and set(stages) == {0, 1, 2, 3}
    assert max(stages.count(g) for g in range(4)) - min(stages.count(g) for g in range(4)) <= 1

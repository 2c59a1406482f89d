"""The seeded input generator: published SplitMix64 outputs, determinism and distributions."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # SplitMix64 from state 0: the first outputs of the reference generator
    w = synth.stream(0, 0, 2)
    assert int(w[0]) == 0xE220A8397B1DCDAF
    assert int(w[1]) == 0x6E789E6AA1B965F4


def test_streams_are_pure_functions_of_their_key():
    a = synth.codes(1000, 3, 17, synth.GATE_CODES, 64, 256)
    b = synth.codes(1000, 3, 17, synth.GATE_CODES, 64, 256)
    c = synth.codes(1000, 3, 18, synth.GATE_CODES, 64, 256)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    s = synth.stream(synth.stream_key(1, 2, 3, 4), 0, 100)
    assert np.array_equal(s[10:20], synth.stream(synth.stream_key(1, 2, 3, 4), 10, 10))


def test_code_and_scale_distributions():
    c = synth.codes(1000, 0, 0, synth.GATE_CODES, 2048, 4096)
    nib = np.concatenate([(c & 15).ravel(), (c >> 4).ravel()])
    hist = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(hist - 1 / 16) < 0.002)
    s = synth.scales(1000, 0, 0, synth.GATE_SCALES, 2048, 4096, -6, 0)
    assert set(np.unique(s)) == {0x08, 0x10, 0x18, 0x20, 0x28, 0x30, 0x38}
    s = synth.scales(1001, 0, 0, synth.GATE_SCALES, 128, 256, -4, 2)
    assert set(np.unique(s)) <= {0x18, 0x20, 0x28, 0x30, 0x38, 0x40, 0x48}


def test_normals_and_bf16():
    x = synth.bf16_bits_to_f32(synth.activations(1002, 0, 64, 4096)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    f = np.array([1.0, 1.00390625, 1.005859375, -2.0, np.inf, 3.4e38], dtype=np.float32)
    b = synth.f32_to_bf16_bits(f)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 1.5*2^-8 rounds up; 3.4e38 rounds to +Inf
    assert list(b) == [0x3F80, 0x3F80, 0x3F81, 0xC000, 0x7F80, 0x7F80]


def test_routing_shapes():
    lg = synth.logits_same(1003, 0, 4, 256)
    assert np.all(lg == lg[0])
    d = synth.logits_disjoint(3, 16, 4)
    order = np.argsort(-d, axis=1, kind="stable")[:, :4]
    assert order.tolist() == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]]


def test_plant_positions():
    x = synth.activations(1004, 0, 16, 4096)
    xp, (nr, nc), (ir, ic) = synth.plant_nan_inf(1004, 0, x)
    assert nr != ir
    f = synth.bf16_bits_to_f32(xp)
    assert np.isnan(f[nr, nc]) and f[ir, ic] == np.inf
    assert int(np.sum(~np.isfinite(f))) == 2


def test_fp8_generators():
    w = synth.fp8_weights(5, 1, 64, 512)
    assert w.shape == (64, 512) and w.dtype == np.uint8
    assert not np.any((w == 0x7F) | (w == 0xFF))          # no NaN codes
    assert np.unique(w).size == 254
    assert np.array_equal(w, synth.fp8_weights(5, 1, 64, 512))
    assert not np.array_equal(w, synth.fp8_weights(5, 2, 64, 512))
    s = synth.fp8_scales(5, 1, 300, 512, -10, -6)
    assert s.shape == (3, 4) and s.dtype == np.float32
    e = np.log2(s)
    assert np.all(e == np.round(e)) and e.min() >= -10 and e.max() <= -6


def test_general_and_mixed_scales():
    # any_scales: every non-NaN E4M3FN byte is possible, NaN bytes never appear
    a = synth.any_scales(5, 0, 1, synth.GATE_SCALES, 512, 4096)
    assert not np.any((a == 0x7F) | (a == 0xFF))
    assert np.unique(a).size == 254
    # mixed_scales: power-of-two draw except where the rule puts general bytes
    N, K = 40, 32 * 9
    m = synth.mixed_scales(5, 0, 1, synth.UP_SCALES, N, K, -4, 2)
    p = synth.scales(5, 0, 1, synth.UP_SCALES, N, K, -4, 2)
    g = synth.any_scales(5, 0, 1, synth.UP_SCALES, N, K)
    for n in range(N):
        for j in range(K // 32):
            want = g[n, j] if (j % 3 == 0 or (j % 3 == 1 and n % 5 == 0)) else p[n, j]
            assert m[n, j] == want
    ex = synth.expert_mixed(5, 0, 1, 64, 32, -4, 2)
    plain = synth.expert(5, 0, 1, 64, 32, -4, 2)
    for name in ("gate_codes", "up_codes", "down_codes"):
        assert np.array_equal(ex[name], plain[name])

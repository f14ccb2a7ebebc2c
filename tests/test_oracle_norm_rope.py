"""Pins for the fp64 oracle of the q/k head RMSNorm + RoPE + paged store step.
CPU only.

Each test names the passage it follows.  Page titles are abbreviated:
[Intro] = "大模型推理入门与 nano-vLLM 源码详解"; [Analysis] = "nano-vllm 技术分析";
[Pico #8] = "Pico-vLLM 开发日志 #8 更多Triton Kernel和性能优化".  Every pin is a
value the pages print, a closed form, or a property of the definition, chosen so
that a plausible slip in the oracle (a dropped eps, a wrong sign, adjacent
instead of half-split pairs, a wrong frequency exponent, rotating before the
norm, normalising over the wrong axis, touching V) fails at least one of them.
"""

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def tol(decimals):
    return 0.5 * 10.0 ** (-decimals) + 1e-12


def f32_raw(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------------------- RMSNorm


def test_rmsnorm_page_example():
    """[Intro §19.3, §19.4]: [1, 2, 3] with eps ignored and gamma = 1."""
    g = golden("intro_s19_4_rmsnorm.json")
    x = np.array(g["x"])
    y = oracle.rms_norm(x, None, 0.0)
    assert np.max(np.abs(y - np.array(g["y"]))) <= tol(g["decimals"])
    assert abs(np.mean(x * x) - g["mean_square"]) < 1e-12
    assert abs(math.sqrt(np.mean(x * x)) - g["rms"]) <= tol(5)
    # the example keeps the 1:2:3 ratio and the output mean square is 1
    assert np.allclose(y / y[0], [1.0, 2.0, 3.0], rtol=0, atol=1e-14)
    assert abs(np.mean(y * y) - 1.0) < 1e-14


def test_rmsnorm_scale_invariance():
    """[Intro §19.3]: scaling [1, 2, 3] by ten gives the same output (eps ignored)."""
    g = golden("intro_s19_4_rmsnorm.json")
    a = oracle.rms_norm(np.array(g["x"]), None, 0.0)
    b = oracle.rms_norm(np.array(g["scaled_x"]), None, 0.0)
    assert np.max(np.abs(a - b)) < 1e-15


def test_rmsnorm_eps_closed_form():
    """[Intro §19.3]: eps sits inside the root, next to the mean square.

    A constant vector c has mean square c*c, so y = gamma * c / sqrt(c*c + eps);
    the zero vector maps to zero, not NaN."""
    for c, eps in [(0.5, 1e-6), (3.0, 0.25), (1e-3, 1e-6)]:
        x = np.full(128, c)
        w = np.linspace(-2.0, 2.0, 128)
        y = oracle.rms_norm(x, w, eps)
        assert np.allclose(y, w * c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)
    assert np.all(oracle.rms_norm(np.zeros(64), None, 1e-6) == 0.0)


def test_rmsnorm_weight_scales_each_feature():
    """[Intro §19.3]: gamma multiplies feature by feature after the common
    scale; dividing it out leaves a unit mean square."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 128))
    w = rng.uniform(0.5, 1.5, 128)
    y = oracle.rms_norm(x, w, 0.0)
    assert np.allclose(np.mean((y / w) ** 2, axis=-1), 1.0, rtol=1e-13)


def test_rmsnorm_is_per_head():
    """[Intro §12.2, §19.3, §19.8]: the q/k norm takes each head of each token
    on its own; scaling one head changes no other head's output."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 4, 128))
    y = oracle.rms_norm(x, None, 0.0)
    x2 = x.copy()
    x2[1, 2] *= 7.0
    y2 = oracle.rms_norm(x2, None, 0.0)
    assert np.max(np.abs(y - y2)) < 1e-14
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)


# ----------------------------------------------------------------------------- RoPE


def test_rotate_pair_page_example():
    """[Intro §19.7]: [1, 0] turned by 90 degrees is [0, 1], length still 1."""
    g = golden("intro_s19_7_rope_pair.json")
    a, b = oracle.rotate_pair(g["pair"][0], g["pair"][1], math.radians(g["phi_degrees"]))
    assert abs(a - g["rotated"][0]) < 1e-15 and abs(b - g["rotated"][1]) < 1e-15
    assert abs(math.hypot(a, b) - 1.0) < 1e-15


def test_rope_identity_at_position_zero():
    """[Intro §19.7]: the angle is the position times the frequency, so
    position 0 leaves every vector unchanged."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 128))
    assert np.array_equal(oracle.rope(x, [0, 0], 1e6), x)


def test_rope_half_split_pairs_and_unit_first_frequency():
    """[Intro §19.7; Analysis §4.4]: feature 0 pairs with feature 64 (not 1),
    and pair 0's frequency is theta**0 = 1, so position 1 turns it by one
    radian whatever theta is."""
    g = golden("intro_s19_7_rope_pair.json")
    d = g["head_dim"]
    x = np.zeros((1, 1, d))
    x[0, 0, 0] = 1.0
    for theta in (g["rope_theta"], 10000.0):
        y = oracle.rope(x, [1], theta)[0, 0]
        assert abs(y[0] - math.cos(1.0)) < 1e-15 and abs(y[d // 2] - math.sin(1.0)) < 1e-15
        others = np.delete(y, [0, d // 2])
        assert np.all(others == 0.0)
    # the second feature of the head pairs with feature d/2 + 1
    x = np.zeros((1, 1, d))
    x[0, 0, 1] = 1.0
    y = oracle.rope(x, [3], 1e6)[0, 0]
    assert set(np.nonzero(y)[0].tolist()) == set(g["pairs_of_feature_0_and_1"][1])


def test_rope_frequency_at_quarter_pair():
    """[Analysis §4.4]: pair i turns at theta**(-2i/d); pair d/4 therefore turns
    at theta**(-1/2) radians per position (0.01 for theta = 1e4, 0.001 for
    theta = 1e6), so positions 100 and 1000 turn it by exactly one radian."""
    d = 128
    for theta, p in ((1e4, 100), (1e6, 1000)):
        x = np.zeros((1, 1, d))
        x[0, 0, d // 4] = 1.0
        y = oracle.rope(x, [p], theta)[0, 0]
        assert abs(y[d // 4] - math.cos(1.0)) < 1e-12
        assert abs(y[d // 4 + d // 2] - math.sin(1.0)) < 1e-12


def test_rope_frequencies_are_geometric():
    """[Analysis §4.4]: successive pairs slow down by a constant factor, from
    1 at pair 0 to theta**(-(d-2)/d) at the last pair."""
    w = oracle.rope_frequencies(128, 1e6)
    assert w[0] == 1.0 and w.shape == (64,)
    ratio = w[1:] / w[:-1]
    assert np.allclose(ratio, ratio[0], rtol=1e-12, atol=0)
    assert abs(w[-1] - 1e6 ** (-126 / 128)) < 1e-18


def test_rope_preserves_pair_lengths():
    """[Intro §19.7]: a rotation keeps each pair's length."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 4, 128))
    y = oracle.rope(x, [0, 1, 17, 4095, 40959], 1e6)
    lx = np.hypot(x[..., :64], x[..., 64:])
    ly = np.hypot(y[..., :64], y[..., 64:])
    assert np.allclose(lx, ly, rtol=1e-13, atol=0)


def test_rope_dot_depends_on_relative_position():
    """[Intro §19.7]: q at p and k at j score by the angle difference, so
    shifting both positions by the same amount keeps q.k."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    dots = []
    for shift in (0, 1, 250, 3000):
        qr = oracle.rope(q, [5 + shift], 1e6)
        kr = oracle.rope(k, [9 + shift], 1e6)
        dots.append(float(np.sum(qr * kr)))
    assert np.allclose(dots, dots[0], rtol=1e-11, atol=1e-11)
    # ...but the offset itself matters
    far = float(np.sum(oracle.rope(q, [5], 1e6) * oracle.rope(k, [60], 1e6)))
    assert abs(far - dots[0]) > 1e-3


def test_rope_matches_complex_multiplication():
    """[Intro §19.7]: turning [a, b] by phi is multiplying a + ib by e^(i phi)."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 2, 64))
    pos = [2, 31, 777]
    w = oracle.rope_frequencies(64, 5e5)
    z = (x[..., :32] + 1j * x[..., 32:]) * np.exp(1j * np.outer(pos, w))[:, None, :]
    y = oracle.rope(x, pos, 5e5)
    assert np.allclose(y[..., :32], z.real, rtol=0, atol=1e-13)
    assert np.allclose(y[..., 32:], z.imag, rtol=0, atol=1e-13)


def test_norm_comes_before_rotation():
    """[Intro §12.2, §19.7]: Q and K are normalised, then rotated.  With a
    non-uniform gamma the order is visible: rotating after the norm keeps
    each pair's length as the normalised vector had it (position 0 output)."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 16, 128))
    k = rng.standard_normal((2, 8, 128))
    qw = rng.uniform(0.2, 2.0, 128)
    kw = rng.uniform(0.2, 2.0, 128)
    q0, k0 = oracle.qk_norm_rope(q, k, qw, kw, [0, 0], 1e-6, 1e6)
    q7, k7 = oracle.qk_norm_rope(q, k, qw, kw, [7, 300], 1e-6, 1e6)
    for a, b in ((q0, q7), (k0, k7)):
        la = np.hypot(a[..., :64], a[..., 64:])
        lb = np.hypot(b[..., :64], b[..., 64:])
        assert np.allclose(la, lb, rtol=1e-12, atol=0)
    # and position 0 is the plain per-head norm with each side's own gamma
    assert np.allclose(q0, oracle.rms_norm(q, qw, 1e-6), rtol=0, atol=1e-14)
    assert np.allclose(k0, oracle.rms_norm(k, kw, 1e-6), rtol=0, atol=1e-14)


def test_q_and_k_are_both_normalised_and_rotated():
    """[Intro §12.2, §19.3, §19.7]: a head holding one spike c at feature 0 has
    mean square c*c/d, so the norm (gamma 1, eps 0) makes the spike sqrt(d);
    position 1 then turns pair 0 by one radian -- for Q and for K alike."""
    d = 128
    q = np.zeros((1, 2, d))
    k = np.zeros((1, 1, d))
    q[0, :, 0] = [3.0, 0.25]
    k[0, 0, 0] = 40.0
    qr, kr = oracle.qk_norm_rope(q, k, None, None, [1], 0.0, 1e6)
    for y in (qr[0, 0], qr[0, 1], kr[0, 0]):
        assert abs(y[0] - math.sqrt(d) * math.cos(1.0)) < 1e-13
        assert abs(y[d // 2] - math.sqrt(d) * math.sin(1.0)) < 1e-13
        assert np.count_nonzero(y) == 2


# ----------------------------------------------------------------------------- split and store


def test_split_qkv_order():
    """[Analysis §4.2]: the fused projection row is Q heads, then K, then V."""
    hq, hkv, d = 4, 2, 8
    row = np.concatenate([np.full(d, 100 + h) for h in range(hq)]
                         + [np.full(d, 200 + h) for h in range(hkv)]
                         + [np.full(d, 300 + h) for h in range(hkv)])
    q, k, v = oracle.split_qkv(np.stack([row, row + 1000]), hq, hkv, d)
    assert q.shape == (2, hq, d) and k.shape == (2, hkv, d) and v.shape == (2, hkv, d)
    assert q[1, 3, 0] == 1103 and k[0, 1, 5] == 201 and v[1, 0, 7] == 1300


def test_store_routes_rotated_k_and_raw_v():
    """[Pico #8 §1; Intro §12.2, §19.7]: Q comes back as rotated values, the
    cache gets rotated K and the untouched V bits at each token's slot; slot -1
    writes nothing and every other slot keeps its bits."""
    rng = np.random.default_rng(12)
    hq, hkv, d, bs, nb = 4, 2, 16, 4, 3
    t = 3
    qkv = rng.standard_normal((t, (hq + 2 * hkv) * d)).astype(np.float32)
    qw = rng.uniform(0.5, 1.5, d).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, d).astype(np.float32)
    kc = f32_raw(rng.standard_normal((nb, bs, hkv, d)))
    vc = f32_raw(rng.standard_normal((nb, bs, hkv, d)))
    slots = [9, -1, 2]
    pos = [40, 41, 5]
    q_rot, k_rot, kc2, vc2 = oracle.qk_norm_rope_store(
        f32_raw(qkv), "f32", hq, hkv, d, f32_raw(qw), f32_raw(kw), pos, slots, 1e-6, 1e6, kc, vc)
    assert q_rot.shape == (t, hq, d) and k_rot.shape == (t, hkv, d)
    v_new = qkv[:, (hq + hkv) * d:].reshape(t, hkv, d)
    assert np.array_equal(vc2[9 // bs, 9 % bs], f32_raw(v_new[0]))
    assert np.array_equal(vc2[2 // bs, 2 % bs], f32_raw(v_new[2]))
    assert np.array_equal(kc2[9 // bs, 9 % bs], k_rot[0])
    assert np.array_equal(kc2[2 // bs, 2 % bs], k_rot[2])
    untouched = [s for s in range(nb * bs) if s not in (9, 2)]
    for s in untouched:
        assert np.array_equal(vc2[s // bs, s % bs], vc[s // bs, s % bs])
        assert np.array_equal(kc2[s // bs, s % bs], kc[s // bs, s % bs].view(np.float32))
    # V is neither normalised nor rotated; K is: its heads now have the norm's
    # mean square (through gamma) and differ from the raw K
    k_raw = qkv[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d).astype(np.float64)
    assert not np.allclose(k_rot, k_raw)
    lk = np.hypot(k_rot[..., : d // 2], k_rot[..., d // 2:])
    ln = oracle.rms_norm(k_raw, kw.astype(np.float64), 1e-6)
    assert np.allclose(lk, np.hypot(ln[..., : d // 2], ln[..., d // 2:]), rtol=1e-12)


def test_store_without_norm_weights_only_rotates():
    """[Analysis §4.2]: a model whose projection has a bias has no q/k norm;
    both weights absent means rotation only (position 0: Q unchanged)."""
    rng = np.random.default_rng(13)
    hq, hkv, d = 2, 1, 8
    qkv = rng.standard_normal((2, (hq + 2 * hkv) * d)).astype(np.float32)
    kc = np.zeros((1, 4, hkv, d), dtype=np.uint32)
    vc = np.zeros_like(kc)
    q_rot, k_rot, _, _ = oracle.qk_norm_rope_store(
        f32_raw(qkv), "f32", hq, hkv, d, None, None, [0, 2], [0, 1], 1e-6, 1e6, kc, vc)
    assert np.array_equal(q_rot[0], qkv[0, : hq * d].reshape(hq, d).astype(np.float64))
    expect = oracle.rope(qkv[1:2, : hq * d].reshape(1, hq, d), [2], 1e6)
    assert np.array_equal(q_rot[1:2], expect)

"""Pins of the oracle's building blocks against closed forms, hand-derived values,
invariants and brute-force loops.  CPU only."""

import math

import numpy as np
import pytest

from oracle import (causal_attention, layer_windows, linear, relu2, rms_norm, rope, rope_tables, sample,
                    softcap)


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RMSNorm -----------
def test_rms_norm_hand_value():
    # [3, 4]: mean square 12.5, so the result is [3, 4] / sqrt(12.5).
    y = rms_norm(np.array([3.0, 4.0]), 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    assert abs(y[0] - 0.848528137423857) < 1e-14
    assert abs(y[1] - 1.131370849898476) < 1e-14


def test_rms_norm_unit_rms_and_closed_form():
    x = rng().standard_normal((5, 7, 96)) * 3.7
    y = rms_norm(x, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=0, atol=1e-14)
    eps = 1e-2
    ms = np.mean(x * x, -1)
    y = rms_norm(x, eps)
    assert np.allclose(np.mean(y * y, -1), ms / (ms + eps), rtol=0, atol=1e-12)


def test_rms_norm_scale_invariance_and_direction():
    x = rng(1).standard_normal((4, 64))
    assert np.allclose(rms_norm(x * 123.0, 0.0), rms_norm(x, 0.0), atol=1e-14)
    # Output is a positive multiple of the input (no parameters, no shift).
    y = rms_norm(x, 1e-6)
    ratio = y / x
    assert np.all(ratio > 0)
    assert np.allclose(ratio, ratio[:, :1], rtol=1e-13)


# ---------------------------------------------------------------- RoPE --------------
def test_rope_hand_value_hd4():
    # hd = 4, base = 100: pair frequencies 100^0 = 1 and 100^(-1/2) = 0.1.
    # Pair (x0, x2) turns by 1 rad at position 1, pair (x1, x3) by 0.1 rad.
    cos, sin = rope_tables(3, 4, 100.0)
    x = np.array([1.0, 2.0, 3.0, 4.0])
    y = rope(x, 1, cos, sin)
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.1), math.sin(0.1)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 1 * s1 + 3 * c1, 2 * s2 + 4 * c2]
    assert np.allclose(y, want, rtol=0, atol=1e-15)
    # Position 2 turns by twice the angle.
    y2 = rope(x, 2, cos, sin)
    assert abs(y2[0] - (math.cos(2) - 3 * math.sin(2))) < 1e-15


def test_rope_hd2_is_plane_rotation():
    cos, sin = rope_tables(50, 2, 10000.0)
    for p in (0, 1, 7, 49):
        y = rope(np.array([1.0, 0.0]), p, cos, sin)
        assert np.allclose(y, [math.cos(p), math.sin(p)], atol=1e-15)


def test_rope_complex_form():
    # Pair i of (x_i, x_{i+hd/2}) read as x_i + j x_{i+hd/2} is multiplied by
    # exp(j p base^(-2i/hd)).
    hd, base = 128, 10000.0
    cos, sin = rope_tables(300, hd, base)
    x = rng(2).standard_normal(hd)
    for p in (0, 5, 299):
        y = rope(x, p, cos, sin)
        z = x[:hd // 2] + 1j * x[hd // 2:]
        theta = p * base ** (-np.arange(hd // 2) * 2.0 / hd)
        w = z * np.exp(1j * theta)
        assert np.allclose(y[:hd // 2], w.real, atol=1e-12)
        assert np.allclose(y[hd // 2:], w.imag, atol=1e-12)


def test_rope_invariants():
    hd = 64
    cos, sin = rope_tables(4096, hd, 10000.0)
    x = rng(3).standard_normal((10, hd))
    pos = np.arange(10) * 37
    y = rope(x, pos[:, None][:, 0], cos, sin)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    assert np.array_equal(rope(x, np.zeros(10, int), cos, sin), x)
    # composition: rope(rope(x, a), b) = rope(x, a + b)
    a, b = 123, 456
    assert np.allclose(rope(rope(x, a, cos, sin), b, cos, sin), rope(x, a + b, cos, sin),
                       atol=1e-12)
    # relative position: <rope(q, m), rope(k, n)> depends on m - n only.
    q, k = rng(4).standard_normal((2, hd))
    d1 = rope(q, 100, cos, sin) @ rope(k, 40, cos, sin)
    d2 = rope(q, 1100, cos, sin) @ rope(k, 1040, cos, sin)
    assert abs(d1 - d2) < 1e-11


def test_rope_then_norm_commutes():
    hd = 128
    cos, sin = rope_tables(64, hd, 10000.0)
    x = rng(5).standard_normal((16, hd))
    pos = np.arange(16)
    for eps in (0.0, 1e-6, 0.5):
        a = rms_norm(rope(x, pos, cos, sin), eps)
        b = rope(rms_norm(x, eps), pos, cos, sin)
        assert np.allclose(a, b, atol=1e-14)


# ---------------------------------------------------------------- ReLU^2, softcap ---
def test_relu2_values():
    z = np.array([-3.0, -0.0, 0.0, 0.5, 2.0])
    assert np.array_equal(relu2(z), [0.0, 0.0, 0.0, 0.25, 4.0])


def test_softcap_properties():
    cap = 15.0
    z = np.linspace(-2000, 2000, 40001)
    y = softcap(z, cap)
    assert np.all(np.abs(y) <= cap)
    assert np.all(np.diff(y) >= 0)  # monotone: argmax is unchanged
    small = np.linspace(-10, 10, 2001)
    err = np.abs(softcap(small, cap) - small)
    assert np.all(err <= np.abs(small) ** 3 / (3 * cap * cap) + 1e-15)
    assert softcap(np.array([0.0]), cap)[0] == 0.0
    # odd function, and tanh(1) at z = cap
    assert np.allclose(softcap(-z, cap), -y)
    assert abs(softcap(np.array([cap]), cap)[0] - cap * math.tanh(1.0)) < 1e-14
    v = rng(6).standard_normal((3, 100)) * 40
    assert np.array_equal(np.argmax(softcap(v, cap), -1), np.argmax(v, -1))


# ---------------------------------------------------------------- linear ------------
def test_linear_matches_loop():
    x = rng(7).standard_normal((3, 5))
    w = rng(8).standard_normal((4, 5))  # [out, in]
    y = linear(x, w)
    for i in range(3):
        for o in range(4):
            acc = 0.0
            for j in range(5):
                acc += x[i, j] * w[o, j]
            assert abs(y[i, o] - acc) < 1e-13


# ---------------------------------------------------------------- attention ---------
def brute_attention(q, k, v, q_pos, window=-1):
    """Triple loop from the definition: softmax over visible keys of q.k/sqrt(hd); with a
    window w >= 0 the visible keys of a query at position p are max(0, p - w) .. p."""
    tq, n_head, hd = q.shape
    n_kv = k.shape[1]
    out = np.zeros_like(q)
    for t in range(tq):
        for h in range(n_head):
            g = h * n_kv // n_head
            first = 0 if window < 0 else max(0, q_pos[t] - window)
            keys = list(range(first, q_pos[t] + 1))
            scores = []
            for j in keys:
                s = 0.0
                for c in range(hd):
                    s += q[t, h, c] * k[j, g, c]
                scores.append(s / math.sqrt(hd))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = sum(w)
            for c in range(hd):
                out[t, h, c] = sum(w[i] * v[j, g, c] for i, j in enumerate(keys)) / z
    return out


@pytest.mark.parametrize("n_head,n_kv", [(3, 1), (2, 2), (4, 2)])
def test_attention_brute_force(n_head, n_kv):
    r = rng(9)
    t, hd = 6, 8
    q = r.standard_normal((t, n_head, hd))
    k = r.standard_normal((t, n_kv, hd))
    v = r.standard_normal((t, n_kv, hd))
    pos = np.arange(t)
    assert np.allclose(causal_attention(q, k, v, pos), brute_attention(q, k, v, pos),
                       rtol=0, atol=1e-13)
    # queries placed later in a longer key sequence (decode form)
    q2 = r.standard_normal((2, n_head, hd))
    pos2 = np.array([3, 5])
    assert np.allclose(causal_attention(q2, k, v, pos2), brute_attention(q2, k, v, pos2),
                       rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [0, 1, 3])
@pytest.mark.parametrize("n_head,n_kv", [(3, 1), (4, 2)])
def test_windowed_attention_brute_force(n_head, n_kv, window):
    r = rng(11)
    t, hd = 7, 8
    q = r.standard_normal((t, n_head, hd))
    k = r.standard_normal((t, n_kv, hd))
    v = r.standard_normal((t, n_kv, hd))
    pos = np.arange(t)
    assert np.allclose(causal_attention(q, k, v, pos, window),
                       brute_attention(q, k, v, pos, window), rtol=0, atol=1e-13)
    q2 = r.standard_normal((2, n_head, hd))
    pos2 = np.array([4, 6])
    assert np.allclose(causal_attention(q2, k, v, pos2, window),
                       brute_attention(q2, k, v, pos2, window), rtol=0, atol=1e-13)


def test_window_special_cases():
    r = rng(12)
    t, hd = 6, 8
    q = r.standard_normal((t, 4, hd))
    k = r.standard_normal((t, 2, hd))
    v = r.standard_normal((t, 2, hd))
    pos = np.arange(t)
    # window 0: a query sees only its own key, so the output is its group's value
    y = causal_attention(q, k, v, pos, 0)
    assert np.allclose(y, np.repeat(v, 2, axis=1), rtol=0, atol=1e-15)
    # a window reaching past position 0 changes nothing
    full = causal_attention(q, k, v, pos)
    assert np.array_equal(causal_attention(q, k, v, pos, t - 1), full)
    assert np.array_equal(causal_attention(q, k, v, pos, 10 * t), full)
    # window 1 at position p: the two-key softmax in closed form
    y1 = causal_attention(q, k, v, pos, 1)
    p, h, g = 4, 3, 1
    s0 = q[p, h] @ k[p - 1, g] / math.sqrt(hd)
    s1 = q[p, h] @ k[p, g] / math.sqrt(hd)
    a = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.allclose(y1[p, h], a * v[p - 1, g] + (1 - a) * v[p, g], rtol=0, atol=1e-14)


def test_layer_windows_pattern():
    assert layer_windows("SSSL", 6, 128) == [128, 128, 128, -1, 128, 128]
    assert layer_windows("L", 3, 64) == [-1, -1, -1]
    assert layer_windows("SL", 3, 0) == [0, -1, 0]
    with pytest.raises(ValueError):
        layer_windows("SXL", 3, 8)


def test_attention_special_cases():
    r = rng(10)
    q = r.standard_normal((1, 3, 8))
    k = r.standard_normal((1, 1, 8))
    v = r.standard_normal((1, 1, 8))
    # one visible key: output is that value for every head
    y = causal_attention(q, k, v, np.array([0]))
    assert np.allclose(y, np.broadcast_to(v[0, 0], (1, 3, 8)), atol=1e-15)
    # identical keys: output is the mean of the visible values
    t = 5
    k = np.broadcast_to(r.standard_normal(8), (t, 1, 8)).copy()
    v = r.standard_normal((t, 1, 8))
    q = r.standard_normal((t, 2, 8))
    y = causal_attention(q, k, v, np.arange(t))
    for i in range(t):
        assert np.allclose(y[i], np.mean(v[:i + 1, 0], axis=0), atol=1e-14)


def test_attention_mqa_equals_replicated_mha():
    r = rng(11)
    t, h, hd = 7, 4, 16
    q = r.standard_normal((t, h, hd))
    k = r.standard_normal((t, 1, hd))
    v = r.standard_normal((t, 1, hd))
    pos = np.arange(t)
    mqa = causal_attention(q, k, v, pos)
    mha = causal_attention(q, np.repeat(k, h, axis=1), np.repeat(v, h, axis=1), pos)
    assert np.allclose(mqa, mha, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- sampling ----------
def test_sample_greedy_limits():
    r = rng(13)
    logits = r.standard_normal((6, 40)) * 3
    greedy = np.argmax(logits, -1)
    u = r.random(6)
    assert np.array_equal(sample(logits, 0.0, 0, u), greedy)        # temperature 0
    assert np.array_equal(sample(logits, 1.0, 1, u), greedy)        # top-1
    assert np.array_equal(sample(logits, 1e-4, 0, u), greedy)       # vanishing temperature
    assert np.array_equal(sample(logits, 0.7, 40, u), sample(logits, 0.7, 0, u))  # k = V


def test_sample_two_tokens_closed_form():
    l0, l1, t = 0.3, 1.1, 0.8
    p0 = 1.0 / (1.0 + math.exp((l1 - l0) / t))
    logits = np.array([[l0, l1]])
    for u in (0.0, p0 - 1e-9, p0 + 1e-9, 0.999):
        assert sample(logits, t, 0, np.array([u]))[0] == (0 if u < p0 else 1)


def test_sample_frequencies_on_a_grid():
    """u on a uniform grid of N points: token i is drawn for the points inside its slice of
    the cumulative distribution, so its count is N p_i within one."""
    r = rng(14)
    z = r.standard_normal(12)
    t, k, n = 1.3, 5, 20000
    keep = np.argsort(z)[::-1][:k]
    e = np.exp(z[keep] / t)
    probs = np.zeros(12)
    probs[keep] = e / e.sum()
    u = (np.arange(n) + 0.5) / n
    got = sample(np.broadcast_to(z, (n, 12)), t, k, u)
    counts = np.bincount(got, minlength=12)
    assert np.all(np.abs(counts - n * probs) <= 1.0)


def test_sample_ties_nan_and_inf():
    row = np.array([[1.0, 2.0, 2.0, 2.0, -np.inf, np.nan, 0.5]])
    # top-2 keeps every logit tied with the 2nd largest: three equal tokens
    drawn = {int(sample(row, 1.0, 2, np.array([u]))[0]) for u in (0.1, 0.5, 0.9)}
    assert drawn == {1, 2, 3}
    # NaN and -inf never drawn, even at the top of the distribution
    assert sample(row, 5.0, 0, np.array([0.999999]))[0] == 6
    assert sample(np.array([[-np.inf, np.nan]]), 1.0, 0, np.array([0.5]))[0] == 0

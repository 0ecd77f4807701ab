"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages state (fixtures under tests/golden/), closed forms, invariants the pages
name (p-RoPE leaves 75 % of dims alone and preserves norms, rotated q.k depends
only on the offset, a window >= T is full causal, GQA equals repeated KV heads,
masks equal brute-force enumeration), textbook special cases and a library
routine (torch CPU fp64 scaled_dot_product_attention).

Pairing convention (adjacent dims vs. half split) and the frequency denominator
are readings the pages do not fix: parity unpinned for those two choices; the
tests below pin everything else about the rotation.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import inputs
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- RoPE ----

@pytest.mark.parametrize("case", _gold("prope_dims.json")["cases"])
def test_prope_untouched_dims_from_pages(case):
    """p = 0.25: exactly the first quarter of dims move, the rest are
    bit-identical at every position (p-RoPE section of the pages)."""
    g = _gold("prope_dims.json")
    D = case["head_dim"]
    R = int(g["p"] * D)
    assert R == case["rotated_dims"] and D - R == case["unrotated_dims"]
    x = rng.standard_normal((6, 3, D))
    pos = [0, 1, 7, 1000, 65536, 131072]
    y = oracle.rope(x, pos, R, g["theta"])
    assert np.array_equal(y[:, :, R:], x[:, :, R:])
    # every rotated pair actually moves at a nonzero position (pair 0 turns by
    # `pos` radians, so it moves whenever pos is not a multiple of 2*pi)
    assert np.all(np.abs(y[1:, :, :2] - x[1:, :, :2]).sum(-1) > 0)


def test_rope_identity_at_position_zero_and_p_zero():
    x = rng.standard_normal((4, 2, 64))
    assert np.array_equal(oracle.rope(x, [0] * 4, 64, 1e4), x)
    assert np.array_equal(oracle.rope(x, [5, 9, 100, 7], 0, 1e4), x)


def test_rope_preserves_pair_norms():
    x = rng.standard_normal((5, 4, 128))
    y = oracle.rope(x, [3, 17, 255, 4096, 131072], 128, 1e6)
    nx = np.hypot(x[..., 0::2], x[..., 1::2])
    ny = np.hypot(y[..., 0::2], y[..., 1::2])
    np.testing.assert_allclose(ny, nx, rtol=1e-12, atol=0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-12)


@pytest.mark.parametrize("D,R,theta", [(128, 32, 1e6), (512, 128, 1e6), (256, 256, 1e4)])
def test_rope_relative_position(D, R, theta):
    """(R_m q).(R_n k) depends only on n - m (shift both by c)."""
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for m, n, c in [(0, 5, 11), (100, 37, 1000), (4000, 4095, 60000), (7, 7, 123456)]:
        a = np.dot(oracle.rope(q, [m], R, theta).ravel(), oracle.rope(k, [n], R, theta).ravel())
        b = np.dot(oracle.rope(q, [m + c], R, theta).ravel(), oracle.rope(k, [n + c], R, theta).ravel())
        assert abs(a - b) <= 1e-9 * (1 + abs(a))


@pytest.mark.parametrize("D,R,theta", [(16, 16, 1e4), (128, 32, 1e6), (512, 128, 1e6)])
def test_rope_matches_textbook_complex_form(D, R, theta):
    """Textbook RoPE: view dims (2p, 2p+1) as z_p = x_2p + i x_2p+1 and
    multiply by exp(i * pos * theta^(-2p/D)); p-RoPE keeps that for the first
    R/2 pairs and leaves the remaining pairs unrotated."""
    x = rng.standard_normal((3, 2, D))
    pos = [1, 250, 131072]
    y = oracle.rope(x, pos, R, theta)
    for n, m in enumerate(pos):
        for h in range(2):
            for p in range(D // 2):
                z = complex(x[n, h, 2 * p], x[n, h, 2 * p + 1])
                if p < R // 2:
                    z *= cmath.exp(1j * m * theta ** (-2.0 * p / D))
                assert abs(z.real - y[n, h, 2 * p]) < 1e-9
                assert abs(z.imag - y[n, h, 2 * p + 1]) < 1e-9


def test_rope_frequency_schedule():
    """Angles at position 1 recovered by atan2: pair 0 turns by exactly 1 rad,
    consecutive pairs form a geometric series of ratio theta^(-2/D) (so the
    frequency decreases along the vector), and pairs past R/2 do not turn."""
    D, R, theta = 64, 48, 1e4
    x = np.zeros((1, D // 2, D))
    for p in range(D // 2):
        x[0, p, 2 * p] = 1.0  # unit vector on pair p, one head per pair
    y = oracle.rope(x, [1], R, theta)
    ang = np.array([math.atan2(y[0, p, 2 * p + 1], y[0, p, 2 * p]) for p in range(D // 2)])
    assert abs(ang[0] - 1.0) < 1e-15
    ratio = ang[1:R // 2] / ang[:R // 2 - 1]
    np.testing.assert_allclose(ratio, theta ** (-2.0 / D), rtol=1e-12)
    assert np.all(ang[R // 2:] == 0.0)


def test_rope_large_position_closed_form():
    """Pair 0 at position 131072 turns by 131072 rad: compare with math.cos/sin."""
    x = np.zeros((1, 1, 8))
    x[0, 0, 0] = 1.0
    y = oracle.rope(x, [131072], 8, 1e6)
    assert abs(y[0, 0, 0] - math.cos(131072.0)) < 1e-12
    assert abs(y[0, 0, 1] - math.sin(131072.0)) < 1e-12


# ------------------------------------------------------------ the masks ----

def _visible_sets(T, W):
    """Read the oracle's effective mask: scale 0 makes every visible key weigh
    the same, and one-hot values V = I report each key's weight."""
    q = rng.standard_normal((1, T, 1, 4))
    k = rng.standard_normal((1, T, 1, 4))
    v = np.eye(T).reshape(1, T, 1, T)
    o = oracle.prefill(q, k, v, window=W, scale=0.0, rotary_dims=0)[0, :, 0, :]
    return o


@pytest.mark.parametrize("T", [1, 2, 7, 33, 64])
def test_mask_brute_force(T):
    for W in sorted({1, 2, 3, max(1, T - 1), T, T + 5, 0}):
        o = _visible_sets(T, W)
        for i in range(T):
            allowed = [j for j in range(T) if j <= i and (W == 0 or i - j < W)]
            expect = np.zeros(T)
            expect[allowed] = 1.0 / len(allowed)
            np.testing.assert_allclose(o[i], expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", _gold("window_ranges.json")["cases"])
def test_window_ranges_from_pages(case):
    """First/last visible key for the window sizes the pages give."""
    W, i = case["window"], case["query"]
    T = i + 1
    # Only row i matters: ask the oracle for that one row, keys 0..i.
    q = np.zeros((1, 1, 1, 1))
    k = np.zeros((1, T, 1, 1))
    v = np.arange(T, dtype=np.float64).reshape(1, T, 1, 1)
    v2 = v ** 2
    vv = np.concatenate([np.ones_like(v), v, v2], axis=3)
    o = oracle.prefill(q, k, vv, window=W, scale=1.0, rotary_dims=0, rows=[i])[0, 0, 0]
    # Uniform weights over keys a..b: mean = (a+b)/2, count from the variance.
    a, b = case["first_key"], case["last_key"]
    assert abs(o[0] - 1.0) < 1e-12
    assert abs(o[1] - (a + b) / 2) < 1e-9
    n = b - a + 1
    assert abs(o[2] - (o[1] ** 2 + (n * n - 1) / 12.0)) < 1e-6 * (1 + o[2])


def test_window_at_least_T_is_causal():
    B, T, H, D = 2, 40, 2, 16
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    causal = oracle.prefill(q, k, v, window=0, scale=0.3, rotary_dims=16, theta=1e4)
    for W in (T, T + 1, 10 * T):
        np.testing.assert_array_equal(
            oracle.prefill(q, k, v, window=W, scale=0.3, rotary_dims=16, theta=1e4), causal)


# ------------------------------------------------- softmax closed forms ----

def test_window_one_returns_own_value():
    B, T, H, D = 1, 20, 3, 8
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    o = oracle.prefill(q, k, v, window=1, scale=0.7, rotary_dims=8, theta=1e4)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


def test_constant_values_give_constant_output():
    B, T, H, D = 1, 30, 2, 8
    q, k = rng.standard_normal((B, T, H, D)), rng.standard_normal((B, T, H, D))
    v = np.full((B, T, H, 5), 3.25)
    o = oracle.prefill(q, k, v, window=7, scale=1.3, rotary_dims=8, theta=1e4)
    np.testing.assert_allclose(o, 3.25, rtol=1e-14)


def test_zero_scale_gives_mean_of_visible_values():
    """scale = 0 makes every visible key weigh the same: o_i is the plain mean
    of v_j over j in (i - W, i]."""
    B, T, Hq, Hkv, D = 2, 23, 4, 2, 8
    q, k = rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, 6))
    for W in (0, 5):
        o = oracle.prefill(q, k, v, window=W, scale=0.0, rotary_dims=8, theta=1e4)
        for i in range(T):
            lo = 0 if W == 0 else max(0, i - W + 1)
            mean = v[:, lo:i + 1].mean(axis=1)               # [B, Hkv, 6]
            np.testing.assert_allclose(o[:, i], np.repeat(mean, Hq // Hkv, axis=1),
                                       rtol=0, atol=1e-13)


def test_first_token_sees_only_itself():
    q, k, v = (rng.standard_normal((2, 5, 4, 8)) for _ in range(3))
    o = oracle.prefill(q, k, v, window=0, scale=0.5, rotary_dims=8, theta=1e6)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-14)


def test_two_token_closed_form():
    """Row 1 of a 2-token, 1-dim problem without RoPE: weights
    e^{s q k_j} / (e^{s q k_0} + e^{s q k_1})."""
    q = np.array([0.0, 1.5]).reshape(1, 2, 1, 1)
    k = np.array([0.4, -0.9]).reshape(1, 2, 1, 1)
    v = np.array([2.0, -1.0]).reshape(1, 2, 1, 1)
    s = 0.8
    o = oracle.prefill(q, k, v, window=0, scale=s, rotary_dims=0)[0, 1, 0, 0]
    e0, e1 = math.exp(s * 1.5 * 0.4), math.exp(s * 1.5 * -0.9)
    assert abs(o - (2.0 * e0 - 1.0 * e1) / (e0 + e1)) < 1e-14


# ----------------------------------------------- library routine + GQA ----

def _torch_sdpa(q, k, v, W, scale, G):
    """torch CPU fp64 SDPA with repeat_interleave'd KV and a boolean mask."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)  # B H T D
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    T = q.shape[1]
    i = torch.arange(T).view(T, 1)
    j = torch.arange(T).view(1, T)
    mask = j <= i
    if W > 0:
        mask &= (i - j) < W
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("B,T,Hq,Hkv,Dk,Dv,W", [
    (1, 9, 1, 1, 8, 8, 0), (2, 33, 4, 2, 16, 8, 5), (1, 40, 8, 1, 32, 16, 0),
    (2, 17, 6, 3, 8, 12, 1), (1, 64, 16, 8, 16, 16, 20)])
def test_oracle_matches_torch_sdpa(B, T, Hq, Hkv, Dk, Dv, W):
    q = rng.standard_normal((B, T, Hq, Dk))
    k = rng.standard_normal((B, T, Hkv, Dk))
    v = rng.standard_normal((B, T, Hkv, Dv))
    scale = 1 / math.sqrt(Dk)
    ref = _torch_sdpa(q, k, v, W, scale, Hq // Hkv)
    o = oracle.prefill(q, k, v, window=W, scale=scale, rotary_dims=0)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_oracle_with_rope_matches_torch_on_prerotated_inputs():
    """RoPE inside the oracle equals rotating q and k first (positions pos0+t)
    and running the library routine without RoPE."""
    B, T, Hq, Hkv, D, R, theta, pos0 = 1, 24, 4, 1, 32, 8, 1e6, 1000
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    pos = np.arange(T) + pos0
    qr = oracle.rope(q[0], pos, R, theta)[None]
    kr = oracle.rope(k[0], pos, R, theta)[None]
    ref = _torch_sdpa(qr, kr, v, 0, 0.2, Hq // Hkv)
    o = oracle.prefill(q, k, v, window=0, scale=0.2, rotary_dims=R, theta=theta, pos0=pos0)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_gqa_equals_repeated_heads():
    B, T, Hq, Hkv, D = 2, 21, 8, 2, 16
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    v = rng.standard_normal((B, T, Hkv, D))
    kw = dict(window=6, scale=0.25, rotary_dims=8, theta=1e6)
    a = oracle.prefill(q, k, v, **kw)
    b = oracle.prefill(q, np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2), **kw)
    np.testing.assert_array_equal(a, b)


def test_position_offset_invariance():
    """Rotating q and k with a common offset pos0 leaves every score, hence
    every output, unchanged (relative-position property)."""
    q, k, v = (rng.standard_normal((1, 16, 2, 32)) for _ in range(3))
    kw = dict(window=0, scale=0.3, rotary_dims=32, theta=1e4)
    np.testing.assert_allclose(oracle.prefill(q, k, v, pos0=0, **kw),
                               oracle.prefill(q, k, v, pos0=5000, **kw), atol=1e-11)


def test_row_subset_equals_full():
    q, k, v = (rng.standard_normal((2, 30, 4, 16)) for _ in range(3))
    kw = dict(window=7, scale=0.3, rotary_dims=16, theta=1e4)
    full = oracle.prefill(q, k, v, **kw)
    rows = [0, 6, 7, 29, 13]
    sub = oracle.prefill(q[:, rows], k, v, rows=rows, **kw)
    np.testing.assert_array_equal(sub, full[:, rows])


# ------------------------------------------------- K = V (keys as values) ----
# Reading: the values are the keys after RoPE, the rows the cache holds.

def test_kv_shared_first_token_returns_its_own_key():
    """Token 0 sees only itself and RoPE at position 0 is the identity, so its
    output is its own unrotated key (per KV head, for each of its G heads)."""
    q = rng.standard_normal((2, 5, 8, 16))
    k = rng.standard_normal((2, 5, 2, 16))
    o = oracle.prefill_kv_shared(q, k, window=0, scale=0.3, rotary_dims=8, theta=1e4)
    np.testing.assert_allclose(o[:, 0], np.repeat(k[:, 0], 4, axis=1), atol=1e-14)


def test_kv_shared_two_token_closed_form():
    """One rotary pair (D = 2): its frequency is 1 under any schedule, so
    rope(x, pos) = x e^{i pos} as a complex number. Row 1 weights the rotated
    keys r_0 = k_0, r_1 = k_1 e^{i}; scores are Re(q_1 e^{i} conj(r_j))."""
    q1, k0, k1, s = complex(0.7, -1.1), complex(0.4, 0.9), complex(-1.3, 0.2), 0.8
    q = np.array([[0.0, 0.0], [q1.real, q1.imag]]).reshape(1, 2, 1, 2)
    k = np.array([[k0.real, k0.imag], [k1.real, k1.imag]]).reshape(1, 2, 1, 2)
    o = oracle.prefill_kv_shared(q, k, window=0, scale=s, rotary_dims=2, theta=1e6)[0, 1, 0]
    rot = cmath.exp(1j)
    r0, r1, qr = k0, k1 * rot, q1 * rot
    s0, s1 = s * (qr * r0.conjugate()).real, s * (qr * r1.conjugate()).real
    e0, e1 = math.exp(s0), math.exp(s1)
    want = (e0 * r0 + e1 * r1) / (e0 + e1)
    assert abs(complex(o[0], o[1]) - want) < 1e-14


def test_kv_shared_zero_scale_is_mean_of_visible_rotated_keys():
    """Equal weights: o_i is the mean of the rotated keys i sees (window 3)."""
    T, D, R, th = 9, 8, 4, 1e4
    q = rng.standard_normal((1, T, 2, D))
    k = rng.standard_normal((1, T, 1, D))
    o = oracle.prefill_kv_shared(q, k, window=3, scale=0.0, rotary_dims=R, theta=th)
    kr = oracle.rope(k[0], np.arange(T), R, th)[:, 0]
    for i in range(T):
        want = kr[max(0, i - 2):i + 1].mean(axis=0)
        np.testing.assert_allclose(o[0, i, 0], want, atol=1e-14)
        np.testing.assert_allclose(o[0, i, 1], want, atol=1e-14)


def test_kv_shared_matches_torch_sdpa_with_rotated_keys_as_values():
    B, T, Hq, Hkv, D, W, R, th = 2, 30, 8, 1, 16, 0, 4, 1e6
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    pos = np.tile(np.arange(T), B)
    qr = oracle.rope(q.reshape(B * T, Hq, D), pos, R, th).reshape(B, T, Hq, D)
    kr = oracle.rope(k.reshape(B * T, Hkv, D), pos, R, th).reshape(B, T, Hkv, D)
    o = oracle.prefill_kv_shared(q, k, window=W, scale=0.25, rotary_dims=R, theta=th)
    np.testing.assert_allclose(o, _torch_sdpa(qr, kr, kr, W, 0.25, Hq // Hkv), atol=1e-12)


def test_kv_shared_output_stays_in_the_keys_hull():
    """A convex combination of rotated keys: no coordinate leaves the range the
    visible keys span, and RoPE keeps key norms, so |o_i| <= max_j |k_j|."""
    q = rng.standard_normal((1, 40, 4, 32)) * 3
    k = rng.standard_normal((1, 40, 2, 32))
    o = oracle.prefill_kv_shared(q, k, window=0, scale=1.0, rotary_dims=32, theta=1e4)
    kmax = np.linalg.norm(k, axis=-1).max()
    assert np.linalg.norm(o, axis=-1).max() <= kmax + 1e-12


@pytest.mark.parametrize("W", [0, 7])
def test_kv_shared_decode_equals_last_prefill_row(W):
    """Decode with one cache passed as both K and V (rotated keys) equals the
    last row of the K = V prefill over the same tokens."""
    L, Hq, Hkv, D, R, th = 25, 8, 1, 16, 4, 1e6
    q = rng.standard_normal((1, L + 1, Hq, D))
    k = rng.standard_normal((1, L + 1, Hkv, D))
    ref = oracle.prefill_kv_shared(q, k, window=W, scale=0.3, rotary_dims=R, theta=th)[0, L]
    kr = oracle.rope(k[0], np.arange(L + 1), R, th)
    out = oracle.decode(q[:, L], kr, kr, [0], [L + 1], window=W, scale=0.3,
                        rotary_dims=R, theta=th)[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- decode ----

@pytest.mark.parametrize("W", [0, 1, 5, 64])
def test_decode_equals_last_prefill_row(W):
    """Decode at kv_len = L+1 with pre-rotated cache keys equals the last row
    of a prefill over the same L+1 tokens that rotates keys itself."""
    L, Hq, Hkv, Dk, Dv, R, theta = 40, 8, 2, 32, 16, 16, 1e6
    q = rng.standard_normal((1, L + 1, Hq, Dk))
    k = rng.standard_normal((1, L + 1, Hkv, Dk))
    v = rng.standard_normal((1, L + 1, Hkv, Dv))
    ref = oracle.prefill(q, k, v, window=W, scale=0.2, rotary_dims=R, theta=theta)[0, L]
    k_rot = oracle.rope(k[0], np.arange(L + 1), R, theta)
    out = oracle.decode(q[:, L], k_rot, v[0], [0], [L + 1], window=W, scale=0.2,
                        rotary_dims=R, theta=theta)[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_decode_ragged_and_empty():
    Hq, Hkv, D = 4, 2, 8
    lens = [0, 1, 9, 30]
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    kc = rng.standard_normal((sum(lens), Hkv, D))
    vc = rng.standard_normal((sum(lens), Hkv, D))
    q = rng.standard_normal((4, Hq, D))
    out = oracle.decode(q, kc, vc, offs, lens, window=4, scale=0.5, rotary_dims=8, theta=1e4)
    assert np.all(out[0] == 0.0)
    np.testing.assert_allclose(out[1], np.repeat(vc[0], Hq // Hkv, axis=0), atol=1e-14)
    for b in (2, 3):
        n = lens[b]
        full = oracle.decode_one(q[b], kc[offs[b]:offs[b] + n], vc[offs[b]:offs[b] + n],
                                 kv_len=n, row0=0, window=4, scale=0.5, rotary_dims=8, theta=1e4)
        np.testing.assert_allclose(out[b], full, atol=1e-14)


def test_decode_rejects_visible_rows_before_row0():
    q = rng.standard_normal((2, 8))
    kc = rng.standard_normal((5, 1, 8))
    with pytest.raises(RuntimeError):
        oracle.decode_one(q, kc, kc, kv_len=10, row0=5, window=6, scale=1.0)


# ------------------------------------------------ verify (several tokens) ----

def test_verify_one_token_is_decode():
    lens, Hq, Hkv, D = [3, 17, 40], 8, 2, 16
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    kc = rng.standard_normal((sum(lens), Hkv, D))
    vc = rng.standard_normal((sum(lens), Hkv, D))
    q = rng.standard_normal((3, Hq, D))
    a = oracle.decode(q, kc, vc, offs, lens, window=5, scale=0.3, rotary_dims=8, theta=1e4)
    b = oracle.verify(q[:, None], kc, vc, offs, lens, window=5, scale=0.3, rotary_dims=8,
                      theta=1e4)
    np.testing.assert_allclose(b[:, 0], a, rtol=0, atol=1e-14)


@pytest.mark.parametrize("W", [0, 3, 9])
def test_verify_rows_equal_the_last_prefill_rows(W):
    """The n_q new tokens of a sequence are the last n_q rows of a prefill
    over the whole sequence (keys cached rotated, queries unrotated)."""
    T, n_q, Hq, Hkv, D, R, th = 30, 5, 4, 2, 16, 8, 1e6
    q = rng.standard_normal((1, T, Hq, D))
    k = rng.standard_normal((1, T, Hkv, D))
    v = rng.standard_normal((1, T, Hkv, D))
    ref = oracle.prefill(q, k, v, window=W, scale=0.25, rotary_dims=R, theta=th)[0, T - n_q:]
    kr = oracle.rope(k[0], np.arange(T), R, th)
    out = oracle.verify(q[:, T - n_q:], kr, v[0], [0], [T], window=W, scale=0.25,
                        rotary_dims=R, theta=th)[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_verify_first_draft_token_ignores_later_ones():
    """Causal within the draft: changing the rows of later new tokens leaves
    token 0's output alone, and token n_q-1 sees them all."""
    T, n_q, D = 12, 3, 8
    kc = rng.standard_normal((T, 1, D))
    vc = rng.standard_normal((T, 1, D))
    q = rng.standard_normal((1, n_q, 2, D))
    a = oracle.verify(q, kc, vc, [0], [T], window=0, scale=0.5)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[T - 2:] += 3.0
    vc2[T - 2:] -= 5.0
    b = oracle.verify(q, kc2, vc2, [0], [T], window=0, scale=0.5)
    np.testing.assert_allclose(a[0, 0], b[0, 0], rtol=0, atol=1e-14)
    assert np.abs(a[0, 1] - b[0, 1]).max() > 1e-3 and np.abs(a[0, 2] - b[0, 2]).max() > 1e-3


# ------------------------------------- drafter cross-attention into a cache ----

def _drafter_cache(T, Hkv, D, R, th):
    """Cache rows 0..T-1 built from unrotated keys turned at their positions."""
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    return k, oracle.rope(k, np.arange(T), R, th), v


def test_cross_attend_at_the_cache_end_is_decode():
    """A query at position kv_len - 1 over the cache is a plain decode (the C
    path), for every window."""
    lens, Hq, Hkv, D = [3, 17, 40], 8, 2, 16
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    kc = rng.standard_normal((sum(lens), Hkv, D))
    vc = rng.standard_normal((sum(lens), Hkv, D))
    q = rng.standard_normal((3, Hq, D))
    for W in (0, 1, 5, 100):
        a = oracle.decode(q, kc, vc, offs, lens, window=W, scale=0.3, rotary_dims=8, theta=1e4)
        b = oracle.cross_attend(q, kc, vc, offs, lens, [n - 1 for n in lens], window=W,
                                scale=0.3, rotary_dims=8, theta=1e4)
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)


def test_cross_attend_depends_on_relative_positions():
    """Without a window only q_pos - (key position) enters: shifting the query
    and every cached key by s leaves the output unchanged, and moving the
    query alone changes it."""
    T, Hq, Hkv, D, R, th, s = 20, 4, 2, 16, 16, 1e4, 37
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    q = rng.standard_normal((1, Hq, D))
    a = oracle.cross_attend(q, oracle.rope(k, np.arange(T), R, th), v, [0], [T], [T + 2],
                            window=0, scale=0.4, rotary_dims=R, theta=th)
    b = oracle.cross_attend(q, oracle.rope(k, np.arange(T) + s, R, th), v, [0], [T], [T + 2 + s],
                            window=0, scale=0.4, rotary_dims=R, theta=th)
    c = oracle.cross_attend(q, oracle.rope(k, np.arange(T), R, th), v, [0], [T], [T + 5],
                            window=0, scale=0.4, rotary_dims=R, theta=th)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    assert np.abs(a - c).max() > 1e-3


def test_cross_attend_window_edge():
    """Query at p past the cache, window W: row p - W + 1 is the first visible
    one. Poisoning the rows before it (NaN) changes nothing; changing that row
    changes the output."""
    T, Hq, Hkv, D, R, th, W, p = 30, 2, 1, 8, 8, 1e4, 10, 31
    _, kc, vc = _drafter_cache(T, Hkv, D, R, th)
    q = rng.standard_normal((1, Hq, D))
    kw = dict(window=W, scale=0.5, rotary_dims=R, theta=th)
    a = oracle.cross_attend(q, kc, vc, [0], [T], [p], **kw)
    kp, vp = kc.copy(), vc.copy()
    kp[: p - W + 1] = np.nan
    vp[: p - W + 1] = np.nan
    b = oracle.cross_attend(q, kp, vp, [0], [T], [p], **kw)
    np.testing.assert_allclose(a, b, rtol=0, atol=0)
    vc2 = vc.copy()
    vc2[p - W + 1] += 4.0
    c = oracle.cross_attend(q, kc, vc2, [0], [T], [p], **kw)
    assert np.abs(a - c).max() > 1e-3


@pytest.mark.parametrize("W", [0, 7])
def test_cross_attend_past_the_cache_is_a_narrower_decode(W):
    """A query d positions past the cache end equals the decode (C path, no
    rotation) of the query turned at its own position, with the window
    narrowed by d: the rows it may see are the cache's last W - d."""
    T, Hq, Hkv, D, R, th = 25, 4, 1, 16, 16, 1e6
    _, kc, vc = _drafter_cache(T, Hkv, D, R, th)
    q = rng.standard_normal((1, Hq, D))
    for d in (1, 2, 3):
        a = oracle.cross_attend(q, kc, vc, [0], [T], [T - 1 + d], window=W, scale=0.3,
                                rotary_dims=R, theta=th)
        qr = oracle.rope(q, [T - 1 + d], R, th)
        b = oracle.decode(qr, kc, vc, [0], [T], window=(W - d if W > 0 else 0), scale=0.3)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ----------------------------------------------------- 2-D RoPE (patches) ----

def test_rope_2d_one_pair_per_half_closed_form():
    """D = 4: pair 0 of each half turns by its coordinate in radians (pair 0
    has frequency 1 under any schedule)."""
    x = rng.standard_normal((3, 2, 4))
    pxy = np.array([[0, 0], [3, 1], [7, 12]])
    y = oracle.rope_2d(x, pxy, 2, 1e4)
    for n in range(3):
        for hh in range(2):
            a = complex(x[n, hh, 0], x[n, hh, 1]) * cmath.exp(1j * pxy[n, 0])
            b = complex(x[n, hh, 2], x[n, hh, 3]) * cmath.exp(1j * pxy[n, 1])
            assert abs(complex(y[n, hh, 0], y[n, hh, 1]) - a) < 1e-13
            assert abs(complex(y[n, hh, 2], y[n, hh, 3]) - b) < 1e-13


def test_rope_2d_each_half_follows_its_own_coordinate():
    x = rng.standard_normal((4, 3, 32))
    pxy = np.array([[5, 9], [0, 4], [7, 0], [2, 2]])
    y = oracle.rope_2d(x, pxy, 8, 1e4)                           # 8 of each half's 16 dims
    np.testing.assert_array_equal(y[1, :, :16], x[1, :, :16])   # x = 0: first half still
    np.testing.assert_array_equal(y[2, :, 16:], x[2, :, 16:])   # y = 0: second half still
    pxy2 = pxy.copy()
    pxy2[:, 1] += 6                                              # move y only
    y2 = oracle.rope_2d(x, pxy2, 8, 1e4)
    np.testing.assert_array_equal(y2[:, :, :16], y[:, :, :16])
    assert np.abs(y2[:, :, 16:] - y[:, :, 16:]).max() > 1e-3
    # dims past rotary_dims in each half are untouched, norms per half kept
    np.testing.assert_array_equal(y[:, :, 8:16], x[:, :, 8:16])
    np.testing.assert_array_equal(y[:, :, 24:], x[:, :, 24:])
    for s0 in (slice(0, 16), slice(16, 32)):
        np.testing.assert_allclose(np.linalg.norm(y[:, :, s0], axis=-1),
                                   np.linalg.norm(x[:, :, s0], axis=-1), rtol=1e-13)


def test_rope_2d_scores_depend_only_on_the_offset():
    """<R(x1, y1) q, R(x2, y2) k> depends only on (x2 - x1, y2 - y1)."""
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    def score(a, b):
        return float(np.sum(oracle.rope_2d(q, [a], 64 // 2, 100.0) *
                            oracle.rope_2d(k, [b], 64 // 2, 100.0)))
    s0 = score((3, 4), (10, 6))
    for dx, dy in [(5, 0), (0, 9), (17, 23)]:
        assert abs(score((3 + dx, 4 + dy), (10 + dx, 6 + dy)) - s0) < 1e-10
    assert abs(score((3, 4), (10, 7)) - s0) > 1e-6


# ------------------------------------------------------------ int8 cache ----
# The scheme (per row and head, symmetric, scale = max|x| / 127) is this
# build's reading: the pages give none, so the scheme itself is parity unpinned;
# these pins fix that the codes realise it.

def test_kv_quantize_int8_bounds_and_extremes():
    x = rng.standard_normal((50, 3, 64)).astype(np.float32) * rng.uniform(0.01, 50, (50, 3, 1)).astype(np.float32)
    x[7, 1] = 0.0
    codes, s = oracle.kv_quantize_int8(x)
    assert codes.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(codes.astype(int)).max() <= 127
    amax = np.abs(x).max(-1)
    np.testing.assert_allclose(s, amax / 127, rtol=1e-7)
    # the largest magnitude of each (row, head) lands on +-127 with its sign
    idx = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0].astype(int)
    sign = np.sign(np.take_along_axis(x, idx[..., None], -1)[..., 0]).astype(int)
    ok = amax > 0
    assert np.all(top[ok] == 127 * sign[ok])
    # round to nearest: dequantised error at most half a step (+ fp32 slack)
    err = np.abs(oracle.kv_dequantize_int8(codes, s) - x)
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-5))
    assert np.all(codes[7, 1] == 0) and s[7, 1] == 0


def test_kv_quantize_int8_exact_grid_and_ties():
    """Values already on the grid come back exactly; exact half steps round
    to even."""
    s0 = np.float32(0.25)
    k = np.arange(-127, 128, dtype=np.float32)
    x = (k * s0).reshape(1, 1, -1)
    codes, s = oracle.kv_quantize_int8(x)
    assert s[0, 0] == np.float32(127 * 0.25 / 127)
    np.testing.assert_array_equal(codes[0, 0].astype(int), k.astype(int))
    x2 = np.array([[[127.0, 0.5, 1.5, 2.5, -0.5, -1.5]]], dtype=np.float32)  # s = 1
    c2, _ = oracle.kv_quantize_int8(x2)
    assert c2[0, 0].tolist() == [127, 0, 2, 2, 0, -2]


def test_decode_int8_equals_decode_of_dequantised_cache():
    lens, Hq, Hkv, D = [5, 40], 4, 2, 16
    offs = [0, 5]
    kc = rng.standard_normal((45, Hkv, D))
    vc = rng.standard_normal((45, Hkv, D))
    q = rng.standard_normal((2, Hq, D))
    kq, ks = oracle.kv_quantize_int8(kc)
    vq, vs = oracle.kv_quantize_int8(vc)
    a = oracle.decode_int8(q, kq, ks, vq, vs, offs, lens, window=0, scale=0.3)
    b = oracle.decode(q, kq.astype(np.float64) * ks[..., None], vq.astype(np.float64) * vs[..., None],
                      offs, lens, window=0, scale=0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
    # and stays within the quantisation error of the unquantised decode
    c = oracle.decode(q, kc, vc, offs, lens, window=0, scale=0.3)
    assert np.abs(a - c).max() < 0.05


def test_workload_shapes_follow_the_pages():
    """Head ratios, head dims, windows and the local:global layer pattern of
    every workload match what the pages state (tests/golden/gqa_ratios.json)."""
    g = json.load(open(os.path.join(GOLD, "gqa_ratios.json")))
    loc, glo = inputs.LOCAL, inputs.GLOBAL
    assert loc["Hq"] // loc["Hkv"] == g["local"]["q_per_kv"]
    assert loc["Dk"] == loc["Dv"] == g["local"]["head_dim"]
    assert glo["Hq"] // glo["Hkv"] == g["global"]["q_per_kv"]
    assert glo["Dk"] == g["global"]["key_dim"]
    sm = g["small_model"]
    for shape, key in ((inputs.SMALL_LOCAL, "local_head_dim"), (inputs.SMALL_GLOBAL, "global_key_dim")):
        assert (shape["Hq"], shape["Hkv"]) == (sm["q_heads"], sm["kv_heads"])
        assert shape["Dk"] == sm[key]
    wl = inputs.WORKLOADS
    assert wl["local_prefill"]["case"].window in g["local"]["windows"]
    big, small = wl["stack"]["case"], wl["small_stack"]["case"]
    for st, ref in ((big, g["large_model"]), (small, sm)):
        kinds = [c.window > 0 for c, _ in st.layers]
        assert kinds[:st.n_local] == [True] * st.n_local and not kinds[st.n_local]
        assert st.n_local == ref["local_per_global"]
        assert st.window == ref["window"]

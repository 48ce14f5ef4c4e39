"""Pins of the oracle's verify attention (oracle/attention.py): closed forms
(one visible key returns its value; equal keys average the values), the
causal limit (keys beyond a query's position do not change it), the
grouped-query head mapping, and torch's float64 scaled-dot-product attention
with an explicit mask as an independent library reference."""
import numpy as np
import torch

import oracle

RNG = np.random.default_rng(55)


def bits(x):
    return oracle.f32_to_bf16(np.asarray(x, dtype=np.float32))


def val(b):
    return oracle.bf16_to_f32(b).astype(np.float64)


def rand_case(B=2, T=3, Hq=4, Hkv=2, Dh=16, Lmax=20):
    q = bits(RNG.standard_normal((B, T, Hq, Dh)))
    k = bits(RNG.standard_normal((B, Hkv, Lmax, Dh)))
    v = bits(RNG.standard_normal((B, Hkv, Lmax, Dh)))
    return q, k, v


def test_single_visible_key_returns_its_value():
    q, k, v = rand_case(B=1, T=1, Hq=2, Hkv=1)
    o = val(oracle.verify_attention(q, k, v, [1]))
    np.testing.assert_array_equal(o[0, 0, 0], val(v)[0, 0, 0])
    np.testing.assert_array_equal(o[0, 0, 1], val(v)[0, 0, 0])


def test_equal_keys_average_the_values():
    q, k, v = rand_case(B=1, T=1, Hq=1, Hkv=1, Lmax=8)
    k[:] = k[:, :, :1]                      # every key the same
    o = val(oracle.verify_attention(q, k, v, [8]))
    want = val(oracle.glue._f64_to_bf16_bits(val(v)[0, 0].mean(axis=0)))
    np.testing.assert_array_equal(o[0, 0, 0], want)


def test_causal_limit_and_group_mapping():
    q, k, v = rand_case(B=2, T=3, Hq=4, Hkv=2, Lmax=20)
    L = [10, 20]
    o = oracle.verify_attention(q, k, v, L)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 10:] = bits(RNG.standard_normal(k2[0, :, 10:].shape))   # beyond L_0
    v2[0, :, 10:] = bits(RNG.standard_normal(v2[0, :, 10:].shape))
    np.testing.assert_array_equal(oracle.verify_attention(q, k2, v2, L), o)
    # query 0 of sequence 1 sees keys 0..17 only; changing key 18 leaves it alone
    k3 = k.copy()
    k3[1, :, 18] = bits(RNG.standard_normal(k3[1, :, 18].shape))
    o3 = oracle.verify_attention(q, k3, v, L)
    np.testing.assert_array_equal(o3[1, 0], o[1, 0])
    assert not np.array_equal(o3[1, 1], o[1, 1])
    # heads 0, 1 read kv head 0; changing kv head 1 leaves them alone
    k4 = k.copy()
    k4[:, 1] = bits(RNG.standard_normal(k4[:, 1].shape))
    o4 = oracle.verify_attention(q, k4, v, L)
    np.testing.assert_array_equal(o4[:, :, :2], o[:, :, :2])


def test_against_torch_sdpa_float64():
    B, T, Hq, Hkv, Dh, Lmax = 2, 5, 8, 2, 64, 40
    q, k, v = rand_case(B, T, Hq, Hkv, Dh, Lmax)
    L = [33, 40]
    o = val(oracle.verify_attention(q, k, v, L))
    for b in range(B):
        qt = torch.from_numpy(val(q)[b]).permute(1, 0, 2)                      # Hq T Dh
        kt = torch.from_numpy(val(k)[b, :, :L[b]]).repeat_interleave(Hq // Hkv, 0)
        vt = torch.from_numpy(val(v)[b, :, :L[b]]).repeat_interleave(Hq // Hkv, 0)
        pos = torch.arange(L[b])[None, :]
        last = L[b] - T + torch.arange(T)[:, None]
        mask = pos <= last                                                      # T x L
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        ref = ref.permute(1, 0, 2).numpy()                                       # T Hq Dh
        got = o[b]
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-12)


def test_qk_norm_rope_position_zero_and_rotation_identities():
    B, T, Hq, Hkv = 2, 3, 4, 2
    x = bits(RNG.standard_normal((B * T, (Hq + 2 * Hkv) * 128)) * 2)
    g = bits(np.ones(128))
    q, k, v = oracle.qk_norm_rope(x, B, T, Hq, Hkv, g, g, 1e-6, [0, 0], 1e6)
    xr = x.reshape(B, T, Hq + 2 * Hkv, 128)
    # v passes through
    np.testing.assert_array_equal(v, xr[:, :, Hq + Hkv:])
    # position 0: no rotation, only the norm
    qn = oracle.rmsnorm(xr[:, 0, :Hq].reshape(-1, 128), g, 1e-6).reshape(B, Hq, 128)
    np.testing.assert_array_equal(q[:, 0], qn)
    # a rotation keeps each pair's norm (up to the bf16 roundings)
    h = val(oracle.rmsnorm(xr[:, :, :Hq].reshape(-1, 128), g, 1e-6)).reshape(B, T, Hq, 128)
    r = val(q)
    n_in = h[..., :64] ** 2 + h[..., 64:] ** 2
    n_out = r[..., :64] ** 2 + r[..., 64:] ** 2
    assert np.all(np.abs(n_out - n_in) <= 2.0 ** -6 * n_in + 1e-6)


def test_qk_norm_rope_known_angle():
    # dim pair d = 0 rotates by the position itself (base^0 = 1); at p = 3:
    # (x1, x2) -> (x1 cos 3 - x2 sin 3, x2 cos 3 + x1 sin 3)
    B, T, Hq, Hkv = 1, 1, 1, 1
    row = np.zeros((1, 3 * 128), dtype=np.float32)
    row[0, 0] = 1.0                         # q: x1 = 1 at d = 0, so its norm is sqrt(1/128)
    row[0, 128] = 1.0                       # k likewise
    x = bits(row)
    g = bits(np.ones(128))
    q, k, _ = oracle.qk_norm_rope(x, B, T, Hq, Hkv, g, g, 0.0, [3], 1e6)
    n = np.sqrt(128.0)                       # the normed x1 before its bf16 rounding
    n_bf = val(oracle.glue._f64_to_bf16_bits(np.array([n])))[0]
    assert val(q)[0, 0, 0, 0] == val(oracle.glue._f64_to_bf16_bits(np.array([n_bf * np.cos(3)])))[0]
    assert val(q)[0, 0, 0, 64] == val(oracle.glue._f64_to_bf16_bits(np.array([n_bf * np.sin(3)])))[0]


# ---------------------------------------------------------------------------
# Rotary angles for every dimension pair, pinned element by element.
#
# Reading (the pages give no attention formula; the workloads follow Qwen3's
# rotate-half RoPE in fp32 inference): pair (d, d + 64) of a head at
# position p turns by a = fp32(fp32(p) * fp32(base^(-d/64))).  The expected
# outputs below are built per element with math.pow / math.cos / math.sin
# and a bf16 rounding written here from its definition (8 significant bits,
# nearest, ties to even), not with the oracle's vectorised helpers.  Each
# plausible slip — exponent -d/128, a float64 angle, the pairs rotated the
# other way — is checked to change at least one of these outputs.
# ---------------------------------------------------------------------------
import math  # noqa: E402


def _bf16_round(x: float) -> float:
    if x == 0.0:
        return 0.0
    m, e = math.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)   # round(): ties to even on floats


def _angle_fp32(p: int, d: int, base: float, denom: float = 64.0) -> float:
    f = float(np.float32(math.pow(base, -d / denom)))
    return float(np.float32(float(np.float32(p)) * f))   # exact product, one fp32 rounding


def _rope_case(starts, T):
    """q head h holds a lone 1 at dim h (x1 of pair h); k head h holds a lone
    1 at dim 64 + h (x2 of pair h); gamma = 1, eps = 0, so every normed
    nonzero is bf16(sqrt(128))."""
    B, H = len(starts), 64
    rows = np.zeros((B * T, 3 * H * 128), dtype=np.float32)
    for h in range(H):
        rows[:, h * 128 + h] = 1.0
        rows[:, (H + h) * 128 + 64 + h] = 1.0
    rows[:, 2 * H * 128:] = RNG.standard_normal((B * T, H * 128))
    g = bits(np.ones(128))
    q, k, _ = oracle.qk_norm_rope(bits(rows), B, T, H, H, g, g, 0.0, starts, 1e6)
    return val(q), val(k)


def _expected(starts, T, angle):
    n = _bf16_round(math.sqrt(128.0))
    B, H = len(starts), 64
    q = np.zeros((B, T, H, 128))
    k = np.zeros((B, T, H, 128))
    for b in range(B):
        for i in range(T):
            p = starts[b] + i
            for h in range(H):
                a = angle(p, h)
                c, s = math.cos(a), math.sin(a)
                q[b, i, h, h] = _bf16_round(n * c)
                q[b, i, h, 64 + h] = _bf16_round(n * s)
                k[b, i, h, h] = _bf16_round(-n * s)
                k[b, i, h, 64 + h] = _bf16_round(n * c)
    return q, k


def test_qk_norm_rope_every_pair_fp32_angle():
    starts, T = [1, 99998, 4097], 2           # positions 1, 2, 99998, 99999, 4097, 4098
    q, k = _rope_case(starts, T)
    qe, ke = _expected(starts, T, lambda p, d: _angle_fp32(p, d, 1e6))
    np.testing.assert_array_equal(q, qe)
    np.testing.assert_array_equal(k, ke)

    # the pins discriminate: each slip changes some output
    q128, _ = _expected(starts, T, lambda p, d: _angle_fp32(p, d, 1e6, denom=128.0))
    assert not np.array_equal(q, q128)
    q64, _ = _expected(starts, T, lambda p, d: float(p) * math.pow(1e6, -d / 64.0))
    assert not np.array_equal(q, q64)
    qrev, _ = _expected(starts, T, lambda p, d: -_angle_fp32(p, d, 1e6))
    assert not np.array_equal(q, qrev)


def test_qk_norm_rope_fp32_angle_differs_from_fp64_at_large_positions():
    # near position 1e5 the fp32 rounding of the angle (up to ~4e-3 rad) is
    # larger than a bf16 step of the rotated values for some pairs: the
    # reading is visible in the outputs, not only in the angles
    starts, T = [99999], 1
    q, _ = _rope_case(starts, T)
    q64, _ = _expected(starts, T, lambda p, d: float(p) * math.pow(1e6, -d / 64.0))
    diff = np.count_nonzero(q != q64)
    assert diff > 0
    angles32 = [_angle_fp32(99999, d, 1e6) for d in range(64)]
    angles64 = [99999.0 * math.pow(1e6, -d / 64.0) for d in range(64)]
    assert max(abs(a - b) for a, b in zip(angles32, angles64)) > 1e-3

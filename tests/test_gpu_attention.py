"""GPU parity of the verified block's attention (w8a8_verify_attention,
through the C ABI) against the oracle's float64 computation
(oracle.verify_attention).

Bar: every bf16 output within 1e-2 relative / 1e-3 absolute of the oracle
(the stated bf16 tolerance); the fraction of bit-identical outputs is
reported.  Shapes: the Qwen3-8B heads (32 query, 8 kv, dim 128) at M = 5
(1 sequence, T = 5) over 4096 cached positions, the 32B heads (64 / 8) at
T = 8, 32 sequences of T = 9 with ragged lengths, and lengths at the edges
(exactly T, a split boundary, Lmax)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8

W_ATT = 9


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def draw(shape, index, scale=1.0):
    z = synth.rng(W_ATT, 30, index).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return synth.to_bf16_bits(z)


def v_blocked(v):
    """The blocked V-cache layout of the C ABI, by numpy axis permutation:
    position p = 16 blk + 4 g + kk, dim d = 16 db + c goes to element
    ((g * 16 + c) * 8 + db) * 4 + kk of block blk."""
    B, H, L, D = v.shape
    x = v.reshape(B, H, L // 16, 4, 4, 8, 16)          # blk, g, kk, db, c
    return np.ascontiguousarray(x.transpose(0, 1, 2, 3, 6, 5, 4)).reshape(B, H, L, D)


def test_pack_v_cache():
    announce("pack_v_cache")
    v = draw((3, 2, 48, 128), 20)
    np.testing.assert_array_equal(host(w8.pack_v_cache(dev_bf16(v))), v_blocked(v))
    # the layout formula of the C ABI, element by element on a few positions
    got = host(w8.pack_v_cache(dev_bf16(v))).reshape(3, 2, -1)
    for p, d in [(0, 0), (5, 17), (15, 127), (16, 1), (47, 64)]:
        e = (p // 16) * 2048 + ((p % 16 // 4) * 16 + d % 16) * 32 + (d // 16) * 4 + p % 4
        assert got[1, 1, e] == v[1, 1, p, d]


def run_attention(q, k, v, lengths):
    out = w8.verify_attention(dev_bf16(q), dev_bf16(k), dev_bf16(v_blocked(v)), dev(lengths))
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("B,T,Hq,Hkv,Lmax,lengths", [
    (1, 5, 32, 8, 4096, [4096]),
    (1, 5, 32, 8, 4096, [1000]),
    (1, 8, 64, 8, 2048, [2048]),
    (32, 9, 32, 8, 608, None),                  # ragged lengths
    (3, 4, 16, 4, 704, [4, 64 + 2, 704]),        # exactly T; straddling a split; Lmax
    (2, 3, 16, 4, 256, [128, 131]),              # ending on / just past a split
    (2, 1, 8, 8, 64, [1, 64]),
    (2, 5, 16, 4, 32768, [32768, 20011]),        # several blocks per split
])
def test_verify_attention(B, T, Hq, Hkv, Lmax, lengths):
    announce(f"verify_attention B={B} T={T} Hq={Hq} Hkv={Hkv} Lmax={Lmax}")
    q = draw((B, T, Hq, 128), 1)
    k = draw((B, Hkv, Lmax, 128), 2)
    v = draw((B, Hkv, Lmax, 128), 3)
    if lengths is None:
        lengths = synth.rng(W_ATT, 31, B).integers(T, Lmax + 1, size=B)
    lengths = np.asarray(lengths, dtype=np.int32)
    want = oracle.verify_attention(q, k, v, lengths)
    got = run_attention(q, k, v, lengths)
    g = oracle.bf16_to_f32(got).astype(np.float64)
    w = oracle.bf16_to_f32(want).astype(np.float64)
    assert np.all(np.abs(g - w) <= 1e-3 + 1e-2 * np.abs(w))
    print(f"[gpu] bit-identical fraction {np.mean(got == want):.4f}", flush=True)


def test_verify_attention_sharp_softmax():
    """Large scores (a nearly one-hot softmax) and all-equal keys."""
    announce("verify_attention sharp and flat softmax")
    B, T, Hq, Hkv, Lmax = 2, 5, 8, 2, 304
    q = draw((B, T, Hq, 128), 4, scale=3.0)
    k = draw((B, Hkv, Lmax, 128), 5, scale=3.0)
    v = draw((B, Hkv, Lmax, 128), 6)
    k[1] = k[1, :, :1]                          # sequence 1: every key equal
    lengths = np.array([300, 257], dtype=np.int32)
    want = oracle.verify_attention(q, k, v, lengths)
    g = oracle.bf16_to_f32(run_attention(q, k, v, lengths)).astype(np.float64)
    w = oracle.bf16_to_f32(want).astype(np.float64)
    assert np.all(np.abs(g - w) <= 1e-3 + 1e-2 * np.abs(w))


def test_verify_attention_ignores_positions_past_length():
    """Cache positions >= L_b may hold any bits (here NaN and Inf in K and
    V): the output equals the one over a clean cache."""
    announce("verify_attention with NaN/Inf past the lengths")
    B, T, Hq, Hkv, Lmax = 2, 5, 32, 8, 320
    q = draw((B, T, Hq, 128), 7)
    k = draw((B, Hkv, Lmax, 128), 8)
    v = draw((B, Hkv, Lmax, 128), 9)
    lengths = np.array([77, 250], dtype=np.int32)
    want = oracle.verify_attention(q, k, v, lengths)
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(lengths):
        k2[b, :, L:] = 0x7FC0                    # NaN
        v2[b, :, L:] = 0x7F80                    # +Inf
        v2[b, :, L::3] = 0xFFC1                  # NaN with another payload
    got = run_attention(q, k2, v2, lengths)
    np.testing.assert_array_equal(got, run_attention(q, k, v, lengths))
    g = oracle.bf16_to_f32(got).astype(np.float64)
    w = oracle.bf16_to_f32(want).astype(np.float64)
    assert np.all(np.abs(g - w) <= 1e-3 + 1e-2 * np.abs(w))


@pytest.mark.parametrize("B,T,Hq,Hkv,Lmax,lengths", [(2, 5, 32, 8, 304, [300, 123]),
                                                     (1, 3, 8, 2, 100000, [99999]),
                                                     (3, 1, 4, 4, 16, [1, 16, 7])])
def test_qk_norm_rope_append(B, T, Hq, Hkv, Lmax, lengths):
    announce(f"qk_norm_rope_append B={B} T={T} Hq={Hq} Hkv={Hkv} Lmax={Lmax}")
    qkv = draw((B * T, (Hq + 2 * Hkv) * 128), 10, scale=2.0)
    qg = synth.to_bf16_bits(synth.rng(W_ATT, 32, 0).uniform(0.5, 1.5, 128).astype(np.float32))
    kg = synth.to_bf16_bits(synth.rng(W_ATT, 32, 1).uniform(0.5, 1.5, 128).astype(np.float32))
    kc0 = draw((B, Hkv, Lmax, 128), 11)
    vc0 = draw((B, Hkv, Lmax, 128), 12)
    lengths = np.asarray(lengths, dtype=np.int32)
    kc, vc = dev_bf16(kc0), dev_bf16(v_blocked(vc0))
    q = w8.qk_norm_rope_append(dev_bf16(qkv), dev_bf16(qg), dev_bf16(kg), dev(lengths), kc, vc,
                               T=T, Hq=Hq, Hkv=Hkv, eps=1e-6, rope_base=1e6)
    torch.cuda.synchronize()
    start = lengths - T
    q_r, k_r, v_r = oracle.qk_norm_rope(qkv, B, T, Hq, Hkv, qg, kg, 1e-6, start, 1e6)

    def close(got, want):
        g = oracle.bf16_to_f32(got).astype(np.float64)
        w = oracle.bf16_to_f32(want).astype(np.float64)
        assert np.all(np.abs(g - w) <= 1e-3 + 1e-2 * np.abs(w))
        return np.mean(got == want)

    fq = close(host(q), q_r)
    kh, vh = host(kc), host(vc)
    want_k, want_v = kc0.copy(), vc0.copy()
    for b in range(B):
        for i in range(T):
            want_k[b, :, start[b] + i] = k_r[b, i]
            want_v[b, :, start[b] + i] = v_r[b, i]
    fk = close(kh, want_k)
    np.testing.assert_array_equal(vh, v_blocked(want_v))
    touched = np.zeros(kh.shape[:3], dtype=bool)
    for b in range(B):
        touched[b, :, start[b]:start[b] + T] = True
    np.testing.assert_array_equal(kh[~touched], kc0[~touched])
    print(f"[gpu] bit-identical q {fq:.4f} k(all) {fk:.6f}", flush=True)

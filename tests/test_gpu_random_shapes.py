"""Seeded random shapes for the W8A8 linear (plain and smoothed), the W4A8
linear, the LM-head verification, the two-pass argmax and acceptance on
planted ties, the stochastic acceptance, the fused BF16 glue and the
verified block's attention with its q/k norm, rotary embedding and cache
append, GPU against the CPU oracle: bit for bit, except the glue's bf16
rows and the attention outputs, which carry the tolerance of their own
tests (1e-2 relative / 1e-3 absolute).

The fixed-shape parity tests pin the workloads' shapes and the edges each
kernel path was written for; these draw (M, N, K) at random over the whole
range the dispatch covers (1..16 rows on the skinny kernel, 17..300 rows
on the batched kernels, ragged N, K any multiple of 16), plus skinny draws
aimed at its plan boundaries (the split tail past whole rounds over the
CUs, the k split of narrow long reductions), so that a boundary nobody
thought of still meets the oracle.  The draws are seeded and printed, so a
failure names its shape.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import sample as S
from tests.gpu_util import announce, dev, dev_bf16, gpu_available, host

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


def _draw_shapes(seed: int, n: int, rows: tuple, max_mnk: float) -> list:
    """n shapes (M, N, K) with M in rows, N in [1, 40000], K a multiple of 16
    in [16, 26624], M*N*K <= max_mnk (the oracle's product stays seconds)."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(r.integers(rows[0], rows[1] + 1))
        N = int(np.exp(r.uniform(0.0, np.log(40000.0))))
        K = 16 * int(np.exp(r.uniform(0.0, np.log(26624 / 16))))
        if M * N * K <= max_mnk:
            out.append((M, N, K))
    return out


def _plan_edges(seed: int) -> list:
    """Skinny shapes aimed at the plan boundaries: outputs a few tiles
    past whole rounds over 256 CUs with long K (the split tail), and narrow
    outputs with long K (the k split), at random row counts."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(4):
        tiles = 256 * int(r.integers(1, 3)) + int(r.integers(1, 256))
        out.append((int(r.integers(1, 17)), 16 * tiles - int(r.integers(0, 16)),
                    64 * int(r.integers(80, 129)) + 16 * int(r.integers(0, 4))))
    for _ in range(3):
        out.append((int(r.integers(1, 17)), int(r.integers(1, 513)),
                    16 * int(r.integers(1024, 1665))))
    return out


SKINNY = _draw_shapes(31, 12, (1, 16), 1.5e9) + _plan_edges(33)
BATCHED = _draw_shapes(32, 10, (17, 300), 3.0e9)


def _linear(M, N, K, seed, tiled):
    bits = synth.activations_bf16(seed, M, K, outliers=True)
    w = synth.weights_f32(seed, N, K)
    xq_ref, xs_ref = oracle.quantize_act(bits)
    wq_ref, ws_ref = oracle.quantize_weight(w)
    acc_ref, y32_ref, y_ref = oracle.w8a8_linear(xq_ref, xs_ref, wq_ref, ws_ref)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq, ws = w8.quantize_weight(dev(w), tiled=tiled)
    yb, yf, acc = w8.linear(xq, xs, wq, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(xq), xq_ref)
    np.testing.assert_array_equal(host(acc), acc_ref)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_ref.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_ref)


@pytest.mark.parametrize("M,N,K", SKINNY)
@pytest.mark.parametrize("tiled", [True, False])
def test_random_skinny_linear(M, N, K, tiled):
    announce(f"random skinny linear M={M} N={N} K={K} tiled={tiled} "
             f"workspace {w8.linear_workspace_bytes(M, N, K)} B")
    _linear(M, N, K, seed=M * 7919 + N * 31 + K, tiled=tiled)


@pytest.mark.parametrize("M,N,K", BATCHED)
def test_random_batched_linear(M, N, K):
    announce(f"random batched linear M={M} N={N} K={K} "
             f"workspace {w8.linear_workspace_bytes(M, N, K)} B")
    _linear(M, N, K, seed=M * 7919 + N * 31 + K, tiled=True)


@pytest.mark.parametrize("M,N,K", BATCHED[:5])
def test_random_batched_tiled_activations(M, N, K):
    """The batched kernels' tiled-activation path on the same draws."""
    announce(f"random tiled-activation linear M={M} N={N} K={K}")
    seed = M * 7919 + N * 31 + K
    bits = synth.activations_bf16(seed, M, K, outliers=True)
    w = synth.weights_f32(seed, N, K)
    xq_ref, xs_ref = oracle.quantize_act(bits)
    wq_ref, ws_ref = oracle.quantize_weight(w)
    acc_ref, y32_ref, y_ref = oracle.w8a8_linear(xq_ref, xs_ref, wq_ref, ws_ref)
    xt, xs = w8.quantize_act_tiled(dev_bf16(bits))
    wq, ws = w8.quantize_weight(dev(w), tiled=True)
    yb, yf, acc = w8.linear_tiled_act(xt, xs, wq, ws, K=K, want_bf16=True, want_f32=True,
                                      want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_ref)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_ref.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_ref)


@pytest.mark.parametrize("B,G,V,K", [(1, 4, 77777, 1040), (2, 6, 30011, 2064), (1, 15, 5003, 4160),
                                     (9, 2, 12007, 528), (24, 11, 3001, 1024)])
def test_random_lm_head_verify(B, G, V, K):
    """The fused LM-head verification (skinny up to 16 rows, batched above)
    at odd vocabularies and K, drafts with spread accepted lengths."""
    announce(f"random lm_head_verify B={B} G={G} V={V} K={K}")
    R = B * (G + 1)
    bits = synth.activations_bf16(V + K, R, K)
    w = synth.weights_f32(V + K, V, K)
    xq_ref, xs_ref = oracle.quantize_act(bits)
    wq_ref, ws_ref = oracle.quantize_weight(w)
    _, y32_ref, _ = oracle.w8a8_linear(xq_ref, xs_ref, wq_ref, ws_ref)
    am0 = oracle.argmax_rows(y32_ref).reshape(B, G + 1)
    draft = synth.draft_ids(V, B, G, V)
    for b in range(B):
        p = (3 * b + 1) % (G + 1)
        draft[b, :p] = am0[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y32_ref, draft)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wt, ws = w8.quantize_weight(dev(w), tiled=True)
    _, am, al, nt = w8.lm_head_verify(xq, xs, wt, ws, dev(draft))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(am), am_r)
    np.testing.assert_array_equal(host(al), al_r)
    np.testing.assert_array_equal(host(nt), nt_r)


def _w4_draws(seed: int, n: int) -> list:
    """W4A8 shapes: M in [1, 48] (skinny and batched), N in [1, 20000], K a
    multiple of 16 in [16, 16384] (int4 k pairs of 128 padded), M*N*K <= 1e9."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(r.integers(1, 49))
        N = int(np.exp(r.uniform(0.0, np.log(20000.0))))
        K = 16 * int(np.exp(r.uniform(0.0, np.log(16384 / 16))))
        if M * N * K <= 1.0e9:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _w4_draws(34, 8))
def test_random_w4_linear(M, N, K):
    announce(f"random w4 linear M={M} N={N} K={K}")
    seed = M * 7919 + N * 31 + K + 1
    bits = synth.activations_bf16(seed, M, K, outliers=True)
    w = synth.weights_f32(seed, N, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    q_r, s_r = oracle.quantize_weight_int4(w)
    acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, q_r, s_r)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq4, ws = w8.quantize_weight_w4(dev(w))
    yb, yf, acc = w8.linear_w4(xq, xs, wq4, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_r)


def _sample_draws(seed: int, n: int) -> list:
    """Stochastic acceptance: B in [1, 8], G in [0, 12], V in [1, 200000],
    T log-uniform in [0.05, 4]."""
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 9)), int(r.integers(0, 13)),
             int(np.exp(r.uniform(0.0, np.log(200000.0)))),
             float(np.float32(np.exp(r.uniform(np.log(0.05), np.log(4.0))))))
            for _ in range(n)]


@pytest.mark.parametrize("B,G,V,t", _sample_draws(35, 8))
def test_random_verify_sample(B, G, V, t):
    """Drafts agreeing with the row argmax for a spread of prefix lengths
    (likely acceptances at low T), the rest random; random words."""
    announce(f"random verify_sample B={B} G={G} V={V} T={t}")
    r = np.random.default_rng(B * 1000003 + G * 1009 + V)
    R = B * (G + 1)
    y = (r.standard_normal((R, V), dtype=np.float32) * np.float32(2.0)).astype(np.float32)
    am = oracle.argmax_rows(y).reshape(B, G + 1)
    d = r.integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):
        p = (2 * b + 1) % (G + 1)
        d[b, :p] = am[b, :p]
    ua = r.integers(0, 1 << 32, size=(B, G), dtype=np.uint64).astype(np.uint32)
    us = r.integers(0, 1 << 64, size=(B,), dtype=np.uint64)
    al_r, nt_r = S.verify_sample(y, d, t, ua, us)
    ua_t = torch.from_numpy(ua.view(np.int32).reshape(B, G).copy()).cuda()
    us_t = torch.from_numpy(us.view(np.int64).copy()).cuda()
    al, nt = w8.verify_sample(dev(y), dev(d), t, ua_t, us_t)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(al), al_r)
    np.testing.assert_array_equal(host(nt), nt_r)


def _glue_draws(seed: int, n: int) -> list:
    """Glue widths: M in [1, 300], D a multiple of 16 in [16, 32768]
    (log-uniform), smoothing on about half of them."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(np.exp(r.uniform(0.0, np.log(300.0))))
        D = 16 * int(np.exp(r.uniform(0.0, np.log(32768 / 16))))
        if M * D <= 2_000_000:
            out.append((M, D, bool(r.integers(0, 2))))
    return out


def _check_glue_codes(xq, xsc, rows_gpu, rows_oracle, smooth):
    """The codes: bit-exact against the oracle's quantizer on the kernel's own
    bf16 rows (the same decision in the same precision), and against the
    all-oracle chain on every row whose bf16 values equal the oracle's; the
    bf16 rows within 1e-2 relative / 1e-3 absolute, >= 99% bit-identical."""
    got = oracle.bf16_to_f32(rows_gpu).astype(np.float64)
    want = oracle.bf16_to_f32(rows_oracle).astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-3 + 1e-2 * np.abs(want))
    assert np.mean(rows_gpu == rows_oracle) >= 0.99
    q_k, s_k = oracle.quantize_act(rows_gpu, smooth=smooth)
    np.testing.assert_array_equal(xq, q_k)
    np.testing.assert_array_equal(xsc.view(np.uint32), s_k.view(np.uint32))
    same = np.all(rows_gpu == rows_oracle, axis=1)
    q_o, s_o = oracle.quantize_act(rows_oracle, smooth=smooth)
    np.testing.assert_array_equal(xq[same], q_o[same])
    np.testing.assert_array_equal(xsc[same].view(np.uint32), s_o[same].view(np.uint32))
    print(f"[gpu] glue rows identical to the oracle's: {int(same.sum())} of {len(same)}", flush=True)


@pytest.mark.parametrize("M,D,smooth", _glue_draws(36, 6))
def test_random_residual_rmsnorm_quant(M, D, smooth):
    announce(f"random residual_rmsnorm_quant M={M} D={D} smooth={smooth}")
    seed = M * 7919 + D
    h = oracle.f32_to_bf16(oracle.bf16_to_f32(synth.activations_bf16(seed, M, D))
                           * np.float32(4.0))
    delta = synth.activations_bf16(seed + 1, M, D, outliers=True)
    gamma = oracle.f32_to_bf16(np.random.default_rng(seed).uniform(0.5, 1.5, D).astype(np.float32))
    s = synth.smoothing_vector(seed, D) if smooth else None
    eps = 1e-6
    xq, xsc, normed, h_out = w8.residual_rmsnorm_quant(
        dev_bf16(h), dev_bf16(gamma), eps, delta=dev_bf16(delta),
        smooth=None if s is None else dev(s), want_normed=True)
    torch.cuda.synchronize()
    h1 = oracle.residual_add(h, delta)
    np.testing.assert_array_equal(host(h_out), h1)
    _check_glue_codes(host(xq), host(xsc), host(normed), oracle.rmsnorm(h1, gamma, eps), s)


@pytest.mark.parametrize("M,F,smooth", _glue_draws(37, 6))
def test_random_silu_mul_quant(M, F, smooth):
    announce(f"random silu_mul_quant M={M} F={F} smooth={smooth}")
    seed = M * 7919 + F + 2
    g = oracle.f32_to_bf16(oracle.bf16_to_f32(synth.activations_bf16(seed, M, F))
                           * np.float32(3.0))
    u = synth.activations_bf16(seed + 1, M, F)
    s = synth.smoothing_vector(seed, F) if smooth else None
    xq, xsc, act = w8.silu_mul_quant(dev_bf16(g), dev_bf16(u),
                                     smooth=None if s is None else dev(s), want_act=True)
    torch.cuda.synchronize()
    _check_glue_codes(host(xq), host(xsc), host(act), oracle.silu_mul(g, u), s)


def _attention_draws(seed: int, n: int) -> list:
    """B in [1, 8] sequences of T in [1, 8] verified positions; kv heads in
    {1, 2, 4, 8} with a query group of at most 64 / T rows; Lmax a multiple
    of 16 up to 16384; ragged lengths in [T, Lmax]; B*Hq*T*Lmax <= 2e7 (the
    float64 oracle stays seconds)."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, T = int(r.integers(1, 9)), int(r.integers(1, 9))
        Hkv = int(r.choice([1, 2, 4, 8]))
        g = int(r.integers(1, 64 // T + 1))
        Lmax = 16 * int(np.exp(r.uniform(np.log((T + 15) // 16), np.log(1024))))
        lengths = [int(x) for x in r.integers(T, Lmax + 1, size=B)]
        if B * Hkv * g * T * Lmax <= 2.0e7:
            out.append((B, T, Hkv * g, Hkv, Lmax, lengths))
    return out


@pytest.mark.parametrize("B,T,Hq,Hkv,Lmax,lengths", _attention_draws(38, 6))
def test_random_verify_attention(B, T, Hq, Hkv, Lmax, lengths):
    announce(f"random verify_attention B={B} T={T} Hq={Hq} Hkv={Hkv} Lmax={Lmax} lengths={lengths}")
    r = np.random.default_rng(B * 131 + T * 17 + Hq * 7 + Lmax)
    q, k, v = (synth.to_bf16_bits(r.standard_normal(shape, dtype=np.float32))
               for shape in ((B, T, Hq, 128), (B, Hkv, Lmax, 128), (B, Hkv, Lmax, 128)))
    lengths = np.asarray(lengths, dtype=np.int32)
    want = oracle.verify_attention(q, k, v, lengths)
    out = w8.verify_attention(dev_bf16(q), dev_bf16(k), w8.pack_v_cache(dev_bf16(v)), dev(lengths))
    torch.cuda.synchronize()
    got = host(out)
    g = oracle.bf16_to_f32(got).astype(np.float64)
    w = oracle.bf16_to_f32(want).astype(np.float64)
    assert np.all(np.abs(g - w) <= 1e-3 + 1e-2 * np.abs(w))
    print(f"[gpu] bit-identical fraction {np.mean(got == want):.4f}", flush=True)


def _append_draws(seed: int, n: int) -> list:
    """B in [1, 8], T in [1, 8], kv heads in {1, 2, 4, 8} with groups of
    1-8, Lmax a multiple of 16 up to 131072 (log-uniform), ragged lengths
    in [T, Lmax], rotary base 1e4 or 1e6; B*Hkv*Lmax <= 5e5."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, T = int(r.integers(1, 9)), int(r.integers(1, 9))
        Hkv = int(r.choice([1, 2, 4, 8]))
        Hq = Hkv * int(r.integers(1, 9))
        Lmax = 16 * int(np.exp(r.uniform(0.0, np.log(8192))))
        lengths = [int(x) for x in r.integers(T, Lmax + 1, size=B)]
        base = float(r.choice([1.0e4, 1.0e6]))
        if Lmax >= T and B * Hkv * Lmax <= 5.0e5:
            out.append((B, T, Hq, Hkv, Lmax, lengths, base))
    return out


@pytest.mark.parametrize("B,T,Hq,Hkv,Lmax,lengths,base", _append_draws(39, 6))
def test_random_qk_norm_rope_append(B, T, Hq, Hkv, Lmax, lengths, base):
    announce(f"random qk_norm_rope_append B={B} T={T} Hq={Hq} Hkv={Hkv} Lmax={Lmax} "
             f"lengths={lengths} base={base:g}")
    r = np.random.default_rng(B * 131 + T * 17 + Hq * 7 + Lmax + 1)

    def bf(shape, scale=1.0):
        return synth.to_bf16_bits(r.standard_normal(shape, dtype=np.float32) * np.float32(scale))

    qkv = bf((B * T, (Hq + 2 * Hkv) * 128), 2.0)
    qg = synth.to_bf16_bits(r.uniform(0.5, 1.5, 128).astype(np.float32))
    kg = synth.to_bf16_bits(r.uniform(0.5, 1.5, 128).astype(np.float32))
    kc0, vc0 = bf((B, Hkv, Lmax, 128)), bf((B, Hkv, Lmax, 128))
    lengths = np.asarray(lengths, dtype=np.int32)
    kc, vc = dev_bf16(kc0), w8.pack_v_cache(dev_bf16(vc0))
    q = w8.qk_norm_rope_append(dev_bf16(qkv), dev_bf16(qg), dev_bf16(kg), dev(lengths), kc, vc,
                               T=T, Hq=Hq, Hkv=Hkv, eps=1e-6, rope_base=base)
    torch.cuda.synchronize()
    start = lengths - T
    q_r, k_r, v_r = oracle.qk_norm_rope(qkv, B, T, Hq, Hkv, qg, kg, 1e-6, start, base)
    want_k, want_v = kc0.copy(), vc0.copy()
    for b in range(B):
        for i in range(T):
            want_k[b, :, start[b] + i] = k_r[b, i]
            want_v[b, :, start[b] + i] = v_r[b, i]
    fractions = []
    for got, want in ((host(q), q_r), (host(kc), want_k)):
        g = oracle.bf16_to_f32(got).astype(np.float64)
        w = oracle.bf16_to_f32(want).astype(np.float64)
        assert np.all(np.abs(g - w) <= 1e-3 + 1e-2 * np.abs(w))
        fractions.append(float(np.mean(got == want)))
    print(f"[gpu] bit-identical q {fractions[0]:.6f} k(all) {fractions[1]:.6f}", flush=True)
    np.testing.assert_array_equal(host(vc), host(w8.pack_v_cache(dev_bf16(want_v))))
    touched = np.zeros((B, Hkv, Lmax), dtype=bool)
    for b in range(B):
        touched[b, :, start[b]:start[b] + T] = True
    np.testing.assert_array_equal(host(kc)[~touched], kc0[~touched])


@pytest.mark.parametrize("M,N,K", _draw_shapes(40, 6, (1, 64), 1.5e9))
def test_random_smoothed_linear(M, N, K):
    """Online smoothing at random shapes: activations multiplied and weights
    divided by one positive per-channel vector before quantization, then the
    linear; codes, scales, int32 sums and outputs bit-exact."""
    announce(f"random smoothed linear M={M} N={N} K={K}")
    seed = M * 7919 + N * 31 + K + 3
    bits = synth.activations_bf16(seed, M, K, outliers=True)
    w = synth.weights_f32(seed, N, K)
    s = synth.smoothing_vector(seed, K)
    xq_r, xs_r = oracle.quantize_act(bits, smooth=s)
    wq_r, ws_r = oracle.quantize_weight(w, smooth=s)
    acc_r, y32_r, y_r = oracle.w8a8_linear(xq_r, xs_r, wq_r, ws_r)
    sd = dev(s)
    xq, xs = w8.quantize_act(dev_bf16(bits), sd)
    wq, ws = w8.quantize_weight(dev(w), sd, tiled=True)
    yb, yf, acc = w8.linear(xq, xs, wq, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(xq), xq_r)
    np.testing.assert_array_equal(host(xs).view(np.uint32), xs_r.view(np.uint32))
    np.testing.assert_array_equal(host(ws).view(np.uint32), ws_r.view(np.uint32))
    np.testing.assert_array_equal(host(acc), acc_r)
    np.testing.assert_array_equal(host(yf).view(np.uint32), y32_r.view(np.uint32))
    np.testing.assert_array_equal(host(yb), y_r)


def _head_draws(seed: int, n: int) -> list:
    """LM-head verifications: B in [1, 8], G in [0, 10], V in [1, 160000],
    K a multiple of 16 in [16, 8192]; R*V*K <= 2e9."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, G = int(r.integers(1, 9)), int(r.integers(0, 11))
        V = int(np.exp(r.uniform(0.0, np.log(160000.0))))
        K = 16 * int(np.exp(r.uniform(0.0, np.log(8192 / 16))))
        if B * (G + 1) * V * K <= 2.0e9:
            out.append((B, G, V, K))
    return out


@pytest.mark.parametrize("B,G,V,K", _head_draws(41, 6))
def test_random_lm_head_argmax_w4(B, G, V, K):
    """The W4A8 LM head with the argmax folded in, then accept_from_keys."""
    announce(f"random lm_head_argmax_w4 B={B} G={G} V={V} K={K}")
    R = B * (G + 1)
    bits = synth.activations_bf16(V + K + 5, R, K)
    w = synth.weights_f32(V + K + 5, V, K)
    xq_r, xs_r = oracle.quantize_act(bits)
    q_r, s_r = oracle.quantize_weight_int4(w)
    _, y32_r, _ = oracle.w8a8_linear(xq_r, xs_r, q_r, s_r)
    am0 = oracle.argmax_rows(y32_r).reshape(B, G + 1)
    draft = synth.draft_ids(V + K + 5, B, G, V)
    for b in range(B):
        p = (3 * b + 2) % (G + 1)
        draft[b, :p] = am0[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y32_r, draft)
    xq, xs = w8.quantize_act(dev_bf16(bits))
    wq4, ws = w8.quantize_weight_w4(dev(w))
    wsp = w8.Workspace()
    w8.lm_head_argmax_w4(xq, xs, wq4, ws, workspace=wsp)
    am, al, nt = w8.accept_from_keys(dev(draft), workspace=wsp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(am), am_r)
    np.testing.assert_array_equal(host(al), al_r)
    np.testing.assert_array_equal(host(nt), nt_r)


@pytest.mark.parametrize("R,V,t", [(int(a), int(b), float(np.float32(c))) for a, b, c in zip(
    np.random.default_rng(42).integers(1, 40, 6),
    np.exp(np.random.default_rng(43).uniform(0.0, np.log(200000.0), 6)).astype(int) + 1,
    np.exp(np.random.default_rng(44).uniform(np.log(0.05), np.log(4.0), 6)))])
def test_random_sample_weights(R, V, t):
    """The fixed-point softmax numerators of the stochastic acceptance, every
    weight bit-exact, at random row counts, vocabularies and temperatures."""
    announce(f"random sample_weights R={R} V={V} T={t}")
    y = (np.random.default_rng(R * 100003 + V).standard_normal((R, V), dtype=np.float32)
         * np.float32(3.0)).astype(np.float32)
    w = host(w8.sample_weights(dev(y), t)).view(np.uint64)
    inv_t = S.inv_temperature(t)
    for r in range(R):
        np.testing.assert_array_equal(w[r], S.fixed_weights(y[r], inv_t))


@pytest.mark.parametrize("B,G,V", [(int(a), int(b), int(c)) for a, b, c in zip(
    np.random.default_rng(45).integers(1, 9, 6), np.random.default_rng(46).integers(0, 12, 6),
    np.exp(np.random.default_rng(47).uniform(0.0, np.log(300000.0), 6)).astype(int) + 1)])
def test_random_verify_accept_ties(B, G, V):
    """The two-pass argmax and greedy acceptance on fp32 logits, with the
    row maximum planted at two to four random positions per row (so ties
    straddle the 4096-logit chunks of the first pass), -0/+0 pairs, and
    drafts that agree with a spread of prefix lengths: argmax (lowest index
    on ties), accepted lengths and next tokens exact."""
    announce(f"random verify_accept ties B={B} G={G} V={V}")
    r = np.random.default_rng(B * 7 + G * 131 + V)
    R = B * (G + 1)
    y = r.standard_normal((R, V), dtype=np.float32)
    for i in range(R):
        top = np.float32(10.0 + r.integers(0, 3))
        y[i, r.integers(0, V, size=int(r.integers(2, 5)))] = top
        if V > 2:
            y[i, r.integers(0, V, size=2)] = np.float32([-0.0, 0.0])
    am0 = oracle.argmax_rows(y).reshape(B, G + 1)
    d = r.integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):
        p = (5 * b + 1) % (G + 1)
        d[b, :p] = am0[b, :p]
    am_r, al_r, nt_r = oracle.verify_accept(y, d)
    am, al, nt = w8.verify_accept(dev(y), dev(d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(am), am_r)
    np.testing.assert_array_equal(host(al), al_r)
    np.testing.assert_array_equal(host(nt), nt_r)

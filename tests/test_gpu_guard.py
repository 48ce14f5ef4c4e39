"""Guard bands around every output and workspace (GPU, through the C ABI).

Each output tensor and each workspace handed to the library is the middle
of a larger device buffer whose bytes before and after are a sentinel
(0xA5).  After the call, every sentinel byte must be intact: a store past a
ragged M or N tail (or past the end of a workspace) would otherwise land
silently in the caching allocator.  The interior must equal what the same
call writes into a fresh, unguarded allocation (bit for bit; the parity
tests compare those with the oracle), and the zero-on-exit workspaces (the
split-K partials and the LM-head argmax keys) must be zero again.

Paths covered: the skinny kernel (row-major and tiled weights, with and
without the split-K handoff), the register-fragment batched kernel, the
LDS-pipelined 16 x 16 and 32 x 32 kernels (including the 96-row form with
the argmax fold), tiled activations, the LM-head argmax keys at 5 and 288
rows, the two-pass verify_accept, the quantizers, the W4A8 kernels, the
fused glue (residual + RMSNorm + quantize, SwiGLU + quantize), the q/k norm
+ rotary + cache append with both caches guarded, the verified block's
attention and its workspace, and the stochastic acceptance and its weights."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import announce, dev, dev_bf16, gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    import w8a8_quantized_verification_amd as w8

PAD = 4096          # bytes of sentinel before and after (keeps 256-byte alignment)
FILL = 0xA5
W_GUARD = 31


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no ROCm GPU")


class Guarded:
    """A device tensor of ``shape``/``dtype`` placed between two sentinel
    bands of PAD bytes."""

    def __init__(self, shape, dtype, zero=False):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = n
        self.raw = torch.full((2 * PAD + n,), FILL, dtype=torch.uint8, device="cuda:0")
        inner = self.raw[PAD:PAD + n]
        if zero:
            inner.zero_()
        self.t = inner.view(dtype).view(shape) if n else inner.view(dtype)

    def intact(self) -> bool:
        return bool((self.raw[:PAD] == FILL).all()) and bool((self.raw[PAD + self.nbytes:] == FILL).all())


class GuardedWorkspace(w8.Workspace if gpu_available() else object):
    """A Workspace whose buffers are exactly the requested size, each
    between sentinel bands (a larger request makes a new guarded buffer)."""

    def __init__(self):
        super().__init__()
        self.bufs = {}
        self.all = []

    def get(self, nbytes, device, use):
        if nbytes == 0:
            return None
        g = self.bufs.get(use)
        if g is None or g.nbytes < nbytes:
            g = Guarded((nbytes,), torch.uint8, zero=True)
            self.bufs[use] = g
            self.all.append((use, g))
        return g.t

    def check(self):
        for use, g in self.all:
            assert g.intact(), f"workspace '{use}' guard band overwritten"
            if use in ("zeroed", "keys"):
                assert not bool(g.t.any()), f"workspace '{use}' not left zero-filled"


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    a = a.contiguous().view(torch.uint8)
    b = b.contiguous().view(torch.uint8)
    return bool(torch.equal(a, b))


def int8_weights(N, K, index, tiled=True):
    w = dev(synth.weights_f32(W_GUARD, N, K, tensor_index=index))
    return w8.quantize_weight(w, tiled=tiled)


def act(M, K, index):
    return dev_bf16(synth.activations_bf16(W_GUARD, M, K, index=index, outliers=True))


def run_linear_guarded(xq, xs, wq, ws, M, N, wsp):
    outs = {"y_bf16": Guarded((M, N), torch.bfloat16), "y_f32": Guarded((M, N), torch.float32),
            "acc": Guarded((M, N), torch.int32)}
    w8.linear(xq, xs, wq, ws, y_bf16=outs["y_bf16"].t, y_f32=outs["y_f32"].t, acc=outs["acc"].t,
              workspace=wsp)
    return outs


def check_linear(xq, xs, wq, ws, M, N, label):
    wsp = GuardedWorkspace()
    outs = run_linear_guarded(xq, xs, wq, ws, M, N, wsp)
    ref = w8.linear(xq, xs, wq, ws, want_bf16=True, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    for (name, g), r in zip(outs.items(), ref):
        assert g.intact(), f"{label}: {name} guard band overwritten"
        assert same_bits(g.t, r), f"{label}: {name} differs from the unguarded call"
    wsp.check()


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("N", [1, 17, 4099])
@pytest.mark.parametrize("tiled", [True, False])
def test_guard_skinny_linear(M, N, tiled):
    K = 4096
    announce(f"guard skinny linear M={M} N={N} K={K} tiled={tiled} "
             f"split-K workspace {w8.linear_workspace_bytes(M, N, K)} B")
    wq, ws = int8_weights(N, K, 1 + N, tiled=tiled)
    xq, xs = w8.quantize_act(act(M, K, M))
    check_linear(xq, xs, wq, ws, M, N, f"skinny M={M} N={N}")


@pytest.mark.parametrize("M,N,K", [(8, 5120, 8192), (7, 4100, 6144)])
@pytest.mark.parametrize("tiled", [True, False])
def test_guard_skinny_split_tail(M, N, K, tiled):
    # the tiles past the last whole round over the CUs are split across
    # workgroups (their partials go through the workspace)
    announce(f"guard skinny split tail M={M} N={N} K={K} tiled={tiled} "
             f"workspace {w8.linear_workspace_bytes(M, N, K)} B")
    assert w8.linear_workspace_bytes(M, N, K) > 0
    wq, ws = int8_weights(N, K, 7 + N, tiled=tiled)
    xq, xs = w8.quantize_act(act(M, K, M + 3))
    check_linear(xq, xs, wq, ws, M, N, f"split tail M={M} N={N}")


@pytest.mark.parametrize("split", [2, 4, 8])
def test_guard_skinny_forced_split_k(split, monkeypatch):
    M, N, K = 5, 4099, 4160          # K not a multiple of 128: ragged k slices too
    monkeypatch.setenv("W8A8_SPLITK", str(split))
    announce(f"guard skinny forced split-K={split} M={M} N={N} K={K}")
    assert w8.linear_workspace_bytes(M, N, K) > 0
    wq, ws = int8_weights(N, K, 50 + split)
    xq, xs = w8.quantize_act(act(M, K, 3))
    check_linear(xq, xs, wq, ws, M, N, f"split-K {split}")


@pytest.mark.parametrize("M,N,K,tiled", [
    (17, 17, 4096, True),        # register-fragment kernel, narrow grid
    (97, 4099, 4096, True),      # LDS 16 x 16, k-sliced
    (289, 4099, 4096, True),
    (289, 12293, 4096, True),    # LDS 32 x 32 (64-row workgroups)
    (289, 4099, 4112, True),     # K not a multiple of 64: register-fragment kernel
    (97, 4099, 4096, False),     # row-major weights
    (288, 4096, 12288, True),    # LDS 32 x 32, k split across two workgroups (workspace)
    (280, 4004, 8256, True),     # the same, ragged M, N and an odd step count
])
def test_guard_batched_linear(M, N, K, tiled):
    announce(f"guard batched linear M={M} N={N} K={K} tiled={tiled}")
    wq, ws = int8_weights(N, K, 100 + M, tiled=tiled)
    xq, xs = w8.quantize_act(act(M, K, M))
    check_linear(xq, xs, wq, ws, M, N, f"batched M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(17, 4099, 4096), (289, 4099, 4096), (289, 12293, 4096),
                                   (289, 1029, 12288), (97, 17, 256), (288, 4096, 12288),
                                   (280, 4004, 8208)])
def test_guard_tiled_activations(M, N, K):
    announce(f"guard tiled activations M={M} N={N} K={K}")
    x = act(M, K, 7)
    xt = Guarded(w8.tiled_shape(M, K), torch.int8)
    xs = Guarded((M,), torch.float32)
    w8.quantize_act_tiled(x, xq_tiled=xt.t, x_scale=xs.t)
    xt_ref, xs_ref = w8.quantize_act_tiled(x)
    wq, ws = int8_weights(N, K, 200 + M)
    outs = {"y_bf16": Guarded((M, N), torch.bfloat16), "y_f32": Guarded((M, N), torch.float32),
            "acc": Guarded((M, N), torch.int32)}
    wsp = GuardedWorkspace()
    w8.linear_tiled_act(xt.t, xs.t, wq, ws, K=K, y_bf16=outs["y_bf16"].t, y_f32=outs["y_f32"].t,
                        acc=outs["acc"].t, workspace=wsp)
    ref = w8.linear_tiled_act(xt_ref, xs_ref, wq, ws, K=K, want_f32=True, want_acc=True)
    torch.cuda.synchronize()
    wsp.check()
    assert xt.intact() and xs.intact()
    assert same_bits(xt.t, xt_ref) and same_bits(xs.t, xs_ref)
    for (name, g), r in zip(outs.items(), ref):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, r), f"{name} differs from the unguarded call"


@pytest.mark.parametrize("M,K", [(5, 4096), (289, 4112), (8, 25600), (1, 16)])
def test_guard_quantize_act(M, K):
    announce(f"guard quantize_act M={M} K={K}")
    x = act(M, K, 11)
    xq, xs = Guarded((M, K), torch.int8), Guarded((M,), torch.float32)
    w8.quantize_act(x, xq=xq.t, x_scale=xs.t)
    rq, rs = w8.quantize_act(x)
    torch.cuda.synchronize()
    assert xq.intact() and xs.intact()
    assert same_bits(xq.t, rq) and same_bits(xs.t, rs)


def test_guard_quantize_weight_tiled_ragged():
    N, K = 4099, 4112
    announce(f"guard quantize_weight tiled N={N} K={K}")
    w = dev(synth.weights_f32(W_GUARD, N, K, tensor_index=300))
    wq, ws = Guarded(w8.tiled_shape(N, K), torch.int8), Guarded((N,), torch.float32)
    w8.quantize_weight(w, tiled=True, wq=wq.t, w_scale=ws.t)
    rq, rs = w8.quantize_weight(w, tiled=True)
    torch.cuda.synchronize()
    assert wq.intact() and ws.intact()
    assert same_bits(wq.t, rq) and same_bits(ws.t, rs)


@pytest.mark.parametrize("B,G,V,K", [(1, 4, 151941, 256), (32, 8, 151941, 256), (2, 7, 4099, 4096),
                                     (3, 0, 17, 64)])
def test_guard_lm_head_verify(B, G, V, K):
    R = B * (G + 1)
    announce(f"guard lm_head_verify B={B} G={G} V={V} K={K} (rows {R})")
    wq, ws = int8_weights(V, K, 400 + B)
    xq, xs = w8.quantize_act(act(R, K, 12))
    draft = dev(synth.draft_ids(W_GUARD, B, G, V))
    wsp = GuardedWorkspace()
    lg, am = Guarded((R, V), torch.float32), Guarded((R,), torch.int32)
    al, nt = Guarded((B,), torch.int32), Guarded((B,), torch.int32)
    w8.lm_head_verify(xq, xs, wq, ws, draft, logits=lg.t, argmax=am.t, accept_len=al.t,
                      next_token=nt.t, workspace=wsp)
    ref = w8.lm_head_verify(xq, xs, wq, ws, draft, want_logits=True)
    torch.cuda.synchronize()
    for name, g, r in (("logits", lg, ref[0]), ("argmax", am, ref[1]), ("accept_len", al, ref[2]),
                       ("next_token", nt, ref[3])):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, r), f"{name} differs from the unguarded call"
    wsp.check()


@pytest.mark.parametrize("B,G,V,K", [(32, 8, 151941, 256), (32, 8, 12293, 4096), (1, 16, 4099, 4096)])
def test_guard_lm_head_argmax_tiled_act(B, G, V, K):
    R = B * (G + 1)
    announce(f"guard lm_head_argmax_tiled_act B={B} G={G} V={V} K={K} (rows {R})")
    wq, ws = int8_weights(V, K, 500 + B)
    xt, xs = w8.quantize_act_tiled(act(R, K, 13))
    draft = dev(synth.draft_ids(W_GUARD, B, G, V, index=1))
    wsp = GuardedWorkspace()
    lg = Guarded((R, V), torch.float32)
    w8.lm_head_argmax_tiled_act(xt, xs, wq, ws, K=K, logits=lg.t, workspace=wsp)
    am, al, nt = (Guarded((R,), torch.int32), Guarded((B,), torch.int32),
                  Guarded((B,), torch.int32))
    w8.accept_from_keys(draft, argmax=am.t, accept_len=al.t, next_token=nt.t, workspace=wsp)
    ref_lg = torch.empty(R, V, dtype=torch.float32, device="cuda:0")
    w8.lm_head_argmax_tiled_act(xt, xs, wq, ws, K=K, logits=ref_lg)
    ref = w8.accept_from_keys(draft)
    torch.cuda.synchronize()
    assert lg.intact() and same_bits(lg.t, ref_lg)
    for name, g, r in (("argmax", am, ref[0]), ("accept_len", al, ref[1]), ("next_token", nt, ref[2])):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, r), f"{name} differs from the unguarded call"
    wsp.check()


@pytest.mark.parametrize("B,G,V", [(1, 4, 151941), (32, 8, 4099), (2, 0, 1)])
def test_guard_verify_accept(B, G, V):
    R = B * (G + 1)
    announce(f"guard verify_accept B={B} G={G} V={V}")
    logits = dev(synth.rng(W_GUARD, 60, V).standard_normal((R, V)).astype(np.float32))
    draft = dev(synth.draft_ids(W_GUARD, B, G, V, index=2))
    wsp = GuardedWorkspace()
    am, al, nt = (Guarded((R,), torch.int32), Guarded((B,), torch.int32),
                  Guarded((B,), torch.int32))
    w8.verify_accept(logits, draft, argmax=am.t, accept_len=al.t, next_token=nt.t, workspace=wsp)
    ref = w8.verify_accept(logits, draft)
    torch.cuda.synchronize()
    for name, g, r in (("argmax", am, ref[0]), ("accept_len", al, ref[1]), ("next_token", nt, ref[2])):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, r), f"{name} differs from the unguarded call"
    for use, g in wsp.all:
        assert g.intact(), f"workspace '{use}' guard band overwritten"


@pytest.mark.parametrize("M,N,K", [(5, 4099, 4096), (16, 17, 4224), (1, 151941, 256)])
def test_guard_w4a8(M, N, K):
    announce(f"guard W4A8 M={M} N={N} K={K}")
    w = dev(synth.weights_f32(W_GUARD, N, K, tensor_index=600 + M))
    wq4, ws = w8.quantize_weight_w4(w)
    xq, xs = w8.quantize_act(act(M, K, 14))
    outs = {"y_bf16": Guarded((M, N), torch.bfloat16), "y_f32": Guarded((M, N), torch.float32),
            "acc": Guarded((M, N), torch.int32)}
    w8.linear_w4(xq, xs, wq4, ws, y_bf16=outs["y_bf16"].t, y_f32=outs["y_f32"].t, acc=outs["acc"].t)
    ref = w8.linear_w4(xq, xs, wq4, ws, want_f32=True, want_acc=True)
    wsp = GuardedWorkspace()
    lg = Guarded((M, N), torch.float32)
    w8.lm_head_argmax_w4(xq, xs, wq4, ws, logits=lg.t, workspace=wsp)
    draft = dev(synth.draft_ids(W_GUARD, 1, M - 1, N, index=3))
    am, al, nt = w8.accept_from_keys(draft, workspace=wsp)
    ref_lg = torch.empty(M, N, dtype=torch.float32, device="cuda:0")
    w8.lm_head_argmax_w4(xq, xs, wq4, ws, logits=ref_lg)
    ram, ral, rnt = w8.accept_from_keys(draft)
    torch.cuda.synchronize()
    for (name, g), r in zip(outs.items(), ref):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, r), f"{name} differs from the unguarded call"
    assert lg.intact() and same_bits(lg.t, ref_lg)
    assert same_bits(am, ram) and same_bits(al, ral) and same_bits(nt, rnt)
    wsp.check()


@pytest.mark.parametrize("M,D", [(1, 16), (7, 4112), (289, 4096)])
def test_guard_residual_rmsnorm_quant(M, D):
    announce(f"guard residual_rmsnorm_quant M={M} D={D}")
    h, delta = act(M, D, 20), act(M, D, 21)
    gamma = dev_bf16(synth.activations_bf16(W_GUARD, 1, D, index=22)[0])
    s = dev(synth.smoothing_vector(W_GUARD, D))
    g = {"xq": Guarded((M, D), torch.int8), "x_scale": Guarded((M,), torch.float32),
         "normed": Guarded((M, D), torch.bfloat16), "h_out": Guarded((M, D), torch.bfloat16)}
    w8.residual_rmsnorm_quant(h, gamma, 1e-6, delta=delta, smooth=s, h_out=g["h_out"].t,
                              normed=g["normed"].t, xq=g["xq"].t, x_scale=g["x_scale"].t)
    ref = w8.residual_rmsnorm_quant(h, gamma, 1e-6, delta=delta, smooth=s, want_normed=True)
    torch.cuda.synchronize()
    for (name, gd), r in zip(g.items(), ref):
        assert gd.intact(), f"{name} guard band overwritten"
        assert same_bits(gd.t, r), f"{name} differs from the unguarded call"


@pytest.mark.parametrize("M,F", [(1, 16), (5, 12304), (289, 3088)])
def test_guard_silu_mul_quant(M, F):
    announce(f"guard silu_mul_quant M={M} F={F}")
    gu = act(M, 2 * F, 23)                      # a fused [gate;up] output: column halves
    gate, up = gu[:, :F], gu[:, F:]
    g = {"xq": Guarded((M, F), torch.int8), "x_scale": Guarded((M,), torch.float32),
         "act": Guarded((M, F), torch.bfloat16)}
    w8.silu_mul_quant(gate, up, act=g["act"].t, xq=g["xq"].t, x_scale=g["x_scale"].t)
    ref = w8.silu_mul_quant(gate, up, want_act=True)
    torch.cuda.synchronize()
    for (name, gd), r in zip(g.items(), ref):
        assert gd.intact(), f"{name} guard band overwritten"
        assert same_bits(gd.t, r), f"{name} differs from the unguarded call"


def _bf16_normal(shape, index, scale=1.0):
    z = synth.rng(W_GUARD, 40, index).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return dev_bf16(synth.to_bf16_bits(z))


@pytest.mark.parametrize("B,T,Hq,Hkv,Lmax,lengths", [(3, 5, 16, 4, 304, [300, 5, 123]),
                                                     (1, 8, 64, 8, 4096, [4096]),
                                                     (2, 1, 8, 8, 64, [1, 64])])
def test_guard_verify_attention_and_append(B, T, Hq, Hkv, Lmax, lengths):
    """The attention output and workspace, and the q output of the q/k norm +
    rotary + cache append with both caches inside guard bands (rows past
    each sequence's block untouched)."""
    announce(f"guard verify_attention B={B} T={T} Hq={Hq} Hkv={Hkv} Lmax={Lmax}")
    lengths = dev(np.asarray(lengths, dtype=np.int32))
    qkv = _bf16_normal((B * T, (Hq + 2 * Hkv) * 128), 1, 2.0)
    qg, kg = _bf16_normal((128,), 2), _bf16_normal((128,), 3)
    k0, v0 = _bf16_normal((B, Hkv, Lmax, 128), 4), w8.pack_v_cache(_bf16_normal((B, Hkv, Lmax, 128), 5))
    kc, vc = Guarded((B, Hkv, Lmax, 128), torch.bfloat16), Guarded((B, Hkv, Lmax, 128), torch.bfloat16)
    kc.t.copy_(k0)
    vc.t.copy_(v0)
    qo = Guarded((B, T, Hq, 128), torch.bfloat16)
    w8.qk_norm_rope_append(qkv, qg, kg, lengths, kc.t, vc.t, T=T, Hq=Hq, Hkv=Hkv, q_out=qo.t)
    k1, v1 = k0.clone(), v0.clone()
    q1 = w8.qk_norm_rope_append(qkv, qg, kg, lengths, k1, v1, T=T, Hq=Hq, Hkv=Hkv)
    wsp = GuardedWorkspace()
    out = Guarded((B, T, Hq, 128), torch.bfloat16)
    w8.verify_attention(qo.t, kc.t, vc.t, lengths, out=out.t, workspace=wsp)
    ref = w8.verify_attention(q1, k1, v1, lengths)
    torch.cuda.synchronize()
    for name, g, r in (("q_out", qo, q1), ("k_cache", kc, k1), ("v_cache", vc, v1), ("out", out, ref)):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, r), f"{name} differs from the unguarded call"
    wsp.check()


@pytest.mark.parametrize("B,G,V,t", [(3, 4, 4099, 1.0), (1, 0, 1, 0.7), (32, 8, 151941, 0.3)])
def test_guard_verify_sample(B, G, V, t):
    announce(f"guard verify_sample B={B} G={G} V={V} T={t}")
    R = B * (G + 1)
    y = dev(synth.rng(W_GUARD, 41, V).standard_normal((R, V), dtype=np.float32))
    d = dev(synth.draft_ids(W_GUARD, B, G, V, index=5))
    r = synth.rng(W_GUARD, 42, V)
    ua = torch.from_numpy(r.integers(0, 1 << 32, size=(B, G), dtype=np.uint64)
                          .astype(np.uint32).view(np.int32).copy()).cuda()
    us = torch.from_numpy(r.integers(0, 1 << 64, size=(B,), dtype=np.uint64).view(np.int64).copy()).cuda()
    wsp = GuardedWorkspace()
    al, nt = Guarded((B,), torch.int32), Guarded((B,), torch.int32)
    w8.verify_sample(y, d, t, ua, us, accept_len=al.t, next_token=nt.t, workspace=wsp)
    ral, rnt = w8.verify_sample(y, d, t, ua, us)
    wts = Guarded((R, V), torch.int64)
    w8.sample_weights(y, t, weights=wts.t, workspace=wsp)
    rw = w8.sample_weights(y, t)
    torch.cuda.synchronize()
    for name, g, ref in (("accept_len", al, ral), ("next_token", nt, rnt), ("weights", wts, rw)):
        assert g.intact(), f"{name} guard band overwritten"
        assert same_bits(g.t, ref), f"{name} differs from the unguarded call"
    wsp.check()

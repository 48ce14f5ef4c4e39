"""The C ABI without a GPU: the library loads, exports every function that
include/w8a8.h declares, and rejects bad arguments on the host before
anything is enqueued (no call here reaches a kernel launch)."""
import ctypes

import pytest

from w8a8_quantized_verification_amd import _lib

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
A16 = 0x10000  # fake, 16-byte aligned addresses: validation never dereferences them
A16b = 0x20000


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_version_and_status_strings(lib):
    assert lib.w8a8_abi_version() == 1
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, 99):
        assert lib.w8a8_status_string(s)


def q_act(lib, x=A16, smooth=None, M=5, K=4096, xq=A16b, xs=A16):
    return lib.w8a8_quantize_act(x, smooth, M, K, xq, xs, None)


def test_quantize_act_validation(lib):
    assert q_act(lib, xs=None) == INVALID
    assert q_act(lib, x=None) == INVALID
    assert q_act(lib, K=17) == INVALID
    assert q_act(lib, K=-16) == INVALID
    assert q_act(lib, M=-1) == INVALID
    assert q_act(lib, K=133144 + 16) == INVALID
    assert q_act(lib, x=A16 + 2) == INVALID          # misaligned input
    assert q_act(lib, smooth=A16 + 4) == INVALID     # misaligned smoothing vector
    assert q_act(lib, K=24) == INVALID
    assert b"K must be a multiple of 16" in lib.w8a8_last_error()
    # empty problem: a no-op that needs no pointers
    assert q_act(lib, x=None, M=0, xq=None, xs=None) == OK
    assert lib.w8a8_last_error() == b""


def test_quantize_weight_validation(lib):
    f = lib.w8a8_quantize_weight
    assert f(A16, None, 10, 4096, A16b, None, None) == INVALID
    assert f(A16 + 8, None, 10, 4096, A16b, A16, None) == INVALID
    assert f(None, None, 0, 4096, None, None, None) == OK


def lin(lib, xq=A16, xs=A16, wq=A16b, ws=A16, M=5, N=4096, K=4096, yb=A16, yf=None, acc=None,
        work=None, wbytes=0):
    return lib.w8a8_linear(xq, xs, wq, ws, M, N, K, yb, yf, acc, work, wbytes, None)


def test_linear_validation(lib):
    assert lin(lib, yb=None) == INVALID                 # no output requested
    assert lin(lib, K=4100) == INVALID
    assert lin(lib, K=133144 + 16) == INVALID
    assert lin(lib, xq=A16 + 1) == INVALID
    assert lin(lib, wq=A16 + 8) == INVALID
    assert lin(lib, yf=A16 + 2) == INVALID
    assert lin(lib, N=-3) == INVALID
    assert lin(lib, M=0, xq=None, xs=None, wq=None, ws=None, yb=None) == OK
    assert lin(lib, N=0) == OK


def test_linear_workspace(lib):
    # an output of one 16-channel tile splits K across workgroups and needs
    # scratch; the LM head and the layer shapes do not
    need = lib.w8a8_linear_workspace_bytes(5, 16, 25600)
    assert need >= 5 * 16 * 4
    assert lib.w8a8_linear_workspace_bytes(5, 151936, 4096) == 0
    assert lib.w8a8_linear_workspace_bytes(5, 1024, 4096) == 0
    assert lib.w8a8_linear_workspace_bytes(0, 16, 25600) == 0
    assert lin(lib, N=16, K=25600, work=None) == WORKSPACE
    assert lin(lib, N=16, K=25600, work=A16, wbytes=need - 1) == WORKSPACE
    assert lin(lib, N=16, K=25600, work=A16 + 16, wbytes=need) == INVALID  # alignment


def test_batched_split_workspace(lib):
    # above 16 rows, tiled weights: a long reduction on a mid-size grid
    # (288 x 4096, 192 k steps) is split across workgroups and needs the
    # workspace; K = 4096 (64 steps), row-major weights and row-major
    # activations with K % 64 != 0 do not split
    need = lib.w8a8_linear_tiled_act_workspace_bytes(288, 4096, 12288)
    assert need >= 288 * 4096 * 4
    assert lib.w8a8_linear_workspace_bytes(288, 4096, 12288) == need
    assert lib.w8a8_linear_tiled_act_workspace_bytes(288, 4096, 4096) == 0
    assert lib.w8a8_linear_tiled_act_workspace_bytes(288, 4096, 8208) > 0
    assert lib.w8a8_linear_workspace_bytes(288, 4096, 8208) == 0
    assert lib.w8a8_linear_tiled_act_workspace_bytes(17, 4096, 12288) == 0
    assert lib.w8a8_linear_tiled_act_workspace_bytes(0, 4096, 12288) == 0
    f = lib.w8a8_linear_tiled_act
    args = (A16, A16, A16b, A16, 288, 4096, 12288, A16, None, None)
    assert f(*args, None, 0, None) == WORKSPACE
    assert f(*args, A16, need - 1, None) == WORKSPACE
    assert f(*args, A16 + 16, need, None) == INVALID     # 256-byte alignment
    assert b"256-byte" in lib.w8a8_last_error()
    assert f(A16, A16, A16b, A16, 288, 4096, 12288, None, None, None, A16, need, None) == INVALID
    assert lib.w8a8_linear_tiled(A16, A16, A16b, A16, 288, 4096, 12288, A16, None, None, None, 0,
                                 None) == WORKSPACE
    assert f(None, None, None, None, 0, 4096, 12288, None, None, None, None, 0, None) == OK


def test_linear_workspace_split_tail(lib, monkeypatch):
    # 320 tiles of 128 k steps over 256 CUs: the 64 tiles past the last whole
    # round are split, so the call needs the split workspace; short tiles
    # (K = 4096) and outputs narrower than the CUs do not split their tail
    assert lib.w8a8_linear_workspace_bytes(8, 5120, 8192) >= 8 * 5120 * 4
    assert lib.w8a8_linear_workspace_bytes(5, 6144, 4096) == 0
    assert lib.w8a8_linear_workspace_bytes(5, 1024, 8192) == 0
    monkeypatch.setenv("W8A8_TAIL", "-1")
    assert lib.w8a8_linear_workspace_bytes(8, 5120, 8192) == 0


def test_linear_workspace_follows_split_override(lib, monkeypatch):
    monkeypatch.setenv("W8A8_SPLITK", "4")
    assert lib.w8a8_linear_workspace_bytes(5, 1024, 4096) >= 5 * 1024 * 4
    monkeypatch.delenv("W8A8_SPLITK")
    assert lib.w8a8_linear_workspace_bytes(5, 1024, 4096) == 0


def va(lib, logits=A16, V=151936, draft=A16, B=1, G=4, am=None, al=A16, nt=A16b, work=A16,
       wbytes=None):
    if wbytes is None:
        wbytes = lib.w8a8_verify_accept_workspace_bytes(B, G, V)
    return lib.w8a8_verify_accept(logits, V, draft, B, G, am, al, nt, work, wbytes, None)


def test_verify_accept_validation(lib):
    assert lib.w8a8_verify_accept_workspace_bytes(1, 4, 151936) > 0
    assert va(lib, G=256) == INVALID
    assert va(lib, G=-1) == INVALID
    assert va(lib, V=0) == INVALID
    assert va(lib, draft=None) == INVALID
    assert va(lib, al=None) == INVALID
    assert va(lib, logits=A16 + 2) == INVALID
    assert va(lib, work=None) == WORKSPACE
    assert va(lib, wbytes=8) == WORKSPACE
    assert va(lib, B=0, logits=None, draft=None, al=None, nt=None, work=None) == OK


def vs(lib, logits=A16, V=151936, draft=A16, B=1, G=4, T=1.0, ua=A16, us=A16, al=A16, nt=A16,
       work=A16, wbytes=None):
    if wbytes is None:
        wbytes = lib.w8a8_verify_sample_workspace_bytes(B, G, V)
    return lib.w8a8_verify_sample(logits, V, draft, B, G, T, ua, us, al, nt, work, wbytes, None)


def test_verify_sample_validation(lib):
    assert lib.w8a8_verify_sample_workspace_bytes(1, 4, 151936) > 0
    assert lib.w8a8_verify_sample_workspace_bytes(1, 4, (1 << 23) + 1) == 0
    for bad_t in (0.0, -1.0, float("inf"), float("nan"), 1e-40):
        assert vs(lib, T=bad_t) == INVALID
    assert vs(lib, V=(1 << 23) + 1, wbytes=1 << 30) == INVALID
    assert vs(lib, G=256) == INVALID
    assert vs(lib, ua=None) == INVALID
    assert vs(lib, us=None) == INVALID
    assert vs(lib, us=A16 + 4) == INVALID
    assert vs(lib, nt=None) == INVALID
    assert vs(lib, work=None) == WORKSPACE
    assert vs(lib, wbytes=8) == WORKSPACE
    assert vs(lib, work=A16 + 16) == INVALID
    assert vs(lib, B=0, logits=None, draft=None, ua=None, us=None, al=None, nt=None,
              work=None) == OK
    f = lib.w8a8_sample_weights
    need = lib.w8a8_sample_weights_workspace_bytes(3, 1000)
    assert need > 0
    assert f(A16, 3, 1000, 1.0, A16 + 4, A16, need, None) == INVALID
    assert f(A16, 3, 1000, 0.0, A16, A16, need, None) == INVALID
    assert f(A16, 3, 1000, 1.0, A16, A16, 8, None) == WORKSPACE
    assert f(None, 0, 1000, 1.0, None, None, 0, None) == OK


def test_w4a8_validation(lib):
    assert lib.w8a8_w4_weight_bytes(151936, 4096) == 151936 * 4096 // 2
    assert lib.w8a8_w4_weight_bytes(17, 80) == 32 * 128 // 2
    q = lib.w8a8_quantize_weight_w4
    assert q(A16, None, 512, 250, A16b, A16, None) == INVALID        # K % 16
    assert q(A16 + 4, None, 512, 256, A16b, A16, None) == INVALID    # w alignment
    assert q(A16, None, 512, 256, None, A16, None) == INVALID
    assert q(None, None, 0, 256, None, None, None) == OK
    f = lib.w8a8_linear_w4
    assert f(A16, A16, A16b, A16, 5, 512, 256, None, None, None, None) == INVALID   # no output
    assert f(A16, A16, A16b + 8, A16, 5, 512, 256, A16, None, None, None) == INVALID
    assert f(A16, A16, A16b, A16, 5, 512, 136000, A16, None, None, None) == INVALID  # K too big
    assert f(None, None, None, None, 0, 512, 256, None, None, None, None) == OK
    g = lib.w8a8_lm_head_argmax_w4
    need = lib.w8a8_lm_head_verify_workspace_bytes(1, 4, 151936, 4096)
    assert g(A16, A16, A16b, A16, 5, 151936, 4096, None, A16, 8, None) == WORKSPACE
    assert g(A16, A16, A16b, A16, 5, 151936, 4096, None, A16 + 16, need, None) == INVALID
    assert g(A16, A16, A16b, A16, 5, 0, 4096, None, A16, need, None) == INVALID


def test_glue_validation(lib):
    f = lib.w8a8_residual_rmsnorm_quant
    assert f(A16, None, A16, 1e-6, None, 5, 4008, None, None, A16b, A16, None) == INVALID  # D % 16
    assert f(A16, None, A16, 1e-6, None, 5, 40000, None, None, A16b, A16, None) == INVALID  # > 32768
    assert f(A16, None, A16, -1.0, None, 5, 4096, None, None, A16b, A16, None) == INVALID   # eps
    assert f(A16 + 8, None, A16, 1e-6, None, 5, 4096, None, None, A16b, A16, None) == INVALID
    assert f(None, None, A16, 1e-6, None, 5, 4096, None, None, A16b, A16, None) == INVALID
    assert f(None, None, None, 1e-6, None, 0, 4096, None, None, None, None, None) == OK
    g = lib.w8a8_silu_mul_quant
    assert g(A16, A16b, 100, None, 5, 128, None, A16, A16, None) == INVALID   # stride < F
    assert g(A16, A16b, 132, None, 5, 128, None, A16, A16, None) == INVALID   # stride % 8
    assert g(A16, None, 256, None, 5, 128, None, A16, A16, None) == INVALID
    assert g(None, None, 256, None, 0, 128, None, None, None, None) == OK


def test_verify_attention_validation(lib):
    f = lib.w8a8_verify_attention
    need = lib.w8a8_verify_attention_workspace_bytes(1, 8, 4096)
    assert need > 0
    args = dict(q=A16, k=A16b, v=A16, ln=A16, B=1, T=5, Hq=32, Hkv=8, Dh=128, L=4096, out=A16,
                w=A16, wb=need)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["ln"], a["B"], a["T"], a["Hq"], a["Hkv"], a["Dh"],
                 a["L"], a["out"], a["w"], a["wb"], None)
    assert call(Dh=64) == UNSUPPORTED
    assert call(T=17) == UNSUPPORTED          # 17 * 4 > 64 query rows per kv head
    assert call(Hq=30) == INVALID
    assert call(L=4) == INVALID
    assert call(L=4100) == INVALID            # not a multiple of 16
    assert lib.w8a8_verify_attention_workspace_bytes(1, 8, 4100) == 0
    assert call(q=A16 + 8) == INVALID
    assert call(ln=None) == INVALID
    assert call(wb=8) == WORKSPACE
    assert call(B=0, q=None, k=None, v=None, ln=None, out=None, w=None) == OK


def test_pack_v_cache_validation(lib):
    f = lib.w8a8_pack_v_cache
    assert f(A16, 1, 8, 4096, 64, A16b, None) == UNSUPPORTED
    assert f(A16, 1, 8, 4100, 128, A16b, None) == INVALID
    assert f(A16, 1, 8, 4096, 128, None, None) == INVALID
    assert f(A16, 1, 8, 4096, 128, A16b + 8, None) == INVALID       # output 16-byte alignment
    assert f(A16, 1, 1, 64, 128, A16 + 64, None) == INVALID         # overlap
    assert f(None, 0, 8, 4096, 128, None, None) == OK


def test_lm_head_argmax_timed_validation(lib):
    """The kernel-timestamped LM-head launch: both events required, M <= 16,
    and the checks of w8a8_lm_head_argmax before any launch."""
    ws = 32 * 64 * 256
    EV0, EV1 = 0x30000, 0x40000   # fake handles: validation never touches them

    def f(M=5, ev0=EV0, ev1=EV1, wsb=ws, xq=A16):
        return lib.w8a8_lm_head_argmax_timed(xq, A16, A16b, A16, M, 151936, 4096, None, A16, wsb,
                                             ev0, ev1, None)

    assert f(ev0=None) == INVALID
    assert f(ev1=None) == INVALID
    assert f(M=17) == UNSUPPORTED
    assert f(wsb=ws // 64) == WORKSPACE
    assert f(xq=A16 + 4) == INVALID
    assert f(M=0, ev0=EV0) == OK


def test_lm_head_argmax_tiled_act_validation(lib):
    f = lib.w8a8_lm_head_argmax_tiled_act
    ws = 288 * 64 * 256
    assert f(None, A16, A16b, A16, 288, 151936, 4096, None, A16, ws, None) == INVALID
    assert f(A16 + 4, A16, A16b, A16, 288, 151936, 4096, None, A16, ws, None) == INVALID
    assert f(A16, A16, A16b, A16, 288, 151936, 4100, None, A16, ws, None) == INVALID
    assert f(A16, A16, A16b, A16, 288, 0, 4096, None, A16, ws, None) == INVALID
    assert f(A16, A16, A16b, A16, 288, 151936, 4096, None, A16, ws - 1, None) == WORKSPACE
    assert f(A16, A16, A16b, A16, 288, 151936, 4096, None, A16 + 16, ws, None) == INVALID
    assert f(None, None, None, None, 0, 151936, 4096, None, None, 0, None) in (OK, WORKSPACE)


def test_bf16_linear_validation(lib):
    f = lib.w8a8_bf16_linear
    assert f(A16, A16b, 17, 512, 256, A16, None, None) == UNSUPPORTED
    assert f(A16, A16b, 5, 512, 250, A16, None, None) == INVALID
    assert f(A16, A16b, 5, 512, 256, None, None, None) == INVALID
    assert f(A16 + 2, A16b, 5, 512, 256, A16, None, None) == INVALID
    assert f(None, None, 0, 512, 256, None, None, None) == OK


def test_bf16_tiled_validation(lib):
    assert lib.w8a8_bf16_tiled_weight_bytes(151936, 4096) == 9496 * 128 * 1024
    assert lib.w8a8_bf16_tiled_weight_bytes(17, 48) == 2 * 2 * 1024
    assert lib.w8a8_bf16_tiled_weight_bytes(0, 48) == 0
    t = lib.w8a8_tile_weight_bf16
    assert t(A16, 17, 40, A16b, None) == INVALID          # K % 16
    assert t(A16 + 2, 17, 48, A16b, None) == INVALID      # misaligned
    assert t(None, 17, 48, A16b, None) == INVALID
    assert t(None, 0, 48, None, None) == OK
    f = lib.w8a8_bf16_linear_tiled
    assert f(A16, A16b, 17, 512, 256, A16, None, None) == UNSUPPORTED
    assert f(A16, A16b, 5, 512, 250, A16, None, None) == INVALID
    assert f(A16, A16b, 5, 512, 256, None, None, None) == INVALID
    assert f(A16 + 2, A16b, 5, 512, 256, A16, None, None) == INVALID
    assert f(None, None, 0, 512, 256, None, None, None) == OK


def test_last_error_is_per_call(lib):
    assert q_act(lib, K=24) == INVALID
    assert lib.w8a8_last_error()
    assert q_act(lib, M=0) == OK
    assert lib.w8a8_last_error() == b""


def test_python_binding_rejects_cpu_tensors():
    import torch
    import w8a8_quantized_verification_amd as w
    x = torch.zeros(5, 256, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="ROCm device"):
        w.quantize_act(x)


def test_workspace_keeps_keys_apart_from_split_k_partials():
    """The LM-head argmax keys stay non-zero between its two phases, so they
    must not share a buffer with the split-K partials that a linear between
    the phases would add onto (host-side bookkeeping; CPU tensors stand in
    for device buffers)."""
    import torch
    import w8a8_quantized_verification_amd as w
    ws = w.Workspace()
    cpu = torch.device("cpu")
    zeroed = ws.get(4096, cpu, use="zeroed")
    keys = ws.get(4096, cpu, use="keys")
    verify = ws.get(4096, cpu, use="verify")
    ptrs = {zeroed.data_ptr(), keys.data_ptr(), verify.data_ptr()}
    assert len(ptrs) == 3
    keys.fill_(7)                                    # keys left behind by phase 1
    again = ws.get(4096, cpu, use="zeroed")          # a split-K linear in between
    assert again.data_ptr() == zeroed.data_ptr() and not bool(again.any())
    assert ws.get(4096, cpu, use="keys").data_ptr() == keys.data_ptr()
    with pytest.raises(ValueError, match="unknown workspace use"):
        ws.get(16, cpu, use="partials")


def test_python_binding_uses_keys_slot_for_the_argmax_phases():
    """Every LM-head argmax / acceptance binding takes the keys slot, and the
    split-K linear the zeroed slot (read from the binding's source)."""
    import inspect
    import w8a8_quantized_verification_amd.api as api
    for fn in (api.lm_head_verify, api.lm_head_argmax, api.lm_head_argmax_tiled_act,
               api.accept_from_keys, api.lm_head_argmax_w4):
        src = inspect.getsource(fn)
        assert 'use="keys"' in src and 'use="zeroed"' not in src, fn.__name__
    assert 'use="zeroed"' in inspect.getsource(api.linear)


def test_hbm_read_probe_validation(lib):
    sink = 4096
    # ragged size, NULL sink, NULL buffer with bytes > 0, misalignment, one event alone
    assert lib.w8a8_hbm_read_probe(16, 24, sink, None, None, None) == INVALID
    assert lib.w8a8_hbm_read_probe(16, 32, None, None, None, None) == INVALID
    assert lib.w8a8_hbm_read_probe(None, 32, sink, None, None, None) == INVALID
    assert lib.w8a8_hbm_read_probe(8, 32, sink, None, None, None) == INVALID
    assert lib.w8a8_hbm_read_probe(16, 32, 2, None, None, None) == INVALID
    assert lib.w8a8_hbm_read_probe(16, 32, sink, 1, None, None) == INVALID
    assert b"both events" in lib.w8a8_last_error()

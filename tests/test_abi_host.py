"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before any HIP
call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import lm_head_top_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdtopk.h")

KD_OK, KD_ERR_INVALID_ARG, KD_ERR_UNSUPPORTED, KD_ERR_WORKSPACE, KD_ERR_HIP = range(5)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kd.lib_path()):
        pytest.skip("libkdtopk.so not built")
    return kd.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("kd_topk_kl_forward", "kd_topk_kl_backward", "kd_topk_kl_workspace_size",
                 "kd_topk_kl_validate", "kd_status_string", "kd_last_hip_error"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.kd_status_string(0) == b"ok"
    assert lib.kd_status_string(3) == b"workspace too small"
    assert lib.kd_status_string(5) == b"cached id outside [0, V)"
    assert lib.kd_status_string(6) == b"device bounds check failed"
    assert lib.kd_status_string(99) == b"unknown status"


def test_debug_library_exports_the_same_symbols(lib):
    path = kd.debug_lib_path()
    if not os.path.exists(path):
        pytest.skip("libkdtopk_debug.so not built")
    dbg = ctypes.CDLL(path)
    for name in _declared_functions():
        assert hasattr(dbg, name), name
    dbg.kd_topk_kl_workspace_size.restype = ctypes.c_size_t
    args = (ctypes.c_int64(8192), ctypes.c_int64(4096), ctypes.c_int64(131072), ctypes.c_int32(100),
            ctypes.c_int64(1024))
    assert dbg.kd_topk_kl_workspace_size(*args) == lib.kd_topk_kl_workspace_size(8192, 4096, 131072, 100, 1024)


def test_validate_env_does_not_touch_argument_checks(lib, monkeypatch):
    # KD_VALIDATE=1 runs only after the host checks pass, so a rejected call
    # still returns its status before any HIP call
    monkeypatch.setenv("KD_VALIDATE", "1")
    assert lib.kd_topk_kl_forward(None, None, None, None, 1, 8, 8, 1, 1.0, 1, None, None, None,
                                  None, 0, None) == KD_ERR_INVALID_ARG
    assert lib.kd_last_hip_error() == b""


def test_last_hip_error_is_empty_without_a_failed_launch(lib):
    # argument errors are not HIP errors
    assert lib.kd_topk_kl_forward(None, None, None, None, 1, 8, 8, 1, 1.0, 1, None, None, None,
                                  None, 0, None) == KD_ERR_INVALID_ARG
    assert lib.kd_last_hip_error() == b""


def test_workspace_size_scales_with_chunk_not_N(lib):
    f = kd.workspace_size
    a = f(8192, 4096, 131072, 100, 1024)
    b = f(32768, 4096, 131072, 100, 1024)
    # only the 4-byte-per-row KL buffer grows with N
    assert 0 <= b - a <= 4 * (32768 - 8192) + 512
    # a group holds 8192 positions at chunk 1024 (8 chunks) and at 2048 (4)
    c = f(8192, 4096, 131072, 100, 2048)
    assert c == a
    # one chunk of 12288 positions is a group of its own: 4096 more G rows
    d = f(32768, 4096, 131072, 100, 12288)
    assert d > b + 131072 * 4096 * 2 - (64 << 20)
    # never O(N V): the dense fp32 grid at 32K x 131072 would be 16 GiB; the
    # workspace holds the G rows of one group of g chunks feeding the dH and
    # dW GEMMs (g = 8 at chunk 1024) plus per-chunk buffers: O(g chunk V)
    V, c, g = 131072, 1024, 8
    assert b <= g * c * V * 2 + (256 << 20)


def test_workspace_size_rejects(lib):
    f = kd.workspace_size
    assert f(10, 12, 100, 5, 4) == 0          # D not a multiple of 8
    assert f(10, 16, 100, 0, 4) == 0          # K = 0
    assert f(10, 16, 100, 101, 4) == 0        # K > V
    assert f(10, 16, 100, 5, 0) == 0          # chunk = 0
    assert f(10, 16, 1000, 257, 4) == 0       # K > KD_MAX_K
    assert f(10, 16, (1 << 20) + 1, 5, 4) == 0
    assert f(-1, 16, 100, 5, 4) == 0
    assert f(0, 16, 100, 5, 4) > 0            # empty batch is valid


def test_keep_logits_workspace_adds_one_fp32_grid(lib):
    base = kd.workspace_size(8192, 4096, 131072, 100, 1024)
    kept = kd.keep_logits_workspace_size(8192, 4096, 131072, 100, 1024)
    assert 0 <= kept - base - 8192 * 131072 * 4 <= 512
    # V = 201088 keeps rows of Vp = 201216 (V rounded up to 256)
    b2 = kd.workspace_size(1000, 64, 201088, 8, 256)
    k2 = kd.keep_logits_workspace_size(1000, 64, 201088, 8, 256)
    assert 0 <= k2 - b2 - 1000 * 201216 * 4 <= 512
    assert kd.keep_logits_workspace_size(10, 12, 100, 5, 4) == 0   # D not a multiple of 8


def test_keep_logits_entry_points_reject(lib):
    v = ctypes.c_void_p
    ok = 1 << 24
    f = lib.kd_topk_kl_forward_keep_logits
    assert f(v(ok), v(ok), v(ok), v(ok), 4, 16, 64, 3, 1.0, 2, v(0), v(ok), v(0), v(ok), 1 << 30,
             v(0)) == KD_ERR_INVALID_ARG                                     # no loss
    assert f(v(ok), v(ok), v(ok), v(ok), 4, 16, 64, 3, 1.0, 2, v(ok), v(ok), v(0), v(ok), 16,
             v(0)) == KD_ERR_WORKSPACE
    b = lib.kd_topk_kl_backward_keep_logits
    assert b(v(ok), v(ok), v(ok), v(ok), v(ok), v(0), 4, 16, 64, 3, 1.0, 2, v(ok), v(0), v(ok), 1 << 30,
             v(0)) == KD_ERR_INVALID_ARG                                     # no dW
    assert b(v(ok), v(ok), v(ok), v(ok), v(ok), v(0), 4, 16, 64, 3, 1.0, 2, v(ok), v(ok), v(ok), 16,
             v(0)) == KD_ERR_WORKSPACE
    assert b(v(ok), v(ok), v(ok), v(ok), v(ok), v(0), 4, 16, 64, 3, 0.0, 2, v(ok), v(ok), v(ok), 1 << 30,
             v(0)) == KD_ERR_INVALID_ARG                                     # T = 0


def test_workspace_size_limits_of_32bit_operand_offsets(lib):
    f = kd.workspace_size
    # a chunk whose G rows exceed 2^31 elements is accepted (its gradient GEMMs
    # run in row blocks): 16384 x 131072 bf16 is 4 GiB of G
    big = f(32768, 4096, 131072, 100, 16384)
    assert big >= 16384 * 131072 * 2
    assert f(4096, 64, 1 << 20, 8, 4096) >= 4096 * (1 << 20) * 2
    # W [V, D] and one chunk of H [chunk, D] are read whole through 32-bit offsets
    assert f(16, 8192, (1 << 18) + 256, 5, 16) == 0      # V * D > 2^31 - 64
    assert f(1 << 20, 4096, 1024, 5, 1 << 19) == 0        # chunk * D > 2^31 - 64
    assert f(1 << 20, 4096, 1024, 5, (1 << 19) - 256) > 0
    assert f(16, 4096, 1 << 19, 5, 16) == 0                # V * D = 2^31
    assert f(16, 4096, (1 << 19) - 256, 5, 16) > 0


def _fwd(lib, **kw):
    a = dict(H=8192 * 16, W=8192 * 16, idx=1 << 20, t=1 << 21, N=4, D=16, V=64, K=3, T=1.0,
             chunk=2, loss=1 << 22, lse=1 << 23, row_kl=0, ws=1 << 24, ws_bytes=1 << 30, stream=0)
    a.update(kw)
    v = ctypes.c_void_p
    return lib.kd_topk_kl_forward(v(a["H"]), v(a["W"]), v(a["idx"]), v(a["t"]), a["N"], a["D"],
                                  a["V"], a["K"], a["T"], a["chunk"], v(a["loss"]), v(a["lse"]),
                                  v(a["row_kl"]), v(a["ws"]), a["ws_bytes"], v(a["stream"]))


def _bwd(lib, **kw):
    a = dict(H=8192 * 16, W=8192 * 16, idx=1 << 20, t=1 << 21, lse=1 << 23, g=0, N=4, D=16, V=64,
             K=3, T=1.0, chunk=2, dH=1 << 25, dW=1 << 26, ws=1 << 24, ws_bytes=1 << 30, stream=0)
    a.update(kw)
    v = ctypes.c_void_p
    return lib.kd_topk_kl_backward(v(a["H"]), v(a["W"]), v(a["idx"]), v(a["t"]), v(a["lse"]),
                                   v(a["g"]), a["N"], a["D"], a["V"], a["K"], a["T"], a["chunk"],
                                   v(a["dH"]), v(a["dW"]), v(a["ws"]), a["ws_bytes"], v(a["stream"]))


@pytest.mark.parametrize("kw,want", [
    (dict(H=0), KD_ERR_INVALID_ARG),
    (dict(W=0), KD_ERR_INVALID_ARG),
    (dict(idx=0), KD_ERR_INVALID_ARG),
    (dict(t=0), KD_ERR_INVALID_ARG),
    (dict(loss=0), KD_ERR_INVALID_ARG),
    (dict(lse=0), KD_ERR_INVALID_ARG),
    (dict(H=8192 * 16 + 2), KD_ERR_INVALID_ARG),      # misaligned bf16 rows
    (dict(idx=(1 << 20) + 2), KD_ERR_INVALID_ARG),
    (dict(row_kl=(1 << 22) + 1), KD_ERR_INVALID_ARG),
    (dict(T=0.0), KD_ERR_INVALID_ARG),
    (dict(T=-1.0), KD_ERR_INVALID_ARG),
    (dict(T=float("inf")), KD_ERR_INVALID_ARG),
    (dict(T=float("nan")), KD_ERR_INVALID_ARG),
    (dict(N=-1), KD_ERR_INVALID_ARG),
    (dict(D=12), KD_ERR_INVALID_ARG),
    (dict(K=0), KD_ERR_INVALID_ARG),
    (dict(K=65), KD_ERR_INVALID_ARG),
    (dict(V=1000, K=300), KD_ERR_UNSUPPORTED),
    (dict(V=(1 << 20) + 8), KD_ERR_UNSUPPORTED),
    (dict(chunk=0), KD_ERR_INVALID_ARG),
    (dict(ws=0), KD_ERR_WORKSPACE),
    (dict(ws_bytes=16), KD_ERR_WORKSPACE),
    (dict(ws=(1 << 24) + 16), KD_ERR_INVALID_ARG),
])
def test_forward_rejects_before_any_hip_call(lib, kw, want):
    assert _fwd(lib, **kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(dW=0), KD_ERR_INVALID_ARG),
    (dict(dH=0), KD_ERR_INVALID_ARG),
    (dict(lse=0), KD_ERR_INVALID_ARG),
    (dict(dW=(1 << 26) + 4), KD_ERR_INVALID_ARG),
    (dict(g=(1 << 27) + 2), KD_ERR_INVALID_ARG),
    (dict(T=0.0), KD_ERR_INVALID_ARG),
    (dict(K=65), KD_ERR_INVALID_ARG),
    (dict(ws_bytes=1), KD_ERR_WORKSPACE),
])
def test_backward_rejects_before_any_hip_call(lib, kw, want):
    assert _bwd(lib, **kw) == want


def _fwd_noalloc(lib, **kw):
    a = dict(H=8192 * 16, W=8192 * 16, idx=1 << 20, t=1 << 21, N=4, D=16, V=64, K=3, T=1.0,
             chunk=2, loss=1 << 22, lse=1 << 23, row_kl=0, stream=0)
    a.update(kw)
    v = ctypes.c_void_p
    return lib.kd_topk_kl_forward_noalloc(v(a["H"]), v(a["W"]), v(a["idx"]), v(a["t"]), a["N"], a["D"],
                                          a["V"], a["K"], a["T"], a["chunk"], v(a["loss"]), v(a["lse"]),
                                          v(a["row_kl"]), v(a["stream"]))


@pytest.mark.parametrize("kw,want", [
    (dict(H=0), KD_ERR_INVALID_ARG),
    (dict(loss=0), KD_ERR_INVALID_ARG),
    (dict(lse=0), KD_ERR_INVALID_ARG),
    (dict(idx=(1 << 20) + 2), KD_ERR_INVALID_ARG),
    (dict(T=0.0), KD_ERR_INVALID_ARG),
    (dict(K=65), KD_ERR_INVALID_ARG),
    (dict(V=(1 << 20) + 8), KD_ERR_UNSUPPORTED),
    # forward scratch beyond the library's 64 MiB array: 512 vocab tiles x
    # 16384 positions of (max, sum exp) partials alone take 64 MiB
    (dict(N=32768, D=64, V=131072, K=4, chunk=16384), KD_ERR_WORKSPACE),
])
def test_forward_noalloc_rejects_before_any_hip_call(lib, kw, want):
    assert _fwd_noalloc(lib, **kw) == want


def test_backward_empty_batch_is_a_no_op(lib):
    # N = 0: nothing to accumulate, nothing enqueued
    assert _bwd(lib, N=0, H=0, W=0, idx=0, t=0, lse=0, dH=0, ws=0, ws_bytes=0) == KD_OK


def test_validate_rejects(lib):
    v = ctypes.c_void_p
    assert lib.kd_topk_kl_validate(v(1 << 20), 4, 3, 64, v(0), v(0)) == KD_ERR_INVALID_ARG
    assert lib.kd_topk_kl_validate(v(1 << 20), 4, 0, 64, v(1 << 21), v(0)) == KD_ERR_INVALID_ARG
    assert lib.kd_topk_kl_validate(v(0), 4, 3, 64, v(1 << 21), v(0)) == KD_ERR_INVALID_ARG


def test_profile_api(lib):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    assert lib.kd_profile_enable(1 << 11) == KD_ERR_INVALID_ARG
    assert lib.kd_profile_read(-1, ctypes.byref(ms), ctypes.byref(n)) == KD_ERR_INVALID_ARG
    assert lib.kd_profile_enable(0) == KD_OK
    assert lib.kd_profile_enable(0x7FF) == KD_OK
    assert lib.kd_profile_enable(0) == KD_OK
    assert lib.kd_profile_read(1, ctypes.byref(ms), ctypes.byref(n)) == KD_OK
    assert n.value == 0 and ms.value == 0.0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    mod = importlib.reload(kd)
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "_HERE", str(tmp_path))
    with pytest.raises(ImportError):
        mod.load_library()
    monkeypatch.undo()
    importlib.reload(kd)


def test_one_hip_runtime_in_the_process():
    """Loading the library binds it to the HIP runtime torch uses, whatever was
    imported first (checked in a fresh interpreter)."""
    import subprocess
    import sys
    code = ("import lm_head_top_amd as kd; kd.load_library(); "
            "m = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))")
    if not os.path.exists(kd.lib_path()):
        pytest.skip("libkdtopk.so not built")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_topk_select_rejects(lib):
    vp = ctypes.c_void_p
    ok = vp(256)
    f = lib.kd_topk_select
    assert f(ok, 2, 4, 100, 10, ok, ok, None) == KD_ERR_INVALID_ARG      # dtype
    assert f(ok, 0, 4, 100, 101, ok, ok, None) == KD_ERR_INVALID_ARG     # K > V
    assert f(ok, 0, 4, 100, 0, ok, ok, None) == KD_ERR_INVALID_ARG       # K = 0
    assert f(ok, 0, -1, 100, 10, ok, ok, None) == KD_ERR_INVALID_ARG     # N < 0
    assert f(ok, 0, 4, 1000, 257, ok, ok, None) == KD_ERR_UNSUPPORTED    # K > KD_MAX_K
    assert f(ok, 0, 4, 1 << 31, 10, ok, ok, None) == KD_ERR_UNSUPPORTED  # V >= 2^31
    assert f(vp(2), 0, 4, 100, 10, ok, ok, None) == KD_ERR_INVALID_ARG   # fp32 needs 4-byte alignment
    assert f(None, 1, 4, 100, 10, ok, ok, None) == KD_ERR_INVALID_ARG    # null logits
    assert f(None, 0, 0, 100, 10, None, None, None) == KD_OK             # empty: nothing to do


def test_keep_workspace_is_order_N_times_V(lib):
    """The kept-gradient comparator holds G for every position: its workspace
    grows by about 2 V bytes per position (bf16 G), unlike the fused one."""
    f = kd.keep_workspace_size
    a = f(8192, 4096, 131072, 100, 1024)
    b = f(16384, 4096, 131072, 100, 1024)
    per_pos = (b - a) / 8192
    assert 2 * 131072 <= per_pos <= 2 * 131072 + 16
    assert a > kd.workspace_size(8192, 4096, 131072, 100, 1024)
    assert f(-1, 8, 8, 1, 1) == 0


def test_keep_entry_points_reject(lib):
    vp = ctypes.c_void_p
    ok = vp(256)
    assert lib.kd_topk_kl_backward_keep(ok, ok, None, 16, 8, 64, 4, 1.0, 8, ok, ok, ok, 16,
                                        None) == KD_ERR_WORKSPACE
    assert lib.kd_topk_kl_backward_keep(ok, ok, None, 16, 8, 64, 4, 1.0, 8, ok, vp(4), ok, 1 << 30,
                                        None) == KD_ERR_INVALID_ARG  # dW misaligned
    assert lib.kd_topk_kl_forward_keep(ok, ok, ok, ok, 16, 8, 64, 4, 1.0, 8, ok, ok, None, ok, 16,
                                       None) == KD_ERR_WORKSPACE
    assert lib.kd_topk_kl_forward_keep(ok, ok, ok, ok, 16, 7, 64, 4, 1.0, 8, ok, ok, None, ok, 1 << 30,
                                       None) == KD_ERR_INVALID_ARG  # D % 8


def test_dense_entry_points_reject(lib):
    vp = ctypes.c_void_p
    ok = vp(256)
    assert kd.dense_workspace_size(8192, 4096, 131070, 1024) == 0          # V % 4 != 0
    assert kd.dense_workspace_size(8192, 4096, 131072, 1024) > 0
    f = lib.kd_dense_kl_forward
    assert f(ok, ok, ok, 2, 16, 8, 64, 1.0, 8, ok, ok, ok, None, ok, 1 << 30, None) == KD_ERR_INVALID_ARG
    assert f(ok, ok, vp(264), 0, 16, 8, 64, 1.0, 8, ok, ok, ok, None, ok, 1 << 30,
             None) == KD_ERR_INVALID_ARG                                    # fp32 teacher not 16-byte aligned
    assert f(ok, ok, ok, 0, 16, 8, 64, 1.0, 8, ok, ok, ok, None, ok, 16, None) == KD_ERR_WORKSPACE
    b = lib.kd_dense_kl_backward
    assert b(ok, ok, ok, 0, ok, ok, None, 16, 8, 64, 1.0, 8, ok, vp(8), ok, 1 << 30,
             None) == KD_ERR_INVALID_ARG                                    # dW misaligned


def test_ext_entry_points_reject(lib):
    vp = ctypes.c_void_p
    ok = vp(256)
    f = lib.kd_topk_kl_forward_ex
    # H, W, idx, t, N, D, V, K, T, chunk, row_weight, labels, kd_w, ce_w, flags, loss, lse, row_loss, ws, bytes, s
    args = [ok, ok, ok, ok, 16, 8, 64, 4, 1.0, 8, None, None, 1.0, 0.0, 0, ok, ok, None, ok, 1 << 30, None]

    def fwd(kw):
        a = list(args)
        for k, v in kw.items():
            a[k] = v
        return f(*a)
    assert fwd({14: 2}) == KD_ERR_INVALID_ARG                 # unknown flag bit
    assert fwd({12: float("nan")}) == KD_ERR_INVALID_ARG      # kd_weight not finite
    assert fwd({13: float("inf")}) == KD_ERR_INVALID_ARG      # ce_weight not finite
    assert fwd({10: vp(258)}) == KD_ERR_INVALID_ARG           # row_weight misaligned
    assert fwd({11: vp(258)}) == KD_ERR_INVALID_ARG           # labels misaligned
    assert fwd({18: ok, 19: 16}) == KD_ERR_WORKSPACE
    b = lib.kd_topk_kl_backward_ex
    # H, W, idx, t, lse, g, N, D, V, K, T, chunk, row_weight, labels, kd_w, ce_w, flags, dH, dW, ws, bytes, s
    bargs = [ok, ok, ok, ok, ok, None, 16, 8, 64, 4, 1.0, 8, None, None, 1.0, 0.0, 0, ok, ok, ok, 1 << 30,
             None]

    def bwd(kw):
        a = list(bargs)
        for k, v in kw.items():
            a[k] = v
        return b(*a)
    assert bwd({16: 4}) == KD_ERR_INVALID_ARG
    assert bwd({18: vp(8)}) == KD_ERR_INVALID_ARG             # dW misaligned
    assert bwd({13: vp(2)}) == KD_ERR_INVALID_ARG             # labels misaligned
    assert bwd({20: 16}) == KD_ERR_WORKSPACE
    assert bwd({6: 0, 0: None, 1: None, 2: None, 3: None, 4: None, 17: None, 19: None,
                  20: 0}) == KD_OK                               # N = 0: nothing enqueued

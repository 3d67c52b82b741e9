"""The C ABI without a GPU: the library loads, exports every function that
include/mha.h declares, and its synchronous validation returns the documented
status codes before any device work."""
import ctypes
import os
import re

import pytest

from masked_head_attention_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 20  # a fake, 16-byte-aligned "device" address: never dereferenced


def _declared():
    with open(os.path.join(ROOT, "include", "mha.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mha_[a-z_]+)\s*\(", src)))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the binding raises: no call has a fallback."""
    import masked_head_attention_amd as M

    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "libmha.so"))
    with pytest.raises(ImportError, match="missing"):
        _abi.lib()
    with pytest.raises(ImportError, match="missing"):
        M.init()
    with pytest.raises(ImportError, match="missing"):
        M.prenorm_cross_workspace_size(2, 4, 8, 8, 64, M.BF16)


def test_exports_every_declared_symbol():
    lib = _abi.lib()
    names = _declared()
    assert "mha_fwd" in names and "mha_prenorm_cross_fwd" in names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _abi.SIGNATURES, n


def _fwd(q=A, k=A, v=A, mask=None, kind=0, B=1, H=1, Lq=4, Lk=4, D=64, scale=0.125, dtype=1,
         out=A):
    return _abi.STATUS[_abi.lib().mha_fwd(q, k, v, mask, kind, B, H, Lq, Lk, D, scale, dtype,
                                          None, out)]


def _pre(x=A, k=A, v=A, mask=None, kind=0, gamma=A, beta=A, eps=1e-5, residual=None, B=1, H=2,
         Lq=4, Lk=4, D=64, scale=0.125, dtype=2, out=A):
    return _abi.STATUS[_abi.lib().mha_prenorm_cross_fwd(x, k, v, mask, kind, gamma, beta, eps,
                                                        residual, B, H, Lq, Lk, D, scale, dtype,
                                                        None, out)]


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), "MHA_E_DTYPE"),
    (dict(kind=32), "MHA_E_MASK"),
    (dict(kind=_abi.KEEP | _abi.ADDITIVE, mask=A), "MHA_E_MASK"),
    (dict(kind=_abi.KEEP | _abi.PADDING, mask=A), "MHA_E_MASK"),
    (dict(kind=_abi.PER_HEAD), "MHA_E_MASK"),
    (dict(kind=_abi.PER_HEAD | _abi.PADDING, mask=A), "MHA_E_MASK"),
    (dict(kind=_abi.KEEP, mask=None), "MHA_E_NULL"),
    (dict(kind=_abi.KEEP, mask=A + 4), "MHA_E_ALIGN"),
    (dict(kind=_abi.KEEP | _abi.PER_HEAD, mask=A, B=1 << 20, H=1 << 20, Lq=1 << 12, Lk=1 << 12),
     "MHA_E_OVERFLOW"),
    (dict(kind=_abi.PADDING | _abi.ADDITIVE, mask=A), "MHA_E_MASK"),
    (dict(kind=0, mask=A), "MHA_E_MASK"),
    (dict(kind=_abi.PADDING, mask=None), "MHA_E_NULL"),
    (dict(kind=_abi.ADDITIVE, mask=None), "MHA_E_NULL"),
    (dict(B=-1), "MHA_E_SHAPE"),
    (dict(Lk=-3), "MHA_E_SHAPE"),
    (dict(D=48), "MHA_E_UNSUPPORTED"),
    (dict(D=256), "MHA_E_UNSUPPORTED"),
    (dict(scale=float("nan")), "MHA_E_ARG"),
    (dict(scale=float("inf")), "MHA_E_ARG"),
    (dict(scale=-0.5), "MHA_E_ARG"),
    (dict(q=None), "MHA_E_NULL"),
    (dict(out=None), "MHA_E_NULL"),
    (dict(k=None), "MHA_E_NULL"),
    (dict(q=A + 8), "MHA_E_ALIGN"),
    (dict(out=A + 2), "MHA_E_ALIGN"),
    (dict(kind=_abi.ADDITIVE, mask=A + 4), "MHA_E_ALIGN"),
    (dict(kind=_abi.PADDING, mask=A + 2), "MHA_E_ALIGN"),
    (dict(B=1 << 30, H=1 << 30, Lq=1 << 20), "MHA_E_OVERFLOW"),
    (dict(B=1 << 16, H=1 << 14, Lq=1 << 12), "MHA_E_OVERFLOW"),
    # 32-bit buffer ranges: one head's K/V, 32 rows of the additive mask
    (dict(B=1, H=1, Lq=1, Lk=(1 << 24), D=128), "MHA_E_OVERFLOW"),
    (dict(B=1, H=1, Lq=1, Lk=(1 << 26), D=16, kind=_abi.ADDITIVE, mask=A, dtype=1),
     "MHA_E_OVERFLOW"),
    # empty calls succeed without touching a device
    (dict(B=0), "MHA_OK"),
    (dict(H=0, q=None, k=None, v=None, out=None), "MHA_OK"),
    (dict(Lq=0), "MHA_OK"),
])
def test_fwd_validation(kw, status):
    assert _fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(eps=float("nan")), "MHA_E_ARG"),
    (dict(eps=-1e-5), "MHA_E_ARG"),
    (dict(gamma=None), "MHA_E_NULL"),
    (dict(beta=None), "MHA_E_NULL"),
    (dict(x=None), "MHA_E_NULL"),
    (dict(residual=A + 8), "MHA_E_ALIGN"),
    (dict(H=1025, D=64), "MHA_E_SHAPE"),
    (dict(Lq=0), "MHA_OK"),
])
def test_prenorm_validation(kw, status):
    assert _pre(**kw) == status


def test_valid_call_without_gpu_reports_no_device():
    """A call that passes validation goes on to the device; here there is none.
    The arguments are fake addresses, so the call must never reach a GPU: the
    test is skipped where one is visible, and the child process hides them all."""
    import subprocess
    import sys
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: fake pointers must not reach it")
    code = ("import ctypes; from masked_head_attention_amd import _abi; "
            f"print(_abi.STATUS[_abi.lib().mha_fwd({A},{A},{A},None,1,1,1,4,4,64,0.125,1,None,{A})])")
    env = {**os.environ, "HIP_VISIBLE_DEVICES": "", "ROCR_VISIBLE_DEVICES": "",
           "CUDA_VISIBLE_DEVICES": ""}
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       env=env, timeout=120)
    out = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    assert out == "MHA_E_NO_DEVICE", (out, r.stderr)


def test_tile_config_and_status_strings():
    lib = _abi.lib()
    r, k = ctypes.c_int(), ctypes.c_int()
    # float32: 16 rows x 16 keys (one 16x16x4 MFMA tile); 16-bit: 32 rows x 64 keys
    for dt, shape in ((0, (16, 16)), (1, (32, 64)), (2, (32, 64))):
        for D in (16, 32, 64, 128):
            assert lib.mha_tile_config(dt, D, 0, ctypes.byref(r), ctypes.byref(k)) == 0
            assert (r.value, k.value) == shape
    assert lib.mha_tile_config(1, 40, 0, ctypes.byref(r), ctypes.byref(k)) == 5
    assert lib.mha_tile_config(7, 64, 0, ctypes.byref(r), ctypes.byref(k)) == 3
    assert lib.mha_tile_config(1, 64, 32, ctypes.byref(r), ctypes.byref(k)) == 4  # E_MASK
    for code, name in _abi.STATUS.items():
        assert lib.mha_status_str(code).decode().startswith(name)
    assert lib.mha_set_debug_counters(None) == 0
    assert lib.mha_set_debug_counters(A + 4) == _abi.STATUS_CODE["MHA_E_ALIGN"]


def _softmax(s=A, p=A, rows=4, cols=64, scale=1.0, dtype=1):
    return _abi.STATUS[_abi.lib().mha_softmax_rows(s, p, rows, cols, scale, dtype, None)]


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), "MHA_E_DTYPE"),
    (dict(rows=-1), "MHA_E_SHAPE"),
    (dict(cols=-2), "MHA_E_SHAPE"),
    (dict(scale=float("nan")), "MHA_E_ARG"),
    (dict(scale=-1.0), "MHA_E_ARG"),
    (dict(s=None), "MHA_E_NULL"),
    (dict(p=None), "MHA_E_NULL"),
    (dict(s=A + 1), "MHA_E_ALIGN"),
    (dict(p=A + 2, dtype=0), "MHA_E_ALIGN"),
    (dict(rows=1 << 40, cols=1 << 30), "MHA_E_OVERFLOW"),
    (dict(rows=1 << 36, cols=1), "MHA_E_OVERFLOW"),
    # empty calls succeed without touching a device
    (dict(rows=0, s=None, p=None), "MHA_OK"),
    (dict(cols=0), "MHA_OK"),
])
def test_softmax_validation(kw, status):
    assert _softmax(**kw) == status


def _dec(q=A, k=A, v=A, lens=None, B=2, H=4, Lk=4096, D=128, scale=0.125, dtype=1, ws=A,
         ws_bytes=1 << 30, out=A, lse=None):
    return _abi.STATUS[_abi.lib().mha_decode_fwd(q, k, v, lens, B, H, Lk, D, scale, dtype, ws,
                                                 ws_bytes, None, out, lse)]


def _ws(B, H, Lk, D, dtype=1):
    n = ctypes.c_size_t(0)
    st = _abi.STATUS[_abi.lib().mha_decode_workspace_size(B, H, Lk, D, dtype, ctypes.byref(n))]
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), "MHA_E_DTYPE"),
    (dict(B=-1), "MHA_E_SHAPE"),
    (dict(Lk=-1), "MHA_E_SHAPE"),
    (dict(D=96), "MHA_E_UNSUPPORTED"),
    (dict(scale=float("nan")), "MHA_E_ARG"),
    (dict(scale=-1.0), "MHA_E_ARG"),
    (dict(q=None), "MHA_E_NULL"),
    (dict(out=None), "MHA_E_NULL"),
    (dict(v=None), "MHA_E_NULL"),
    (dict(k=A + 8), "MHA_E_ALIGN"),
    (dict(lens=A + 2), "MHA_E_ALIGN"),
    (dict(lse=A + 1), "MHA_E_ALIGN"),
    (dict(ws=None), "MHA_E_WORKSPACE"),
    (dict(ws=A + 4), "MHA_E_WORKSPACE"),
    (dict(ws_bytes=16), "MHA_E_WORKSPACE"),
    (dict(B=1, H=1, Lk=1 << 24, D=128), "MHA_E_OVERFLOW"),
    # empty calls succeed without touching a device
    (dict(B=0), "MHA_OK"),
    (dict(H=0, q=None, out=None), "MHA_OK"),
])
def test_decode_validation(kw, status):
    assert _dec(**kw) == status


def _dec_noalloc(q=A, k=A, v=A, lens=None, B=2, H=4, Lk=4096, D=128, scale=0.125, dtype=1,
                 out=A, lse=None):
    return _abi.STATUS[_abi.lib().mha_decode_fwd_noalloc(q, k, v, lens, B, H, Lk, D, scale,
                                                         dtype, None, out, lse)]


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), "MHA_E_DTYPE"),
    (dict(B=-1), "MHA_E_SHAPE"),
    (dict(D=96), "MHA_E_UNSUPPORTED"),
    (dict(scale=float("nan")), "MHA_E_ARG"),
    (dict(q=None), "MHA_E_NULL"),
    (dict(out=None), "MHA_E_NULL"),
    (dict(k=A + 8), "MHA_E_ALIGN"),
    (dict(lens=A + 2), "MHA_E_ALIGN"),
    (dict(B=1, H=1, Lk=1 << 24, D=128), "MHA_E_OVERFLOW"),
    # more partial results than the static scratch holds: refused before any HIP call
    (dict(B=64, H=64, Lk=8192, D=128), "MHA_E_SCRATCH"),
    (dict(B=0), "MHA_OK"),
])
def test_decode_noalloc_validation(kw, status):
    assert _dec_noalloc(**kw) == status


def test_noalloc_scratch_limit():
    n = ctypes.c_size_t(0)
    assert _abi.lib().mha_noalloc_scratch_bytes(ctypes.byref(n)) == 0
    assert n.value == 16 << 20
    assert _abi.lib().mha_noalloc_scratch_bytes(None) == _abi.STATUS_CODE["MHA_E_NULL"]
    # the largest call that fits uses at most that many bytes of partial results
    st, need = _ws(64, 64, 8192, 128)
    assert st == "MHA_OK" and need > n.value
    st, need = _ws(16, 32, 4096, 128)
    assert st == "MHA_OK" and 0 < need <= n.value


def test_decode_workspace_size():
    # one split per head when the cache is short: no workspace
    assert _ws(2, 4, 37, 128) == ("MHA_OK", 0)
    assert _ws(0, 4, 4096, 128) == ("MHA_OK", 0)
    # split keys: B*H*nsplit partial rows of D floats plus (m, l)
    st, n = _ws(16, 32, 4096, 128)
    assert st == "MHA_OK" and n > 0 and n % (16 * 32 * 130 * 4) == 0
    nsplit = n // (16 * 32 * 130 * 4)
    assert nsplit > 1 and 4096 % nsplit == 0
    # fewer heads: more splits per head to fill the GPU, never below 64-key chunks
    st, n1 = _ws(1, 2, 4096, 128)
    assert st == "MHA_OK" and n1 // (2 * 130 * 4) == 4096 // 64
    assert _ws(1, 1, 10, 48)[0] == "MHA_E_UNSUPPORTED"
    assert _ws(1, 1, 10, 64, dtype=9)[0] == "MHA_E_DTYPE"
    assert _ws(1, -1, 10, 64)[0] == "MHA_E_SHAPE"


def _bwd(q=A, k=A, v=A, dout=A, mask=None, kind=0, B=1, H=2, Lq=8, Lk=8, D=64, scale=0.125,
         dtype=1, ws=A, ws_bytes=1 << 20, dq=A, dk=A, dv=A):
    return _abi.STATUS[_abi.lib().mha_bwd(q, k, v, dout, mask, kind, B, H, Lq, Lk, D, scale,
                                          dtype, ws, ws_bytes, None, dq, dk, dv)]


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), "MHA_E_DTYPE"),
    (dict(dtype=0, D=48), "MHA_E_UNSUPPORTED"),
    (dict(D=48), "MHA_E_UNSUPPORTED"),
    (dict(kind=_abi.ADDITIVE | _abi.PADDING, mask=A), "MHA_E_MASK"),
    (dict(kind=_abi.PER_HEAD), "MHA_E_MASK"),
    (dict(kind=_abi.KEEP, mask=A + 4), "MHA_E_ALIGN"),
    (dict(kind=64), "MHA_E_MASK"),
    (dict(kind=0, mask=A), "MHA_E_MASK"),
    (dict(kind=_abi.PADDING), "MHA_E_NULL"),
    (dict(kind=_abi.PADDING, mask=A + 2), "MHA_E_ALIGN"),
    (dict(B=-1), "MHA_E_SHAPE"),
    (dict(scale=float("inf")), "MHA_E_ARG"),
    (dict(dout=None), "MHA_E_NULL"),
    (dict(dk=None), "MHA_E_NULL"),
    (dict(dout=A + 8), "MHA_E_ALIGN"),
    (dict(ws=None), "MHA_E_WORKSPACE"),
    (dict(ws_bytes=8), "MHA_E_WORKSPACE"),
    (dict(Lk=1 << 24, D=128), "MHA_E_OVERFLOW"),
    (dict(B=0), "MHA_OK"),
    (dict(Lq=0, Lk=0), "MHA_OK"),
    (dict(Lk=0, k=None, v=None, dk=None, dv=None, ws=None, ws_bytes=0), "MHA_E_WORKSPACE"),
])
def test_bwd_validation(kw, status):
    assert _bwd(**kw) == status


def test_bwd_workspace_size():
    n = ctypes.c_size_t(0)
    assert _abi.lib().mha_bwd_workspace_size(2, 3, 100, 1, ctypes.byref(n)) == 0
    assert n.value == 2 * 3 * 100 * 8
    assert _abi.STATUS[_abi.lib().mha_bwd_workspace_size(2, -3, 100, 1, ctypes.byref(n))] == \
        "MHA_E_SHAPE"


def _pre_ws(workspace=A, workspace_bytes=1 << 40, x=A, k=A, v=A, mask=None, kind=0, gamma=A,
            beta=A, eps=1e-5, residual=None, B=1, H=2, Lq=4, Lk=4, D=64, scale=0.125, dtype=2,
            out=A):
    return _abi.STATUS[_abi.lib().mha_prenorm_cross_fwd_ws(
        x, k, v, mask, kind, gamma, beta, eps, residual, B, H, Lq, Lk, D, scale, dtype,
        workspace, workspace_bytes, None, out)]


def _pre_ws_size(B, H, Lq, Lk, D, dtype=2):
    n = ctypes.c_size_t(0)
    st = _abi.lib().mha_prenorm_cross_workspace_size(B, H, Lq, Lk, D, dtype, ctypes.byref(n))
    return _abi.STATUS[st], n.value


def test_prenorm_workspace_size():
    """bfloat16: two float16 copies of [B,H,Lk,D], B*H*4 int32 flags and B*Lq
    float32 pairs, each part rounded up to 256 bytes; every other dtype, or no
    queries or keys, needs none."""
    kv = (2 * 16 * 2048 * 64 * 2 + 255) // 256 * 256
    assert _pre_ws_size(2, 16, 2048, 2048, 64) == (
        "MHA_OK", 2 * kv + (2 * 16 * 16 + 255) // 256 * 256 + 2 * 2048 * 8)
    assert _pre_ws_size(1, 1, 5, 3, 16) == ("MHA_OK", 2 * 256 + 256 + 256)
    assert _pre_ws_size(2, 16, 2048, 2048, 64, dtype=1) == ("MHA_OK", 0)
    assert _pre_ws_size(2, 16, 2048, 2048, 64, dtype=0) == ("MHA_OK", 0)
    assert _pre_ws_size(2, 16, 2048, 0, 64) == ("MHA_OK", 0)
    assert _pre_ws_size(2, 16, 0, 2048, 64) == ("MHA_OK", 0)
    assert _pre_ws_size(0, 16, 2048, 2048, 64) == ("MHA_OK", 0)
    assert _pre_ws_size(1, 1, 10, 10, 48)[0] == "MHA_E_UNSUPPORTED"
    assert _pre_ws_size(1, 1, 10, 10, 64, dtype=9)[0] == "MHA_E_DTYPE"
    assert _pre_ws_size(1, -1, 10, 10, 64)[0] == "MHA_E_SHAPE"
    assert _pre_ws_size(1, 1, -10, 10, 64)[0] == "MHA_E_SHAPE"
    assert _pre_ws_size(1 << 30, 1 << 30, 4, 1 << 20, 64)[0] == "MHA_E_OVERFLOW"
    assert _abi.lib().mha_prenorm_cross_workspace_size(1, 1, 1, 1, 64, 2, None) == \
        _abi.STATUS_CODE["MHA_E_NULL"]


@pytest.mark.parametrize("kw,status", [
    # the checks of mha_prenorm_cross_fwd come first
    (dict(dtype=3), "MHA_E_DTYPE"),
    (dict(eps=-1e-5), "MHA_E_ARG"),
    (dict(gamma=None), "MHA_E_NULL"),
    # bfloat16 without a mask tensor needs the workspace
    (dict(workspace=None), "MHA_E_WORKSPACE"),
    (dict(workspace=A + 8), "MHA_E_WORKSPACE"),
    (dict(workspace_bytes=2559), "MHA_E_WORKSPACE"),
    # empty calls succeed without touching a device or the workspace
    (dict(Lq=0, workspace=None), "MHA_OK"),
    (dict(B=0, workspace=None), "MHA_OK"),
])
def test_prenorm_ws_validation(kw, status):
    assert _pre_ws_size(1, 2, 4, 4, 64)[1] == 2560  # the size the short-workspace case misses by one
    assert _pre_ws(**kw) == status

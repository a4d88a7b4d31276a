"""The C-ABI library without a GPU: it loads, exports every symbol include/fa.h declares, and
rejects invalid arguments with the documented status before making any HIP call."""

import ctypes
import math
import os
import re

import pytest
import torch

from io_aware_attention_02_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
OK, INVALID, UNSUPPORTED, HIPERR, TOO_LARGE = 0, 1, 2, 3, 4
P = 0x100000  # a 16-byte-aligned stand-in for a device pointer; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.library_path()):
        pytest.skip("libfa.so not built")
    return _binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == ["fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_fp8",
                                     "fa_fwd_unfused",
                                     "fa_fwd_unfused_workspace_bytes", "fa_paged_decode",
                                     "fa_paged_decode_noalloc",
                                     "fa_paged_decode_workspace_bytes", "fa_paged_prefill",
                                     "fa_paged_prefill_workspace_bytes", "fa_status_str"]


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert _binding.fa_status_str(OK) == "ok"
    assert _binding.fa_status_str(INVALID) == "invalid argument"
    assert _binding.fa_status_str(UNSUPPORTED) == "unsupported configuration"
    assert _binding.fa_status_str(HIPERR) == "HIP runtime error"
    assert "static scratch" in _binding.fa_status_str(TOO_LARGE)
    assert _binding.fa_status_str(99) == "unknown status"


def test_workspace_bytes(lib):
    # 64 sequences x 32 heads x ceil(2048*16/512)=64 ranges x (128 + 2) floats
    # 32768 tokens = 64 ranges of 512, raised to 71 (7 mod 8) so ranges spread over the 8 XCDs
    assert lib.fa_paged_decode_workspace_bytes(64, 32, 128, 2048, 16) == 64 * 32 * 71 * 130 * 4
    assert lib.fa_paged_decode_workspace_bytes(2, 1, 128, 224, 16) == 2 * 7 * 130 * 4   # 7 ranges
    assert lib.fa_paged_decode_workspace_bytes(2, 1, 128, 256, 16) == 2 * 15 * 130 * 4  # 8 -> 15
    assert lib.fa_paged_decode_workspace_bytes(1, 1, 64, 1, 16) == 66 * 4
    assert lib.fa_paged_decode_workspace_bytes(0, 32, 128, 2048, 16) == 0
    assert lib.fa_paged_decode_workspace_bytes(4, 32, 128, -1, 16) == 0
    # Chunked prefill: at most 2048 split partials of 128 rows (1024 of 256 rows when max_q >=
    # 256) x (d + 2) floats, plus the plan (a few ints per sequence and 8 per work item),
    # whatever the lengths.
    for d in (64, 128):
        partials = 2048 * 128 * (d + 2) * 4
        small = lib.fa_paged_prefill_workspace_bytes(1, 16, 8, 8, d, 1)
        big = lib.fa_paged_prefill_workspace_bytes(64, 1024, 32, 8, d, 2048)
        assert partials < small < partials + (1 << 20)
        assert small < big < partials + (1 << 24)
        assert small % 256 == 0 and big % 256 == 0
    assert lib.fa_paged_prefill_workspace_bytes(0, 16, 8, 8, 128, 1) == 0
    assert lib.fa_paged_prefill_workspace_bytes(1, 16, 8, 3, 128, 1) == 0


def _fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=8, Hkv=2, N=128, d=128, scale=0.1, causal=0,
             seq_lens=None, dtype=0, stream=None)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"],
                      a["d"], a["scale"], a["causal"], a["seq_lens"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(Hkv=0), INVALID), (dict(N=0), INVALID),
    (dict(d=0), INVALID), (dict(H=8, Hkv=3), INVALID),
    (dict(q=P + 8), INVALID), (dict(o=P + 4), INVALID), (dict(lse=P + 2), INVALID),
    (dict(seq_lens=P + 1), INVALID),
    (dict(scale=-0.5), INVALID), (dict(scale=math.nan), INVALID), (dict(scale=math.inf), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(dtype=2), UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20), UNSUPPORTED),
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status


def _fp8(lib, **kw):
    a = dict(q=P, k=P, v=P, qs=0.01, ks=0.01, vs=0.01, o=P, lse=P, B=1, H=8, Hkv=2, N=128, d=128,
             scale=0.1, causal=0, seq_lens=None, stream=None)
    a.update(kw)
    return lib.fa_fwd_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["o"], a["lse"],
                          a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"],
                          a["seq_lens"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(Hkv=0), INVALID), (dict(N=0), INVALID),
    (dict(d=0), INVALID), (dict(H=8, Hkv=3), INVALID),
    (dict(k=P + 8), INVALID), (dict(o=P + 4), INVALID), (dict(lse=P + 2), INVALID),
    (dict(seq_lens=P + 1), INVALID),
    (dict(scale=-0.5), INVALID), (dict(qs=math.nan), INVALID), (dict(ks=-1.0), INVALID),
    (dict(vs=math.inf), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20), UNSUPPORTED),
])
def test_fp8_rejects(lib, kw, status):
    assert _fp8(lib, **kw) == status


def test_bwd_workspace_bytes(lib):
    # two fp32 per query row (D and the base-2 LSE), each array rounded up to 256 bytes
    assert lib.fa_bwd_workspace_bytes(1, 8, 16384) == 2 * 8 * 16384 * 4
    assert lib.fa_bwd_workspace_bytes(1, 1, 3) == 512
    assert lib.fa_bwd_workspace_bytes(0, 8, 16) == 0
    assert lib.fa_bwd_workspace_bytes(2, 8, -1) == 0


def _bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=8, Hkv=2, N=128, d=128,
             scale=0.1, causal=0, seq_lens=None, dtype=0, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                      a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"],
                      a["seq_lens"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(do=None), INVALID), (dict(dq=None), INVALID), (dict(dk=None), INVALID),
    (dict(dv=None), INVALID), (dict(ws=None), INVALID),
    (dict(B=0), INVALID), (dict(N=-3), INVALID), (dict(H=8, Hkv=3), INVALID),
    (dict(dq=P + 8), INVALID), (dict(do=P + 4), INVALID), (dict(lse=P + 2), INVALID),
    (dict(ws=P + 8), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=math.nan), INVALID),
    (dict(wsb=100), INVALID),
    (dict(dtype=1), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20, wsb=1 << 62), UNSUPPORTED),
])
def test_bwd_rejects(lib, kw, status):
    assert _bwd(lib, **kw) == status


def test_unfused_workspace_bytes(lib):
    # fp32 scores and bf16 probabilities: 6 bytes per (batch, head, query, key)
    assert lib.fa_fwd_unfused_workspace_bytes(1, 8, 16384) == 6 * 8 * 16384 * 16384
    assert lib.fa_fwd_unfused_workspace_bytes(0, 8, 16) == 0


def _unf(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=8, Hkv=2, N=128, d=128, scale=0.1, causal=0, ws=P,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.fa_fwd_unfused(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                              a["N"], a["d"], a["scale"], a["causal"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(ws=None), INVALID),
    (dict(B=0), INVALID), (dict(H=8, Hkv=3), INVALID), (dict(o=P + 4), INVALID),
    (dict(scale=-2.0), INVALID), (dict(wsb=1000), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(N=100), UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20, wsb=1 << 62), UNSUPPORTED),
])
def test_unfused_rejects(lib, kw, status):
    assert _unf(lib, **kw) == status


def _pre(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, sl=P, ql=P, o=P, lse=P, S=4, Q=64, Hq=32, Hkv=8, d=128, bs=16,
             M=64, nb=256, scale=0.1, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.fa_paged_prefill(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["ql"], a["o"], a["lse"],
                                a["S"], a["Q"], a["Hq"], a["Hkv"], a["d"], a["bs"], a["M"], a["nb"],
                                a["scale"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(bt=None), INVALID),
    (dict(sl=None), INVALID), (dict(ql=None), INVALID), (dict(o=None), INVALID),
    (dict(lse=None), INVALID), (dict(S=0), INVALID), (dict(Q=0), INVALID), (dict(M=-1), INVALID),
    (dict(Hq=32, Hkv=5), INVALID), (dict(scale=math.inf), INVALID), (dict(q=P + 8), INVALID),
    (dict(ql=P + 2), INVALID), (dict(lse=P + 1), INVALID), (dict(ws=None), INVALID),
    (dict(ws=P + 8), INVALID), (dict(wsb=1 << 20), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(bs=8), UNSUPPORTED),
    (dict(S=1 << 20, Q=1 << 20, Hq=1 << 8, Hkv=1 << 8), UNSUPPORTED),
    (dict(M=1 << 28), UNSUPPORTED),
])
def test_paged_prefill_rejects(lib, kw, status):
    assert _pre(lib, **kw) == status


def _dec(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, sl=P, o=P, lse=P, S=4, Hq=32, Hkv=8, d=128, bs=16, M=64,
             nb=256, scale=0.1, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.fa_paged_decode(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"], a["S"],
                               a["Hq"], a["Hkv"], a["d"], a["bs"], a["M"], a["nb"], a["scale"],
                               a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vc=None), INVALID),
    (dict(bt=None), INVALID), (dict(sl=None), INVALID), (dict(o=None), INVALID),
    (dict(ws=None), INVALID), (dict(S=0), INVALID), (dict(Hq=0), INVALID), (dict(M=0), INVALID),
    (dict(nb=0), INVALID), (dict(Hq=32, Hkv=5), INVALID), (dict(scale=-1.0), INVALID),
    (dict(kc=P + 8), INVALID), (dict(ws=P + 4), INVALID), (dict(bt=P + 2), INVALID),
    (dict(lse=P + 1), INVALID), (dict(wsb=1000), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(bs=32), UNSUPPORTED), (dict(Hq=64, Hkv=2), UNSUPPORTED),
    (dict(S=1 << 20, M=1 << 14), UNSUPPORTED),
])
def test_decode_rejects(lib, kw, status):
    assert _dec(lib, **kw) == status


def _dec_noalloc(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, sl=P, o=P, lse=P, S=4, Hq=32, Hkv=8, d=128, bs=16, M=64,
             nb=256, scale=0.1, stream=None)
    a.update(kw)
    return lib.fa_paged_decode_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"],
                                       a["lse"], a["S"], a["Hq"], a["Hkv"], a["d"], a["bs"],
                                       a["M"], a["nb"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(bt=None), INVALID), (dict(o=None), INVALID),
    (dict(S=0), INVALID), (dict(nb=0), INVALID), (dict(Hq=32, Hkv=5), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(kc=P + 8), INVALID), (dict(sl=P + 2), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(bs=32), UNSUPPORTED), (dict(Hq=64, Hkv=2), UNSUPPORTED),
    (dict(S=1 << 20, M=1 << 14), UNSUPPORTED),
    # 64 sequences x 32 heads with a 65536-token table need 144 MB of partials: over 80 MiB
    (dict(S=64, Hq=32, M=4096), TOO_LARGE),
])
def test_decode_noalloc_rejects(lib, kw, status):
    assert _dec_noalloc(lib, **kw) == status


def test_decode_noalloc_limit_is_the_documented_scratch(lib):
    # The decode workload (64 sequences x 32 heads, 32768-token tables, d = 128) fits the scratch.
    assert lib.fa_paged_decode_workspace_bytes(64, 32, 128, 2048, 16) <= 80 << 20
    assert lib.fa_paged_decode_workspace_bytes(64, 32, 128, 4096, 16) > 80 << 20


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_call_without_a_device_reports_hip_error(lib):
    # Arguments pass validation, so the call reaches the runtime, which has no device.
    assert _fwd(lib) == HIPERR
    assert _dec(lib) == HIPERR
    assert _bwd(lib) == HIPERR
    assert _pre(lib) == HIPERR
    assert _unf(lib) == HIPERR
    assert _fp8(lib) == HIPERR
    assert _dec_noalloc(lib) == HIPERR


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "_LIB", None)
    monkeypatch.setattr(_binding, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _binding.load_library()

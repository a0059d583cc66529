"""Host-side checks of libfa.so that need no GPU: the library loads, exports
every entry point include/fa.h declares, and rejects invalid arguments on the
host before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("fa_fwd", "fa_bwd", "fa_fwd_varlen", "fa_bwd_varlen", "fa_fwd_kvcache",
              "fa_bwd_workspace_size", "fa_kvcache_workspace_size", "fa_status_string"):
        assert n in names


@pytest.fixture(scope="module")
def lib():
    import io_aware_exact_qk_amd as fa
    return fa.lib()


def test_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), f"libfa.so does not export {n}"


def test_status_strings(lib):
    assert lib.fa_status_string(0) == b"ok"
    assert lib.fa_status_string(1) == b"invalid argument"
    assert lib.fa_status_string(2) == b"unsupported configuration"
    assert lib.fa_status_string(99) == b"unknown status"


def test_workspace_sizes(lib):
    # two float32 row arrays (row term, LSE in log2 units), each padded to 256 bytes
    assert lib.fa_bwd_workspace_size(2, 512, 512, 16, 16, 128, 0) == 2 * (2 * 16 * 512 * 4)
    # varlen backward: two row arrays, then the 128-row query-tile list and the
    # 256-key tile list (8 bytes per entry, at most (total + nseq (tile - 1)) / tile entries)
    rows = 2 * 12032  # 1000 * 3 * 4 = 12000 rounded up to 256
    q_list = -(-((1000 + 5 * 127) // 128) * 8 // 256) * 256
    k_list = -(-((900 + 5 * 255) // 256) * 8 // 256) * 256
    assert lib.fa_bwd_varlen_workspace_size(5, 1000, 900, 3, 128, 0) == rows + q_list + k_list
    assert lib.fa_fwd_varlen_workspace_size(5, 1000, 3, 128) == q_list
    assert lib.fa_fwd_varlen_workspace_size(5, 0, 3, 128) == 0
    assert lib.fa_kvcache_workspace_size(8, 1, 32, 128, 1) == 0
    assert lib.fa_kvcache_workspace_size(8, 1, 32, 128, 16) == 8 * 32 * 16 * 128 * 4 + 8 * 32 * 16 * 4
    # num_splits = 0 (automatic) is sized for the largest automatic choice, 32
    assert lib.fa_kvcache_workspace_size(8, 1, 32, 128, 0) == 8 * 32 * 32 * 128 * 4 + 8 * 32 * 32 * 4


# Fake, 16-byte aligned "device" addresses: the calls below must fail in
# host-side validation, before any HIP call could touch them.
A = 1 << 20
F = ctypes.c_void_p(A)


def _fwd(lib, **kw):
    a = dict(B=1, Sq=8, Sk=8, Hq=4, Hkv=2, D=128, dtype=1, scale=0.125, causal=0, wl=-1, wr=-1,
             softcap=0.0, alibi=None, q=F, out=F)
    a.update(kw)
    return lib.fa_fwd(a["q"], F, F, a["out"], F, a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"],
                      a["dtype"], a["scale"], a["causal"], a["wl"], a["wr"], a["softcap"], a["alibi"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), 1), (dict(Hkv=0), 1), (dict(dtype=2), 1), (dict(scale=0.0), 1),
    (dict(scale=float("inf")), 1), (dict(wl=-2), 1), (dict(softcap=-1.0), 1),
    (dict(softcap=float("nan")), 1), (dict(B=0), 1), (dict(Sq=0), 1),
    (dict(q=ctypes.c_void_p(A + 8)), 1), (dict(out=None), 1), (dict(D=80), 2), (dict(D=48), 2),
])
def test_fwd_rejects_invalid(lib, kw, status):
    assert _fwd(lib, **kw) == status


@pytest.mark.parametrize("p", [1.0, -0.01, float("nan"), 255.5 / 256])
def test_dropout_rejects_probability(lib, p):
    st = lib.fa_fwd_dropout(F, F, F, F, F, 1, 8, 8, 2, 2, 128, 1, ctypes.c_float(0.1), 0, -1, -1,
                            ctypes.c_float(0.0), None, ctypes.c_float(p), ctypes.c_ulonglong(1),
                            ctypes.c_ulonglong(0), None)
    assert st == 1


def test_bwd_rejects_small_workspace(lib):
    st = lib.fa_bwd(F, F, F, F, F, F, F, F, F, 1, 8, 8, 2, 2, 128, 1, 0.1, 0, -1, -1, 0.0, None, 0,
                    F, 16, None)
    assert st == 3
    st = lib.fa_bwd(F, F, F, F, F, F, F, F, F, 1, 8, 8, 2, 2, 128, 1, 0.1, 0, -1, -1, 0.0, None, 0,
                    None, 1 << 20, None)
    assert st == 3


def test_kvcache_rejects(lib):
    def call(**kw):
        a = dict(page=256, rd=0, cos=None, sin=None, Sq=1, splits=1, wl=-1, softcap=0.0, Hq=32, Hkv=8,
                 knew=F, vnew=F)
        a.update(kw)
        return lib.fa_fwd_kvcache(F, a["knew"], a["vnew"], F, F, F, F, 4, a["page"], a["cos"], a["sin"],
                                  a["rd"], F, F, 2, a["Sq"], a["Hq"], a["Hkv"], 128, 1, 0.088, 1, a["wl"],
                                  -1, a["softcap"], None, a["splits"], None, 0, None)
    assert call(page=48) == 1
    assert call(page=0) == 1
    assert call(cos=F, sin=None, rd=128) == 1
    assert call(cos=F, sin=F, rd=24) == 1
    assert call(cos=F, sin=F, rd=256) == 1
    assert call(knew=None) == 1
    assert call(splits=-1) == 1
    assert call(Sq=2, Hq=32, Hkv=1) == 2  # 32 query heads x 2 new tokens > 32 MFMA columns
    assert call(Hq=66, Hkv=1) == 2
    assert call(splits=4) == 3  # needs a workspace
    assert call(splits=0) == 3  # the automatic count here is 4: needs a workspace
    assert call(splits=4, wl=5, softcap=3.0) == 3


def test_varlen_rejects(lib):
    st = lib.fa_fwd_varlen(F, F, F, F, F, F, F, 0, 8, 8, 8, 8, 2, 2, 128, 1, 0.1, 0, -1, -1, 0.0, None, F,
                           1 << 20, None)
    assert st == 1  # nseq = 0
    st = lib.fa_fwd_varlen(F, F, F, F, F, None, F, 1, 8, 8, 8, 8, 2, 2, 128, 1, 0.1, 0, -1, -1, 0.0, None, F,
                           1 << 20, None)
    assert st == 1  # cu_seqlens_q missing
    st = lib.fa_fwd_varlen(F, F, F, F, F, F, F, 1, 8, 8, 8, 8, 2, 2, 128, 1, 0.1, 0, -1, -1, 0.0, None, None,
                           0, None)
    assert st == 3  # the tile list needs a workspace


def test_noalloc_rejects_requests_beyond_its_scratch(lib):
    """fa_fwd_kvcache_noalloc refuses, on the host, partials larger than its
    static scratch (B * Sq_new * Hq * splits * (D + 1) * 4 bytes > 8 MiB)."""
    assert lib.fa_kvcache_noalloc_max_bytes() == 8 << 20
    assert lib.fa_status_string(5).startswith(b"request exceeds the static scratch")
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: the call is refused first
    B, Sq, Hq, Hkv, D, splits = 64, 1, 64, 8, 128, 32
    assert lib.fa_kvcache_workspace_size(B, Sq, Hq, D, splits) > (8 << 20)
    st = lib.fa_fwd_kvcache_noalloc(p, None, None, p, p, p, p, 300, 256, None, None, 0, p, p,
                                    B, Sq, Hq, Hkv, D, 1, 0.088, 1, -1, -1, 0.0, None, splits, None)
    assert st == 5

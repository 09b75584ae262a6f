"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and rejects
bad arguments with the documented status before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

from causal_flashattention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "cfa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    names = declared_functions()
    assert "attn_fwd" in names and "attn_bwd" in names and "mx_quantize" in names
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings():
    L = _lib.lib()
    assert L.cfa_status_string(0) == b"CFA_OK"
    assert L.cfa_status_string(5) == b"CFA_ERR_WORKSPACE"
    assert L.cfa_version() >> 16 == 1


def test_workspace_sizes():
    L = _lib.lib()
    assert L.cfa_workspace_bytes(0, 8192, 9, 16, 16, 128, 1) > 0
    assert L.cfa_workspace_bytes(1, 8192, 9, 16, 16, 128, 1) >= 16 * 8192 * 4
    assert L.cfa_workspace_bytes(0, 8192, 9, 16, 5, 128, 1) == 0       # hq % hkv
    assert L.cfa_workspace_bytes(0, 8192, 9, 16, 16, 96, 1) == 0       # head dim
    assert L.cfa_workspace_bytes(1, 256, 1, 1, 1, 64, 0) == 0          # fp32 is forward-only
    assert L.cfa_workspace_bytes(2, 256, 1, 1, 1, 64, 1) == 0          # no such pass
    assert L.mx_padded_tokens(100, 3) == 128 + 96
    sb = ctypes.c_size_t(0)
    assert L.mx_quantize_bytes(0, 100, 3, 2, 128, ctypes.byref(sb)) == 100 * 2 * 128 and sb.value == 100 * 2 * 4
    for axis in (1, 2):
        assert L.mx_quantize_bytes(axis, 100, 3, 2, 128, ctypes.byref(sb)) == 2 * 128 * (128 + 96)
        assert sb.value == 2 * 128 * (128 + 96) // 32
    assert L.mx_quantize_bytes(3, 100, 3, 2, 128, ctypes.byref(sb)) == 0 and sb.value == 0
    assert L.mx_quantize_bytes(0, 100, 3, 2, 96, None) == 0


def _fwd(**over):
    L = _lib.lib()
    cu_h = np.array([0, 40, 100], dtype=np.int32)
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, cu_h=cu_h.ctypes.data, n_docs=2, T=100, maxs=0,
             hq=4, hkv=2, d=128, scale=0.088, causal=1, dtype=1, saved=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return L.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["cu_h"], a["n_docs"], a["T"], a["maxs"],
                      a["hq"], a["hkv"], a["d"], a["scale"], a["causal"], a["dtype"], a["saved"], a["ws"], a["wsb"],
                      a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(ws=None), 1),
    (dict(hkv=3), 2), (dict(n_docs=0), 2), (dict(T=-1), 2), (dict(scale=float("nan")), 2), (dict(scale=0.0), 2),
    (dict(d=96), 3), (dict(dtype=7), 3), (dict(dtype=2, d=64), 3), (dict(dtype=0, d=256), 3),
    (dict(dtype=2, d=256), 3), (dict(dtype=3, d=64), 3), (dict(dtype=4, d=64), 3), (dict(dtype=5, d=64), 3),
    (dict(dtype=6), 3),
    (dict(q=FAKE + 8), 4), (dict(ws=FAKE + 16), 4),
    (dict(wsb=16), 5),
])
def test_fwd_rejects(over, status):
    assert _fwd(**over) == status
    assert _lib.lib().cfa_last_error()


def test_fwd_rejects_bad_host_cu():
    for bad in ([1, 40, 100], [0, 50, 40], [0, 40, 99]):
        arr = np.array(bad, dtype=np.int32)
        assert _fwd(cu_h=arr.ctypes.data) == 2
    arr = np.array([0, 40, 100], dtype=np.int32)
    assert _fwd(cu_h=arr.ctypes.data, maxs=50) == 2     # a document longer than max_seqlen


def test_bwd_rejects():
    L = _lib.lib()
    cu_h = np.array([0, 100], dtype=np.int32)
    args = [FAKE] * 6 + [None] + [FAKE] * 4 + [FAKE, cu_h.ctypes.data, 1, 100, 0, 4, 2, 128, 0.088, 1, 1, FAKE,
                                                1 << 30, None]   # dlse (index 6) may be NULL
    bad = list(args); bad[7] = None                      # saved may be NULL for bf16: not an error by itself
    bad[8] = None                                        # dq NULL
    assert L.attn_bwd(*bad) == 1
    bad = list(args); bad[21] = 0                        # dtype fp32 is forward-only
    assert L.attn_bwd(*bad) == 3
    bad = list(args); bad[23] = 8                        # workspace too small
    assert L.attn_bwd(*bad) == 5
    bad = list(args); bad[6] = FAKE + 4                  # a misaligned dlse
    assert L.attn_bwd(*bad) == 4
    # MX without saved: the workspace must also hold the re-quantised Q_d, K_d, V_d
    ws1 = L.cfa_workspace_bytes(1, 100, 1, 4, 2, 128, 2)
    sv = L.cfa_saved_bytes(100, 1, 4, 2, 128, 2)
    assert sv > 0
    bad = list(args); bad[7] = None; bad[21] = 2; bad[23] = ws1
    assert L.attn_bwd(*bad) == 5
    assert b"cfa_saved_bytes" in L.cfa_last_error()
    bad = list(args); bad[7] = FAKE + 16; bad[21] = 2   # a given saved must be 256-byte aligned
    assert L.attn_bwd(*bad) == 4


def test_mx_quantize_rejects():
    L = _lib.lib()
    assert L.mx_quantize(FAKE, 100, 2, 128, FAKE, None, 1, 3, FAKE, FAKE, 0, None, 0, None) == 2   # axis
    assert L.mx_quantize(FAKE, 100, 2, 128, FAKE, None, 1, 2, FAKE, FAKE, 160, None, 0, None) == 1   # workspace
    assert L.mx_quantize(FAKE, 100, 2, 96, FAKE, None, 1, 0, FAKE, FAKE, 0, None, 0, None) == 3    # d
    assert L.mx_quantize(FAKE, 100, 2, 128, FAKE, None, 1, 1, FAKE, FAKE, 100, FAKE, 1 << 20, None) == 2  # t_pad
    assert L.mx_quantize(FAKE, 100, 2, 128, FAKE, None, 1, 1, FAKE, FAKE, 160, None, 0, None) == 1   # workspace


def test_kernel_events_hook_validates():
    L = _lib.lib()
    assert L.cfa_set_kernel_events(None, 2) == 1
    assert L.cfa_set_kernel_events(None, 0) == 0


def test_decode_rejects():
    L = _lib.lib()
    cu_h = np.array([0, 40, 100], dtype=np.int32)

    def call(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, o=FAKE, lse=FAKE, cu=FAKE, cu_h=cu_h.ctypes.data, B=2,
                 Tk=100, hq=8, hkv=2, d=128, scale=0.088, kv=2, ws=FAKE, wsb=1 << 30)
        a.update(over)
        return L.attn_decode(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], a["lse"], a["cu"], a["cu_h"], a["B"],
                             a["Tk"], a["hq"], a["hkv"], a["d"], a["scale"], a["kv"], a["ws"], a["wsb"], None)
    assert call(q=None) == 1
    assert call(ks=None) == 1                            # an MXFP8 cache needs its scales
    assert call(hkv=3) == 2 and call(B=0) == 2 and call(scale=-1.0) == 2
    assert call(cu_h=np.array([0, 50, 99], dtype=np.int32).ctypes.data) == 2
    assert call(d=256) == 3 and call(kv=0) == 3
    assert call(o=FAKE + 4) == 4
    assert call(wsb=64) == 5
    assert L.cfa_decode_workspace_bytes(2, 100, 8, 2, 128, 2) > 0
    assert L.cfa_decode_workspace_bytes(2, 100, 8, 2, 96, 2) == 0


def test_narrow_mx_sizes_and_quantiser_rejects():
    L = _lib.lib()
    # saved buffer: Q_d and K_d copies; E2M1 rows d/2 bytes, both 6-bit types 3d/4, E4M3 d
    sb = {dt: L.cfa_saved_bytes(4096, 3, 8, 2, 128, dt) for dt in (2, 3, 4, 5)}
    assert sb[4] == sb[5] and sb[3] < sb[4] < sb[2]
    assert L.cfa_saved_bytes(4096, 3, 8, 2, 128, 1) == 0          # bf16 saves nothing
    assert L.cfa_saved_bytes(4096, 3, 8, 2, 64, 5) == 0           # the MX paths take d = 128 only
    for fn in (L.mx_quantize_fp4, L.mx_quantize_fp6, L.mx_quantize_fp6_e3m2):
        assert fn(FAKE, 100, 2, 96, FAKE, FAKE, None) == 3        # head dim
        assert fn(FAKE, -1, 2, 128, FAKE, FAKE, None) == 2        # negative token count
        assert fn(None, 100, 2, 128, FAKE, FAKE, None) == 1       # NULL input
        assert fn(FAKE + 8, 100, 2, 128, FAKE, FAKE, None) == 4   # misaligned input
        assert fn(FAKE, 0, 2, 128, FAKE, FAKE, None) == 0         # nothing to do: no launch
        assert L.cfa_last_error() is not None



def test_mx_paths_reject_token_counts_past_32_bit_column_offsets():
    """Token-blocked MX rows are addressed as channel·t_pad + column in 32 bits: d·t_pad must
    stay below 2^31 (t_pad = 32·ceil(T/32) + 32·n_docs), checked before any launch."""
    L = _lib.lib()
    big = (1 << 31) // 128                              # t_pad·128 = 2^31 exactly at one document
    for dt in (2, 3, 4, 5):
        assert _fwd(dtype=dt, T=big - 32, n_docs=1, cu_h=None, hq=1, hkv=1, saved=FAKE) == 3
        assert b"2^31" in L.cfa_last_error()
        assert L.cfa_workspace_bytes(0, big - 32, 1, 1, 1, 128, dt) == 0
        assert L.cfa_workspace_bytes(0, big - 64, 1, 1, 1, 128, dt) > 0   # t_pad·d = 2^31 − 4096
    assert L.cfa_workspace_bytes(0, big - 32, 1, 1, 1, 128, 1) > 0       # bf16 has no such rows


def test_noalloc_backward_rejects_sizes_beyond_its_array():
    """attn_bwd_noalloc checks the workspace its sizes need against its fixed 64 MiB array before
    any HIP call: 2^20 tokens × 32 heads of D alone is 128 MiB."""
    L = _lib.lib()
    args = [FAKE] * 6 + [None, None] + [FAKE] * 3 + [FAKE, None, 1, 1 << 20, 0, 32, 8, 128, 0.088, 1, 1, None]
    assert L.attn_bwd_noalloc(*args) == 5
    assert b"64" in L.cfa_last_error() or b"67108864" in L.cfa_last_error()
    bad = list(args); bad[21] = 0                        # fp32 is forward-only, checked first
    assert L.attn_bwd_noalloc(*bad) == 3


def test_mx_head_limits_of_the_operand_passes():
    """The operand passes address a block's rows as a 32-bit offset r·h·d (r < 32): the MX paths
    take hq <= 65536, and mx_quantize axes 1, 2 take h <= 65536, rejected before any launch."""
    L = _lib.lib()
    assert _fwd(dtype=2, T=64, n_docs=1, cu_h=None, hq=65536 * 2, hkv=1, saved=FAKE) == 3
    assert b"65536" in L.cfa_last_error()
    assert L.cfa_workspace_bytes(0, 64, 1, 65536 * 2, 1, 128, 2) == 0
    assert L.cfa_workspace_bytes(0, 64, 1, 65536, 1, 128, 2) > 0
    assert L.mx_quantize(FAKE, 64, 65537, 128, FAKE, None, 1, 1, FAKE, FAKE, 96, FAKE, 1 << 20, None) == 3
    assert b"65536" in L.cfa_last_error()


def test_head_limit_of_the_tile_copies():
    """Every attention path stages a tile's rows at 32-bit offsets row·hq·d·2 bytes: hq above 65536
    is rejected before any launch (bf16 forward and backward, cross-attention), 65536 is taken."""
    L = _lib.lib()
    assert _fwd(dtype=1, T=64, n_docs=1, cu_h=None, hq=65537, hkv=1) == 3
    assert b"65536" in L.cfa_last_error()
    assert L.cfa_workspace_bytes(1, 64, 1, 65537, 1, 128, 1) == 0
    assert L.cfa_workspace_bytes(1, 64, 1, 65536, 1, 128, 1) > 0
    assert L.cfa_cross_workspace_bytes(1, 64, 64, 1, 65537, 1, 128) == 0

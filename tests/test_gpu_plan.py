"""The work-list builder on the GPU: device-side validation of cu_seqlens and the schedule switch.

A device-only cu_seqlens (no host copy) is checked by the plan kernel: a malformed one raises a
flag bit, read back with cfa_device_error, and every document becomes empty, so no kernel writes
an output row. The schedule (longest first, or index order under CFA_SCHED=naive) decides only
which workgroup computes a tile, so results are bit-identical under either.
"""
import os

import numpy as np
import pytest
import torch

import causal_flashattention_amd as cfa
from causal_flashattention_amd import workloads as W

from gpu_helpers import DEV, announce, to_dev

SENT = 7.0                       # finite sentinel: an untouched output keeps it


def _inputs(T, hq, hkv, seed):
    w = W.make_random(seed=seed, lengths=[T], hq=hq, hkv=hkv)
    return to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.do), w.scale


@pytest.mark.gpu
@pytest.mark.parametrize("mx", [False, "mxfp8"])
@pytest.mark.parametrize("bad,bit", [([0, 100, 50, 200], 2), ([0, 200, 0, 200], 2),
                                     ([1, 100, 150, 200], 1), ([0, 100, 150, 190], 4)])
def test_malformed_device_cu_seqlens_flags_and_writes_nothing(mx, bad, bit):
    announce("plan flag", mx, bad)
    T, hq, hkv = 200, 4, 1                    # bf16: the head-split reduce kernel runs too
    q, k, v, do, sc = _inputs(T, hq, hkv, 31)
    cu = torch.tensor(bad, dtype=torch.int32, device=DEV)
    n_docs = len(bad) - 1
    dt = cfa.CFA_MXFP8 if mx else cfa.CFA_BF16
    ws0 = torch.empty(cfa.workspace_bytes(0, T, n_docs, hq, hkv, 128, dt), dtype=torch.uint8, device=DEV)
    ws1 = torch.empty(cfa.workspace_bytes(1, T, n_docs, hq, hkv, 128, dt), dtype=torch.uint8, device=DEV)
    o = torch.full_like(q, SENT)
    lse = torch.full((hq, T), SENT, dtype=torch.float32, device=DEV)
    _, _, saved = cfa.attn_fwd(q, k, v, cu, scale=sc, mx=mx, out=o, lse=lse, workspace=ws0)
    f0 = cfa.device_error(ws0)
    assert f0 & bit, f0
    assert bool(torch.all(o == SENT)) and bool(torch.all(lse == SENT))
    dq, dk, dv = torch.full_like(q, SENT), torch.full_like(k, SENT), torch.full_like(v, SENT)
    # o is the sentinel: finite, so D = rowsum(dO·O) is finite and nothing else reads it
    cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=sc, mx=mx, saved=saved, dq=dq, dk=dk, dv=dv, workspace=ws1)
    f1 = cfa.device_error(ws1)
    assert f1 == f0
    for t in (dq, dk, dv):
        assert bool(torch.all(t == SENT))


@pytest.mark.gpu
def test_well_formed_device_cu_seqlens_leaves_flag_clear():
    announce("plan flag clear")
    T, hq, hkv = 200, 4, 1
    q, k, v, do, sc = _inputs(T, hq, hkv, 32)
    cu = torch.tensor([0, 100, 100, 200], dtype=torch.int32, device=DEV)
    ws = torch.empty(cfa.workspace_bytes(1, T, 3, hq, hkv, 128, cfa.CFA_BF16), dtype=torch.uint8, device=DEV)
    o, lse, _ = cfa.attn_fwd(q, k, v, cu, scale=sc, workspace=ws)
    assert cfa.device_error(ws) == 0
    cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=sc, workspace=ws)
    assert cfa.device_error(ws) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("mx", [False, "mxfp8"])
def test_naive_schedule_gives_identical_results(mx):
    """Documents of mixed lengths (ties in the length buckets, empty and short documents):
    the index-order schedule gives bit-identical outputs to the longest-first one."""
    announce("naive schedule", mx)
    lengths = [300, 5, 0, 1000, 130, 300, 64, 0, 1, 700]
    w = W.make_random(seed=33, lengths=lengths, hq=4, hkv=2)
    q, k, v, do = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.do)
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(DEV)

    def run():
        o, lse, saved = cfa.attn_fwd(q, k, v, cu, scale=w.scale, mx=mx)
        g = cfa.attn_bwd(q, k, v, o, lse, do, cu, scale=w.scale, mx=mx, saved=saved)
        torch.cuda.synchronize()
        return [t.cpu() for t in (o, lse, *g)]
    a = run()
    old = os.environ.get("CFA_SCHED")
    os.environ["CFA_SCHED"] = "naive"
    try:
        b = run()
    finally:
        if old is None:
            del os.environ["CFA_SCHED"]
        else:
            os.environ["CFA_SCHED"] = old
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


@pytest.mark.gpu
@pytest.mark.parametrize("mx", [False, "mxfp8"])
def test_debug_check_fails_malformed_call_before_any_kernel(monkeypatch, mx):
    """CFA_DEBUG_CHECK=1: a malformed device cu_seqlens fails the call with CFA_ERR_SHAPE (the
    flag read back right after the plan kernel); a well-formed one runs as without the switch."""
    announce("debug check", mx)
    T, hq, hkv = 200, 4, 1
    q, k, v, do, sc = _inputs(T, hq, hkv, 33)
    dt = cfa.CFA_MXFP8 if mx else cfa.CFA_BF16
    good = torch.tensor([0, 100, 100, 200], dtype=torch.int32, device=DEV)
    ref_o, ref_lse, ref_saved = cfa.attn_fwd(q, k, v, good, scale=sc, mx=mx)
    ref_grads = cfa.attn_bwd(q, k, v, ref_o, ref_lse, do, good, scale=sc, mx=mx, saved=ref_saved)
    monkeypatch.setenv("CFA_DEBUG_CHECK", "1")
    bad = torch.tensor([0, 100, 50, 200], dtype=torch.int32, device=DEV)
    ws0 = torch.empty(cfa.workspace_bytes(0, T, 3, hq, hkv, 128, dt), dtype=torch.uint8, device=DEV)
    o = torch.full_like(q, SENT)
    lse = torch.full((hq, T), SENT, dtype=torch.float32, device=DEV)
    with pytest.raises(cfa.CfaError) as ei:
        cfa.attn_fwd(q, k, v, bad, scale=sc, mx=mx, out=o, lse=lse, workspace=ws0)
    assert ei.value.name == "CFA_ERR_SHAPE" and "flag 2" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(o == SENT)) and bool(torch.all(lse == SENT))
    dq, dk, dv = torch.full_like(q, SENT), torch.full_like(k, SENT), torch.full_like(v, SENT)
    with pytest.raises(cfa.CfaError):
        cfa.attn_bwd(q, k, v, ref_o, ref_lse, do, bad, scale=sc, mx=mx, saved=ref_saved, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.all(t == SENT))
    o2, lse2, saved2 = cfa.attn_fwd(q, k, v, good, scale=sc, mx=mx)
    grads2 = cfa.attn_bwd(q, k, v, o2, lse2, do, good, scale=sc, mx=mx, saved=saved2)
    assert torch.equal(o2, ref_o) and torch.equal(lse2, ref_lse)
    for a, b in zip(grads2, ref_grads):
        assert torch.equal(a, b)

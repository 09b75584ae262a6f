"""Attention oracle fed with MX-quantised operand copies (forward and backward).

TEST INFRASTRUCTURE ONLY (see the package docstring).

FLAMIA page, "FLAMIA Mimarisi ve Temel Tasarım İlkeleri": an MXFP8 path whose quantised
operands are reused across matrix orientations (token-block scaling), with safeguards so that
a shared scale never carries a later token's data into an earlier query, and with the forward
and backward passes numerically consistent. The page gives no mechanism; the reading here is:

* Every MX GEMM is blocked along its contraction axis. QKᵀ and dO·Vᵀ contract over the head
  dim: their operands are the d-blocked copies ``X_d``. P·V and Pᵀ·dO contract over tokens:
  their V / dO operands are the token-blocked, document-local copies ``X_t``.
* A d-block holds one token's channels, so it cannot leak. A token block can: its scale mixes
  32 neighbouring tokens. Pairs (i, j) lying in the same doc-local C×C tile (C = 128) -- the
  diagonal tiles of the causal mask -- therefore use the unquantised bf16 values ``X_b`` in
  every token-contracted GEMM, and only pairs in off-diagonal tiles use ``X_t``. When
  ``causal`` is false no tile is treated as diagonal.
* The two products with dS (dS·K and dSᵀ·Q) are not MX products: the page fixes no precision
  per product, dS needs more significant bits than one E4M3 rounding keeps, and a two-term
  E4M3 dS costs the matrix cores as much as bf16 on the target hardware. Their K / Q operands
  are the bf16 values ``X_b`` for every pair.
* The backward reuses the forward's ``Q_d``/``K_d`` bytes, so it sees the same scores.

Computed exactly in float64 from the decoded copies (the decoding is exact):

    S_ij  = scale·Q_d[i]·K_d[j]                        P = softmax(S + mask) (two-pass)
    O[i]  = Σ_j P_ij·(diag ? V_b[j] : V_t[j])           LSE_i = max + ln(sum)
    dP_ij = dO_d[i]·V_d[j]                              D_i = dO_b[i]·O[i]
    dS_ij = P_ij·(dP_ij − D_i) + P_ij·dLSE_i             (dLSE optional, else 0)
    dV[j] = Σ_{h in group} Σ_i P_ij·(diag ? dO_b[i] : dO_t[i])
    dQ[i] = scale·Σ_j dS_ij·K_b[j]
    dK[j] = scale·Σ_{h in group} Σ_i dS_ij·Q_b[i]

Not modelled: the rounding of P and dS before a matrix-core product and fp32 accumulation on
the device.

MXFP4/FP8 variant (``qk="e2m1"``): the page names a mixed NVFP4/FP8 path without saying which
products take FP4. The reading here: the score product QKᵀ -- the one whose operands both
passes share through ``saved`` -- takes E2M1 d-blocked copies ``Q_d``, ``K_d`` (same block rule
with the E2M1 top exponent, see ``oracle.mx``); every other product is the MXFP8 path above.
MXFP6/FP8 variants (``qk="e2m3"`` or ``"e3m2"``): the same with E2M3 or E3M2 copies of Q and K.
"""

import numpy as np

from . import attention as _att
from . import mx as _mx

DIAG_TILE = 128


def operand_copies(x_b, cu_seqlens):
    """Decoded d-blocked and token-blocked copies of a bf16-valued tensor [T, h, d]."""
    cd, sd = _mx.quantize_d(x_b)
    ct, st = _mx.quantize_t(x_b, cu_seqlens)
    return _mx.dequantize_d(cd, sd), _mx.dequantize_t(ct, st, cu_seqlens)


def qk_copy(x_b, qk):
    """Decoded d-blocked copy used by QKᵀ: E4M3 (``qk="e4m3"``), E2M1 (``"e2m1"``), E2M3
    (``"e2m3"``) or E3M2 (``"e3m2"``)."""
    if qk == "e2m1":
        c, s = _mx.quantize_d_fp4(x_b)
        return _mx.dequantize_d_fp4(c, s)
    if qk in ("e2m3", "e3m2"):
        c, s = _mx.quantize_d_fp6(x_b, qk)
        return _mx.dequantize_d_fp6(c, s, qk)
    assert qk == "e4m3"
    c, s = _mx.quantize_d(x_b)
    return _mx.dequantize_d(c, s)


def diag_pairs(n_rows, row0, n_cols, causal, tile=DIAG_TILE):
    """Boolean [rows, cols]: true where doc-local query i and key j share a tile×tile tile."""
    if not causal:
        return np.zeros((n_rows, n_cols), dtype=bool)
    i = (row0 + np.arange(n_rows))[:, None] // tile
    j = np.arange(n_cols)[None, :] // tile
    return i == j


def attn_mx_fwd(q_b, k_b, v_b, cu_seqlens, scale, causal=True, tile=DIAG_TILE,
                row_block=_att.ROW_BLOCK, qk="e4m3"):
    """Forward with MX operands; returns o [T, hq, d], lse [hq, T] (float64)."""
    q_b = np.asarray(q_b, np.float64)
    k_b = np.asarray(k_b, np.float64)
    v_b = np.asarray(v_b, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, hq, d = q_b.shape
    hkv = k_b.shape[1]
    group = hq // hkv
    q_d = qk_copy(q_b, qk)
    k_d = qk_copy(k_b, qk)
    _, v_t = operand_copies(v_b, cu)
    o = np.zeros((T, hq, d))
    lse = np.zeros((hq, T))
    for n in range(len(cu) - 1):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        L = s1 - s0
        if L == 0:
            continue
        for h in range(hq):
            g = h // group
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                p, rl = _att._probabilities(q_d[s0 + r0:s0 + r1, h], k_d[s0:s1, g], scale, r0, causal)
                dg = diag_pairs(r1 - r0, r0, L, causal, tile)
                o[s0 + r0:s0 + r1, h] = np.where(dg, p, 0.0) @ v_b[s0:s1, g] + \
                    np.where(dg, 0.0, p) @ v_t[s0:s1, g]
                lse[h, s0 + r0:s0 + r1] = rl
    return o, lse


def attn_mx_bwd(q_b, k_b, v_b, do_b, cu_seqlens, scale, causal=True, tile=DIAG_TILE,
                row_block=_att.ROW_BLOCK, dlse=None, qk="e4m3"):
    """Backward with MX operands; returns dq [T, hq, d], dk, dv [T, hkv, d] (float64)."""
    q_b = np.asarray(q_b, np.float64)
    k_b = np.asarray(k_b, np.float64)
    v_b = np.asarray(v_b, np.float64)
    do_b = np.asarray(do_b, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, hq, d = q_b.shape
    hkv = k_b.shape[1]
    group = hq // hkv
    q_d, k_d = qk_copy(q_b, qk), qk_copy(k_b, qk)
    v_d, v_t = operand_copies(v_b, cu)
    do_d, do_t = operand_copies(do_b, cu)
    dlse = np.zeros((hq, T)) if dlse is None else np.asarray(dlse, np.float64)
    dq = np.zeros((T, hq, d))
    dk = np.zeros((T, hkv, d))
    dv = np.zeros((T, hkv, d))
    for n in range(len(cu) - 1):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        L = s1 - s0
        if L == 0:
            continue
        for h in range(hq):
            g = h // group
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = slice(s0 + r0, s0 + r1)
                p, _ = _att._probabilities(q_d[rows, h], k_d[s0:s1, g], scale, r0, causal)
                dg = diag_pairs(r1 - r0, r0, L, causal, tile)
                p_diag, p_off = np.where(dg, p, 0.0), np.where(dg, 0.0, p)
                o = p_diag @ v_b[s0:s1, g] + p_off @ v_t[s0:s1, g]
                D = np.sum(do_b[rows, h] * o, axis=1)
                dp = do_d[rows, h] @ v_d[s0:s1, g].T
                ds = p * (dp - D[:, None]) + p * dlse[h, rows][:, None]
                dv[s0:s1, g] += p_diag.T @ do_b[rows, h] + p_off.T @ do_t[rows, h]
                dq[rows, h] = scale * (ds @ k_b[s0:s1, g])
                dk[s0:s1, g] += scale * (ds.T @ q_b[rows, h])
    return dq, dk, dv


def attn_mx_rows(q_b, k_b, v_b, do_b, rows, scale, causal=True, tile=DIAG_TILE, qk="e4m3"):
    """Selected query rows of ONE document with MX operands (doc-local arrays).

    The MX counterpart of ``oracle.attention.attn_rows`` for documents too long for the full
    oracle: the quantised copies are built for the whole document (blocks are doc-local), then
    each selected row follows the definitions in the module docstring. Returns
    ``o [n, hq, d], lse [hq, n], dq [n, hq, d]`` and the partial ``dk, dv [L, hkv, d]`` summed
    over the selected rows only.
    """
    q_b = np.asarray(q_b, np.float64)
    k_b = np.asarray(k_b, np.float64)
    v_b = np.asarray(v_b, np.float64)
    do_b = np.asarray(do_b, np.float64)
    rows = np.asarray(rows, np.int64)
    L, hq, d = q_b.shape
    hkv = k_b.shape[1]
    group = hq // hkv
    cu = np.array([0, L])
    q_d, k_d = qk_copy(q_b, qk), qk_copy(k_b, qk)
    v_d, v_t = operand_copies(v_b, cu)
    do_d, do_t = operand_copies(do_b, cu)
    n = len(rows)
    o = np.zeros((n, hq, d))
    lse = np.zeros((hq, n))
    dq = np.zeros((n, hq, d))
    dk = np.zeros_like(k_b)
    dv = np.zeros_like(v_b)
    for h in range(hq):
        g = h // group
        for r0 in range(0, n, 256):
            rs = rows[r0:r0 + 256]
            s = scale * (q_d[rs, h] @ k_d[:, g].T)
            mask = np.zeros_like(s)
            if causal:
                mask[np.arange(L)[None, :] > rs[:, None]] = -np.inf
            z = s + mask
            m = z.max(axis=1)
            e = np.exp(z - m[:, None])
            l = e.sum(axis=1)
            p = e / l[:, None]
            if causal:
                dg = (rs[:, None] // tile) == (np.arange(L)[None, :] // tile)
            else:
                dg = np.zeros_like(p, dtype=bool)
            p_diag, p_off = np.where(dg, p, 0.0), np.where(dg, 0.0, p)
            ob = p_diag @ v_b[:, g] + p_off @ v_t[:, g]
            o[r0:r0 + len(rs), h] = ob
            lse[h, r0:r0 + len(rs)] = m + np.log(l)
            D = np.sum(do_b[rs, h] * ob, axis=1)
            ds = p * (do_d[rs, h] @ v_d[:, g].T - D[:, None])
            dq[r0:r0 + len(rs), h] = scale * (ds @ k_b[:, g])
            dk[:, g] += scale * (ds.T @ q_b[rs, h])
            dv[:, g] += p_diag.T @ do_b[rs, h] + p_off.T @ do_t[rs, h]
    return o, lse, dq, dk, dv

"""Naive float64 attention over packed documents: forward and exact gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain NumPy, float64, explicit mask.

Layout: packed tokens × heads × head-dim, row-major. ``q`` is ``[T, hq, d]``; ``k`` and ``v``
are ``[T, hkv, d]``. Document ``n`` owns packed rows ``cu_seqlens[n] .. cu_seqlens[n+1]-1``;
attention never crosses a document boundary (document-local, packed layout: FLAMIA page,
"FLAMIA Mimarisi ve Temel Tasarım İlkeleri"). Query head ``h`` reads kv head
``h // (hq // hkv)`` (consecutive query heads share a kv head).
"""

import numpy as np

ROW_BLOCK = 512  # query rows per explicit score block (memory bound only; rows are independent)


def _check(q, k, v, cu_seqlens):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, hq, d = q.shape
    assert k.shape[0] == T and v.shape[0] == T and k.shape == v.shape and k.shape[2] == d
    hkv = k.shape[1]
    assert hq % hkv == 0
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    return q, k, v, cu, T, hq, hkv, d


def causal_mask(n_rows, row0, n_cols, causal):
    """Explicit additive mask: 0 where key j may be seen by query i, -inf where j > i.

    "GPT Kernel Programlama" §4: a query must not see later tokens, so their scores are set to
    minus infinity before the softmax. ``i`` and ``j`` are document-local indices; ``row0`` is
    the first query row of the block.
    """
    m = np.zeros((n_rows, n_cols), dtype=np.float64)
    if causal:
        i = (row0 + np.arange(n_rows))[:, None]
        j = np.arange(n_cols)[None, :]
        m[j > i] = -np.inf
    return m


def _probabilities(qb, kd, scale, row0, causal):
    """Scores, explicit mask and the two-pass (max, then sum) softmax of one row block.

    "GPT Kernel Programlama" §3 (S = Q·Kᵀ/√d, here with the scale passed in), §4 (mask),
    §5 (subtract the row maximum, exponentiate, divide by the row sum).
    Returns P and the row log-sum-exp m + ln(l) of the masked, scaled scores.
    """
    s = scale * (qb @ kd.T)
    z = s + causal_mask(qb.shape[0], row0, kd.shape[0], causal)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    return p, m + np.log(l)


def attn_fwd(q, k, v, cu_seqlens, scale, causal=True, row_block=ROW_BLOCK):
    """Forward pass: O = softmax(scale·QKᵀ + mask)·V per document and head; also LSE.

    "GPT Kernel Programlama" §2 (the three equations), §6 (O[i,r] = Σ_j P[i,j]·V[j,r]);
    "FlashAttention (HU)", "A szabványos attention problematikája" (softmax(QKᵀ/√d_k)V).

    Returns ``o [T, hq, d]`` and ``lse [hq, T]`` (natural log of Σ_j exp(scaled masked score)).
    Rows of empty documents do not exist; a packed token belongs to exactly one document.
    """
    q, k, v, cu, T, hq, hkv, d = _check(q, k, v, cu_seqlens)
    group = hq // hkv
    o = np.zeros((T, hq, d), dtype=np.float64)
    lse = np.zeros((hq, T), dtype=np.float64)
    for n in range(len(cu) - 1):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        L = s1 - s0
        if L == 0:
            continue
        for h in range(hq):
            g = h // group
            kd = k[s0:s1, g, :]
            vd = v[s0:s1, g, :]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                p, rl = _probabilities(q[s0 + r0:s0 + r1, h, :], kd, scale, r0, causal)
                o[s0 + r0:s0 + r1, h, :] = p @ vd
                lse[h, s0 + r0:s0 + r1] = rl
    return o, lse


def attn_bwd(q, k, v, do, cu_seqlens, scale, causal=True, row_block=ROW_BLOCK, dlse=None):
    """Exact gradient of ``attn_fwd`` for upstream gradients ``do`` (of O) and ``dlse`` (of LSE).

    The pages only name the backward pass (FLAMIA page, "FLAMIA Mimarisi ve Temel Tasarım
    İlkeleri": forward and backward must agree numerically); these are the derivatives of the
    forward definition above, with the oracle's own float64 O and P:

        D_i    = Σ_r dO[i,r]·O[i,r]
        dP_ij  = Σ_r dO[i,r]·V[j,r]
        dS_ij  = P_ij·(dP_ij − D_i) + P_ij·dLSE_i
        dQ[i]  = scale·Σ_j dS_ij·K[j]
        dK[j]  = scale·Σ_{h in group} Σ_i dS_ij·Q[i]
        dV[j]  = Σ_{h in group} Σ_i P_ij·dO[i]

    The dLSE term is the derivative of LSE_i = log Σ_j exp(S_ij), which is P_ij (the pages do
    not name an LSE gradient; ``dlse [hq, T]`` defaults to zero).
    Returns ``dq [T, hq, d]``, ``dk, dv [T, hkv, d]``.
    """
    q, k, v, cu, T, hq, hkv, d = _check(q, k, v, cu_seqlens)
    do = np.asarray(do, dtype=np.float64)
    assert do.shape == q.shape
    dlse = np.zeros((hq, T)) if dlse is None else np.asarray(dlse, dtype=np.float64)
    assert dlse.shape == (hq, T)
    group = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for n in range(len(cu) - 1):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        L = s1 - s0
        if L == 0:
            continue
        for h in range(hq):
            g = h // group
            kd = k[s0:s1, g, :]
            vd = v[s0:s1, g, :]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                qb = q[s0 + r0:s0 + r1, h, :]
                dob = do[s0 + r0:s0 + r1, h, :]
                p, _ = _probabilities(qb, kd, scale, r0, causal)
                ob = p @ vd
                D = np.sum(dob * ob, axis=1)
                dp = dob @ vd.T
                ds = p * (dp - D[:, None]) + p * dlse[h, s0 + r0:s0 + r1][:, None]
                dq[s0 + r0:s0 + r1, h, :] = scale * (ds @ kd)
                dk[s0:s1, g, :] += scale * (ds.T @ qb)
                dv[s0:s1, g, :] += p.T @ dob
    return dq, dk, dv


def attn_rows(q, k, v, do, rows, scale, causal=True):
    """Selected query rows of ONE document (doc-local arrays), forward and backward by definition.

    For large documents where the full oracle is too slow: every quantity of query row i
    depends only on row i's softmax over keys 0..i (or all keys when not causal), so rows can
    be computed one block at a time. ``q, do [L, hq, d]``, ``k, v [L, hkv, d]``; ``rows`` is a
    sorted 1-D array of doc-local query indices. Returns

        o [len(rows), hq, d], lse [hq, len(rows)], dq [len(rows), hq, d],
        dk_part, dv_part [L, hkv, d] -- the contributions of the selected rows only; for a key j
        they are the complete dK/dV when ``rows`` covers every query that can see j.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    rows = np.asarray(rows, np.int64)
    L, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    n = len(rows)
    o = np.zeros((n, hq, d))
    lse = np.zeros((hq, n))
    dq = np.zeros((n, hq, d))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        g = h // group
        for r0 in range(0, n, 256):
            rs = rows[r0:r0 + 256]
            s = scale * (q[rs, h] @ k[:, g].T)
            mask = np.zeros_like(s)
            if causal:
                mask[np.arange(L)[None, :] > rs[:, None]] = -np.inf
            z = s + mask
            m = z.max(axis=1)
            e = np.exp(z - m[:, None])
            l = e.sum(axis=1)
            p = e / l[:, None]
            ob = p @ v[:, g]
            o[r0:r0 + len(rs), h] = ob
            lse[h, r0:r0 + len(rs)] = m + np.log(l)
            D = np.sum(do[rs, h] * ob, axis=1)
            ds = p * (do[rs, h] @ v[:, g].T - D[:, None])
            dq[r0:r0 + len(rs), h] = scale * (ds @ k[:, g])
            dk[:, g] += scale * (ds.T @ q[rs, h])
            dv[:, g] += p.T @ do[rs, h]
    return o, lse, dq, dk, dv


def attn_key_block(q, k, v, do, k0, k1, scale, causal=True, row_block=256, q_range=None):
    """dK and dV of keys k0..k1-1 of ONE document (doc-local arrays), summed over every query.

    For documents too long for the full oracle, when a block of keys is to be checked
    completely: dK_j and dV_j sum over all queries i that see key j (i >= j when causal), and
    each term needs that query's whole softmax row (its normaliser) and its O_i (for D_i). So
    every query row that can see the block is formed in full, as in ``attn_bwd`` -- scores of
    the keys the row may see, explicit mask, two-pass softmax ("GPT Kernel Programlama"
    §3-§6) -- and only the block's columns of P and dS enter the sums (the derivatives of
    ``attn_bwd``). A causal row i is formed over keys 0..r1-1 of its row block (r1 > i): the
    keys past i are masked, so their probabilities are exact zeros either way.
    ``q, do [L, hq, d]``, ``k, v [L, hkv, d]``. Returns ``dk, dv [k1 - k0, hkv, d]``.
    ``q_range = (a, b)`` sums over queries a..b-1 only (the sums split by query ranges add up
    to the whole).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    L, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    assert 0 <= k0 <= k1 <= L
    nk = k1 - k0
    dk = np.zeros((nk, hkv, d))
    dv = np.zeros((nk, hkv, d))
    first_row = k0 if causal else 0
    qa, qb = (0, L) if q_range is None else q_range
    for h in range(hq):
        g = h // group
        for r0 in range(max(first_row, qa), qb, row_block):
            r1 = min(qb, r0 + row_block)
            cols = r1 if causal else L
            p, _ = _probabilities(q[r0:r1, h], k[:cols, g], scale, r0, causal)
            o = p @ v[:cols, g]
            D = np.sum(do[r0:r1, h] * o, axis=1)
            pb = np.zeros((r1 - r0, nk))
            c1 = min(k1, cols)
            pb[:, :c1 - k0] = p[:, k0:c1]
            dp = do[r0:r1, h] @ v[k0:k1, g].T
            ds = pb * (dp - D[:, None])
            dv[:, g] += pb.T @ do[r0:r1, h]
            dk[:, g] += scale * (ds.T @ q[r0:r1, h])
    return dk, dv


# ---------------------------------------------------------------- cross-attention
def cross_mask(Lq, Lk, causal):
    """Explicit additive mask of one document with separate query and key lengths.

    Causal: query i sees key j iff j <= i + (Lk - Lq), the causal rule with the queries aligned to
    the end of the keys (the queries are the last Lq positions of a sequence of Lk): for Lq = Lk it
    is the self-attention mask of "GPT Kernel Programlama" §4, and a single query sees every key
    (decoding). Queries with i + Lk - Lq < 0 see no key.
    """
    m = np.zeros((Lq, Lk), dtype=np.float64)
    if causal:
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        m[j > i + (Lk - Lq)] = -np.inf
    return m


def attn_cross(q, k, v, do, cu_q, cu_k, scale, causal=True, dlse=None):
    """Attention of packed query documents on packed key/value documents (document n: query rows
    cu_q[n]..cu_q[n+1]-1, key rows cu_k[n]..cu_k[n+1]-1), forward and exact gradient.

    Per document and head, with M the mask of ``cross_mask``: S = scale·QKᵀ + M, P = softmax(S)
    by rows (two-pass, §5), O = PV, LSE = log Σ exp(S); a row that sees no key has the empty sum:
    O = 0, LSE = -inf, P = 0, and so no gradient. Gradient as in ``attn_bwd`` (D_i = dO_i·O_i −
    dLSE_i, dS = P∘(dP − D)). ``do`` may be None (forward only). Returns o, lse, dq, dk, dv.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    cq = np.asarray(cu_q, np.int64)
    ck = np.asarray(cu_k, np.int64)
    Tq, hq, d = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    assert len(cq) == len(ck) and cq[-1] == Tq and ck[-1] == Tk and v.shape == k.shape
    group = hq // hkv
    o = np.zeros((Tq, hq, d))
    lse = np.full((hq, Tq), -np.inf)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlse = np.zeros((hq, Tq)) if dlse is None else np.asarray(dlse, np.float64)
    for n in range(len(cq) - 1):
        q0, q1, k0, k1 = int(cq[n]), int(cq[n + 1]), int(ck[n]), int(ck[n + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0:
            continue
        M = cross_mask(Lq, Lk, causal)
        for h in range(hq):
            g = h // group
            if Lk == 0:
                continue
            z = scale * (q[q0:q1, h] @ k[k0:k1, g].T) + M
            seen = np.isfinite(z).any(axis=1)
            m = np.where(seen, z.max(axis=1), 0.0)
            e = np.where(seen[:, None], np.exp(z - m[:, None]), 0.0)
            l = e.sum(axis=1)
            p = np.where(seen[:, None], e / np.where(seen, l, 1.0)[:, None], 0.0)
            ob = p @ v[k0:k1, g]
            o[q0:q1, h] = ob
            lse[h, q0:q1] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
            if do is None:
                continue
            dob = np.asarray(do, np.float64)[q0:q1, h]
            D = np.sum(dob * ob, axis=1) - dlse[h, q0:q1]
            ds = p * (dob @ v[k0:k1, g].T - D[:, None])
            dq[q0:q1, h] = scale * (ds @ k[k0:k1, g])
            dk[k0:k1, g] += scale * (ds.T @ q[q0:q1, h])
            dv[k0:k1, g] += p.T @ dob
    return o, lse, dq, dk, dv

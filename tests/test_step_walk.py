"""CPU model of the dK/dV kernels' step walk (host logic, no GPU).

A dK/dV work item visits, for its key tile, every (query head h, first query q0) step: the query
heads of its group (or of its head split) outer and the query tiles ascending from the diagonal
inner; with dQ inside the pass, the query tiles from the document end down to the diagonal with
the heads inner. The kernels do not divide the step index by the tile count at each step: they
start from the first position and advance it by one step per iteration (an add and a compare on
the scalar unit). This test runs that advance rule next to the closed form (step -> (h, q0) by
division) over many shapes, ragged tails and empty cases, and checks that the two visit the same
positions in the same order."""
import itertools

import pytest


def closed_form(st, h_lo, n_h, q_begin, n_qt, bm, fq):
    if fq:
        return h_lo + st % n_h, q_begin + (n_qt - 1 - st // n_h) * bm
    return h_lo + st // n_qt, q_begin + (st % n_qt) * bm


def walk(h_lo, n_h, q_begin, n_qt, bm, fq, n_steps):
    """The kernels' rule: first position, then one advance per step."""
    h, q0 = h_lo, (q_begin + (n_qt - 1) * bm if fq else q_begin)
    q_end = q_begin + n_qt * bm
    out = []
    for _ in range(n_steps):
        out.append((h, q0))
        if fq:
            h += 1
            if h == h_lo + n_h:
                h, q0 = h_lo, q0 - bm
        else:
            q0 += bm
            if q0 >= q_end:
                q0, h = q_begin, h + 1
    return out


@pytest.mark.parametrize("fq", [False, True])
def test_walk_matches_division(fq):
    bm = 64
    for L, t, kt, g, G, causal in itertools.product([0, 1, 63, 64, 65, 200, 1000], [0, 1, 3], [128],
                                                     [0, 2], [1, 4, 8], [False, True]):
        q_begin = t * kt if causal else 0
        n_qt = max(0, (L - q_begin + bm - 1) // bm)
        n_h = G
        h_lo = g * G
        n_steps = n_qt * n_h
        expect = [closed_form(st, h_lo, n_h, q_begin, n_qt, bm, fq) for st in range(n_steps)]
        assert walk(h_lo, n_h, q_begin, n_qt, bm, fq, n_steps) == expect, (L, t, g, G, causal)
        # every step starts inside the document and every (head, tile) pair appears once
        assert len(set(expect)) == n_steps
        assert all(q_begin <= q0 < max(L, q_begin + 1) for _, q0 in expect)


def test_mx_walk_on_document_length():
    """The MX dK/dV kernel wraps at the document length L instead of the tile end; both give the
    same positions because the last tile starts below L and the next would start at or past it."""
    bm = 64
    for L in range(1, 700, 7):
        for t in range(0, (L + 127) // 128):
            q_begin = t * 128
            n_qt = (L - q_begin + bm - 1) // bm
            h, q0, seen = 0, q_begin, []
            for _ in range(n_qt * 3):
                seen.append((h, q0))
                q0 += bm
                if q0 >= L:
                    q0, h = q_begin, h + 1
            assert seen == [closed_form(st, 0, 3, q_begin, n_qt, bm, False) for st in range(n_qt * 3)]

"""CPU model of the fused backward's schedule: per-XCD claims of key tiles and ordered dQ sums.

The persistent dK/dV/dQ kernel hands out key tiles through one 64-bit word per XCD (high half:
chain + 1, low half: next tile; atomic increment) and a global chain counter; the workgroup that
draws the first tile past a chain's end takes the next chain and publishes it, later drawers wait
for the word to change. Tile t of a chain adds into each (query head, query tile) block only after
tile t - 1 has (a count per block). This model runs the same protocol as interleaved
generators -- every atomic step is one scheduling point, the interleaving random -- and checks
that every tile is processed exactly once, that every block receives its key tiles in the order
0, 1, 2, ..., and that the system never deadlocks, whatever the number of workgroups per XCD
(including XCDs with none, or one workgroup that must run a whole chain alone)."""
import random

import pytest

END = 0x7fffffff


class Machine:
    def __init__(self, chains, n_xcd):
        self.chains = chains                 # list of (n_tiles, n_query_tiles)
        self.word = [(0, 0)] * n_xcd         # (hi, lo)
        self.counter = 0
        self.cnt = {}                        # (chain, query tile) -> tiles added so far
        self.order = {}                      # (chain, query tile) -> list of tiles in adding order
        self.done = set()

    def tiles(self, c):
        return self.chains[c][0]


def workgroup(m, x, log):
    """One persistent workgroup on XCD x; yields at every atomic step or wait poll."""
    while True:
        # claim
        while True:
            hi, lo = m.word[x]
            m.word[x] = (hi, lo + 1)                        # atomic add on the low half
            yield
            if hi == END:
                return
            n = 0 if hi == 0 else m.tiles(hi - 1)
            if lo < n:
                chain, tile = hi - 1, lo
                break
            if lo == n:
                got = None
                while True:
                    c = m.counter
                    m.counter += 1                          # atomic add on the chain counter
                    yield
                    if c >= len(m.chains):
                        m.word[x] = (END, 0)
                        yield
                        return
                    if m.tiles(c) > 0:
                        got = c
                        break
                m.word[x] = (got + 1, 1)                    # atomic exchange: tile 0 taken
                yield
                chain, tile = got, 0
                break
            while m.word[x][0] == hi:                       # another workgroup is claiming
                yield
        # process: query tiles from the last down to this tile's diagonal (causal, 2 per key tile)
        assert (chain, tile) not in m.done
        n_qt = m.chains[chain][1]
        for qt in range(n_qt - 1, 2 * tile - 1, -1):
            key = (chain, qt)
            while m.cnt.get(key, 0) < tile:                 # wait for tile - 1
                yield
            m.order.setdefault(key, []).append(tile)        # add this tile's part
            yield
            m.cnt[key] = tile + 1                           # hand over
            yield
        m.done.add((chain, tile))
        log.append((x, chain, tile))


def run(chains, wgs_per_xcd, seed, max_steps=2_000_000):
    rng = random.Random(seed)
    m = Machine(chains, len(wgs_per_xcd))
    log = []
    live = [workgroup(m, x, log) for x, n in enumerate(wgs_per_xcd) for _ in range(n)]
    steps = 0
    while live:
        i = rng.randrange(len(live))
        try:
            next(live[i])
        except StopIteration:
            live.pop(i)
        steps += 1
        assert steps < max_steps, "no progress: deadlock"
    return m, log


def doc_chains(lengths, hkv):
    out = []
    for L in sorted(lengths, reverse=True):                 # longest first, as the plan orders them
        for _ in range(hkv):
            out.append(((L + 127) // 128, (L + 63) // 64))
    return out


@pytest.mark.parametrize("wgs", [[4, 4, 4, 4], [1, 0, 3, 0], [0, 0, 0, 1], [6, 1, 0, 2], [2] * 8])
@pytest.mark.parametrize("lengths,hkv", [([1000], 2), ([300, 0, 129, 1, 64, 700], 2), ([0, 0], 3), ([5000], 1)])
def test_claims_cover_every_tile_once_in_order(wgs, lengths, hkv):
    chains = doc_chains(lengths, hkv)
    for seed in range(3):
        m, log = run(chains, wgs, seed)
        want = {(c, t) for c, (n, _) in enumerate(chains) for t in range(n)}
        assert m.done == want
        assert len(log) == len(want)
        for (c, qt), tiles in m.order.items():
            # key tiles 0 .. diagonal, each once, in order
            assert tiles == list(range(min(qt // 2, chains[c][0] - 1) + 1)), (c, qt, tiles)
        # all tiles of a chain ran on one XCD
        xcds = {}
        for x, c, t in log:
            xcds.setdefault(c, set()).add(x)
        assert all(len(v) == 1 for v in xcds.values())

"""Seeded synthetic workloads shared by the tests, the bench and the oracle's callers.

Holds no attention or quantisation arithmetic: it draws document lengths and N(0,1) tensors,
rounds float32 to bf16 (round to nearest even, bit arithmetic) and counts causal FLOPs.

RNG: ``numpy.random.Generator(PCG64(seed))``. Draw order: document lengths, then Q, K, V, dO
as float32 standard normals in C order ``[T, H, d]``, then (heavy-tailed workload only) the
outlier channels and the shuffle of the document list.

Workloads (d = 128 unless stated):

1. ``fp32_single``   T=256, one document, hq=hkv=1, d=64, fp32, scale 1/8, forward only.
2. ``bf16_packed``   T=8192, hq=hkv=16, lengths uniform integers in [64, 2048].
3. ``bf16_gqa32k``   T=32768, one document, hq=32, hkv=8 (GQA group 4).
4. ``mxfp8_packed``  T=65536, hq=hkv=32, lengths floor(exp(U(ln 128, ln 16384))), MXFP8.
5. ``heavy_tail``    T=131072, hq=hkv=16, four 16384-token documents plus documents of
   uniform length [32, 128] filling the rest, shuffled; Q/K/V get 2 outlier channels per head
   (1% of 128, rounded up) scaled by 20 before the bf16 cast.

Packed workloads draw lengths until the total is reached and truncate the last document.
"""

from dataclasses import dataclass, field
import math

import numpy as np

NAMES = {1: "fp32_single", 2: "bf16_packed", 3: "bf16_gqa32k", 4: "mxfp8_packed", 5: "heavy_tail"}


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    """Exact float64 value of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def causal_flops_fwd(cu_seqlens, hq, d, causal=True):
    """Algorithmic forward FLOPs: two GEMMs over the causal pairs, 4·d·hq·Σ L(L+1)/2."""
    L = np.diff(np.asarray(cu_seqlens, dtype=np.int64)).astype(np.float64)
    pairs = np.sum(L * (L + 1) / 2) if causal else np.sum(L * L)
    return 4.0 * d * hq * float(pairs)


def causal_flops_fwd_bwd(cu_seqlens, hq, d, causal=True):
    """Forward plus backward: 3.5 × forward (2 + 5 GEMMs)."""
    return 3.5 * causal_flops_fwd(cu_seqlens, hq, d, causal)


@dataclass
class Workload:
    name: str
    total_tokens: int
    hq: int
    hkv: int
    d: int
    dtype: str                 # "f32", "bf16" or "mxfp8"
    scale: float
    cu_seqlens: np.ndarray     # int32 [n_docs + 1]
    q: np.ndarray              # uint16 bf16 bits, or float32 for dtype "f32"
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray = None
    causal: bool = True
    info: dict = field(default_factory=dict)

    @property
    def n_docs(self):
        return len(self.cu_seqlens) - 1

    @property
    def max_seqlen(self):
        return int(np.max(np.diff(self.cu_seqlens))) if self.n_docs else 0

    def f64(self, name):
        """Exact float64 values of one input tensor ('q', 'k', 'v', 'do')."""
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f64(a)
        return a.astype(np.float64)

    def flops_fwd(self):
        return causal_flops_fwd(self.cu_seqlens, self.hq, self.d, self.causal)

    def flops_fwd_bwd(self):
        return causal_flops_fwd_bwd(self.cu_seqlens, self.hq, self.d, self.causal)


def _fill_lengths(draw, total):
    lengths = []
    s = 0
    while s < total:
        L = int(draw())
        L = min(L, total - s)
        lengths.append(L)
        s += L
    return lengths


def cu_from_lengths(lengths):
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def _normals(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_workload(k, seed=None, with_grad=True):
    """Workload number k (1..5) drawn from PCG64(seed), seed defaulting to k."""
    seed = k if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    d = 64 if k == 1 else 128
    if k == 1:
        T, hq, hkv, dtype = 256, 1, 1, "f32"
        lengths = [256]
    elif k == 2:
        T, hq, hkv, dtype = 8192, 16, 16, "bf16"
        lengths = _fill_lengths(lambda: rng.integers(64, 2049), T)
    elif k == 3:
        T, hq, hkv, dtype = 32768, 32, 8, "bf16"
        lengths = [T]
    elif k == 4:
        T, hq, hkv, dtype = 65536, 32, 32, "mxfp8"
        lengths = _fill_lengths(lambda: math.floor(math.exp(rng.uniform(math.log(128), math.log(16384)))), T)
    elif k == 5:
        T, hq, hkv, dtype = 131072, 16, 16, "bf16"
        lengths = [16384] * 4 + _fill_lengths(lambda: rng.integers(32, 129), T - 4 * 16384)
    else:
        raise ValueError(f"no workload {k}")
    q = _normals(rng, (T, hq, d))
    kk = _normals(rng, (T, hkv, d))
    v = _normals(rng, (T, hkv, d))
    do = _normals(rng, (T, hq, d)) if (with_grad and k != 1) else None
    if k == 5:
        n_out = math.ceil(0.01 * d)
        for a in (q, kk, v):
            for h in range(a.shape[1]):
                ch = rng.choice(d, size=n_out, replace=False)
                a[:, h, ch] *= 20.0
        order = rng.permutation(len(lengths))
        lengths = [lengths[i] for i in order]
    cu = cu_from_lengths(lengths)
    if dtype != "f32":
        q, kk, v = f32_to_bf16_bits(q), f32_to_bf16_bits(kk), f32_to_bf16_bits(v)
        do = f32_to_bf16_bits(do) if do is not None else None
    return Workload(name=NAMES[k], total_tokens=T, hq=hq, hkv=hkv, d=d, dtype=dtype,
                    scale=1.0 / math.sqrt(d), cu_seqlens=cu, q=q, k=kk, v=v, do=do,
                    info={"config": k, "seed": seed})


def make_random(seed, lengths, hq, hkv, d=128, dtype="bf16", scale=None, causal=True,
                value_scale=1.0, with_grad=True):
    """Small ad-hoc workload with given document lengths (for parity and edge-case tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = int(sum(lengths))
    q = _normals(rng, (T, hq, d)) * np.float32(value_scale)
    kk = _normals(rng, (T, hkv, d)) * np.float32(value_scale)
    v = _normals(rng, (T, hkv, d))
    do = _normals(rng, (T, hq, d)) if with_grad else None
    if dtype != "f32":
        q, kk, v = f32_to_bf16_bits(q), f32_to_bf16_bits(kk), f32_to_bf16_bits(v)
        do = f32_to_bf16_bits(do) if do is not None else None
    return Workload(name="random", total_tokens=T, hq=hq, hkv=hkv, d=d, dtype=dtype,
                    scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                    cu_seqlens=cu_from_lengths(lengths), q=q, k=kk, v=v, do=do, causal=causal,
                    info={"seed": seed, "lengths": list(lengths)})


# ---------------------------------------------------------------- decoding over a KV cache
@dataclass
class DecodeWorkload:
    """One new query token per sequence over a packed KV cache.

    ``q [B, hq, d]`` bf16 bits; the cache ``k, v [Tk, hkv, d]`` holds bf16 bits (kv "bf16") or
    E4M3 codes (kv "mxfp8", with E8M0 block scales ``k_scales, v_scales [Tk, hkv, d/32]``);
    sequence ``b`` owns cache rows ``cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1``.
    """
    name: str
    hq: int
    hkv: int
    d: int
    kv: str
    scale: float
    cu_seqlens_k: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_scales: np.ndarray = None
    v_scales: np.ndarray = None
    info: dict = field(default_factory=dict)

    @property
    def n_seqs(self):
        return len(self.cu_seqlens_k) - 1

    @property
    def total_k(self):
        return int(self.cu_seqlens_k[-1])

    def kv_bytes(self):
        """Bytes of the cache read once (codes and scales, or bf16), K and V."""
        per = self.d * (1 + 1 / 32) if self.kv == "mxfp8" else 2 * self.d
        return 2.0 * self.total_k * self.hkv * per


def make_decode(seed, lengths, hq, hkv, d=128, kv="bf16", scale=None):
    """Seeded decode inputs. Draw order: Q (N(0,1) → bf16), then K, V: bf16 N(0,1) values, or
    E4M3 codes uniform over the 254 finite byte values with E8M0 scale bytes uniform in
    [117, 124] (2^-10 .. 2^-3), drawn K codes, K scales, V codes, V scales."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = len(lengths)
    Tk = int(sum(lengths))
    q = f32_to_bf16_bits(_normals(rng, (B, hq, d)))
    ks = vs = None
    if kv == "bf16":
        k = f32_to_bf16_bits(_normals(rng, (Tk, hkv, d)))
        v = f32_to_bf16_bits(_normals(rng, (Tk, hkv, d)))
    elif kv == "mxfp8":
        def codes():
            c = rng.integers(0, 254, size=(Tk, hkv, d), dtype=np.int64)
            c = c + (c >= 0x7F)                   # skip 0x7F; 0xFF is never drawn (max 254)
            return c.astype(np.uint8)

        def scales():
            return rng.integers(117, 125, size=(Tk, hkv, d // 32)).astype(np.uint8)
        k, ks = codes(), scales()
        v, vs = codes(), scales()
    else:
        raise ValueError(kv)
    return DecodeWorkload(name="decode", hq=hq, hkv=hkv, d=d, kv=kv,
                          scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                          cu_seqlens_k=cu_from_lengths(lengths), q=q, k=k, v=v, k_scales=ks, v_scales=vs,
                          info={"seed": seed, "lengths": list(lengths)})


def decode_batch_lengths(seed, n_seqs, lo=512, hi=32768):
    """Context lengths of a serving batch: floor(exp(U(ln lo, ln hi))) per sequence."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi))))) for _ in range(n_seqs)]


def reorder_documents(w, order):
    """The same documents packed in another order: document ``order[i]`` of ``w`` becomes
    document ``i``, its tokens moving with it (Q, K, V and dO rows alike)."""
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    order = [int(i) for i in order]
    if sorted(order) != list(range(w.n_docs)):
        raise ValueError("order must be a permutation of the document indices")
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order]) if order else np.zeros(0, np.int64)

    def take(a):
        return None if a is None else np.ascontiguousarray(a[rows])
    lengths = [int(cu[i + 1] - cu[i]) for i in order]
    info = dict(w.info)
    info["doc_order"] = "permuted"
    return Workload(name=w.name, total_tokens=w.total_tokens, hq=w.hq, hkv=w.hkv, d=w.d, dtype=w.dtype,
                    scale=w.scale, cu_seqlens=cu_from_lengths(lengths), q=take(w.q), k=take(w.k),
                    v=take(w.v), do=take(w.do), causal=w.causal, info=info)


def longest_last(w):
    """``w`` with its documents sorted by length, shortest first (ties keep their order): the
    packing order that is worst for a scheduler that hands out work in document order."""
    L = np.diff(np.asarray(w.cu_seqlens, dtype=np.int64))
    out = reorder_documents(w, np.argsort(L, kind="stable"))
    out.info["doc_order"] = "longest_last"
    return out

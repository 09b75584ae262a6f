// Recomputing causal attention backward for gfx950 (bf16 MFMA), deterministic.
//
// The pages only name the backward pass (FLAMIA page, "FLAMIA Mimarisi ve Temel Tasarım
// İlkeleri": forward and backward must agree numerically). The kernels compute the exact
// derivative of the forward definition ("GPT Kernel Programlama" §2-§6), recomputing the
// probabilities tile by tile from the saved row log-sum-exp instead of storing P:
//   P_ij  = exp(scale·q_i·k_j − LSE_i)           (0 where key j is masked)
//   D_i   = Σ_r dO_ir O_ir − dLSE_i               -- bwd_pre_kernel (dLSE optional, else 0)
//   dP_ij = dO_i·v_j,  dS_ij = P_ij (dP_ij − D_i)
//   dV_j  = Σ_{h in group} Σ_i P_ij dO_i           -- attn_bwd_dkdv_pair_kernel
//   dK_j  = scale Σ_{h in group} Σ_i dS_ij q_i     -- attn_bwd_dkdv_pair_kernel
//   dQ_i  = scale Σ_j dS_ij k_j                    -- attn_bwd_dq_kernel (separate pass)
// No floating-point atomics: each output element is summed by one lane in a fixed order, so
// reruns are bit-identical and a token never receives contributions through shared state.
//
// dK/dV kernel: wave pairs own 32 keys of one kv head each (K or V rows in registers as MFMA B
// operands) and walk the query tiles of every query head of the group, from the diagonal to the
// end of the document (details at the kernel):
//   S  = Q Kᵀ        A = Q tile rows (LDS)          -> lane holds one key, 16 queries
//   dP = dO Vᵀ       A = dO tile rows (LDS)
//   dVᵀ += dOᵀ P     A = dOᵀ via ds_read_b64_tr_b16, B = P as computed (bf16)
//   dKᵀ += Qᵀ dS     A = Qᵀ via ds_read_b64_tr_b16, B = dS as computed (bf16)
// dQ kernel: the forward's layout (a wave owns 32 queries, Qᵀ and dOᵀ fragments in registers),
// key tiles of 64 double-buffered in LDS:
//   Sᵀ = K Qᵀ, dPᵀ = V dOᵀ (A = K / V tile rows), dQᵀ += Kᵀ dSᵀ (A = Kᵀ via transposing reads).
#include "cfa_device.h"

namespace cfa {

// ------------------------------------------------------------------ D = rowsum(dO ∘ O) − dLSE
// 16 lanes per (token, head) row of 128 (8 lanes for d = 64), 16 bytes per lane. A gradient
// dLSE_i flowing into the row log-sum-exp adds P_ij·dLSE_i to dS_ij (∂LSE_i/∂S_ij = P_ij), which
// is the same as lowering D_i by dLSE_i.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                      const float* __restrict__ dlse, float* __restrict__ delta,
                                                      int total_tokens, int hq) {
  constexpr int LPR = D / 8;  // lanes per row
  const long row = (long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  const long rows = (long)total_tokens * hq;
  float acc = 0.f;
  if (row < rows) {
    const i32x4 a = *(const i32x4*)(o + row * D + sub * 8);
    const i32x4 b = *(const i32x4*)(dout + row * D + sub * 8);
    const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && sub == 0) {
    const int t = (int)(row / hq), h = (int)(row % hq);
    const size_t i = (size_t)h * total_tokens + t;
    delta[i] = dlse ? acc - dlse[i] : acc;
  }
}

template <int D>
struct BwdTile {
  using S = SwzTile<D>;                     // tiles read row-wise and transposed (cfa_device.h)
  static constexpr int RSTR = S::STR;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
};

// ------------------------------------------------------------------ dK / dV, wave pairs
// 2·NP waves own 32·NP keys of one kv head, as NP pairs of 32 keys (d = 64 and 128: 4 pairs, two
// waves per SIMD; d = 256: 2 pairs, one wave per SIMD with twice the registers). In a pair, the "P wave" (w < NP)
// holds K and computes S = Q Kᵀ, P = exp(S − LSE), dVᵀ += dOᵀ P; the "dS wave" (w + NP) holds V
// and computes dP = dO Vᵀ, dS = P (dP − D), dKᵀ += Qᵀ dS with the bf16 P that its partner left
// in LDS one step earlier. A step is 64 queries (d = 64, 128; 32 for d = 256) of one query head,
// taken as two 32-query blocks: the longer step leaves the copies of the next one more time. Running the dS wave one step behind removes every wait between the
// two inside a step; the two waves of a pair sit on the same SIMD, so one wave's exponentials
// and packing overlap the other's matrix products. Each wave holds one accumulator (dVᵀ or
// dKᵀ) and one operand set (K or V), which is what brings two waves per SIMD within the
// register file. Staging buffers: step i (Q, dO tiles, LSE·log2 e, D) lives in buffer i mod 3
// and P of step i in exchange buffer i mod 3, so the loop is unrolled three times and every
// buffer is a distinct static array (no aliasing between the copies in flight and the reads).
//
// Head split (n_split > 1, for grids too small to fill the chip, e.g. MQA): workgroup
// (item, split, kv head) runs only query heads [G·split/n_split, G·(split+1)/n_split) of the group
// and writes its unscaled fp32 dKᵀ / dVᵀ sums to part_dk / part_dv [n_split][T][hkv][d]; the
// reduce kernel adds the splits in index order (deterministic) and writes bf16.
//
// Cross-attention (CROSS = true): the work list is built on the key documents, `qdoc[doc]` gives
// the query rows, off = Lk - Lq and key j is seen by query i iff j <= i + off; LSE = -inf (a query
// that sees no key) is read as +inf so that its P is 0. total_tokens counts query rows (LSE, D),
// total_k key rows (partial sums).
template <int D, int NP, bool CROSS, bool SPLIT>
__global__ __launch_bounds__(128 * NP, 1) void attn_bwd_dkdv_pair_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, Plan plan, int total_tokens, int hq, int hkv,
    float scale, int causal, int n_split, float* __restrict__ part_dk, float* __restrict__ part_dv,
    const int2* __restrict__ qdoc, int total_k) {
  using C = BwdTile<D>;
  constexpr int KT = 32 * NP;                     // keys per workgroup
  constexpr int QBS = D <= 128 ? 2 : 1;           // 32-query blocks per step (a longer step hides the copies)
  constexpr int BM = 32 * QBS;                    // queries per step
  constexpr int TILE = BM * C::RSTR;              // 16 KB
  constexpr int STAGE = 2 * TILE + 2 * BM * 4;    // Q, dO, LSE·log2 e, D
  constexpr int XP = NP * QBS * 2 * 64;           // i32x4 per exchange buffer: bf16 P [pair][qb][u][lane]
  constexpr int SB = D == 256 ? 4 : C::DS;        // k-steps per operand batch
  constexpr int DBC = D == 256 ? 4 : C::DB;       // d blocks per transposed-read batch
  __shared__ __attribute__((aligned(16))) char st_a[STAGE];
  __shared__ __attribute__((aligned(16))) char st_b[STAGE];
  __shared__ __attribute__((aligned(16))) char st_c[STAGE];
  __shared__ i32x4 xp_a[XP];
  __shared__ i32x4 xp_b[XP];
  __shared__ i32x4 xp_c[XP];

  const int ns = SPLIT ? n_split : 1;             // the unsplit instantiation keeps plain indexing
  const int p = blockIdx.x / (hkv * ns), g = blockIdx.x % hkv, split = SPLIT ? (blockIdx.x / hkv) % ns : 0;
  int s0, L, t, doc;
  if (!decode_item(plan, p, KT, false, s0, L, t, &doc)) return;
  // key rows [s0, s0 + L); query rows [q_s0, q_s0 + Lq); off = L - Lq (0 for self-attention)
  int q_s0 = s0, Lq = L;
  if constexpr (CROSS) {
    const int2 qd = qdoc[doc];
    q_s0 = qd.x;
    Lq = qd.y;
  }
  const int off = CROSS ? L - Lq : 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, half = lane >> 5;
  const int pair = w % NP;
  const bool ds_wave = w >= NP;
  const int G = hq / hkv;
  const int h_lo = SPLIT ? g * G + (G * split) / ns : g * G;  // this split's query heads
  const int n_h = SPLIT ? g * G + (G * (split + 1)) / ns - h_lo : G;
  const int kw0 = t * KT + 32 * pair;             // first doc-local key of this pair
  const int mykey = kw0 + (lane & 31);
  const float sl2 = scale * LOG2E;
  const SwzOffsets<D> so(lane);

  // B operand rows (lane: key mykey, d = 16s + 8·half ..): K for the P wave, V for the dS wave
  bf16x8 kv[C::DS];
  {
    const bool ok = mykey < L;
    const __bf16* src = ds_wave ? v : k;
    const size_t ro = ((size_t)(s0 + (ok ? mykey : 0)) * hkv + g) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < C::DS; ++s)
      kv[s] = __builtin_bit_cast(bf16x8, ok ? *(const i32x4*)(src + ro + 16 * s) : i32x4{0, 0, 0, 0});
  }
  f32x16 acc[C::DB];                              // dVᵀ (P wave) or dKᵀ (dS wave)
#pragma unroll
  for (int b = 0; b < C::DB; ++b) acc[b] = f32x16{};

  const int q_begin = causal ? (CROSS ? max(0, t * KT - off) : t * KT) : 0;
  const int n_qt = CROSS ? max(0, (Lq - q_begin + BM - 1) / BM) : (L - q_begin + BM - 1) / BM;
  const int n_steps = n_qt * n_h;
  const int wave_first_q = causal ? kw0 - off : 0;

  // Step st -> buffer: P waves copy the Q tile, dS waves the dO tile (direct global -> LDS);
  // lanes 0..31 of wave 0 fetch LSE and D into registers, written by stage_finish. Rows past
  // the document end are clamped into it and masked (P = 0).
  float lreg = 0.f, dreg = 0.f;
  // d = 64: 144-byte padded rows (no swizzle), staged through registers: the role's NP waves
  // load the BM × D tile as 16-byte chunks (TR per lane) and stage_finish writes them
  constexpr int TR = D < 128 ? BM * D / 8 / (64 * NP) : 1;
  i32x4 treg[TR];
  auto stage = [&](int st, char* buf) {
    const int h = h_lo + st / n_qt;
    const int q0 = q_begin + (st % n_qt) * BM;
    const __bf16* src = ds_wave ? dout : q;
    if constexpr (D >= 128) {
      stage_rows_lds<BM, NP, D>(buf + (ds_wave ? TILE : 0), (const char*)(src + ((size_t)(q_s0 + q0) * hq + h) * D),
                                (uint32_t)hq * D * 2, Lq - 1 - q0, pair, lane);
    } else {
#pragma unroll
      for (int i = 0; i < TR; ++i) {
        const int c = pair * 64 + lane + 64 * NP * i, row = c / (D / 8), col = c % (D / 8);
        treg[i] = *(const i32x4*)(src + ((size_t)(q_s0 + q0 + min(row, Lq - 1 - q0)) * hq + h) * D + 8 * col);
      }
    }
    if (threadIdx.x < BM) {
      const size_t li = (size_t)h * total_tokens + q_s0 + min(q0 + (int)threadIdx.x, Lq - 1);
      lreg = lse[li];
      if (CROSS && lreg == -INFINITY) lreg = INFINITY;
      dreg = delta[li];
    }
  };
  auto stage_finish = [&](char* buf) {
    if constexpr (D < 128) {
#pragma unroll
      for (int i = 0; i < TR; ++i) {
        const int c = pair * 64 + lane + 64 * NP * i;
        *(i32x4*)(buf + (ds_wave ? TILE : 0) + C::S::chunk(c / (D / 8), c % (D / 8))) = treg[i];
      }
    }
    if (threadIdx.x < BM) {
      float* lb = (float*)(buf + 2 * TILE);
      lb[threadIdx.x] = lreg * LOG2E;
      lb[BM + threadIdx.x] = -dreg;               // -D: the dP accumulator starts from it
    }
  };
  auto active = [&](int st) {
    const int q0 = q_begin + (st % n_qt) * BM;
    return q0 + BM - 1 >= wave_first_q && kw0 < L;
  };

  // P wave, step st: per 32-query block, S, P (bf16, to the exchange buffer and the dV product),
  // dVᵀ += dOᵀ P
  auto step_p = [&](int st, const char* buf, i32x4* xw) __attribute__((always_inline)) {
    const int q0 = q_begin + (st % n_qt) * BM;
    const char* ob = buf + TILE;
    const f32x4* l2 = (const f32x4*)(buf + 2 * TILE);
    const bool masked = (causal && q0 + off < kw0 + 31) || q0 + BM > Lq;   // wave-uniform
#pragma unroll
    for (int qb = 0; qb < QBS; ++qb) {
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int sc = 0; sc < C::DS; sc += SB) {
        i32x4 fq[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) fq[s] = *(const i32x4*)(buf + 32 * qb * C::RSTR + so.row[sc + s]);
#pragma unroll
        for (int s = 0; s < SB; ++s) sacc = mfma32(as_bf16x8(fq[s]), kv[sc + s], sacc);
        if constexpr (D == 128) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        }
      }
      // masked scores -> -inf, so P = 2^(s·c − LSE·log2 e) is exactly 0 there
      if (masked) {
        // element j holds query qb0 + c_j, c_j = 8(j/4) + j%4: masked below lo (causal: the
        // query precedes this lane's key) or above hi (past the document end)
        const int qb0 = q0 + 32 * qb + 4 * half;
        const int lo = causal ? mykey - off - qb0 : -1, hi = Lq - 1 - qb0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int c = 8 * (j >> 2) + (j & 3);
          if ((c < lo) | (c > hi)) sacc[j] = -INFINITY;
        }
      }
      i32x4 pw[2];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {            // rows 32·qb + 8·jj + 4·half + u
        const f32x4 lr = l2[8 * qb + 2 * jj + half];
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = exp2_fast(fmaf(sacc[4 * jj + u], sl2, -lr[u]));
        pw[jj >> 1][2 * (jj & 1)] = (int)pack_bf16x2(x[0], x[1]);
        pw[jj >> 1][2 * (jj & 1) + 1] = (int)pack_bf16x2(x[2], x[3]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) xw[((pair * QBS + qb) * 2 + u) * 64 + lane] = pw[u];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int rb = (32 * qb + 16 * kk) * C::RSTR;
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw[kk]);
#pragma unroll
        for (int dc = 0; dc < C::DB; dc += DBC) {
          bf16x8 ao[DBC];
#pragma unroll
          for (int i = 0; i < DBC; ++i)
            ao[i] = concat_tr(lds_read_tr16(ob + rb + so.tr0[dc + i]), lds_read_tr16(ob + rb + so.tr1[dc + i]));
#pragma unroll
          for (int i = 0; i < DBC; ++i) acc[dc + i] = mfma32(ao[i], pf, acc[dc + i]);
        }
      }
    }
  };

  // dS wave, step st (one iteration after its P wave): per 32-query block, dP − D (the product
  // accumulates onto −D, read from the stage as the accumulator's start), dS = P (dP − D) with the
  // bf16 P of its partner, dKᵀ += Qᵀ dS
  auto step_ds = [&](int st, const char* buf, const i32x4* xr) __attribute__((always_inline)) {
    const char* ob = buf + TILE;
    const f32x4* db = (const f32x4*)(buf + 2 * TILE + BM * 4);
#pragma unroll
    for (int qb = 0; qb < QBS; ++qb) {
      f32x16 pacc;                                // element 4jj + u: query 32qb + 8jj + 4·half + u
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 nd = db[8 * qb + 2 * jj + half];
#pragma unroll
        for (int u = 0; u < 4; ++u) pacc[4 * jj + u] = nd[u];
      }
#pragma unroll
      for (int sc = 0; sc < C::DS; sc += SB) {
        i32x4 fo[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) fo[s] = *(const i32x4*)(ob + 32 * qb * C::RSTR + so.row[sc + s]);
#pragma unroll
        for (int s = 0; s < SB; ++s) pacc = mfma32(as_bf16x8(fo[s]), kv[sc + s], pacc);
        if constexpr (D == 128) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        }
      }
      bf16x8 sf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const i32x4 pw = xr[((pair * QBS + qb) * 2 + u) * 64 + lane];
        i32x4 us;
#pragma unroll
        for (int e = 0; e < 4; ++e) {             // word e: rows of jj = 2u + e/2, values (e%2)·2, +1
          const int jj = 2 * u + (e >> 1), j0 = 4 * jj + 2 * (e & 1);
          const float p0 = __builtin_bit_cast(float, (uint32_t)pw[e] << 16);
          const float p1 = __builtin_bit_cast(float, (uint32_t)pw[e] & 0xFFFF0000u);
          us[e] = (int)pack_bf16x2(p0 * pacc[j0], p1 * pacc[j0 + 1]);
        }
        sf[u] = __builtin_bit_cast(bf16x8, us);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int rb = (32 * qb + 16 * kk) * C::RSTR;
#pragma unroll
        for (int dc = 0; dc < C::DB; dc += DBC) {
          bf16x8 aq[DBC];
#pragma unroll
          for (int i = 0; i < DBC; ++i)
            aq[i] = concat_tr(lds_read_tr16(buf + rb + so.tr0[dc + i]), lds_read_tr16(buf + rb + so.tr1[dc + i]));
#pragma unroll
          for (int i = 0; i < DBC; ++i) acc[dc + i] = mfma32(aq[i], sf[kk], acc[dc + i]);
        }
      }
    }
  };

  // Iteration i: copy step i+1 into `nxt`; P waves run step i on `cur`; dS waves run step i-1
  // on `prv`. The conditions depend on i only, so every wave meets the same barriers.
  auto iter = [&](int i, char* cur, char* prv, char* nxt, i32x4* xcur, const i32x4* xprv)
      __attribute__((always_inline)) {
    if (i + 1 < n_steps) stage(i + 1, nxt);
    if (!ds_wave) {
      if (i < n_steps && active(i)) step_p(i, cur, xcur);
    } else {
      if (i >= 1 && active(i - 1)) step_ds(i - 1, prv, xprv);
    }
    if (i + 1 < n_steps) stage_finish(nxt);
    wait_vmem();
    __syncthreads();
  };

  if (n_steps > 0) {
    stage(0, st_a);
    stage_finish(st_a);
  }
  wait_vmem();
  __syncthreads();
  for (int i = 0; i <= n_steps; i += 3) {
    iter(i, st_a, st_c, st_b, xp_a, xp_c);
    if (i + 1 <= n_steps) iter(i + 1, st_b, st_a, st_c, xp_b, xp_a);
    if (i + 2 <= n_steps) iter(i + 2, st_c, st_b, st_a, xp_c, xp_b);
  }

  // dS wave: dK = scale·dKᵀ; P wave: dV (lane: key mykey, d = 32 db + 8 jg + 4·half + 0..3)
  if (mykey < L) {
    const size_t row = ((size_t)(s0 + mykey) * hkv + g) * D + 4 * half;
    if (SPLIT) {
      float* dst = (ds_wave ? part_dk : part_dv) + (size_t)split * (CROSS ? total_k : total_tokens) * hkv * D + row;
#pragma unroll
      for (int dbk = 0; dbk < C::DB; ++dbk)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg)
          *(f32x4*)(dst + 32 * dbk + 8 * jg) =
              f32x4{acc[dbk][4 * jg], acc[dbk][4 * jg + 1], acc[dbk][4 * jg + 2], acc[dbk][4 * jg + 3]};
    } else {
      const float f = ds_wave ? scale : 1.f;
      __bf16* dst = (ds_wave ? dk : dv) + row;
#pragma unroll
      for (int dbk = 0; dbk < C::DB; ++dbk)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          i32x2 u;
          u.x = (int)pack_bf16x2(acc[dbk][4 * jg] * f, acc[dbk][4 * jg + 1] * f);
          u.y = (int)pack_bf16x2(acc[dbk][4 * jg + 2] * f, acc[dbk][4 * jg + 3] * f);
          *(i32x2*)(dst + 32 * dbk + 8 * jg) = u;
        }
    }
  }
}

// Sum of the head-split partial sums in split order: dK = scale·Σ_s part_dk[s], dV = Σ_s part_dv[s]
// (bf16). One lane per 4 consecutive elements. Nothing is written when the plan flagged a
// malformed cu_seqlens (every document empty: no partial sum was produced).
__global__ __launch_bounds__(256) void dkdv_split_reduce_kernel(const float* __restrict__ part_dk,
                                                                const float* __restrict__ part_dv,
                                                                __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                                                                long n, int n_split, float scale,
                                                                const int* __restrict__ flag) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n || *flag != 0) return;
  f32x4 a = *(const f32x4*)(part_dk + i), b = *(const f32x4*)(part_dv + i);
  for (int sp = 1; sp < n_split; ++sp) {
    a += *(const f32x4*)(part_dk + (size_t)sp * n + i);
    b += *(const f32x4*)(part_dv + (size_t)sp * n + i);
  }
  *(i32x2*)(dk + i) = i32x2{(int)pack_bf16x2(a[0] * scale, a[1] * scale), (int)pack_bf16x2(a[2] * scale, a[3] * scale)};
  *(i32x2*)(dv + i) = i32x2{(int)pack_bf16x2(b[0], b[1]), (int)pack_bf16x2(b[2], b[3])};
}



// ------------------------------------------------------------------ dQ
// Cross-attention (CROSS = true): work list on the query documents, `kdoc[doc]` = key rows.
// HPB query heads of one kv group per workgroup (4 waves each, 32 queries per wave): the K/V
// tiles are staged once for all of them (HPB = 2 halves the copies per product).
template <int D, bool CROSS, int HPB>
__global__ __launch_bounds__(256 * HPB, D == 256 ? 1 : 2 / HPB) void attn_bwd_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dq, Plan plan, int total_tokens, int hq, int hkv, float scale, int causal,
    const int2* __restrict__ kdoc) {
  static_assert(HPB == 1 || D == 128, "two heads per workgroup at d = 128 only");
  using C = BwdTile<D>;
  constexpr int BN = 64;
  constexpr int TILE = BN * C::RSTR;
  constexpr int STAGE = 2 * TILE;
  constexpr int CH = BN * D / 8;
  constexpr int PT = CH / 256;
  constexpr int SB = D == 256 ? 4 : C::DS;       // k-steps per operand batch
  // two separate buffers so that the compiler sees the copy into one never aliases the other
  __shared__ __attribute__((aligned(16))) char lds_a[STAGE];
  __shared__ __attribute__((aligned(16))) char lds_b[STAGE];

  const int n_hb = hq / HPB;
  const int p = blockIdx.x / n_hb, hb = blockIdx.x % n_hb;
  int s0, L, t, doc;
  if (!decode_item(plan, p, 128, true, s0, L, t, &doc)) return;
  int k_s0 = s0, Lk = L;                         // key rows (cross-attention: their own documents)
  if constexpr (CROSS) {
    const int2 kd = kdoc[doc];
    k_s0 = kd.x;
    Lk = kd.y;
  }
  const int off = CROSS ? Lk - L : 0;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5;
  const int h = hb * HPB + (w >> 2);             // this wave's query head
  const int g = h / (hq / hkv);
  const int wr0 = t * 128 + 32 * (w & 3);
  const int qrow = wr0 + (lane & 31);
  const int kv_end = causal ? (CROSS ? min(Lk, min(L, (t + 1) * 128) + off) : min(L, (t + 1) * 128)) : Lk;
  const int n_kt = (CROSS && kv_end <= 0) ? 0 : (kv_end + BN - 1) / BN;
  const int wave_last_key = causal ? (CROSS ? min(Lk, min(L, wr0 + 32) + off) : min(L, wr0 + 32)) - 1 : Lk - 1;
  const float sl2 = scale * LOG2E;
  const SwzOffsets<D> so(lane);

  bf16x8 qf[C::DS], of[C::DS];
  float lse2 = INFINITY, dl = 0.f;
  {
    const bool ok = qrow < L;
    const size_t ro = ((size_t)(s0 + (ok ? qrow : 0)) * hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, ok ? *(const i32x4*)(q + ro + 16 * s) : i32x4{0, 0, 0, 0});
      of[s] = __builtin_bit_cast(bf16x8, ok ? *(const i32x4*)(dout + ro + 16 * s) : i32x4{0, 0, 0, 0});
    }
    if (ok) {
      lse2 = lse[(size_t)h * total_tokens + s0 + qrow] * LOG2E;
      if (CROSS && lse2 == -INFINITY) lse2 = INFINITY;      // a row that sees no key: P = 0
      dl = delta[(size_t)h * total_tokens + s0 + qrow];
    }
  }
  f32x16 dqa[C::DB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) dqa[b] = f32x16{};

  // K/V tile kt -> LDS buffer; keys past kv_end are clamped into the document (masked, P = 0)
  auto stage = [&](int kt, char* kb) {
    const int k0 = kt * BN;
    char* vb = kb + TILE;
    if constexpr (D >= 128) {
      const size_t row0 = ((size_t)(k_s0 + k0) * hkv + g) * D;
      const uint32_t stride = (uint32_t)hkv * D * 2;
      stage_rows_lds<BN, 4 * HPB, D>(kb, (const char*)(k + row0), stride, kv_end - 1 - k0, w, lane);
      stage_rows_lds<BN, 4 * HPB, D>(vb, (const char*)(v + row0), stride, kv_end - 1 - k0, w, lane);
    } else {
      i32x4 kreg[PT], vreg[PT];
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int key = c / (D / 8), col = c % (D / 8);
        const size_t eo = ((size_t)(k_s0 + min(k0 + key, kv_end - 1)) * hkv + g) * D + col * 8;
        kreg[i] = *(const i32x4*)(k + eo);
        vreg[i] = *(const i32x4*)(v + eo);
      }
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int key = c / (D / 8), col = c % (D / 8);
        *(i32x4*)(kb + C::S::chunk(key, col)) = kreg[i];
        *(i32x4*)(vb + C::S::chunk(key, col)) = vreg[i];
      }
    }
  };

  auto iter = [&](int kt, const char* kb, char* nxt) __attribute__((always_inline)) {
    const int k0 = kt * BN;
    if (kt + 1 < n_kt) stage(kt + 1, nxt);
    if (k0 <= wave_last_key) {
      const char* vb = kb + TILE;
      const bool need_mask = causal ? (k0 + BN - 1 > wr0 + off) : (k0 + BN > Lk);
      bf16x8 sf[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // Sᵀ = K Qᵀ and dPᵀ = V dOᵀ for one 32-key block, operand rows read as a batch (d = 256:
        // four batches of 4 k-steps)
        f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
        for (int sc = 0; sc < C::DS; sc += SB) {
          i32x4 fk[SB], fv[SB];
#pragma unroll
          for (int s = 0; s < SB; ++s) {
            fk[s] = *(const i32x4*)(kb + b * 32 * C::RSTR + so.row[sc + s]);
            fv[s] = *(const i32x4*)(vb + b * 32 * C::RSTR + so.row[sc + s]);
          }
#pragma unroll
          for (int s = 0; s < SB; ++s) {
            sacc = mfma32(as_bf16x8(fk[s]), qf[sc + s], sacc);
            pacc = mfma32(as_bf16x8(fv[s]), of[sc + s], pacc);
          }
          if constexpr (D <= 128) {
            // keep ~4 operand reads in flight ahead of the products (occupancy 2 register budget)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < C::DS - 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
        }
        // masked scores -> -inf (wave-uniform branch: diagonal or document-end tiles only),
        // so P = 2^(s·c − LSE·log2 e) is exactly 0 there
        if (need_mask) {
          // keys above lim are masked; element j holds key k0 + 32b + 4·half + 8(j/4) + j%4
          const int r = (causal ? qrow + off : Lk - 1) - (k0 + 32 * b + 4 * half);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (8 * (j >> 2) + (j & 3) > r) sacc[j] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const float x0 = exp2_fast(fmaf(sacc[j], sl2, -lse2));
          const float x1 = exp2_fast(fmaf(sacc[j + 1], sl2, -lse2));
          const int fi = 2 * b + (j >> 3);
          i32x4 us = __builtin_bit_cast(i32x4, sf[fi]);
          us[(j & 7) >> 1] = (int)pack_bf16x2(x0 * (pacc[j] - dl), x1 * (pacc[j + 1] - dl));
          sf[fi] = __builtin_bit_cast(bf16x8, us);
        }
      }
      // dQᵀ += Kᵀ dSᵀ (Kᵀ through transposing reads, batched per kk)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int rb = (32 * (kk >> 1) + 16 * (kk & 1)) * C::RSTR;
        bf16x8 ak[C::DB];
#pragma unroll
        for (int dbk = 0; dbk < C::DB; ++dbk)
          ak[dbk] = concat_tr(lds_read_tr16(kb + rb + so.tr0[dbk]), lds_read_tr16(kb + rb + so.tr1[dbk]));
#pragma unroll
        for (int dbk = 0; dbk < C::DB; ++dbk) dqa[dbk] = mfma32(ak[dbk], sf[kk], dqa[dbk]);
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (n_kt > 0) stage(0, lds_a);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    iter(kt, lds_a, lds_b);
    if (kt + 1 < n_kt) iter(kt + 1, lds_b, lds_a);
  }

  if (qrow < L) {
    __bf16* dst = dq + ((size_t)(s0 + qrow) * hq + h) * D + 4 * half;
#pragma unroll
    for (int dbk = 0; dbk < C::DB; ++dbk)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        i32x2 u;
        u.x = (int)pack_bf16x2(dqa[dbk][4 * jg] * scale, dqa[dbk][4 * jg + 1] * scale);
        u.y = (int)pack_bf16x2(dqa[dbk][4 * jg + 2] * scale, dqa[dbk][4 * jg + 3] * scale);
        *(i32x2*)(dst + 32 * dbk + 8 * jg) = u;
      }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_bwd_pre(const void* o, const void* dout, const float* dlse, float* delta, int total_tokens, int hq,
                          int d, hipStream_t stream) {
  const long rows = (long)total_tokens * hq;
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (d / 8);
  const long grid = (rows + rpb - 1) / rpb;
  if (d == 256)
    hipLaunchKernelGGL(bwd_pre_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, (const __bf16*)o,
                       (const __bf16*)dout, dlse, delta, total_tokens, hq);
  else if (d == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, (const __bf16*)o,
                       (const __bf16*)dout, dlse, delta, total_tokens, hq);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, (const __bf16*)o,
                       (const __bf16*)dout, dlse, delta, total_tokens, hq);
  return hipGetLastError();
}

template <int D, bool CROSS>
static hipError_t launch_dkdv_d(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* delta, void* dk, void* dv, const Plan& plan_any, const int* pref_base,
                                int T, int hq, int hkv, float scale, int causal, int n_split, float* part,
                                hipStream_t stream, const int2* qdoc, int Tk) {
  constexpr int NP = D == 256 ? 2 : 4;            // wave pairs per workgroup
  constexpr int KT = D == 256 ? 64 : 128;         // keys per workgroup
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(KT) * (plan.n_docs + 1);
  const long items = (long)(Tk + KT - 1) / KT + plan.n_docs;   // key tiles (plan on the key documents)
  {
    const long grid = items * hkv * n_split;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const long n = (long)Tk * hkv * D;
    float* pdk = n_split > 1 ? part : nullptr;
    float* pdv = n_split > 1 ? part + (size_t)n_split * n : nullptr;
    if (n_split > 1)
      hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<D, NP, CROSS, true>), dim3((unsigned)grid), dim3(128 * NP), 0,
                         stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, lse, delta,
                         (__bf16*)dk, (__bf16*)dv, plan, T, hq, hkv, scale, causal, n_split, pdk, pdv, qdoc, Tk);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<D, NP, CROSS, false>), dim3((unsigned)grid), dim3(128 * NP), 0,
                         stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, lse, delta,
                         (__bf16*)dk, (__bf16*)dv, plan, T, hq, hkv, scale, causal, 1, pdk, pdv, qdoc, Tk);
    if (n_split > 1 && n > 0)
      hipLaunchKernelGGL(dkdv_split_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, pdk,
                         pdv, (__bf16*)dk, (__bf16*)dv, n, n_split, scale, plan.header);
  }
  return hipGetLastError();
}

int dkdv_head_split(int hq, int hkv, int d) {
  (void)d;
  const int G = hq / hkv;
  return std::max(1, std::min(G, 8 / hkv));
}

template <int D>
static hipError_t launch_dq_d(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              const float* delta, void* dq, const Plan& plan, int T, int hq, int hkv, float scale,
                              int causal, hipStream_t stream, const int2* kdoc) {
  const long items = (long)(T + 127) / 128 + plan.n_docs;
  // two query heads of a kv group per workgroup where the group has an even size (d = 128)
  constexpr int HP2 = D == 128 ? 2 : 1;
  const int hpb = (D == 128 && (hq / hkv) % 2 == 0) ? 2 : 1;
  auto kern = hpb == 2 ? (kdoc ? attn_bwd_dq_kernel<D, true, HP2> : attn_bwd_dq_kernel<D, false, HP2>)
                       : (kdoc ? attn_bwd_dq_kernel<D, true, 1> : attn_bwd_dq_kernel<D, false, 1>);
  const long grid = items * (hq / hpb);
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256 * hpb), 0, stream, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, (const __bf16*)dout, lse, delta, (__bf16*)dq, plan, T, hq, hkv, scale, causal,
                     kdoc);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* delta, void* dk, void* dv, const Plan& plan_any, const int* pref_base, int T,
                           int hq, int hkv, int d, float scale, int causal, int n_split, float* part,
                           hipStream_t stream, const int2* qdoc, int Tk) {
  if (!qdoc) Tk = T;
#define CFA_DKDV(DD, NS, PP)                                                                                  \
  (qdoc ? launch_dkdv_d<DD, true>(q, k, v, dout, lse, delta, dk, dv, plan_any, pref_base, T, hq, hkv, scale, causal, \
                                  NS, PP, stream, qdoc, Tk)                                                    \
        : launch_dkdv_d<DD, false>(q, k, v, dout, lse, delta, dk, dv, plan_any, pref_base, T, hq, hkv, scale,   \
                                   causal, NS, PP, stream, qdoc, Tk))
  if (d == 128) return CFA_DKDV(128, n_split, part);
  if (d == 256) return CFA_DKDV(256, n_split, part);
  return CFA_DKDV(64, 1, nullptr);
#undef CFA_DKDV
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         const float* delta, void* dq, const Plan& plan_any, const int* pref_base, int T, int hq,
                         int hkv, int d, float scale, int causal, hipStream_t stream, const int2* kdoc) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(128) * (plan.n_docs + 1);
  if (d == 128) return launch_dq_d<128>(q, k, v, dout, lse, delta, dq, plan, T, hq, hkv, scale, causal, stream, kdoc);
  if (d == 256) return launch_dq_d<256>(q, k, v, dout, lse, delta, dq, plan, T, hq, hkv, scale, causal, stream, kdoc);
  return launch_dq_d<64>(q, k, v, dout, lse, delta, dq, plan, T, hq, hkv, scale, causal, stream, kdoc);
}

}  // namespace cfa

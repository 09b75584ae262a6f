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
//
// dQ inside this pass (FQ, self-attention at d = 128): dQ_i = scale·Σ_j dS_ij k_j is the one
// gradient that sums over key tiles, which different workgroups own. Each workgroup adds its key
// tile's part of every (query head, 64-query tile) block into an fp32 sum in the workspace, and
// the tiles of a document add in key-tile order 0, 1, 2, ...: tile t waits until tile t − 1 has
// added (a count per block piece), so the sum has one fixed order and reruns are bit-identical.
// Tile 0 writes the block, the last tile that sees it (the diagonal one when causal) writes dQ
// as bf16. To keep tile t just behind tile t − 1, every key tile of a document walks the same
// query tiles in the same order: from the document end down to its own diagonal, query heads
// inner. The part itself, dQᵀ = Kᵀ dSᵀ over the workgroup's 128 keys, is split over the 8 waves by
// head-dim columns (16 each, v_mfma_f32_16x16x32_bf16): A = Kᵀ (registers, read once from a
// staged K tile), B = dSᵀ, which the dS wave writes over its partner's P in the exchange tile
// (rows = keys), so no extra LDS is needed. Waits: a tile waits only on the tile of its
// document handed out just before it, which a running workgroup holds (see the claim below),
// so every wait ends; each one is bounded anyway and raises bit 3 of the plan flag if it gives up.
struct FusedDq {
  float* acc;                 // [T][hq][D] fp32 running dQ / scale of the key tiles added so far
  int* cnt;                   // [t_pad/32][hq][8]: key tiles that have added into each 16-column piece
  __bf16* dq;                 // dQ output [T][hq][D]
  const int* padoff;          // plan: first 32-token block of each document
  int* header;                // plan header: [0] flag, [2] chain counter, [16, 48) per-XCD claim words
  i32x4* kt;                  // [grid][8 waves][4 pairs][64 lanes]: each workgroup's Kᵀ operands
  unsigned long long acc_bytes;
  int n_chains;               // documents × kv heads × head splits
};

constexpr int FUSED_MAX_GRID = 256;           // persistent workgroups (Kᵀ operand slots) at most

constexpr int SPIN_LIMIT = 1 << 20;          // ~1 s of polling: far beyond any legitimate wait
constexpr int SC1 = 16;                       // buffer access cache policy: device scope (sc1)
constexpr int CLAIM_END = 0x7fffffff;

// Index of the XCD (accelerator complex die) the calling wave runs on; the CUs of one XCD share
// one L2 cache.
__device__ inline int xcc_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

// Byte offset of bf16 column c (c % 4 == 0) of row r in a 128-row × 64-column exchange tile with
// 128-byte rows whose 32-byte units are XOR-swizzled by f(r): the transposing reads of the dQ
// product (rows 8g + 0..3 of four lane groups, 32 bytes each) then fall into distinct bank
// groups within each half of the wave.
__device__ inline int xt_off(int r, int c) {
  const int f = ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
  return r * 128 + ((((c >> 4) ^ f) & 3) << 5) + ((c & 15) << 1);
}

typedef __attribute__((address_space(3))) char lds_char;

// The exchange tile's LDS address as an opaque scalar: the three exchange buffers are then
// addressed through one set of lane offsets (plus immediates) instead of a set per buffer.
__device__ inline lds_char* lds_opaque(const void* p) {
  uint32_t a = (uint32_t)(uintptr_t)(const lds_char*)p;
  asm volatile("" : "+s"(a));
  return (lds_char*)(uintptr_t)a;
}

// The lane index as a value the compiler cannot hoist: addresses derived from it are recomputed
// where they are used instead of being held in registers across the whole persistent loop.
__device__ inline int lane_here() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// Wait until *cnt >= target (device-coherent polling); bounded. A wait that gives up raises bit 3
// of the plan flag, after which every wait returns at once (the results are then invalid, and the
// pass still ends promptly).
__device__ inline void wait_count(const int* cnt, int target, int* flag) {
  for (int n = 0;; ++n) {
    const int c = __builtin_amdgcn_readfirstlane(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (c >= target) return;
    if ((n & 255) == 255 &&
        (__builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & 8))
      return;
    if (n >= SPIN_LIMIT) {
      if ((threadIdx.x & 63) == 0) atomicOr(flag, 8);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

template <int D, int NP>
struct DkdvLds {
  using C = BwdTile<D>;
  static constexpr int QBS = D <= 128 ? 2 : 1;
  static constexpr int BM = 32 * QBS;
  static constexpr int TILE = BM * C::RSTR;
  static constexpr int STAGE = 2 * TILE + 2 * BM * 4;   // Q, dO, LSE·log2 e, D
  static constexpr int XP = NP * QBS * 2 * 64;          // i32x4 per exchange buffer (16 KB at d = 128)
};

// One work item: 32·NP keys [t·32·NP, ...) of document `doc` (rows s0 .. s0 + L − 1), kv head g,
// head split `split`.
template <int D, int NP, bool CROSS, bool SPLIT, bool FQ>
__device__ __forceinline__ void dkdv_item(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int total_tokens, int hq, int hkv, float scale, int causal,
    int n_split, float* __restrict__ part_dk, float* __restrict__ part_dv, const int2* __restrict__ qdoc,
    int total_k, const FusedDq& fq, int s0, int L, int t, int doc, int g, int split, char* st_a, char* st_b,
    char* st_c, i32x4* xp_a, i32x4* xp_b, i32x4* xp_c) {
  using C = BwdTile<D>;
  using X = DkdvLds<D, NP>;
  static_assert(!FQ || (D == 128 && NP == 4 && !CROSS), "dQ inside the pass: self-attention at d = 128");
  constexpr int KT = 32 * NP;                     // keys per workgroup
  constexpr int QBS = X::QBS;                     // 32-query blocks per step (a longer step hides the copies)
  constexpr int BM = X::BM;                       // queries per step
  constexpr int TILE = X::TILE;                   // 16 KB
  // k-steps per operand batch (fused mode: 4, leaving room for the dQ product's operands)
  constexpr int SB = (D == 256 || FQ) ? 4 : C::DS;
  constexpr int DBC = D == 256 ? 4 : C::DB;       // d blocks per transposed-read batch

  const int ns = SPLIT ? n_split : 1;             // the unsplit instantiation keeps plain indexing
  // key rows [s0, s0 + L); query rows [q_s0, q_s0 + Lq); off = L - Lq (0 for self-attention)
  int q_s0 = s0, Lq = L;
  if constexpr (CROSS) {
    const int2 qd = qdoc[doc];
    q_s0 = __builtin_amdgcn_readfirstlane(qd.x);
    Lq = __builtin_amdgcn_readfirstlane(qd.y);
  }
  const int off = CROSS ? L - Lq : 0;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5;
  const int pair = w % NP;
  const bool ds_wave = w >= NP;
  const int G = __builtin_amdgcn_readfirstlane(hq / hkv);
  // this split's query heads
  const int h_lo = SPLIT ? __builtin_amdgcn_readfirstlane(g * G + (G * split) / ns) : g * G;
  const int n_h = SPLIT ? __builtin_amdgcn_readfirstlane(g * G + (G * (split + 1)) / ns) - h_lo : G;
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
  const int n_qt =
      __builtin_amdgcn_readfirstlane(CROSS ? max(0, (Lq - q_begin + BM - 1) / BM) : (L - q_begin + BM - 1) / BM);
  const int n_steps = n_qt * n_h;
  const int wave_first_q = causal ? kw0 - off : 0;

  // A step's position (query head, first doc-local query of the step). Steps run the query heads
  // outer and the query tiles ascending from the diagonal; with dQ inside the pass, the query
  // tiles from the document end down to the diagonal with the heads inner (the order every key
  // tile of the document shares). The loop walks them one per iteration (uniform values, no
  // division per step).
  struct Pos {
    int h, q0;
  };
  const Pos first_pos{h_lo, FQ ? q_begin + (n_qt - 1) * BM : q_begin};
  const int q_end = q_begin + n_qt * BM;
  auto next_pos = [&](Pos ps) {
    if constexpr (FQ) {
      if (++ps.h == h_lo + n_h) {
        ps.h = h_lo;
        ps.q0 -= BM;
      }
    } else {
      ps.q0 += BM;
      if (ps.q0 >= q_end) {
        ps.q0 = q_begin;
        ++ps.h;
      }
    }
    return ps;
  };

  // dQ product A operands: element e of operand kk is K[key 32kk + 8(lane/16) + e][d 16w + lane%16]
  // (keys of this workgroup; zero past the document end), read transposed from the K tile staged
  // once into a free stage buffer and kept in this workgroup's slot of the workspace (registers
  // are full), from where each dQ part reloads them (coalesced, from L2)
  i32x4* const kt_slot = FQ ? fq.kt + (size_t)blockIdx.x * (8 * NP * 64) : nullptr;
  if constexpr (FQ) {
    stage_rows_lds<KT, 2 * NP, D>(st_c, (const char*)(k + ((size_t)(s0 + t * KT) * hkv + g) * D),
                                  (uint32_t)hkv * D * 2, L - 1 - t * KT, w, lane);
    wait_vmem();
    __syncthreads();
    const int gi = lane >> 4, ii = lane & 15;
#pragma unroll
    for (int kk = 0; kk < NP; ++kk) {
      const int r = 32 * kk + 8 * gi + (ii >> 2), col = 16 * w + 4 * (ii & 3);
      i32x4 u = __builtin_bit_cast(i32x4, concat_tr(lds_read_tr16(st_c + C::S::elem(r, col)),
                                                    lds_read_tr16(st_c + C::S::elem(r + 4, col))));
      const int key0 = t * KT + 32 * kk + 8 * gi;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key0 + e >= L) u[e >> 1] &= (e & 1) ? 0x0000FFFF : (int)0xFFFF0000;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(kt_slot + w * NP * 64, 0, NP * 64 * 16, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(u, rk, (kk * 64 + lane) * 16, 0, SC1);
    }
    wait_vmem();
    __syncthreads();
  }

  // exchange-tile lane offset (xt_off with the row swizzle folded in) of this lane's key row and
  // 32-byte unit u (u = 2qb + jj/2) of its P / dS words (+16 bytes for odd jj)
  auto xo = [&](int u) {
    const int l = lane_here();
    const int xrow = 32 * pair + (l & 31);
    const int fx = ((xrow >> 1) & 1) | (((xrow >> 3) & 1) << 1);
    return xrow * 128 + (((u ^ fx) & 3) << 5) + 8 * (l >> 5);
  };

  // Step st -> buffer: P waves copy the Q tile, dS waves the dO tile (direct global -> LDS);
  // lanes 0..31 of wave 0 fetch LSE and D into registers, written by stage_finish. Rows past
  // the document end are clamped into it and masked (P = 0).
  float lreg = 0.f, dreg = 0.f;
  // d = 64: 144-byte padded rows (no swizzle), staged through registers: the role's NP waves
  // load the BM × D tile as 16-byte chunks (TR per lane) and stage_finish writes them
  constexpr int TR = D < 128 ? BM * D / 8 / (64 * NP) : 1;
  i32x4 treg[TR];
  // d >= 128: the step tiles' copies (lane offsets fixed for the whole item)
  const RowCopies<BM, NP, D >= 128 ? D : 128> rc((uint32_t)hq * D * 2, pair, lane);
  auto stage = [&](Pos ps, char* buf) {
    const int h = ps.h, q0 = ps.q0;
    const __bf16* src = ds_wave ? dout : q;
    if constexpr (D >= 128) {
      // rows past the document end read zeros (those queries are masked: P = 0, dS = 0)
      rc.copy(buf + (ds_wave ? TILE : 0), src + ((size_t)(q_s0 + q0) * hq + h) * D, Lq - 1 - q0, pair);
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
  auto active = [&](Pos ps) { return ps.q0 + BM - 1 >= wave_first_q && kw0 < L; };

  // P wave, step st: per 32-query block, S, P (bf16, to the exchange buffer and the dV product),
  // dVᵀ += dOᵀ P
  auto step_p = [&](int q0, const char* buf, i32x4* xw) __attribute__((always_inline)) {
    const char* ob = buf + TILE;
    const f32x4* l2 = (const f32x4*)(buf + 2 * TILE);
    const bool masked = (causal && q0 + off < kw0 + 31) || q0 + BM > Lq;   // wave-uniform
#pragma unroll
    for (int qb = 0; qb < QBS; ++qb) {
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int sc = 0; sc < C::DS; sc += SB) {
        i32x4 fq_[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) fq_[s] = *(const i32x4*)(buf + 32 * qb * C::RSTR + so.row[sc + s]);
#pragma unroll
        for (int s = 0; s < SB; ++s) sacc = mfma32(as_bf16x8(fq_[s]), kv[sc + s], sacc);
        if constexpr (D == 128 && !FQ) {
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
      if constexpr (FQ) {                         // rows = keys: the dS wave overwrites them in place
        lds_char* xb = lds_opaque(xw);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(__attribute__((address_space(3))) i32x2*)(xb + xo(2 * qb + (jj >> 1)) + 16 * (jj & 1)) =
              i32x2{pw[jj >> 1][2 * (jj & 1)], pw[jj >> 1][2 * (jj & 1) + 1]};
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) xw[((pair * QBS + qb) * 2 + u) * 64 + lane] = pw[u];
      }
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
  // bf16 P of its partner, dKᵀ += Qᵀ dS; with dQ inside the pass, dS (bf16) replaces P in the
  // exchange tile for the dQ product
  auto step_ds = [&](const char* buf, i32x4* xr) __attribute__((always_inline)) {
    const char* ob = buf + TILE;
    const f32x4* db = (const f32x4*)(buf + 2 * TILE + BM * 4);
    lds_char* xb = FQ ? lds_opaque(xr) : nullptr;
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
        if constexpr (D == 128 && !FQ) {
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
        i32x4 pw;
        if constexpr (FQ) {
          typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
          const int o = xo(2 * qb + u);
          const i32x2 a = *(const lds_i32x2*)(xb + o);
          const i32x2 b = *(const lds_i32x2*)(xb + o + 16);
          pw = i32x4{a.x, a.y, b.x, b.y};
        } else {
          pw = xr[((pair * QBS + qb) * 2 + u) * 64 + lane];
        }
        i32x4 us;
#pragma unroll
        for (int e = 0; e < 4; ++e) {             // word e: rows of jj = 2u + e/2, values (e%2)·2, +1
          const int jj = 2 * u + (e >> 1), j0 = 4 * jj + 2 * (e & 1);
          const float p0 = __builtin_bit_cast(float, (uint32_t)pw[e] << 16);
          const float p1 = __builtin_bit_cast(float, (uint32_t)pw[e] & 0xFFFF0000u);
          us[e] = (int)pack_bf16x2(p0 * pacc[j0], p1 * pacc[j0 + 1]);
        }
        sf[u] = __builtin_bit_cast(bf16x8, us);
        if constexpr (FQ) {                       // each lane rewrites exactly the words it read
          typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
          const int o = xo(2 * qb + u);
          *(lds_i32x2*)(xb + o) = i32x2{us[0], us[1]};
          *(lds_i32x2*)(xb + o + 16) = i32x2{us[2], us[3]};
        }
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

  // dQ part of step s for this wave's 16 head-dim columns 16w .. 16w + 15 over the 64 queries of
  // the step, from the dSᵀ tile `xt` of that step: wait for the previous key tile's part, add this
  // tile's, hand over (or write dQ). Lane l holds columns 16w + 4(l/16) + 0..3 of query row
  // q0 + 16·sb + l%16 (sub-block sb of 16 queries).
  auto dq_phase = [&](Pos ps, const void* xt_buf) __attribute__((always_inline)) {
    const lds_char* xt = lds_opaque(xt_buf);
    const int h = ps.h, q0 = ps.q0;
    const int l = lane_here(), gi = l >> 4, ii = l & 15;
    const int kt_last = causal ? q0 / KT : (L + KT - 1) / KT - 1;
    const bool first = t == 0, last = t == kt_last;
    int* cnt = fq.cnt + ((size_t)(fq.padoff[doc] / 32 + q0 / 32) * hq + h) * 8 + w;
    const size_t row0 = (size_t)(s0 + q0) * hq + h;
    // the block's rows q0 .. q0 + 63 of head h: buffer offsets from row q0 (raw buffer accesses
    // past the end of the buffer read 0 / write nothing)
    const unsigned long long rem = fq.acc_bytes - row0 * D * sizeof(float);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        fq.acc + row0 * D, 0, (int)(rem < 0x7fffffffull ? rem : 0x7fffffffull), 0x00020000);
    const int lo0 = (ii * hq * D + 16 * w + 4 * gi) * (int)sizeof(float), sb_step = 16 * hq * D * (int)sizeof(float);
    // Hand-over, reading side: the sums travel as device-scope accesses (sc1), coherent on their
    // own whichever CU or XCD wrote them (a plain load could hit an older copy left in this CU's
    // L1 by an earlier tile of the chain)
    if (!first) wait_count(cnt, t, fq.header);
    f32x4 c[4];                                   // the products accumulate onto the running sums
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
      c[sb] = first ? f32x4{}
                    : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo0 + sb * sb_step, 0,
                                                                                     SC1));
    // this wave's Kᵀ operands (written by this wave at the item's start)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(kt_slot + w * NP * 64, 0, NP * 64 * 16, 0x00020000);
    bf16x8 kT[NP];
#pragma unroll
    for (int kk = 0; kk < NP; ++kk)
      kT[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, (kk * 64 + l) * 16, 0, SC1));
    const int rr = 8 * gi + (ii >> 2);
    const int fd = ((rr >> 1) & 1) | (((rr >> 3) & 1) << 1);
#pragma unroll
    for (int kk = 0; kk < NP; ++kk) {
      const int pk0 = t * KT + 32 * kk;           // pair kk's first key
      if ((causal ? q0 + BM - 1 >= pk0 : true) && pk0 < L) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          // rows 32kk + 8(l/16) + (l%16)/4 and + 4 (keys), columns 16sb + 4(l%4) (queries)
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const lds_char* a0 = xt + rr * 128 + (((sb ^ fd) & 3) << 5) + 8 * (ii & 3) + 4096 * kk;
          const bf16x8 b = concat_tr(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0),
                                     __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 512)));
          c[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kT[kk], b, c[sb], 0, 0, 0);
          // one operand pair in flight per product: the phase runs beside the partner wave's
          // step, with little register room left
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
    if (last) {
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(fq.dq + row0 * D, 0, 0x7fffffff, 0x00020000);
      const int qo0 = (ii * hq * D + 16 * w + 4 * gi) * 2, qsb = 16 * hq * D * 2;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        if (q0 + 16 * sb + ii < L)
          __builtin_amdgcn_raw_buffer_store_b64(
              i32x2{(int)pack_bf16x2(c[sb][0] * scale, c[sb][1] * scale), (int)pack_bf16x2(c[sb][2] * scale, c[sb][3] * scale)},
              rq, qo0 + sb * qsb, 0, 0);
    } else {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        if (q0 + 16 * sb + ii < L)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, c[sb]), rs, lo0 + sb * sb_step, 0, SC1);
    }
    wait_vmem();                                  // this wave's stores are done before the hand-over
    if (!last && l == 0) __hip_atomic_store(cnt, t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // Iteration i: copy step i+1 into `nxt`; P waves run step i on `cur`; dS waves run step i-1
  // on `prv`; with dQ inside the pass, every wave then adds its dQ part of step i-2 (dSᵀ in
  // `xdq`; one call site for both roles keeps the register count within two waves per SIMD).
  // The conditions depend on i only, so every wave meets the same barriers.
  // Positions of steps i + 1 (staged in iteration i), i (P waves), i − 1 (dS waves) and i − 2
  // (dQ parts), shifted by one step per iteration.
  Pos p_next = first_pos, p_cur = first_pos, p_prv = first_pos, p_dq = first_pos;
  auto iter = [&](int i, char* cur, char* prv, char* nxt, i32x4* xcur, i32x4* xprv, const i32x4* xdq)
      __attribute__((always_inline)) {
    if (i + 1 < n_steps) stage(p_next, nxt);
    if (!per_lane(ds_wave)) {
      if (i < n_steps && active(p_cur)) step_p(p_cur.q0, cur, xcur);
    } else {
      if (i >= 1 && i - 1 < n_steps && active(p_prv)) step_ds(prv, xprv);
    }
    if (i + 1 < n_steps) stage_finish(nxt);
    if constexpr (FQ) {
      if (i >= 2 && i - 2 < n_steps) dq_phase(p_dq, xdq);
    }
    p_dq = p_prv;
    p_prv = p_cur;
    p_cur = p_next;
    p_next = next_pos(p_next);
    wait_vmem();
    __syncthreads();
  };

  if (n_steps > 0) {
    stage(first_pos, st_a);
    stage_finish(st_a);
  }
  p_next = next_pos(first_pos);
  wait_vmem();
  __syncthreads();
  const int last_i = n_steps + (FQ ? 1 : 0);
  for (int i = 0; i <= last_i; i += 3) {
    iter(i, st_a, st_c, st_b, xp_a, xp_c, xp_b);
    if (i + 1 <= last_i) iter(i + 1, st_b, st_a, st_c, xp_b, xp_a, xp_c);
    if (i + 2 <= last_i) iter(i + 2, st_c, st_b, st_a, xp_c, xp_b, xp_a);
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

// One workgroup per (key tile, head split, kv head) of the work list.
template <int D, int NP, bool CROSS, bool SPLIT>
__global__ __launch_bounds__(128 * NP, 1) void attn_bwd_dkdv_pair_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, Plan plan, int total_tokens, int hq, int hkv,
    float scale, int causal, int n_split, float* __restrict__ part_dk, float* __restrict__ part_dv,
    const int2* __restrict__ qdoc, int total_k) {
  using X = DkdvLds<D, NP>;
  __shared__ __attribute__((aligned(16))) char st_a[X::STAGE];
  __shared__ __attribute__((aligned(16))) char st_b[X::STAGE];
  __shared__ __attribute__((aligned(16))) char st_c[X::STAGE];
  __shared__ i32x4 xp_a[X::XP];
  __shared__ i32x4 xp_b[X::XP];
  __shared__ i32x4 xp_c[X::XP];
  const int ns = SPLIT ? n_split : 1;
  // work-item values are the same in every lane; readfirstlane keeps them (and all derived from
  // them) in scalar registers
  const int p = __builtin_amdgcn_readfirstlane(blockIdx.x / (hkv * ns));
  const int g = __builtin_amdgcn_readfirstlane(blockIdx.x % hkv);
  const int split = SPLIT ? __builtin_amdgcn_readfirstlane((blockIdx.x / hkv) % ns) : 0;
  int s0, L, t, doc;
  if (!decode_item(plan, p, 32 * NP, false, s0, L, t, &doc)) return;
  dkdv_item<D, NP, CROSS, SPLIT, false>(q, k, v, dout, lse, delta, dk, dv, total_tokens, hq, hkv, scale, causal,
                                               n_split, part_dk, part_dv, qdoc, total_k, FusedDq{}, s0, L, t, doc, g,
                                               split, st_a, st_b, st_c, xp_a, xp_b, xp_c);
}

// Claims the next key tile for this XCD (one thread of the workgroup). Chains are (document,
// kv head, head split) in longest-first document order; a chain's key tiles are handed out in
// order from a 64-bit word of this XCD (high half: chain + 1, low half: next tile) by atomic
// increment, so all tiles of a chain go to workgroups of one XCD and tile t is handed out after
// tile t − 1, to a running workgroup. The thread that draws the first tile past a chain's end
// takes the next chain from the global counter and publishes it (with tile 0 taken); threads
// that drew later wait for the word to change. Returns false when no chain is left.
__device__ inline bool claim_tile(const FusedDq& fq, const Plan& pl, int per_doc, int kt, int& chain, int& tile) {
  unsigned long long* word = (unsigned long long*)(fq.header + 16) + (xcc_id() & 15);
  auto tiles_of = [&](int c) { return (pl.docinfo[pl.order[c / per_doc]].y + kt - 1) / kt; };
  for (int spins = 0;;) {
    const unsigned long long old = atomicAdd(word, 1ull);
    const int hi = (int)(old >> 32), lo = (int)(old & 0xffffffffull);
    if (hi == CLAIM_END) return false;
    const int n = hi == 0 ? 0 : tiles_of(hi - 1);
    if (lo < n) {
      chain = hi - 1;
      tile = lo;
      return true;
    }
    if (lo == n) {
      for (;;) {
        const int c = atomicAdd(fq.header + 2, 1);
        if (c >= fq.n_chains) {
          atomicExch(word, (unsigned long long)CLAIM_END << 32);
          return false;
        }
        if (tiles_of(c) > 0) {
          atomicExch(word, ((unsigned long long)(c + 1) << 32) | 1ull);
          chain = c;
          tile = 0;
          return true;
        }
      }
    }
    while ((int)(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) == hi) {
      if (++spins > SPIN_LIMIT) {
        atomicOr(fq.header, 8);
        return false;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// dK, dV and dQ in one pass (self-attention, d = 128): a persistent grid, one workgroup per CU,
// each claiming key tiles of its XCD until none is left.
template <bool SPLIT>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, Plan plan, int total_tokens, int hq, int hkv,
    float scale, int causal, int n_split, float* __restrict__ part_dk, float* __restrict__ part_dv, FusedDq fq) {
  using X = DkdvLds<128, 4>;
  __shared__ __attribute__((aligned(16))) char st_a[X::STAGE];
  __shared__ __attribute__((aligned(16))) char st_b[X::STAGE];
  __shared__ __attribute__((aligned(16))) char st_c[X::STAGE];
  __shared__ i32x4 xp_a[X::XP];
  __shared__ i32x4 xp_b[X::XP];
  __shared__ i32x4 xp_c[X::XP];
  __shared__ int claim[2];
  const int ns = SPLIT ? n_split : 1;
  const int per_doc = hkv * ns;
  for (;;) {
    if (threadIdx.x == 0) {
      int c = -1, tl = 0;
      if (!claim_tile(fq, plan, per_doc, 128, c, tl)) c = -1;
      claim[0] = c;
      claim[1] = tl;
    }
    __syncthreads();
    const int c = __builtin_amdgcn_readfirstlane(claim[0]), t = __builtin_amdgcn_readfirstlane(claim[1]);
    __syncthreads();
    if (c < 0) return;
    const int doc = __builtin_amdgcn_readfirstlane(plan.order[c / per_doc]);
    const int r = c % per_doc;
    const int2 di = plan.docinfo[doc];
    dkdv_item<128, 4, false, SPLIT, true>(
        q, k, v, dout, lse, delta, dk, dv, total_tokens, hq, hkv, scale, causal, n_split, part_dk, part_dv, nullptr,
        total_tokens, fq, __builtin_amdgcn_readfirstlane(di.x), __builtin_amdgcn_readfirstlane(di.y), t, doc, r % hkv,
        r / hkv, st_a, st_b, st_c, xp_a, xp_b, xp_c);
  }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int* __restrict__ p, long n) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) *(i32x4*)(p + i) = i32x4{0, 0, 0, 0};
  else for (long j = i; j < n; ++j) p[j] = 0;
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
  // work-item values are the same in every lane; readfirstlane keeps them in scalar registers
  const int p = __builtin_amdgcn_readfirstlane(blockIdx.x / n_hb), hb = __builtin_amdgcn_readfirstlane(blockIdx.x % n_hb);
  int s0, L, t, doc;
  if (!decode_item(plan, p, 128, true, s0, L, t, &doc)) return;
  int k_s0 = s0, Lk = L;                         // key rows (cross-attention: their own documents)
  if constexpr (CROSS) {
    const int2 kd = kdoc[doc];
    k_s0 = __builtin_amdgcn_readfirstlane(kd.x);
    Lk = __builtin_amdgcn_readfirstlane(kd.y);
  }
  const int off = CROSS ? Lk - L : 0;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5;
  const int h = hb * HPB + (w >> 2);             // this wave's query head
  const int g = __builtin_amdgcn_readfirstlane(h / (hq / hkv));
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
  // d >= 128: lane offsets of the tile copies, fixed for the whole key loop
  // two heads per workgroup: only waves 0..3 copy, so the other wave of each SIMD starts its
  // products while they issue the copies
  const RowCopies<BN, 4, D >= 128 ? D : 128> rc((uint32_t)hkv * D * 2, w & 3, lane);
  auto stage = [&](int kt, char* kb) {
    const int k0 = kt * BN;
    char* vb = kb + TILE;
    if constexpr (D >= 128) {
      // keys past kv_end read zeros (masked: P = 0)
      const size_t row0 = ((size_t)(k_s0 + k0) * hkv + g) * D;
      if (w < 4) {
        rc.copy(kb, k + row0, kv_end - 1 - k0, w);
        rc.copy(vb, v + row0, kv_end - 1 - k0, w);
      }
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

hipError_t launch_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              const float* delta, void* dq, void* dk, void* dv, const Plan& plan, int T, int hq, int hkv,
                              float scale, int causal, int n_split, float* part, float* dq_acc, int* cnt, long n_cnt,
                              const int* padoff, int* header, void* kt, int n_cu, hipStream_t stream) {
  if (n_cnt > 0)
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((n_cnt / 4 + 255) / 256 + 1)), dim3(256), 0, stream, cnt, n_cnt);
  FusedDq fq;
  fq.acc = dq_acc;
  fq.cnt = cnt;
  fq.dq = (__bf16*)dq;
  fq.padoff = padoff;
  fq.header = header;
  fq.kt = (i32x4*)kt;
  fq.acc_bytes = (unsigned long long)T * hq * 128 * sizeof(float);
  fq.n_chains = plan.n_docs * hkv * n_split;
  const long n = (long)T * hkv * 128;
  float* pdk = n_split > 1 ? part : nullptr;
  float* pdv = n_split > 1 ? part + (size_t)n_split * n : nullptr;
  const dim3 grid((unsigned)std::max(1, std::min(n_cu, FUSED_MAX_GRID))), block(512);
#define CFA_FUSED(SP)                                                                                     \
  hipLaunchKernelGGL((attn_bwd_dkdv_dq_kernel<SP>), grid, block, 0, stream, (const __bf16*)q, (const __bf16*)k, \
                     (const __bf16*)v, (const __bf16*)dout, lse, delta, (__bf16*)dk, (__bf16*)dv, plan, T, hq, hkv, \
                     scale, causal, n_split, pdk, pdv, fq)
  if (n_split > 1) CFA_FUSED(true);
  else CFA_FUSED(false);
#undef CFA_FUSED
  if (n_split > 1 && n > 0)
    hipLaunchKernelGGL(dkdv_split_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, pdk, pdv,
                       (__bf16*)dk, (__bf16*)dv, n, n_split, scale, plan.header);
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

// Fused causal attention forward for gfx950: bf16 MFMA path and an fp32 path.
//
// What is computed (per document, query head h, kv head g = h / (hq/hkv)):
//   S = scale·Q Kᵀ, masked by index (key j visible to query i iff j <= i), P = softmax(S),
//   O = P V, LSE = ln Σ_j exp(S_ij)   -- "GPT Kernel Programlama" §2-§6.
// How: Q/K/V are cut into tiles that live on chip; each workgroup walks the key tiles of its
// query tile with a running row maximum and running sum (online softmax) and writes O once;
// tiles wholly above the diagonal are skipped -- "GPT Kernel Programlama" §4 and §7,
// "FlashAttention (HU)" sections "Tiling és blokkos feldolgozás", "Online Softmax-számítás",
// "Műveletek összevonása egyetlen CUDA-kernelbe".
//
// bf16 kernel layout (d = 64, 128 or 256), one workgroup = NW waves of 64 lanes (8 for d = 128, 4
// for 64 and 256; d = 256 holds a 128-register Oᵀ accumulator per wave, so one wave per SIMD):
//  * Each wave owns 32 query rows of one head. HPW heads of one GQA group share a workgroup
//    (HPW = 1, 2 or 4), so a K/V tile staged in LDS serves 32·NW (row, head) pairs: with 8 waves
//    each staged byte feeds twice the products of a 4-wave workgroup (one workgroup per CU).
//  * Scores are formed transposed, Sᵀ = K Qᵀ, with v_mfma_f32_32x32x16_bf16: the wave's Qᵀ
//    fragment stays in registers for the whole key loop, and each lane ends up holding one
//    query column, so the row max and row sum are in-lane plus one swap between lane halves.
//  * The probabilities in that layout are already the B operand of Oᵀ += Vᵀ Pᵀ (only a
//    convert to bf16); Vᵀ comes from the row-major V tile through ds_read_b64_tr_b16.
//  * K/V tiles of 64 keys are double-buffered in LDS: the next tile's global loads are in
//    flight while the current tile is multiplied.
//  * exp2 with scale·log2(e) folded into the exponent; LSE converted back to natural log.
// Cross-attention (CROSS = true): the work list is built on the query documents and `kdoc[doc]`
// gives the document's key rows (start, length); with off = Lk - Lq, query i sees key j iff
// j <= i + off (causal) -- the causal rule with the queries at the end of the keys. A row that
// sees no key gets O = 0 and LSE = -inf, and the running maximum starts from -inf without NaN.
#include "cfa_device.h"

namespace cfa {

template <int D>
struct FwdTile {
  static constexpr int BN = 64;                  // keys per tile
  using S = SwzTile<D>;                          // swizzled rows, see cfa_device.h
  static constexpr int KBYTES = BN * S::STR;
  static constexpr int VBYTES = BN * S::STR;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int CHUNKS = BN * D / 8;      // 16-byte chunks per tile and tensor
  static constexpr int PER_THREAD = CHUNKS / 256;
  static constexpr int DS = D / 16;              // k-steps of the QKᵀ MFMA
  static constexpr int DB = D / 32;              // 32-wide d blocks of Oᵀ
};

// The running maximum is only moved when a tile's maximum exceeds it by more than this (log2
// units), which skips most rescalings of the O accumulator.
constexpr float RESCALE_LOG2 = 8.f;

template <int D, int HPW, int NW, bool CROSS>
__global__ __launch_bounds__(64 * NW, D == 256 ? 1 : 8 / NW) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, Plan plan, int total_tokens, int hq, int hkv,
    int n_hb, float scale_log2, int causal, const int2* __restrict__ kdoc) {
  using C = FwdTile<D>;
  constexpr int BMW = 32 * NW / HPW;  // query rows per workgroup
  // two separate LDS buffers (not one array indexed at run time) so that the compiler can
  // tell that the copy into one buffer never aliases the reads of the other
  __shared__ __attribute__((aligned(16))) char lds_a[C::STAGE];
  __shared__ __attribute__((aligned(16))) char lds_b[C::STAGE];

  const int wid = blockIdx.x;
  // work-item values are the same in every lane; readfirstlane keeps them in scalar registers
  const int p = __builtin_amdgcn_readfirstlane(wid / n_hb), hb = __builtin_amdgcn_readfirstlane(wid % n_hb);
  int s0, L, t, doc;
  if (!decode_item(plan, p, BMW, true, s0, L, t, &doc)) return;
  // query rows [s0, s0 + L), key rows [k_s0, k_s0 + Lk); off = 0 for self-attention
  int k_s0 = s0, Lk = L;
  if constexpr (CROSS) {
    const int2 kd = kdoc[doc];
    k_s0 = __builtin_amdgcn_readfirstlane(kd.x);
    Lk = __builtin_amdgcn_readfirstlane(kd.y);
  }
  const int off = CROSS ? Lk - L : 0;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = __builtin_amdgcn_readfirstlane(hq / hkv);
  const int h = hb * HPW + (w % HPW);
  const int g = __builtin_amdgcn_readfirstlane(h / G);
  const int wr0 = t * BMW + 32 * (w / HPW);      // first doc-local row of this wave
  const int wg_rows_end = min(L, (t + 1) * BMW);
  // keys the workgroup needs (cross-attention: possibly none)
  const int kv_end = causal ? (CROSS ? min(Lk, wg_rows_end + off) : wg_rows_end) : Lk;
  const int n_kt = (CROSS && kv_end <= 0) ? 0 : (kv_end + C::BN - 1) / C::BN;
  const int wave_last_key = causal ? (CROSS ? min(Lk, min(L, wr0 + 32) + off) : min(L, wr0 + 32)) - 1 : Lk - 1;
  const int qrow = wr0 + (lane & 31);            // this lane's query (doc-local)
  const int half = lane >> 5;
  const SwzOffsets<D> so(lane);

  // ---- Qᵀ fragments (B operand): lane holds Q[qrow][16s + 8·half .. +8]
  bf16x8 qf[C::DS];
  {
    const bool ok = qrow < L;
    const __bf16* src = q + ((size_t)(s0 + (ok ? qrow : 0)) * hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      i32x4 u = ok ? *(const i32x4*)(src + 16 * s) : i32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- staging of one K/V tile into an LDS buffer: [K rows][V rows]. d >= 128: direct global ->
  // LDS copies shared out among the NW waves (no registers, completion tracked by vmcnt);
  // d = 64: through registers. Keys past kv_end are clamped into the document: they are masked
  // (P = 0).
  // d >= 128: lane offsets of the tile copies, fixed for the whole key loop
  // with two waves per SIMD (NW = 8), only waves 0..3 copy: the other wave of each SIMD starts
  // its products while they issue the copies
  constexpr int CW = NW == 8 ? 4 : NW;
  const RowCopies<C::BN, CW, D >= 128 ? D : 128> rc((uint32_t)hkv * D * 2, w % CW, lane);
  auto stage = [&](int kt, char* kb) {
    const int k0 = kt * C::BN;
    char* vb = kb + C::KBYTES;
    if constexpr (D >= 128) {
      // keys past kv_end read zeros (masked: P = 0)
      const size_t row0 = ((size_t)(k_s0 + k0) * hkv + g) * D;
      if (w < CW) {
        rc.copy(kb, k + row0, kv_end - 1 - k0, w);
        rc.copy(vb, v + row0, kv_end - 1 - k0, w);
      }
    } else {
      i32x4 kreg[C::PER_THREAD], vreg[C::PER_THREAD];
#pragma unroll
      for (int i = 0; i < C::PER_THREAD; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int key = c / (D / 8), col = c % (D / 8);
        const size_t eo = ((size_t)(k_s0 + min(k0 + key, kv_end - 1)) * hkv + g) * D + col * 8;
        kreg[i] = *(const i32x4*)(k + eo);
        vreg[i] = *(const i32x4*)(v + eo);
      }
#pragma unroll
      for (int i = 0; i < C::PER_THREAD; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int key = c / (D / 8), col = c % (D / 8);
        *(i32x4*)(kb + C::S::chunk(key, col)) = kreg[i];
        *(i32x4*)(vb + C::S::chunk(key, col)) = vreg[i];
      }
    }
  };

  if (!CROSS || n_kt > 0) stage(0, lds_a);
  wait_vmem();
  __syncthreads();

  // the 64-key tile at doc-local key k0, its K rows at kb and V rows at vb
  auto subtile = [&](int k0, const char* kb, const char* vb) __attribute__((always_inline)) {
    if (k0 <= wave_last_key) {
      // ---- Sᵀ = K Qᵀ for the tile's two 32-key blocks: operand rows read as a batch (d = 256:
      // four batches of 4 k-steps), the two accumulators interleaved so consecutive MFMAs are
      // independent
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      constexpr int SB = D == 256 ? 4 : C::DS;
#pragma unroll
      for (int sc = 0; sc < C::DS; sc += SB) {
        i32x4 fk[2][SB];
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
          for (int b = 0; b < 2; ++b) fk[b][s] = *(const i32x4*)(kb + b * 32 * C::S::STR + so.row[sc + s]);
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
          for (int b = 0; b < 2; ++b) sacc[b] = mfma32(as_bf16x8(fk[b][s]), qf[sc + s], sacc[b]);
        if constexpr (D <= 128) {
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::DS - 4, 0);
        }
      }
      // ---- online softmax on this lane's query column. The maximum is taken on the raw scores
      // (scale_log2 > 0) and the scale is folded into the exponent, p = 2^(s·c − m). Masking
      // is a separate, wave-uniform branch taken only by tiles that cross the diagonal or the
      // document end.
      const bool need_mask = causal ? (k0 + C::BN - 1 > wr0 + off) : (k0 + C::BN > Lk);
      if (need_mask) {
        // keys above lim are masked; element j of block b holds key k0 + 32b + 4·half + c_j,
        // c_j = 8(j/4) + j%4, so one compare of the constant c_j per element
        const int lim = causal ? qrow + off : Lk - 1;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int r = lim - (k0 + 32 * b + 4 * half);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (8 * (j >> 2) + (j & 3) > r) sacc[b][j] = -INFINITY;
        }
      }
      const float mt = wave_max_xor32(max32(sacc[0], sacc[1])) * scale_log2;
      // Lazy rescaling: the reference maximum only moves when the tile's maximum exceeds it
      // by more than RESCALE_LOG2 (then P <= 2^RESCALE_LOG2, harmless in fp32 / bf16); LSE and
      // O are exact for any reference value.
      const bool upd = mt > m_run + RESCALE_LOG2;
      if (__any(upd)) {
        const float m_new = upd ? mt : m_run;
        // a row that has seen no key yet keeps m = -inf (cross-attention only): factor 1, not NaN
        const float alpha = (CROSS && m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
      }
      // four partial row sums (short add chains), each started by its first term rather than by
      // adding it to 0 (the terms are >= +0, so the sums are the same)
      float ls4[4];
      bf16x8 pf[4];
      const float m_use = (CROSS && m_run == -INFINITY) ? 0.f : m_run;   // all -inf scores -> p = 0
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const float p0 = exp2_fast(fmaf(sacc[b][j], scale_log2, -m_use));
          const float p1 = exp2_fast(fmaf(sacc[b][j + 1], scale_log2, -m_use));
          if (b == 0 && j < 8) ls4[j >> 1] = p0 + p1;
          else ls4[(j >> 1) & 3] += p0 + p1;
          const uint32_t pk = pack_bf16x2(p0, p1);
          i32x4 u = __builtin_bit_cast(i32x4, pf[2 * b + (j >> 3)]);
          u[(j & 7) >> 1] = (int)pk;
          pf[2 * b + (j >> 3)] = __builtin_bit_cast(bf16x8, u);
        }
      l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
      // ---- Oᵀ += Vᵀ Pᵀ; Vᵀ fragments via transposing LDS reads
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int rb = (32 * (kk >> 1) + 16 * (kk & 1)) * C::S::STR;
        bf16x8 av[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          av[db] = concat_tr(lds_read_tr16(vb + rb + so.tr0[db]), lds_read_tr16(vb + rb + so.tr1[db]));
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] = mfma32(av[db], pf[kk], oacc[db]);
      }
    }
  };
  // one key tile: copy tile kt+1 into `nxt` while multiplying tile kt from `cur`
  auto iter = [&](int kt, const char* cur, char* nxt) __attribute__((always_inline)) {
    if (kt + 1 < n_kt) stage(kt + 1, nxt);
    subtile(kt * C::BN, cur, cur + C::KBYTES);
    wait_vmem();
    __syncthreads();
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    iter(kt, lds_a, lds_b);
    if (kt + 1 < n_kt) iter(kt + 1, lds_b, lds_a);
  }

  // ---- epilogue: O = Oᵀ / l, LSE = (m + log2 l)·ln 2
  const float l_tot = wave_sum_xor32(l_run);
  if (qrow < L) {
    const float inv = (CROSS && !(l_tot > 0.f)) ? 0.f : 1.f / l_tot;
    __bf16* dst = o + ((size_t)(s0 + qrow) * hq + h) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        i32x2 u;
        u.x = (int)pack_bf16x2(oacc[db][4 * jg] * inv, oacc[db][4 * jg + 1] * inv);
        u.y = (int)pack_bf16x2(oacc[db][4 * jg + 2] * inv, oacc[db][4 * jg + 3] * inv);
        *(i32x2*)(dst + 32 * db + 8 * jg) = u;
      }
    if (half == 0)
      lse[(size_t)h * total_tokens + s0 + qrow] =
          (CROSS && !(l_tot > 0.f)) ? -INFINITY : (m_run + __log2f(l_tot)) * LN2;
  }
}

// ------------------------------------------------------------------ fp32 path
// One wave per workgroup, one query row per lane, 64-row query tiles, key tiles of KT keys in
// LDS; plain fp32 FMA arithmetic with the same online softmax.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, Plan plan, int total_tokens, int hq, int hkv,
    float scale_log2, int causal) {
  constexpr int KT = (D <= 64) ? 64 : 32;
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[KT][D + 1];
  const int p = blockIdx.x / hq, h = blockIdx.x % hq;
  int s0, L, t;
  if (!decode_item(plan, p, 64, true, s0, L, t)) return;
  const int g = h / (hq / hkv);
  const int lane = threadIdx.x;
  const int qrow = t * 64 + lane;
  const bool ok = qrow < L;
  float qr[D], acc[D];
  for (int r = 0; r < D; ++r) {
    qr[r] = ok ? q[((size_t)(s0 + qrow) * hq + h) * D + r] : 0.f;
    acc[r] = 0.f;
  }
  const int kv_end = causal ? min(L, (t + 1) * 64) : L;
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = 0; k0 < kv_end; k0 += KT) {
    __syncthreads();
    for (int i = lane; i < KT * D; i += 64) {
      const int key = i / D, r = i % D;
      const bool in = k0 + key < kv_end;
      const size_t off = ((size_t)(s0 + (in ? k0 + key : 0)) * hkv + g) * D + r;
      ks[key][r] = in ? k[off] : 0.f;
      vs[key][r] = in ? v[off] : 0.f;
    }
    __syncthreads();
    float s[KT];
    float mt = -INFINITY;
    for (int j = 0; j < KT; ++j) {
      float x = 0.f;
      for (int r = 0; r < D; ++r) x = fmaf(qr[r], ks[j][r], x);
      x *= scale_log2;
      const int key = k0 + j;
      const bool masked = (key >= kv_end) || (causal && key > qrow);
      s[j] = masked ? -INFINITY : x;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2_fast(m_run - m_new);
    l_run *= alpha;
    for (int r = 0; r < D; ++r) acc[r] *= alpha;
    for (int j = 0; j < KT; ++j) {
      const float pj = exp2_fast(s[j] - m_new);
      l_run += pj;
      for (int r = 0; r < D; ++r) acc[r] = fmaf(pj, vs[j][r], acc[r]);
    }
    m_run = m_new;
  }
  if (ok) {
    const float inv = 1.f / l_run;
    for (int r = 0; r < D; ++r) o[((size_t)(s0 + qrow) * hq + h) * D + r] = acc[r] * inv;
    lse[(size_t)h * total_tokens + s0 + qrow] = (m_run + __log2f(l_run)) * LN2;
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, const Plan& plan_any,
                           const int* pref_base, int total_tokens, int hq, int hkv, int d, float scale, int causal,
                           hipStream_t stream, const int2* kdoc) {
  const int G = hq / hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  const int nw = (d == 128) ? 8 : 4;              // waves per workgroup (one K/V tile for all of them)
  const int rows = 32 * nw / hpw;
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(rows) * (plan.n_docs + 1);
  const int n_hb = hq / hpw;
  // upper bound of items for this tile height: ceil(T/rows) + n_docs
  const long items = (long)(total_tokens + rows - 1) / rows + plan.n_docs;
  const long grid = items * n_hb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const float sl2 = scale * LOG2E;
  const __bf16* Q = (const __bf16*)q;
  const __bf16* K = (const __bf16*)k;
  const __bf16* V = (const __bf16*)v;
  __bf16* O = (__bf16*)o;
#define CFA_FWD_LAUNCH(DD, HH, NN)                                                                         \
  do {                                                                                                     \
    if (kdoc)                                                                                              \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, HH, NN, true>), dim3((unsigned)grid), dim3(64 * NN), 0, stream, \
                         Q, K, V, O, lse, plan, total_tokens, hq, hkv, n_hb, sl2, causal, kdoc);          \
    else                                                                                                   \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, HH, NN, false>), dim3((unsigned)grid), dim3(64 * NN), 0,      \
                         stream, Q, K, V, O, lse, plan, total_tokens, hq, hkv, n_hb, sl2, causal, kdoc);  \
  } while (0)
  if (d == 128) {
    if (hpw == 4) CFA_FWD_LAUNCH(128, 4, 8);
    else if (hpw == 2) CFA_FWD_LAUNCH(128, 2, 8);
    else CFA_FWD_LAUNCH(128, 1, 8);
  } else if (d == 256) {
    if (hpw == 4) CFA_FWD_LAUNCH(256, 4, 4);
    else if (hpw == 2) CFA_FWD_LAUNCH(256, 2, 4);
    else CFA_FWD_LAUNCH(256, 1, 4);
  } else {
    if (hpw == 4) CFA_FWD_LAUNCH(64, 4, 4);
    else if (hpw == 2) CFA_FWD_LAUNCH(64, 2, 4);
    else CFA_FWD_LAUNCH(64, 1, 4);
  }
#undef CFA_FWD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, const Plan& plan_any,
                          const int* pref_base, int total_tokens, int hq, int hkv, int d, float scale, int causal,
                          hipStream_t stream) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(64) * (plan.n_docs + 1);
  const long items = (long)(total_tokens + 63) / 64 + plan.n_docs;
  const long grid = items * hq;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const float sl2 = scale * LOG2E;
  if (d == 64)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (float*)o, lse, plan, total_tokens, hq, hkv, sl2, causal);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(64), 0, stream, (const float*)q,
                       (const float*)k, (const float*)v, (float*)o, lse, plan, total_tokens, hq, hkv, sl2, causal);
  return hipGetLastError();
}

}  // namespace cfa

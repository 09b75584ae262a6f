// Split-KV decoding for gfx950: one new query token per sequence over a packed KV cache, held
// in bf16 or in the MX format (E4M3 codes with one E8M0 scale per 32 channels of a token).
//
// What is computed (per sequence b, query head h, kv head g = h / (hq/hkv)): the query sees
// every cached key of its sequence (the current token's included), s_j = scale·q·K_j,
// o = softmax(s)·V, lse = ln Σ_j exp(s_j) -- the last row of a causal document ("GPT Kernel
// Programlama" §4-§6). The cache is read through flash attention with a quantised V, as local
// inference engines do ("Flash Attention", ai.ozdemir.be, "Tanım" and "Gerçek dünyadan örnek").
//
// The pass is bound by reading the cache once from HBM (no reuse across sequences), so the
// design keeps every cache byte to one read and makes the arithmetic cheap next to it:
//  * Workgroup = (1024-key chunk of one sequence, kv head g, block of up to 32 query heads of g's
//    group). The group's query heads play the 32 query columns of the forward kernel's
//    transposed product, so each K/V byte read serves all of them.
//  * 4 waves × 256 keys. A wave loads its keys' rows 32 at a time into registers (the next
//    blocks' loads in flight during the current block's products), converts them to bf16
//    (MX: v_cvt_scalef32_pk_bf16_fp8 with the block scale; E4M3 × 2^e is exact in bf16) into its
//    own swizzled LDS region, then Sᵀ = K Qᵀ and Oᵀ += Vᵀ Pᵀ with v_mfma_f32_32x32x16_bf16 and an
//    online softmax per column. No barrier inside the key loop.
//  * The four waves merge (max, sum, Oᵀ) through LDS; the workgroup writes one partial per
//    query head; the combine kernel merges a sequence's chunks in chunk order (deterministic).
#include "cfa_device.h"

namespace cfa {

constexpr int DEC_CHUNK = 1024;  // keys per workgroup
constexpr int DEC_SUB = 32;     // keys per wave block

// Partial slot of chunk t of a sequence whose cache starts at token s0 (sequence index b):
// floor((s0 + 1024 t) / 1024) + b, injective over all (b, t) and below ceil(Tk/1024) + n_seqs.
__device__ inline int dec_slot(int s0, int t, int b) { return (s0 + DEC_CHUNK * t) / DEC_CHUNK + b; }

template <int D, bool MX>
struct DecLoads {
  // one 32-key block of K or V rows per wave: lane i loads 16 bytes per row piece
  static constexpr int BYTES_PER_ROW = MX ? D : 2 * D;
  static constexpr int LPR = BYTES_PER_ROW / 16;  // lanes per row
  static constexpr int ROWS_PER_LOAD = 64 / LPR;
  static constexpr int NL = DEC_SUB / ROWS_PER_LOAD;
};

template <int D, bool MX>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(
    const __bf16* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const uint8_t* __restrict__ ksc, const uint8_t* __restrict__ vsc, float* __restrict__ part_o,
    float2* __restrict__ part_ml, Plan plan, int hq, int hkv, int n_hb, float scale_log2) {
  using S = SwzTile<D>;
  using LD = DecLoads<D, MX>;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int SUBB = DEC_SUB * S::STR;                 // one 32-key bf16 tile
  constexpr int STAGE_BYTES = 4 * 2 * SUBB;              // per wave: K tile, V tile
  constexpr int MERGE_BYTES = 4 * 32 * (D + 1) * 4;      // per wave: Oᵀ as [column][d + 1]
  constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  __shared__ float mw[4][32], lw[4][32];

  // Workgroups are dealt to the 8 XCDs round-robin. All (kv head, head block) workgroups of one
  // chunk go to the same XCD back to back, so the cache rows of a chunk ([key][hkv][d], all kv
  // heads contiguous) are read by one XCD at nearly the same time.
  const int HB = hkv * n_hb;
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  const int p = (r / HB) * 8 + xcd;
  const int g = (r % HB) / n_hb, hb = (r % HB) % n_hb;
  int s0, L, t, b;
  if (!decode_item(plan, p, DEC_CHUNK, false, s0, L, t, &b)) return;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5;
  const int G = hq / hkv;
  const int col = lane & 31;                            // query column: head g·G + 32·hb + col
  const bool col_ok = 32 * hb + col < G;
  const int h = g * G + 32 * hb + col;
  const int k1 = min(L, (t + 1) * DEC_CHUNK);           // end of this chunk's keys
  constexpr int WK = DEC_CHUNK / 4, NB = WK / DEC_SUB;  // keys and 32-key blocks per wave
  const int kw0 = t * DEC_CHUNK + WK * w;               // this wave's first key
  const SwzOffsets<D> so(lane);
  char* kt = lds + w * 2 * SUBB;
  char* vt = kt + SUBB;

  bf16x8 qf[DS];
  {
    const __bf16* src = q + ((size_t)b * hq + (col_ok ? h : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, col_ok ? *(const i32x4*)(src + 16 * s) : i32x4{0, 0, 0, 0});
  }
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- raw rows of a 32-key block (keys past k1 repeat key k1 - 1: masked below). MX: two
  // blocks of codes in flight ahead of the block being converted; bf16: one block ahead (its rows
  // take twice the registers).
  constexpr int NBUF = MX ? 2 : 1;
  i32x4 kraw[NBUF][LD::NL], vraw[NBUF][LD::NL];
  int kscw[NBUF][LD::NL], vscw[NBUF][LD::NL];   // MX: the row's D/32 scale bytes (D = 128: one word)
  auto load = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < LD::NL; ++i) {
      const int key = min(kb + i * LD::ROWS_PER_LOAD + lane / LD::LPR, k1 - 1);
      const size_t row = (size_t)(s0 + key) * hkv + g;
      const int piece = lane % LD::LPR;
      kraw[buf][i] = *(const i32x4*)(kc + row * LD::BYTES_PER_ROW + 16 * piece);
      vraw[buf][i] = *(const i32x4*)(vc + row * LD::BYTES_PER_ROW + 16 * piece);
      if constexpr (MX) {
        if constexpr (D == 128) {
          kscw[buf][i] = *(const int*)(ksc + row * 4);
          vscw[buf][i] = *(const int*)(vsc + row * 4);
        } else {
          kscw[buf][i] = ksc[row * (D / 32) + piece / 2];
          vscw[buf][i] = vsc[row * (D / 32) + piece / 2];
        }
      }
    }
  };
  // ---- registers -> bf16 rows in this wave's LDS tiles
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LD::NL; ++i) {
      const int r = i * LD::ROWS_PER_LOAD + lane / LD::LPR;
      const int piece = lane % LD::LPR;
      if constexpr (MX) {
        // 16 codes = half of one 32-channel block: scale byte piece / 2 of the row
        const int sh = D == 128 ? 8 * (piece >> 1) : 0;
        const float ksf = pow2i(((kscw[buf][i] >> sh) & 0xFF) - 127);
        const float vsf = pow2i(((vscw[buf][i] >> sh) & 0xFF) - 127);
        i32x4 ko[2], vo[2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {                   // 4 codes per 32-bit word
          ko[u >> 1][2 * (u & 1)] = fp8x2_to_bf16x2_scaled<false>(kraw[buf][i][u], ksf);
          ko[u >> 1][2 * (u & 1) + 1] = fp8x2_to_bf16x2_scaled<true>(kraw[buf][i][u], ksf);
          vo[u >> 1][2 * (u & 1)] = fp8x2_to_bf16x2_scaled<false>(vraw[buf][i][u], vsf);
          vo[u >> 1][2 * (u & 1) + 1] = fp8x2_to_bf16x2_scaled<true>(vraw[buf][i][u], vsf);
        }
        *(i32x4*)(kt + S::chunk(r, 2 * piece)) = ko[0];
        *(i32x4*)(kt + S::chunk(r, 2 * piece + 1)) = ko[1];
        *(i32x4*)(vt + S::chunk(r, 2 * piece)) = vo[0];
        *(i32x4*)(vt + S::chunk(r, 2 * piece + 1)) = vo[1];
      } else {
        *(i32x4*)(kt + S::chunk(r, piece)) = kraw[buf][i];
        *(i32x4*)(vt + S::chunk(r, piece)) = vraw[buf][i];
      }
    }
  };

  // ---- one 32-key block from the LDS tiles: Sᵀ = K Qᵀ, online softmax, Oᵀ += Vᵀ Pᵀ
  auto block = [&](int kb) {
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) sacc = mfma32(as_bf16x8(*(const i32x4*)(kt + so.row[s])), qf[s], sacc);
    if (kb + DEC_SUB > k1) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (kb + 8 * (j >> 2) + 4 * half + (j & 3) >= k1) sacc[j] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[j]);
    mt = wave_max_xor32(mt) * scale_log2;
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2_fast(m_run - m_new);      // 0 on the first block (m_run = -inf)
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
    bf16x8 pf[2];
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const float p0 = exp2_fast(fmaf(sacc[j], scale_log2, -m_run));
      const float p1 = exp2_fast(fmaf(sacc[j + 1], scale_log2, -m_run));
      ls += p0 + p1;
      i32x4 u = __builtin_bit_cast(i32x4, pf[j >> 3]);
      u[(j & 7) >> 1] = (int)pack_bf16x2(p0, p1);
      pf[j >> 3] = __builtin_bit_cast(bf16x8, u);
    }
    l_run += ls;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int rb = 16 * kk * S::STR;
      bf16x8 av[DB];
#pragma unroll
      for (int i = 0; i < DB; ++i)
        av[i] = concat_tr(lds_read_tr16(vt + rb + so.tr0[i]), lds_read_tr16(vt + rb + so.tr1[i]));
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] = mfma32(av[i], pf[kk], oacc[i]);
    }
  };

  if (kw0 < k1) {
    const int nb = min(NB, (k1 - kw0 + DEC_SUB - 1) / DEC_SUB);   // this wave's blocks (1 .. NB)
    load(kw0, 0);
    if (MX && nb > 1) load(kw0 + DEC_SUB, 1);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i < nb) {
        if (i > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's tile reads are done
        store(MX ? (i & 1) : 0);
        // refill the raw registers just converted: block i + 2 (MX) or i + 1 (bf16)
        if (MX && i + 2 < nb) load(kw0 + (i + 2) * DEC_SUB, i & 1);
        if (!MX && i + 1 < nb) load(kw0 + (i + 1) * DEC_SUB, 0);
        block(kw0 + i * DEC_SUB);
      }
    }
  }

  // ---- merge the four waves: column maximum M, sum Σ_w l_w 2^(m_w - M), Oᵀ likewise
  const float l_tot = wave_sum_xor32(l_run);
  if (half == 0) {
    mw[w][col] = m_run;
    lw[w][col] = l_tot;
  }
  __syncthreads();                                      // also: every wave is done with its tiles
  float M = mw[0][col];
#pragma unroll
  for (int i = 1; i < 4; ++i) M = fmaxf(M, mw[i][col]);
  const float f = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - M);
  float* ot = (float*)lds + (size_t)w * 32 * (D + 1);  // this wave's Oᵀ as [column][d]
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) ot[col * (D + 1) + 32 * i + 8 * (j >> 2) + 4 * half + (j & 3)] = oacc[i][j] * f;
  __syncthreads();
  const int slot = dec_slot(s0, t, b);
  const int ncol = min(32, G - 32 * hb);
  for (int e = threadIdx.x; e < ncol * D; e += 256) {
    const int c = e / D, d = e % D;
    const float* src = (const float*)lds + c * (D + 1) + d;
    const float sum = src[0] + src[32 * (D + 1)] + src[2 * 32 * (D + 1)] + src[3 * 32 * (D + 1)];
    part_o[((size_t)slot * hq + g * G + 32 * hb + c) * D + d] = sum;
  }
  if (w == 0 && half == 0 && col_ok) {
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum += (mw[i][col] == -INFINITY) ? 0.f : lw[i][col] * exp2_fast(mw[i][col] - M);
    part_ml[(size_t)slot * hq + h] = float2{M, lsum};
  }
}

// Merge of a sequence's chunk partials: lane group c (of CL) folds chunks c, c + CL, ... with
// the online rule (m, l, o) <- (max, l·2^(m-m') + l_t·2^(m_t-m'), o·2^(m-m') + o_t·2^(m_t-m')), then
// the CL group results are folded in group order through LDS (a fixed order: deterministic).
// o = o / l, lse = (m + log2 l) ln 2; a sequence without keys gets o = 0, lse = -inf. One
// workgroup of 256 threads per (sequence, query head): D/4 threads per group, 4 channels each.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(const float* __restrict__ part_o,
                                                                  const float2* __restrict__ part_ml,
                                                                  __bf16* __restrict__ o, float* __restrict__ lse,
                                                                  Plan plan, int n_seqs, int hq) {
  constexpr int DQ = D / 4, CL = 256 / DQ;
  __shared__ float4 so4[CL][DQ];
  __shared__ float2 sml[CL];
  const int b = blockIdx.x / hq, h = blockIdx.x % hq;
  const int c0 = threadIdx.x / DQ, dq = threadIdx.x % DQ;
  const int2 di = plan.docinfo[b];
  const int s0 = di.x, L = di.y;
  const int n_ch = (L + DEC_CHUNK - 1) / DEC_CHUNK;
  const int base = dec_slot(s0, 0, b);
  float m = -INFINITY, l = 0.f;
  float4 acc = float4{0.f, 0.f, 0.f, 0.f};
  for (int c = c0; c < n_ch; c += CL) {
    const float2 ml = part_ml[(size_t)(base + c) * hq + h];
    const float4 ot = *(const float4*)(part_o + ((size_t)(base + c) * hq + h) * D + 4 * dq);
    const float mn = fmaxf(m, ml.x);
    const float a = (m == -INFINITY) ? 0.f : exp2_fast(m - mn), f = exp2_fast(ml.x - mn);
    l = l * a + ml.y * f;
    acc = acc * a + ot * f;
    m = mn;
  }
  so4[c0][dq] = acc;
  if (dq == 0) sml[c0] = float2{m, l};
  __syncthreads();
  if (c0 == 0) {
    for (int c = 1; c < CL; ++c) {
      const float2 ml = sml[c];
      if (ml.x == -INFINITY) continue;
      const float mn = fmaxf(m, ml.x);
      const float a = (m == -INFINITY) ? 0.f : exp2_fast(m - mn), f = exp2_fast(ml.x - mn);
      l = l * a + ml.y * f;
      acc = acc * a + so4[c][dq] * f;
      m = mn;
    }
    const float inv = n_ch > 0 ? 1.f / l : 0.f;
    __bf16* dst = o + ((size_t)b * hq + h) * D + 4 * dq;
    *(i32x2*)dst = i32x2{(int)pack_bf16x2(acc.x * inv, acc.y * inv), (int)pack_bf16x2(acc.z * inv, acc.w * inv)};
    if (dq == 0) lse[(size_t)h * n_seqs + b] = n_ch > 0 ? (m + __log2f(l)) * LN2 : -INFINITY;
  }
}

size_t decode_partial_slots(int total_k, int n_seqs) {
  return (size_t)(total_k + DEC_CHUNK - 1) / DEC_CHUNK + (size_t)n_seqs;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const uint8_t* ks, const uint8_t* vs,
                         const Plan& plan_any, const int* pref_base, int n_seqs, int total_k, int hq, int hkv, int d,
                         float scale, bool mx, float* part_o, void* part_ml, hipStream_t stream) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(DEC_CHUNK) * (plan.n_docs + 1);
  const int G = hq / hkv;
  const int n_hb = (G + 31) / 32;
  const long grid = (long)((decode_partial_slots(total_k, n_seqs) + 7) / 8) * 8 * hkv * n_hb;
  if (total_k == 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const float sl2 = scale * LOG2E;
  const __bf16* Q = (const __bf16*)q;
  const uint8_t* K = (const uint8_t*)k;
  const uint8_t* V = (const uint8_t*)v;
  float2* ML = (float2*)part_ml;
#define CFA_DEC_LAUNCH(DD, MM)                                                                             \
  hipLaunchKernelGGL((attn_decode_kernel<DD, MM>), dim3((unsigned)grid), dim3(256), 0, stream, Q, K, V, ks, vs, \
                     part_o, ML, plan, hq, hkv, n_hb, sl2)
  if (d == 128) {
    if (mx) CFA_DEC_LAUNCH(128, true);
    else CFA_DEC_LAUNCH(128, false);
  } else {
    if (mx) CFA_DEC_LAUNCH(64, true);
    else CFA_DEC_LAUNCH(64, false);
  }
#undef CFA_DEC_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode_combine(const float* part_o, const void* part_ml, void* o, float* lse, const Plan& plan,
                                 int n_seqs, int hq, int d, hipStream_t stream) {
  const long grid = (long)n_seqs * hq;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (d == 128)
    hipLaunchKernelGGL(attn_decode_combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                       (const float2*)part_ml, (__bf16*)o, lse, plan, n_seqs, hq);
  else
    hipLaunchKernelGGL(attn_decode_combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                       (const float2*)part_ml, (__bf16*)o, lse, plan, n_seqs, hq);
  return hipGetLastError();
}

}  // namespace cfa

// MXFP8 causal attention forward for gfx950 (d = 128).
//
// The MXFP8 path with token-block scaling, causal-leakage safeguards and forward/backward
// consistency is named on the FLAMIA page ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri"); the
// page gives no mechanism. This kernel implements the reading in which every product is
// blocked along its contraction axis:
//  * S = scale·Q Kᵀ contracts over d: E4M3 operands Q_d, K_d with one E8M0 scale per token and
//    32 channels (a scale never mixes tokens), on every tile, through
//    v_mfma_scale_f32_32x32x64_f8f6f4. The backward reuses the very same Q_d/K_d bytes.
//  * O += P V contracts over keys. Off the diagonal, V_t carries one scale per channel and
//    32 doc-local keys, and P̃ (at most 2^0.8 after the lazily moved running-max shift) is
//    encoded E4M3 with the fixed scale 2^-8 (P̃·2^8 <= 445.7 < 448; the 2^8 is folded into the
//    exponent). On the
//    diagonal 128×128 tile of each document the token blocks would share a scale between a
//    query and keys after it, so there P and V stay bf16 and use v_mfma_f32_32x32x16_bf16.
// Work list, online softmax, Sᵀ orientation and the two static LDS buffers filled by direct
// global -> LDS copies follow the bf16 kernel in attn_fwd.hip.
//
// MXFP4/FP8 (QF = 1): the score product takes E2M1 copies Q_d, K_d (two codes per byte,
// 64-byte rows for d = 128, blocks of 32 channels with E8M0 scales) through the same
// instruction with format code 4 on both operands; the rest is the MXFP8 path unchanged.
// MXFP6/FP8 (QF = 2): E2M3 copies, 96-byte rows whose blocks are a 16-byte part (the first 64
// bytes, staged and read exactly like the E2M1 rows) and an 8-byte part (the last 32 bytes,
// staged as two 16-byte chunks per row, chunk-major), format code 2. QF = 3: E3M2 copies in
// the same storage, format code 3.
//
// LDS tile (64 keys): K_d codes as 128-byte rows whose 16-byte chunks are XOR-swizzled with
// (row / 2) % 8 (FP4: 64-byte rows swizzled with (row / 4) % 4), then 4 scale bytes per key; then either the bf16 V rows of a diagonal tile
// (SwzTile<128>) or the V_t codes as 64-byte channel rows swizzled with (row / 4) % 4 and the
// 2 × 128 scale bytes of the tile's two key blocks. Both swizzles send the 16 rows read by a
// 16-lane group to 16 distinct 16-byte bank groups. V_t comes in the kernels' token-blocked
// layout (mx_quantize.hip): the bytes 16g..16g+15 of each 32-key block hold exactly the keys
// whose probabilities lane group g holds, so no data is permuted on chip.
#include "cfa_device.h"
#include "cfa_mx.h"

namespace cfa {

// The running maximum moves only when a tile's maximum exceeds it by more than 0.8 (log2
// units), so P̃ <= 2^0.8 = 1.741 and P̃·2^8 <= 445.7 still fits E4M3 (max 448) with the same
// fixed scale 2^-8: small probabilities keep exactly the range they have with threshold 0,
// while the rescaling of O (64 multiplies per lane) runs on far fewer tiles. A larger
// threshold would need a smaller fixed scale and push small probabilities into E4M3's
// subnormal range.
constexpr float RESCALE_LOG2_MX = 0.8f;

template <int QF>
struct MxFwdTile {
  static constexpr int BN = 64;
  static constexpr int D = 128;
  static constexpr int KROW = QF == 0 ? D : D / 2;   // bytes of one K_d row (6-bit: its 16-byte parts)
  static constexpr int OFF_KB = BN * KROW;           // K_d codes: 64 rows
  static constexpr int OFF_KSC = OFF_KB + (QF >= 2 ? BN * D / 4 : 0);   // 6-bit: 8-byte parts [chunk][row]
  static constexpr int OFF_V = OFF_KSC + BN * 4;     // K_d scales: 4 B per key
  static constexpr int OFF_VTSC = OFF_V + D * 64;    // V_t codes: 128 channel rows × 64 B
  static constexpr int STAGE = OFF_V + BN * 256;     // union with the bf16 V rows (64 × 256 B)
};

template <int HPW, int QF>
__global__ __launch_bounds__(256, 2) void attn_fwd_mx_kernel(
    const __bf16* __restrict__ q, uint8_t* __restrict__ qd, uint8_t* __restrict__ qd_sc, const uint8_t* __restrict__ kd,
    const uint8_t* __restrict__ kd_sc, const uint8_t* __restrict__ vt, const uint8_t* __restrict__ vt_sc,
    const __bf16* __restrict__ v, __bf16* __restrict__ o, float* __restrict__ lse, Plan plan,
    const int* __restrict__ padoff, int total_tokens, int t_pad, int hq, int hkv, int n_hb, float scale_log2,
    int causal) {
  using C = MxFwdTile<QF>;
  constexpr bool FP4 = QF == 1, FP6 = QF >= 2, NARROW = QF != 0;   // QF 2, 3: E2M3, E3M2
  constexpr int QROW = FP4 ? 64 : FP6 ? 96 : 128;     // bytes of one Q_d / K_d row in HBM
  constexpr int D = C::D;
  constexpr int BMW = 128 / HPW;
  __shared__ __attribute__((aligned(16))) char lds_a[C::STAGE];
  __shared__ __attribute__((aligned(16))) char lds_b[C::STAGE];

  const int wid = blockIdx.x;
  // work-item values are the same in every lane; readfirstlane keeps them in scalar registers
  const int p = __builtin_amdgcn_readfirstlane(wid / n_hb), hb = __builtin_amdgcn_readfirstlane(wid % n_hb);
  int s0, L, t, doc;
  if (!decode_item(plan, p, BMW, true, s0, L, t, &doc)) return;
  const int pcol = padoff[doc];                 // first token-blocked column of the document
  const int lp = 32 * ((L + 31) / 32);          // padded document length (columns)
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5, r32 = lane & 31;
  const int G = __builtin_amdgcn_readfirstlane(hq / hkv);
  const int h = hb * HPW + (w % HPW);
  const int g = __builtin_amdgcn_readfirstlane(h / G);
  const int wr0 = t * BMW + 32 * (w / HPW);
  const int wg_rows_end = min(L, (t + 1) * BMW);
  const int kv_end = causal ? wg_rows_end : L;
  const int n_kt = (kv_end + C::BN - 1) / C::BN;
  const int wave_last_key = causal ? min(L, wr0 + 32) - 1 : L - 1;
  const int qrow = wr0 + r32;
  const int diag_blk = causal ? (t * BMW) / 128 : -1;   // the wg's 128-row block
  const SwzOffsets<D> so(lane);
  int ko[2][2], vo[2];                          // lane-constant swizzled chunk offsets
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      ko[s][u] = NARROW ? 16 * ((2 * s + half) ^ vt_swz(r32)) : 16 * ((4 * s + 2 * u + half) ^ kd_swz(r32));
#pragma unroll
  for (int u = 0; u < 2; ++u) vo[u] = 16 * ((2 * u + half) ^ vt_swz(r32));

  // ---- Q quantised here, from the bf16 rows this wave owns (fused quantisation: Q is read once,
  // by the kernel that uses it), into the B operand of Sᵀ = K Qᵀ for the two 64-channel halves s,
  // and written out as the d-blocked Q_d (and scales) that the backward reuses. Lane (qrow, half)
  // supplies the scale of block 2s + half. E4M3: the operand holds channels 64s + 16·half + 0..15
  // (block 2s) and 64s + 32 + 16·half + 0..15 (block 2s + 1), so each block's maximum meets its
  // other 16 channels in the partner lane (l ^ 32); E2M1 / 6-bit: the lane holds all 32 channels
  // of block 2s + half.
  i32x8 qa[2];
  int qs[2];
  {
    const bool ok = qrow < L;
    const size_t row = (size_t)(s0 + (ok ? qrow : 0)) * hq + h;
    const __bf16* qr = q + row * D;
    auto ld = [&](int c) { return ok ? *(const i32x4*)(qr + c) : i32x4{0, 0, 0, 0}; };   // 8 channels from c
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (QF == 0) {
        uint32_t wa[8], wb[8];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const i32x4 ua = ld(64 * s + 16 * half + 8 * c), ub = ld(64 * s + 32 + 16 * half + 8 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wa[4 * c + e] = (uint32_t)ua[e];
            wb[4 * c + e] = (uint32_t)ub[e];
          }
        }
        const uint32_t ma = pair_max32_u(amax_bits<8>(wa)), mb = pair_max32_u(amax_bits<8>(wb));
        const int ea = e4m3_block_exp(ma), eb = e4m3_block_exp(mb);
        const bool bada = ma >= 0x7F80u, badb = mb >= 0x7F80u;
        const i32x4 lo = {bad_or(bada, 0x7F7F7F7F, e4m3_encode4(wa[0], wa[1], ea)),
                          bad_or(bada, 0x7F7F7F7F, e4m3_encode4(wa[2], wa[3], ea)),
                          bad_or(bada, 0x7F7F7F7F, e4m3_encode4(wa[4], wa[5], ea)),
                          bad_or(bada, 0x7F7F7F7F, e4m3_encode4(wa[6], wa[7], ea))};
        const i32x4 hi = {bad_or(badb, 0x7F7F7F7F, e4m3_encode4(wb[0], wb[1], eb)),
                          bad_or(badb, 0x7F7F7F7F, e4m3_encode4(wb[2], wb[3], eb)),
                          bad_or(badb, 0x7F7F7F7F, e4m3_encode4(wb[4], wb[5], eb)),
                          bad_or(badb, 0x7F7F7F7F, e4m3_encode4(wb[6], wb[7], eb))};
        qa[s] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        qs[s] = half ? (badb ? 0xFF : eb + 127) : (bada ? 0xFF : ea + 127);
        if (ok) {
          *(i32x4*)(qd + row * D + 64 * s + 16 * half) = lo;
          *(i32x4*)(qd + row * D + 64 * s + 32 + 16 * half) = hi;
        }
      } else {
        uint32_t w[16];                           // block 2s + half: channels 64s + 32·half + 0..31
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const i32x4 u = ld(64 * s + 32 * half + 8 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[4 * c + e] = (uint32_t)u[e];
        }
        const uint32_t m = amax_bits<16>(w);
        const bool bad = m >= 0x7F80u;
        if constexpr (FP4) {
          const int e = e2m1_block_exp(m);
          const i32x4 c4 = {bad_or(bad, 0, (int)e2m1_encode8(w, e)), bad_or(bad, 0, (int)e2m1_encode8(w + 4, e)),
                            bad_or(bad, 0, (int)e2m1_encode8(w + 8, e)), bad_or(bad, 0, (int)e2m1_encode8(w + 12, e))};
          qa[s] = fp4_operand(c4);
          qs[s] = bad ? 0xFF : e + 127;
          if (ok) *(i32x4*)(qd + row * (D / 2) + 32 * s + 16 * half) = c4;
        } else {
          const int e = e6_block_exp<QF>(m);
          u32x6 cw = e6_encode32<QF>(w, e);
          if (bad) cw = u32x6{0u, 0u, 0u, 0u, 0u, 0u};
          const i32x4 lo = {(int)cw[0], (int)cw[1], (int)cw[2], (int)cw[3]};
          const i32x2 hi = {(int)cw[4], (int)cw[5]};
          qa[s] = fp6_operand(lo, hi);
          qs[s] = bad ? 0xFF : e + 127;
          if (ok) {
            uint8_t* rp = qd + row * QROW;
            *(i32x4*)(rp + 16 * (2 * s + half)) = lo;
            *(i32x2*)(rp + D / 2 + 8 * (2 * s + half)) = hi;
          }
        }
      }
      if (ok) qd_sc[row * 4 + 2 * s + half] = (uint8_t)qs[s];
    }
  }
  f32x16 oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto tile_is_diag = [&](int kt) { return (kt * C::BN) / 128 == diag_blk; };
  // Tile kt -> LDS with direct copies. Keys past kv_end are clamped into the document (K_d,
  // bf16 V) or into its last token block (V_t); they are masked (P = 0).
  // Addresses: a wave-uniform 64-bit tile base plus a 32-bit lane offset within the tile.
  const uint32_t tok_b = (uint32_t)hkv * D;     // bytes between consecutive tokens of K_d (E4M3)
  auto stage = [&](int kt, char* tb) {
    const int k0 = kt * C::BN;
    const int rmax = kv_end - 1 - k0;
    const size_t tok0 = (size_t)(s0 + k0) * hkv + g;
    if constexpr (NARROW) {                     // K_d codes: 4 blocks of 16 rows, 1 per wave
      const uint8_t* kdb = kd + tok0 * QROW;
      const uint32_t rs = (uint32_t)hkv * QROW;
      const int r = 16 * w + (lane >> 2);
      g2lds16(kdb + ((uint32_t)min(r, rmax) * rs + 16 * ((lane & 3) ^ vt_swz(r))), tb + w * 1024);
      if (FP6 && w < 2)                         // 8-byte parts: chunk w of every row (lane = row)
        g2lds16(kdb + ((uint32_t)min(lane, rmax) * rs + D / 2 + 16 * w), tb + C::OFF_KB + w * 1024);
    } else {
      const uint8_t* kdb = kd + tok0 * D;
#pragma unroll
      for (int j = 0; j < 2; ++j) {             // K_d codes: 8 blocks of 8 rows, 2 per wave
        const int I = 2 * w + j, r = 8 * I + (lane >> 3);
        g2lds16(kdb + ((uint32_t)min(r, rmax) * tok_b + 16 * ((lane & 7) ^ kd_swz(r))), tb + I * 1024);
      }
    }
    if (w == 0) g2lds4(kd_sc + tok0 * 4 + (uint32_t)min(lane, rmax) * (uint32_t)hkv * 4, tb + C::OFF_KSC);
    if (tile_is_diag(kt)) {
      stage_rows_lds<C::BN>(tb + C::OFF_V, (const char*)(v + tok0 * D), tok_b * 2, rmax, w, lane);
    } else {
      const uint8_t* vtb = vt + (size_t)g * D * t_pad + pcol + k0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {             // V_t codes: 8 blocks of 16 channel rows, 2 per wave
        const int I = 2 * w + j, r = 16 * I + (lane >> 2);
        const int col = min(16 * ((lane & 3) ^ vt_swz(r)), lp - 16 - k0);
        g2lds16(vtb + (uint32_t)(r * t_pad + col), tb + C::OFF_V + I * 1024);
      }
      if (w == 1 && lane < 16) {                // V_t scales of the two key blocks
        const int blk = min((k0 >> 5) + (lane >> 3), lp / 32 - 1);
        g2lds16(vt_sc + ((size_t)g * (t_pad / 32) + (pcol >> 5) + blk) * D + 16 * (lane & 7), tb + C::OFF_VTSC);
      }
    }
  };

  stage(0, lds_a);
  wait_vmem();
  __syncthreads();

  auto iter = [&](int kt, const char* tb, char* nxt) __attribute__((always_inline)) {
    const int k0 = kt * C::BN;
    if (kt + 1 < n_kt) stage(kt + 1, nxt);
    if (k0 <= wave_last_key) {
      // ---- Sᵀ = K_d Q_dᵀ (scaled fp8, or fp4), the two 32-key blocks interleaved
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      int ksc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) ksc[b] = *(const int*)(tb + C::OFF_KSC + (32 * b + r32) * 4) >> (8 * half);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const char* kr = tb + (32 * b + r32) * C::KROW;
          // key block 2s + half's scale: byte 2s of the shifted word (the product's byte select)
          if constexpr (FP4) {
            sacc[b] = mfma32_scale_byte<4, 4>(fp4_operand(*(const i32x4*)(kr + ko[s][0])), ksc[b], 2 * s, qa[s], qs[s],
                                              sacc[b]);
          } else if constexpr (FP6) {
            const i32x2 hi = *(const i32x2*)(tb + C::OFF_KB + 16 * (64 * s + 32 * b + r32) + 8 * half);
            sacc[b] = mfma32_scale_byte<QF, QF>(fp6_operand(*(const i32x4*)(kr + ko[s][0]), hi), ksc[b], 2 * s, qa[s],
                                                qs[s], sacc[b]);
          } else {
            const i32x4 lo = *(const i32x4*)(kr + ko[s][0]);
            const i32x4 hi = *(const i32x4*)(kr + ko[s][1]);
            sacc[b] = mfma32_scale_byte<0, 0>(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, ksc[b], 2 * s,
                                              qa[s], qs[s], sacc[b]);
          }
        }
      // ---- online softmax: maximum on the raw scores (scale_log2 > 0), scale folded into the
      // exponent, masks only on tiles crossing the diagonal or the document end (wave-uniform)
      const bool need_mask = causal ? (k0 + C::BN - 1 > wr0) : (k0 + C::BN > L);
      if (need_mask) {
        const int lim = causal ? qrow : L - 1;      // keys above lim are masked (see attn_fwd.hip)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int r = lim - (k0 + 32 * b + 4 * half);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (8 * (j >> 2) + (j & 3) > r) sacc[b][j] = -INFINITY;
        }
      }
      const float mt = wave_max_xor32(max32(sacc[0], sacc[1])) * scale_log2;
      const bool upd = mt > m_run + RESCALE_LOG2_MX;
      if (__any(upd)) {
        const float m_new = upd ? mt : m_run;
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      }
      const bool diag = per_lane(tile_is_diag(kt));
      // diagonal tiles: P̃ (bf16); other tiles: P̃·2^8 (E4M3 with scale 2^-8)
      const float bias = diag ? -m_run : 8.f - m_run;
      // four partial row sums (short add chains), each started by its first term rather than by
      // adding it to 0 (the terms are >= +0, so the sums are the same)
      float ls4[4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pj = exp2_fast(fmaf(sacc[b][j], scale_log2, bias));
          sacc[b][j] = pj;
          if (b == 0 && j < 4) ls4[j] = pj;
          else ls4[j & 3] += pj;
        }
      const float ls = (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
      l_run += diag ? ls : ls * (1.f / 256.f);
      if (diag) {
        bf16x8 pf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          i32x4 u;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            u[e] = (int)pack_bf16x2(sacc[kk >> 1][8 * (kk & 1) + 2 * e], sacc[kk >> 1][8 * (kk & 1) + 2 * e + 1]);
          pf[kk] = __builtin_bit_cast(bf16x8, u);
        }
        const char* vb = tb + C::OFF_V;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int rb = (32 * (kk >> 1) + 16 * (kk & 1)) * 256;
          bf16x8 av[4];
#pragma unroll
          for (int db = 0; db < 4; ++db)
            av[db] = concat_tr(lds_read_tr16(vb + rb + so.tr0[db]), lds_read_tr16(vb + rb + so.tr1[db]));
#pragma unroll
          for (int db = 0; db < 4; ++db) oacc[db] = mfma32(av[db], pf[kk], oacc[db]);
        }
      } else {
        i32x8 pb;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[4 * b + e] = pack_fp8x4(sacc[b][4 * e], sacc[b][4 * e + 1], sacc[b][4 * e + 2], sacc[b][4 * e + 3]);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ch = 32 * db + r32;
          const char* vr = tb + C::OFF_V + ch * 64;
          const i32x4 lo = *(const i32x4*)(vr + vo[0]);
          const i32x4 hi = *(const i32x4*)(vr + vo[1]);
          const int sa = *(const uint8_t*)(tb + C::OFF_VTSC + half * 128 + ch);
          oacc[db] = mfma32_mx(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, sa, pb, 127 - 8, oacc[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    iter(kt, lds_a, lds_b);
    if (kt + 1 < n_kt) iter(kt + 1, lds_b, lds_a);
  }

  const float l_tot = wave_sum_xor32(l_run);
  if (qrow < L) {
    const float inv = 1.f / l_tot;
    __bf16* dst = o + ((size_t)(s0 + qrow) * hq + h) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        i32x2 u;
        u.x = (int)pack_bf16x2(oacc[db][4 * jg] * inv, oacc[db][4 * jg + 1] * inv);
        u.y = (int)pack_bf16x2(oacc[db][4 * jg + 2] * inv, oacc[db][4 * jg + 3] * inv);
        *(i32x2*)(dst + 32 * db + 8 * jg) = u;
      }
    if (half == 0) lse[(size_t)h * total_tokens + s0 + qrow] = (m_run + __log2f(l_tot)) * LN2;
  }
}

hipError_t launch_fwd_mx(const void* q, uint8_t* qd, uint8_t* qd_sc, const uint8_t* kd, const uint8_t* kd_sc,
                         const uint8_t* vt, const uint8_t* vt_sc, const void* v, void* o, float* lse,
                         const Plan& plan_any, const int* pref_base, const int* padoff, int total_tokens, int t_pad,
                         int hq, int hkv, float scale, int causal, int qf, hipStream_t stream) {
  const int G = hq / hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  const int rows = 128 / hpw;
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(rows) * (plan.n_docs + 1);
  const int n_hb = hq / hpw;
  const long grid = ((long)(total_tokens + rows - 1) / rows + plan.n_docs) * n_hb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const float sl2 = scale * LOG2E;
#define CFA_MXF_LAUNCH(HH, F4)                                                                                 \
  hipLaunchKernelGGL((attn_fwd_mx_kernel<HH, F4>), dim3((unsigned)grid), dim3(256), 0, stream, (const __bf16*)q, qd,   \
                     qd_sc, kd, kd_sc,                                                                           \
                     vt, vt_sc, (const __bf16*)v, (__bf16*)o, lse, plan, padoff, total_tokens, t_pad, hq, hkv, n_hb, sl2, \
                     causal)
  if (qf == 1) {
    if (hpw == 4) CFA_MXF_LAUNCH(4, 1);
    else if (hpw == 2) CFA_MXF_LAUNCH(2, 1);
    else CFA_MXF_LAUNCH(1, 1);
  } else if (qf == 2) {
    if (hpw == 4) CFA_MXF_LAUNCH(4, 2);
    else if (hpw == 2) CFA_MXF_LAUNCH(2, 2);
    else CFA_MXF_LAUNCH(1, 2);
  } else if (qf == 3) {
    if (hpw == 4) CFA_MXF_LAUNCH(4, 3);
    else if (hpw == 2) CFA_MXF_LAUNCH(2, 3);
    else CFA_MXF_LAUNCH(1, 3);
  } else {
    if (hpw == 4) CFA_MXF_LAUNCH(4, 0);
    else if (hpw == 2) CFA_MXF_LAUNCH(2, 0);
    else CFA_MXF_LAUNCH(1, 0);
  }
#undef CFA_MXF_LAUNCH
  return hipGetLastError();
}

}  // namespace cfa

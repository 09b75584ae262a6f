// MXFP8 causal attention backward for gfx950 (d = 128), deterministic.
//
// Same derivative and work split as the bf16 backward (attn_bwd.hip); the operands follow the
// MXFP8 reading of the FLAMIA page ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri": token-block
// scaling reused across matrix orientations, causal-leakage safeguards, exact forward/backward
// consistency), each product blocked along its contraction axis:
//  * S = Q_d K_dᵀ from the forward's own Q_d/K_d bytes, so P = exp(S − LSE) reproduces the
//    forward's probabilities; dP = dO_d V_dᵀ. Both contract over d (scale per token).
//  * dV += Pᵀ dO contracts over tokens. Off the diagonal 128×128 tile it uses the token-blocked
//    copy dO_t (one scale per channel and 32 doc-local tokens) and P (normalised, so ~1/L)
//    encoded E4M3 with an MX scale computed in registers per 32 contraction elements; on the
//    diagonal tile it stays bf16 (bf16 MFMA, transposing LDS reads), so no scale spans a
//    query's future.
//  * dK += dSᵀ Q and dQ += dS K take bf16 dS and the bf16 Q / K rows on every tile. dS needs
//    about 8 significant bits here (one E4M3 rounding, relative error up to 2^-4, alone costs
//    ~3% rel-L2 in dQ and dK), and on gfx950 two E4M3 products (value and rounding residual)
//    over 64 contraction elements take exactly the matrix-core time of bf16 products over the
//    same 64, while the second term's block maxima, encoding and residual cost ~75 vector
//    instructions per 32×32 block; the bf16 pack costs 8.
// Token-blocked tiles are staged with the 4-byte chunk order (0,2,4,6,1,3,5,7) per 32-token
// block so that the A operand read at offset 16h matches the lane's P register order.
#include "cfa_device.h"
#include "cfa_kernels.h"

namespace cfa {

// One 32-element contraction block, this lane's 16 values: encode x·2^-e into the 4 words the
// lane contributes to a B operand (exponents from fit_exp keep |x|·2^-e <= 448).
__device__ inline i32x4 encode16(const f32x16& x, int e) {
  const float s = pow2i(e);
  i32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = pack_fp8x4_scaled(x[4 * k], x[4 * k + 1], x[4 * k + 2], x[4 * k + 3], s);
  return r;
}

// Largest of 16 non-negative values (probabilities): two v_max3 chains, then their maximum.
__device__ inline float max16_nonneg(const f32x16& x) {
  float m[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    m[k] = fmaxf(fmaxf(x[8 * k], x[8 * k + 1]), x[8 * k + 2]);
    m[k] = fmaxf(fmaxf(m[k], x[8 * k + 3]), x[8 * k + 4]);
    m[k] = fmaxf(fmaxf(m[k], x[8 * k + 5]), x[8 * k + 6]);
    m[k] = fmaxf(m[k], x[8 * k + 7]);
  }
  return fmaxf(m[0], m[1]);
}

// Block exponent for values quantised inside the kernel (P): the smallest e with
// amax·2^-e <= 448, so the largest element is never clipped (the operand rule of mx_quantize
// may clip it by up to 1/8, which the oracle models for Q/K/V/dO but not here). Read off the
// bits of amax >= 0: for amax in [2^E, 2^(E+1)), amax·2^-(E-8) = 1.m·2^8 exceeds 448 = 1.75·2^8
// exactly when the mantissa field exceeds 0x600000. Zero and subnormal amax give -127.
__device__ inline int fit_exp(float amax) {
  const uint32_t b = __builtin_bit_cast(uint32_t, amax);
  const int e = (int)(b >> 23) - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return min(max(e, -127), 127);
}

__device__ inline i32x8 load_a_fp8(const char* row, int half) {
  const i32x4 lo = *(const i32x4*)(row + 16 * half);
  const i32x4 hi = *(const i32x4*)(row + 32 + 16 * half);
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// ------------------------------------------------------------------ dK / dV (wave pairs)
// 8 waves own 128 keys of one kv head as 4 pairs of 32 keys; a step is 64 queries of one query
// head (two 32-query blocks: one MX block along the token-contracted products).
//  * P wave (w < 4): K_d of its keys in registers. S = Q_d K_dᵀ (scaled fp8), P = exp(S − LSE),
//    P to the exchange buffer (bf16), dVᵀ += dO_tᵀ P with P MX-encoded per 32-query block, or
//    dOᵀ P in bf16 on diagonal steps.
//  * dS wave (w + 4), one step behind: V_d in registers. dP = dO_d V_dᵀ, dS = P (dP − D) with
//    its partner's P, dKᵀ += Qᵀ dS in bf16 (transposing reads of the bf16 Q rows).
// Each role stages its own operands by direct global -> LDS copies into two static buffers:
//   P wave:  [Q_d codes 64 × 128 B][Q_d scales 64 × 4][LSE·log2 e][dO_t 128 × 64 B + 2 × 128 scales | bf16 dO rows]
//   dS wave: [dO_d codes][dO_d scales][D][bf16 Q rows]
// Iteration i: P waves copy step i+1 and compute step i; dS waves copy step i and compute step
// i−1 (P of step i−1 sits in exchange buffer (i−1) mod 2). Every buffer is a separate static
// array and the loop is unrolled twice, so no copy in flight aliases a buffer being read.
struct MxDkdvTile {
  static constexpr int BM = 64;
  static constexpr int OFF_SC = BM * 128;            // d-blocked codes: 64 rows × 128 B (kd_swz)
  static constexpr int OFF_ROW = OFF_SC + BM * 4;    // 4 scale bytes per row
  static constexpr int OFF_U = OFF_ROW + BM * 4;     // LSE·log2 e or D: 64 floats
  static constexpr int OFF_TSC = OFF_U + 128 * 64;   // token-blocked codes: 128 rows × 64 B (vt_swz)
  static constexpr int BUF = OFF_U + BM * 256;       // union with 64 bf16 rows (SwzTile<128>)
  static constexpr int XP = 4 * 4 * 64;              // exchange: i32x4 [pair][2·qb + u][lane]
};

// QF = 1 (MXFP4/FP8 path): the P wave's score product takes E2M1 Q_d rows (64 bytes, swizzled
// with (row / 4) % 4) and E2M1 K_d registers; QF = 2 (MXFP6/FP8): E2M3 rows, whose 16-byte parts
// are staged like the E2M1 rows and whose 8-byte parts follow chunk-major (two 16-byte chunks
// per row); QF = 3: E3M2 in the same storage; everything else is unchanged.
template <int QF>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_mx_kernel(
    const uint8_t* __restrict__ qd, const uint8_t* __restrict__ qd_sc, const uint8_t* __restrict__ kd,
    const uint8_t* __restrict__ kd_sc, const uint8_t* __restrict__ dod, const uint8_t* __restrict__ dod_sc,
    const uint8_t* __restrict__ vd, const uint8_t* __restrict__ vd_sc, const uint8_t* __restrict__ dot,
    const uint8_t* __restrict__ dot_sc, const __bf16* __restrict__ q, const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, __bf16* __restrict__ dk, __bf16* __restrict__ dv, Plan plan,
    const int* __restrict__ padoff, int total_tokens, int t_pad, int hq, int hkv, float scale, int causal) {
  using C = MxDkdvTile;
  constexpr int D = 128, BM = C::BM;
  __shared__ i32x4 xp_a[C::XP];
  __shared__ i32x4 xp_b[C::XP];
  __shared__ __attribute__((aligned(16))) char pb_a[C::BUF];
  __shared__ __attribute__((aligned(16))) char pb_b[C::BUF];
  __shared__ __attribute__((aligned(16))) char sb_a[C::BUF];
  __shared__ __attribute__((aligned(16))) char sb_b[C::BUF];

  const int p = __builtin_amdgcn_readfirstlane(blockIdx.x / hkv), g = __builtin_amdgcn_readfirstlane(blockIdx.x % hkv);
  int s0, L, t, doc;
  if (!decode_item(plan, p, 128, false, s0, L, t, &doc)) return;
  const int pcol = padoff[doc];
  const int lp = 32 * ((L + 31) / 32);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5,
            r32 = lane & 31;
  const int pair = w & 3;
  const bool ds_wave = w >= 4;
  const int G = __builtin_amdgcn_readfirstlane(hq / hkv);
  const int kw0 = t * 128 + 32 * pair;
  const int mykey = kw0 + r32;
  const float sl2 = scale * LOG2E;
  int ko[2][2], to[2], kq[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u) ko[s][u] = 16 * ((4 * s + 2 * u + half) ^ kd_swz(r32));
#pragma unroll
  for (int u = 0; u < 2; ++u) to[u] = 16 * ((2 * u + half) ^ vt_swz(r32));
#pragma unroll
  for (int s = 0; s < 2; ++s) kq[s] = 16 * ((2 * s + half) ^ vt_swz(r32));
  constexpr bool FP4 = QF == 1, FP6 = QF >= 2;   // QF 2, 3: E2M3, E3M2
  constexpr int F6 = FP6 ? QF : 2;                // 6-bit format code (any valid one when unused)
  constexpr int QROW = FP4 ? 64 : FP6 ? 96 : 128;  // bytes of one Q_d / K_d row in HBM
  const bool narrow_role = QF != 0 && !ds_wave;    // this wave's score operands are E2M1 / E2M3

  // B operand rows of key mykey: K_d (P wave) or V_d (dS wave)
  i32x8 kvb[2];
  int kvs[2];
  {
    const bool ok = mykey < L;
    const uint8_t* src = ds_wave ? vd : kd;
    const uint8_t* ssrc = ds_wave ? vd_sc : kd_sc;
    const size_t row = (size_t)(s0 + (ok ? mykey : 0)) * hkv + g;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (FP4 && narrow_role)
        kvb[s] = ok ? fp4_operand(*(const i32x4*)(kd + row * (D / 2) + 32 * s + 16 * half)) : i32x8{};
      else if (FP6 && narrow_role)
        kvb[s] = ok ? fp6_operand(*(const i32x4*)(kd + row * QROW + 16 * (2 * s + half)),
                                  *(const i32x2*)(kd + row * QROW + D / 2 + 8 * (2 * s + half)))
                    : i32x8{};
      else
        kvb[s] = ok ? load_a_fp8((const char*)(src + row * D + 64 * s), half) : i32x8{};
      kvs[s] = ok ? ssrc[row * 4 + 2 * s + half] : 127;
    }
  }
  f32x16 acc[4];                                  // dVᵀ (P wave) or dKᵀ (dS wave)
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};

  const int q_begin = causal ? t * 128 : 0;
  const int n_qt = __builtin_amdgcn_readfirstlane((L - q_begin + BM - 1) / BM);
  const int n_steps = n_qt * G;
  const int wave_first_q = causal ? kw0 : 0;
  // A step's position: its query head and first doc-local query. Steps run query tiles ascending
  // from the diagonal with the heads outer; each role walks them one per iteration (uniform
  // values, no division per step).
  struct Pos {
    int h, q0;
  };
  auto next_pos = [&](Pos ps) {
    ps.q0 += BM;
    if (ps.q0 >= L) {
      ps.q0 = q_begin;
      ++ps.h;
    }
    return ps;
  };
  auto step_is_diag = [&](int q0) { return causal && (q0 >> 7) == t; };
  auto active = [&](int q0) { return q0 + BM - 1 >= wave_first_q && kw0 < L; };

  // Operands of the step at position ps for this wave's role -> buffer. Rows past the document
  // end are clamped into it (d-blocked, bf16) or into its last token block (token-blocked); they
  // are masked. Each wave fetches the step's 64 LSE or D values into a register; the second
  // wave of each role writes them to the buffer after the step's compute (stage_finish).
  float rreg = 0.f;
  // Lane offsets of the copies from a step's first row (first column for the token-blocked
  // copy), the same for every step; a step whose 64 queries all lie inside the document uses
  // them as they are (rows past the document end only occur on its last step, which clamps).
  const uint32_t tok_b = (uint32_t)hq * D;
  const uint32_t nrs = (uint32_t)hq * QROW;       // narrow Q_d row stride
  uint32_t dof[2], tof[2];
  const uint32_t nof = (uint32_t)(16 * pair + (lane >> 2)) * nrs + 16 * ((lane & 3) ^ vt_swz(16 * pair + (lane >> 2)));
  const uint32_t nof6 = (uint32_t)lane * nrs + D / 2 + 16 * pair;
  const uint32_t sof = (uint32_t)lane * (uint32_t)hq * 4;
  const uint32_t tsof = (uint32_t)(lane >> 3) * D + 16 * (lane & 7);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int I = 2 * pair + j, r = 8 * I + (lane >> 3), rt = 16 * I + (lane >> 2);
    dof[j] = (uint32_t)r * tok_b + 16 * ((lane & 7) ^ kd_swz(r));
    tof[j] = (uint32_t)(rt * t_pad) + 16 * ((lane & 3) ^ vt_swz(rt));
  }
  const RowCopies<BM, 4, 128> rows((uint32_t)hq * D * 2, pair, lane);
  auto stage = [&](Pos ps, char* buf) {
    const int h = ps.h, q0 = ps.q0;
    const int rmax = L - 1 - q0;
    const size_t tok0 = (size_t)(s0 + q0) * hq + h;
    // every wave loads the step's LSE or D row (one load site, so the register needs no copy
    // between the two staging paths below, which would wait for the tile copies); pair 1 stores it
    rreg = (ds_wave ? delta : lse)[(size_t)h * total_tokens + s0 + q0 + min(lane, rmax)];
    if (rmax >= BM - 1) {                       // the whole step lies inside the document
      if (narrow_role) {
        const auto rs = rsrc_at(qd + tok0 * QROW, 0x7fffffffu);
        b2lds16(rs, nof, buf + pair * 1024);
        if (FP6 && pair < 2) b2lds16(rs, nof6, buf + 4096 + pair * 1024);
      } else {
        const auto rs = rsrc_at((ds_wave ? dod : qd) + tok0 * D, 0x7fffffffu);
#pragma unroll
        for (int j = 0; j < 2; ++j) b2lds16(rs, dof[j], buf + (2 * pair + j) * 1024);
      }
      if (pair == 0) b2lds4(rsrc_at((ds_wave ? dod_sc : qd_sc) + tok0 * 4, 0x7fffffffu), sof, buf + C::OFF_SC);
      if (ds_wave || step_is_diag(q0)) {
        rows.copy(buf + C::OFF_U, (ds_wave ? q : dout) + tok0 * D, rmax, pair);
      } else {
        const auto rs = rsrc_at(dot + (size_t)h * D * t_pad + pcol + q0, 0x7fffffffu);
#pragma unroll
        for (int j = 0; j < 2; ++j) b2lds16(rs, tof[j], buf + C::OFF_U + (2 * pair + j) * 1024);
        if (pair == 2 && lane < 16)
          b2lds16(rsrc_at(dot_sc + ((size_t)h * (t_pad / 32) + ((pcol + q0) >> 5)) * D, 0x7fffffffu), tsof,
                  buf + C::OFF_TSC);
      }
      return;
    }
    // the document's last step: rows past its end are clamped into it (d-blocked, bf16) or into
    // its last token block (token-blocked); they are masked
    if (narrow_role) {                          // E2M1 / E2M3 Q_d codes: 4 blocks of 16 rows of 64 B
      const uint8_t* dsrc = qd + tok0 * QROW;
      const int r = 16 * pair + (lane >> 2);
      g2lds16(dsrc + ((uint32_t)min(r, rmax) * nrs + 16 * ((lane & 3) ^ vt_swz(r))), buf + pair * 1024);
      if (FP6 && pair < 2)                      // E2M3 8-byte parts: chunk `pair` of every row
        g2lds16(dsrc + ((uint32_t)min(lane, rmax) * nrs + D / 2 + 16 * pair), buf + 4096 + pair * 1024);
    } else {
      const uint8_t* dsrc = (ds_wave ? dod : qd) + tok0 * D;
#pragma unroll
      for (int j = 0; j < 2; ++j) {             // d-blocked codes: 8 blocks of 8 rows
        const int I = 2 * pair + j, r = 8 * I + (lane >> 3);
        g2lds16(dsrc + ((uint32_t)min(r, rmax) * tok_b + 16 * ((lane & 7) ^ kd_swz(r))), buf + I * 1024);
      }
    }
    if (pair == 0)
      g2lds4((ds_wave ? dod_sc : qd_sc) + tok0 * 4 + (uint32_t)min(lane, rmax) * (uint32_t)hq * 4, buf + C::OFF_SC);
    if (ds_wave || step_is_diag(q0)) {
      stage_rows_lds<BM>(buf + C::OFF_U, (const char*)((ds_wave ? q : dout) + tok0 * D), tok_b * 2, rmax, pair, lane);
    } else {
      const uint8_t* tsrc = dot + (size_t)h * D * t_pad + pcol + q0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {             // token-blocked codes: 8 blocks of 16 channel rows
        const int I = 2 * pair + j, r = 16 * I + (lane >> 2);
        const int col = min(16 * ((lane & 3) ^ vt_swz(r)), lp - 16 - q0);
        g2lds16(tsrc + (uint32_t)(r * t_pad + col), buf + C::OFF_U + I * 1024);
      }
      if (pair == 2 && lane < 16) {
        const int blk = min((q0 >> 5) + (lane >> 3), lp / 32 - 1);
        g2lds16(dot_sc + ((size_t)h * (t_pad / 32) + (pcol >> 5) + blk) * D + 16 * (lane & 7), buf + C::OFF_TSC);
      }
    }
  };
  auto stage_finish = [&](char* buf) {
    if (pair == 1) ((float*)(buf + C::OFF_ROW))[lane] = ds_wave ? -rreg : rreg * LOG2E;   // dS wave: -D
  };

  // scores of 32-query block qb of the step against this pair's keys (A = d-blocked rows),
  // accumulated onto a0
  auto dscores = [&](const char* buf, int qb, f32x16 a0) __attribute__((always_inline)) {
    const int qr = 32 * qb + r32;
    // the row's four block scales; this lane's blocks are 2s + half (s = 0, 1): bytes 2s of scw
    const int scw = *(const int*)(buf + C::OFF_SC + qr * 4) >> (8 * half);
    f32x16 a = a0;
    if (FP4 && narrow_role) {
      const char* rp = buf + qr * (D / 2);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        a = mfma32_scale_byte<4, 4>(fp4_operand(*(const i32x4*)(rp + kq[s])), scw, 2 * s, kvb[s], kvs[s], a);
    } else if (FP6 && narrow_role) {
      const char* rp = buf + qr * (D / 2);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        a = mfma32_scale_byte<F6, F6>(
            fp6_operand(*(const i32x4*)(rp + kq[s]), *(const i32x2*)(buf + 4096 + 16 * (64 * s + qr) + 8 * half)),
            scw, 2 * s, kvb[s], kvs[s], a);
    } else {
      const char* rp = buf + qr * 128;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const i32x4 lo = *(const i32x4*)(rp + ko[s][0]), hi = *(const i32x4*)(rp + ko[s][1]);
        a = mfma32_scale_byte<0, 0>(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, scw, 2 * s, kvb[s],
                                    kvs[s], a);
      }
    }
    return a;
  };

  // P wave, step st; the two query blocks one after the other
  auto step_p = [&](int q0, const char* buf, i32x4* xw) __attribute__((always_inline)) {
    const bool diag = per_lane(step_is_diag(q0));
    const bool masked = (causal && q0 < kw0 + 31) || q0 + BM > L;   // wave-uniform
    const f32x4* l2 = (const f32x4*)(buf + C::OFF_ROW);
    i32x4 pw[4];                                // bf16 P: exchange words and diagonal B operands
    i32x8 pb8;                                  // E4M3 P (off-diagonal steps)
    int psc = 127;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 x = dscores(buf, qb, f32x16{});
      if (masked) {
        // element j holds query qb0 + 8(j/4) + j%4: masked below lo (causal) or above hi
        const int qb0 = q0 + 32 * qb + 4 * half;
        const int lo = causal ? mykey - qb0 : -1, hi = L - 1 - qb0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int c = 8 * (j >> 2) + (j & 3);
          if ((c < lo) | (c > hi)) x[j] = -INFINITY;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 lr = l2[8 * qb + 2 * jj + half];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[4 * jj + u] = exp2_fast(fmaf(x[4 * jj + u], sl2, -lr[u]));
        pw[2 * qb + (jj >> 1)][2 * (jj & 1)] = (int)pack_bf16x2(x[4 * jj], x[4 * jj + 1]);
        pw[2 * qb + (jj >> 1)][2 * (jj & 1) + 1] = (int)pack_bf16x2(x[4 * jj + 2], x[4 * jj + 3]);
      }
      xw[(pair * 4 + 2 * qb) * 64 + lane] = pw[2 * qb];
      xw[(pair * 4 + 2 * qb + 1) * 64 + lane] = pw[2 * qb + 1];
      if (!diag) {                              // MX block of 32 queries: exponent over the lane pair
        float a = max16_nonneg(x);
        a = wave_max_xor32(a);
        const int e = fit_exp(a);
        const i32x4 c = encode16(x, e);
#pragma unroll
        for (int k = 0; k < 4; ++k) pb8[4 * qb + k] = c[k];
        if (half == qb) psc = e + 127;
      }
    }
    if (diag) {
      const SwzOffsets<D> so(lane);
      const char* ob = buf + C::OFF_U;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int rb = (32 * (kk >> 1) + 16 * (kk & 1)) * 256;
        bf16x8 ao[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
          ao[db] = concat_tr(lds_read_tr16(ob + rb + so.tr0[db]), lds_read_tr16(ob + rb + so.tr1[db]));
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma32(ao[db], __builtin_bit_cast(bf16x8, pw[kk]), acc[db]);
      }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int ch = 32 * db + r32;
        const char* rp = buf + C::OFF_U + ch * 64;
        const i32x4 lo = *(const i32x4*)(rp + to[0]), hi = *(const i32x4*)(rp + to[1]);
        const int sa = *(const uint8_t*)(buf + C::OFF_TSC + half * 128 + ch);
        acc[db] = mfma32_mx(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, sa, pb8, psc, acc[db]);
      }
    }
  };

  // dS wave, step st (one iteration after its P wave); the query blocks one after the other.
  // The dP product accumulates onto -D (stored negated in the stage), so x = dP - D.
  auto step_ds = [&](const char* buf, const i32x4* xr) __attribute__((always_inline)) {
    const f32x4* dd = (const f32x4*)(buf + C::OFF_ROW);
    bf16x8 sf[4];                               // bf16 dS, B operands of the dK product
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 nd;                                // element 4m + c: query 32qb + 8m + 4·half + c
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 v4 = dd[8 * qb + 2 * m + half];
#pragma unroll
        for (int c = 0; c < 4; ++c) nd[4 * m + c] = v4[c];
      }
      f32x16 x = dscores(buf, qb, nd);          // dP - D
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const i32x4 pw = xr[(pair * 4 + 2 * qb + u) * 64 + lane];
        i32x4 us;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t word = (uint32_t)pw[2 * jj + e];
            const int j = 8 * u + 4 * jj + 2 * e;
            us[2 * jj + e] = (int)pack_bf16x2(__builtin_bit_cast(float, word << 16) * x[j],
                                              __builtin_bit_cast(float, word & 0xFFFF0000u) * x[j + 1]);
          }
        }
        sf[2 * qb + u] = __builtin_bit_cast(bf16x8, us);
      }
    }
    const SwzOffsets<D> so(lane);
    const char* qb_ = buf + C::OFF_U;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rb = (32 * (kk >> 1) + 16 * (kk & 1)) * 256;
      bf16x8 aq[4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
        aq[db] = concat_tr(lds_read_tr16(qb_ + rb + so.tr0[db]), lds_read_tr16(qb_ + rb + so.tr1[db]));
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = mfma32(aq[db], sf[kk], acc[db]);
    }
  };

  // Iteration i. The two roles run separate loops (so each keeps only its own addresses live);
  // both execute one barrier per iteration, n_steps + 1 iterations after the prologue barrier.
  // pc: position of the step this wave computes in the iteration (P: i, dS: i - 1); pn: of the
  // step it stages (P: i + 1, dS: i).
  Pos pc{g * G, q_begin}, pn = pc;
  auto iter_p = [&](int i, const char* pcur, char* pnxt, i32x4* xw) __attribute__((always_inline)) {
    if (i + 1 < n_steps) stage(pn, pnxt);
    if (i < n_steps && active(pc.q0)) step_p(pc.q0, pcur, xw);
    if (i + 1 < n_steps) stage_finish(pnxt);
    pc = pn;
    pn = next_pos(pn);
    wait_vmem();
    __syncthreads();
  };
  auto iter_ds = [&](int i, char* sload, const char* suse, const i32x4* xr) __attribute__((always_inline)) {
    if (i < n_steps) stage(pn, sload);
    if (i >= 1 && active(pc.q0)) step_ds(suse, xr);
    if (i < n_steps) stage_finish(sload);
    pc = pn;
    pn = next_pos(pn);
    wait_vmem();
    __syncthreads();
  };

  if (!ds_wave) {
    if (n_steps > 0) {
      stage(pn, pb_a);
      stage_finish(pb_a);
    }
    pn = next_pos(pn);
    wait_vmem();
    __syncthreads();
    for (int i = 0; i <= n_steps; i += 2) {
      iter_p(i, pb_a, pb_b, xp_a);
      if (i + 1 <= n_steps) iter_p(i + 1, pb_b, pb_a, xp_b);
    }
  } else {
    wait_vmem();                                // the V_d registers have landed
    __syncthreads();
    for (int i = 0; i <= n_steps; i += 2) {
      iter_ds(i, sb_a, sb_b, xp_b);
      if (i + 1 <= n_steps) iter_ds(i + 1, sb_b, sb_a, xp_a);
    }
  }

  // dS wave: dK = scale·dKᵀ; P wave: dV (lane: key mykey, d = 32 db + 8 jg + 4·half + 0..3)
  if (mykey < L) {
    const float f = ds_wave ? scale : 1.f;
    __bf16* dst = (ds_wave ? dk : dv) + ((size_t)(s0 + mykey) * hkv + g) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        i32x2 u;
        u.x = (int)pack_bf16x2(acc[db][4 * jg] * f, acc[db][4 * jg + 1] * f);
        u.y = (int)pack_bf16x2(acc[db][4 * jg + 2] * f, acc[db][4 * jg + 3] * f);
        *(i32x2*)(dst + 32 * db + 8 * jg) = u;
      }
  }
}

// ------------------------------------------------------------------ dQ
// A wave owns 32 queries of one head (Q_d, dO_d in registers as B operands); the workgroup
// walks key tiles of 64, staged by direct global -> LDS copies into two static buffers:
//   [K_d codes 64 × 128 B][K_d scales 64 × 4][V_d codes][V_d scales][K bf16 rows (SwzTile<128>)]
// (code rows XOR-swizzled as in the MX forward kernel). S and dP are scaled fp8 products; dQ
// takes bf16 dS and the bf16 K rows (transposing reads) on every tile.
struct MxDqTile {
  static constexpr int BN = 64;
  static constexpr int OFF_KDSC = BN * 128;
  static constexpr int OFF_VD = OFF_KDSC + BN * 4;
  static constexpr int OFF_VDSC = OFF_VD + BN * 128;
  static constexpr int OFF_U = OFF_VDSC + BN * 4;
  static constexpr int STAGE = OFF_U + BN * 256;
};

// QF = 1: the score product takes E2M1 K_d rows (64 bytes, swizzled with (row / 4) % 4) and E2M1
// Q_d registers; QF = 2 (E2M3), 3 (E3M2): 6-bit rows, their 8-byte parts chunk-major after the
// 16-byte parts.
template <int QF>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_mx_kernel(
    const uint8_t* __restrict__ qd, const uint8_t* __restrict__ qd_sc, const uint8_t* __restrict__ kd,
    const uint8_t* __restrict__ kd_sc, const uint8_t* __restrict__ dod, const uint8_t* __restrict__ dod_sc,
    const uint8_t* __restrict__ vd, const uint8_t* __restrict__ vd_sc, const __bf16* __restrict__ k,
    const float* __restrict__ lse, const float* __restrict__ delta, __bf16* __restrict__ dq, Plan plan,
    int total_tokens, int hq, int hkv, float scale, int causal) {
  using C = MxDqTile;
  constexpr int D = 128, BN = C::BN;
  constexpr bool FP4 = QF == 1, FP6 = QF >= 2;   // QF 2, 3: E2M3, E3M2
  constexpr int F6 = FP6 ? QF : 2;                // 6-bit format code (any valid one when unused)
  constexpr int QROW = FP4 ? 64 : FP6 ? 96 : 128;  // bytes of one Q_d / K_d row in HBM
  __shared__ __attribute__((aligned(16))) char lds_a[C::STAGE];
  __shared__ __attribute__((aligned(16))) char lds_b[C::STAGE];

  // work-item values are the same in every lane; readfirstlane keeps them in scalar registers
  const int p = __builtin_amdgcn_readfirstlane(blockIdx.x / hq), h = __builtin_amdgcn_readfirstlane(blockIdx.x % hq);
  int s0, L, t, doc;
  if (!decode_item(plan, p, 128, true, s0, L, t, &doc)) return;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = lane >> 5, r32 = lane & 31;
  const int g = __builtin_amdgcn_readfirstlane(h / (hq / hkv));
  const int wr0 = t * 128 + 32 * w;
  const int qrow = wr0 + r32;
  const int kv_end = causal ? min(L, (t + 1) * 128) : L;
  const int n_kt = (kv_end + BN - 1) / BN;
  const int wave_last_key = causal ? min(L, wr0 + 32) - 1 : L - 1;
  const float sl2 = scale * LOG2E;
  int ko[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u) ko[s][u] = 16 * ((4 * s + 2 * u + half) ^ kd_swz(r32));
  int kq[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) kq[s] = 16 * ((2 * s + half) ^ vt_swz(r32));

  i32x8 qa[2], oa[2];
  int qs[2], os[2];
  float lse2 = INFINITY, dl = 0.f;
  {
    const bool ok = qrow < L;
    const size_t row = (size_t)(s0 + (ok ? qrow : 0)) * hq + h;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (FP4)
        qa[s] = ok ? fp4_operand(*(const i32x4*)(qd + row * (D / 2) + 32 * s + 16 * half)) : i32x8{};
      else if constexpr (FP6)
        qa[s] = ok ? fp6_operand(*(const i32x4*)(qd + row * QROW + 16 * (2 * s + half)),
                                 *(const i32x2*)(qd + row * QROW + D / 2 + 8 * (2 * s + half)))
                   : i32x8{};
      else
        qa[s] = ok ? load_a_fp8((const char*)(qd + row * D + 64 * s), half) : i32x8{};
      oa[s] = ok ? load_a_fp8((const char*)(dod + row * D + 64 * s), half) : i32x8{};
      qs[s] = ok ? qd_sc[row * 4 + 2 * s + half] : 127;
      os[s] = ok ? dod_sc[row * 4 + 2 * s + half] : 127;
    }
    if (ok) {
      lse2 = lse[(size_t)h * total_tokens + s0 + qrow] * LOG2E;
      dl = delta[(size_t)h * total_tokens + s0 + qrow];
    }
  }
  f32x16 dqa[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) dqa[b] = f32x16{};

  // key tile -> LDS through buffer resources that end after the document's last row: keys past
  // kv_end read zeros and are masked (P = 0). The lane offsets from a tile's first row are the
  // same for every tile.
  const uint32_t krow_b = (uint32_t)hkv * D;      // bytes between consecutive tokens (codes, bf16/2)
  const uint32_t nrs = (uint32_t)hkv * QROW;      // narrow K_d row stride
  uint32_t dof[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * (2 * w + j) + (lane >> 3);
    dof[j] = (uint32_t)r * krow_b + 16 * ((lane & 7) ^ kd_swz(r));
  }
  const uint32_t nof = (uint32_t)(16 * w + (lane >> 2)) * nrs + 16 * ((lane & 3) ^ vt_swz(16 * w + (lane >> 2)));
  const uint32_t nof6 = (uint32_t)lane * nrs + D / 2 + 16 * w;
  const uint32_t sof = (uint32_t)lane * (uint32_t)hkv * 4;
  const RowCopies<BN, 4, 128> rows(krow_b * 2, w, lane);
  auto stage = [&](int ktile, char* tb) {
    const int k0 = ktile * BN;
    const int rmax = kv_end - 1 - k0;             // last row inside the document
    const size_t tok0 = (size_t)(s0 + k0) * hkv + g;
    auto ends = [&](uint32_t stride, uint32_t row_bytes) {
      return rmax >= BN - 1 ? 0x7fffffffu : (uint32_t)rmax * stride + row_bytes;
    };
    const auto rv = rsrc_at(vd + tok0 * D, ends(krow_b, D));
#pragma unroll
    for (int j = 0; j < 2; ++j) {               // K_d and V_d codes: 8 blocks of 8 rows each
      if constexpr (QF == 0) b2lds16(rsrc_at(kd + tok0 * D, ends(krow_b, D)), dof[j], tb + (2 * w + j) * 1024);
      b2lds16(rv, dof[j], tb + C::OFF_VD + (2 * w + j) * 1024);
    }
    if constexpr (QF != 0) {                    // E2M1 / E2M3 K_d codes: 4 blocks of 16 rows of 64 B
      const auto rk = rsrc_at(kd + tok0 * QROW, ends(nrs, QROW));
      b2lds16(rk, nof, tb + w * 1024);
      if (FP6 && w < 2) b2lds16(rk, nof6, tb + 4096 + w * 1024);   // E2M3 8-byte parts: chunk w of every row
    }
    if (w == 0) b2lds4(rsrc_at(kd_sc + tok0 * 4, ends(hkv * 4, 4)), sof, tb + C::OFF_KDSC);
    if (w == 1) b2lds4(rsrc_at(vd_sc + tok0 * 4, ends(hkv * 4, 4)), sof, tb + C::OFF_VDSC);
    rows.copy(tb + C::OFF_U, k + tok0 * D, rmax, w);
  };

  // dS of one 32-key block b of the tile (this lane: query qrow, keys k0 + 32b + 8(j/4) + 4·half + j%4)
  auto ds_block = [&](const char* tb, int k0, int b, bool need_mask) __attribute__((always_inline)) {
    const int kr = 32 * b + r32;
    // the key's four block scales; this lane's blocks are 2s + half (s = 0, 1): bytes 2s
    const int ksc = *(const int*)(tb + C::OFF_KDSC + kr * 4) >> (8 * half);
    const int vsc = *(const int*)(tb + C::OFF_VDSC + kr * 4) >> (8 * half);
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const char* vp = tb + C::OFF_VD + kr * 128;
      const i32x4 vlo = *(const i32x4*)(vp + ko[s][0]), vhi = *(const i32x4*)(vp + ko[s][1]);
      if constexpr (FP4) {
        sacc = mfma32_scale_byte<4, 4>(fp4_operand(*(const i32x4*)(tb + kr * (D / 2) + kq[s])), ksc, 2 * s, qa[s],
                                       qs[s], sacc);
      } else if constexpr (FP6) {
        sacc = mfma32_scale_byte<F6, F6>(fp6_operand(*(const i32x4*)(tb + kr * (D / 2) + kq[s]),
                                                 *(const i32x2*)(tb + 4096 + 16 * (64 * s + kr) + 8 * half)),
                                     ksc, 2 * s, qa[s], qs[s], sacc);
      } else {
        const char* kp = tb + kr * 128;
        const i32x4 klo = *(const i32x4*)(kp + ko[s][0]), khi = *(const i32x4*)(kp + ko[s][1]);
        sacc = mfma32_scale_byte<0, 0>(i32x8{klo.x, klo.y, klo.z, klo.w, khi.x, khi.y, khi.z, khi.w}, ksc, 2 * s,
                                       qa[s], qs[s], sacc);
      }
      pacc = mfma32_scale_byte<0, 0>(i32x8{vlo.x, vlo.y, vlo.z, vlo.w, vhi.x, vhi.y, vhi.z, vhi.w}, vsc, 2 * s,
                                     oa[s], os[s], pacc);
    }
    if (need_mask) {                     // wave-uniform: diagonal or document-end tiles
      const int r = (causal ? qrow : L - 1) - (k0 + 32 * b + 4 * half);   // keys above are masked
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > r) sacc[j] = -INFINITY;
    }
    f32x16 x;
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = exp2_fast(fmaf(sacc[j], sl2, -lse2)) * (pacc[j] - dl);
    return x;
  };

  // one key tile: bf16 dS and bf16 K (transposing reads)
  auto tile = [&](const char* tb, int k0, bool need_mask) __attribute__((always_inline)) {
    bf16x8 sf[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x16 x = ds_block(tb, k0, b, need_mask);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        i32x4 us;
#pragma unroll
        for (int e = 0; e < 4; ++e) us[e] = (int)pack_bf16x2(x[8 * u + 2 * e], x[8 * u + 2 * e + 1]);
        sf[2 * b + u] = __builtin_bit_cast(bf16x8, us);
      }
    }
    const SwzOffsets<D> so(lane);
    const char* kb = tb + C::OFF_U;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rb = (32 * (kk >> 1) + 16 * (kk & 1)) * 256;
      bf16x8 ak[4];
#pragma unroll
      for (int dbk = 0; dbk < 4; ++dbk)
        ak[dbk] = concat_tr(lds_read_tr16(kb + rb + so.tr0[dbk]), lds_read_tr16(kb + rb + so.tr1[dbk]));
#pragma unroll
      for (int dbk = 0; dbk < 4; ++dbk) dqa[dbk] = mfma32(ak[dbk], sf[kk], dqa[dbk]);
    }
  };

  auto iter = [&](int ktile, const char* tb, char* nxt) __attribute__((always_inline)) {
    const int k0 = ktile * BN;
    if (ktile + 1 < n_kt) stage(ktile + 1, nxt);
    if (k0 <= wave_last_key) {
      const bool need_mask = causal ? (k0 + BN - 1 > wr0) : (k0 + BN > L);
      tile(tb, k0, need_mask);
    }
    wait_vmem();
    __syncthreads();
  };

  if (n_kt > 0) stage(0, lds_a);
  wait_vmem();
  __syncthreads();
  for (int ktile = 0; ktile < n_kt; ktile += 2) {
    iter(ktile, lds_a, lds_b);
    if (ktile + 1 < n_kt) iter(ktile + 1, lds_b, lds_a);
  }

  if (qrow < L) {
    __bf16* dst = dq + ((size_t)(s0 + qrow) * hq + h) * D + 4 * half;
#pragma unroll
    for (int dbk = 0; dbk < 4; ++dbk)
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
hipError_t launch_bwd_dkdv_mx(const MxOperands& m, const void* q, const void* dout, const float* lse,
                              const float* delta, void* dk, void* dv, const Plan& plan_any, const int* pref_base,
                              const int* padoff, int T, int t_pad, int hq, int hkv, float scale, int causal,
                              int qf, hipStream_t stream) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(128) * (plan.n_docs + 1);
  const long grid = ((long)(T + 127) / 128 + plan.n_docs) * hkv;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  auto kern = qf == 1   ? attn_bwd_dkdv_mx_kernel<1>
              : qf == 2 ? attn_bwd_dkdv_mx_kernel<2>
              : qf == 3 ? attn_bwd_dkdv_mx_kernel<3>
                        : attn_bwd_dkdv_mx_kernel<0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, stream, m.qd, m.qd_sc, m.kd, m.kd_sc, m.dod, m.dod_sc,
                     m.vd, m.vd_sc, m.dot, m.dot_sc, (const __bf16*)q, (const __bf16*)dout, lse, delta,
                     (__bf16*)dk, (__bf16*)dv, plan, padoff, T, t_pad, hq, hkv, scale, causal);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_mx(const MxOperands& m, const void* k, const float* lse, const float* delta, void* dq,
                            const Plan& plan_any, const int* pref_base, int T, int hq, int hkv, float scale,
                            int causal, int qf, hipStream_t stream) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(128) * (plan.n_docs + 1);
  const long grid = ((long)(T + 127) / 128 + plan.n_docs) * hq;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  auto kern = qf == 1   ? attn_bwd_dq_mx_kernel<1>
              : qf == 2 ? attn_bwd_dq_mx_kernel<2>
              : qf == 3 ? attn_bwd_dq_mx_kernel<3>
                        : attn_bwd_dq_mx_kernel<0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, stream, m.qd, m.qd_sc, m.kd, m.kd_sc, m.dod, m.dod_sc,
                     m.vd, m.vd_sc, (const __bf16*)k, lse, delta, (__bf16*)dq, plan, T, hq, hkv, scale, causal);
  return hipGetLastError();
}

}  // namespace cfa

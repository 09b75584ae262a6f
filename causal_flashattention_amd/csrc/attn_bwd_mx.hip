// MXFP8 causal attention backward for gfx950 (d = 128), deterministic.
//
// Same derivative and work split as the bf16 backward (attn_bwd.hip); the operands follow the
// MXFP8 reading of the FLAMIA page ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri": token-block
// scaling reused across matrix orientations, causal-leakage safeguards, exact forward/backward
// consistency), each product blocked along its contraction axis:
//  * S = Q_d K_dᵀ from the forward's own Q_d/K_d bytes, so P = exp(S − LSE) reproduces the
//    forward's probabilities; dP = dO_d V_dᵀ. Both contract over d (scale per token).
//  * dV += Pᵀ dO, dK += dSᵀ Q, dQ += dS K contract over tokens. Off the diagonal 128×128 tile
//    they use the token-blocked copies dO_t, Q_t, K_t (one scale per channel and 32 doc-local
//    tokens). P (normalised, so ~1/L) is encoded E4M3 with an MX scale computed in registers
//    per 32 contraction elements; dS as two E4M3 terms (value and rounding residual, each with
//    its own MX scale), two MFMAs with the same A operand, since a single E4M3 rounding of dS
//    (relative error up to 2^-4) alone costs ~3% rel-L2 in dQ and dK when most pairs are off
//    the diagonal. On the diagonal tile everything token-contracted
//    stays bf16 (bf16 MFMA, transposing LDS reads), so no scale spans a query's future.
// Token-blocked tiles are staged with the 4-byte chunk order (0,2,4,6,1,3,5,7) per 32-token
// block so that the A operand read at offset 16h matches the lane's P / dS register order.
#include "cfa_device.h"
#include "cfa_kernels.h"

namespace cfa {

__device__ inline int mx_exp_of(float amax) {
  if (!(amax > 0.f)) return -127;
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  return min(max(ex - 1 - 8, -127), 127);
}

// Encode 2 × 16 values (two 32-element contraction blocks, 16 per lane each) as the B operand:
// bytes 0-15 block 0 with exponent e0, bytes 16-31 block 1 with exponent e1. The exponents come
// from fit_exp, so every scaled value lies within ±448 and needs no clamp.
__device__ inline i32x8 encode_b_fp8(const f32x16& x0, const f32x16& x1, int e0, int e1) {
  i32x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = pack_fp8x4(__builtin_amdgcn_ldexpf(x0[4 * e], -e0), __builtin_amdgcn_ldexpf(x0[4 * e + 1], -e0),
                      __builtin_amdgcn_ldexpf(x0[4 * e + 2], -e0), __builtin_amdgcn_ldexpf(x0[4 * e + 3], -e0));
    r[4 + e] = pack_fp8x4(__builtin_amdgcn_ldexpf(x1[4 * e], -e1), __builtin_amdgcn_ldexpf(x1[4 * e + 1], -e1),
                          __builtin_amdgcn_ldexpf(x1[4 * e + 2], -e1), __builtin_amdgcn_ldexpf(x1[4 * e + 3], -e1));
  }
  return r;
}

// Residual of a B-operand encoding: x - decode(codes)·2^e for both blocks (one fma each).
__device__ inline void residual_fp8(const f32x16& x0, const f32x16& x1, const i32x8& c, int e0, int e1, f32x16& r0,
                                    f32x16& r1) {
  const float p0 = __builtin_amdgcn_ldexpf(1.f, e0), p1 = __builtin_amdgcn_ldexpf(1.f, e1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 a01 = __builtin_amdgcn_cvt_pk_f32_fp8(c[e], false), a23 = __builtin_amdgcn_cvt_pk_f32_fp8(c[e], true);
    const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(c[4 + e], false);
    const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(c[4 + e], true);
    r0[4 * e + 0] = fmaf(-a01.x, p0, x0[4 * e + 0]);
    r0[4 * e + 1] = fmaf(-a01.y, p0, x0[4 * e + 1]);
    r0[4 * e + 2] = fmaf(-a23.x, p0, x0[4 * e + 2]);
    r0[4 * e + 3] = fmaf(-a23.y, p0, x0[4 * e + 3]);
    r1[4 * e + 0] = fmaf(-b01.x, p1, x1[4 * e + 0]);
    r1[4 * e + 1] = fmaf(-b01.y, p1, x1[4 * e + 1]);
    r1[4 * e + 2] = fmaf(-b23.x, p1, x1[4 * e + 2]);
    r1[4 * e + 3] = fmaf(-b23.y, p1, x1[4 * e + 3]);
  }
}

__device__ inline float amax16(const f32x16& x) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 2) m = fmaxf(m, fmaxf(fabsf(x[j]), fabsf(x[j + 1])));   // v_max3 with |.|
  return m;
}

// One 32-element contraction block, this lane's 16 values: encode with exponent e into the
// 4 words the lane contributes to a B operand (exponents from fit_exp: no clamp needed).
__device__ inline i32x4 encode16(const f32x16& x, int e) {
  i32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = pack_fp8x4(__builtin_amdgcn_ldexpf(x[4 * k], -e), __builtin_amdgcn_ldexpf(x[4 * k + 1], -e),
                      __builtin_amdgcn_ldexpf(x[4 * k + 2], -e), __builtin_amdgcn_ldexpf(x[4 * k + 3], -e));
  return r;
}

// x -= decode(c)·2^e in place (the rounding residual of encode16).
__device__ inline void residual16(f32x16& x, const i32x4& c, int e) {
  const float pe = __builtin_amdgcn_ldexpf(1.f, e);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 a01 = __builtin_amdgcn_cvt_pk_f32_fp8(c[k], false), a23 = __builtin_amdgcn_cvt_pk_f32_fp8(c[k], true);
    x[4 * k + 0] = fmaf(-a01.x, pe, x[4 * k + 0]);
    x[4 * k + 1] = fmaf(-a01.y, pe, x[4 * k + 1]);
    x[4 * k + 2] = fmaf(-a23.x, pe, x[4 * k + 2]);
    x[4 * k + 3] = fmaf(-a23.y, pe, x[4 * k + 3]);
  }
}

// Block exponent for values quantised inside the kernel (P, dS): the smallest power of two
// that maps amax to at most 448, so the largest element is never clipped (the operand rule
// of mx_quantize may clip it by up to 1/8, which the oracle models for Q/K/V/dO but not here).
__device__ inline int fit_exp(float amax) {
  int e = mx_exp_of(amax);
  if (amax > 0.f && __builtin_amdgcn_ldexpf(amax, -e) > 448.f) e += 1;
  return e;
}

// Exponents of the two 32-element contraction blocks held by a lane pair (l, l^32).
__device__ inline void block_exps(const f32x16& x0, const f32x16& x1, int& e0, int& e1) {
  float a0 = amax16(x0), a1 = amax16(x1);
  a0 = fmaxf(a0, __shfl_xor(a0, 32));
  a1 = fmaxf(a1, __shfl_xor(a1, 32));
  e0 = fit_exp(a0);
  e1 = fit_exp(a1);
}

// Two E4M3 terms for one B operand: x ≈ hi·2^e + lo·2^(e−4), e the block exponent from
// fit_exp. With every |x|·2^-e <= 448 the rounding residual of hi is at most 16·2^e (half the
// E4M3 spacing 32 of [256, 448]), so residual·2^(4−e) <= 256 fits E4M3 without a second block
// maximum. One E4M3 rounding has a relative error up to 2^-4; the residual term brings it to
// ~2^-8.
struct Fp8Pair {
  i32x8 hi, lo;
  int shi, slo;  // this lane's scale bytes (k-block = l/32)
};

__device__ inline Fp8Pair encode_two_term(const f32x16& x0, const f32x16& x1, int half) {
  Fp8Pair r;
  int e0, e1;
  block_exps(x0, x1, e0, e1);
  r.hi = encode_b_fp8(x0, x1, e0, e1);
  f32x16 r0, r1;
  residual_fp8(x0, x1, r.hi, e0, e1, r0, r1);
  const int f0 = max(e0 - 4, -127), f1 = max(e1 - 4, -127);
  r.lo = encode_b_fp8(r0, r1, f0, f1);
  r.shi = (half ? e1 : e0) + 127;
  r.slo = (half ? f1 : f0) + 127;
  return r;
}

// Block-wise form of encode_two_term for block b (0 or 1) of a B operand: consumes x (its
// storage becomes the residual), writes words 4b..4b+3 of hi and lo and, in the lane group
// that supplies block b's scale (half == b), the two scale bytes.
__device__ inline void encode_two_term_block(f32x16& x, int b, int half, Fp8Pair& r) {
  float a = amax16(x);
  a = fmaxf(a, __shfl_xor(a, 32));
  const int e = fit_exp(a);
  const i32x4 h4 = encode16(x, e);
  residual16(x, h4, e);
  const int f = max(e - 4, -127);
  const i32x4 l4 = encode16(x, f);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r.hi[4 * b + k] = h4[k];
    r.lo[4 * b + k] = l4[k];
  }
  if (half == b) {
    r.shi = e + 127;
    r.slo = f + 127;
  }
}

// Store a 16-byte chunk (16 consecutive tokens of one channel row) of a token-blocked tile into
// LDS with the per-32-block chunk order (0,2,4,6,1,3,5,7).
__device__ inline void store_tblocked(char* rowp, int kc, const i32x4& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q = 4 * kc + e;
    const int bb = q >> 3, qq = q & 7;
    const int pos = (qq & 1) ? 4 + (qq >> 1) : (qq >> 1);
    *(int*)(rowp + 32 * bb + 4 * pos) = v[e];
  }
}

__device__ inline i32x8 load_a_fp8(const char* row, int half) {
  const i32x4 lo = *(const i32x4*)(row + 16 * half);
  const i32x4 hi = *(const i32x4*)(row + 32 + 16 * half);
  return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

struct MxBwdTile {
  static constexpr int D = 128;
  static constexpr int BM = 64;                       // tokens per step / tile
  static constexpr int DSTR = 144;                    // d-blocked code row stride
  static constexpr int DCODES = BM * DSTR;            // 9216
  static constexpr int DSC = BM * 4;                  // 256
  static constexpr int TSTR = 80;                     // token-blocked row stride (64 tokens + 16)
  static constexpr int TCODES = D * TSTR;             // 10240
  static constexpr int TSC = D * 2;                   // 256
  static constexpr int BSTR = D * 2 + 16;             // bf16 row stride (272)
  static constexpr int BTILE = BM * BSTR;             // 17408
};

// ------------------------------------------------------------------ dK / dV
// LDS stage: [Qd codes][Qd sc][dOd codes][dOd sc][union: {Qt, Qt sc, dOt, dOt sc} | {Qb, dOb}][lse2][D]
template <int DUMMY>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_mx_kernel(
    const uint8_t* __restrict__ qd, const uint8_t* __restrict__ qd_sc, const uint8_t* __restrict__ kd,
    const uint8_t* __restrict__ kd_sc, const uint8_t* __restrict__ dod, const uint8_t* __restrict__ dod_sc,
    const uint8_t* __restrict__ vd, const uint8_t* __restrict__ vd_sc, const uint8_t* __restrict__ qt,
    const uint8_t* __restrict__ qt_sc, const uint8_t* __restrict__ dot, const uint8_t* __restrict__ dot_sc,
    const __bf16* __restrict__ q, const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, __bf16* __restrict__ dk, __bf16* __restrict__ dv, Plan plan,
    const int* __restrict__ padoff, int total_tokens, int t_pad, int hq, int hkv, float scale, int causal) {
  using C = MxBwdTile;
  constexpr int D = C::D, BM = C::BM;
  constexpr int O_QDSC = C::DCODES;
  constexpr int O_OD = O_QDSC + C::DSC;
  constexpr int O_ODSC = O_OD + C::DCODES;
  constexpr int O_U = O_ODSC + C::DSC;
  constexpr int O_QT = O_U, O_QTSC = O_QT + C::TCODES, O_OT = O_QTSC + C::TSC, O_OTSC = O_OT + C::TCODES;
  constexpr int O_QB = O_U, O_OB = O_U + C::BTILE;
  constexpr int U_BYTES = (2 * C::BTILE > 2 * (C::TCODES + C::TSC)) ? 2 * C::BTILE : 2 * (C::TCODES + C::TSC);
  constexpr int O_L = O_U + U_BYTES;
  constexpr int STAGE = O_L + 2 * BM * 4;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int p = blockIdx.x / hkv, g = blockIdx.x % hkv;
  int s0, L, t, doc;
  if (!decode_item(plan, p, 128, false, s0, L, t, &doc)) return;
  const int pcol = padoff[doc];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, half = lane >> 5;
  const int G = hq / hkv;
  const int kw0 = t * 128 + 32 * w;
  const int mykey = kw0 + (lane & 31);
  const float sl2 = scale * LOG2E;

  // K_d and V_d of this wave's keys as B operands
  i32x8 kb[2], vb[2];
  int ks[2], vs[2];
  {
    const bool ok = mykey < L;
    const size_t row = (size_t)(s0 + (ok ? mykey : 0)) * hkv + g;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      kb[s] = ok ? load_a_fp8((const char*)(kd + row * D + 64 * s), half) : i32x8{};
      vb[s] = ok ? load_a_fp8((const char*)(vd + row * D + 64 * s), half) : i32x8{};
      ks[s] = ok ? kd_sc[row * 4 + 2 * s + half] : 127;
      vs[s] = ok ? vd_sc[row * 4 + 2 * s + half] : 127;
    }
  }
  f32x16 dka[4], dva[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) { dka[b] = f32x16{}; dva[b] = f32x16{}; }

  const int q_begin = causal ? t * 128 : 0;
  const int n_qt = (L - q_begin + BM - 1) / BM;
  const int n_steps = n_qt * G;
  const int wave_first_q = causal ? kw0 : 0;
  auto step_is_diag = [&](int st) { return causal && ((q_begin + (st % n_qt) * BM) / 128 == t); };

  i32x4 r_qd[2], r_od[2], r_u[8];
  int r_qs = 0, r_os = 0, r_ts = 0;
  float r_l = 0.f, r_d = 0.f;
  auto load_step = [&](int st) {
    const int h = g * G + st / n_qt;
    const int q0 = q_begin + (st % n_qt) * BM;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = c & 7;
      const bool ok = q0 + row < L;
      const size_t off = ((size_t)(s0 + q0 + row) * hq + h) * D + col * 16;
      r_qd[i] = ok ? *(const i32x4*)(qd + off) : i32x4{0, 0, 0, 0};
      r_od[i] = ok ? *(const i32x4*)(dod + off) : i32x4{0, 0, 0, 0};
    }
    if (tid < 64) {
      const bool ok = q0 + tid < L;
      const size_t off = ((size_t)(s0 + q0 + tid) * hq + h) * 4;
      r_qs = ok ? *(const int*)(qd_sc + off) : 0x7f7f7f7f;
      r_os = ok ? *(const int*)(dod_sc + off) : 0x7f7f7f7f;
      r_l = ok ? lse[(size_t)h * total_tokens + s0 + q0 + tid] * LOG2E : INFINITY;
      r_d = ok ? delta[(size_t)h * total_tokens + s0 + q0 + tid] : 0.f;
    }
    if (step_is_diag(st)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, row = c >> 4, col = c & 15;
        const bool ok = q0 + row < L;
        const size_t off = ((size_t)(s0 + q0 + row) * hq + h) * D + col * 8;
        r_u[i] = ok ? *(const i32x4*)(q + off) : i32x4{0, 0, 0, 0};
        r_u[4 + i] = ok ? *(const i32x4*)(dout + off) : i32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, ch = c >> 2, kc = c & 3;
        const bool ok = q0 + 16 * kc < L;
        const size_t off = ((size_t)h * D + ch) * t_pad + pcol + q0 + 16 * kc;
        r_u[i] = ok ? *(const i32x4*)(qt + off) : i32x4{0, 0, 0, 0};
        r_u[2 + i] = ok ? *(const i32x4*)(dot + off) : i32x4{0, 0, 0, 0};
      }
      if (tid < D) {
        const size_t srow = ((size_t)h * D + tid) * (t_pad / 32) + (pcol + q0) / 32;
        const bool ok1 = q0 + 32 < L;
        r_ts = qt_sc[srow] | ((ok1 ? qt_sc[srow + 1] : 127) << 8) | (dot_sc[srow] << 16) |
               ((ok1 ? dot_sc[srow + 1] : 127) << 24);
      }
    }
  };
  auto store_step = [&](int buf, int st) {
    char* sb = smem + buf * STAGE;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = c & 7;
      *(i32x4*)(sb + row * C::DSTR + col * 16) = r_qd[i];
      *(i32x4*)(sb + O_OD + row * C::DSTR + col * 16) = r_od[i];
    }
    if (tid < 64) {
      *(int*)(sb + O_QDSC + tid * 4) = r_qs;
      *(int*)(sb + O_ODSC + tid * 4) = r_os;
      ((float*)(sb + O_L))[tid] = r_l;
      ((float*)(sb + O_L))[BM + tid] = r_d;
    }
    if (step_is_diag(st)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, row = c >> 4, col = c & 15;
        *(i32x4*)(sb + O_QB + row * C::BSTR + col * 16) = r_u[i];
        *(i32x4*)(sb + O_OB + row * C::BSTR + col * 16) = r_u[4 + i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, ch = c >> 2, kc = c & 3;
        store_tblocked(sb + O_QT + ch * C::TSTR, kc, r_u[i]);
        store_tblocked(sb + O_OT + ch * C::TSTR, kc, r_u[2 + i]);
      }
      if (tid < D) {
        *(uint16_t*)(sb + O_QTSC + tid * 2) = (uint16_t)(r_ts & 0xFFFF);
        *(uint16_t*)(sb + O_OTSC + tid * 2) = (uint16_t)(r_ts >> 16);
      }
    }
  };

  if (n_steps > 0) {
    load_step(0);
    store_step(0, 0);
  }
  __syncthreads();
  for (int st = 0; st < n_steps; ++st) {
    if (st + 1 < n_steps) load_step(st + 1);
    const int q0 = q_begin + (st % n_qt) * BM;
    if (q0 + BM - 1 >= wave_first_q && kw0 < L) {
      const char* sb = smem + (st & 1) * STAGE;
      const float* lb = (const float*)(sb + O_L);
      const float* db = lb + BM;
      const bool need_mask = causal && (q0 < kw0 + 31);
      f32x16 pv[2], dsv[2];
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        const int qr = 32 * qb2 + (lane & 31);
        const int qsc = *(const int*)(sb + O_QDSC + qr * 4);
        const int osc = *(const int*)(sb + O_ODSC + qr * 4);
        f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          sacc = mfma32_mx(load_a_fp8(sb + qr * C::DSTR + 64 * s, half), (qsc >> (8 * (2 * s + half))) & 0xFF, kb[s],
                           ks[s], sacc);
          pacc = mfma32_mx(load_a_fp8(sb + O_OD + qr * C::DSTR + 64 * s, half), (osc >> (8 * (2 * s + half))) & 0xFF,
                           vb[s], vs[s], pacc);
        }
        if (need_mask) {                 // wave-uniform: steps that cross the diagonal
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (mykey > q0 + 32 * qb2 + 8 * (j >> 2) + 4 * half + (j & 3)) sacc[j] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int qi_t = 32 * qb2 + 8 * (j >> 2) + 4 * half + (j & 3);
          const float x = exp2_fast(fmaf(sacc[j], sl2, -lb[qi_t]));
          pv[qb2][j] = x;
          dsv[qb2][j] = x * (pacc[j] - db[qi_t]);
        }
      }
      if (step_is_diag(st)) {
        bf16x8 pf[4], sf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          i32x4 up, us;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            up[e] = (int)pack_bf16x2(pv[kk >> 1][8 * (kk & 1) + 2 * e], pv[kk >> 1][8 * (kk & 1) + 2 * e + 1]);
            us[e] = (int)pack_bf16x2(dsv[kk >> 1][8 * (kk & 1) + 2 * e], dsv[kk >> 1][8 * (kk & 1) + 2 * e + 1]);
          }
          pf[kk] = __builtin_bit_cast(bf16x8, up);
          sf[kk] = __builtin_bit_cast(bf16x8, us);
        }
        const char* qbt = sb + O_QB;
        const char* obt = sb + O_OB;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int rbase = 32 * (kk >> 1) + 16 * (kk & 1);
          const int row = rbase + 4 * half + ((lane & 15) >> 2);
          const int dsub = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
          for (int dbk = 0; dbk < 4; ++dbk) {
            const int boff = row * C::BSTR + (32 * dbk + dsub) * 2;
            dva[dbk] = mfma32(concat_tr(lds_read_tr16(obt + boff), lds_read_tr16(obt + boff + 8 * C::BSTR)), pf[kk],
                              dva[dbk]);
            dka[dbk] = mfma32(concat_tr(lds_read_tr16(qbt + boff), lds_read_tr16(qbt + boff + 8 * C::BSTR)), sf[kk],
                              dka[dbk]);
          }
        }
      } else {
        // P (normalised, ~1/L: needs its own block scale) with an MX exponent per (key,
        // 32-query block); dS as two E4M3 terms with MX exponents
        int pe0, pe1;
        block_exps(pv[0], pv[1], pe0, pe1);
        const i32x8 pb = encode_b_fp8(pv[0], pv[1], pe0, pe1);
        const int psc = (half ? pe1 : pe0) + 127;
        const Fp8Pair ds2 = encode_two_term(dsv[0], dsv[1], half);
#pragma unroll
        for (int dbk = 0; dbk < 4; ++dbk) {
          const int ch = 32 * dbk + (lane & 31);
          const int osa = (*(const uint16_t*)(sb + O_OTSC + ch * 2) >> (8 * half)) & 0xFF;
          const int qsa = (*(const uint16_t*)(sb + O_QTSC + ch * 2) >> (8 * half)) & 0xFF;
          dva[dbk] = mfma32_mx(load_a_fp8(sb + O_OT + ch * C::TSTR, half), osa, pb, psc, dva[dbk]);
          const i32x8 aq = load_a_fp8(sb + O_QT + ch * C::TSTR, half);
          dka[dbk] = mfma32_mx(aq, qsa, ds2.hi, ds2.shi, dka[dbk]);
          dka[dbk] = mfma32_mx(aq, qsa, ds2.lo, ds2.slo, dka[dbk]);
        }
      }
    }
    if (st + 1 < n_steps) store_step((st + 1) & 1, st + 1);
    __syncthreads();
  }

  if (mykey < L) {
    const size_t base = ((size_t)(s0 + mykey) * hkv + g) * D + 4 * half;
#pragma unroll
    for (int dbk = 0; dbk < 4; ++dbk)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        i32x2 uk, uv;
        uk.x = (int)pack_bf16x2(dka[dbk][4 * jg] * scale, dka[dbk][4 * jg + 1] * scale);
        uk.y = (int)pack_bf16x2(dka[dbk][4 * jg + 2] * scale, dka[dbk][4 * jg + 3] * scale);
        uv.x = (int)pack_bf16x2(dva[dbk][4 * jg], dva[dbk][4 * jg + 1]);
        uv.y = (int)pack_bf16x2(dva[dbk][4 * jg + 2], dva[dbk][4 * jg + 3]);
        *(i32x2*)(dk + base + 32 * dbk + 8 * jg) = uk;
        *(i32x2*)(dv + base + 32 * dbk + 8 * jg) = uv;
      }
  }
}

// ------------------------------------------------------------------ dQ
// A wave owns 32 queries of one head (Q_d, dO_d in registers as B operands); the workgroup
// walks key tiles of 64, staged by direct global -> LDS copies into two static buffers:
//   [K_d codes 64 × 128 B][K_d scales 64 × 4][V_d codes][V_d scales]
//   [diagonal: K bf16 rows (SwzTile<128>) | otherwise: K_t codes 128 channel rows × 64 B, scales 2 × 128]
// (code rows XOR-swizzled as in the MX forward kernel).
struct MxDqTile {
  static constexpr int BN = 64;
  static constexpr int OFF_KDSC = BN * 128;
  static constexpr int OFF_VD = OFF_KDSC + BN * 4;
  static constexpr int OFF_VDSC = OFF_VD + BN * 128;
  static constexpr int OFF_U = OFF_VDSC + BN * 4;
  static constexpr int OFF_KTSC = OFF_U + 128 * 64;
  static constexpr int STAGE = OFF_U + BN * 256;
};

__global__ __launch_bounds__(256, 2) void attn_bwd_dq_mx_kernel(
    const uint8_t* __restrict__ qd, const uint8_t* __restrict__ qd_sc, const uint8_t* __restrict__ kd,
    const uint8_t* __restrict__ kd_sc, const uint8_t* __restrict__ dod, const uint8_t* __restrict__ dod_sc,
    const uint8_t* __restrict__ vd, const uint8_t* __restrict__ vd_sc, const uint8_t* __restrict__ kt,
    const uint8_t* __restrict__ kt_sc, const __bf16* __restrict__ k, const float* __restrict__ lse,
    const float* __restrict__ delta, __bf16* __restrict__ dq, Plan plan, const int* __restrict__ padoff,
    int total_tokens, int t_pad, int hq, int hkv, float scale, int causal) {
  using C = MxDqTile;
  constexpr int D = 128, BN = C::BN;
  __shared__ __attribute__((aligned(16))) char lds_a[C::STAGE];
  __shared__ __attribute__((aligned(16))) char lds_b[C::STAGE];

  const int p = blockIdx.x / hq, h = blockIdx.x % hq;
  int s0, L, t, doc;
  if (!decode_item(plan, p, 128, true, s0, L, t, &doc)) return;
  const int pcol = padoff[doc];
  const int lp = 32 * ((L + 31) / 32);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, half = lane >> 5, r32 = lane & 31;
  const int g = h / (hq / hkv);
  const int wr0 = t * 128 + 32 * w;
  const int qrow = wr0 + r32;
  const int kv_end = causal ? min(L, (t + 1) * 128) : L;
  const int n_kt = (kv_end + BN - 1) / BN;
  const int wave_last_key = causal ? min(L, wr0 + 32) - 1 : L - 1;
  const float sl2 = scale * LOG2E;
  auto tile_is_diag = [&](int ktile) { return causal && ((ktile * BN) / 128 == t); };
  int ko[2][2], to[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int u = 0; u < 2; ++u) ko[s][u] = 16 * ((4 * s + 2 * u + half) ^ kd_swz(r32));
#pragma unroll
  for (int u = 0; u < 2; ++u) to[u] = 16 * ((2 * u + half) ^ vt_swz(r32));

  i32x8 qa[2], oa[2];
  int qs[2], os[2];
  float lse2 = INFINITY, dl = 0.f;
  {
    const bool ok = qrow < L;
    const size_t row = (size_t)(s0 + (ok ? qrow : 0)) * hq + h;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
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

  // key tile -> LDS; keys past kv_end are clamped into the document (K_d, V_d, bf16 K) or its
  // last token block (K_t); they are masked (P = 0)
  // Addresses: a wave-uniform 64-bit tile base plus a 32-bit lane offset within the tile.
  const uint32_t krow_b = (uint32_t)hkv * D;      // bytes between consecutive tokens (codes, bf16/2)
  auto stage = [&](int ktile, char* tb) {
    const int k0 = ktile * BN;
    const int rmax = kv_end - 1 - k0;             // last row inside the document
    const size_t tok0 = (size_t)(s0 + k0) * hkv + g;
    const uint8_t* kdb = kd + tok0 * D;
    const uint8_t* vdb = vd + tok0 * D;
#pragma unroll
    for (int j = 0; j < 2; ++j) {               // K_d and V_d codes: 8 blocks of 8 rows each
      const int I = 2 * w + j, r = 8 * I + (lane >> 3);
      const uint32_t off = (uint32_t)min(r, rmax) * krow_b + 16 * ((lane & 7) ^ kd_swz(r));
      g2lds16(kdb + off, tb + I * 1024);
      g2lds16(vdb + off, tb + C::OFF_VD + I * 1024);
    }
    const uint32_t soff = (uint32_t)min(lane, rmax) * (uint32_t)hkv * 4;
    if (w == 0) g2lds4(kd_sc + tok0 * 4 + soff, tb + C::OFF_KDSC);
    if (w == 1) g2lds4(vd_sc + tok0 * 4 + soff, tb + C::OFF_VDSC);
    if (tile_is_diag(ktile)) {
      stage_rows_lds<BN>(tb + C::OFF_U, (const char*)(k + tok0 * D), krow_b * 2, rmax, w, lane);
    } else {
      const uint8_t* ktb = kt + (size_t)g * D * t_pad + pcol + k0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {             // K_t codes: 8 blocks of 16 channel rows
        const int I = 2 * w + j, r = 16 * I + (lane >> 2);
        const int col = min(16 * ((lane & 3) ^ vt_swz(r)), lp - 16 - k0);
        g2lds16(ktb + (uint32_t)(r * t_pad + col), tb + C::OFF_U + I * 1024);
      }
      if (w == 2 && lane < 16) {
        const int blk = min((k0 >> 5) + (lane >> 3), lp / 32 - 1);
        g2lds16(kt_sc + ((size_t)g * (t_pad / 32) + (pcol >> 5) + blk) * D + 16 * (lane & 7), tb + C::OFF_KTSC);
      }
    }
  };

  // dS of one 32-key block b of the tile (this lane: query qrow, keys k0 + 32b + 8(j/4) + 4·half + j%4)
  auto ds_block = [&](const char* tb, int k0, int b, bool need_mask) __attribute__((always_inline)) {
    const int kr = 32 * b + r32;
    const int ksc = *(const int*)(tb + C::OFF_KDSC + kr * 4);
    const int vsc = *(const int*)(tb + C::OFF_VDSC + kr * 4);
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const char* kp = tb + kr * 128;
      const char* vp = tb + C::OFF_VD + kr * 128;
      const i32x4 klo = *(const i32x4*)(kp + ko[s][0]), khi = *(const i32x4*)(kp + ko[s][1]);
      const i32x4 vlo = *(const i32x4*)(vp + ko[s][0]), vhi = *(const i32x4*)(vp + ko[s][1]);
      sacc = mfma32_mx(i32x8{klo.x, klo.y, klo.z, klo.w, khi.x, khi.y, khi.z, khi.w},
                       (ksc >> (8 * (2 * s + half))) & 0xFF, qa[s], qs[s], sacc);
      pacc = mfma32_mx(i32x8{vlo.x, vlo.y, vlo.z, vlo.w, vhi.x, vhi.y, vhi.z, vhi.w},
                       (vsc >> (8 * (2 * s + half))) & 0xFF, oa[s], os[s], pacc);
    }
    if (need_mask) {                     // wave-uniform: diagonal or document-end tiles
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + 32 * b + 8 * (j >> 2) + 4 * half + (j & 3);
        if (causal ? (key > qrow) : (key >= L)) sacc[j] = -INFINITY;
      }
    }
    f32x16 x;
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = exp2_fast(fmaf(sacc[j], sl2, -lse2)) * (pacc[j] - dl);
    return x;
  };

  // diagonal tile: bf16 dS and bf16 K (transposing reads)
  auto tile_diag = [&](const char* tb, int k0, bool need_mask) __attribute__((always_inline)) {
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

  // other tiles: two-term E4M3 dS and token-blocked K_t
  auto tile_off = [&](const char* tb, int k0, bool need_mask) __attribute__((always_inline)) {
    Fp8Pair ds2;
    ds2.shi = ds2.slo = 127;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 x = ds_block(tb, k0, b, need_mask);
      encode_two_term_block(x, b, half, ds2);
    }
#pragma unroll
    for (int dbk = 0; dbk < 4; ++dbk) {
      const int ch = 32 * dbk + r32;
      const char* kr = tb + C::OFF_U + ch * 64;
      const i32x4 lo = *(const i32x4*)(kr + to[0]), hi = *(const i32x4*)(kr + to[1]);
      const i32x8 ak = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int ksa = *(const uint8_t*)(tb + C::OFF_KTSC + half * 128 + ch);
      dqa[dbk] = mfma32_mx(ak, ksa, ds2.hi, ds2.shi, dqa[dbk]);
      dqa[dbk] = mfma32_mx(ak, ksa, ds2.lo, ds2.slo, dqa[dbk]);
    }
  };

  auto iter = [&](int ktile, const char* tb, char* nxt) __attribute__((always_inline)) {
    const int k0 = ktile * BN;
    if (ktile + 1 < n_kt) stage(ktile + 1, nxt);
    if (k0 <= wave_last_key) {
      const bool need_mask = causal ? (k0 + BN - 1 > wr0) : (k0 + BN > L);
      if (tile_is_diag(ktile)) tile_diag(tb, k0, need_mask);
      else tile_off(tb, k0, need_mask);
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
static int dkdv_mx_stage() {
  using C = MxBwdTile;
  constexpr int U = (2 * C::BTILE > 2 * (C::TCODES + C::TSC)) ? 2 * C::BTILE : 2 * (C::TCODES + C::TSC);
  return 2 * (C::DCODES + C::DSC) + U + 2 * C::BM * 4;
}

hipError_t launch_bwd_dkdv_mx(const MxOperands& m, const void* q, const void* dout, const float* lse,
                              const float* delta, void* dk, void* dv, const Plan& plan_any, const int* pref_base,
                              const int* padoff, int T, int t_pad, int hq, int hkv, float scale, int causal,
                              hipStream_t stream) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(128) * (plan.n_docs + 1);
  const long grid = ((long)(T + 127) / 128 + plan.n_docs) * hkv;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int lds = 2 * dkdv_mx_stage();
  auto kern = attn_bwd_dkdv_mx_kernel<0>;
  if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds))
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, stream, m.qd, m.qd_sc, m.kd, m.kd_sc, m.dod, m.dod_sc,
                     m.vd, m.vd_sc, m.qt, m.qt_sc, m.dot, m.dot_sc, (const __bf16*)q, (const __bf16*)dout, lse, delta,
                     (__bf16*)dk, (__bf16*)dv, plan, padoff, T, t_pad, hq, hkv, scale, causal);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_mx(const MxOperands& m, const void* k, const float* lse, const float* delta, void* dq,
                            const Plan& plan_any, const int* pref_base, const int* padoff, int T, int t_pad, int hq,
                            int hkv, float scale, int causal, hipStream_t stream) {
  Plan plan = plan_any;
  plan.pref = pref_base + pref_slot(128) * (plan.n_docs + 1);
  const long grid = ((long)(T + 127) / 128 + plan.n_docs) * hq;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(attn_bwd_dq_mx_kernel, dim3((unsigned)grid), dim3(256), 0, stream, m.qd, m.qd_sc, m.kd, m.kd_sc,
                     m.dod, m.dod_sc, m.vd, m.vd_sc, m.kt, m.kt_sc, (const __bf16*)k, lse, delta, (__bf16*)dq, plan,
                     padoff, T, t_pad, hq, hkv, scale, causal);
  return hipGetLastError();
}

}  // namespace cfa

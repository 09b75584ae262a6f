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
//    32 doc-local keys, and P (in [0, 1] after the running-max shift) is encoded E4M3 with the
//    fixed scale 2^-8 (P·256 <= 256 < 448). On the diagonal 128×128 tile of each document the
//    token blocks would share a scale between a query and keys after it, so there P and V stay
//    bf16 and use v_mfma_f32_32x32x16_bf16.
// Everything else (work list, online softmax, double-buffered LDS staging, Sᵀ orientation)
// follows the bf16 kernel in attn_fwd.hip.
//
// Operand staging. K_d rows go to LDS as 128 code bytes (+16 pad) plus 4 scale bytes per key.
// The scaled MFMA takes, per lane, 16 consecutive k bytes twice; the probabilities of lane
// group h hold keys {8·(j/4) + 4h + j%4} of each 32-key block, so the V_t tile is written to
// LDS with its 4-byte chunks of each 32-key block reordered to (0,2,4,6,1,3,5,7): the A read
// at offset 16h then yields exactly the keys whose probabilities the lane holds.
#include "cfa_device.h"

namespace cfa {

// The running maximum moves as soon as a tile's maximum exceeds it (threshold 0, log2 units),
// so P̃ <= 1 and P̃·2^8 fits E4M3 with 2^-8 as its fixed scale; a larger threshold would push
// typical probabilities into E4M3's subnormal range. Only the rescaling of O is skipped when
// no lane's maximum grew.
constexpr float RESCALE_LOG2_MX = 0.f;

struct MxFwdTile {
  static constexpr int BN = 64;
  static constexpr int D = 128;
  static constexpr int KSTR = 144;                 // K_d code row stride (bytes)
  static constexpr int K_CODES = BN * KSTR;        // 9216
  static constexpr int K_SC = BN * 4;              // 256
  static constexpr int VT_STR = 80;                // V_t code row stride: 64 keys + 16 pad
  static constexpr int VT_CODES = D * VT_STR;      // 10240
  static constexpr int VT_SC = D * 2;              // 256 (2 key blocks per channel)
  static constexpr int VB_STR = D * 2 + 32;        // bf16 V row stride (transposed reads)
  static constexpr int VB = BN * VB_STR;           // 18432
  static constexpr int OFF_KSC = K_CODES;
  static constexpr int OFF_VT = OFF_KSC + K_SC;
  static constexpr int OFF_VTSC = OFF_VT + VT_CODES;
  static constexpr int OFF_VB = OFF_VTSC + VT_SC;
  static constexpr int STAGE = OFF_VB + VB;        // 38400
};

template <int HPW>
__global__ __launch_bounds__(256, 2) void attn_fwd_mx_kernel(
    const uint8_t* __restrict__ qd, const uint8_t* __restrict__ qd_sc, const uint8_t* __restrict__ kd,
    const uint8_t* __restrict__ kd_sc, const uint8_t* __restrict__ vt, const uint8_t* __restrict__ vt_sc,
    const __bf16* __restrict__ v, __bf16* __restrict__ o, float* __restrict__ lse, Plan plan,
    const int* __restrict__ padoff, int total_tokens, int t_pad, int hq, int hkv, int n_hb, float scale_log2,
    int causal) {
  using C = MxFwdTile;
  constexpr int D = C::D;
  constexpr int BMW = 128 / HPW;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int wid = blockIdx.x;
  const int p = wid / n_hb, hb = wid % n_hb;
  int s0, L, t, doc;
  if (!decode_item(plan, p, BMW, true, s0, L, t, &doc)) return;
  const int pcol = padoff[doc];                 // first token-blocked column of the document
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, half = lane >> 5;
  const int G = hq / hkv;
  const int h = hb * HPW + (w % HPW);
  const int g = h / G;
  const int wr0 = t * BMW + 32 * (w / HPW);
  const int wg_rows_end = min(L, (t + 1) * BMW);
  const int kv_end = causal ? wg_rows_end : L;
  const int n_kt = (kv_end + C::BN - 1) / C::BN;
  const int wave_last_key = causal ? min(L, wr0 + 32) - 1 : L - 1;
  const int qrow = wr0 + (lane & 31);
  const int diag_blk = causal ? (t * BMW) / 128 : -1;   // the wg's 128-row block

  // ---- Q_d fragments (B operand of Sᵀ = K Qᵀ): two 64-channel halves
  i32x8 qa[2];
  int qs[2];
  {
    const bool ok = qrow < L;
    const size_t row = (size_t)(s0 + (ok ? qrow : 0)) * hq + h;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const i32x4 lo = ok ? *(const i32x4*)(qd + row * D + 64 * s + 16 * half) : i32x4{0, 0, 0, 0};
      const i32x4 hi = ok ? *(const i32x4*)(qd + row * D + 64 * s + 32 + 16 * half) : i32x4{0, 0, 0, 0};
      qa[s] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      qs[s] = ok ? qd_sc[row * 4 + 2 * s + half] : 127;
    }
  }
  f32x16 oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // ---- staging registers
  i32x4 kreg[2], vreg[4];
  int ksreg = 0, vsreg = 0;
  auto tile_is_diag = [&](int kt) { return (kt * C::BN) / 128 == diag_blk; };
  auto load_tile = [&](int kt) {
    const int k0 = kt * C::BN;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // K_d codes: 64 rows × 8 chunks
      const int c = tid + 256 * i, key = c >> 3, col = c & 7;
      const bool ok = k0 + key < kv_end;
      kreg[i] = ok ? *(const i32x4*)(kd + ((size_t)(s0 + k0 + key) * hkv + g) * D + col * 16) : i32x4{0, 0, 0, 0};
    }
    if (tid < 64) {  // K_d scales: one int (4 bytes) per key
      const bool ok = k0 + tid < kv_end;
      ksreg = ok ? *(const int*)(kd_sc + ((size_t)(s0 + k0 + tid) * hkv + g) * 4) : 0x7f7f7f7f;
    }
    if (tile_is_diag(kt)) {  // bf16 V rows: 64 × 16 chunks
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, key = c >> 4, col = c & 15;
        const bool ok = k0 + key < kv_end;
        vreg[i] = ok ? *(const i32x4*)(v + ((size_t)(s0 + k0 + key) * hkv + g) * D + col * 8) : i32x4{0, 0, 0, 0};
      }
    } else {  // V_t codes: 128 channel rows × 4 chunks of 16 keys, and 2 scale bytes per row
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, ch = c >> 2, kc = c & 3;
        const bool ok = k0 + 16 * kc < kv_end;
        vreg[i] = ok ? *(const i32x4*)(vt + ((size_t)g * D + ch) * t_pad + pcol + k0 + 16 * kc) : i32x4{0, 0, 0, 0};
      }
      if (tid < D) {
        const size_t srow = ((size_t)g * D + tid) * (t_pad / 32) + (pcol + k0) / 32;
        const int b0 = vt_sc[srow];
        const int b1 = (k0 + 32 < kv_end) ? vt_sc[srow + 1] : 127;
        vsreg = b0 | (b1 << 8);
      }
    }
  };
  auto store_tile = [&](int buf, int kt) {
    char* st = smem + buf * C::STAGE;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, key = c >> 3, col = c & 7;
      *(i32x4*)(st + key * C::KSTR + col * 16) = kreg[i];
    }
    if (tid < 64) *(int*)(st + C::OFF_KSC + tid * 4) = ksreg;
    if (tile_is_diag(kt)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, key = c >> 4, col = c & 15;
        *(i32x4*)(st + C::OFF_VB + key * C::VB_STR + col * 16) = vreg[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, ch = c >> 2, kc = c & 3;
        // chunk of 16 keys = 4-byte pieces q = 4kc..4kc+3 of the row; piece q (keys 4q..4q+3)
        // of 32-key block bb = q/8 goes to position (q%8 even ? (q%8)/2 : 4 + (q%8)/2)
        char* rowp = st + C::OFF_VT + ch * C::VT_STR;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = 4 * kc + e;
          const int bb = q >> 3, qq = q & 7;
          const int pos = (qq & 1) ? 4 + (qq >> 1) : (qq >> 1);
          *(int*)(rowp + 32 * bb + 4 * pos) = vreg[i][e];
        }
      }
      if (tid < D) *(uint16_t*)(st + C::OFF_VTSC + tid * 2) = (uint16_t)vsreg;
    }
  };

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * C::BN;
    if (kt + 1 < n_kt) load_tile(kt + 1);
    if (k0 <= wave_last_key) {
      const char* st = smem + (kt & 1) * C::STAGE;
      // ---- Sᵀ = K_d Q_dᵀ (scaled fp8)
      f32x16 sacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sacc[b] = f32x16{};
        const int krow = 32 * b + (lane & 31);
        const char* kr = st + krow * C::KSTR;
        const int ksc = *(const int*)(st + C::OFF_KSC + krow * 4);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x4 lo = *(const i32x4*)(kr + 64 * s + 16 * half);
          const i32x4 hi = *(const i32x4*)(kr + 64 * s + 32 + 16 * half);
          const i32x8 a = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const int sa = (ksc >> (8 * (2 * s + half))) & 0xFF;
          sacc[b] = mfma32_mx(a, sa, qa[s], qs[s], sacc[b]);
        }
      }
      // ---- online softmax: maximum on the raw scores (scale_log2 > 0), scale folded into the
      // exponent, masks only on tiles crossing the diagonal or the document end (wave-uniform)
      const bool need_mask = causal ? (k0 + C::BN - 1 > wr0) : (k0 + C::BN > L);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + 32 * b + 8 * (j >> 2) + 4 * half + (j & 3);
            if (causal ? (key > qrow) : (key >= L)) sacc[b][j] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; j += 2) mt = fmaxf(mt, fmaxf(sacc[b][j], sacc[b][j + 1]));
      mt = wave_max_xor32(mt) * scale_log2;
      const bool upd = mt > m_run + RESCALE_LOG2_MX;
      if (__any(upd)) {
        const float m_new = upd ? mt : m_run;
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      }
      float ls = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pj = exp2_fast(fmaf(sacc[b][j], scale_log2, -m_run));
          sacc[b][j] = pj;
          ls += pj;
        }
      l_run += ls;
      if (tile_is_diag(kt)) {
        // ---- diagonal tile: bf16 P and V
        bf16x8 pf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          i32x4 u;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            u[e] = (int)pack_bf16x2(sacc[kk >> 1][8 * (kk & 1) + 2 * e], sacc[kk >> 1][8 * (kk & 1) + 2 * e + 1]);
          pf[kk] = __builtin_bit_cast(bf16x8, u);
        }
        const char* vb = st + C::OFF_VB;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int kbase = 32 * (kk >> 1) + 16 * (kk & 1);
          const int key = kbase + 4 * half + ((lane & 15) >> 2);
          const int dsub = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const char* p0 = vb + key * C::VB_STR + (32 * db + dsub) * 2;
            oacc[db] = mfma32(concat_tr(lds_read_tr16(p0), lds_read_tr16(p0 + 8 * C::VB_STR)), pf[kk], oacc[db]);
          }
        }
      } else {
        // ---- off-diagonal tile: P·2^8 as E4M3 (scale byte 127-8), V_t token-blocked
        i32x8 pb;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[4 * b + e] = pack_fp8x4(sacc[b][4 * e] * 256.f, sacc[b][4 * e + 1] * 256.f,
                                       sacc[b][4 * e + 2] * 256.f, sacc[b][4 * e + 3] * 256.f);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ch = 32 * db + (lane & 31);
          const char* vr = st + C::OFF_VT + ch * C::VT_STR;
          const i32x4 lo = *(const i32x4*)(vr + 16 * half);
          const i32x4 hi = *(const i32x4*)(vr + 32 + 16 * half);
          const i32x8 a = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const int sa = (*(const uint16_t*)(st + C::OFF_VTSC + ch * 2) >> (8 * half)) & 0xFF;
          oacc[db] = mfma32_mx(a, sa, pb, 127 - 8, oacc[db]);
        }
      }
    }
    if (kt + 1 < n_kt) store_tile((kt + 1) & 1, kt + 1);
    __syncthreads();
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

hipError_t launch_fwd_mx(const uint8_t* qd, const uint8_t* qd_sc, const uint8_t* kd, const uint8_t* kd_sc,
                         const uint8_t* vt, const uint8_t* vt_sc, const void* v, void* o, float* lse,
                         const Plan& plan_any, const int* pref_base, const int* padoff, int total_tokens, int t_pad,
                         int hq, int hkv, float scale, int causal, hipStream_t stream) {
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
  const int lds = 2 * MxFwdTile::STAGE;
#define CFA_MXF_LAUNCH(HH)                                                                                    \
  do {                                                                                                        \
    auto kern = attn_fwd_mx_kernel<HH>;                                                                       \
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds))              \
      return hipErrorInvalidConfiguration;                                                                    \
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, stream, qd, qd_sc, kd, kd_sc, vt, vt_sc,   \
                       (const __bf16*)v, (__bf16*)o, lse, plan, padoff, total_tokens, t_pad, hq, hkv, n_hb, sl2, \
                       causal);                                                                               \
  } while (0)
  if (hpw == 4) CFA_MXF_LAUNCH(4);
  else if (hpw == 2) CFA_MXF_LAUNCH(2);
  else CFA_MXF_LAUNCH(1);
#undef CFA_MXF_LAUNCH
  return hipGetLastError();
}

}  // namespace cfa

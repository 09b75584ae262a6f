// MX quantiser for gfx950: bf16 -> FP8 E4M3 (or FP4 E2M1, FP6 E2M3 / E3M2) codes + E8M0 scales,
// one scale per 32.
//
// The MXFP8 attention path and its document-local token-block scaling are named on the FLAMIA
// page ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri"); the bit-level rule is the public MX one:
// per block, amax = max|x|, e = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for a zero
// block), scale byte e + 127; elements x·2^-e saturated to ±448 and rounded to nearest E4M3
// (ties to even, sign of zero kept); a block holding NaN/Inf gets scale 0xFF and codes 0x7F.
//
// The E4M3 and E2M1 encoders work on the bf16 bit patterns, two elements per 32-bit word:
//  * amax: the magnitude bits (x & 0x7FFF) order finite values, Inf (0x7F80) and NaN (above)
//    like their magnitudes, so a packed 16-bit maximum gives the block's largest magnitude and
//    its non-finite test (>= 0x7F80) at once, and e = max(E - 135, -127) from its exponent
//    field E (E4M3; E - 129 for E2M1, whose top exponent is 2);
//  * elements: v_cvt_scalef32_pk_{fp8,fp4}_bf16 divides two bf16 values by the f32 scale 2^e and
//    rounds to nearest even. An in-bounds probe over every bf16 pattern and exponents -127..127
//    matched the f32 path (ldexp, clamp, v_cvt_pk_fp8_f32 / the E2M1 grid) bit for bit, except
//    that the FP8 form does not saturate: scaled magnitudes from 464 up become NaN. The E4M3 path
//    therefore clamps magnitudes to 448·2^e first, in the bf16 domain (a packed 16-bit minimum
//    against the bit pattern ((e + 135) << 7) | 0x60 of 448·2^e; power-of-two scaling makes the
//    two clamps the same). E2M1 saturates at ±6 in the instruction itself.
//
// The kernels are HBM-bound streaming passes (2 bytes read, 1 + 1/32 bytes written per element
// for E4M3):
//  * along d: 4 lanes per 32-channel block, 16 bytes per lane, amax by two lane swaps;
//  * along doc-local tokens: a workgroup per (128 padded columns, head) stages the 128 × d tile
//    in LDS and each lane encodes whole 32-token blocks of one channel (details at
//    encode_t_group);
//  * fused: one pass per direction writes the copies the attention kernels need but do not make
//    themselves (details at mx_prep_fwd_kernel and mx_prep_bwd_kernel; the MX forward kernel
//    quantises Q from the rows it reads).
#include "cfa_device.h"
#include "cfa_mx.h"

namespace cfa {

__global__ __launch_bounds__(256) void mx_quantize_d_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, long n_blocks) {
  const long blk = (long)blockIdx.x * 64 + threadIdx.x / 4;
  const int sub = threadIdx.x & 3;
  i32x4 u = i32x4{0, 0, 0, 0};
  if (blk < n_blocks) u = *(const i32x4*)(x + blk * 32 + sub * 8);
  const uint32_t w[4] = {(uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w};
  const uint32_t ab = quad_max(amax_bits<4>(w));
  if (blk >= n_blocks) return;
  const bool bad = ab >= 0x7F80u;
  const int e = e4m3_block_exp(ab);
  const i32x2 c = {bad_or(bad, 0x7F7F7F7F, e4m3_encode4(w[0], w[1], e)), bad_or(bad, 0x7F7F7F7F, e4m3_encode4(w[2], w[3], e))};
  *(i32x2*)(codes + blk * 32 + sub * 8) = c;
  if (sub == 0) scales[blk] = bad ? 0xFF : (uint8_t)(e + 127);
}

// E2M1 (MXFP4) along d: the same block rule with the E2M1 top exponent 2, e = floor(log2 amax) - 2;
// elements x·2^-e clamped to ±6 and rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to
// the even code (mantissa bit 0); sign kept (also of zero). A NaN/Inf block gets scale 0xFF and
// codes 0. Codes are packed two per byte, element 2i in the low nibble: [T, h, d/2].
__global__ __launch_bounds__(256) void mx_quantize_d_fp4_kernel(const __bf16* __restrict__ x,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales, long n_blocks) {
  const long blk = (long)blockIdx.x * 64 + threadIdx.x / 4;
  const int sub = threadIdx.x & 3;
  i32x4 u = i32x4{0, 0, 0, 0};
  if (blk < n_blocks) u = *(const i32x4*)(x + blk * 32 + sub * 8);
  const uint32_t w[4] = {(uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w};
  const uint32_t ab = quad_max(amax_bits<4>(w));
  if (blk >= n_blocks) return;
  const bool bad = ab >= 0x7F80u;
  const int e = e2m1_block_exp(ab);
  *(uint32_t*)(codes + blk * 16 + sub * 4) = (uint32_t)bad_or(bad, 0, (int)e2m1_encode8(w, e));
  if (sub == 0) scales[blk] = bad ? 0xFF : (uint8_t)(e + 127);
}

// E2M3 (FP6) element of an already-scaled value |y| <= 7.5: the magnitudes form a grid of step
// 1/8 on [0, 2), 1/4 on [2, 4) and 1/2 on [4, 7.5], one code per grid point, so rounding the
// position within the binade to the nearest even integer is round-to-nearest, ties to the even
// code. y is a bf16 value times a power of two: every product and difference below is exact.
__device__ inline int e2m3_code(float y) {
  const float a = fabsf(y);
  const int c = a < 2.f ? (int)rintf(a * 8.f) : a < 4.f ? 16 + (int)rintf((a - 2.f) * 4.f)
                                                          : 24 + (int)rintf((a - 4.f) * 2.f);
  return c | (__builtin_signbit(y) ? 32 : 0);
}

// E3M2 (FP6) element of an already-scaled value |y| <= 28: four codes per binade [2^t, 2^(t+1))
// for t >= -2 (step 2^(t-2)), and step 1/16 on [0, 0.5) (subnormals and the first binade), so
// code = round(|y|·2^(2-t)) + 4t + 8 with t = max(floor(log2 |y|), -2); a round-up to the next
// power of two lands on that binade's first code. rintf ties to even, and 4t + 8 is even, so
// ties go to the even code. Every product is exact (scaling by a power of two).
__device__ inline int e3m2_code(float y) {
  const float a = fabsf(y);
  const int t = a < 0.25f ? -2 : __builtin_amdgcn_frexp_expf(a) - 1;
  const int c = (int)rintf(__builtin_amdgcn_ldexpf(a, 2 - t)) + 4 * t + 8;
  return c | (__builtin_signbit(y) ? 32 : 0);
}

// Block exponent with top exponent EMAX: floor(log2 amax) - EMAX clamped to [-127, 127], -127
// for a zero block.
template <int EMAX>
__device__ inline int mx_exponent_top(float amax) {
  if (!(amax > 0.f)) return -127;
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  return min(max(ex - 1 - EMAX, -127), 127);
}

// Two lanes per block of 32 elements, 16 elements (96 code bits) each. Block b of a row is the
// 192-bit little-endian number whose bits 6i..6i+5 hold code i; its bytes 0-15 go to the row's
// 16-byte part [16b, 16b+16), bytes 16-23 to its 8-byte part [d/2 + 8b, d/2 + 8b + 8); a row
// (one token and head) is 3d/4 bytes. Lane 0 owns bytes 0-11 (one 12-byte store), lane 1 bytes
// 12-23 (4 bytes ending the 16-byte part, 8 bytes the 8-byte part). FMT 2: E2M3 (top exponent
// 2, saturation at 7.5); FMT 3: E3M2 (top exponent 4, saturation at 28).
template <int FMT>
__global__ __launch_bounds__(256) void mx_quantize_d_fp6_kernel(const __bf16* __restrict__ x,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales, long n_blocks, int nb) {
  const long blk = (long)blockIdx.x * 128 + threadIdx.x / 2;
  const int sub = threadIdx.x & 1;
  float v[16];
  float amax = 0.f;
  bool bad = false;
  if (blk < n_blocks) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 u = __builtin_bit_cast(bf16x8, *(const i32x4*)(x + blk * 32 + sub * 16 + 8 * hh));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[8 * hh + e] = (float)u[e];
        bad |= !__builtin_isfinite(v[8 * hh + e]);
        amax = fmaxf(amax, fabsf(v[8 * hh + e]));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.f;
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  int badi = bad ? 1 : 0;
  badi |= __shfl_xor(badi, 1);
  if (blk >= n_blocks) return;
  constexpr float VMAX = FMT == 2 ? 7.5f : 28.f;
  const int e = mx_exponent_top<FMT == 2 ? 2 : 4>(amax);
  uint32_t w[3] = {0u, 0u, 0u};                  // this lane's 96 code bits, little endian
  if (!badi) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float y = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[j], -e), -VMAX), VMAX);
      const uint32_t c = (uint32_t)(FMT == 2 ? e2m3_code(y) : e3m2_code(y));
      const int bit = 6 * j;
      w[bit >> 5] |= c << (bit & 31);
      if ((bit & 31) > 26) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));   // a code across two words
    }
  }
  const long row = blk / nb;
  const int b = (int)(blk % nb);
  uint8_t* rowp = codes + row * (long)(24 * nb);
  if (sub == 0) {
    uint32_t* dst = (uint32_t*)(rowp + 16 * b);
    dst[0] = w[0];
    dst[1] = w[1];
    dst[2] = w[2];
    scales[blk] = badi ? 0xFF : (uint8_t)(e + 127);
  } else {
    *(uint32_t*)(rowp + 16 * b + 12) = w[0];
    *(i32x2*)(rowp + 16 * nb + 8 * b) = i32x2{(int)w[1], (int)w[2]};
  }
}

// ------------------------------------------------------------------ token-blocked copies
// A workgroup owns one head and the 128 padded columns [128g, 128g + 128): up to four 32-token
// blocks, each inside one document (blocks never straddle documents; a document's last block is
// zero-padded). Owning four blocks gives every channel row 128 contiguous code bytes, so the
// codes leave as whole 128-byte lines from one workgroup instead of 32-byte pieces from four.
struct BlockGroup {
  int tok0[4];   // packed row of the block's first token
  int ntok[4];   // real tokens in the block
  bool live[4];  // the block lies below the last document's padded end (its bytes are written)
};

// a[b] for a lane-dependent b, as a select chain (an indexed private array would live in scratch)
template <class T>
__device__ inline T sel4(const T (&a)[4], int b) {
  return b == 0 ? a[0] : b == 1 ? a[1] : b == 2 ? a[2] : a[3];
}

__device__ inline BlockGroup block_group(int g, const int2* __restrict__ docinfo, const int* __restrict__ padoff,
                                         int n_docs) {
  BlockGroup bg;
  const int total_cols = __builtin_amdgcn_readfirstlane(padoff[n_docs]);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = 128 * g + 32 * b;
    bg.live[b] = col < total_cols;
    bg.ntok[b] = 0;
    bg.tok0[b] = 0;
    if (bg.live[b]) {
      // the document holding column col: padoff[n] <= col < padoff[n+1] (the last such n, so
      // that empty documents, which own no column, are skipped)
      int lo = 0, hi = n_docs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (padoff[mid] <= col) lo = mid; else hi = mid - 1;
      }
      const int2 di = docinfo[lo];
      const int b0 = col - padoff[lo];
      bg.ntok[b] = __builtin_amdgcn_readfirstlane(min(32, di.y - b0));
      bg.tok0[b] = __builtin_amdgcn_readfirstlane(di.x + b0);
    }
  }
  return bg;
}

// Token-blocked E4M3 encoding of one 128-column group of one head from a bf16 tile in LDS
// (tile row r = column 128g + r, RSTR elements per row, rows past a block's tokens hold zeros).
// KL selects the layout:
//  * KL = false (public): codes [h, d, t_pad] in token order, scales [h, d, t_pad/32];
//  * KL = true (attention kernels' internal copies): within each 32-token block the 4-byte
//    pieces (4 tokens each) are stored in the order 0,2,4,6,1,3,5,7 -- the order in which a
//    matrix-core lane group holds probabilities (tokens 8m + 4g + 0..3 for lane group g) --
//    and scales are block-major [h, t_pad/32, d], so a block's D scale bytes are contiguous.
// 256 threads: 256/D lanes per channel, each encoding 4·D/256 whole blocks of its channel (no
// cross-lane reduction); the bytes meet in the LDS staging rows `ost` (D rows of OSTR bytes,
// which may alias the tile: they are written after a barrier that ends the tile reads) and
// leave as 16-byte stores, eight lanes per 128-byte row segment. Padding tokens of a partial
// block encode 0x00. Ends with the workgroup's stores issued (no barrier after).
template <int D, bool KL>
__device__ inline void encode_t_group(const __bf16* tile, int rstr, uint8_t* ost, const BlockGroup& bg, int g,
                                      int head, int t_pad, uint8_t* __restrict__ codes,
                                      uint8_t* __restrict__ scales) {
  constexpr int OSTR = 144;                         // 128 bytes + 16 (spreads LDS banks)
  constexpr int LPC = 256 / D;                      // lanes per channel
  constexpr int BPL = 4 / LPC;                      // blocks per lane
  const int c = threadIdx.x % D;
  const int part = threadIdx.x / D;
  i32x4 out[BPL][2];
#pragma unroll
  for (int j = 0; j < BPL; ++j) {
    const int b = part * BPL + j;
    const unsigned short* t16 = (const unsigned short*)tile + 32 * b * rstr + c;
    uint32_t w[16];                                 // bytes 2k, 2k + 1 of the block: tokens tk, tk + 1
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = 2 * k;
      const int tk = KL ? 4 * ((i >> 2) < 4 ? 2 * (i >> 2) : 2 * (i >> 2) - 7) + (i & 3) : i;
      w[k] = (uint32_t)t16[tk * rstr] | ((uint32_t)t16[(tk + 1) * rstr] << 16);
    }
    const uint32_t ab = amax_bits<16>(w);
    const bool bad = ab >= 0x7F80u;
    const int e = e4m3_block_exp(ab);
    // rows past the block's tokens hold +0, which encodes as 0x00
#pragma unroll
    for (int q = 0; q < 2; ++q)
      out[j][q] = i32x4{e4m3_encode4(w[8 * q], w[8 * q + 1], e), e4m3_encode4(w[8 * q + 2], w[8 * q + 3], e),
                        e4m3_encode4(w[8 * q + 4], w[8 * q + 5], e), e4m3_encode4(w[8 * q + 6], w[8 * q + 7], e)};
    if (bad) {
      // a NaN/Inf block: 0x7F for the block's tokens, 0x00 for the padding rows
      const int nt = sel4(bg.ntok, b);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        out[j][q] = i32x4{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
#pragma unroll
        for (int i = 16 * q; i < 16 * q + 16; ++i) {
          const int tk = KL ? 4 * ((i >> 2) < 4 ? 2 * (i >> 2) : 2 * (i >> 2) - 7) + (i & 3) : i;
          if (tk >= nt) out[j][q][(i / 4) % 4] &= ~(0xFF << (8 * (i % 4)));
        }
      }
    }
    if (sel4(bg.live, b)) {
      const uint8_t sb = bad ? 0xFF : (uint8_t)(e + 127);
      const int pb = 4 * g + b;
      if (KL) scales[((size_t)head * (t_pad / 32) + pb) * D + c] = sb;
      else scales[((size_t)head * D + c) * (t_pad / 32) + pb] = sb;
    }
  }
  __syncthreads();                                  // every lane is done reading the tile
#pragma unroll
  for (int j = 0; j < BPL; ++j) {
    const int b = part * BPL + j;
    *(i32x4*)(ost + c * OSTR + 32 * b) = out[j][0];
    *(i32x4*)(ost + c * OSTR + 32 * b + 16) = out[j][1];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const int row = threadIdx.x / 8 + 32 * p;
    const int piece = threadIdx.x % 8;
    if (sel4(bg.live, piece / 2)) {
      const i32x4 u = *(const i32x4*)(ost + row * OSTR + 16 * piece);
      // channel row head·D + row; the in-head offset fits 32 bits (D·t_pad < 2^31 is checked on the host)
      *(i32x4*)(codes + (size_t)head * D * t_pad + (uint32_t)(row * t_pad + 128 * g + 16 * piece)) = u;
    }
  }
}

// 16-byte chunk `col` of row r of a block: token tok0 + r of head `head` (h heads). The load
// reads token tok0 + min(r, ntok - 1) (tok0 itself for a dead block, whose tok0 is 0; callers run
// only when the tensor has tokens), so it never leaves the tensor and needs no branch; MASK gives
// zeros for r >= ntok (the rows a token-blocked tile pads with). The block's base address is
// uniform and the lane's offset fits 32 bits (r < 32, h <= 65536 is checked on the host).
template <int D, bool MASK>
__device__ inline i32x4 load_row_chunk(const __bf16* __restrict__ x, int h, int head, int tok0, int r, int ntok,
                                       int col) {
  const char* base = (const char*)(x + ((size_t)tok0 * h + head) * D);
  const int rr = min(r, max(ntok - 1, 0));
  i32x4 u = *(const i32x4*)(base + (uint32_t)(rr * h * D + col * 8) * 2u);
  if (MASK) {
    const int m = r < ntok ? -1 : 0;
    u = i32x4{u.x & m, u.y & m, u.z & m, u.w & m};
  }
  return u;
}

// Load the 128 × D tile of one head and group into LDS (zeros for rows past a block's tokens).
template <int D>
__device__ inline void load_group_tile(const __bf16* __restrict__ x, int h, int head, const BlockGroup& bg,
                                       __bf16* tile, int rstr) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per token row
  constexpr int RPI = 256 / CPR;                    // rows per iteration (16 or 32)
#pragma unroll
  for (int i = 0; i < 128 * CPR / 256; ++i) {
    const int col = threadIdx.x % CPR;
    const int row = RPI * i + threadIdx.x / CPR;
    const int b = RPI * i / 32, r = RPI * i % 32 + threadIdx.x / CPR;   // b known at compile time
    *(i32x4*)(tile + row * rstr + col * 8) = load_row_chunk<D, true>(x, h, head, bg.tok0[b], r, bg.ntok[b], col);
  }
}

// grid: h·ceil(t_pad / 128) workgroups (workgroup g·h + head), 256 threads; D = head dim (64 or
// 128). Heads vary fastest, so the workgroups in flight together read whole token rows (h·D
// contiguous elements) of a few groups.
template <int D, bool KL>
__global__ __launch_bounds__(256, 4) void mx_quantize_t_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, const int2* __restrict__ docinfo,
                                                            const int* __restrict__ padoff, int n_docs, int h,
                                                            int t_pad) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int RSTR = D + 8;                      // bf16 elements per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) __bf16 tile[128 * RSTR];   // staging rows alias it
  uint8_t* ost = (uint8_t*)tile;
  static_assert(D * 144 <= 128 * RSTR * 2, "staging rows fit in the tile");
  const int g = blockIdx.x / h;
  const int hh = blockIdx.x % h;
  const BlockGroup bg = block_group(g, docinfo, padoff, n_docs);
  if (!bg.live[0]) return;
  load_group_tile<D>(x, h, hh, bg, tile, RSTR);
  __syncthreads();
  encode_t_group<D, KL>(tile, RSTR, ost, bg, g, hh, t_pad, codes, scales);
}

// ------------------------------------------------------------------ fused operand preparation
// d-blocked copy of the 128 token rows of one head and group. Four lanes per 32-element block,
// eight elements (16 bytes) per lane, chunk i of the lane: row = tid/16 + 16 i, 16-byte chunk
// tid % 16 of the row. The raw chunks are loaded by the caller (all loads in flight at once).
// QF: 0 E4M3, 1 E2M1, 2 E2M3, 3 E3M2 (the same block rules as the single-format kernels above).
template <int QF>
__device__ inline void quant_d_chunks(const i32x4* raw, const BlockGroup& bg, int h, int head,
                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int D = 128;
  const int ch = threadIdx.x % 16;
  const int sub = ch % 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = i / 2, r = 16 * (i % 2) + threadIdx.x / 16;   // row 32 b + r = tid/16 + 16 i
    const uint32_t w[4] = {(uint32_t)raw[i].x, (uint32_t)raw[i].y, (uint32_t)raw[i].z, (uint32_t)raw[i].w};
    const uint32_t ab = quad_max(amax_bits<4>(w));
    const bool bad = ab >= 0x7F80u;
    if (r >= bg.ntok[b]) continue;
    // (token, head) row tok0 + r: a uniform block base plus a 32-bit lane offset
    const size_t row0 = (size_t)bg.tok0[b] * h + head;
    const uint32_t rh = (uint32_t)(r * h);
    uint8_t* sc = scales + row0 * (D / 32) + rh * (D / 32) + ch / 4;
    if (QF == 0) {
      const int e = e4m3_block_exp(ab);
      const i32x2 c = {bad_or(bad, 0x7F7F7F7F, e4m3_encode4(w[0], w[1], e)),
                       bad_or(bad, 0x7F7F7F7F, e4m3_encode4(w[2], w[3], e))};
      *(i32x2*)(codes + row0 * D + (rh * D + ch * 8)) = c;
      if (sub == 0) *sc = bad ? 0xFF : (uint8_t)(e + 127);
    } else if (QF == 1) {
      const int e = e2m1_block_exp(ab);
      *(uint32_t*)(codes + row0 * (D / 2) + (rh * (D / 2) + ch * 4)) = (uint32_t)bad_or(bad, 0, (int)e2m1_encode8(w, e));
      if (sub == 0) *sc = bad ? 0xFF : (uint8_t)(e + 127);
    } else {
      // 6-bit codes: block kb of a row is the 192-bit number with code i at bits 6i..6i+5; its
      // bytes 0-15 sit at row bytes [16 kb, 16 kb + 16), bytes 16-23 at [D/2 + 8 kb, D/2 + 8 kb + 8).
      // This lane's eight codes are block bits 48 sub .. 48 sub + 47, i.e. block bytes 6 sub .. 6 sub + 5.
      constexpr float VMAX = QF == 2 ? 7.5f : 28.f;
      const int e = mx_exponent_top<QF == 2 ? 2 : 4>(__builtin_bit_cast(float, ab << 16));
      const bf16x8 u = __builtin_bit_cast(bf16x8, raw[i]);
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (float)u[k];
      uint64_t bits = 0;
      if (!bad) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float y = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[j], -e), -VMAX), VMAX);
          bits |= (uint64_t)(QF == 2 ? e2m3_code(y) : e3m2_code(y)) << (6 * j);
        }
      }
      const int kb = ch / 4;
      uint8_t* rowp = codes + row0 * (3 * D / 4) + rh * (3 * D / 4);
      const uint32_t lo4 = (uint32_t)bits, hi2 = (uint32_t)(bits >> 32) & 0xFFFFu;
      const uint32_t lo2 = (uint32_t)bits & 0xFFFFu, hi4 = (uint32_t)(bits >> 16);
      // block bytes 6 sub .. 6 sub + 5 as one 4-byte and one 2-byte store, both naturally aligned
      if (sub == 0) {
        *(uint32_t*)(rowp + 16 * kb) = lo4;
        *(uint16_t*)(rowp + 16 * kb + 4) = (uint16_t)hi2;
      } else if (sub == 1) {
        *(uint16_t*)(rowp + 16 * kb + 6) = (uint16_t)lo2;
        *(uint32_t*)(rowp + 16 * kb + 8) = hi4;
      } else if (sub == 2) {
        *(uint32_t*)(rowp + 16 * kb + 12) = lo4;
        *(uint16_t*)(rowp + D / 2 + 8 * kb) = (uint16_t)hi2;
      } else {
        *(uint16_t*)(rowp + D / 2 + 8 * kb + 2) = (uint16_t)lo2;
        *(uint32_t*)(rowp + D / 2 + 8 * kb + 4) = hi4;
      }
      if (sub == 0) *sc = bad ? 0xFF : (uint8_t)(e + 127);
    }
  }
}

// 6-bit score copies, one whole 32-channel block per lane (e6_encode32, cfa_mx.h).
// Lane mapping: (row, block) pair tid + 256 j (j = 0, 1) is row 64 j + tid/4, block tid % 4; the
// row's 32-token block is 2 j + tid/128 and its row within it (tid/4) % 32.
template <int D>
__device__ inline void load_blocks6(const __bf16* __restrict__ x, int h, int head, const BlockGroup& bg,
                                    i32x4 (&raw)[2][4]) {
  const int kb = threadIdx.x % 4, r = (threadIdx.x / 4) % 32, hi = threadIdx.x >= 128;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int b0 = 2 * j;                         // block 2j (tid < 128) or 2j + 1
    const int tok0 = hi ? bg.tok0[b0 + 1] : bg.tok0[b0], nt = hi ? bg.ntok[b0 + 1] : bg.ntok[b0];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[j][c] = load_row_chunk<D, false>(x, h, head, tok0, r, nt, 4 * kb + c);
  }
}

template <int QF>
__device__ inline void quant6_blocks(const i32x4 (&raw)[2][4], const BlockGroup& bg, int h, int head,
                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int D = 128;
  const int kb = threadIdx.x % 4, r = (threadIdx.x / 4) % 32, hi = threadIdx.x >= 128;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int b0 = 2 * j;
    const int tok0 = hi ? bg.tok0[b0 + 1] : bg.tok0[b0], nt = hi ? bg.ntok[b0 + 1] : bg.ntok[b0];
    if (r >= nt) continue;
    uint32_t w[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[4 * c] = (uint32_t)raw[j][c].x;
      w[4 * c + 1] = (uint32_t)raw[j][c].y;
      w[4 * c + 2] = (uint32_t)raw[j][c].z;
      w[4 * c + 3] = (uint32_t)raw[j][c].w;
    }
    const uint32_t ab = amax_bits<16>(w);
    const bool bad = ab >= 0x7F80u;
    const int e = e6_block_exp<QF>(ab);
    u32x6 cw = e6_encode32<QF>(w, e);
    if (bad) cw = u32x6{0u, 0u, 0u, 0u, 0u, 0u};
    const size_t row0 = (size_t)tok0 * h + head;
    uint8_t* rowp = codes + row0 * (3 * D / 4) + (uint32_t)(r * h) * (3 * D / 4);
    *(i32x4*)(rowp + 16 * kb) = i32x4{(int)cw[0], (int)cw[1], (int)cw[2], (int)cw[3]};
    *(i32x2*)(rowp + D / 2 + 8 * kb) = i32x2{(int)cw[4], (int)cw[5]};
    scales[row0 * (D / 32) + (uint32_t)(r * h) * (D / 32) + kb] = bad ? 0xFF : (uint8_t)(e + 127);
  }
}

// The lane's eight chunks (row tid/16 + 16 i, 16-byte chunk tid % 16) of one head and group; MASK:
// zeros in rows past a block's tokens (needed only where the rows feed a token-blocked tile).
template <int D, bool MASK>
__device__ inline void load_chunks(const __bf16* __restrict__ x, int h, int head, const BlockGroup& bg, i32x4* raw) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = i / 2, r = 16 * (i % 2) + threadIdx.x / 16;   // row 32 b + r = tid/16 + 16 i
    raw[i] = load_row_chunk<D, MASK>(x, h, head, bg.tok0[b], r, bg.ntok[b], threadIdx.x % 16);
  }
}

// Forward operand copies in one pass over K and V (each read once): workgroup g·hkv + head of
// hkv·ceil(t_pad/128) (heads fastest) writes K_d (score format QF), V_d (E4M3, the dP operand of
// the backward) and the kernel-layout V_t (E4M3) of kv head `head` over the tokens of padded
// columns [128g, 128g + 128). Q is quantised by the MX forward kernel, which reads it anyway.
template <int QF>
__global__ __launch_bounds__(256, 3) void mx_prep_fwd_kernel(const __bf16* __restrict__ k,
                                                          const __bf16* __restrict__ v, MxPrepOut out,
                                                          const int2* __restrict__ docinfo,
                                                          const int* __restrict__ padoff, int n_docs, int hkv,
                                                          int t_pad) {
  constexpr int D = 128, RSTR = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 tile[128 * RSTR];   // staging rows alias it
  uint8_t* ost = (uint8_t*)tile;
  static_assert(D * 144 <= 128 * RSTR * 2, "staging rows fit in the tile");
  const int g = blockIdx.x / hkv;
  const int head = blockIdx.x % hkv;
  const BlockGroup bg = block_group(g, docinfo, padoff, n_docs);
  if (!bg.live[0]) return;
  i32x4 rv[8];
  if constexpr (QF >= 2) {                        // 6-bit score copies: one block per lane
    i32x4 rk[2][4];
    load_blocks6<D>(k, hkv, head, bg, rk);
    load_chunks<D, true>(v, hkv, head, bg, rv);
    quant6_blocks<QF>(rk, bg, hkv, head, out.b_codes, out.b_scales);
  } else {
    i32x4 rk[8];
    load_chunks<D, false>(k, hkv, head, bg, rk);
    load_chunks<D, true>(v, hkv, head, bg, rv);
    quant_d_chunks<QF>(rk, bg, hkv, head, out.b_codes, out.b_scales);
  }
  quant_d_chunks<0>(rv, bg, hkv, head, out.c_codes, out.c_scales);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = threadIdx.x / 16 + 16 * i;
    *(i32x4*)(tile + row * RSTR + (threadIdx.x % 16) * 8) = rv[i];   // zeros past a block's tokens
  }
  __syncthreads();
  encode_t_group<D, true>(tile, RSTR, ost, bg, g, head, t_pad, out.t_codes, out.t_scales);
}

// Backward preparation in one pass over O and dO: workgroup g·hq + head (heads fastest) writes, for the tokens of padded columns [128g, 128g + 128) and query head `head`,
//   D_i = Σ_r dO_ir O_ir − dLSE_i  (delta [hq, T]; 16 lanes per row, each summing 8 products in
//        order, then a butterfly over offsets 8, 4, 2, 1: the summation order of bwd_pre_kernel),
//   dO_d (E4M3, d-blocked) and the kernel-layout dO_t (E4M3, token-blocked).
__global__ __launch_bounds__(256, 4) void mx_prep_bwd_kernel(const __bf16* __restrict__ o,
                                                          const __bf16* __restrict__ dout,
                                                          const float* __restrict__ dlse, float* __restrict__ delta,
                                                          MxPrepOut out, const int2* __restrict__ docinfo,
                                                          const int* __restrict__ padoff, int n_docs,
                                                          int total_tokens, int hq, int t_pad) {
  constexpr int D = 128, RSTR = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 tile[128 * RSTR];   // staging rows alias it
  uint8_t* ost = (uint8_t*)tile;
  static_assert(D * 144 <= 128 * RSTR * 2, "staging rows fit in the tile");
  const int g = blockIdx.x / hq;
  const int head = blockIdx.x % hq;
  const BlockGroup bg = block_group(g, docinfo, padoff, n_docs);
  if (!bg.live[0]) return;
  i32x4 ro[8], rd[8];
  load_chunks<D, false>(o, hq, head, bg, ro);
  load_chunks<D, true>(dout, hq, head, bg, rd);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = threadIdx.x / 16 + 16 * i;
    *(i32x4*)(tile + row * RSTR + (threadIdx.x % 16) * 8) = rd[i];
    const bf16x8 x = __builtin_bit_cast(bf16x8, ro[i]), y = __builtin_bit_cast(bf16x8, rd[i]);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    const int b = i / 2, r = 16 * (i % 2) + threadIdx.x / 16;
    if (threadIdx.x % 16 == 0 && r < bg.ntok[b]) {
      const size_t di = (size_t)head * total_tokens + bg.tok0[b] + r;
      delta[di] = dlse ? acc - dlse[di] : acc;
    }
  }
  quant_d_chunks<0>(rd, bg, hq, head, out.a_codes, out.a_scales);
  __syncthreads();
  encode_t_group<D, true>(tile, RSTR, ost, bg, g, head, t_pad, out.t_codes, out.t_scales);
}

hipError_t launch_mx_quantize_d(const void* x, long n_elems, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const long n_blocks = n_elems / 32;
  if (n_blocks == 0) return hipSuccess;
  const long grid = (n_blocks + 63) / 64;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mx_quantize_d_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const __bf16*)x, codes, scales,
                     n_blocks);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_d_fp4(const void* x, long n_elems, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const long n_blocks = n_elems / 32;
  if (n_blocks == 0) return hipSuccess;
  const long grid = (n_blocks + 63) / 64;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mx_quantize_d_fp4_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const __bf16*)x, codes,
                     scales, n_blocks);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_d_fp6(const void* x, long n_elems, int d, int fmt, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream) {
  const long n_blocks = n_elems / 32;
  if (n_blocks == 0) return hipSuccess;
  if (fmt != 2 && fmt != 3) return hipErrorInvalidValue;
  const long grid = (n_blocks + 127) / 128;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fmt == 2 ? mx_quantize_d_fp6_kernel<2> : mx_quantize_d_fp6_kernel<3>, dim3((unsigned)grid),
                     dim3(256), 0, stream, (const __bf16*)x, codes, scales, n_blocks, d / 32);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_t(const void* x, int total_tokens, int h, int d, const void* ws, int n_docs,
                                uint8_t* codes, uint8_t* scales, int t_pad, bool kernel_layout, hipStream_t stream) {
  const PlanLayout lay(n_docs);
  const char* b = (const char*)ws;
  const int2* docinfo = (const int2*)(b + lay.docinfo);
  const int* padoff = (const int*)(b + lay.padoff);
  const long ng = ((long)t_pad + 127) / 128;        // 128-column groups covering every padded block
  if (ng == 0 || h == 0 || total_tokens == 0) return hipSuccess;
  if (ng * h > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(ng * h));             // heads fastest: neighbouring workgroups read one token row
#define CFA_MXQT(DD, KK)                                                                                     \
  hipLaunchKernelGGL((mx_quantize_t_kernel<DD, KK>), grid, dim3(256), 0, stream, (const __bf16*)x, codes, scales, \
                     docinfo, padoff, n_docs, h, t_pad)
  if (d == 128 && kernel_layout) CFA_MXQT(128, true);
  else if (d == 128) CFA_MXQT(128, false);
  else if (d == 64 && kernel_layout) CFA_MXQT(64, true);
  else if (d == 64) CFA_MXQT(64, false);
  else return hipErrorInvalidValue;
#undef CFA_MXQT
  return hipGetLastError();
}

hipError_t launch_mx_prep_fwd(const void* k, const void* v, int total_tokens, int hkv, const void* ws, int n_docs,
                              int qf, const MxPrepOut& out, int t_pad, hipStream_t stream) {
  const PlanLayout lay(n_docs);
  const char* b = (const char*)ws;
  const long ng = ((long)t_pad + 127) / 128;
  if (ng == 0 || total_tokens == 0) return hipSuccess;
  if (ng * hkv > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(ng * hkv));           // heads fastest: neighbouring workgroups read one token row
  auto kern = qf == 1 ? mx_prep_fwd_kernel<1> : qf == 2 ? mx_prep_fwd_kernel<2> : qf == 3 ? mx_prep_fwd_kernel<3>
                                                                                         : mx_prep_fwd_kernel<0>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, (const __bf16*)k, (const __bf16*)v, out,
                     (const int2*)(b + lay.docinfo), (const int*)(b + lay.padoff), n_docs, hkv, t_pad);
  return hipGetLastError();
}

hipError_t launch_mx_prep_bwd(const void* o, const void* dout, const float* dlse, float* delta, int total_tokens,
                              int hq, const void* ws, int n_docs, const MxPrepOut& out, int t_pad,
                              hipStream_t stream) {
  const PlanLayout lay(n_docs);
  const char* b = (const char*)ws;
  const long ng = ((long)t_pad + 127) / 128;
  if (ng == 0 || total_tokens == 0) return hipSuccess;
  if (ng * hq > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(ng * hq));            // heads fastest: neighbouring workgroups read one token row
  hipLaunchKernelGGL(mx_prep_bwd_kernel, grid, dim3(256), 0, stream, (const __bf16*)o, (const __bf16*)dout, dlse,
                     delta, out, (const int2*)(b + lay.docinfo), (const int*)(b + lay.padoff), n_docs, total_tokens,
                     hq, t_pad);
  return hipGetLastError();
}

}  // namespace cfa

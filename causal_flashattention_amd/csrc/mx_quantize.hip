// MX quantiser for gfx950: bf16 -> FP8 E4M3 (or FP4 E2M1) codes + E8M0 scales, one scale per 32.
//
// The MXFP8 attention path and its document-local token-block scaling are named on the FLAMIA
// page ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri"); the bit-level rule is the public MX one:
// per block, amax = max|x|, e = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for a zero
// block), scale byte e + 127; elements x·2^-e saturated to ±448 and rounded to nearest E4M3
// (ties to even, sign of zero kept; v_cvt_pk_fp8_f32 rounds to nearest even and does not
// saturate, hence the clamp); a block holding NaN/Inf gets scale 0xFF and codes 0x7F.
//
// Both kernels are HBM-bound streaming passes (2 bytes read, 1 + 1/32 bytes written per
// element):
//  * along d: 4 lanes per 32-channel block, 16 bytes per lane, amax by two lane swaps;
//  * along doc-local tokens: a workgroup per (32-token block, head) reads the 32 × d tile with
//    16-byte loads into LDS, each lane reduces 16 tokens of one channel, the two lanes of a
//    channel meet in LDS, and each lane writes 16 code bytes of its channel row in the
//    transposed [h, d, t_pad] layout.
#include "cfa_device.h"

namespace cfa {

__device__ inline int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int ex = __builtin_amdgcn_frexp_expf(amax);  // amax = f·2^ex, f in [0.5, 1)
  return min(max(ex - 1 - 8, -127), 127);
}

// Quantise 8 values with a shared exponent e into 8 E4M3 bytes (little-endian in a uint2).
__device__ inline i32x2 mx_encode8(const float* x, int e) {
  i32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(__builtin_amdgcn_ldexpf(x[4 * w + i], -e), -448.f), 448.f);
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);   // bytes 0, 1
    word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);     // bytes 2, 3
    r[w] = word;
  }
  return r;
}

__global__ __launch_bounds__(256) void mx_quantize_d_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, long n_blocks) {
  const long blk = (long)blockIdx.x * 64 + threadIdx.x / 4;
  const int sub = threadIdx.x & 3;
  float v[8];
  float amax = 0.f;
  bool bad = false;
  if (blk < n_blocks) {
    const bf16x8 u = __builtin_bit_cast(bf16x8, *(const i32x4*)(x + blk * 32 + sub * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)u[e];
      bad |= !__builtin_isfinite(v[e]);
      amax = fmaxf(amax, fabsf(v[e]));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  int badi = bad ? 1 : 0;
  badi |= __shfl_xor(badi, 1);
  badi |= __shfl_xor(badi, 2);
  if (blk >= n_blocks) return;
  const int e = mx_exponent(amax);
  i32x2 c = badi ? i32x2{0x7F7F7F7F, 0x7F7F7F7F} : mx_encode8(v, e);
  *(i32x2*)(codes + blk * 32 + sub * 8) = c;
  if (sub == 0) scales[blk] = badi ? 0xFF : (uint8_t)(e + 127);
}

// E2M1 (MXFP4) along d: the same block rule with the E2M1 top exponent 2, e = floor(log2 amax) - 2;
// elements x·2^-e clamped to ±6 and rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to
// the even code (mantissa bit 0); sign kept (also of zero). A NaN/Inf block gets scale 0xFF and
// codes 0. Codes are packed two per byte, element 2i in the low nibble: [T, h, d/2].
__device__ inline int mx_exponent_fp4(float amax) {
  if (!(amax > 0.f)) return -127;
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  return min(max(ex - 1 - 2, -127), 127);
}
__device__ inline int e2m1_code(float y) {
  const float a = fabsf(y);
  const int c = a <= 0.25f ? 0 : a < 0.75f ? 1 : a <= 1.25f ? 2 : a < 1.75f ? 3
              : a <= 2.5f ? 4 : a < 3.5f ? 5 : a <= 5.f ? 6 : 7;
  return c | (__builtin_signbit(y) ? 8 : 0);
}

__global__ __launch_bounds__(256) void mx_quantize_d_fp4_kernel(const __bf16* __restrict__ x,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales, long n_blocks) {
  const long blk = (long)blockIdx.x * 64 + threadIdx.x / 4;
  const int sub = threadIdx.x & 3;
  float v[8];
  float amax = 0.f;
  bool bad = false;
  if (blk < n_blocks) {
    const bf16x8 u = __builtin_bit_cast(bf16x8, *(const i32x4*)(x + blk * 32 + sub * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)u[e];
      bad |= !__builtin_isfinite(v[e]);
      amax = fmaxf(amax, fabsf(v[e]));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  int badi = bad ? 1 : 0;
  badi |= __shfl_xor(badi, 1);
  badi |= __shfl_xor(badi, 2);
  if (blk >= n_blocks) return;
  const int e = mx_exponent_fp4(amax);
  uint32_t word = 0;
  if (!badi) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      word |= (uint32_t)e2m1_code(fminf(fmaxf(__builtin_amdgcn_ldexpf(v[j], -e), -6.f), 6.f)) << (4 * j);
  }
  *(uint32_t*)(codes + blk * 16 + sub * 4) = word;
  if (sub == 0) scales[blk] = badi ? 0xFF : (uint8_t)(e + 127);
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

// grid: (padded 32-token blocks upper bound) × h; block 256 threads; D = head dim (64 or 128).
// The 32 × D tile is read with 16-byte loads along channels into LDS, then each lane of the
// first 2·D threads reduces 16 tokens of one channel; the two lanes of a channel meet in LDS.
// KL selects the layout:
//  * KL = false (public): codes [h, d, t_pad] in token order, scales [h, d, t_pad/32];
//  * KL = true (attention kernels' internal copies): within each 32-token block the 4-byte
//    pieces (4 tokens each) are stored in the order 0,2,4,6,1,3,5,7 -- the order in which a
//    matrix-core lane group holds probabilities (tokens 8m + 4g + 0..3 for lane group g) --
//    and scales are block-major [h, t_pad/32, d], so a block's 128 scale bytes are contiguous.
//    Lane group g (g = 0, 1) then handles exactly the tokens stored in bytes 16g..16g+15.
template <int D, bool KL>
__global__ __launch_bounds__(256) void mx_quantize_t_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, const int2* __restrict__ docinfo,
                                                            const int* __restrict__ padoff, int n_docs, int h,
                                                            int t_pad) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int RSTR = D + 8;                      // bf16 elements per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) __bf16 tile[32 * RSTR];
  __shared__ float s_amax[2][D];
  __shared__ int s_bad[2][D];
  const int pb = blockIdx.x;           // padded block index (column pb*32)
  const int hh = blockIdx.y;
  const int total_cols = padoff[n_docs];
  if (pb * 32 >= total_cols) return;
  // document holding column pb*32: padoff[n] <= pb*32 < padoff[n+1]
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (padoff[mid] <= pb * 32) lo = mid; else hi = mid - 1;
  }
  const int2 di = docinfo[lo];
  const int b0 = pb * 32 - padoff[lo];            // doc-local first token of this block
  const int ntok = min(32, di.y - b0);            // real tokens in the block
  constexpr int CPR = D / 8;                      // 16-byte chunks per token row
#pragma unroll
  for (int i = 0; i < (32 * CPR + 255) / 256; ++i) {
    const int cidx = threadIdx.x + 256 * i;
    if (cidx < 32 * CPR) {
      const int row = cidx / CPR, col = cidx % CPR;
      i32x4 u = i32x4{0, 0, 0, 0};
      if (row < ntok) u = *(const i32x4*)(x + ((size_t)(di.x + b0 + row) * h + hh) * D + col * 8);
      *(i32x4*)(tile + row * RSTR + col * 8) = u;
    }
  }
  __syncthreads();
  const int c = threadIdx.x % D;                  // channel
  const int half = threadIdx.x / D;               // lane group: 16 of the 32 tokens
  const bool active = threadIdx.x < 2 * D;
  auto token = [&](int i) { return KL ? 8 * (i >> 2) + 4 * half + (i & 3) : 16 * half + i; };
  float v[16];
  float amax = 0.f;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float val = active ? (float)tile[token(i) * RSTR + c] : 0.f;
    v[i] = val;
    bad |= !__builtin_isfinite(val);
    amax = fmaxf(amax, fabsf(val));
  }
  if (active) { s_amax[half][c] = amax; s_bad[half][c] = bad; }
  __syncthreads();
  if (!active) return;
  amax = fmaxf(s_amax[0][c], s_amax[1][c]);
  bad = s_bad[0][c] | s_bad[1][c];
  const int e = mx_exponent(amax);
  i32x4 out;
  if (bad) {
    out = i32x4{0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F, 0x7F7F7F7F};
  } else {
    const i32x2 lo8 = mx_encode8(v, e), hi8 = mx_encode8(v + 8, e);
    out = i32x4{lo8.x, lo8.y, hi8.x, hi8.y};
  }
  // padding tokens of a partial last block encode 0x00 (not -0 or NaN)
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (token(i) >= ntok) out[i / 4] &= ~(0xFF << (8 * (i % 4)));
  const size_t row = (size_t)hh * D + c;
  *(i32x4*)(codes + row * t_pad + pb * 32 + 16 * half) = out;
  const uint8_t sb = bad ? 0xFF : (uint8_t)(e + 127);
  if (half == 0) {
    if (KL) scales[((size_t)hh * (t_pad / 32) + pb) * D + c] = sb;
    else scales[row * (t_pad / 32) + pb] = sb;
  }
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
  const long nb = (long)(total_tokens + 31) / 32 + n_docs;   // bound on padded blocks
  if (nb == 0 || h == 0) return hipSuccess;
  const dim3 grid((unsigned)nb, (unsigned)h);
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

}  // namespace cfa

// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers, the work-list
// decode, bf16 packing and the workspace layout. No host logic lives here.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------- workspace layout
// All sections 256-byte aligned. The plan part is shared by every pass:
//   header   int[64]              [0] flag (bit0 cu[0]!=0, bit1 decreasing, bit2 cu[n]!=T:
//                                  every document was made empty; bit3: a bounded wait of the
//                                  fused backward gave up), [2] chain counter, [16, 48) per-XCD
//                                  claim words of the fused backward; all but [0] zeroed by the plan
//   docinfo  int2[n_docs]         (first packed row, length) after clamping
//   order    int[n_docs]          documents sorted by length, longest first
//   pref     int[4][n_docs+1]     item prefix over `order` for tiles of 32, 64, 128, 256 rows
//   padoff   int[n_docs+1]        MX token-block column offsets P_n (document order)
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PlanLayout {
  size_t header, docinfo, order, pref, padoff, end;
  __host__ __device__ explicit PlanLayout(int n_docs) {
    header = 0;
    docinfo = align256(header + 64 * sizeof(int));
    order = align256(docinfo + size_t(n_docs) * 2 * sizeof(int));
    pref = align256(order + size_t(n_docs) * sizeof(int));
    padoff = align256(pref + 6 * size_t(n_docs + 1) * sizeof(int));
    end = align256(padoff + size_t(n_docs + 1) * sizeof(int));
  }
};

// Output sections of the fused MX operand preparation kernels: up to three d-blocked copies
// (a, b, c: codes and scales) and one kernel-layout token-blocked copy (t).
struct MxPrepOut {
  uint8_t *a_codes, *a_scales, *b_codes, *b_scales, *c_codes, *c_scales, *t_codes, *t_scales;
};

struct Plan {
  const int* header;     // header[0]: the validation flag (non-zero: every document is empty)
  const int2* docinfo;
  const int* order;
  const int* pref;  // prefix for the kernel's tile size, n_docs+1 entries
  int n_docs;
};

__host__ __device__ inline int pref_slot(int tile_rows) {
  return tile_rows == 32 ? 0 : tile_rows == 64 ? 1 : tile_rows == 128 ? 2 : tile_rows == 256 ? 3 : tile_rows == 512 ? 4 : 5;
}

// Decode work item p (0-based position in the longest-first list) into a document and a tile.
// Returns false when p is past the end of the list (the grid is sized by an upper bound).
// `expensive_first`: tile index counts down from the document's last tile (forward, dQ: the
// tile with the most causal key tiles first); otherwise it counts up (dK/dV: key tile 0 sees
// every query tile).
__device__ inline bool decode_item(const Plan& pl, int p, int tile_rows, bool expensive_first,
                                   int& s0, int& L, int& tile, int* doc_out = nullptr) {
  const int total = pl.pref[pl.n_docs];
  if (p >= total) return false;
  int lo = 0, hi = pl.n_docs - 1;  // find i: pref[i] <= p < pref[i+1]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pl.pref[mid] <= p) lo = mid; else hi = mid - 1;
  }
  // every value here is the same in all lanes (p is per workgroup); readfirstlane tells the
  // compiler so, which keeps the work-item arithmetic and everything derived from it scalar
  const int doc = __builtin_amdgcn_readfirstlane(pl.order[lo]);
  if (doc_out) *doc_out = doc;
  const int2 di = pl.docinfo[doc];
  s0 = __builtin_amdgcn_readfirstlane(di.x);
  L = __builtin_amdgcn_readfirstlane(di.y);
  const int nt = (L + tile_rows - 1) / tile_rows;
  const int j = p - __builtin_amdgcn_readfirstlane(pl.pref[lo]);
  tile = __builtin_amdgcn_readfirstlane(expensive_first ? (nt - 1 - j) : j);
  return true;
}

// ---------------------------------------------------------------- MFMA wrappers
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane i receives
// element (i % 4) of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ inline i16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds_ptr));
}

__device__ inline bf16x8 concat_tr(i16x4 a, i16x4 b) {
  i32x2 ua = __builtin_bit_cast(i32x2, a);
  i32x2 ub = __builtin_bit_cast(i32x2, b);
  i32x4 u = {ua.x, ua.y, ub.x, ub.y};
  return __builtin_bit_cast(bf16x8, u);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; a in bits 15:0.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Scaled FP8 MFMA, E4M3 operands, E8M0 scales (bits 7:0 of sa / sb). Operand layout per lane l:
// row (A) or column (B) l%32; bytes 0-15 hold k = 16·(l/32) + 0..15, bytes 16-31 hold
// k = 32 + 16·(l/32) + 0..15; lane l supplies the scale of row/column l%32 for k-block l/32.
__device__ inline f32x16 mfma32_mx(i32x8 a, int sa, i32x8 b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Scaled MFMA with E2M1 (FP4, format code 4) A and B: operand layout per lane l: row/column l%32,
// k = 32·(l/32) + 0..31 in bytes 0-15, element 2i in the low nibble of byte i (bytes 16-31
// unused); scales as above (pinned by a probe against a CPU product, also mixed with an E4M3 B).
__device__ inline f32x16 mfma32_mx_fp4(i32x8 a, int sa, i32x8 b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
__device__ inline i32x8 fp4_operand(i32x4 u) { return i32x8{u.x, u.y, u.z, u.w, 0, 0, 0, 0}; }

// Scaled MFMA with 6-bit A and B, FMT = the instruction's format code: 2 = E2M3, 3 = E3M2. Per
// lane l, row/column l%32, k = 32·(l/32) + i for the code at bits 6i..6i+5 of the 192-bit
// little-endian operand in dwords 0-5 (pinned for E2M3 by a probe against a CPU product with
// per-block scales; E3M2 differs only in how a code decodes); scales as above. The operand is
// assembled from a block's 16-byte part (dwords 0-3) and 8-byte part (dwords 4-5).
template <int FMT>
__device__ inline f32x16 mfma32_mx_fp6(i32x8 a, int sa, i32x8 b, int sb, f32x16 c) {
  static_assert(FMT == 2 || FMT == 3, "6-bit format codes are 2 (E2M3) and 3 (E3M2)");
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, sa, 0, sb);
}
__device__ inline i32x8 fp6_operand(i32x4 lo, i32x2 hi) { return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, 0, 0}; }

// Scaled MFMA (A format FA, B format FB) whose A scale is byte `sel` of `sa_word`, picked by the
// instruction's byte select, so a lane holding a token's four block scales in one word needs no
// shift and mask per product. `sel` must be a compile-time constant after unrolling.
template <int FA, int FB>
__device__ inline f32x16 mfma32_scale_byte(i32x8 a, int sa_word, int sel, i32x8 b, int sb, f32x16 c) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa_word, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 1, sa_word, 0, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 2, sa_word, 0, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 3, sa_word, 0, sb);
  }
}

// Four floats -> four E4M3 bytes (round to nearest even; inputs must already lie in ±448).
// The first conversion writes bytes 0-1 and keeps bytes 2-3 of its `old` operand, which the
// second one overwrites: any register will do, and b's (usually dead afterwards) saves a move.
__device__ inline int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, b), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

typedef __attribute__((ext_vector_type(2))) short i16x2;

// Four floats -> four E4M3 bytes of x / s for a power of two s, in two v_cvt_scalef32_pk_fp8_f32
// (round to nearest even, no saturation: callers keep |x / s| <= 448).
__device__ inline int pack_fp8x4_scaled(float a, float b, float c, float d, float s) {
  // `old` as in pack_fp8x4: its bytes 2-3 are overwritten by the second conversion
  i16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(i16x2, b), a, b, s, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, s, true);
  return __builtin_bit_cast(int, w);
}

// Two E4M3 bytes (bytes 0-1, or 2-3 when HI) -> floats × s for a power of two s.
template <bool HI>
__device__ inline f32x2 unpack_fp8x2_scaled(int word, float s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, s, HI);
}

// Two E4M3 bytes (bytes 0-1, or 2-3 when HI) -> bf16 pair × s (s a power of two), packed in one
// 32-bit word with byte 0 (2) in the low half; exact whenever the products are normal bf16
// values (E4M3 has 3 mantissa bits): bit-identical to unpack_fp8x2_scaled + pack_bf16x2.
template <bool HI>
__device__ inline int fp8x2_to_bf16x2_scaled(int word, float s) {
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, s, HI));
}

// 2^e as a float for -126 <= e <= 127 (exponent field only); 2^-127 is built by ldexp.
__device__ inline float pow2i(int e) { return e >= -126 ? __builtin_bit_cast(float, (e + 127) << 23) : 0x1p-127f; }

// LDS layout of a bf16 tile with rows of D elements that is read both row-wise (ds_read_b128:
// 16 lanes take one 16-byte chunk of 16 consecutive rows) and transposed (ds_read_b64_tr_b16:
// 32 lanes take 4 rows × 4 consecutive chunks). For D = 128, rows are 256 bytes (no padding)
// and chunk c of row r is stored at chunk position c ^ f(r), f(r) = 4·(r%4) + (r/4)%4:
// f is a bijection on 16 consecutive rows (row reads hit 16 distinct chunk slots) and, for
// 4 rows r ≡ 0..3 (mod 4), moves the 4-chunk group by a different multiple of 4 (transposed
// reads hit 16 distinct slots), so both patterns cover the 64 banks once. D = 256: rows of 512
// bytes, each 256-byte half swizzled as a D = 128 row (a 512-byte stride maps onto the banks as
// a 256-byte one). D = 64 uses a padded 144-byte row instead.
template <int D>
struct SwzTile {
  static constexpr bool SWZ = D >= 128;
  static constexpr int STR = SWZ ? 2 * D : D * 2 + 16;
  __device__ static inline int f(int r) { return SWZ ? (4 * (r & 3) + ((r >> 2) & 3)) : 0; }
  // byte offset of 16-byte chunk c of row r
  __device__ static inline int chunk(int r, int c) {
    return SWZ ? r * STR + ((c >> 4) << 8) + (((c & 15) ^ f(r)) << 4) : r * STR + (c << 4);
  }
  // byte offset of element d of row r (d % 4 == 0 for 8-byte transposed reads)
  __device__ static inline int elem(int r, int d) { return chunk(r, d >> 3) + ((d & 7) << 1); }
};

// Lane-constant byte offsets of the two read patterns on a SwzTile (row blocks of 32 rows and
// 16-row groups move the offsets by whole rows, which never changes f, so the swizzle is folded
// into these few registers and the rest are immediate offsets):
//  row reads:   lane reads chunk 2s + half of row (lane & 31)               -> row[s]
//  transposed:  lane reads d = 32·db + 16·((lane>>4)&1) + 4·(lane&3) of rows
//               4·half + (lane&15)/4 (+0 and +8)                            -> tr0[db], tr1[db]
template <int D>
struct SwzOffsets {
  int row[D / 16];
  int tr0[D / 32], tr1[D / 32];
  __device__ explicit SwzOffsets(int lane) {
    using S = SwzTile<D>;
    constexpr int W = D < 128 ? D : 128;          // d = 256: the upper half is the lower + 256 B
    const int half = lane >> 5;
#pragma unroll
    for (int s = 0; s < W / 16; ++s) row[s] = S::chunk(lane & 31, 2 * s + half);
    const int r = 4 * half + ((lane & 15) >> 2);
    const int dsub = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < W / 32; ++db) {
      tr0[db] = S::elem(r, 32 * db + dsub);
      tr1[db] = S::elem(r + 8, 32 * db + dsub);
    }
#pragma unroll
    for (int s = W / 16; s < D / 16; ++s) row[s] = row[s - W / 16] + 256;
#pragma unroll
    for (int db = W / 32; db < D / 32; ++db) {
      tr0[db] = tr0[db - W / 32] + 256;
      tr1[db] = tr1[db - W / 32] + 256;
    }
  }
};

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): the wave writes
// 1 KB at lds_wave_base + 16·lane; lds_wave_base must be the same for the whole wave.
__device__ inline void g2lds16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// Direct global -> LDS copy of 4 bytes per lane: LDS[lds_wave_base + 4·lane].
__device__ inline void g2lds4(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}

// Raw buffer resource over the `bytes` bytes from `base` (reads past them return zeros). Both are
// read from the first lane, so the resource lives in scalar registers: they must be the same in
// every lane.
__device__ inline __amdgpu_buffer_rsrc_t rsrc_at(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc((void*)u, 0, __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
// g2lds16 through a buffer resource: the source is the resource base + voff (a 32-bit lane
// offset), so copies whose lane offsets repeat need no per-copy address arithmetic.
__device__ inline void b2lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, 0, 0, 0);
}
__device__ inline void b2lds4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 4, voff, 0, 0, 0);
}

// XOR swizzles of the 16-byte chunks of E4M3 code tiles in LDS, chosen so that the 16 rows
// read by a 16-lane group at one logical chunk land in 16 distinct 16-byte bank groups:
// d-blocked rows of 128 bytes (8 chunks): rows r and r+1 share a 256-byte bank window, so the
// chunk moves with r/2; token-blocked rows of 64 bytes (4 chunks): 4 rows share a window.
__device__ inline int kd_swz(int r) { return (r >> 1) & 7; }
__device__ inline int vt_swz(int r) { return (r >> 2) & 3; }

// A wave-uniform condition handed to the compiler as a per-lane value: a branch on it is then
// compiled with exec masks and both arms keep one register assignment (on a scalar branch the
// register allocator may copy every accumulator register at the join of the two arms).
__device__ inline bool per_lane(bool b) {
  int v = b;
  asm volatile("" : "+v"(v));
  return v != 0;
}

// Wait until every vector-memory operation of this wave has completed. The builtin lets the
// compiler's wait insertion know that every earlier load has landed, so it adds no wait of its
// own for them later; the empty asm statements keep memory accesses from moving across it.
__device__ inline void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt not waited for
  asm volatile("" ::: "memory");
}
// Wait until at most N vector-memory operations of this wave are outstanding (the N most recent
// may still be in flight).
template <int N>
__device__ inline void wait_vmem_keep() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Workgroup barrier after this wave's LDS operations have completed, without the fence of
// __syncthreads (which would also wait for every outstanding global -> LDS copy). Used where
// the caller has already waited for the copies that the other waves are about to read.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Stage ROWS rows of D bf16 (D = 128: 256 bytes, 256: 512 bytes) into a SwzTile<D> LDS tile
// with direct loads. Called by NW waves; wave w copies the 1 KB blocks
// [w·ROWS/(RB·NW), (w+1)·ROWS/(RB·NW)), block I holding the RB = 1024 / (2·D) rows RB·I ...
// Lane i fills physical chunk i % (D/8) of row RB·I + i / (D/8), i.e. the logical chunk whose
// swizzled position that is: the swizzle is applied on the global side. Tile row r is read from
// base + min(r, rmax)·stride: `base` is wave-uniform (the tile's first row), so each copy is a
// scalar base plus a 32-bit lane offset; rows past rmax repeat row rmax.
template <int ROWS, int NW = 4, int D = 128>
__device__ inline void stage_rows_lds(char* tile, const char* base, uint32_t stride, int rmax, int wave, int lane) {
  static_assert(D == 128 || D == 256, "rows of 256 or 512 bytes");
  constexpr int LPR = D / 8, RB = 64 / LPR;
  static_assert(ROWS % (RB * NW) == 0, "NW waves × RB rows per block");
  constexpr int PER_WAVE = ROWS / (RB * NW);
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int I = wave * PER_WAVE + j;
    const int r = RB * I + lane / LPR;
    const int pc = lane % LPR;                    // physical chunk
    const uint32_t c = (uint32_t)((pc & 16) | ((pc & 15) ^ SwzTile<D>::f(r)));
    g2lds16(base + ((uint32_t)min(r, rmax) * stride + c * 16), tile + I * 1024);
  }
}

// The copies of stage_rows_lds<ROWS, NW, D> as buffer loads: the lane offsets from a tile's first
// row are computed once (they repeat from tile to tile), and each tile gets a scalar resource
// that ends after row rmax, so rows past it read zeros instead of repeating row rmax (callers
// mask those rows). No per-copy address arithmetic is left in a loop over tiles.
template <int ROWS, int NW, int D>
struct RowCopies {
  static_assert(D == 128 || D == 256, "rows of 256 or 512 bytes");
  static constexpr int LPR = D / 8, RB = 64 / LPR, PER_WAVE = ROWS / (RB * NW);
  static_assert(ROWS % (RB * NW) == 0, "NW waves × RB rows per block");
  uint32_t off[PER_WAVE];
  uint32_t stride;
  __device__ RowCopies(uint32_t row_stride, int wave, int lane) : stride(row_stride) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int r = RB * (wave * PER_WAVE + j) + lane / LPR, pc = lane % LPR;
      off[j] = (uint32_t)r * stride + 16 * (uint32_t)((pc & 16) | ((pc & 15) ^ SwzTile<D>::f(r)));
    }
  }
  // tile rows 0..ROWS-1 from `base` (row r at base + r·stride; wave-uniform), rows past rmax zero
  __device__ void copy(char* tile, const void* base, int rmax, int wave) const {
    const uint32_t bytes = rmax >= ROWS - 1 ? 0x7fffffffu : rmax < 0 ? 0u : (uint32_t)rmax * stride + D * 2;
    const auto rs = rsrc_at(base, bytes);
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) b2lds16(rs, off[j], tile + (wave * PER_WAVE + j) * 1024);
  }
};

__device__ inline bf16x8 as_bf16x8(const i32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// 2^x with the bare v_exp_f32: results below 2^-126 may flush to zero, which is negligible in
// every use here (probabilities and rescale factors next to a row sum of at least 1).
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of the 32 values of two 16-element accumulators: four independent v_max3 chains of
// 8 values (short dependency chains), then their maximum. Exact, so the order does not matter.
__device__ inline float max32(const f32x16& a, const f32x16& b) {
  float m[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    m[k] = fmaxf(fmaxf(a[4 * k], a[4 * k + 1]), a[4 * k + 2]);
    m[k] = fmaxf(fmaxf(m[k], a[4 * k + 3]), b[4 * k]);
    m[k] = fmaxf(fmaxf(m[k], b[4 * k + 1]), b[4 * k + 2]);
    m[k] = fmaxf(m[k], b[4 * k + 3]);
  }
  return fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
}

// Reductions over the lane pair (l, l ^ 32) with one v_permlane32_swap (no LDS round trip).
// With x in both operands, the first result holds, in the upper half-wave, the lower half's
// values (the lower half keeps its own) and the second result the converse, so the pair
// maximum / sum is one operation on the two results in every lane; addition being commutative,
// both lanes of a pair get the identical sum.
__device__ inline f32x2 pair_swap32(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return f32x2{__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1])};
}
__device__ inline float wave_max_xor32(float x) {
  const f32x2 r = pair_swap32(x);
  return fmaxf(r.x, r.y);
}
__device__ inline float wave_sum_xor32(float x) {
  const f32x2 r = pair_swap32(x);
  return r.x + r.y;
}

}  // namespace cfa

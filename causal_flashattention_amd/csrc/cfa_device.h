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
//   header   int[64]              flag (bit0 cu[0]!=0, bit1 decreasing, bit2 cu[n]!=T), spare
//   docinfo  int2[n_docs]         (first packed row, length) after clamping
//   order    int[n_docs]          documents sorted by length, longest first
//   pref     int[3][n_docs+1]     item prefix over `order` for tiles of 32, 64, 128 rows
//   padoff   int[n_docs+1]        MX token-block column offsets P_n (document order)
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PlanLayout {
  size_t header, docinfo, order, pref, padoff, end;
  __host__ __device__ explicit PlanLayout(int n_docs) {
    header = 0;
    docinfo = align256(header + 64 * sizeof(int));
    order = align256(docinfo + size_t(n_docs) * 2 * sizeof(int));
    pref = align256(order + size_t(n_docs) * sizeof(int));
    padoff = align256(pref + 3 * size_t(n_docs + 1) * sizeof(int));
    end = align256(padoff + size_t(n_docs + 1) * sizeof(int));
  }
};

struct Plan {
  const int2* docinfo;
  const int* order;
  const int* pref;  // prefix for the kernel's tile size, n_docs+1 entries
  int n_docs;
};

__host__ __device__ inline int pref_slot(int tile_rows) { return tile_rows == 32 ? 0 : (tile_rows == 64 ? 1 : 2); }

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
  const int doc = pl.order[lo];
  if (doc_out) *doc_out = doc;
  const int2 di = pl.docinfo[doc];
  s0 = di.x;
  L = di.y;
  const int nt = (L + tile_rows - 1) / tile_rows;
  const int j = p - pl.pref[lo];
  tile = expensive_first ? (nt - 1 - j) : j;
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

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Scaled FP8 MFMA, E4M3 operands, E8M0 scales (bits 7:0 of sa / sb). Operand layout per lane l:
// row (A) or column (B) l%32; bytes 0-15 hold k = 16·(l/32) + 0..15, bytes 16-31 hold
// k = 32 + 16·(l/32) + 0..15; lane l supplies the scale of row/column l%32 for k-block l/32.
__device__ inline f32x16 mfma32_mx(i32x8 a, int sa, i32x8 b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Four floats -> four E4M3 bytes (round to nearest even; inputs must already lie in ±448).
__device__ inline int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ inline float wave_max_xor32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ inline float wave_sum_xor32(float x) { return x + __shfl_xor(x, 32); }

}  // namespace cfa

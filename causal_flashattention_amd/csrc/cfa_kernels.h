// Launchers of the gfx950 kernels, called by the C-ABI host code.
#pragma once
#include <hip/hip_runtime.h>

#include "cfa_device.h"

namespace cfa {

// MX-quantised operands of the MXFP8 backward (codes + scales): d-blocked *_d, token-blocked *_t.
struct MxOperands {
  const uint8_t *qd, *qd_sc, *kd, *kd_sc, *dod, *dod_sc, *vd, *vd_sc;
  const uint8_t *dot, *dot_sc;
};

// naive: documents in index order (a diagnostic for the scheduler's effect); otherwise longest
// first, ties by document index.
hipError_t launch_plan(const int* cu, int n_docs, int total_tokens, void* ws, hipStream_t stream, bool naive = false);

// kdoc != nullptr: cross-attention; the plan is built on the query documents and kdoc[n] =
// (first key row, key count) of document n.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, const Plan& plan,
                           const int* pref_base, int total_tokens, int hq, int hkv, int d, float scale, int causal,
                           hipStream_t stream, const int2* kdoc = nullptr);

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, const Plan& plan,
                          const int* pref_base, int total_tokens, int hq, int hkv, int d, float scale, int causal,
                          hipStream_t stream);

hipError_t launch_bwd_pre(const void* o, const void* dout, const float* dlse, float* delta, int total_tokens, int hq,
                          int d, hipStream_t stream);

// Cross-attention (qdoc / kdoc != nullptr): the dK/dV plan is built on the key documents and
// qdoc[n] = (first query row, query count); the dQ plan on the query documents and kdoc[n] =
// (first key row, key count); T counts query rows, Tk key rows.
// n_split > 1: the query heads of each group are split over n_split workgroups whose fp32
// partial sums go to `part` (2·n_split·T·hkv·d floats, see dkdv_head_split) and are reduced in
// split order.
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* delta, void* dk, void* dv, const Plan& plan, const int* pref_base, int T,
                           int hq, int hkv, int d, float scale, int causal, int n_split, float* part,
                           hipStream_t stream, const int2* qdoc = nullptr, int Tk = 0);

// dK, dV and dQ in one pass (bf16 self-attention, d = 128): dQ is summed over the key tiles in a
// fixed order in dq_acc (float [T][hq][128]) with the counts `cnt` (n_cnt = (t_pad/32)·hq·8 ints,
// zeroed here) and written as bf16 by the last key tile of each query block. `header` is the
// plan header (claim words and chain counter, zeroed by the plan kernel; bit 3 of header[0]
// reports a bounded wait that gave up). kt: FUSED_KT_BYTES of scratch. n_cu: workgroups of the
// persistent grid (at most 256).
hipError_t launch_bwd_dkdv_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              const float* delta, void* dq, void* dk, void* dv, const Plan& plan, int T, int hq, int hkv,
                              float scale, int causal, int n_split, float* part, float* dq_acc, int* cnt, long n_cnt,
                              const int* padoff, int* header, void* kt, int n_cu, hipStream_t stream);
// Bytes of the fused pass's per-workgroup Kᵀ operand slots (256 workgroups × 32 KB).
constexpr size_t FUSED_KT_BYTES = size_t(256) * 8 * 4 * 64 * 16;

// Head split of the bf16 dK/dV pass// Head split of the bf16 dK/dV pass (1 = none): with fewer than 8 kv heads the (key tile,
// kv head) grid is split further over the query heads of each group, up to 8 workgroups per key
// tile (MQA: min(hq, 8)). It depends on the head configuration only, never on the token count or
// the documents, so a document's dK/dV are bit-identical whatever it is packed with.
int dkdv_head_split(int hq, int hkv, int d);

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         const float* delta, void* dq, const Plan& plan, const int* pref_base, int T, int hq,
                         int hkv, int d, float scale, int causal, hipStream_t stream,
                         const int2* kdoc = nullptr);

// Decoding over a packed KV cache (bf16 or MX codes + E8M0 scales): per-chunk partials, then
// their merge in chunk order. part_o: float [slots][hq][d], part_ml: float2 [slots][hq], with
// slots = decode_partial_slots(total_k, n_seqs).
size_t decode_partial_slots(int total_k, int n_seqs);
hipError_t launch_decode(const void* q, const void* k, const void* v, const uint8_t* ks, const uint8_t* vs,
                         const Plan& plan, const int* pref_base, int n_seqs, int total_k, int hq, int hkv, int d,
                         float scale, bool mx, float* part_o, void* part_ml, hipStream_t stream);
hipError_t launch_decode_combine(const float* part_o, const void* part_ml, void* o, float* lse, const Plan& plan,
                                 int n_seqs, int hq, int d, hipStream_t stream);

hipError_t launch_mx_quantize_d(const void* x, long n_elems, uint8_t* codes, uint8_t* scales, hipStream_t stream);
// E2M1 codes packed two per byte ([n_elems / 2] bytes), E8M0 scales [n_elems / 32].
hipError_t launch_mx_quantize_d_fp4(const void* x, long n_elems, uint8_t* codes, uint8_t* scales, hipStream_t stream);
// 6-bit codes [n_elems/d rows][3d/4 bytes] (each block of 32 as a 16-byte and an 8-byte part);
// fmt = MFMA format code: 2 = E2M3, 3 = E3M2
hipError_t launch_mx_quantize_d_fp6(const void* x, long n_elems, int d, int fmt, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream);

// kernel_layout: the attention kernels' internal token-blocked layout (pieces of 4 tokens in
// the order 0,2,4,6,1,3,5,7 within each 32-token block; scales [h, t_pad/32, d]); otherwise the
// public layout of mx_quantize.
hipError_t launch_mx_quantize_t(const void* x, int total_tokens, int h, int d, const void* ws, int n_docs,
                                uint8_t* codes, uint8_t* scales, int t_pad, bool kernel_layout, hipStream_t stream);
// Fused MX operand preparation (one pass each, grid ceil(t_pad/128) × hq):
//   forward : out.b = K_d (score format qf), out.c = V_d (E4M3), out.t = V_t (grid over kv heads;
//             Q is quantised by the MX forward kernel itself);
//   backward: delta = rowsum(dO∘O) − dLSE, out.a = dO_d, out.t = dO_t (E4M3).
hipError_t launch_mx_prep_fwd(const void* k, const void* v, int total_tokens, int hkv, const void* ws, int n_docs,
                              int qf, const MxPrepOut& out, int t_pad, hipStream_t stream);
hipError_t launch_mx_prep_bwd(const void* o, const void* dout, const float* dlse, float* delta, int total_tokens,
                              int hq, const void* ws, int n_docs, const MxPrepOut& out, int t_pad,
                              hipStream_t stream);

// fp4: Q_d, K_d are E2M1 copies (mx_quantize_fp4 layout) and the score product runs on FP4.
// The MX forward quantises Q itself (bf16 q in; Q_d codes and scales written to qd, qd_sc).
hipError_t launch_fwd_mx(const void* q, uint8_t* qd, uint8_t* qd_sc, const uint8_t* kd, const uint8_t* kd_sc,
                         const uint8_t* vt, const uint8_t* vt_sc, const void* v, void* o, float* lse,
                         const Plan& plan, const int* pref_base, const int* padoff, int total_tokens, int t_pad,
                         int hq, int hkv, float scale, int causal, int qf, hipStream_t stream);

hipError_t launch_bwd_dkdv_mx(const MxOperands& m, const void* q, const void* dout, const float* lse,
                              const float* delta, void* dk, void* dv, const Plan& plan, const int* pref_base,
                              const int* padoff, int T, int t_pad, int hq, int hkv, float scale, int causal, int qf, hipStream_t stream);

hipError_t launch_bwd_dq_mx(const MxOperands& m, const void* k, const float* lse, const float* delta, void* dq,
                            const Plan& plan, const int* pref_base, int T, int hq, int hkv, float scale, int causal,
                            int qf, hipStream_t stream);

}  // namespace cfa

/*
 * cfa.h -- C ABI of the causal packed flash-attention library for AMD MI355X (gfx950).
 *
 * What the calls compute (sources are web pages, cited by title and section):
 *
 *   S = scale * Q K^T,  P = softmax(S + causal mask),  O = P V
 *     "GPT Kernel Programlama: MatMul, Softmax ve Attention Hesabı" (dehayz.com), §2 and §3
 *     (the equations and the score sum), §4 (a query never sees later tokens; the mask is
 *     applied by index and never stored), §5 (softmax with the row maximum subtracted),
 *     §6 (the value sum), §7 (tiles of Q/K/V on chip, online softmax, O written once).
 *     "FlashAttention (HU)" (systems-analysis.info), sections "Tiling és blokkos feldolgozás",
 *     "Online Softmax-számítás", "Műveletek összevonása egyetlen CUDA-kernelbe".
 *   Packed variable-length documents, document-local attention, an MXFP8 path with
 *   document-local token-block scales, a causal-leakage safeguard and forward/backward
 *   consistency:
 *     "FLAMIA: Blackwell Üzerinde Hızlı ve Nedensel Olarak Güvenli Eğitim İçin Flash
 *     Mikro-Ölçeklemeli Dikkat Mekanizması" (blog.edumints.com), section "FLAMIA Mimarisi ve
 *     Temel Tasarım İlkeleri".
 *
 * Conventions for every call
 * --------------------------
 *  - Tensors are packed tokens x heads x head-dim, row-major and contiguous:
 *      q, o, dout, dq : [total_tokens, hq,  d]
 *      k, v, dk, dv   : [total_tokens, hkv, d]
 *      lse            : [hq, total_tokens] float32, natural log of sum_j exp(scaled masked score)
 *    Element type: float32 for CFA_F32, bfloat16 (raw 16-bit patterns) otherwise.
 *  - cu_seqlens: int32 [n_docs + 1] in DEVICE memory, cu[0] = 0, non-decreasing,
 *    cu[n_docs] = total_tokens. Document n owns packed rows cu[n] .. cu[n+1]-1; attention
 *    never crosses documents. Empty documents are allowed. cu_seqlens_host is an optional
 *    host copy: when given it is validated before anything is launched.
 *  - Query head h reads kv head h / (hq / hkv) (consecutive query heads share a kv head).
 *  - causal != 0: doc-local key j is visible to doc-local query i iff j <= i.
 *  - Ownership: the caller owns every buffer. The library allocates no device memory, keeps no
 *    state between calls (apart from the thread-local error text and the optional timing events
 *    of cfa_set_kernel_events) and never synchronises the stream; every call only enqueues work on
 *    `stream` (a hipStream_t; NULL is the default stream). Inputs are never written.
 *  - Pointers must be 16-byte aligned. Scratch memory is the caller's `workspace`, at least
 *    cfa_workspace_bytes(...) bytes, 256-byte aligned.
 *  - Errors: every precondition the host can check is checked before any launch; on failure the
 *    call returns a non-zero cfa_status, writes nothing, and cfa_last_error() describes it.
 *    A device-only cu_seqlens that turns out malformed (cu[0] != 0, a decreasing entry or
 *    cu[n_docs] != total_tokens) raises a flag in the workspace, readable with
 *    cfa_device_error(), and makes every document empty: attn_fwd / attn_bwd / the cross calls
 *    then write no row of o, lse, dq, dk, dv (decoding writes each sequence's empty result,
 *    o = 0 and lse = -inf).
 *  - CFA_SCHED=naive in the environment (a diagnostic) schedules documents in index order
 *    instead of longest first; results are bit-identical either way.
 *  - CFA_DEBUG_CHECK=1 in the environment (a diagnostic) makes every call that checks a device
 *    cu_seqlens synchronise on `stream` right after that check and, when it raised the flag,
 *    return CFA_ERR_SHAPE before any other kernel runs (outputs untouched). Not for stream
 *    capture: the check reads the flag back to the host.
 *  - hq <= 65536 on every path (the kernels address the rows of a staged tile with 32-bit
 *    offsets; CFA_ERR_UNSUPPORTED otherwise).
 *  - Size limits of the MX dtypes (CFA_ERR_UNSUPPORTED otherwise): d = 128, hq <= 65536 and
 *    d·(32·ceil(total_tokens/32) + 32·n_docs) < 2^31.
 */
#ifndef CFA_H
#define CFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* CFA_MXFP4: the MXFP8 path with the score product QK^T on E2M1 copies of Q and K (mx_quantize_fp4),
 * a reading of the mixed NVFP4/FP8 path the FLAMIA page names ("FLAMIA Mimarisi ve Temel Tasarım
 * İlkeleri"). CFA_MXFP6: the same with E2M3 copies (mx_quantize_fp6); CFA_MXFP6_E3M2: with E3M2
 * copies (mx_quantize_fp6_e3m2), the other 6-bit MX element type. */
typedef enum {
  CFA_F32 = 0,
  CFA_BF16 = 1,
  CFA_MXFP8 = 2,
  CFA_MXFP4 = 3,
  CFA_MXFP6 = 4,
  CFA_MXFP6_E3M2 = 5
} cfa_dtype;

typedef enum {
  CFA_OK = 0,
  CFA_ERR_NULL = 1,         /* a required pointer is NULL */
  CFA_ERR_SHAPE = 2,        /* inconsistent sizes or a malformed host cu_seqlens */
  CFA_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head dim, dtype/pass combination) */
  CFA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned (workspace: 256) */
  CFA_ERR_WORKSPACE = 5,    /* workspace smaller than cfa_workspace_bytes() */
  CFA_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed */
} cfa_status;

/* Library version, (major << 16) | minor. */
int cfa_version(void);

/* Human-readable name of a status code. Static storage. */
const char* cfa_status_string(int status);

/* Detail of the last failure on the calling thread (thread-local, static storage). */
const char* cfa_last_error(void);

/* Scratch bytes needed by attn_fwd (pass 0) or attn_bwd (pass 1) for these sizes. Depends only
 * on the sizes (and, for the bf16 backward at d = 128, on CFA_DQ_MODE below), never on the values
 * of cu_seqlens. Returns 0 for invalid sizes.
 * CFA_DQ_MODE=fused in the environment: the bf16 backward at d = 128 sums dQ inside the dK/dV
 * pass, in key-tile order (deterministic), instead of a separate dQ pass that recomputes S and dP;
 * its workspace then also holds fp32 dQ sums [total_tokens, hq, d]. Measured slower on MI355X, so
 * it is off by default. */
size_t cfa_workspace_bytes(int pass, int total_tokens, int n_docs, int hq, int hkv, int d, int dtype);

/* Bytes of the forward-to-backward buffer `saved` (the MX dtypes only): the d-blocked E4M3, E2M1,
 * E2M3 or E3M2 copies of Q and K with their scales, reused by the backward so both passes see
 * identical scores (Q_d is written by the forward attention kernel from the Q rows it quantises
 * for itself), and the d-blocked E4M3 copy of V (the backward's dP operand), which the forward
 * writes in the same pass that reads V for its token-blocked copy -- quantised operands reused in
 * another orientation instead of being quantised again (FLAMIA page, "FLAMIA Mimarisi ve Temel
 * Tasarım İlkeleri": token-block scaling, fused quantisation). Layout, each section
 * starting at a 256-byte boundary: Q_d codes [T, hq, c], Q_d scales [T, hq, d/32], K_d codes
 * [T, hkv, c], K_d scales [T, hkv, d/32], V_d codes [T, hkv, d], V_d scales [T, hkv, d/32], with
 * c = d (E4M3), d/2 (E2M1) or 3d/4 (6-bit) bytes as mx_quantize and mx_quantize_fp4/fp6 store
 * them. 0 for the other dtypes and for invalid sizes. */
size_t cfa_saved_bytes(int total_tokens, int n_docs, int hq, int hkv, int d, int dtype);

/*
 * Forward pass. Writes o and lse.
 *   max_seqlen : upper bound on any document length (0 = unknown; then total_tokens is used).
 *   scale      : multiplier of Q K^T (usually 1/sqrt(d)); finite and > 0.
 *   dtype      : CFA_F32 (d = 64 or 128), CFA_BF16 (d = 64, 128 or 256; 256 is FlashAttention-2's
 *                extension, "FlashAttention (HU)", FlashAttention-2 (2023)), CFA_MXFP8 (d = 128).
 *                CFA_MXFP4 / CFA_MXFP6 / CFA_MXFP6_E3M2 (d = 128): as CFA_MXFP8 with an E2M1 / E2M3
 *                / E3M2 score product.
 *   saved      : the MX dtypes: cfa_saved_bytes() bytes written here for attn_bwd;
 *                otherwise NULL.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
             int n_docs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
             float scale, int causal, int dtype, void* saved,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass: dq, dk, dv (same layouts and element type as q, k, v) from q, k, v, the
 * forward's o and lse, and the upstream gradients dout (of O) and dlse (of LSE). dtype CFA_BF16,
 * CFA_MXFP8, CFA_MXFP4, CFA_MXFP6 or CFA_MXFP6_E3M2 (CFA_F32 is forward-only).
 *   dlse  : float32 [hq, total_tokens] like lse, or NULL for no gradient into lse. The pages do
 *           not name it; it is the exact derivative of the lse output the forward returns:
 *           d lse_i / d S_ij = P_ij, so it enters as dS_ij = P_ij (dP_ij - (D_i - dlse_i)) with
 *           D_i = sum_r dout_ir o_ir. Shares the 16-byte alignment rule.
 *   saved : the MX dtypes: the buffer attn_fwd filled, unmodified; otherwise NULL. An MX call
 *           may also pass NULL: the backward then quantises Q, K and V again (the same bytes
 *           the forward wrote, so the results are bit-identical) into the workspace, which must
 *           then hold cfa_workspace_bytes(1, ...) + cfa_saved_bytes(...) bytes.
 * Deterministic: two calls on the same inputs give bit-identical outputs.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, const float* dlse, const void* saved, void* dq, void* dk, void* dv,
             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
             int n_docs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
             float scale, int causal, int dtype,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * MX quantiser: bf16 x [total_tokens, h, d] -> E4M3 codes + E8M0 scales, one scale per block of
 * 32 elements. Rule per block: amax = max|x|; e = floor(log2 amax) - 8 clamped to [-127, 127]
 * (e = -127 for an all-zero block); scale byte e + 127; element = x * 2^-e saturated to +-448
 * and rounded to nearest E4M3 (ties to even, sign of zero kept); a block holding NaN or Inf gets
 * scale byte 0xFF and codes 0x7F.
 *   axis 0 : blocks of 32 channels along d.   codes [T, h, d], scales [T, h, d/32].
 *   axis 1 : blocks of 32 doc-local tokens.   codes [h, d, t_pad], scales [h, d, t_pad/32],
 *            document n starting at column P_n = sum_{m<n} 32*ceil(L_m/32); a document's last
 *            block holds only its own tokens; padding columns get code 0x00 and belong to no
 *            scale. t_pad is the row stride of both outputs: a multiple of 32 and at least
 *            mx_padded_tokens(total_tokens, n_docs) (columns past P_{n_docs} are left as is).
 *   axis 2 : the axis-1 blocks in the layout the attention kernels stage for themselves: codes
 *            [h, d, t_pad] with the 4-token pieces of each 32-token block stored in the order
 *            0,2,4,6,1,3,5,7 (bytes 16g..16g+15 of a block hold the tokens a matrix-core lane
 *            group g reads), scales block-major [h, t_pad/32, d].
 * d·t_pad must stay below 2^31 and h at most 65536 (axes 1, 2; CFA_ERR_UNSUPPORTED otherwise).
 * Token-block scaling of this kind, with blocks that never cross a document, is the FLAMIA
 * page's document-local scaling ("FLAMIA Mimarisi ve Temel Tasarım İlkeleri"); the element and
 * scale rules are the OCP MX definitions of E4M3 and E8M0 (the page names MXFP8 only).
 * workspace: at least mx_workspace_bytes(n_docs) bytes (axes 1, 2; may be NULL for axis 0).
 */
int mx_quantize(const void* x, int total_tokens, int h, int d,
                const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int n_docs, int axis,
                uint8_t* codes, uint8_t* scales, int t_pad,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cross-attention (bf16): packed query documents attend to their own packed key/value documents.
 * Document n owns query rows cu_seqlens_q[n] .. cu_seqlens_q[n+1]-1 of q, o, dout, dq (total_q
 * rows) and key rows cu_seqlens_k[n] .. cu_seqlens_k[n+1]-1 of k, v, dk, dv (total_k rows); both
 * arrays follow the cu_seqlens rules (device memory, optional host copies validated first).
 * causal != 0: with Lq, Lk the document's lengths, query i sees key j iff j <= i + (Lk - Lq) --
 * the queries are the last Lq positions of the Lk keys, which is the rule of "GPT Kernel
 * Programlama" §4 when Lq = Lk and decoding when Lq = 1. A query that sees no key (i < Lq - Lk,
 * or Lk = 0) gets o = 0, lse = -inf and no gradient. lse: [hq, total_q]; dlse as in attn_bwd.
 * d = 64, 128 or 256. The pages do not name cross-attention; the definitions are those of
 * attn_fwd / attn_bwd with the mask above.
 * Scratch: cfa_cross_workspace_bytes(pass 0 = forward, 1 = backward, ...). cfa_device_error on
 * this workspace reports cu_seqlens_q only (a malformed device cu_seqlens_k is clamped the same
 * way, its documents becoming empty).
 */
size_t cfa_cross_workspace_bytes(int pass, int total_q, int total_k, int n_docs, int hq, int hkv, int d);
int attn_fwd_cross(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
                   int n_docs, int total_q, int total_k, int hq, int hkv, int d, float scale, int causal,
                   void* workspace, size_t workspace_bytes, void* stream);
int attn_bwd_cross(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, const float* dlse, void* dq, void* dk, void* dv,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
                   int n_docs, int total_q, int total_k, int hq, int hkv, int d, float scale, int causal,
                   void* workspace, size_t workspace_bytes, void* stream);
/*
 * MXFP4 quantiser along d: bf16 x [total_tokens, h, d] -> E2M1 codes packed two per byte
 * (element 2i in the low nibble) [total_tokens, h, d/2] + E8M0 scales [total_tokens, h, d/32].
 * Per 32-channel block: e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for a zero block);
 * elements x * 2^-e saturated to +-6 and rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6
 * (ties to the even code; sign of zero kept); a NaN/Inf block gets scale 0xFF and codes 0. The
 * score operands of the CFA_MXFP4 attention path are these copies of Q and K.
 */
int mx_quantize_fp4(const void* x, int total_tokens, int h, int d, uint8_t* codes, uint8_t* scales, void* stream);
/*
 * MXFP6 quantiser along d (E2M3 elements: 1 sign, 2 exponent bits with bias 1, 3 mantissa bits;
 * magnitudes 0..1.875 in steps of 1/8, 2..3.75 in 1/4, 4..7.5 in 1/2): bf16 x [total_tokens, h,
 * d] -> codes [total_tokens, h, 3d/4] bytes + E8M0 scales [total_tokens, h, d/32]. Per 32-channel
 * block b: e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for a zero block); elements
 * x * 2^-e saturated to +-7.5 and rounded to the nearest E2M3 value (ties to the even code; sign of
 * zero kept); a NaN/Inf block gets scale 0xFF and codes 0. Block b is the 192-bit little-endian
 * number with code i in bits 6i..6i+5; its bytes 0-15 are stored at [16b, 16b+16) of the row and
 * its bytes 16-23 at [d/2 + 8b, d/2 + 8b + 8) -- the two parts of the matrix-core operand of
 * v_mfma_scale_f32_32x32x64_f8f6f4 with format code 2. x and codes: 16-byte aligned. The score
 * operands of the CFA_MXFP6 attention path are these copies of Q and K.
 */
int mx_quantize_fp6(const void* x, int total_tokens, int h, int d, uint8_t* codes, uint8_t* scales, void* stream);
/*
 * The same quantiser and storage with E3M2 elements (1 sign, 3 exponent bits with bias 3, 2
 * mantissa bits; magnitudes 0..0.4375 in steps of 1/16, then four per binade [2^k, 2^(k+1)) up
 * to 16, 20, 24, 28): e = floor(log2 amax) - 4, elements saturated to +-28 and rounded to the
 * nearest E3M2 value (ties to the even code). Matrix-core format code 3. The score operands of
 * the CFA_MXFP6_E3M2 attention path are these copies of Q and K.
 */
int mx_quantize_fp6_e3m2(const void* x, int total_tokens, int h, int d, uint8_t* codes, uint8_t* scales,
                         void* stream);
/* Upper bound of P_{n_docs} for any cu_seqlens with these sizes, rounded up to 32:
 * 32*ceil(total_tokens/32) + 32*n_docs. */
int mx_padded_tokens(int total_tokens, int n_docs);

/* Scratch bytes of mx_quantize along tokens. */
size_t mx_workspace_bytes(int n_docs);

/* Output sizes of mx_quantize: returns the bytes of `codes` and, when scale_bytes is not NULL,
 * stores the bytes of `scales` there (one E8M0 byte per 32 codes). Axis 0: h·d·total_tokens
 * codes; axes 1, 2: h·d·t_pad codes with t_pad = mx_padded_tokens(total_tokens, n_docs), the
 * smallest row stride that holds any cu_seqlens of these sizes. 0 (and 0 scale bytes) for an
 * invalid axis or sizes (n_docs < 1, h < 1, d other than 64 or 128, as mx_quantize). */
size_t mx_quantize_bytes(int axis, int total_tokens, int n_docs, int h, int d, size_t* scale_bytes);

/*
 * Decoding: one new query token per sequence over a packed KV cache (the current token's K/V
 * already appended), the last row of a causal document -- "GPT Kernel Programlama" §4-§6 -- read
 * through flash attention from a quantised cache as local inference engines do ("Flash
 * Attention", ai.ozdemir.be, sections "Tanım" and "Gerçek dünyadan örnek", which name an 8-bit
 * cache type at about half the memory of f16; here: the MX format below, 8.25 bits per element).
 *   q, o        : [n_seqs, hq, d] bf16; lse: [hq, n_seqs] float32 (natural log).
 *   k_cache,
 *   v_cache     : [total_k, hkv, d]; kv_dtype CFA_BF16: bf16 values; CFA_MXFP8: E4M3 codes with
 *                 k_scales / v_scales [total_k, hkv, d/32] E8M0 bytes (mx_quantize axis 0);
 *                 element value = code * 2^(scale - 127). Scales are NULL for CFA_BF16.
 *   cu_seqlens_k: int32 [n_seqs + 1] in device memory (same rules as cu_seqlens); sequence b
 *                 owns cache rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 and its query sees all
 *                 of them. A sequence with no rows gets o = 0 and lse = -inf.
 *   d           : 64 or 128. Query head h reads kv head h / (hq / hkv).
 * Work is split over 1024-key chunks; the chunk partials are merged in chunk order, so results
 * are deterministic. Scratch: cfa_decode_workspace_bytes() bytes (256-byte aligned); no other
 * allocation. Errors as for the other calls.
 */
size_t cfa_decode_workspace_bytes(int n_seqs, int total_k, int hq, int hkv, int d, int kv_dtype);
int attn_decode(const void* q, const void* k_cache, const void* v_cache, const uint8_t* k_scales,
                const uint8_t* v_scales, void* o, float* lse, const int32_t* cu_seqlens_k,
                const int32_t* cu_seqlens_k_host, int n_seqs, int total_k, int hq, int hkv, int d,
                float scale, int kv_dtype, void* workspace, size_t workspace_bytes, void* stream);
/*
 * Per-kernel timing for measurement tools. While set on the calling thread, the attention
 * calls record events[2*i] on their stream just before launching their i-th main kernel and
 * events[2*i+1] just after it (the work-list kernel is not counted). Kernel order:
 *   attn_fwd: 0 = forward attention (MX dtypes: it also quantises Q), 1 = (MX dtypes) the one pass
 *             that quantises K and V;
 *   attn_bwd: 0 = D = rowsum(dO*O) (MX dtypes: the one pass that also writes both dO copies),
 *             1 = dK/dV, 2 = dQ;
 *   attn_decode: 0 = chunk partials, 1 = their merge.
 * Entries may be NULL (not recorded). The caller owns the hipEvent_t handles and keeps the
 * array alive while it is set; n_pairs = 0 (events NULL) switches recording off.
 */
int cfa_set_kernel_events(void* const* events, int n_pairs);

/*
 * Reads the device-side validation flag left in `workspace` by the last attn_fwd / attn_bwd /
 * mx_quantize call that used it. Synchronises `stream`. *flag = 0: cu_seqlens was well formed;
 * otherwise bit 0 = cu[0] != 0, bit 1 = a decreasing entry, bit 2 = cu[n_docs] != total_tokens.
 */
int cfa_device_error(const void* workspace, void* stream, int* flag);

/*
 * attn_bwd for callers that cannot allocate device memory (code under stream capture, serving
 * loops, harnesses that forbid hipMalloc): the same computation, outputs and errors as attn_bwd,
 * with the scratch taken from a fixed array inside the library instead of a caller workspace.
 * Each GPU the library runs on holds one such array of 64 MiB (67108864 bytes) until the
 * process ends; its address is looked up once per device on the first call
 * with that device current (no allocation). Where attn_bwd's workspace for these sizes fits in
 * the array the results are attn_bwd's bit for bit; under CFA_DQ_MODE=fused a bf16 call at
 * d = 128 whose fp32 dQ sums do not fit runs dQ as a separate pass instead (results within
 * rounding of attn_bwd's); sizes that do not fit either way are rejected with CFA_ERR_WORKSPACE
 * before any launch. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller. Nothing in the array needs to start at zero (every
 * call clears or writes what it reads). The validation flag of a device-only cu_seqlens is kept
 * in the array and is not readable through cfa_device_error.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, const float* dlse, const void* saved, void* dq, void* dk, void* dv,
                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                     int n_docs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
                     float scale, int causal, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CFA_H */

// Work-list ("plan") builder: one workgroup turns cu_seqlens into the longest-first schedule.
//
// Documents are independent and a document's tiles cost up to its length, so long documents
// go first (workload-aware scheduling over packed documents: FLAMIA page, "FLAMIA Mimarisi ve
// Temel Tasarım İlkeleri"). Documents are bucketed by ceil(L/128) (capped), bucket order is
// descending; the order inside a bucket is whatever the atomics give: it only decides *which*
// workgroup computes a tile, never how, so results stay bit-identical between runs.
#include "cfa_device.h"

namespace cfa {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 4096;

__device__ inline void block_exclusive_scan_desc(int* a, int n, int* tmp) {
  // exclusive scan of a[0..n) in DESCENDING index order: a[i] <- sum_{j>i} a[j]; n <= 4096
  const int tid = threadIdx.x;
  constexpr int PER = PLAN_BUCKETS / PLAN_THREADS;  // 4
  int loc[PER];
  int s = 0;
  for (int e = PER - 1; e >= 0; --e) {
    int i = tid * PER + e;
    int v = (i < n) ? a[i] : 0;
    loc[e] = s;
    s += v;
  }
  tmp[tid] = s;
  __syncthreads();
  // suffix sums over threads (Hillis-Steele)
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    int v = (tid + off < PLAN_THREADS) ? tmp[tid + off] : 0;
    __syncthreads();
    tmp[tid] += v;
    __syncthreads();
  }
  int after = (tid + 1 < PLAN_THREADS) ? tmp[tid + 1] : 0;
  __syncthreads();
  for (int e = 0; e < PER; ++e) {
    int i = tid * PER + e;
    if (i < n) a[i] = loc[e] + after;
  }
  __syncthreads();
}

// Exclusive prefix (ascending) of values produced by f(i) for i in [0, n), written to out[0..n]
// (out[n] = total). Chunks of PLAN_THREADS; `carry` and `tmp` are LDS scratch.
template <typename F>
__device__ inline void block_prefix(int n, F f, int* out, int* tmp) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < n; base += PLAN_THREADS) {
    int i = base + tid;
    int v = (i < n) ? f(i) : 0;
    tmp[tid] = v;
    __syncthreads();
    for (int off = 1; off < PLAN_THREADS; off <<= 1) {
      int u = (tid >= off) ? tmp[tid - off] : 0;
      __syncthreads();
      tmp[tid] += u;
      __syncthreads();
    }
    if (i < n) out[i] = carry + tmp[tid] - v;
    int chunk_total = tmp[PLAN_THREADS - 1];
    __syncthreads();
    carry += chunk_total;
  }
  if (tid == 0) out[n] = carry;
  __syncthreads();
}

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const int* __restrict__ cu, int n_docs, int total_tokens,
                                                            char* __restrict__ ws) {
  __shared__ int hist[PLAN_BUCKETS];
  __shared__ int tmp[PLAN_THREADS];
  __shared__ int sflag;
  const PlanLayout lay(n_docs);
  int* header = (int*)(ws + lay.header);
  int2* docinfo = (int2*)(ws + lay.docinfo);
  int* order = (int*)(ws + lay.order);
  int* pref = (int*)(ws + lay.pref);
  int* padoff = (int*)(ws + lay.padoff);
  const int tid = threadIdx.x;
  for (int i = tid; i < PLAN_BUCKETS; i += PLAN_THREADS) hist[i] = 0;
  if (tid == 0) sflag = 0;
  __syncthreads();
  // 1. validate and clamp documents; histogram of length buckets
  int flag = 0;
  for (int n = tid; n < n_docs; n += PLAN_THREADS) {
    int a = cu[n], b = cu[n + 1];
    if (n == 0 && a != 0) flag |= 1;
    if (b < a) flag |= 2;
    if (n == n_docs - 1 && b != total_tokens) flag |= 4;
    int s0 = min(max(a, 0), total_tokens);
    int s1 = min(max(b, 0), total_tokens);
    int L = max(s1 - s0, 0);
    docinfo[n] = make_int2(s0, L);
    int key = min((L + 127) / 128, PLAN_BUCKETS - 1);
    atomicAdd(&hist[key], 1);
  }
  if (flag) atomicOr(&sflag, flag);
  __syncthreads();
  // 2. bucket start positions, longest bucket first
  block_exclusive_scan_desc(hist, PLAN_BUCKETS, tmp);
  // 3. place documents
  for (int n = tid; n < n_docs; n += PLAN_THREADS) {
    int L = docinfo[n].y;
    int key = min((L + 127) / 128, PLAN_BUCKETS - 1);
    int pos = atomicAdd(&hist[key], 1);
    order[pos] = n;
  }
  __threadfence_block();
  __syncthreads();
  // 4. item prefixes for tile heights 32, 64, 128, 256 over the sorted order
  for (int s = 0; s < 4; ++s) {
    const int rows = 32 << s;
    block_prefix(n_docs, [&](int i) { int L = docinfo[order[i]].y; return (L + rows - 1) / rows; },
                 pref + s * (n_docs + 1), tmp);
  }
  // 5. MX token-block column offsets, document order
  block_prefix(n_docs, [&](int i) { int L = docinfo[i].y; return (L + 31) / 32 * 32; }, padoff, tmp);
  if (tid == 0) header[0] = sflag;
}

hipError_t launch_plan(const int* cu, int n_docs, int total_tokens, void* ws, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, cu, n_docs, total_tokens, (char*)ws);
  return hipGetLastError();
}

}  // namespace cfa

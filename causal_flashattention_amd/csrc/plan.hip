// Work-list ("plan") builder: one workgroup turns cu_seqlens into the longest-first schedule.
//
// Documents are independent and a document's tiles cost up to its length, so long documents
// go first (workload-aware scheduling over packed documents: FLAMIA page, "FLAMIA Mimarisi ve
// Temel Tasarım İlkeleri"). Documents are bucketed by ceil(L/128) (capped); buckets run in
// descending order and documents of one bucket in ascending index order (a stable counting
// sort), so the schedule itself is a function of cu_seqlens alone. The order only decides
// *which* workgroup computes a tile, never how, so results are bit-identical under any order.
// `naive` (a diagnostic) keeps the documents in index order instead.
//
// A device-only cu_seqlens is validated here: any malformed entry (cu[0] != 0, a decrease,
// cu[n] != total) raises a flag bit and makes every document empty, so no kernel of the pass
// reads or writes a token row (overlapping documents could otherwise write one row from
// several workgroups, and their padded MX offsets could run past the workspace).
#include "cfa_device.h"

namespace cfa {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 4096;

// Inclusive sum over the lanes of a wave up to this lane (lane shuffles, no barrier).
__device__ inline int wave_incl_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Exclusive sum of one value per thread over the threads of the block in thread order, and the
// block total. `wt` is LDS scratch of PLAN_THREADS / 64 ints. Two barriers (the second lets the
// next call reuse `wt`).
__device__ inline int block_excl_sum(int v, int* wt, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) wt[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < PLAN_THREADS / 64; ++w) {
    const int x = wt[w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// block_excl_sum for N values per thread at once (one exchange of wave totals for all N).
// `wt` holds N · PLAN_THREADS / 64 ints.
template <int N>
__device__ inline void block_excl_sum_n(const int (&v)[N], int (&ex)[N], int (&total)[N], int* wt) {
  constexpr int NW = PLAN_THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int c = 0; c < N; ++c) {
    incl[c] = wave_incl_sum(v[c]);
    if (lane == 63) wt[c * NW + wave] = incl[c];
  }
  __syncthreads();
  int before[N], all[N];
#pragma unroll
  for (int c = 0; c < N; ++c) before[c] = all[c] = 0;
#pragma unroll 1
  for (int w = 0; w < NW; ++w) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const int x = wt[c * NW + w];
      before[c] += w < wave ? x : 0;
      all[c] += x;
    }
  }
#pragma unroll
  for (int c = 0; c < N; ++c) {
    ex[c] = before[c] + incl[c] - v[c];
    total[c] = all[c];
  }
  __syncthreads();
}

__device__ inline void block_exclusive_scan_desc(int* a, int n, int* tmp) {
  // exclusive scan of a[0..n) in DESCENDING index order: a[i] <- sum_{j>i} a[j]; n <= 4096.
  // Thread t holds the PER buckets from (PLAN_THREADS - 1 - t)·PER up, so the threads before it
  // hold exactly the higher buckets.
  constexpr int PER = PLAN_BUCKETS / PLAN_THREADS;  // 4
  const int r = PLAN_THREADS - 1 - (int)threadIdx.x;
  int loc[PER];
  int s = 0;
  for (int e = PER - 1; e >= 0; --e) {
    const int i = r * PER + e;
    const int v = (i < n) ? a[i] : 0;
    loc[e] = s;
    s += v;
  }
  int total;
  const int after = block_excl_sum(s, tmp, total);
  for (int e = 0; e < PER; ++e) {
    const int i = r * PER + e;
    if (i < n) a[i] = loc[e] + after;
  }
  __syncthreads();
}

__device__ inline int length_bucket(int L) { return min((L + 127) / 128, PLAN_BUCKETS - 1); }

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const int* __restrict__ cu, int n_docs, int total_tokens,
                                                            int naive, char* __restrict__ ws) {
  __shared__ int hist[PLAN_BUCKETS];
  __shared__ int tmp[PLAN_THREADS];
  __shared__ int sflag;
  const PlanLayout lay(n_docs);
  int* header = (int*)(ws + lay.header);
  int2* docinfo = (int2*)(ws + lay.docinfo);
  int* order = (int*)(ws + lay.order);
  int* pref = (int*)(ws + lay.pref);
  int* padoff = (int*)(ws + lay.padoff);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < PLAN_BUCKETS; i += PLAN_THREADS) hist[i] = 0;
  if (tid == 0) sflag = 0;
  if (tid > 0 && tid < 64) header[tid] = 0;       // chain counter and claim words of the fused backward
  __syncthreads();
  // 1. validate; clamp each document into [0, total]
  int flag = 0;
  for (int n = tid; n < n_docs; n += PLAN_THREADS) {
    int a = cu[n], b = cu[n + 1];
    if (n == 0 && a != 0) flag |= 1;
    if (b < a) flag |= 2;
    if (n == n_docs - 1 && b != total_tokens) flag |= 4;
    int s0 = min(max(a, 0), total_tokens);
    int s1 = min(max(b, 0), total_tokens);
    docinfo[n] = make_int2(s0, max(s1 - s0, 0));
  }
  if (flag) atomicOr(&sflag, flag);
  __syncthreads();
  // 2. a malformed cu_seqlens empties every document; histogram of length buckets
  const bool bad = sflag != 0;
  for (int n = tid; n < n_docs; n += PLAN_THREADS) {
    int2 di = docinfo[n];
    if (bad) docinfo[n] = make_int2(di.x, 0);
    atomicAdd(&hist[length_bucket(bad ? 0 : di.y)], 1);
  }
  __syncthreads();
  // 3. bucket start positions, longest bucket first
  block_exclusive_scan_desc(hist, PLAN_BUCKETS, tmp);
  // 4. place documents: bucket start + the number of lower-indexed documents of the same bucket
  //    (chunks of PLAN_THREADS in index order; rank within a wave by lane exchange, then the
  //    waves of a chunk in turn)
  for (int base = 0; base < n_docs; base += PLAN_THREADS) {
    const int n = base + tid;
    const bool ok = n < n_docs;
    const int key = ok ? length_bucket(docinfo[n].y) : -1;
    int rank = 0;
    for (int j = 0; j < 64; ++j) {
      const int other = __shfl(key, j, 64);
      rank += (j < lane && other == key) ? 1 : 0;
    }
    const int n_waves = min(PLAN_THREADS, n_docs - base + 63) / 64;   // waves holding documents
    for (int w = 0; w < n_waves; ++w) {
      if (wave == w && ok) order[naive ? n : hist[key] + rank] = n;
      __syncthreads();
      if (wave == w && ok) atomicAdd(&hist[key], 1);
      __syncthreads();
    }
  }
  __threadfence_block();
  __syncthreads();
  // 5. item prefixes for tile heights 32, 64, ..., 1024 over the sorted order, and 6. the MX
  // token-block column offsets in document order: one pass (each document's lengths are read
  // once; the seven scans share it)
  constexpr int NS = 6;
  int carry[NS + 1];
#pragma unroll
  for (int c = 0; c <= NS; ++c) carry[c] = 0;
  for (int base = 0; base < n_docs; base += PLAN_THREADS) {
    const int i = base + tid;
    const bool ok = i < n_docs;
    const int Ls = ok ? docinfo[order[i]].y : 0;     // sorted order
    const int Li = ok ? docinfo[i].y : 0;            // document order
    int v[NS + 1], ex[NS + 1], total[NS + 1];
#pragma unroll
    for (int c = 0; c < NS; ++c) v[c] = (Ls + (32 << c) - 1) / (32 << c);
    v[NS] = (Li + 31) / 32 * 32;
    block_excl_sum_n<NS + 1>(v, ex, total, tmp);
#pragma unroll
    for (int c = 0; c <= NS; ++c) {
      if (ok) (c < NS ? pref + c * (n_docs + 1) : padoff)[i] = carry[c] + ex[c];
      carry[c] += total[c];
    }
  }
  if (tid == 0) {
    for (int c = 0; c < NS; ++c) pref[c * (n_docs + 1) + n_docs] = carry[c];
    padoff[n_docs] = carry[NS];
  }
  if (tid == 0) header[0] = sflag;
}

hipError_t launch_plan(const int* cu, int n_docs, int total_tokens, void* ws, hipStream_t stream, bool naive) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, cu, n_docs, total_tokens, naive ? 1 : 0,
                     (char*)ws);
  return hipGetLastError();
}

}  // namespace cfa

// Token permutation by expert: a stable counting sort of the (token, slot)
// pairs by expert id, plus the tile lists of the grouped expert GEMMs.
//
// The grouping is what a grouped matmul over experts needs (sglang-jax issue
// "[Feature] Support Step 3.5 Flash (StepFun) Model", "Implementation
// strategy": grouped matmul first, checked against a per-expert loop).
//
// Three kernels, none with floating-point work and none order-dependent:
//  rank     one wave per chunk of pairs: per-expert counts of the chunk and
//           each pair's rank among the chunk's pairs of the same expert
//           (wave ballots over the expert-id bits; pairs in ascending id).
//  scan     one block: per-expert exclusive prefix over chunks, expert
//           offsets (exclusive prefix over experts) and the GEMM tile list.
//  scatter  position = offset[e] + chunk base[e] + rank.

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// hist is [E][C]: hist[e * C + c] = pairs of expert e in chunk c.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                  int chunk, int C, int32_t* __restrict__ rank,
                                                  int32_t* __restrict__ hist) {
  __shared__ int32_t cnt[kMaxExperts];
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int q0 = c * chunk;
  const int q1 = min(P, q0 + chunk);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int q = q0; q < q1; q += 64) {
    const int p = q + lane;
    const int e_in = p < q1 ? ids[p] : -1;
    const bool valid = e_in >= 0 && e_in < E;  // out-of-range ids are not counted
    const int e = valid ? e_in : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      peers &= bit ? ones : ~ones;
    }
    int base = 0;
    if (valid) base = cnt[e];
    __syncthreads();
    if (valid) {
      rank[p] = base + __popcll(peers & below);
      const int leader = __ffsll(static_cast<unsigned long long>(peers)) - 1;
      if (lane == leader) cnt[e] = base + __popcll(peers);
    }
    __syncthreads();
  }
  for (int e = lane; e < E; e += 64) hist[static_cast<int64_t>(e) * C + c] = cnt[e];
}

// Exclusive prefix sum over the 1024 threads of a block; returns the total
// in *total.
__device__ int block_excl_scan(int v, int* smem, int* total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) smem[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int wv = lane < 16 ? smem[lane] : 0;
    int wincl = wv;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(wincl, off);
      if (lane >= off) wincl += o;
    }
    if (lane < 16) smem[16 + lane] = wincl - wv;
    if (lane == 15) smem[32] = wincl;
  }
  __syncthreads();
  const int r = smem[16 + wid] + incl - v;
  *total = smem[32];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ hist, int C, int E,
                                                    int P, int64_t T, int bm, int with_shared,
                                                    int32_t* __restrict__ base,
                                                    int32_t* __restrict__ offsets,
                                                    int2* __restrict__ tiles,
                                                    int32_t* __restrict__ ntiles) {
  __shared__ int32_t count[kMaxExperts];
  __shared__ int smem[40];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  // Per-expert prefix over chunks (16 waves, one expert at a time each).
  for (int e = wid; e < E; e += 16) {
    int run = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < C ? hist[static_cast<int64_t>(e) * C + c] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (c < C) base[static_cast<int64_t>(e) * C + c] = run + incl - v;
      run += __shfl(incl, 63);
    }
    if (lane == 0) count[e] = run;
  }
  __syncthreads();
  // Expert offsets.
  const int ce = tid < E ? count[tid] : 0;
  int tot = 0;
  const int off = block_excl_scan(ce, smem, &tot);
  if (tid < E) offsets[tid] = off;
  if (tid == 0) offsets[E] = tot;
  // Tile list: routed tiles expert by expert, then the shared expert's.
  const int nt = tid < E ? (ce + bm - 1) / bm : 0;
  int ntot = 0;
  const int tstart = block_excl_scan(nt, smem, &ntot);
  for (int i = 0; i < nt; ++i) tiles[tstart + i] = make_int2(tid, off + i * bm);
  const int nshared = with_shared ? static_cast<int>((T + bm - 1) / bm) : 0;
  for (int i = tid; i < nshared; i += 1024) tiles[ntot + i] = make_int2(E, i * bm);
  if (tid == 0) *ntiles = ntot + nshared;
  (void)P;
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ offsets, int P,
                                                      int E, int C, int chunk,
                                                      int32_t* __restrict__ sorted,
                                                      int32_t* __restrict__ pos) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  const int e = ids[p];
  if (e < 0 || e >= E) return;  // not counted by the rank kernel
  const int c = p / chunk;
  const int i = offsets[e] + base[static_cast<int64_t>(e) * C + c] + rank[p];
  sorted[i] = p;
  pos[p] = i;
}

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_fill_zero(int32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  fill_zero_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int64_t T, int bm, int with_shared,
                          int32_t* rank, int32_t* hist, int32_t* base, int32_t* offsets,
                          int32_t* sorted, int32_t* pos, int2* tiles, int32_t* ntiles,
                          hipStream_t stream, hipEvent_t* ev) {
  const int C = (P + kPermuteChunk - 1) / kPermuteChunk;
  if (ev) hipEventRecord(ev[0], stream);
  rank_kernel<<<C, 64, 0, stream>>>(ids, P, E, kPermuteChunk, C, rank, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev) hipEventRecord(ev[1], stream);
  scan_kernel<<<1, 1024, 0, stream>>>(hist, C, E, P, T, bm, with_shared, base, offsets, tiles,
                                      ntiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev) hipEventRecord(ev[2], stream);
  scatter_kernel<<<(P + 255) / 256, 256, 0, stream>>>(ids, rank, base, offsets, P, E, C,
                                                      kPermuteChunk, sorted, pos);
  return hipGetLastError();
}

}  // namespace moe

// Token permutation by expert: a stable counting sort of the (token, slot)
// pairs by expert id, plus the tile list of the grouped expert GEMMs.
//
// The grouping is what a grouped matmul over experts needs (sglang-jax issue
// "[Feature] Support Step 3.5 Flash (StepFun) Model", "Implementation
// strategy": grouped matmul first, checked against a per-expert loop).
//
// The pairs are cut into spans.  Inside a span, one wave walks the pairs
// in ascending id, 64 at a time: lanes holding the same expert find each
// other by ballots over the bits of the expert id, so each pair gets its
// rank among the chunk's earlier pairs of its expert and the chunk gets
// per-expert counts.  An exclusive prefix over chunks (per expert) and over
// experts then places every pair: position = offset[e] + base[e][c] + rank.
// Nothing here depends on timing, so the permutation is deterministic.
//
// Chunks are ranked by whole blocks: each of 16 waves ranks a span of the
// chunk and one thread per expert prefixes the waves' counts.  Small batches
// (<= 4096 pairs) run all of it in one block; larger ones use three kernels
// (rank, scan, scatter).

#include "common.h"
#include "kernels.h"
#include "permute_ops.h"

namespace moe {

namespace {

constexpr int kSmallPairs = 4096;

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
    const int wv = lane < 16 ? smem[lane] : 0;
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

// Offsets from per-expert counts (one per thread, experts 0..E-1), then the
// tile list: routed tiles expert by expert, then the shared expert's.
// queue (may be null): the big-tile GEMMs' work-queue counters, zeroed here.
__device__ void offsets_and_tiles(int count, int E, int64_t T, int bm, int with_shared,
                                  int* smem, int32_t* offsets, int32_t* offs_lds,
                                  int2* tiles, int32_t* ntiles, uint32_t* queue) {
  const int tid = threadIdx.x;
  int tot = 0;
  const int off = block_excl_scan(tid < E ? count : 0, smem, &tot);
  if (tid < E) {
    offsets[tid] = off;
    if (offs_lds) offs_lds[tid] = off;
  }
  if (tid == 0) offsets[E] = tot;
  const int nt = tid < E ? (count + bm - 1) / bm : 0;
  int ntot = 0;
  const int tstart = block_excl_scan(nt, smem, &ntot);
  for (int i = 0; i < nt; ++i) tiles[tstart + i] = make_int2(tid, off + i * bm);
  const int nshared = with_shared ? static_cast<int>((T + bm - 1) / bm) : 0;
  for (int i = tid; i < nshared; i += 1024) tiles[ntot + i] = make_int2(E, i * bm);
  if (tid == 0) *ntiles = ntot + nshared;
  if (queue && tid < kQueueWords) queue[tid] = 0u;
}

// Ranks of the n <= kSmallPairs pairs staged in sid[0..n) among the earlier
// pairs of the same expert: each of the 16 waves ranks a contiguous span,
// then one thread per expert prefixes the waves' counts.  run[e] enters as
// the count of pairs ranked before this span and leaves advanced; srank[q]
// receives the rank.  wcnt must be zero on entry and is left zero.
__device__ void block_rank(const int32_t* sid, int n, int E, int nbits,
                           int32_t (*wcnt)[kMaxExperts], int32_t* run, int32_t* srank) {
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int CH = ((n + 15) / 16 + 63) / 64 * 64;  // pairs per wave
  const int q0 = min(n, wid * CH), q1 = min(n, q0 + CH);
  rank_span(sid + q0, q0, q1, E, nbits, wcnt[wid], srank, 0);
  __syncthreads();
  if (tid < E) {
    int c = run[tid];
    for (int w = 0; w < 16; ++w) {
      const int t = wcnt[w][tid];
      wcnt[w][tid] = c;
      c += t;
    }
    run[tid] = c;
  }
  __syncthreads();
  for (int q = tid; q < n; q += 1024) {
    const int e = sid[q];
    if (e >= 0 && e < E) srank[q] += wcnt[q / CH][e];
  }
  __syncthreads();
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
  __syncthreads();
}

// ---------------------------------------------------------------- small

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ ids, int P, int E, int64_t T, int bm, int with_shared,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ pos,
    int2* __restrict__ tiles, int32_t* __restrict__ ntiles, uint32_t* __restrict__ queue,
    const float* __restrict__ topk_w, float* __restrict__ w_sorted) {
  __shared__ int32_t sid[kSmallPairs];
  __shared__ int32_t srank[kSmallPairs];
  __shared__ int32_t wcnt[16][kMaxExperts];
  __shared__ int32_t run[kMaxExperts];
  __shared__ int smem[40];
  constexpr int PER = kSmallPairs / 1024;  // pairs per thread
  const int tid = threadIdx.x;
  // The gating weights are requested with the ids, so the scatter at the
  // end does not wait for a second round trip.
  float wv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p = tid + 1024 * j;
    if (p < P) {
      sid[p] = ids[p];
      wv[j] = w_sorted ? topk_w[p] : 0.f;
    }
  }
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
  for (int e = tid; e < E; e += 1024) run[e] = 0;
  __syncthreads();
  block_rank(sid, P, E, id_bits(E), wcnt, run, srank);
  const int count = tid < E ? run[tid] : 0;
  offsets_and_tiles(count, E, T, bm, with_shared, smem, offsets, run, tiles, ntiles, queue);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p = tid + 1024 * j;
    if (p >= P) continue;
    const int e = sid[p];
    if (e < 0 || e >= E) continue;
    const int i = run[e] + srank[p];
    sorted[i] = p;
    pos[p] = i;
    if (w_sorted) w_sorted[i] = wv[j];
  }
}

// ---------------------------------------------------------------- large

// One block per chunk of pairs: ranks within the chunk and the chunk's
// per-expert counts.  hist is [E][Cp]: hist[e * Cp + c] = pairs of expert e
// in chunk c (rows padded to Cp, a multiple of 4, for 16-byte loads).
__global__ __launch_bounds__(1024) void rank_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                    int chunk, int Cp, int32_t* __restrict__ rank,
                                                    int32_t* __restrict__ hist) {
  __shared__ int32_t sid[kSmallPairs];
  __shared__ int32_t srank[kSmallPairs];
  __shared__ int32_t wcnt[16][kMaxExperts];
  __shared__ int32_t run[kMaxExperts];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
  for (int e = tid; e < E; e += 1024) run[e] = 0;
  const int nbits = id_bits(E);
  const int q_end = min(P, (c + 1) * chunk);
  for (int q0 = c * chunk; q0 < q_end; q0 += kSmallPairs) {
    const int n = min(q_end - q0, kSmallPairs);
    int v[kSmallPairs / 1024];
#pragma unroll
    for (int i = 0; i < kSmallPairs / 1024; ++i) {
      const int q = tid + 1024 * i;
      v[i] = q < n ? ids[q0 + q] : -1;
    }
#pragma unroll
    for (int i = 0; i < kSmallPairs / 1024; ++i) sid[tid + 1024 * i] = v[i];
    __syncthreads();
    block_rank(sid, n, E, nbits, wcnt, run, srank);
    for (int q = tid; q < n; q += 1024) rank[q0 + q] = srank[q];
    __syncthreads();
  }
  for (int e = tid; e < E; e += 1024) hist[static_cast<int64_t>(e) * Cp + c] = run[e];
}

// One block, one thread per expert: the expert's chunk counts (C <= 64,
// row stride Cp) come in with 16-byte loads, all in flight together, and
// are prefixed in registers.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ hist, int C, int Cp,
                                                    int E, int64_t T, int bm, int with_shared,
                                                    int32_t* __restrict__ base,
                                                    int32_t* __restrict__ offsets,
                                                    int2* __restrict__ tiles,
                                                    int32_t* __restrict__ ntiles,
                                                    uint32_t* __restrict__ queue) {
  __shared__ int smem[40];
  const int e = threadIdx.x;
  int count = 0;
  if (e < E) {
    const int4* src = reinterpret_cast<const int4*>(hist + static_cast<int64_t>(e) * Cp);
    int4* dst = reinterpret_cast<int4*>(base + static_cast<int64_t>(e) * Cp);
    int4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (4 * i < C) {
        int4 t = src[i];  // padding columns past C are not written by the rank kernel
        if (4 * i + 1 >= C) t.y = 0;
        if (4 * i + 2 >= C) t.z = 0;
        if (4 * i + 3 >= C) t.w = 0;
        v[i] = t;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (4 * i < C) {
        int4 o;
        o.x = count; count += v[i].x;
        o.y = count; count += v[i].y;
        o.z = count; count += v[i].z;
        o.w = count; count += v[i].w;
        dst[i] = o;
      }
    }
  }
  offsets_and_tiles(count, E, T, bm, with_shared, smem, offsets, nullptr, tiles, ntiles, queue);
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ offsets, int P,
                                                      int E, int Cp, int chunk,
                                                      int32_t* __restrict__ sorted,
                                                      int32_t* __restrict__ pos,
                                                      const float* __restrict__ topk_w,
                                                      float* __restrict__ w_sorted) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  const int e = ids[p];
  if (e < 0 || e >= E) return;  // not counted by the rank kernel
  const int c = p / chunk;
  const int i = offsets[e] + base[static_cast<int64_t>(e) * Cp + c] + rank[p];
  sorted[i] = p;
  pos[p] = i;
  if (w_sorted) w_sorted[i] = topk_w[p];
}

// Tile list of a single group of T rows (the dense FFN): (group, first row).
__global__ void dense_tiles_kernel(int2* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                   uint32_t* __restrict__ queue, int n, int bm, int group) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) tiles[i] = make_int2(group, i * bm);
  if (i == 0) *ntiles = n;
  if (queue && i < kQueueWords) queue[i] = 0u;
}

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int permute_hist_stride(int P) {
  const int chunk = permute_chunk(P);
  const int C = (P + chunk - 1) / chunk;
  return (C + 3) / 4 * 4;
}

int permute_chunk(int P) {
  // At most 64 chunks, each a multiple of the LDS staging size.
  const int per = (P + 63) / 64;
  return std::max(kSmallPairs, (per + kSmallPairs - 1) / kSmallPairs * kSmallPairs);
}

hipError_t launch_dense_tiles(int2* tiles, int32_t* ntiles, uint32_t* queue, int64_t T, int bm,
                              int group, hipStream_t stream) {
  const int n = static_cast<int>((T + bm - 1) / bm);
  const int threads = std::max(n, kQueueWords);
  dense_tiles_kernel<<<(threads + 255) / 256, 256, 0, stream>>>(tiles, ntiles, queue, n, bm,
                                                                group);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  fill_zero_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int64_t T, int bm, int with_shared,
                          int32_t* rank, int32_t* hist, int32_t* base, int32_t* offsets,
                          int32_t* sorted, int32_t* pos, int2* tiles, int32_t* ntiles,
                          uint32_t* queue, const float* topk_w, float* w_sorted,
                          hipStream_t stream, hipEvent_t* ev) {
  if (P <= kSmallPairs) {
    if (ev) hipEventRecord(ev[0], stream);
    permute_small_kernel<<<1, 1024, 0, stream>>>(ids, P, E, T, bm, with_shared, offsets, sorted,
                                                 pos, tiles, ntiles, queue, topk_w, w_sorted);
    if (ev) {
      hipEventRecord(ev[1], stream);
      hipEventRecord(ev[2], stream);
    }
    return hipGetLastError();
  }
  const int chunk = permute_chunk(P);
  const int C = (P + chunk - 1) / chunk;
  const int Cp = permute_hist_stride(P);
  if (ev) hipEventRecord(ev[0], stream);
  rank_kernel<<<C, 1024, 0, stream>>>(ids, P, E, chunk, Cp, rank, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev) hipEventRecord(ev[1], stream);
  scan_kernel<<<1, 1024, 0, stream>>>(hist, C, Cp, E, T, bm, with_shared, base, offsets, tiles,
                                      ntiles, queue);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev) hipEventRecord(ev[2], stream);
  scatter_kernel<<<(P + 255) / 256, 256, 0, stream>>>(ids, rank, base, offsets, P, E, Cp, chunk,
                                                      sorted, pos, topk_w, w_sorted);
  return hipGetLastError();
}

}  // namespace moe

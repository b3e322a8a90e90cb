// Ranking helpers of the stable counting sort by expert (wave ballots over
// the bits of the expert id), shared by the permutation kernels and the
// fused decode kernel.

#pragma once

#include "common.h"

namespace moe {

namespace {

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Lanes of the wave holding the same expert id as this lane (valid lanes only).
__device__ __forceinline__ uint64_t peers_of(int e, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    peers &= bit ? ones : ~ones;
  }
  return peers;
}

__device__ __forceinline__ int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

// Ranks of pairs [q0, q1) (ids staged in LDS at sid[q - q0]) among the
// wave's earlier pairs of the same expert; cnt[e] carries the running count.
// rank_out is indexed by q - rank_base.
__device__ __forceinline__ void rank_span(const int32_t* sid, int q0, int q1, int E, int nbits,
                                          int32_t* cnt, int32_t* rank_out, int rank_base) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lanes_below(lane);
  for (int q = q0; q < q1; q += 64) {
    const int p = q + lane;
    const int e_in = p < q1 ? sid[p - q0] : -1;
    const bool valid = e_in >= 0 && e_in < E;  // out-of-range ids are not counted
    const int e = valid ? e_in : 0;
    const uint64_t peers = peers_of(e, valid, nbits);
    int base = 0;
    if (valid) base = cnt[e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      rank_out[p - rank_base] = base + __popcll(peers & below);
      const int leader = __ffsll(static_cast<unsigned long long>(peers)) - 1;
      if (lane == leader) cnt[e] = base + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

}  // namespace moe

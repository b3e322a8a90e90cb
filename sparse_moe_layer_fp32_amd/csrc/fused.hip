// Single-launch MoE layer forward for small batches (decoding).
//
// The sglang-jax issue "[Feature] Support Step 3.5 Flash (StepFun) Model"
// maps the layer onto a grouped-matmul expert path first and names a fused
// expert backend as the later performance switch ("Reuse map",
// "Implementation strategy").  This is that switch on one GPU: every step of
// the layer runs inside one persistent grid, so a decoding batch pays one
// launch, and the steps overlap where their data allow (the shared expert
// runs while the router decides; down tiles start as soon as their rows'
// gate/up tiles are done, while other gate/up tiles still stream).
//
// Work is a queue of units in eight phases:
//   0 router logit tiles (64 tokens x 64 experts x one k split)
//   1 shared-expert gate/up tiles          4 shared-expert down tiles
//   2 top-k, one token per wave            5 routed gate/up tiles
//   3 the permutation (one block)          6 routed down tiles
//                                          7 combine rows
// Each phase has a ticket counter.  A block takes the next ticket of its
// phase and moves on when the phase has none left; a unit that needs
// results of others waits for a counter that those units raise when done.
// Units only ever wait for units of earlier phases, whose tickets were all
// taken, by blocks that were running when they took them; so every wait
// ends without any assumption about how many blocks are resident.  Waits
// are bounded all the same: one that runs out records a flag in the status
// word, skips its unit's work and still raises its own counter, so the
// grid always drains.
//
// Every unit computes exactly what the multi-launch path computes (same
// router tiles and k splits, same top-k keys and sums, the same k order for
// every GEMM output, same combine order), so the two give bit-identical
// outputs.
//
// Memory ordering: a finished unit waits for its own stores, meets the
// block barrier, and one thread raises the counter with an agent-scope
// release; a waiting unit polls with relaxed loads and takes an
// agent-scope acquire fence once the count is reached.  The control words
// are zero before the launch; the last block to leave zeroes them again.

#include "expert_tile.h"
#include "permute_ops.h"
#include "router_ops.h"

namespace moe {

namespace {

constexpr int kFT = 256;  // threads per block (4 waves)
// GEMM tiles of 64 rows, one block per CU, each keeping 80-120 KB of weights
// in flight: gate/up 128 weight rows at k step 128 with a 3-deep ring (H is
// a multiple of 128); down 256 output columns (the four waves side by side)
// at k step 64 with a 3-deep ring when H is a multiple of 256, else 128
// columns with a 6-deep ring (I is a multiple of 64).
using GuCfg = Cfg<64, 128, 128, 2, 2, 3>;
using DnCfg = Cfg<64, 128, 64, 2, 2, 6>;
using DnWideCfg = Cfg<64, 256, 64, 1, 4, 3>;
constexpr int kDnLds = DnCfg::LDS_BYTES > DnWideCfg::LDS_BYTES ? DnCfg::LDS_BYTES : DnWideCfg::LDS_BYTES;
constexpr int kGemmLds = GuCfg::LDS_BYTES > kDnLds ? GuCfg::LDS_BYTES : kDnLds;
constexpr int kPermLds = (2 * kFusedMaxPairs + 4 * kMaxExperts + kMaxExperts + 16) * 4;
constexpr int kTopkLds = 4 * kMaxExperts * (4 + 8);  // per wave: logits and keys
static_assert(kTopkLds <= kGemmLds, "top-k LDS");
constexpr int kFusedLds = kGemmLds > kRouterTileLds ? (kGemmLds > kPermLds ? kGemmLds : kPermLds)
                                                    : (kRouterTileLds > kPermLds ? kRouterTileLds
                                                                                 : kPermLds);
constexpr uint32_t kSpinLimit = 1u << 20;  // polls before a wait gives up (~1 s)

enum Phase : int {
  kPhRouter,
  kPhSharedGu,
  kPhTopk,
  kPhPermute,
  kPhSharedDown,
  kPhGu,
  kPhDown,
  kPhCombine,
  kNumPhases
};
static_assert(kNumPhases <= kCtlRouterDone - kCtlTicket, "ticket words");

// Unit counts that do not depend on the routing.
struct Shape {
  int T, P, S;
  int nnt;       // router expert tiles
  int n_router;  // router units
  int ns;        // shared row tiles (0 without a shared expert)
  int ntg_s;     // shared gate/up column tiles per row tile
  int ntg;       // routed gate/up column tiles per row tile
  int ntd;       // down column tiles per row tile
  int dn_wide;   // down tiles of 256 columns (else 128)
  int n_topk, n_comb;
};

__device__ __forceinline__ Shape shape_of(const FusedArgs& f) {
  Shape s;
  s.T = static_cast<int>(f.g.T);
  s.P = s.T * f.g.k;
  s.S = f.S;
  const int nmt = (s.T + 63) / 64;
  s.nnt = (f.g.E + 63) / 64;
  s.n_router = nmt * s.nnt * f.S;
  s.ns = f.g.Is > 0 ? nmt : 0;
  s.ntg_s = f.g.Is / 64;
  s.ntg = f.g.I / 64;
  s.dn_wide = f.g.H % 256 == 0;
  s.ntd = f.g.H / (s.dn_wide ? 256 : 128);
  s.n_topk = (s.T + 3) / 4;
  s.n_comb = static_cast<int>((static_cast<int64_t>(s.T) * (f.g.H / 8) + kFT - 1) / kFT);
  return s;
}

__device__ __forceinline__ int phase_units(const Shape& s, int phase, int nr) {
  switch (phase) {
    case kPhRouter: return s.n_router;
    case kPhSharedGu: return s.ns * s.ntg_s;
    case kPhTopk: return s.n_topk;
    case kPhPermute: return 1;
    case kPhSharedDown: return s.ns * s.ntd;
    case kPhGu: return nr * s.ntg;
    case kPhDown: return nr * s.ntd;
    default: return s.n_comb;
  }
}

// A routed tile as the permutation writes it (checked, so that control words
// that were not zero before the launch cannot send a tile outside the
// buffers).
__device__ __forceinline__ bool tile_ok(int2 tile, int E, int P) {
  return tile.x >= 0 && tile.x < E && tile.y >= 0 && tile.y < P;
}

__device__ __forceinline__ uint32_t load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The control code runs on all 64 lanes of one wave and keeps every value
// that a loop or branch depends on uniform across the wave (lane 0 does the
// atomics, readlane hands the result to the others).  A loop that only some
// lanes of a wave run must not hold or precede a block barrier: the compiler
// may then let the other lanes go on through the barrier without them (with
// the tickets taken by thread 0 alone, it did: the rest of the block went on
// to the hand-over barrier and re-read the previous ticket, forever).
__device__ __forceinline__ uint32_t wave_load(const uint32_t* p) {
  return __builtin_amdgcn_readfirstlane(load_relaxed(p));
}

__device__ __forceinline__ uint32_t wave_fetch_add(uint32_t* p, uint32_t v) {
  uint32_t r = 0;
  if ((threadIdx.x & 63) == 0)
    r = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readlane(r, 0);
}

// One whole wave: wait until ctl[word] >= target, then acquire.  On running
// out, record `flag` and return false.
__device__ bool wave_wait_count(uint32_t* ctl, int word, uint32_t target, uint32_t flag) {
  for (uint32_t i = 0; wave_load(ctl + word) < target; ++i) {
    if (i == kSpinLimit) {
      if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(ctl + kCtlStatus, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// The whole block waits (wave 0 polls); true when the count was reached.
__device__ __forceinline__ bool block_wait(uint32_t* ctl, int word, uint32_t target, uint32_t flag,
                                           int* s_ok) {
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wid == 0) {
    const bool ok = wave_wait_count(ctl, word, target, flag);
    if (threadIdx.x == 0) *s_ok = ok ? 1 : 0;
  }
  __syncthreads();
  return *s_ok != 0;
}

// The block's unit is done: its stores are complete, then one release.
__device__ __forceinline__ void block_signal(uint32_t* ctl, int word) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(ctl + word, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix sum over the block's 256 threads; *total receives the sum.
__device__ int scan256(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      tmp[4 + w] = run;
      run += tmp[w];
    }
    tmp[8] = run;
  }
  __syncthreads();
  const int r = tmp[4 + wid] + incl - v;
  *total = tmp[8];
  __syncthreads();
  return r;
}

// The permutation of the P = T k pairs by expert (a stable counting sort:
// each wave ranks a contiguous span of pairs, then the spans' counts are
// prefixed per expert), the expert offsets, the gating weights in expert
// order, and the routed row tiles of 64 rows.  Returns the tile count.
__device__ int fused_permute(const FusedArgs& f, const Shape& s, uint8_t* smem) {
  int32_t* sid = reinterpret_cast<int32_t*>(smem);       // [kFusedMaxPairs]
  int32_t* srank = sid + kFusedMaxPairs;                 // [kFusedMaxPairs]
  int32_t* wcnt = srank + kFusedMaxPairs;                // [4][kMaxExperts]
  int32_t* offs = wcnt + 4 * kMaxExperts;                // [kMaxExperts]
  int* tmp = offs + kMaxExperts;                         // [16]
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = s.P, E = f.g.E;
  for (int p = tid; p < P; p += kFT) sid[p] = f.ids[p];
  for (int i = tid; i < 4 * kMaxExperts; i += kFT) wcnt[i] = 0;
  __syncthreads();
  const int CH = ((P + 3) / 4 + 63) / 64 * 64;  // pairs per wave
  const int q0 = min(P, wid * CH), q1 = min(P, q0 + CH);
  rank_span(sid + q0, q0, q1, E, id_bits(E), wcnt + wid * kMaxExperts, srank, 0);
  __syncthreads();
  // Thread tid owns experts 4 tid .. 4 tid + 3: their counts (with the
  // per-wave prefixes left in wcnt) and row tiles.
  int cnt[4], ntl[4], csum = 0, tsum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    int c = 0;
    if (e < E)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int v = wcnt[w * kMaxExperts + e];
        wcnt[w * kMaxExperts + e] = c;
        c += v;
      }
    cnt[j] = c;
    ntl[j] = (c + 63) / 64;
    csum += c;
    tsum += ntl[j];
  }
  int ctot, ttot;
  int co = scan256(csum, tmp, &ctot);
  int to = scan256(tsum, tmp, &ttot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < E) {
      offs[e] = co;
      f.offsets[e] = co;
      for (int i = 0; i < ntl[j] && to + i < f.tile_cap; ++i)
        f.tiles[to + i] = make_int2(e, co + 64 * i);
    }
    co += cnt[j];
    to += ntl[j];
  }
  if (tid == 0) f.offsets[E] = ctot;
  __syncthreads();
  for (int p = tid; p < P; p += kFT) {
    const int e = sid[p];
    if (e < 0 || e >= E) continue;
    const int i = offs[e] + wcnt[(p / CH) * kMaxExperts + e] + srank[p];
    f.sorted[i] = p;
    f.pos[p] = i;
    f.w_sorted[i] = f.w[p];
  }
  return min(ttot, f.tile_cap);
}

// A down tile (direct stores: the waves go on to other units).
__device__ __forceinline__ void down_tile(const ExpertArgs& g, uint8_t* smem, TileCoord tc, int e,
                                          int row0, int wide) {
  if (wide)
    gemm_tile<1, 64, 256, 64, 1, 4, 3, 0, 0, false>(g, smem, tc, e, row0);
  else
    gemm_tile<1, 64, 128, 64, 2, 2, 6, 0, 0, false>(g, smem, tc, e, row0);
}

__global__ __launch_bounds__(kFT) void fused_kernel(FusedArgs f) {
  // One LDS array for everything, the hand-over words in its last 16 bytes:
  // with a second __shared__ variable the compiler makes every LDS read that
  // follows a weight DMA wait for all DMAs in flight (vmcnt(0)), which drains
  // the GEMM rings at every k substep (the GEMM units ran 2-3x slower).
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kFusedLds + 16];
  int* const s_ctl = reinterpret_cast<int*>(smem + kFusedLds);
  const int tid = threadIdx.x;
  uint32_t* ctl = f.ctl;
  const Shape s = shape_of(f);
  const int E = f.g.E, H = f.g.H;

  int phase = 0, nr = -1;
  for (;;) {
    // Next ticket (wave 0), handed to the block through LDS.
    if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) {
      int t = -1;
      while (phase < kNumPhases) {
        if ((phase == kPhGu || phase == kPhDown) && nr < 0) {
          // Without the permutation there are no routed tiles to run.
          nr = wave_wait_count(ctl, kCtlPermDone, 1, kStPerm)
                   ? min(static_cast<int>(wave_load(ctl + kCtlNtiles)), f.tile_cap)
                   : 0;
        }
        const int units = phase_units(s, phase, nr);
        if (units > 0) {
          t = static_cast<int>(wave_fetch_add(ctl + kCtlTicket + phase, 1u));
          if (t < units) break;
        }
        ++phase;
      }
      if (tid == 0) {
        s_ctl[0] = phase;
        s_ctl[1] = t;
        s_ctl[2] = nr;
      }
    }
    __syncthreads();
    phase = s_ctl[0];
    const int t = s_ctl[1];
    nr = s_ctl[2];
    __syncthreads();
    if (phase >= kNumPhases) break;

    switch (phase) {
      case kPhRouter: {
        const int sp = t % s.S, r = t / s.S;
        router_tile(f.g.x, f.wg, f.zpart, s.T, H, E, H / s.S, s.S, r % s.nnt, r / s.nnt, sp, smem);
        block_signal(ctl, kCtlRouterDone);
        break;
      }
      case kPhSharedGu: {
        const int j = t / s.ntg_s;
        gemm_tile<0, 64, 128, 128, 2, 2, 3, 0>(f.g, smem, TileCoord{0, t % s.ntg_s}, E, 64 * j);
        block_signal(ctl, kCtlSharedGu + j);
        break;
      }
      case kPhTopk: {
        block_wait(ctl, kCtlRouterDone, s.n_router, kStRouter, &s_ctl[3]);
        const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int tok = 4 * t + wv;
        float* zl = reinterpret_cast<float*>(smem) + wv * kMaxExperts;
        uint64_t* kl = reinterpret_cast<uint64_t*>(smem + 4 * kMaxExperts * 4) + wv * kMaxExperts;
        if (tok < s.T)
          topk_wave_lds(f.zpart, f.pl, f.bias, E, f.g.k, f.scaling, f.renorm, f.ids, f.w, tok,
                        zl, kl);
        block_signal(ctl, kCtlTopkDone);
        break;
      }
      case kPhPermute: {
        block_wait(ctl, kCtlTopkDone, s.n_topk, kStTopk, &s_ctl[3]);
        const int ntiles = fused_permute(f, s, smem);
        if (tid == 0) ctl[kCtlNtiles] = static_cast<uint32_t>(ntiles);
        block_signal(ctl, kCtlPermDone);
        break;
      }
      case kPhSharedDown: {
        const int j = t / s.ntd;
        if (block_wait(ctl, kCtlSharedGu + j, s.ntg_s, kStSharedGu, &s_ctl[3]))
          down_tile(f.g, smem, TileCoord{0, t % s.ntd}, E, 64 * j, s.dn_wide);
        block_signal(ctl, kCtlDownDone);
        break;
      }
      case kPhGu: {
        const int i = t / s.ntg;
        const int2 tile = f.tiles[i];
        if (tile_ok(tile, E, s.P))
          gemm_tile<0, 64, 128, 128, 2, 2, 3, 0>(f.g, smem, TileCoord{0, t % s.ntg}, tile.x,
                                                tile.y);
        block_signal(ctl, kCtlTileGu + i);
        break;
      }
      case kPhDown: {
        const int i = t / s.ntd;
        if (block_wait(ctl, kCtlTileGu + i, s.ntg, kStGu, &s_ctl[3])) {
          const int2 tile = f.tiles[i];
          if (tile_ok(tile, E, s.P))
            down_tile(f.g, smem, TileCoord{0, t % s.ntd}, tile.x, tile.y, s.dn_wide);
        }
        block_signal(ctl, kCtlDownDone);
        break;
      }
      default: {
        if (block_wait(ctl, kCtlDownDone, (s.ns + nr) * s.ntd, kStDown, &s_ctl[3]))
          combine_row(f.g.o_routed, f.g.o_shared, f.pos, f.g.k, s.T, H, s.P, f.y,
                      static_cast<int64_t>(t) * kFT + tid);
        break;
      }
    }
  }

  // The last block to leave zeroes the control words for the next launch.
  if (tid == 0)
    s_ctl[3] = __hip_atomic_fetch_add(ctl + kCtlExit, 1u, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (s_ctl[3])
    for (int i = tid; i < kCtlReset; i += kFT) ctl[i] = 0;
}

int fused_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;  // one block per CU (the GEMM rings take most of the LDS)
}

}  // namespace

hipError_t launch_fused(const FusedArgs& f, hipStream_t stream) {
  fused_kernel<<<fused_grid(), kFT, 0, stream>>>(f);
  return hipGetLastError();
}

}  // namespace moe

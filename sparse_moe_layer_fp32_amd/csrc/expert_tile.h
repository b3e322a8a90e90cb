// Grouped SwiGLU expert GEMMs of the MoE layer on gfx950 matrix cores.
//
// Each routed expert is a SwiGLU MLP H -> I -> H (sglang-jax issue
// "[Feature] Support Step 3.5 Flash (StepFun) Model", "Model configuration"
// and "Reuse map": SiLU of the gate times up, optionally clamped; llm-atlas
// Step-3.5-Flash card, raw fields moe_intermediate_size 1280 and
// share_expert_dim 1280).  The pairs were sorted by expert, so expert e owns
// rows [offsets[e], offsets[e+1]) of the sorted order; the shared expert is
// one more group whose rows are the tokens themselves.
//
// gate/up: h[r] = SiLU(min(g, L)) * clamp(u, -L, L) with g = W_gate[e] x_r,
//          u = W_up[e] x_r (no clamp when L <= 0); x rows are gathered by
//          token from the sorted pairs; h is stored bf16 in sorted order.
// down:    o[r] = w_r * (W_down[e] h[r]), bf16, sorted order; w_r is the
//          pair's gating weight (1 for the shared expert).
//
// Mainloop (one template for both GEMMs and both tile shapes):
//  * bf16 x bf16 -> fp32 on v_mfma_f32_32x32x16_bf16; every operand is
//    k-contiguous in memory (weights are out x in), so A and B fragments are
//    plain 16-byte LDS reads.
//  * Tiles are copied HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging): one wave instruction fills 1 KiB of LDS (4, 8 or 16 rows of
//    a 128-, 64- or 32-wide k step); rows are gathered per lane, so
//    the token gather of the gate/up GEMM costs nothing extra.  The 16-byte
//    chunks of a row are XOR-swizzled so that the 64 lanes of a fragment
//    read hit all 64 LDS banks once (no bank conflicts).
//  * An S-stage ring (or a split ring, A and B in rings of their own: Cfg):
//    stages kt+1 .. kt+S-2 are in flight while stage kt is multiplied;
//    per-wave `s_waitcnt vmcnt` plus a bare s_barrier order the ring (no full
//    fence, which would drain the prefetches).
//  * Work comes from a device-side tile list (no host synchronisation); units
//    are spread over the 8 XCDs in contiguous ranges (the big tiles: a queue
//    per XCD, with stealing) and walked in groups of 8 row tiles so that
//    co-resident blocks share operands in their L2.
//
// Two tile families: 256 x 256 (one block per CU, 8 waves of 128 x 64) for
// many rows per expert, and 64-row tiles with 3- or 4-deep rings for few rows
// per expert, where the GEMMs stream weights at HBM rate.

#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int GROUP_M = 8;    // row tiles per scheduling group

// CPOL is the load's cache policy: 0, or kCpolNt for data read once (the
// non-temporal hint: the lines are the first to go from the caches).
template <int CPOL = 0>
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)lds_wave_base, 16, 0, CPOL);
}
constexpr int kCpolNt = 2;  // gfx950 cache-policy bit NT

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct TileCoord {
  int mt, nt;
};

__device__ __forceinline__ TileCoord tile_of(int u, int ntiles, int NT) {
  const int group = u / (GROUP_M * NT);
  const int first = group * GROUP_M;
  const int gm = min(GROUP_M, ntiles - first);
  const int within = u - group * GROUP_M * NT;
  return {first + within % gm, within / gm};
}

// Scheduling groups that follow the experts: the tile list holds each
// expert's row tiles consecutively and in row order, so the tiles of one
// expert are cut into groups of at most GROUP_M, and unit u's group is
// found from the tile u / NT (a group of gm tiles owns the gm NT units from
// its first tile times NT on).  Inside a group the row tile runs fastest,
// so blocks running together share the expert's weight column tiles and
// each row tile's activations; a group never mixes experts, whose weight
// tiles nothing would share.
template <int BM>
__device__ __forceinline__ TileCoord tile_of_expert(int u, int NT, const int2* tiles,
                                                    const int32_t* offsets, int E, int64_t T) {
  const int t = u / NT;
  const int2 tile = tiles[t];
  const bool shared = tile.x == E;
  const int base = shared ? 0 : offsets[tile.x];
  const int64_t n = shared ? T : offsets[tile.x + 1] - base;
  const int i = (tile.y - base) / BM;  // the tile's index among its expert's
  const int gi = i / GROUP_M * GROUP_M;
  const int first = t - (i - gi);
  const int gm = static_cast<int>(min<int64_t>(GROUP_M, (n + BM - 1) / BM - gi));
  const int within = u - first * NT;
  return {first + within % gm, within / gm};
}

// AV = 1 (split ring): A goes through its own 2-deep LDS ring, one k step
// ahead; B through an S-deep ring, S-1 steps ahead.
template <int BM, int BN, int BK, int WM, int WN, int S, int WF = 0, int AV = 0>
struct Cfg {
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int MB = BM / WM / 32;     // 32-row blocks per wave
  static constexpr int NB = BN / WN / 32;     // 32-col blocks per wave
  static constexpr int CH = BK / 8;           // 16-byte chunks per A row (bf16)
  static constexpr int ROWB = BK * 2;         // bytes per A row
  static constexpr int RPI = 64 / CH;         // A rows filled by one DMA instruction
  static constexpr int BROWB = WF ? BK : BK * 2;  // bytes per B row (e4m3 or bf16)
  static constexpr int CHB = BROWB / 16;      // 16-byte chunks per B row
  static constexpr int RPIB = 64 / CHB;       // B rows filled by one DMA instruction
  static constexpr int JA = BM / RPI / NW;    // A DMA instructions per wave per stage
  static constexpr int JB = BN / RPIB / NW;   // B DMA instructions per wave per stage
  static constexpr int NI = JA + JB;
  static constexpr int KS = BK / 16;          // MFMA k-substeps per stage
  static constexpr int STAGE_BYTES = BM * ROWB + BN * BROWB;
  static constexpr int A_BYTES = BM * ROWB;   // one A buffer (AV)
  static constexpr int B_BYTES = BN * BROWB;  // one B buffer (AV)
  static constexpr int LDS_BYTES = AV ? 2 * A_BYTES + S * B_BYTES : S * STAGE_BYTES;
  static_assert(CH == 4 || CH == 8 || CH == 16, "k step of 32, 64 or 128");
  static_assert(CHB == 2 || CHB == 4 || CHB == 8 || CHB == 16, "B row of 32 to 256 bytes");
  static_assert(MB >= 1 && NB >= 1 && JA >= 1 && JB >= 1, "tile shape");
  static_assert(NI * (S > 2 ? S - 2 : 1) <= 63, "vmcnt budget");
  // XOR swizzle of a row's 16-byte chunks.  The LDS serves 16 lanes (256
  // bytes, 64 banks) per cycle; a fragment read has those 16 lanes on 16
  // consecutive rows at one logical chunk.  With 256-byte rows every row
  // spans all banks and row & 15 gives the 16 rows 16 different chunk slots;
  // with 128-byte rows, even and odd rows fall in different bank halves and
  // (row >> 1) & 7 spreads the 8 rows of each half over its 8 chunk slots;
  // with 64-byte rows, row & 3 picks the quarter and (row >> 2) & 3 the
  // slot.  Either way the 16 lanes hit 16 distinct 16-byte bank groups.
  static __device__ __forceinline__ int swz(int row) {
    return CH == 16 ? (row & 15) : CH == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
  }
  // B rows: as above for bf16.  e4m3 fragments are 8-byte reads of 64- or
  // 32-byte rows (32 lanes per cycle); the swizzle spreads the rows that
  // share a bank window over the chunk slots (at most two lanes per bank).
  static __device__ __forceinline__ int swzb(int row) {
    return CHB == 16  ? (row & 15)
           : CHB == 8 ? ((row >> 1) & 7)
           : CHB == 4 ? ((row >> 2) & 3)
                      : ((row >> 3) & 1);
  }
};

// MODE 0: gate/up (+ SwiGLU), MODE 1: down (+ gating weight), MODE 2: the
// router's logits as one dense GEMM over the bf16 planes of its weight.
//
// WF = 1: the routed experts' weights are e4m3 codes (B operand): DMA'd as
// bytes, widened to bf16 exactly after the LDS read, and multiplied by their
// row's scale in the epilogue (a scale per output row factors out of the
// dot product).  The shared expert's tiles (bf16 weights) in such a launch
// take the bf16 body: the choice is made once per block.
//
// STAGED (down only): the output tile leaves through LDS in whole rows, and
// waves without rows end before the epilogue's barriers, so the caller
// ends the block after the tile.  A persistent caller, whose waves go on to
// other work, passes false: direct stores, no barrier after the mainloop.
//
// JOIN (split ring, staged down only): waves without rows do not end after
// the mainloop but pass the epilogue's barriers and help store, for a
// persistent caller whose waves all go on to the next tile.
template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF, int AV = 0,
          bool STAGED = true, bool JOIN = false>
__device__ __forceinline__ void gemm_tile(const ExpertArgs& a, uint8_t* smem, TileCoord tc,
                                          int e, int row0) {
  using C = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  static_assert(AV == 0 || S >= 3, "split ring: B ring of 3 or more");
  static_assert(!JOIN || (AV && MODE == 1 && STAGED), "JOIN: split-ring staged down tiles");
  using BT = typename std::conditional<WF == 1, uint8_t, uint16_t>::type;
  static_assert(WF == 0 || MODE < 2, "e4m3 weights are for the expert GEMMs");
  const bool shared = MODE != 2 && e == a.E;
  const int H = a.H;

  // Problem shape of this group.
  int K, N;  // reduction length, output columns (h cols or d cols)
  if (MODE == 0) {
    K = H;
    N = shared ? a.Is : a.I;
  } else if (MODE == 1) {
    K = shared ? a.Is : a.I;
    N = H;
  } else {
    K = H;
    N = a.Np;
  }
  const int n0 = tc.nt * (MODE == 0 ? BN / 2 : BN);  // first output column
  if (n0 >= N) return;
  const int rows = (shared || MODE == 2) ? static_cast<int>(min<int64_t>(BM, a.T - row0))
                                         : min(BM, a.offsets[e + 1] - row0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // ---- DMA sources.  Instruction j of wave w fills tile rows
  // [RPI (w*J + j), +RPI); lane l writes row RPI(w*J + j) + l/CH at physical
  // chunk l % CH, which holds logical chunk (l % CH) ^ swz(row).
  const int lrow = lane / C::CH;
  const int pchunk = lane % C::CH;
  const uint16_t* abase;
  if (MODE != 1)
    abase = a.x;
  else
    abase = shared ? a.h_shared : a.h_routed;
  uint32_t aoff[C::JA];  // element offsets of the A rows (gathered by token for gate/up)
#pragma unroll
  for (int j = 0; j < C::JA; ++j) {
    const int r = C::RPI * (wid * C::JA + j) + lrow;
    const int lchunk = pchunk ^ C::swz(r);
    const int rr = r < rows ? r : 0;  // rows past the group's end re-read row 0 (one cached line)
    int64_t src_row;
    if (MODE == 0) {
      src_row = shared ? static_cast<int64_t>(row0 + rr) : a.sorted[row0 + rr] / a.k;
      src_row = min<int64_t>(max<int64_t>(src_row, 0), a.T - 1);
    } else {
      src_row = row0 + rr;
    }
    aoff[j] = static_cast<uint32_t>(src_row * K + lchunk * 8);
  }
  // B rows: each wave's rows are consecutive and lie in one matrix (for
  // gate/up the first half of the tile is W_gate, the second W_up).
  const BT* bmat;
  uint32_t boff[C::JB];  // element offsets inside that matrix
  {
    const int lrow_b = lane / C::CHB, pchunk_b = lane % C::CHB;
    const int r0 = C::RPIB * wid * C::JB;  // first B row of this wave
    int mrow;
    if constexpr (WF == 1) {
      const int64_t eo = static_cast<int64_t>(e) * a.I * H;
      if (MODE == 0) {
        const bool up = r0 >= BN / 2;
        bmat = (up ? a.w8_up : a.w8_gate) + eo;
        mrow = n0 + r0 - (up ? BN / 2 : 0);
      } else {
        bmat = a.w8_down + eo;
        mrow = n0 + r0;
      }
    } else if (MODE == 0) {
      const bool up = r0 >= BN / 2;
      bmat = up ? (shared ? a.ws_up : a.w_up + static_cast<int64_t>(e) * a.I * H)
                : (shared ? a.ws_gate : a.w_gate + static_cast<int64_t>(e) * a.I * H);
      mrow = n0 + r0 - (up ? BN / 2 : 0);
    } else if (MODE == 1) {
      bmat = shared ? a.ws_down : a.w_down + static_cast<int64_t>(e) * H * a.I;
      mrow = n0 + r0;
    } else {
      bmat = a.wsplit;
      mrow = n0 + r0;
    }
#pragma unroll
    for (int j = 0; j < C::JB; ++j) {
      const int lchunk = pchunk_b ^ C::swzb(r0 + C::RPIB * j + lrow_b);
      boff[j] = static_cast<uint32_t>((mrow + C::RPIB * j + lrow_b) * K +
                                      lchunk * (16 / static_cast<int>(sizeof(BT))));
    }
  }

  // DMA instruction d (0 <= d < NI) of stage kt: A rows first, then B rows.
  auto issue_one = [&](int kt, int d) {
    uint8_t* st = smem + (kt % S) * C::STAGE_BYTES;
    const int k0 = kt * BK;
    if (d < C::JA) {
      dma16(abase + aoff[d] + k0, st + (wid * C::JA + d) * 1024);
    } else {
      const int j = d - C::JA;
      // Small expert tiles stream weights that no other block reads (few
      // row tiles per expert): non-temporal, so they do not push the
      // activations and outputs out of the caches (decode gate/up and down
      // -10% each) -- when a k step reads whole 128-byte lines: the e4m3
      // rows' 64-byte pieces would have each line fetched twice (+7%).  The
      // router's weight planes are read by every row tile.
      constexpr int bpol = (MODE != 2 && C::BROWB % 128 == 0) ? kCpolNt : 0;
      dma16<bpol>(bmat + boff[j] + k0, st + BM * C::ROWB + (wid * C::JB + j) * 1024);
    }
  };

  // ---- fragment addressing.  Wave (wm, wn) owns rows [wm*BM/WM, +BM/WM).
  const int wm = wid / WN, wn = wid % WN;
  const int fr = lane & 31;
  const int fh = lane >> 5;
  const int fswz = C::swz(fr);  // fragment rows start at multiples of 32
  int a_off[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) a_off[mb] = (wm * (BM / WM) + 32 * mb + fr) * C::ROWB;
  int b_off[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    int brow;
    if (MODE == 0) {
      // blocks 0..NB/2-1 are gate, NB/2.. the matching up blocks
      const int half = C::NB / 2;
      const int hcol = wn * (BN / 2 / WN) + 32 * (nb % half);
      brow = (nb < half ? 0 : BN / 2) + hcol;
    } else {
      brow = wn * (BN / WN) + 32 * nb;
    }
    b_off[nb] = (AV ? 0 : BM * C::ROWB) + (brow + fr) * C::BROWB;
  }

  const int KT = K / BK;
  const bool has_rows = wm * (BM / WM) < rows;  // else: keep the ring going only
  // Down: gating weight of each of this lane's output rows, requested now,
  // used in the epilogue.
  float wt[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int r = wm * (BM / WM) + 32 * mb + fr;
    wt[mb] = (MODE == 1 && !shared && r < rows) ? a.w_sorted[row0 + r] : 1.0f;
  }

  f32x16 acc[C::MB][C::NB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x16{};

  bf16x8 af[2][C::MB], bf[2][C::NB];
  const int fswzb = C::swzb(fr);
  auto load_frags = [&](int kt, int ks, int set) {
    // A and B of stage kt: one ring slot, or (AV) the A and B buffers
    const uint8_t* st =
        AV ? smem + 2 * C::A_BYTES + (kt % S) * C::B_BYTES : smem + (kt % S) * C::STAGE_BYTES;
    const uint8_t* sa = AV ? smem + (kt & 1) * C::A_BYTES : st;
    const int sw = ((2 * ks + fh) ^ fswz) * 16;
    if constexpr (WF == 1) {
      // Logical chunk ks of the e4m3 row holds the 16 codes of k-substep ks;
      // this lane's 8 are half fh.  The whole chunk is read (a single 16-byte
      // LDS read, like the bf16 fragments) and the half selected in registers.
      const int swb = (ks ^ fswzb) * 16;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(st + b_off[nb] + swb);
        bf[set][nb] = fh ? e4m3x8_to_bf16(raw[2], raw[3]) : e4m3x8_to_bf16(raw[0], raw[1]);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
        bf[set][nb] = *reinterpret_cast<const bf16x8*>(st + b_off[nb] + sw);
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      af[set][mb] = *reinterpret_cast<const bf16x8*>(sa + a_off[mb] + sw);
  };
  // The MFMAs of one k-substep; `dma(i)` may issue a refill DMA after MFMA i.
  auto mfmas = [&](int set, auto dma) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        acc[mb][nb] = mfma32(bf[set][nb], af[set][mb], acc[mb][nb]);
        dma(mb * C::NB + nb);
      }
  };
  // A bare barrier orders the ring without draining in-flight prefetches
  // (a full fence would); the "memory" clobber keeps LDS accesses in place.
  auto barrier = [] { asm volatile("s_barrier" ::: "memory"); };

  if constexpr (AV) {
    // Split ring: A has its own 2-deep ring (one stage ahead), B an S-deep
    // ring (S-1 stages ahead), both filled by DMA.  Step kt multiplies A(kt)
    // (A buffer kt & 1) by B(kt) (B slot kt % S).  Right after the barrier
    // that starts it, A(kt+1) is DMA'd into A buffer (kt+1) & 1; between its
    // MFMAs, B(kt+S-1) into B slot (kt-1) % S; both were last read in step
    // kt-1.  At its end, loads returning in order, only B(kt+S-1) may still
    // be in flight (B(kt+1) was issued in an earlier step), and one barrier
    // publishes A(kt+1) and B(kt+1).
    static_assert(S >= 3, "B ring of 3 or more");
    auto a_issue = [&](int kt) {
#pragma unroll
      for (int j = 0; j < C::JA; ++j)
        dma16(abase + aoff[j] + kt * BK, smem + (kt & 1) * C::A_BYTES + (wid * C::JA + j) * 1024);
    };
    auto b_issue = [&](int kt, int j) {
      dma16(bmat + boff[j] + kt * BK,
            smem + 2 * C::A_BYTES + (kt % S) * C::B_BYTES + (wid * C::JB + j) * 1024);
    };
    auto step_end = [&](int kt) {
      if (kt + S - 1 < KT)
        wait_vmcnt<C::JB>();
      else
        wait_vmcnt<0>();
      barrier();
    };
    // Prologue: A(0), B(0 .. S-2); wait for A(0) and B(0).
    a_issue(0);
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < KT)
#pragma unroll
        for (int j = 0; j < C::JB; ++j) b_issue(s, j);
    if (S - 2 < KT)
      wait_vmcnt<(S - 2) * C::JB>();  // B(1 .. S-2) may be in flight
    else
      wait_vmcnt<0>();
    barrier();
    constexpr int MFMAS = C::KS * C::MB * C::NB;
    constexpr int DMA_EVERY = MFMAS / C::JB > 0 ? MFMAS / C::JB : 1;
    if (!has_rows) {
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) a_issue(kt + 1);
        if (kt + S - 1 < KT)
#pragma unroll
          for (int j = 0; j < C::JB; ++j) b_issue(kt + S - 1, j);
        if (kt + 1 < KT) step_end(kt);
      }
      if constexpr (!JOIN) return;
    }
    auto step = [&](int kt, auto REFILL) {
      constexpr bool refill = decltype(REFILL)::value;
      if (kt + 1 < KT) a_issue(kt + 1);
      load_frags(kt, 0, 0);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + 1 < C::KS) load_frags(kt, ks + 1, (ks + 1) & 1);
        mfmas(ks & 1, [&](int i) {
          const int g = ks * C::MB * C::NB + i;
          if (refill && g % DMA_EVERY == DMA_EVERY - 1 && g / DMA_EVERY < C::JB)
            b_issue(kt + S - 1, g / DMA_EVERY);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
      if (refill && MFMAS / DMA_EVERY < C::JB)
#pragma unroll
        for (int j = MFMAS / DMA_EVERY; j < C::JB; ++j) b_issue(kt + S - 1, j);
      if (kt + 1 < KT) step_end(kt);
    };
    if (!JOIN || has_rows) {
      int kt = 0;
      for (; kt + S - 1 < KT; ++kt) step(kt, std::true_type{});
      for (; kt < KT; ++kt) step(kt, std::false_type{});
    }
  } else {
    // Ring of S buffers, S-1 stages in flight: wait for stage kt, barrier
    // (all waves' DMAs of stage kt landed, all waves done with stage kt-1,
    // whose buffer stage kt+S-1 refills), then the stage's MFMAs with the
    // refill DMAs spread between them.
    constexpr int MFMAS = C::KS * C::MB * C::NB;
    constexpr int DMA_EVERY = MFMAS / C::NI > 0 ? MFMAS / C::NI : 1;
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < KT)
#pragma unroll
        for (int d = 0; d < C::NI; ++d) issue_one(s, d);
    auto wait_stage = [&](int kt) {
      if (kt + S - 2 < KT)
        wait_vmcnt<(S - 2) * C::NI>();
      else
        wait_vmcnt<0>();
      barrier();
    };
    if (!has_rows) {
      // Waves without rows keep the same DMA and barrier sequence (a loop of
      // its own: a branch around the MFMAs would move the accumulators).
      for (int kt = 0; kt < KT; ++kt) {
        wait_stage(kt);
        if (kt + S - 1 < KT)
          for (int d = 0; d < C::NI; ++d) issue_one(kt + S - 1, d);
      }
      return;
    }
    // REFILL is a compile-time flag: a runtime branch between the MFMAs
    // would move the accumulators between register files every step.
    auto step = [&](int kt, auto REFILL) {
      constexpr bool refill = decltype(REFILL)::value;
      wait_stage(kt);
      load_frags(kt, 0, 0);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (ks + 1 < C::KS) load_frags(kt, ks + 1, (ks + 1) & 1);
        mfmas(ks & 1, [&](int i) {
          const int g = ks * C::MB * C::NB + i;  // MFMA index in the stage
          if (refill && g % DMA_EVERY == DMA_EVERY - 1 && g / DMA_EVERY < C::NI)
            issue_one(kt + S - 1, g / DMA_EVERY);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
      if (refill && MFMAS / DMA_EVERY < C::NI)  // more DMAs than MFMA slots
#pragma unroll
        for (int d = MFMAS / DMA_EVERY; d < C::NI; ++d) issue_one(kt + S - 1, d);
    };
    int kt = 0;
    for (; kt + S - 1 < KT; ++kt) step(kt, std::true_type{});
    for (; kt < KT; ++kt) step(kt, std::false_type{});
  }
  if (!JOIN && !has_rows) return;

  // ---- epilogue.  The MFMAs take the weight rows as their first operand,
  // so acc[mb][nb] holds the transposed block: lane l owns token row
  // 32 mb + (l % 32) of the wave's rows and, for r = 4g .. 4g+3, the four
  // consecutive output columns 8g + 4(l / 32) + 0..3 of block nb.
  const int row = wm * (BM / WM) + fr;  // + 32 mb
  if (MODE == 2) {
    // fp32 logits, one 16-byte store per group of four
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if (row + 32 * mb >= rows) continue;
      float* zrow = a.zout + static_cast<int64_t>(row0 + row + 32 * mb) * a.Np + n0 +
                    wn * (BN / WN) + 4 * fh;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& v = acc[mb][nb];
          *reinterpret_cast<f32x4*>(zrow + 32 * nb + 8 * g) =
              f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
        }
    }
    return;
  }
  if (MODE == 0) {
    // h after SwiGLU, one 8-byte store per group of four (the SwiGLU work
    // overlaps these stores across waves; staging them costs more than
    // it saves here)
    uint16_t* out = shared ? a.h_shared : a.h_routed;
    const float lim = shared ? a.limit_shared : a.limit;
    const int half = C::NB / 2;
    // e4m3 weights: the scales of this lane's gate and up output rows
    f32x4 sg[C::NB / 2][4], su[C::NB / 2][4];
    if constexpr (WF == 1) {
      const float* sgp = a.s_gate + static_cast<int64_t>(e) * a.I + n0 + wn * (BN / 2 / WN) + 4 * fh;
      const float* sup = a.s_up + static_cast<int64_t>(e) * a.I + n0 + wn * (BN / 2 / WN) + 4 * fh;
#pragma unroll
      for (int nb = 0; nb < half; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          sg[nb][g] = *reinterpret_cast<const f32x4*>(sgp + 32 * nb + 8 * g);
          su[nb][g] = *reinterpret_cast<const f32x4*>(sup + 32 * nb + 8 * g);
        }
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if (row + 32 * mb >= rows) continue;
      uint16_t* orow = out + static_cast<int64_t>(row0 + row + 32 * mb) * N + n0 +
                       wn * (BN / 2 / WN) + 4 * fh;
#pragma unroll
      for (int nb = 0; nb < half; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float gv = acc[mb][nb][4 * g + q], uv = acc[mb][nb + half][4 * g + q];
            if constexpr (WF == 1) {
              gv *= sg[nb][g][q];
              uv *= su[nb][g][q];
            }
            hv[q] = swiglu_f32(gv, uv, lim);
          }
          *reinterpret_cast<uint2*>(orow + 32 * nb + 8 * g) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
    }
    return;
  }
  // Down: o = the sums times the gating weight, then the weight scale for
  // e4m3.
  f32x4 sd[C::NB][4];
  if constexpr (WF == 1) {
    const float* sdp = a.s_down + static_cast<int64_t>(e) * H + n0 + wn * (BN / WN) + 4 * fh;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) sd[nb][g] = *reinterpret_cast<const f32x4*>(sdp + 32 * nb + 8 * g);
  }
  auto o4 = [&](int mb, int nb, int g) {
    const f32x16& v = acc[mb][nb];
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = v[4 * g + q] * wt[mb];
      if constexpr (WF == 1) o[q] *= sd[nb][g][q];
    }
    return make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
  };
  uint16_t* out = shared ? a.o_shared : a.o_routed;
  if constexpr (!STAGED) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if (row + 32 * mb >= rows) continue;
      uint16_t* orow =
          out + static_cast<int64_t>(row0 + row + 32 * mb) * H + n0 + wn * (BN / WN) + 4 * fh;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<uint2*>(orow + 32 * nb + 8 * g) = o4(mb, nb, g);
    }
    return;
  }
  // STAGED: the bf16 tile goes through LDS, free now (no DMA in flight;
  // the barrier below has every wave past its last fragment read), row by
  // row with the 16-byte chunks of row r XOR-rotated by r so the 32 rows of
  // one write instruction land in different banks, then leaves as whole
  // rows: each thread moves 16 bytes, eight threads a 128-byte line.
  // Stored one group of four per lane instead, every store instruction
  // touches 32 rows 2H bytes apart.  Without JOIN, waves without rows have
  // ended here (a barrier waits for the surviving waves only), so the rows
  // are copied out by the waves holding them: those of the first
  // ceil(rows / (BM/WM)) wave rows.  With JOIN every wave is here (the
  // staging loop below skips rows past the group's end).
  constexpr int OCH = BN / 8;  // 16-byte chunks per staged row
  static_assert((OCH & (OCH - 1)) == 0 && OCH >= 4, "power-of-two chunks per row");
  static_assert(BM * BN * 2 <= Cfg<BM, BN, BK, WM, WN, S, 0, AV>::LDS_BYTES,
                "the output tile fits the LDS");
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int r = row + 32 * mb;
    if (r >= rows) continue;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wn * (BN / WN) + 32 * nb + 8 * g + 4 * fh;  // first of the four columns
        *reinterpret_cast<uint2*>(smem + (r * OCH + ((c >> 3) ^ (r & (OCH - 1)))) * 16 +
                                  (c & 4) * 2) = o4(mb, nb, g);
      }
  }
  __syncthreads();
  const int alive = JOIN ? C::THREADS : min(WM, (rows + BM / WM - 1) / (BM / WM)) * WN * 64;
#pragma unroll 4
  for (int i = tid; i < rows * OCH; i += alive) {
    const int r = i / OCH, c = i % OCH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + (r * OCH + (c ^ (r & (OCH - 1)))) * 16);
    *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(row0 + r) * H + n0 + c * 8) = v;
  }
}

// y[t] = o_shared[t] + sum_j o[pos(t, j)] in slot order j = 0..k-1, fp32,
// rounded once to bf16.  Thread idx computes the 8 consecutive outputs
// 8 idx .. 8 idx + 7 of the flattened [T][H] output.
// NT: the o rows are loaded with the non-temporal hint (large batches,
// whose o does not stay in the caches anyway: -8% at T = 8192; decoding
// batches' o is cache-resident and keeps the default).
template <bool NT = false>
__device__ __forceinline__ void combine_row(const uint16_t* __restrict__ o_routed,
                                            const uint16_t* __restrict__ o_shared,
                                            const int32_t* __restrict__ pair_pos, int k,
                                            int64_t T, int H, int P, uint16_t* __restrict__ y,
                                            int64_t idx) {
  const int per_row = H / 8;
  const int64_t t = idx / per_row;
  if (t >= T) return;
  const int d = static_cast<int>(idx - t * per_row) * 8;
  float acc[8];
  if (o_shared) {
    const u32x4* src = reinterpret_cast<const u32x4*>(o_shared + t * H + d);
    const u32x4 v = NT ? __builtin_nontemporal_load(src) : *src;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = bf16_lo(v[q]);
      acc[2 * q + 1] = bf16_hi(v[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  }
  // Slots in chunks of 8: all positions, then all rows, are requested
  // before the first add, so the loads overlap; the adds stay in slot order.
  for (int j0 = 0; j0 < k; j0 += 8) {
    int64_t pos[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pos[j] = j0 + j < k ? min(max(pair_pos[t * k + j0 + j], 0), P - 1) : -1;
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (pos[j] >= 0) {
        const u32x4* src = reinterpret_cast<const u32x4*>(o_routed + pos[j] * H + d);
        v[j] = NT ? __builtin_nontemporal_load(src) : *src;
      }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (pos[j] >= 0)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += bf16_lo(v[j][q]);
          acc[2 * q + 1] += bf16_hi(v[j][q]);
        }
  }
  u32x4 outv;
#pragma unroll
  for (int q = 0; q < 4; ++q) outv[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  *reinterpret_cast<u32x4*>(y + t * H + d) = outv;
}

}  // namespace

}  // namespace moe

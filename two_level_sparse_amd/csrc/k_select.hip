// k_select.hip -- the two selection stages of a decode step.
//
// AsyncTLS pages, section 2A:
//  * coarse block filtering: the Quest upper bound of q.k over a block, from
//    the block's key max/min, recast as a dense GEMM so that the query heads
//    sharing one kv head form the M dimension; top-Kb blocks are kept;
//  * fine token selection: inside the kept blocks, Double-Sparsity style
//    scores on a few INT4 label channels; top-Kt tokens are kept.
//
// k_score_blocks runs the GEMM [q+, q-] . [Kmax; Kmin] on MFMA
// (v_mfma_f32_16x16x32_bf16): rows are the G heads of a pair (zero-padded to
// 16 per m-tile), columns are blocks, k runs over the 2*D summary channels.
// Since Kmax >= Kmin, q+ . Kmax + q- . Kmin = sum_c max(q_c Kmax_c, q_c Kmin_c).
// The epilogue takes the maximum over the heads and writes one fp32 score
// per block. Summary rows are 2*D bf16 contiguous per block, so each lane's
// 16-byte fragment loads are fully used and consecutive blocks are
// consecutive in memory.
//
// The top-k is an exact radix select over order-preserving 32-bit keys of the
// scores, run by one 1024-thread workgroup per row (block_topk). Elements
// equal to the threshold key are taken in index order, which realises the
// lower-index tie rule; the output is written ascending via one block-wide
// scan. The token stage scores its candidates on MFMA in a kernel spread over
// the whole chip (the G heads times r label channels product is a dense
// contraction; INT4 codes are exact in bf16), then selects per pair.
#include <algorithm>

#include "tls_dev.h"
#include "tls_launch.h"
#include "tls_select_dev.h"

namespace tls {

// ----------------------------------------------------------- block scores --

// The scores of NSUB consecutive 16-block tiles of one pair, from tile T0
// (a tile past the last is the last again): best[s] is block 16*(T0+s) + n's
// score in the lanes with kq == 0. The channel loop runs in groups of UNR
// chunks of 32 channels whose loads (summaries and q fragments) are all issued
// before the group's MFMAs. qp: the pair's first head row; sp: its summaries.
template <int MT, int NSUB, int KC, int UNR>
__device__ __forceinline__ void block_tile_scores(float (&best)[NSUB], const uint16_t* qp, const uint16_t* sp,
                                                  int64_t T0, int64_t NB, int G, int D) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int kc = KC > 0 ? KC : D / 32;
  // the tiles in tile-fragment order: lane L reads elements 8L .. 8L+7 of a unit
  const uint16_t* brow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int64_t T = min(T0 + s, summ_tiles(NB) - 1);
    brow[s] = sp + summ_unit(T, 0, 0, kc) + 8 * lane;
  }
  const uint16_t* qrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) qrow[m] = qp + (int64_t)min(m * 16 + n, G - 1) * D;  // rows past G repeat G-1, unused
  f32x4 acc[MT][NSUB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int cb = 0; cb < kc; cb += UNR) {
    u32x4 kmx[UNR][NSUB], kmn[UNR][NSUB], qr[UNR][MT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int off = (cb + u) * 32 + 8 * kq;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        kmx[u][s] = ld16(brow[s] + summ_unit(0, cb + u, 0, kc));
        kmn[u][s] = ld16(brow[s] + summ_unit(0, cb + u, 1, kc));
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) qr[u][m] = ld16(qrow[m] + off);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the group's loads ahead of its MFMAs
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        u32x4 pos, neg;
        split_sign(qr[u][m], pos, neg);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          acc[m][s] = mfma16x16x32(pos, kmx[u][s], acc[m][s]);
          acc[m][s] = mfma16x16x32(neg, kmn[u][s], acc[m][s]);
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    float b = -INFINITY;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m * 16 + 4 * kq + i < G) b = fmaxf(b, acc[m][s][i]);
    best[s] = max_rows(b);
  }
}

// Streaming scorer for small head groups (G <= 48): every summary byte is used
// by at most three 16-row MFMA tiles, so the kernel is a plain HBM stream.
// Each wave scores 16*NSUB consecutive blocks (block_tile_scores). KC = D/32
// when known at compile time (0: from D at run time, with UNR = 1).
// Waves per SIMD the streaming scorer asks of the compiler: one head tile on
// 128 channels fits in 64 registers, so eight workgroups share a CU and the
// 128k launch (2048 workgroups) runs as one round instead of seven per CU
// and a tail; the larger tiles keep the compiler's own choice.
template <int MT, int KC>
constexpr int score_blocks_waves() { return MT == 1 && KC > 0 && KC <= 4 ? 8 : 1; }

template <int MT, int NSUB, int KC, int UNR>
__global__ __launch_bounds__(256, (score_blocks_waves<MT, KC>())) void k_score_blocks(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ summ, float* __restrict__ S,
                                                      int Hq, int Hkv, int G, int D, int64_t NB, int64_t NBs) {
  const int p = blockIdx.y;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t jbase = ((int64_t)blockIdx.x * 4 + wave) * (16 * NSUB);
  if (jbase >= NB) return;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  const uint16_t* sp = summ + (int64_t)p * summ_pair_elems(NBs, D);
  float best[NSUB];
  block_tile_scores<MT, NSUB, KC, UNR>(best, qp, sp, jbase / 16, NB, G, D);
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int64_t j = jbase + s * 16 + n;
    if (kq == 0 && j < NB) S[(int64_t)p * NB + j] = best[s];
  }
}

// LDS-staged scorer for large head groups (G > 48, e.g. MLA's 128 heads on
// one latent kv head): a GEMM with M = G heads, N = blocks, K = 2*D. A
// workgroup of 8 waves scores kLdsTiles tiles of 16 consecutive blocks of one
// pair. Wave w takes head tiles 2*(w&3), 2*(w&3)+1 and one half of the
// channel chunks (w>>2); the two halves' sums meet in LDS at the end.
//
// The contraction streams over the chunks of a half: step g multiplies chunk
// g of the first half (waves 0-3) and chunk KH+g of the second (waves 4-7).
// Everything a step needs -- the wave's own q fragments of its chunk and the
// summary pieces (tile, half, max|min) of both chunks -- goes to one of
// kLdsSlots LDS slots with direct global->LDS 16-byte loads, kLdsSlots-1
// steps ahead of the products, laid out as MFMA fragments (64 lanes x 16
// bytes per piece, read back conflict-free). Only direct loads are in
// flight, so a wave waits with vmcnt for exactly the step it multiplies next
// (plain loads of q beside them would make the compiler wait for all), and
// one barrier per step both publishes the step's pieces and frees the slot
// of the step before for the next issue. Each slot is its own LDS object, so
// reading one slot does not also wait for the loads into the others.
constexpr int kLdsTiles = 4;
constexpr int kLdsWaves = 8;
constexpr int kLdsSlots = 4;

struct LdsScoreSlot {
  u32x4 q[kLdsWaves][2][64];             // wave, head tile of the wave, lane
  u32x4 b[kLdsTiles][2][2][64];          // tile, half, max|min, lane
};

template <int MT, int KC>
__global__ __launch_bounds__(kLdsWaves * 64) void k_score_blocks_lds(const uint16_t* __restrict__ q,
                                                                     const uint16_t* __restrict__ summ,
                                                                     float* __restrict__ S, int Hq, int Hkv, int G,
                                                                     int64_t NB, int64_t NBs) {
  constexpr int D = KC * 32;
  constexpr int MW = 2;       // head tiles per wave
  constexpr int KH = KC / 2;  // steps (chunks per half)
  constexpr int BPW = kLdsTiles * 2 * 2 / kLdsWaves;  // summary pieces per wave and step
  constexpr int LPS = MW + BPW;                       // direct loads per wave and step
  static_assert(MT == 8 && KC % 2 == 0 && kLdsTiles == 4 && BPW == 2, "tile layout");
  // (a slot no step uses is never referenced, and takes no LDS)
  __shared__ LdsScoreSlot s0, s1, s2, s3;
  __shared__ float part[kLdsTiles][4][16];
  // after the products: the second channel half's sums, [tile][head-tile pair][MW][lane]
  static_assert(sizeof(LdsScoreSlot) >= kLdsTiles * 4 * MW * 64 * sizeof(f32x4), "half sums fit a slot");
  f32x4* half1 = reinterpret_cast<f32x4*>(&s0);

  // Workgroup -> (pair, tile group). Workgroups are dealt to the 8 XCDs in
  // turn (linear id mod 8); when the pair count allows, every workgroup of a
  // pair lands on one XCD, whose L2 then serves the pair's q to all of them.
  const int gx = (int)((NB + 16 * kLdsTiles - 1) / (16 * kLdsTiles));  // tile groups per pair
  const int npairs = (int)gridDim.x / gx;
  int p, tg;
  if (npairs % 8 == 0) {
    const int xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
    p = xcd + 8 * (slot / gx);
    tg = slot % gx;
  } else {
    p = (int)blockIdx.x / gx;
    tg = (int)blockIdx.x % gx;
  }
  const int b = p / Hkv, h = p % Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int hp = wave & 3, kh = wave >> 2;  // head-tile pair, channel half
  // A workgroup always loads kLdsTiles tiles; rows past NB repeat row NB-1
  // and are not stored. q rows past G repeat row G-1; their products are
  // left out of the maxima.
  const int64_t t0 = (int64_t)tg * kLdsTiles;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  const uint16_t* sp = summ + (int64_t)p * summ_pair_elems(NBs, D);
  const uint16_t* qr[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) qr[i] = qp + (int64_t)min((2 * hp + i) * 16 + n, G - 1) * D + 8 * kq + kh * KH * 32;
  // this wave's summary pieces x = wave + 8k: (tile x>>2, half (x>>1)&1,
  // max|min x&1), each one 1 KB unit of the tile-fragment order (a tile past
  // the last is the last again; its scores are not stored)
  const uint16_t* br[BPW];
#pragma unroll
  for (int k = 0; k < BPW; ++k) {
    const int x = wave + kLdsWaves * k;
    const int64_t T = min(t0 + (x >> 2), summ_tiles(NB) - 1);
    br[k] = sp + summ_unit(T, ((x >> 1) & 1) * KH, x & 1, KC) + 8 * lane;
  }
  auto slot_of = [&](auto gc) -> LdsScoreSlot& {
    constexpr int sl = decltype(gc)::value % kLdsSlots;
    if constexpr (sl == 0) return s0;
    else if constexpr (sl == 1) return s1;
    else if constexpr (sl == 2) return s2;
    else return s3;
  };
  auto issue = [&](auto gc) {
    constexpr int g = decltype(gc)::value;
    if constexpr (g < KH) {
      LdsScoreSlot& sl = slot_of(gc);
#pragma unroll
      for (int i = 0; i < MW; ++i)
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(qr[i] + g * 32),
                                         (__attribute__((address_space(3))) void*)&sl.q[wave][i][0], 16, 0, 0);
#pragma unroll
      for (int k = 0; k < BPW; ++k) {
        const int x = wave + kLdsWaves * k;
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(br[k] + summ_unit(0, g, 0, KC)),
                                         (__attribute__((address_space(3))) void*)&sl.b[x >> 2][(x >> 1) & 1][x & 1][0],
                                         16, 0, 0);
      }
    }
  };

  // accumulators: one chain per (tile, head tile); a chunk's q+ products go
  // to the eight chains first, then its q- products
  f32x4 acc[kLdsTiles][MW];
#pragma unroll
  for (int t = 0; t < kLdsTiles; ++t)
#pragma unroll
    for (int i = 0; i < MW; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto product = [&](const LdsScoreSlot& sl) {
    // all ten LDS reads first, then one wait (interleaved with the MFMAs the
    // compiler waits for each pair of reads in turn)
    u32x4 qraw[MW], bmx[kLdsTiles], bmn[kLdsTiles];
#pragma unroll
    for (int i = 0; i < MW; ++i) qraw[i] = sl.q[wave][i][lane];
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t) {
      bmx[t] = sl.b[t][kh][0][lane];
      bmn[t] = sl.b[t][kh][1][lane];
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 qpos[MW], qneg[MW];
#pragma unroll
    for (int i = 0; i < MW; ++i) split_sign(qraw[i], qpos[i], qneg[i]);
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t)
#pragma unroll
      for (int i = 0; i < MW; ++i) acc[t][i] = mfma16x16x32(qpos[i], bmx[t], acc[t][i]);
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t)
#pragma unroll
      for (int i = 0; i < MW; ++i) acc[t][i] = mfma16x16x32(qneg[i], bmn[t], acc[t][i]);
  };
  // step g: wait for this wave's loads of step g (the ones issued after it
  // may stay in flight), then a barrier (no fence: it would wait for those
  // too) after which every wave's pieces of step g are in LDS and every wave
  // is done with step g-1, whose slot then takes step g-1+kLdsSlots
  auto step = [&](auto gc) {
    constexpr int g = decltype(gc)::value;
    if constexpr (g < KH) {
      // (the products of step g-1, and with them every read of its slot, stay
      // ahead of this wait and barrier: the slot is refilled right after)
      __builtin_amdgcn_sched_barrier(0);
      constexpr int last_issued = g == 0 ? kLdsSlots - 1 : g + kLdsSlots - 2;
      constexpr int ahead = (last_issued < KH - 1 ? last_issued : KH - 1) - g;
      wait_vmcnt<LPS * ahead>();
      __asm__ volatile("s_barrier" ::: "memory");
      if constexpr (g > 0) issue(std::integral_constant<int, g - 1 + kLdsSlots>{});
      product(slot_of(gc));
    }
  };
  issue(std::integral_constant<int, 0>{});
  issue(std::integral_constant<int, 1>{});
  issue(std::integral_constant<int, 2>{});
  issue(std::integral_constant<int, 3>{});
  static_assert(kLdsSlots == 4 && KH <= 12, "steps unrolled below");
  step(std::integral_constant<int, 0>{});
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 3>{});
  step(std::integral_constant<int, 4>{});
  step(std::integral_constant<int, 5>{});
  step(std::integral_constant<int, 6>{});
  step(std::integral_constant<int, 7>{});
  step(std::integral_constant<int, 8>{});
  step(std::integral_constant<int, 9>{});
  step(std::integral_constant<int, 10>{});
  step(std::integral_constant<int, 11>{});
  // the second channel half hands its sums to the first (through slot 0,
  // once every wave is done reading the slots)
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t)
#pragma unroll
      for (int i = 0; i < MW; ++i) half1[((t * 4 + hp) * MW + i) * 64 + lane] = acc[t][i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t) {
      float best = -INFINITY;
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        const f32x4 sum = acc[t][i] + half1[((t * 4 + hp) * MW + i) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((2 * hp + i) * 16 + 4 * kq + r < G) best = fmaxf(best, sum[r]);
      }
      best = max_rows(best);
      if (kq == 0) part[t][hp][n] = best;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int t = lane >> 4, jj = lane & 15;
    const int64_t j = (t0 + t) * 16 + jj;
    if (t < kLdsTiles && j < NB)
      S[(int64_t)p * NB + j] = fmaxf(fmaxf(part[t][0][jj], part[t][1][jj]), fmaxf(part[t][2][jj], part[t][3][jj]));
  }
}

// Largest divisor of kc whose chunk group keeps at most 24 16-byte loads in
// flight per lane.
constexpr int unroll_for(int kc, int loads_per_chunk) {
  int u = 1;
  for (int d = 1; d <= kc; ++d)
    if (kc % d == 0 && d * loads_per_chunk <= 24) u = d;
  return u;
}

template <int MT, int NSUB, int KC>
static void go_blocks_k(const BlockScoreArgs& a, hipStream_t st) {
  constexpr int UNR = KC > 0 ? unroll_for(KC, 2 * NSUB + MT) : 1;
  const int64_t per_wg = 4 * 16 * NSUB;
  dim3 grid((unsigned)((a.NB + per_wg - 1) / per_wg), (unsigned)a.pairs);
  hipLaunchKernelGGL((k_score_blocks<MT, NSUB, KC, UNR>), grid, dim3(256), 0, st, a.q, a.summ, a.S, a.Hq, a.Hkv, a.G,
                     a.D, a.NB, a.NBs);
}

// Always 8 head tiles: for G < 128 the extra tiles run on clamped q rows and
// are masked; their waves would otherwise idle beside the others.
template <int KC>
static void go_blocks_lds(const BlockScoreArgs& a, hipStream_t st) {
  const int64_t ntiles = (a.NB + 15) / 16;
  const int64_t gx = (ntiles + kLdsTiles - 1) / kLdsTiles;
  hipLaunchKernelGGL((k_score_blocks_lds<8, KC>), dim3((unsigned)(gx * a.pairs)), dim3(kLdsWaves * 64), 0, st, a.q, a.summ,
                     a.S, a.Hq, a.Hkv, a.G, a.NB, a.NBs);
}

template <int MT, int NSUB>
static void go_blocks(const BlockScoreArgs& a, hipStream_t st) {
  if constexpr (MT >= 4) {
    switch (a.D) {
      case 128: go_blocks_lds<4>(a, st); return;
      case 256: go_blocks_lds<8>(a, st); return;
      case 576: go_blocks_lds<18>(a, st); return;
      default: break;
    }
  }
  switch (a.D) {
    case 64: go_blocks_k<MT, NSUB, 2>(a, st); break;
    case 128: go_blocks_k<MT, NSUB, 4>(a, st); break;
    case 256: go_blocks_k<MT, NSUB, 8>(a, st); break;
    case 576: go_blocks_k<MT, NSUB, 18>(a, st); break;
    default: go_blocks_k<MT, NSUB, 0>(a, st); break;
  }
}

// One 16-block tile per wave for a single head tile (twice the workgroups of
// two tiles per wave; 128k: 12.6 us per launch against 13.1).
hipError_t launch_score_blocks(const BlockScoreArgs& a, hipStream_t st) {
  const int mt = (a.G + 15) / 16;
  switch (mt) {
    case 1: go_blocks<1, 1>(a, st); break;
    case 2: go_blocks<2, 2>(a, st); break;
    case 3: go_blocks<3, 1>(a, st); break;
    case 4: go_blocks<4, 1>(a, st); break;
    case 5: go_blocks<5, 1>(a, st); break;
    case 6: go_blocks<6, 1>(a, st); break;
    case 7: go_blocks<7, 1>(a, st); break;
    case 8: go_blocks<8, 1>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


// Top-Kb of the block scores of one pair per workgroup.
template <int PER, int NT>
__global__ __launch_bounds__(NT) void k_topk_blocks(const float* __restrict__ S, int n, int K,
                                                    int32_t* __restrict__ out) {
  __shared__ TopkLds<NT> sh;
  const int row = blockIdx.x;
  float v[PER];
  load_row_f32<PER>(S + (int64_t)row * n, n, threadIdx.x * PER, v);
  uint32_t key[PER];
  int32_t id[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = threadIdx.x * PER + e;
    id[e] = c;
    key[e] = c < n ? order_key(v[e]) : 0u;
  }
  __shared__ uint32_t stage[NT * PER];
  block_topk<PER, NT>(key, id, (uint32_t)K, out + (int64_t)row * K, K, sh, stage);
}

// ----------------------------------------------------------- token stage --
// Candidate c of a pair is token block_idx[c / bs] * bs + c % bs (ascending
// with c); it exists only when that token is < N.

// Label-channel scores of candidates in units of 256 per wave (16 tiles of
// 16). Sixteen candidates times sixteen heads is one MFMA (16x16x32 bf16):
// A = q on the label channels (heads x channels, zero padded to 32 channels),
// B = the candidates' INT4 codes widened to bf16 (exact). The epilogue takes
// the max over the heads and multiplies by the token's scale (non-negative,
// so the order of max and scale is immaterial). A unit's loads go out in two
// dependent batches (block numbers, then codes and scales) before its MFMAs;
// the label-channel -> query chain runs beside them.
// A unit is UT tiles of 16 candidates (one wave); UT/4 groups of four tiles,
// one score per lane each.

template <int UT>
struct UnitLoads {
  uint32_t cw[UT];  // lane (n, kq): code bytes 4kq..4kq+3 of candidate c0 + 16u + n
  float tsc[UT / 4];   // scale of candidate c0 + 64j + lane
  bool ok[UT / 4];     // that candidate exists
};

// Issues the loads of the unit starting at candidate c0. `bidx` is the pair's
// block list (global or LDS).
template <int RB, int UT>
__device__ __forceinline__ void unit_loads(UnitLoads<UT>& L, const int32_t* bidx, const uint8_t* cbase,
                                           const float* sbase, int c0, int ncand, int64_t N, int bs, int bsh,
                                           int rb) {
  const int lane = threadIdx.x & 63, n = lane & 15, kq = lane >> 4;
  int cq[UT], sq[UT / 4], cid[UT], sid[UT / 4];
  if (bsh >= 0) {
#pragma unroll
    for (int u = 0; u < UT; ++u) cq[u] = min(c0 + u * 16 + n, ncand - 1) >> bsh;
#pragma unroll
    for (int j = 0; j < UT / 4; ++j) sq[j] = min(c0 + 64 * j + lane, ncand - 1) >> bsh;
  } else {
#pragma unroll
    for (int u = 0; u < UT; ++u) cq[u] = min(c0 + u * 16 + n, ncand - 1) / bs;
#pragma unroll
    for (int j = 0; j < UT / 4; ++j) sq[j] = min(c0 + 64 * j + lane, ncand - 1) / bs;
  }
#pragma unroll
  for (int u = 0; u < UT; ++u) cid[u] = bidx[cq[u]];
#pragma unroll
  for (int j = 0; j < UT / 4; ++j) sid[j] = bidx[sq[j]];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    const int c = c0 + u * 16 + n;
    const int64_t t = (int64_t)cid[u] * bs + (c - cq[u] * bs);
    const int64_t ts = (c < ncand && t >= 0 && t < N) ? t : 0;  // masked candidates read token 0
    const uint8_t* cp = cbase + ts * rb;
    if constexpr (RB > 0) {
      L.cw[u] = *reinterpret_cast<const uint32_t*>(cp + (4 * kq < RB ? 4 * kq : 0));
    } else {
      uint32_t w = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) w |= (uint32_t)cp[min(4 * kq + e, rb - 1)] << (8 * e);
      L.cw[u] = w;
    }
  }
#pragma unroll
  for (int j = 0; j < UT / 4; ++j) {
    const int c = c0 + 64 * j + lane;
    const int64_t t = (int64_t)sid[j] * bs + (c - sq[j] * bs);
    L.ok[j] = c < ncand && t >= 0 && t < N;
    L.tsc[j] = sbase[L.ok[j] ? t : 0];
  }
}


// Scores of the unit: val[j] for candidate c0 + 64j + lane (0 if it does not
// exist).
template <int MT, int RB, int UT>
__device__ __forceinline__ void unit_scores(float (&val)[UT / 4], const UnitLoads<UT>& L, const u32x4 (&qa)[MT],
                                            int G, int rb) {
  const int lane = threadIdx.x & 63, kq = lane >> 4;
#pragma unroll
  for (int j = 0; j < UT / 4; ++j) {
    // x[jj]: max over the heads this lane holds (rows 4kq .. 4kq+3 of every
    // head tile) for candidate n of tile 4j + jj.
    float x[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t w = L.cw[4 * j + jj];
      if constexpr (RB > 0) {
        if (4 * kq >= RB) w = 0u;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * kq + e >= rb) w &= ~(0xFFu << (8 * e));
      }
      const u32x4 bop = codes_to_bf16(w);  // channels 8kq .. 8kq+7
      float best = -INFINITY;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const f32x4 a = mfma16x16x32(qa[m], bop, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i)
          best = fmaxf(best, a[i]);  // rows past G repeat head G-1
      }
      x[jj] = best;
    }
    // Max across the four 16-lane rows, scattered so that row kq ends with
    // tile 4j + kq: the 32-lane swap pairs rows (0,2) and (1,3) and leaves
    // tiles {0,1} in the low half, {2,3} in the high half; the 16-lane swap
    // then pairs rows (0,1) and (2,3).
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[2]), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]), __float_as_uint(x[3]), false, false);
    const float y0 = fmaxf(__uint_as_float(s02[0]), __uint_as_float(s02[1]));
    const float y1 = fmaxf(__uint_as_float(s13[0]), __uint_as_float(s13[1]));
    const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y0), __float_as_uint(y1), false, false);
    const float best = fmaxf(__uint_as_float(s01[0]), __uint_as_float(s01[1]));
    val[j] = L.ok[j] ? L.tsc[j] * best : 0.0f;
  }
}

// Token scores of 4 units per workgroup (one unit of UT*16 candidates per
// wave), spread over the chip; the scores go to A[pair, candidate] for
// k_topk_tokens.
// The scores of one wave's unit (UT*16 candidates from c0): val[j] belongs to
// candidate cand[j]; qa holds the A fragments (label_q_finish).
// FOLD: the folded form (G <= 8, r = 8 or 16, bs = 64).
template <int MT, int RB, int UT, bool FOLD>
__device__ __forceinline__ void score_unit(float (&val)[UT / 4], int (&cand)[UT / 4], const int32_t* bidx,
                                           const u32x4 (&qa)[MT], const uint8_t* cbase, const float* sbase, int c0,
                                           int kb, int64_t N, int64_t Ns, int G, int bs, int bsh, int r) {
  const int lane = threadIdx.x & 63;
  const int rb = r / 2, ncand = kb * bs;
  if constexpr (FOLD) {
    static_assert(MT == 1 && (RB == 4 || RB == 8), "folded scores: G <= 8, r = 8 or 16");
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(cbase, (int)(Ns * RB));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sbase, (int)(Ns * 4));
    fold_unit<RB, UT / 4>(val, cand, bidx, cr, sr, c0, kb, N, qa[0]);
  } else {
    UnitLoads<UT> L;
    unit_loads<RB, UT>(L, bidx, cbase, sbase, c0, ncand, N, bs, bsh, rb);
    unit_scores<MT, RB, UT>(val, L, qa, G, rb);
#pragma unroll
    for (int j = 0; j < UT / 4; ++j) cand[j] = c0 + 64 * j + lane;
  }
}

// Pair and unit group of a workgroup of a (unit groups, pairs) grid.
// Workgroups are dealt to the 8 XCDs in turn (linear id mod 8); when the pair
// count allows, all of pair p's workgroups land on XCD p mod 8, so that its
// block-score row, label channels and q are fetched into one L2 only.
__device__ __forceinline__ void pair_and_unit(int& p, int& ux) {
  const int nx = (int)gridDim.x;
  if (gridDim.y % 8 == 0) {
    const int l = (int)blockIdx.y * nx + (int)blockIdx.x;
    const int slot = l / 8;
    p = l % 8 + 8 * (slot / nx);
    ux = slot % nx;
  } else {
    p = (int)blockIdx.y;
    ux = (int)blockIdx.x;
  }
}

template <int MT, int RB, int UT, bool FOLD>
__global__ __launch_bounds__(256) void k_score_tokens(const uint16_t* __restrict__ q,
                                                      const int32_t* __restrict__ label_ch,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale,
                                                      const int32_t* __restrict__ block_idx, float* __restrict__ A,
                                                      int Hq, int Hkv, int G, int D, int64_t N, int64_t Ns, int bs,
                                                      int bsh, int r, int kb) {
  int p, ux;
  pair_and_unit(p, ux);
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6;
  const int ncand = kb * bs, rb = r / 2;
  const int c0 = ux * (4 * UT * 16) + wave * (UT * 16);
  const int32_t* lab = label_ch + (int64_t)h * r;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  __shared__ __align__(16) uint16_t sq[MT * 16 * kLabRow];
  u32x4 qa[MT];
  uint32_t hl[2 * MT];
  label_q_issue<MT>(hl, lab, qp, G, D, r);
  label_q_finish<MT, FOLD>(qa, hl, sq, r);
  float val[UT / 4];
  int cand[UT / 4];
  score_unit<MT, RB, UT, FOLD>(val, cand, block_idx + (int64_t)p * kb, qa, codes + (int64_t)p * Ns * rb,
                               scale + (int64_t)p * Ns, c0, kb, N, Ns, G, bs, bsh, r);
  // bounded buffer stores: the hardware drops candidates >= ncand
  const __amdgpu_buffer_rsrc_t arow = make_rsrc(A + (int64_t)p * ncand, ncand * 4);
#pragma unroll
  for (int j = 0; j < UT / 4; ++j)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[j]), arow, cand[j] * 4, 0, 0);
}

// Both selection stages of a pair in one launch after the block scores: every
// token-scoring workgroup first selects its pair's top-Kb blocks from the
// block-score row itself (the same radix select as k_topk_blocks, thread t
// holding blocks [t*per, t*per + per)), keeps the list in LDS for its
// candidate loads, and workgroup 0 of the pair writes it out. The selection
// is repeated by the pair's few scoring workgroups instead of costing a launch
// of its own, which would keep all but one workgroup per pair of the chip idle.
constexpr int kSelMaxBlocks = 4096;  // block-score row per workgroup: 16 per thread
// BSC: the workgroups compute their pair's block scores themselves from the
// summaries (block_tile_scores, the arithmetic of k_score_blocks, so the same
// scores) instead of reading them from S: one head tile, 128 channels, at most
// kSelScoreMaxBlocks blocks, kSelScoreTiles tiles per wave and round. Every
// scoring workgroup of a pair then reads all of the pair's summaries, which
// pays while they are few: graph-replayed steps of 4 x 8 pairs (G = 4, Kb =
// NB/8) took 26.5 / 29.5 / 33.8 / 36.6 us at 128 / 256 / 384 / 512 blocks
// against 29.5 / 31.7 / 34.2 / 35.7 us with the block scorer's launch.
constexpr int kSelScoreMaxBlocks = 384;
constexpr int kSelScoreTiles = 4;

template <int MT, int RB, int UT, int PERB, bool FOLD, bool BSC>
__global__ __launch_bounds__(256) void k_score_tokens_sel(const uint16_t* __restrict__ q,
                                                          const int32_t* __restrict__ label_ch,
                                                          const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ S,
                                                          const uint16_t* __restrict__ summ, int NB, int64_t NBs,
                                                          int32_t* __restrict__ block_idx, float* __restrict__ A,
                                                          int Hq, int Hkv, int G, int D, int64_t N, int64_t Ns, int bs,
                                                          int bsh, int r, int kb) {
  static_assert(!BSC || (MT == 1 && PERB * 256 >= kSelScoreMaxBlocks), "block scores inside: one head tile");
  __shared__ TopkLds<256> sh;
  __shared__ uint32_t stage[256 * PERB];
  __shared__ int32_t sblk[kSelMaxBlocks];
  __shared__ float srow[BSC ? kSelScoreMaxBlocks : 1];
  int p, ux;
  pair_and_unit(p, ux);
  const int tid = threadIdx.x;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = tid >> 6;
  const int ncand = kb * bs, rb = r / 2;
  // the q gathers (label channels, then q on them) go out with the block-score
  // row and land while the blocks are selected: the selection's barriers
  // order LDS only and do not wait for them
  __shared__ __align__(16) uint16_t sq[MT * 16 * kLabRow];
  uint32_t hl[2 * MT];
  {
    const int per = (NB + 255) / 256;
    float v[PERB];
    const int32_t* lab = label_ch + (int64_t)h * r;
    const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
    if constexpr (BSC) {
      label_q_issue<MT>(hl, lab, qp, G, D, r);
      // wave w scores tiles 4w .. 4w+3, then 16 further on, ...
      const uint16_t* sp = summ + (int64_t)p * summ_pair_elems(NBs, D);
      const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), ntiles = (NB + 15) / 16;
      for (int t0 = wv * kSelScoreTiles; t0 < ntiles; t0 += 4 * kSelScoreTiles) {
        float best[kSelScoreTiles];
        block_tile_scores<1, kSelScoreTiles, 4, 4>(best, qp, sp, t0, NB, G, D);
#pragma unroll
        for (int s = 0; s < kSelScoreTiles; ++s) {
          const int j = (t0 + s) * 16 + (tid & 15);
          if ((tid & 63) < 16 && j < NB) srow[j] = best[s];
        }
      }
      lds_sync();
#pragma unroll
      for (int e = 0; e < PERB; ++e) {
        const int c = tid * per + e;
        v[e] = (e < per && c < NB) ? srow[c] : 0.0f;
      }
    } else {
      load_row_f32<PERB>(S + (int64_t)p * NB, NB, tid * per, v);
      label_q_issue<MT>(hl, lab, qp, G, D, r);
    }
    uint32_t key[PERB];
    int32_t id[PERB];
#pragma unroll
    for (int e = 0; e < PERB; ++e) {
      const int c = tid * per + e;
      id[e] = c;
      key[e] = (e < per && c < NB) ? order_key(v[e]) : 0u;
    }
    block_topk<PERB, 256>(key, id, (uint32_t)kb, sblk, kb, sh, stage);
  }
  lds_sync();
  if (ux == 0)
    for (int i = tid; i < kb; i += 256) block_idx[(int64_t)p * kb + i] = sblk[i];
  const int c0 = ux * (4 * UT * 16) + wave * (UT * 16);
  u32x4 qa[MT];
  label_q_finish<MT, FOLD>(qa, hl, sq, r);
  float val[UT / 4];
  int cand[UT / 4];
  score_unit<MT, RB, UT, FOLD>(val, cand, sblk, qa, codes + (int64_t)p * Ns * rb, scale + (int64_t)p * Ns, c0, kb, N,
                               Ns, G, bs, bsh, r);
  const __amdgpu_buffer_rsrc_t arow = make_rsrc(A + (int64_t)p * ncand, ncand * 4);
#pragma unroll
  for (int j = 0; j < UT / 4; ++j)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[j]), arow, cand[j] * 4, 0, 0);
}

// Top-Kt' of the candidate scores of one pair per workgroup; ids are tokens.
template <int PER, int NT>
__global__ __launch_bounds__(NT) void k_topk_tokens(const float* __restrict__ A,
                                                               const int32_t* __restrict__ block_idx,
                                                               int32_t* __restrict__ token_idx, int64_t N, int bs,
                                                               int bsh, int kb, int kt) {
  __shared__ TopkLds<NT> sh;
  const int p = blockIdx.x, tid = threadIdx.x;
  const int ncand = kb * bs;
  const int32_t* bidx = block_idx + (int64_t)p * kb;
  // scores and block numbers of this thread's candidates, all loads in flight together
  float v[PER];
  load_row_f32<PER>(A + (int64_t)p * ncand, ncand, tid * PER, v);
  int bq[PER], bid[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = min(tid * PER + e, ncand - 1);
    bq[e] = bsh >= 0 ? (c >> bsh) : c / bs;
  }
  if (bs % PER == 0) {
    // the thread's elements lie in one block: one load of its number
    const int b0 = bidx[bq[0]];
#pragma unroll
    for (int e = 0; e < PER; ++e) bid[e] = b0;
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) bid[e] = bidx[bq[e]];
  }
  uint32_t key[PER];
  int32_t id[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = tid * PER + e;
    const int64_t t = (int64_t)bid[e] * bs + (c - bq[e] * bs);
    const bool ok = c < ncand && t >= 0 && t < N;
    key[e] = ok ? order_key(v[e]) : 0u;
    id[e] = ok ? (int32_t)t : -1;
  }
  __shared__ uint32_t stage[NT * PER];
  block_topk<PER, NT>(key, id, (uint32_t)kt, token_idx + (int64_t)p * kt, kt, sh, stage);
}

// More candidates than one workgroup holds (16384): an exact top-k in passes.
// Pass 1 keeps the top-Kt' of every chunk of kTopkChunk candidates, as (key,
// token) lists in candidate order; each later pass does the same over chunks
// of the concatenated lists, until one chunk remains, whose selection is the
// result. A chunk's selection is in element order and chunks follow each
// other, so the lists stay in token order and the lower-index tie rule holds
// across passes. With Kt' <= kTopkChunk / 2 every pass at least halves the list.

template <int PER, int NT>
__global__ __launch_bounds__(NT) void k_topk_tokens_chunk(const float* __restrict__ A,
                                                          const int32_t* __restrict__ block_idx,
                                                          uint32_t* __restrict__ okey, int32_t* __restrict__ oid,
                                                          int64_t ostride, int64_t N, int bs, int bsh, int kb, int kt) {
  __shared__ TopkLds<NT> sh;
  const int ch = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  const int ncand = kb * bs, c0 = ch * kTopkChunk, n = min(kTopkChunk, ncand - c0);
  const int32_t* bidx = block_idx + (int64_t)p * kb;
  float v[PER];
  load_row_f32<PER>(A + (int64_t)p * ncand + c0, n, tid * PER, v);
  int bq[PER], bid[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = c0 + min(tid * PER + e, n - 1);
    bq[e] = bsh >= 0 ? (c >> bsh) : c / bs;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) bid[e] = bidx[bq[e]];
  uint32_t key[PER];
  int32_t id[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = c0 + tid * PER + e;
    const int64_t t = (int64_t)bid[e] * bs + (c - bq[e] * bs);
    const bool ok = tid * PER + e < n && t >= 0 && t < N;
    key[e] = ok ? order_key(v[e]) : 0u;
    id[e] = ok ? (int32_t)t : -1;
  }
  const int64_t o = (int64_t)p * ostride + (int64_t)ch * kt;
  __shared__ uint32_t stage[NT * PER];
  block_topk<PER, NT>(key, id, (uint32_t)kt, oid + o, kt, sh, stage, okey + o);
}

// A later pass: chunk blockIdx.x of the (key, id) list of pair blockIdx.y.
// okey == NULL: the last pass, writing the result.
template <int PER, int NT>
__global__ __launch_bounds__(NT) void k_topk_lists(const uint32_t* __restrict__ ikey,
                                                   const int32_t* __restrict__ iid, int64_t istride, int64_t n_in,
                                                   uint32_t* __restrict__ okey, int32_t* __restrict__ oid,
                                                   int64_t ostride, int kt) {
  __shared__ TopkLds<NT> sh;
  const int ch = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  const int64_t c0 = (int64_t)ch * kTopkChunk;
  uint32_t key[PER];
  int32_t id[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int64_t i = c0 + tid * PER + e;
    const bool ok = tid * PER + e < kTopkChunk && i < n_in;
    const int64_t j = (int64_t)p * istride + (ok ? i : 0);
    key[e] = ok ? ikey[j] : 0u;
    id[e] = ok ? iid[j] : -1;
  }
  const int64_t o = (int64_t)p * ostride + (int64_t)ch * kt;
  __shared__ uint32_t stage[NT * PER];
  block_topk<PER, NT>(key, id, (uint32_t)kt, oid + o, kt, sh, stage, okey ? okey + o : nullptr);
}

static int log2_or_neg(int bs) { return (bs & (bs - 1)) == 0 ? __builtin_ctz((unsigned)bs) : -1; }
// Workgroup size for a row of n keys: the fewest threads with at most 8 keys
// each (up to 16 with 1024 threads). Measured on the 128k workload: 2048
// block scores 5.1 us on 256 threads vs 5.4 on 1024; 8192 candidates 9.2 us
// on 1024 vs 9.8 on 512; 4096 candidates (the 32k and 64k latent steps) on
// 1024 threads made those steps 0.3-1 us slower than on 512.
static int topk_threads(int n) { return n <= 256 * 8 ? 256 : n <= 512 * 8 ? 512 : 1024; }
#define TLS_PER_SWITCH(per, NT, MACRO) \
  if (per <= 1) MACRO(1, NT);          \
  else if (per <= 2) MACRO(2, NT);     \
  else if (per <= 4) MACRO(4, NT);     \
  else if (per <= 8) MACRO(8, NT);     \
  else if (per <= 16) MACRO(16, NT);   \
  else return hipErrorInvalidValue;
#define TLS_NT_SWITCH(n, MACRO)                                  \
  {                                                              \
    const int nt_ = topk_threads(n), per_ = (n + nt_ - 1) / nt_; \
    if (nt_ == 256) {                                            \
      TLS_PER_SWITCH(per_, 256, MACRO)                           \
    } else if (nt_ == 512) {                                     \
      TLS_PER_SWITCH(per_, 512, MACRO)                           \
    } else {                                                     \
      TLS_PER_SWITCH(per_, 1024, MACRO)                          \
    }                                                            \
  }

hipError_t launch_topk_blocks(const float* S, int rows, int n, int K, int32_t* out, hipStream_t st) {
#define TLS_GO(P, NT) hipLaunchKernelGGL((k_topk_blocks<P, NT>), dim3(rows), dim3(NT), 0, st, S, n, K, out)
  TLS_NT_SWITCH(n, TLS_GO)
#undef TLS_GO
  return hipGetLastError();
}


// The folded token scores apply: up to 8 heads (one head tile), 8 or 16
// label channels, blocks of 64, and per-pair codes and scales that a buffer
// resource spans.
template <int MT, int RB>
static bool fold_ok(const TokenSelectArgs& a) {
  if constexpr (MT == 1 && (RB == 4 || RB == 8))
    return a.G <= 8 && a.bs == 64 && a.Ns <= (int64_t)0x7FFFFFFF / 4;
  else
    return false;
}

template <int MT, int RB, int UT>
static void go_score_tokens_ut(const TokenSelectArgs& a, float* A, hipStream_t st) {
  const int ncand = a.kb * a.bs;
  dim3 grid((unsigned)((ncand + 64 * UT - 1) / (64 * UT)), (unsigned)a.pairs);
#define TLS_GO(F)                                                                                                 \
  hipLaunchKernelGGL((k_score_tokens<MT, RB, UT, F>), grid, dim3(256), 0, st, a.q, a.label_ch, a.codes, a.scale, \
                     a.block_idx, A, a.Hq, a.Hkv, a.G, a.D, a.N, a.Ns, a.bs, log2_or_neg(a.bs), a.r, a.kb)
  if constexpr (MT == 1 && (RB == 4 || RB == 8)) {
    if (fold_ok<MT, RB>(a)) {
      TLS_GO(true);
      return;
    }
  }
  TLS_GO(false);
#undef TLS_GO
}

// Units of 16 tiles for few head tiles (the unit's loads are its latency);
// units of 4 tiles for many (8 MFMAs per tile: 64-candidate units put four
// times the waves on the chip, 12.7 vs 20.1 us for 128 heads at 4096
// candidates per pair).
template <int MT, int RB>
static void go_score_tokens(const TokenSelectArgs& a, float* A, hipStream_t st) {
  if constexpr (MT >= 4)
    go_score_tokens_ut<MT, RB, 4>(a, A, st);
  else
    go_score_tokens_ut<MT, RB, 16>(a, A, st);
}

template <int MT>
static void go_score_tokens_rb(const TokenSelectArgs& a, float* A, hipStream_t st) {
  switch (a.r) {
    case 8: go_score_tokens<MT, 4>(a, A, st); break;
    case 16: go_score_tokens<MT, 8>(a, A, st); break;
    case 32: go_score_tokens<MT, 16>(a, A, st); break;
    default: go_score_tokens<MT, 0>(a, A, st); break;
  }
}

template <int MT, int RB, int UT>
static void go_score_tokens_sel_ut(const TokenSelectArgs& a, const float* S, int NB, int32_t* block_idx, float* A,
                                   hipStream_t st) {
  const int ncand = a.kb * a.bs;
  dim3 grid((unsigned)((ncand + 64 * UT - 1) / (64 * UT)), (unsigned)a.pairs);
#define TLS_GO(PB, F)                                                                                               \
  hipLaunchKernelGGL((k_score_tokens_sel<MT, RB, UT, PB, F, false>), grid, dim3(256), 0, st, a.q, a.label_ch,      \
                     a.codes, a.scale, S, nullptr, NB, (int64_t)0, block_idx, A, a.Hq, a.Hkv, a.G, a.D, a.N, a.Ns, a.bs, \
                     log2_or_neg(a.bs), a.r, a.kb)
  if constexpr (MT == 1 && (RB == 4 || RB == 8)) {
    if (fold_ok<MT, RB>(a)) {
      if (NB <= 256 * 8)
        TLS_GO(8, true);
      else
        TLS_GO(16, true);
      return;
    }
  }
  if (NB <= 256 * 8)
    TLS_GO(8, false);
  else
    TLS_GO(16, false);
#undef TLS_GO
}

template <int MT, int RB>
static void go_score_tokens_sel(const TokenSelectArgs& a, const float* S, int NB, int32_t* block_idx, float* A,
                                hipStream_t st) {
  if constexpr (MT >= 4) {
    go_score_tokens_sel_ut<MT, RB, 4>(a, S, NB, block_idx, A, st);
  } else {
    // 1024 candidates per workgroup, or 512 where that leaves CUs without a
    // workgroup (each workgroup selects the pair's blocks itself first)
    const int64_t wgs = (int64_t)((a.kb * a.bs + 1023) / 1024) * a.pairs;
    if (wgs < 256)
      go_score_tokens_sel_ut<MT, RB, 8>(a, S, NB, block_idx, A, st);
    else
      go_score_tokens_sel_ut<MT, RB, 16>(a, S, NB, block_idx, A, st);
  }
}

template <int MT>
static void go_score_tokens_sel_rb(const TokenSelectArgs& a, const float* S, int NB, int32_t* block_idx, float* A,
                                   hipStream_t st) {
  switch (a.r) {
    case 8: go_score_tokens_sel<MT, 4>(a, S, NB, block_idx, A, st); break;
    case 16: go_score_tokens_sel<MT, 8>(a, S, NB, block_idx, A, st); break;
    case 32: go_score_tokens_sel<MT, 16>(a, S, NB, block_idx, A, st); break;
    default: go_score_tokens_sel<MT, 0>(a, S, NB, block_idx, A, st); break;
  }
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t token_ws_bytes(int pairs, int64_t ncand, int kt) {
  const size_t scores = round256((size_t)pairs * ncand * sizeof(float));
  if (ncand <= kTopkChunk) return scores;
  if (ncand > kMaxTokenCandidates || kt > kTopkChunk / 2) return 0;
  const int64_t list = (ncand + kTopkChunk - 1) / kTopkChunk * kt;
  return scores + 4 * round256((size_t)pairs * list * 4);  // two (key, id) lists
}

static hipError_t launch_topk_tokens(const TokenSelectArgs& a, float* A, hipStream_t st);

hipError_t launch_select_tokens(const TokenSelectArgs& a, float* A, hipStream_t st) {
  switch ((a.G + 15) / 16) {
    case 1: go_score_tokens_rb<1>(a, A, st); break;
    case 2: go_score_tokens_rb<2>(a, A, st); break;
    case 3: go_score_tokens_rb<3>(a, A, st); break;
    case 4: go_score_tokens_rb<4>(a, A, st); break;
    case 5: go_score_tokens_rb<5>(a, A, st); break;
    case 6: go_score_tokens_rb<6>(a, A, st); break;
    case 7: go_score_tokens_rb<7>(a, A, st); break;
    case 8: go_score_tokens_rb<8>(a, A, st); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_topk_tokens(a, A, st);
}

bool select_fused_ok(int NB, int kb) { return NB <= kSelMaxBlocks && kb <= NB; }

hipError_t launch_select_fused(const TokenSelectArgs& a, const float* S, int NB, int32_t* block_idx, float* A,
                               hipStream_t st) {
  if (!select_fused_ok(NB, a.kb)) return hipErrorInvalidValue;
  switch ((a.G + 15) / 16) {
    case 1: go_score_tokens_sel_rb<1>(a, S, NB, block_idx, A, st); break;
    case 2: go_score_tokens_sel_rb<2>(a, S, NB, block_idx, A, st); break;
    case 3: go_score_tokens_sel_rb<3>(a, S, NB, block_idx, A, st); break;
    case 4: go_score_tokens_sel_rb<4>(a, S, NB, block_idx, A, st); break;
    case 5: go_score_tokens_sel_rb<5>(a, S, NB, block_idx, A, st); break;
    case 6: go_score_tokens_sel_rb<6>(a, S, NB, block_idx, A, st); break;
    case 7: go_score_tokens_sel_rb<7>(a, S, NB, block_idx, A, st); break;
    case 8: go_score_tokens_sel_rb<8>(a, S, NB, block_idx, A, st); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_topk_tokens(a, A, st);
}

bool select_scores_inside_ok(int G, int D, int NB, int kb) {
  return G <= 16 && D == 128 && NB <= kSelScoreMaxBlocks && kb <= NB;
}

template <int RB, int UT>
static void go_select_from_summaries(const TokenSelectArgs& a, const uint16_t* summ, int NB, int64_t NBs,
                                     int32_t* block_idx, float* A, hipStream_t st) {
  const int ncand = a.kb * a.bs;
  dim3 grid((unsigned)((ncand + 64 * UT - 1) / (64 * UT)), (unsigned)a.pairs);
#define TLS_GO(F)                                                                                                  \
  hipLaunchKernelGGL((k_score_tokens_sel<1, RB, UT, 8, F, true>), grid, dim3(256), 0, st, a.q, a.label_ch, a.codes, \
                     a.scale, nullptr, summ, NB, NBs, block_idx, A, a.Hq, a.Hkv, a.G, a.D, a.N, a.Ns, a.bs,         \
                     log2_or_neg(a.bs), a.r, a.kb)
  if constexpr (RB == 4 || RB == 8) {
    if (fold_ok<1, RB>(a)) {
      TLS_GO(true);
      return;
    }
  }
  TLS_GO(false);
#undef TLS_GO
}

template <int RB>
static void go_select_from_summaries_ut(const TokenSelectArgs& a, const uint16_t* summ, int NB, int64_t NBs,
                                        int32_t* block_idx, float* A, hipStream_t st) {
  // the unit size of go_score_tokens_sel for one head tile
  const int64_t wgs = (int64_t)((a.kb * a.bs + 1023) / 1024) * a.pairs;
  if (wgs < 256)
    go_select_from_summaries<RB, 8>(a, summ, NB, NBs, block_idx, A, st);
  else
    go_select_from_summaries<RB, 16>(a, summ, NB, NBs, block_idx, A, st);
}

hipError_t launch_select_from_summaries(const TokenSelectArgs& a, const uint16_t* summ, int NB, int64_t NBs,
                                        int32_t* block_idx, float* A, hipStream_t st) {
  if (!select_scores_inside_ok(a.G, a.D, NB, a.kb)) return hipErrorInvalidValue;
  switch (a.r) {
    case 8: go_select_from_summaries_ut<4>(a, summ, NB, NBs, block_idx, A, st); break;
    case 16: go_select_from_summaries_ut<8>(a, summ, NB, NBs, block_idx, A, st); break;
    case 32: go_select_from_summaries_ut<16>(a, summ, NB, NBs, block_idx, A, st); break;
    default: go_select_from_summaries_ut<0>(a, summ, NB, NBs, block_idx, A, st); break;
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_topk_tokens(a, A, st);
}

// The token top-k over the scores in A (one launch, or passes over chunks).
static hipError_t launch_topk_tokens(const TokenSelectArgs& a, float* A, hipStream_t st) {
  hipError_t e = hipSuccess;
  const int ncand = a.kb * a.bs;
  if (ncand <= kTopkChunk) {
#define TLS_GO(P, NT)                                                                                          \
  hipLaunchKernelGGL((k_topk_tokens<P, NT>), dim3(a.pairs), dim3(NT), 0, st, A, a.block_idx, a.token_idx, a.N, \
                     a.bs, log2_or_neg(a.bs), a.kb, a.kt)
    TLS_NT_SWITCH(ncand, TLS_GO)
#undef TLS_GO
    return hipGetLastError();
  }
  // passes over chunks (workspace: scores, then two (key, id) lists)
  constexpr int NT = kTopkThreads, PER = kTopkChunk / kTopkThreads;
  int64_t nch = (ncand + kTopkChunk - 1) / kTopkChunk;
  const int64_t list = nch * a.kt;
  const size_t lb = round256((size_t)a.pairs * list * 4);
  char* base = reinterpret_cast<char*>(A) + round256((size_t)a.pairs * ncand * sizeof(float));
  uint32_t* key[2] = {reinterpret_cast<uint32_t*>(base), reinterpret_cast<uint32_t*>(base + 2 * lb)};
  int32_t* id[2] = {reinterpret_cast<int32_t*>(base + lb), reinterpret_cast<int32_t*>(base + 3 * lb)};
  hipLaunchKernelGGL((k_topk_tokens_chunk<PER, NT>), dim3((unsigned)nch, (unsigned)a.pairs), dim3(NT), 0, st, A,
                     a.block_idx, key[0], id[0], list, a.N, a.bs, log2_or_neg(a.bs), a.kb, a.kt);
  e = hipGetLastError();
  int64_t n = list;
  int cur = 0;
  while (e == hipSuccess) {
    nch = (n + kTopkChunk - 1) / kTopkChunk;
    if (nch == 1) {  // the last pass writes the result
      hipLaunchKernelGGL((k_topk_lists<PER, NT>), dim3(1, (unsigned)a.pairs), dim3(NT), 0, st, key[cur], id[cur], list,
                         n, nullptr, a.token_idx, (int64_t)a.kt, a.kt);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((k_topk_lists<PER, NT>), dim3((unsigned)nch, (unsigned)a.pairs), dim3(NT), 0, st, key[cur],
                       id[cur], list, n, key[cur ^ 1], id[cur ^ 1], list, a.kt);
    e = hipGetLastError();
    n = nch * a.kt;
    cur ^= 1;
  }
  return e;
}

}  // namespace tls

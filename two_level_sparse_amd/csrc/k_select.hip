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

namespace tls {

// ----------------------------------------------------------- block scores --
// q+ and q- of one A fragment: per 16-bit half, sign set -> negative part.
__device__ __forceinline__ void split_sign(u32x4 raw, u32x4& pos, u32x4& neg) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t mask = ((raw[e] >> 15) & 0x00010001u) * 0xFFFFu;
    neg[e] = raw[e] & mask;
    pos[e] = raw[e] & ~mask;
  }
}

// Streaming scorer for small head groups (G <= 48): every summary byte is used
// by at most three 16-row MFMA tiles, so the kernel is a plain HBM stream.
// Each wave scores 16*NSUB consecutive blocks; the channel loop runs in groups
// of UNR chunks of 32 channels whose loads (summaries and q fragments) are all
// issued before the group's MFMAs. KC = D/32 when known at compile time (0:
// from D at run time, with UNR = 1).
template <int MT, int NSUB, int KC, int UNR>
__global__ __launch_bounds__(256) void k_score_blocks(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ summ, float* __restrict__ S,
                                                      int Hq, int Hkv, int G, int D, int64_t NB, int64_t NBs) {
  const int p = blockIdx.y;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t jbase = ((int64_t)blockIdx.x * 4 + wave) * (16 * NSUB);
  if (jbase >= NB) return;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  const uint16_t* sp = summ + (int64_t)p * NBs * 2 * D;

  const uint16_t* brow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int64_t j = jbase + s * 16 + n;
    brow[s] = sp + (j < NB ? j : NB - 1) * 2 * D;
  }
  const uint16_t* qrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) qrow[m] = qp + (int64_t)min(m * 16 + n, G - 1) * D;  // rows past G repeat G-1, unused
  f32x4 acc[MT][NSUB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunk = KC > 0 ? KC : D / 32;
  for (int cb = 0; cb < nchunk; cb += UNR) {
    u32x4 kmx[UNR][NSUB], kmn[UNR][NSUB], qr[UNR][MT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int off = (cb + u) * 32 + 8 * kq;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        kmx[u][s] = ld16(brow[s] + off);
        kmn[u][s] = ld16(brow[s] + D + off);
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
    float best = -INFINITY;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m * 16 + 4 * kq + i < G) best = fmaxf(best, acc[m][s][i]);
    best = max_rows(best);
    const int64_t j = jbase + s * 16 + n;
    if (kq == 0 && j < NB) S[(int64_t)p * NB + j] = best;
  }
}

// LDS-staged scorer for large head groups (G > 48, e.g. MLA's 128 heads on
// one latent kv head): a GEMM with M = G heads, N = blocks, K = 2*D. A
// workgroup of 8 waves scores kLdsTiles tiles of 16 consecutive blocks of one
// pair. Wave w takes head tiles 2*(w&3), 2*(w&3)+1 and one half of the
// channel chunks (w>>2), whose q fragments it keeps in registers; the two
// halves' sums meet in LDS. The summaries of all the workgroup's tiles go to
// LDS with direct global->LDS 16-byte loads, laid out as B fragments (piece
// (chunk, max|min) = 64 lanes x 16 bytes, read back conflict-free), and are
// read by the 4 waves that share a channel half. q is loaded once per
// workgroup for kLdsTiles tiles of summaries.
constexpr int kLdsTiles = 4;
constexpr int kLdsWaves = 8;

template <int MT, int KC>
__global__ __launch_bounds__(kLdsWaves * 64) void k_score_blocks_lds(const uint16_t* __restrict__ q,
                                                                     const uint16_t* __restrict__ summ,
                                                                     float* __restrict__ S, int Hq, int Hkv, int G,
                                                                     int64_t NB, int64_t NBs) {
  constexpr int D = KC * 32;
  constexpr int MW = 2;                 // head tiles per wave
  constexpr int KH = KC / 2;            // channel chunks per wave
  constexpr int PIECES = 2 * KC;        // per tile
  constexpr int PPW = (PIECES + kLdsWaves - 1) / kLdsWaves;
  constexpr int CG = KH % 3 == 0 ? 3 : KH % 2 == 0 ? 2 : 1;  // chunks per group of LDS reads
  static_assert(MT <= 8 && KC % 2 == 0 && kLdsTiles == 4, "tile layout");
  // tiles 0-1 and 2-3 in two LDS objects, so that reading tiles 0-1 does not
  // wait for the loads of tiles 2-3
  __shared__ u32x4 btA[2][PIECES][64], btB[2][PIECES][64];
  __shared__ float part[kLdsTiles][4][16];
  // after the products: the second channel half's sums, [tile][head-tile pair][MW][lane],
  // in btA when it is large enough
  constexpr int HALF = kLdsTiles * 4 * MW * 64;
  constexpr bool kAlias = 2 * PIECES * 64 >= HALF;
  __shared__ f32x4 half_own[kAlias ? 1 : HALF];
  f32x4* half1 = kAlias ? reinterpret_cast<f32x4*>(&btA[0][0][0]) : half_own;
  auto bt = [&](int t) -> u32x4(*)[64] { return t < 2 ? btA[t] : btB[t - 2]; };
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
  // and are not stored.
  const int64_t t0 = (int64_t)tg * kLdsTiles;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  const uint16_t* sp = summ + (int64_t)p * NBs * 2 * D;

  // Direct loads of tiles [ta, tb): wave w issues pieces w, w+8, ...
  auto issue = [&](int ta, int tb) {
#pragma unroll
    for (int t = ta; t < tb; ++t) {
      const int64_t j = min((t0 + t) * 16 + n, NB - 1);
      const uint16_t* src = sp + j * 2 * D + 8 * kq;
#pragma unroll
      for (int k = 0; k < PPW; ++k) {
        const int pc = wave + kLdsWaves * k;
        if (pc < PIECES)
          __builtin_amdgcn_global_load_lds(
              (__attribute__((address_space(1))) void*)(src + (pc & 1) * D + (pc >> 1) * 32),
              (__attribute__((address_space(3))) void*)&bt(t)[pc][0], 16, 0, 0);
      }
    }
  };
  // Tiles 0 and 1 first, then the q fragments (rows past G repeat row G-1;
  // their products are left out of the maxima), split once into q+ / q-.
  // Waiting for q also waits for those two tiles; tiles 2 and 3 are issued
  // after it and land while tiles 0 and 1 are multiplied.
  issue(0, 2);
  u32x4 qpos[MW][KH], qneg[MW][KH];
  {
    u32x4 raw[MW][KH];
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const uint16_t* qr = qp + (int64_t)min((2 * hp + i) * 16 + n, G - 1) * D + 8 * kq + kh * KH * 32;
#pragma unroll
      for (int c = 0; c < KH; ++c) raw[i][c] = ld16(qr + c * 32);
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int c = 0; c < KH; ++c) split_sign(raw[i][c], qpos[i][c], qneg[i][c]);
  }
  __builtin_amdgcn_sched_barrier(0);
  issue(2, kLdsTiles);
  // tiles 0 and 1 are in LDS for every wave: a barrier without a memory fence
  // (a fence would wait for tiles 2 and 3 as well)
  __asm__ volatile("s_barrier" ::: "memory");

  f32x4 tot[kLdsTiles][MW];
  auto product = [&](int t) {
    // four independent accumulation chains per head tile (q+ / q- terms of
    // even / odd chunks), so that consecutive MFMAs do not wait on each other
    f32x4 acc[MW][4];
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[i][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cg = 0; cg < KH; cg += CG) {
      u32x4 bmx[CG], bmn[CG];
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const int c = kh * KH + cg + u;
        bmx[u] = bt(t)[2 * c][lane];
        bmn[u] = bt(t)[2 * c + 1][lane];
      }
#pragma unroll
      for (int u = 0; u < CG; ++u) {
#pragma unroll
        for (int i = 0; i < MW; ++i) {
          {
            const int a = 2 * (u & 1);
            acc[i][a] = mfma16x16x32(qpos[i][cg + u], bmx[u], acc[i][a]);
            acc[i][a + 1] = mfma16x16x32(qneg[i][cg + u], bmn[u], acc[i][a + 1]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MW; ++i) tot[t][i] = (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
  };
  product(0);
  product(1);
  wait_vmcnt<0>();
  __asm__ volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int t = 2; t < kLdsTiles; ++t) product(t);
  // the second channel half hands its sums to the first (through the tile
  // buffer, once every wave is done reading it)
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t)
#pragma unroll
      for (int i = 0; i < MW; ++i) half1[((t * 4 + hp) * MW + i) * 64 + lane] = tot[t][i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < kLdsTiles; ++t) {
      float best = -INFINITY;
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        const f32x4 sum = tot[t][i] + half1[((t * 4 + hp) * MW + i) * 64 + lane];
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

// ------------------------------------------------------------------ top-k --
// Exact top-k of one row per workgroup of NT threads (256, 512 or 1024);
// keys in registers, thread t owning elements [t*PER, t*PER+PER). Invalid
// elements carry key 0, below every valid key.
constexpr int kTopkThreads = 1024;  // the largest workgroup: 16 keys per thread up to 16384
constexpr int kTopkChunk = 16384;   // the most keys one workgroup selects from

template <int NT>
struct alignas(16) TopkLds {
  uint32_t hist[3][256];  // pass i counts into hist[i % 3]
  uint32_t red[3][NT / 64];
  uint32_t scan[NT / 64];
};

// Block-wide exclusive scan of one uint32 per thread; returns the prefix.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh /* one per wave */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sh[wave] = x;
  lds_sync();
  uint32_t before = 0u;
  for (int w = 0; w < wave; ++w) before += sh[w];
  return before + x - v;
}

// The bin of a 256-bin histogram that holds the krem-th largest key: every
// wave reads the whole histogram and finds it on its own (wave-uniform
// results, no LDS round trip). Lane l holds bins 255-4l .. 252-4l, so an
// exclusive prefix scan over lanes counts the keys in the bins above.
struct BinPick {
  uint32_t bin, above, count;
};
__device__ __forceinline__ BinPick pick_bin(const uint32_t* hist, uint32_t krem) {
  const int lane = threadIdx.x & 63;
  const int b0 = 252 - 4 * lane;
  const u32x4 hb = *reinterpret_cast<const u32x4*>(&hist[b0]);
  const uint32_t mine = hb[0] + hb[1] + hb[2] + hb[3];
  const uint32_t above = wave_incl_scan(mine) - mine;
  const uint64_t hit = __ballot(above < krem && krem <= above + mine);
  const int L = __builtin_ctzll(hit);  // the lane whose 4 bins hold it (one exists: krem <= keys in range)
  uint32_t bin = 0u, ab = 0u, cnt = 0u, run = above;
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (run < krem && krem <= run + hb[i]) {  // true for exactly one bin of lane L
      bin = (uint32_t)(b0 + i);
      ab = run;
      cnt = hb[i];
    }
    run += hb[i];
  }
  return BinPick{readlane(bin, L), readlane(ab, L), readlane(cnt, L)};
}

// Selects the K largest keys (ties: lower element index first) and writes
// their ids ascending to out[0..min(K, valid)), then -1 up to out_len.
// Radix select. The first pass bins the keys' float values linearly between
// the smallest and the largest (a monotone map, so a bin holds one interval
// of keys; binning the raw keys instead would put every float of one binade
// into a single bin). The later passes histogram (key - lo) >> shift, the next
// 8 bits below the top set bit of (hi - lo), over the keys left in [lo, hi].
// The search stops as soon as the chosen bin is taken whole, with the
// threshold at the bin's lower edge and every key equal to it kept. One
// barrier per pass: the histograms rotate over three buffers (a buffer is
// cleared two passes after its last read), and every wave picks the bin.
template <int PER, int NT>
__device__ void block_topk(const uint32_t (&key)[PER], const int32_t (&id)[PER], uint32_t K, int32_t* out,
                           int out_len, TopkLds<NT>& sh, uint32_t* out_key = nullptr) {
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nval = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (key[e] != 0u) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
      ++nval;
    }
  kmin = wave_umin(kmin);
  kmax = wave_umax(kmax);
  nval = wave_usum(nval);
  if (lane == 0) {
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
    sh.red[2][wave] = nval;
  }
  for (int i = tid; i < 512; i += NT) sh.hist[i >> 8][i & 255] = 0u;  // buffers 0 and 1
  lds_sync();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, total = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    lo = min(lo, sh.red[0][w]);
    hi = max(hi, sh.red[1][w]);
    total += sh.red[2][w];
  }
  const uint32_t kk = K < total ? K : total;
  uint32_t thr = 0u, krem = 0u;  // kk == total: keep every valid element
  if (kk < total) {
    krem = kk;
    bool done = false;
    int pass = 0;  // histogram buffer = pass % 3; pass p clears buffer (p + 1) % 3
    const float vlo = key_float(lo), vhi = key_float(hi);
    const float sc = 256.0f / (vhi - vlo);
    if (hi > lo && sc > 0.0f && sc < INFINITY) {
      uint32_t bin[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float x = key[e] != 0u ? (key_float(key[e]) - vlo) * sc : 0.0f;  // in [0, 256]
        bin[e] = min((uint32_t)x, 255u);
        if (key[e] != 0u) atomicAdd(&sh.hist[0][bin[e]], 1u);
      }
      if (tid < 256) sh.hist[2][tid] = 0u;  // (buffer 1 was cleared at the start)
      lds_sync();
      const BinPick pk = pick_bin(sh.hist[0], krem);
      pass = 1;
      const uint32_t d = pk.bin;
      krem -= pk.above;
      // keys of bin d: one interval [lo, hi] (a block reduction; its barrier
      // also orders this pass's histogram reads before buffer 0 is cleared)
      kmin = 0xFFFFFFFFu;
      kmax = 0u;
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (key[e] != 0u && bin[e] == d) {
          kmin = min(kmin, key[e]);
          kmax = max(kmax, key[e]);
        }
      kmin = wave_umin(kmin);
      kmax = wave_umax(kmax);
      if (lane == 0) {
        sh.red[0][wave] = kmin;
        sh.red[1][wave] = kmax;
      }
      lds_sync();
      lo = 0xFFFFFFFFu;
      hi = 0u;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        lo = min(lo, sh.red[0][w]);
        hi = max(hi, sh.red[1][w]);
      }
      if (krem == pk.count) {
        // the whole bin is taken: the threshold is its smallest key
        thr = lo;
        krem = 0xFFFFFFFFu;
        done = true;
      }
    }
    while (!done && hi > lo) {
      const uint32_t diff = hi - lo;
      const int nbits = 32 - __clz(diff);
      const int shift = nbits > 8 ? nbits - 8 : 0;
      uint32_t* hcur = sh.hist[pass % 3];
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (key[e] >= lo && key[e] <= hi) atomicAdd(&hcur[(key[e] - lo) >> shift], 1u);
      if (tid < 256) sh.hist[(pass + 1) % 3][tid] = 0u;  // last read two barriers ago
      lds_sync();
      const BinPick pk = pick_bin(hcur, krem);
      ++pass;
      const uint32_t d = pk.bin;
      krem -= pk.above;
      const uint32_t nlo = lo + (d << shift);
      if (krem == pk.count) {
        // the whole bin is taken: every key in it is >= nlo and every key
        // of a lower bin is < nlo
        thr = nlo;
        krem = 0xFFFFFFFFu;
        done = true;
        break;
      }
      const uint32_t span = shift == 0 ? 0u : ((1u << shift) - 1u);
      hi = (hi - nlo) > span ? nlo + span : hi;
      lo = nlo;
    }
    if (!done) thr = lo;
  }
// Elements above the threshold, plus the first krem equal to it (index
// order), placed by one block-wide scan into an LDS row that goes out in
// coalesced stores (placing straight into global memory would scatter every
// store instruction over the wave's whole output range).
  __shared__ uint32_t stage[NT * PER];
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    gt += (key[e] > thr) ? 1u : 0u;
    eq += (key[e] == thr && key[e] != 0u) ? 1u : 0u;
  }
  const uint32_t pre = block_exclusive_scan(gt | (eq << 16), sh.scan);
  auto place = [&](bool ids) {
    uint32_t eq_before = pre >> 16;
    uint32_t pos = (pre & 0xFFFFu) + min(eq_before, krem);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      bool take = key[e] > thr;
      if (key[e] == thr && key[e] != 0u) {
        take = eq_before < krem;
        ++eq_before;
      }
      if (take) {
        if (pos < kk) stage[pos] = ids ? (uint32_t)id[e] : key[e];  // never more than kk entries
        ++pos;
      }
    }
  };
  place(true);
  lds_sync();
  for (int i = tid; i < out_len; i += NT) out[i] = i < (int)kk ? (int32_t)stage[i] : -1;
  if (out_key) {
    lds_sync();
    place(false);
    lds_sync();
    for (int i = tid; i < out_len; i += NT) out_key[i] = i < (int)kk ? stage[i] : 0u;  // key 0: no element
  }
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
  block_topk<PER, NT>(key, id, (uint32_t)K, out + (int64_t)row * K, K, sh);
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

// A fragments of q on the label channels, in two steps so that the gathers
// can be issued long before the fragments are needed. The workgroup of 256
// threads gathers the matrix of q on the label channels once (MT*16 rows x 32
// channel slots; rows past G repeat head G-1, so the maximum over all rows is
// the heads' maximum; slots past r are zero) and shares it through LDS: every
// wave needs all of it, and a wave gathering it alone makes MT*8 two-byte
// loads per lane at 64 scattered addresses each (for 128 heads the gathers
// alone kept a wave busy for about 6 us). Thread t gathers slot t%32 of rows
// t/32 + 8k (label_q_issue, into registers); label_q_finish writes them to
// LDS and reads the fragments back with one 16-byte read per tile from rows
// of 80 bytes (16 rows at distinct bank offsets).
// Plain form: lane (n, kq) of tile m holds head m*16 + n on channels 8kq ..
// 8kq+7. Folded form (G <= 8, one tile): lane (n, kq) holds head n&7 of half
// n>>3 on k = 8kq .. 8kq+7; half 0 takes channels 0-15 on k 0-15 and half 1
// the same channels on k 16-31, the other quarter of each row is zero.
constexpr int kLabRow = 40;  // uint16 per LDS row: 32 channels and 16 bytes of padding

template <int MT>
__device__ __forceinline__ void label_q_issue(uint32_t (&hl)[2 * MT], const int32_t* lab, const uint16_t* qp, int G,
                                              int D, int r) {
  const int t = threadIdx.x, i = t & 31;
  const int li = lab[min(i, r - 1)];
#pragma unroll
  for (int k = 0; k < 2 * MT; ++k) hl[k] = qp[(int64_t)min((t >> 5) + 8 * k, G - 1) * D + li];
}

template <int MT, bool FOLD>
__device__ __forceinline__ void label_q_finish(u32x4 (&qa)[MT], const uint32_t (&hl)[2 * MT], uint16_t* sq, int r) {
  const int t = threadIdx.x, i = t & 31;
  const int lane = t & 63, n = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int k = 0; k < 2 * MT; ++k) sq[((t >> 5) + 8 * k) * kLabRow + i] = i < r ? (uint16_t)hl[k] : (uint16_t)0;
  lds_sync();
  if constexpr (FOLD) {
    static_assert(MT == 1, "folded scores: one head tile");
    const u32x4 v = *reinterpret_cast<const u32x4*>(&sq[(n & 7) * kLabRow + 8 * (kq & 1)]);
    const bool mine = (kq >> 1) == (n >> 3);
    qa[0] = mine ? v : u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m) qa[m] = *reinterpret_cast<const u32x4*>(&sq[(m * 16 + n) * kLabRow + 8 * kq]);
  }
}

// Eight INT4 codes (one byte per channel pair, low nibble first) widened to
// bf16, exact: the B fragment of one lane.
__device__ __forceinline__ u32x4 codes_to_bf16(uint32_t w) {
  u32x4 bop;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int lo4 = (int)(w << (28 - 8 * e)) >> 28;  // channel 2e of the word
    const int hi4 = (int)(w << (24 - 8 * e)) >> 28;  // channel 2e + 1
    bop[e] = (__float_as_uint((float)lo4) >> 16) | (__float_as_uint((float)hi4) & 0xFFFF0000u);
  }
  return bop;
}

// ---- folded scores: up to 8 heads on 8 or 16 label channels, blocks of 64 ----
// One 16x16x32 MFMA carries two tiles of 16 candidates: rows 0-7 are the
// heads on k 0-15 (tile X's channels), rows 8-15 the same heads on k 16-31
// (tile Y's); B holds tile X's codes on k 0-15 and tile Y's on k 16-31.
// With G <= 8 and r <= 16 none of the product is padding, so every lane
// unpacks codes that count (a plain tile leaves half of k and half of the
// rows empty, and its lanes unpack zeros). A group of 64 candidates is one
// whole block: its codes and scales sit at a block-uniform offset (scalar)
// plus a per-lane constant, so the loads need no per-candidate address
// arithmetic. Rows past G repeat head G-1, which leaves every maximum as it is.
// NG groups of 64 candidates from candidate c0 (a multiple of 64): val[g] is
// the score of candidate cand[g] (0 if it does not exist). Lane (n, kq) ends
// with tile 2(kq&1) + (kq>>1) of its group: the MFMA of tiles 0/1 leaves
// tile 0 on rows 0-1 and tile 1 on rows 2-3, the one of tiles 2/3 likewise,
// and one 16-lane swap of the two (odd rows of the first with even rows of the
// second) pairs each tile's two row halves. `bidx` is the pair's block list.
template <int RB, int NG>
__device__ __forceinline__ void fold_unit(float (&val)[NG], int (&cand)[NG], const int32_t* bidx,
                                          __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr, int c0, int kb,
                                          int64_t N, u32x4 qa) {
  const int lane = threadIdx.x & 63, n = lane & 15, kq = lane >> 4;
  const int tile = 2 * (kq & 1) + (kq >> 1);
  const int voff = (n + 16 * (kq >> 1)) * RB + 4 * (kq & 1);  // tiles 0/1; +32 rows for tiles 2/3
  uint32_t cwa[NG], cwb[NG];
  float tsc[NG];
  int tok0[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int blk = c0 / 64 + g;
    tok0[g] = __builtin_amdgcn_readfirstlane(blk < kb ? bidx[blk] : 0) * 64;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    cwa[g] = __builtin_amdgcn_raw_buffer_load_b32(cr, voff, tok0[g] * RB, 0);
    cwb[g] = __builtin_amdgcn_raw_buffer_load_b32(cr, voff + 32 * RB, tok0[g] * RB, 0);
    tsc[g] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, (16 * tile + n) * 4, tok0[g] * 4, 0));
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const f32x4 a = mfma16x16x32(qa, codes_to_bf16(cwa[g]), f32x4{0.f, 0.f, 0.f, 0.f});
    const f32x4 c = mfma16x16x32(qa, codes_to_bf16(cwb[g]), f32x4{0.f, 0.f, 0.f, 0.f});
    const float xa = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
    const float xc = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(xa), __float_as_uint(xc), false, false);
    const float best = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const int within = 16 * tile + n;
    const bool ok = c0 / 64 + g < kb && (int64_t)tok0[g] + within < N;
    val[g] = ok ? tsc[g] * best : 0.0f;
    cand[g] = c0 + 64 * g + within;
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

template <int MT, int RB, int UT, bool FOLD>
__global__ __launch_bounds__(256) void k_score_tokens(const uint16_t* __restrict__ q,
                                                      const int32_t* __restrict__ label_ch,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale,
                                                      const int32_t* __restrict__ block_idx, float* __restrict__ A,
                                                      int Hq, int Hkv, int G, int D, int64_t N, int64_t Ns, int bs,
                                                      int bsh, int r, int kb) {
  const int p = blockIdx.y;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6;
  const int ncand = kb * bs, rb = r / 2;
  const int c0 = blockIdx.x * (4 * UT * 16) + wave * (UT * 16);
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

template <int MT, int RB, int UT, int PERB, bool FOLD>
__global__ __launch_bounds__(256) void k_score_tokens_sel(const uint16_t* __restrict__ q,
                                                          const int32_t* __restrict__ label_ch,
                                                          const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ S, int NB,
                                                          int32_t* __restrict__ block_idx, float* __restrict__ A,
                                                          int Hq, int Hkv, int G, int D, int64_t N, int64_t Ns, int bs,
                                                          int bsh, int r, int kb) {
  __shared__ TopkLds<256> sh;
  __shared__ int32_t sblk[kSelMaxBlocks];
  const int p = blockIdx.y, tid = threadIdx.x;
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
    load_row_f32<PERB>(S + (int64_t)p * NB, NB, tid * per, v);
    const int32_t* lab = label_ch + (int64_t)h * r;
    const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
    label_q_issue<MT>(hl, lab, qp, G, D, r);
    uint32_t key[PERB];
    int32_t id[PERB];
#pragma unroll
    for (int e = 0; e < PERB; ++e) {
      const int c = tid * per + e;
      id[e] = c;
      key[e] = (e < per && c < NB) ? order_key(v[e]) : 0u;
    }
    block_topk<PERB, 256>(key, id, (uint32_t)kb, sblk, kb, sh);
  }
  lds_sync();
  if (blockIdx.x == 0)
    for (int i = tid; i < kb; i += 256) block_idx[(int64_t)p * kb + i] = sblk[i];
  const int c0 = blockIdx.x * (4 * UT * 16) + wave * (UT * 16);
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
#pragma unroll
  for (int e = 0; e < PER; ++e) bid[e] = bidx[bq[e]];
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
  block_topk<PER, NT>(key, id, (uint32_t)kt, token_idx + (int64_t)p * kt, kt, sh);
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
  block_topk<PER, NT>(key, id, (uint32_t)kt, oid + o, kt, sh, okey + o);
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
  block_topk<PER, NT>(key, id, (uint32_t)kt, oid + o, kt, sh, okey ? okey + o : nullptr);
}

static int log2_or_neg(int bs) { return (bs & (bs - 1)) == 0 ? __builtin_ctz((unsigned)bs) : -1; }
// Workgroup size for a row of n keys: the fewest threads with at most 8 keys
// each (up to 16 with 1024 threads). Measured on the 128k workload: 2048
// block scores 5.1 us on 256 threads vs 5.4 on 1024; 8192 candidates 9.2 us
// on 1024 vs 9.8 on 512.
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
  hipLaunchKernelGGL((k_score_tokens_sel<MT, RB, UT, PB, F>), grid, dim3(256), 0, st, a.q, a.label_ch, a.codes,    \
                     a.scale, S, NB, block_idx, A, a.Hq, a.Hkv, a.G, a.D, a.N, a.Ns, a.bs, log2_or_neg(a.bs), a.r, \
                     a.kb)
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
  if constexpr (MT >= 4)
    go_score_tokens_sel_ut<MT, RB, 4>(a, S, NB, block_idx, A, st);
  else
    go_score_tokens_sel_ut<MT, RB, 16>(a, S, NB, block_idx, A, st);
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

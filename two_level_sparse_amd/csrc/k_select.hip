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
// k_topk is an exact radix select over order-preserving 32-bit keys of the
// scores, run by one 1024-thread workgroup per row. The digit width adapts to
// the key range (histograms of (key - lo) >> shift with 256 bins), so keys that
// share their upper bits do not pile into one bin. Elements equal to the
// threshold key are taken in index order, which realises the lower-index tie
// rule; the output is written ascending via one block-wide scan.
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {

// ----------------------------------------------------------- block scores --
template <int MT, int NSUB>
__global__ __launch_bounds__(256) void k_score_blocks(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ summ, float* __restrict__ S,
                                                      int Hq, int Hkv, int G, int D, int64_t NB) {
  const int p = blockIdx.y;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t jbase = ((int64_t)blockIdx.x * 4 + wave) * (16 * NSUB);
  if (jbase >= NB) return;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  const uint16_t* sp = summ + (int64_t)p * NB * 2 * D;

  const uint16_t* brow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    int64_t j = jbase + s * 16 + n;
    brow[s] = sp + (j < NB ? j : NB - 1) * 2 * D;
  }
  f32x4 acc[MT][NSUB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < D; c0 += 32) {
    const int off = c0 + 8 * kq;
    u32x4 kmx[NSUB], kmn[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      kmx[s] = ld16(brow[s] + off);
      kmn[s] = ld16(brow[s] + D + off);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int g = m * 16 + n;
      u32x4 raw = g < G ? ld16(qp + (int64_t)g * D + off) : u32x4{0u, 0u, 0u, 0u};
      u32x4 pos, neg;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // per 16-bit half: sign set -> negative part, else positive part
        uint32_t sgn = (raw[e] >> 15) & 0x00010001u;
        uint32_t mask = sgn * 0xFFFFu;
        neg[e] = raw[e] & mask;
        pos[e] = raw[e] & ~mask;
      }
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        acc[m][s] = mfma16x16x32(pos, kmx[s], acc[m][s]);
        acc[m][s] = mfma16x16x32(neg, kmn[s], acc[m][s]);
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
    best = fmaxf(best, __shfl_xor(best, 16, 64));
    best = fmaxf(best, __shfl_xor(best, 32, 64));
    const int64_t j = jbase + s * 16 + n;
    if (kq == 0 && j < NB) S[(int64_t)p * NB + j] = best;
  }
}

template <int MT, int NSUB>
static void go_blocks(const BlockScoreArgs& a, hipStream_t st) {
  const int64_t per_wg = 4 * 16 * NSUB;
  dim3 grid((unsigned)((a.NB + per_wg - 1) / per_wg), (unsigned)a.pairs);
  hipLaunchKernelGGL((k_score_blocks<MT, NSUB>), grid, dim3(256), 0, st, a.q, a.summ, a.S, a.Hq, a.Hkv, a.G, a.D,
                     a.NB);
}

hipError_t launch_score_blocks(const BlockScoreArgs& a, hipStream_t st) {
  const int mt = (a.G + 15) / 16;
  switch (mt) {
    case 1: go_blocks<1, 2>(a, st); break;
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

// ----------------------------------------------------------- token scores --
// One thread per candidate. The label-channel query values of the G heads sit
// in LDS (read as broadcasts); the candidate's packed codes are one 8- or
// 16-byte load.
template <int RMAX>
__global__ __launch_bounds__(256) void k_score_tokens(const uint16_t* __restrict__ q,
                                                      const int32_t* __restrict__ label_ch,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale,
                                                      const int32_t* __restrict__ block_idx, float* __restrict__ A,
                                                      int Hq, int Hkv, int G, int D, int64_t N, int bs, int r,
                                                      int kb) {
  __shared__ float ql[128 * RMAX];
  const int p = blockIdx.y;
  const int b = p / Hkv, h = p % Hkv;
  const int32_t* lab = label_ch + (int64_t)h * r;
  const uint16_t* qp = q + ((int64_t)b * Hq + (int64_t)h * G) * D;
  for (int e = threadIdx.x; e < G * RMAX; e += blockDim.x) {
    const int g = e / RMAX, i = e % RMAX;
    ql[e] = i < r ? bf2f(qp[(int64_t)g * D + lab[i]]) : 0.0f;
  }
  __syncthreads();
  const int ncand = kb * bs;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= ncand) return;
  const int64_t t = (int64_t)block_idx[(int64_t)p * kb + c / bs] * bs + c % bs;
  float outv = -INFINITY;
  if (t >= 0 && t < N) {
    const uint8_t* cp = codes + ((int64_t)p * N + t) * (r / 2);
    float cv[RMAX];
#pragma unroll
    for (int i = 0; i < RMAX; i += 2) {
      uint32_t byte = i < r ? cp[i / 2] : 0u;
      cv[i] = (float)((int32_t)(byte << 28) >> 28);
      cv[i + 1] = (float)((int32_t)(byte << 24) >> 28);
    }
    float best = -INFINITY;
    for (int g = 0; g < G; ++g) {
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < RMAX; ++i) dot = fmaf(ql[g * RMAX + i], cv[i], dot);
      best = fmaxf(best, dot);
    }
    outv = scale[(int64_t)p * N + t] * best;
  }
  A[(int64_t)p * ncand + c] = outv;
}

hipError_t launch_score_tokens(const TokenScoreArgs& a, hipStream_t st) {
  const int ncand = a.kb * a.bs;
  dim3 grid((unsigned)((ncand + 255) / 256), (unsigned)a.pairs);
  if (a.r <= 16)
    hipLaunchKernelGGL(k_score_tokens<16>, grid, dim3(256), 0, st, a.q, a.label_ch, a.codes, a.scale, a.block_idx,
                       a.A, a.Hq, a.Hkv, a.G, a.D, a.N, a.bs, a.r, a.kb);
  else
    hipLaunchKernelGGL(k_score_tokens<32>, grid, dim3(256), 0, st, a.q, a.label_ch, a.codes, a.scale, a.block_idx,
                       a.A, a.Hq, a.Hkv, a.G, a.D, a.N, a.bs, a.r, a.kb);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k --
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Block-wide exclusive scan of one uint32 per thread; returns the prefix.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh /* kTopkWaves+1 */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      uint32_t t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[kTopkWaves] = run;
  }
  __syncthreads();
  return sh[wave] + x - v;
}

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ scores, int n, int K,
                                                        const int32_t* __restrict__ block_idx, int kb, int bs,
                                                        int64_t N, int32_t* __restrict__ out, int out_len) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t red[3][kTopkWaves];
  __shared__ uint32_t scan_sh[kTopkWaves + 1];
  __shared__ uint32_t sel[2];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* sc = scores + (int64_t)row * n;

  uint32_t key[PER];
  int32_t id[PER];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nval = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = tid * PER + e;
    key[e] = 0u;
    id[e] = c;
    if (c < n) {
      bool valid = true;
      if (block_idx) {
        const int64_t t = (int64_t)block_idx[(int64_t)row * kb + c / bs] * bs + c % bs;
        valid = t >= 0 && t < N;
        id[e] = (int32_t)t;
      }
      if (valid) {
        key[e] = order_key(sc[c]);
        kmin = min(kmin, key[e]);
        kmax = max(kmax, key[e]);
        ++nval;
      }
    }
  }
  // block-wide min / max / count of the valid keys
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o, 64));
    nval += __shfl_xor(nval, o, 64);
  }
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
    red[2][wave] = nval;
  }
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, total = 0u;
  for (int w = 0; w < kTopkWaves; ++w) {
    lo = min(lo, red[0][w]);
    hi = max(hi, red[1][w]);
    total += red[2][w];
  }
  const uint32_t kk = (uint32_t)K < total ? (uint32_t)K : total;
  uint32_t thr, krem;
  if (kk == total) {  // keep every valid element
    thr = 0u;
    krem = 0u;
  } else {
    krem = kk;
    if (tid == 0) {
      sel[0] = 0u;
      sel[1] = 0u;
    }
    while (hi > lo) {
      const uint32_t diff = hi - lo;
      const int nbits = 32 - __clz(diff);
      const int shift = nbits > 8 ? nbits - 8 : 0;
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (key[e] >= lo && key[e] <= hi && key[e] != 0u) atomicAdd(&hist[(key[e] - lo) >> shift], 1u);
      __syncthreads();
      if (wave == 0) {
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hb[i] = hist[4 * lane + i];
        const uint32_t mine = hb[0] + hb[1] + hb[2] + hb[3];
        uint32_t suf = mine;  // inclusive suffix sum over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          uint32_t y = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += y;
        }
        uint32_t above = suf - mine;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if (above < krem && krem <= above + hb[i]) {
            sel[0] = 4 * lane + i;
            sel[1] = above;
          }
          above += hb[i];
        }
      }
      __syncthreads();
      const uint32_t d = sel[0];
      krem -= sel[1];
      const uint32_t nlo = lo + (d << shift);
      const uint32_t span = shift == 0 ? 0u : ((1u << shift) - 1u);
      hi = (hi - nlo) > span ? nlo + span : hi;
      lo = nlo;
      __syncthreads();
    }
    thr = lo;
  }
  // Elements above the threshold, plus the first krem equal to it (index order).
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    gt += (key[e] > thr) ? 1u : 0u;
    eq += (key[e] == thr && key[e] != 0u) ? 1u : 0u;
  }
  const uint32_t pre = block_exclusive_scan(gt | (eq << 16), scan_sh);
  uint32_t eq_before = pre >> 16;
  uint32_t pos = (pre & 0xFFFFu) + min(eq_before, krem);
  int32_t* o = out + (int64_t)row * out_len;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    bool take = key[e] > thr;
    if (key[e] == thr && key[e] != 0u) {
      take = eq_before < krem;
      ++eq_before;
    }
    if (take) {
      if (pos < kk) o[pos] = id[e];  // never more than kk entries
      ++pos;
    }
  }
  for (int i = (int)kk + tid; i < out_len; i += kTopkThreads) o[i] = -1;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int per = (a.n + kTopkThreads - 1) / kTopkThreads;
  dim3 grid((unsigned)a.rows);
#define TLS_TOPK(P)                                                                                              \
  hipLaunchKernelGGL(k_topk<P>, grid, dim3(kTopkThreads), 0, st, a.scores, a.n, a.K, a.block_idx, a.kb, a.bs, a.N, \
                     a.out, a.out_len)
  if (per <= 1) TLS_TOPK(1);
  else if (per <= 2) TLS_TOPK(2);
  else if (per <= 4) TLS_TOPK(4);
  else if (per <= 8) TLS_TOPK(8);
  else if (per <= 16) TLS_TOPK(16);
  else return hipErrorInvalidValue;
#undef TLS_TOPK
  return hipGetLastError();
}

}  // namespace tls

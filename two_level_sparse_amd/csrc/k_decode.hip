// k_decode.hip -- attention over the kept tokens, split over the token list,
// merged with log-sum-exp.
//
// AsyncTLS pages, section 2A: after the two selection stages, attention is
// computed only over the selected tokens. The G query heads of a pair share
// the gathered K/V rows, so each gathered row is read once per head tile.
//
// k_attend: workgroup = 4 wavefronts = one (pair, head tile, token split).
// A wave owns 64-token chunks of the split:
//   - lane l resolves token l of the chunk (one index load per lane, slot map
//     applied); the chunk is then streamed as four 16-token tiles whose K
//     fragments and V chunks are loaded one tile ahead (double-buffered), with
//     invalid tokens pointed at a real row and masked, so no load is guarded;
//   - q.K^T on MFMA (16x16x32 bf16): A = the tile's query heads (rows, zero
//     padded to 16), B = the 16 gathered key rows (columns);
//   - online softmax per head in the exp2 domain (scale folded with log2 e);
//   - P.V on the vector ALU: a lane owns 8 consecutive value channels of one
//     token per 16-byte load, so one wave load covers 64/(DV/8) whole rows; the
//     probabilities cross from the MFMA layout through LDS.
// The 4 waves merge their (m, l, o) in LDS and the workgroup writes one
// partial. k_merge then combines the splits of every head. (A fused
// last-workgroup merge would need an agent-scope release per workgroup, which
// on this part writes back the XCD's whole L2; a second launch is cheaper.)
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {

template <int D, int DV, int HT, bool PRE, bool SMAP>
__global__ __launch_bounds__(256) void k_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                const int32_t* __restrict__ slot_map,
                                                const int32_t* __restrict__ token_idx, float* __restrict__ part,
                                                int Hq, int Hkv, int G, int row, int v_off, int64_t N, int bs,
                                                int64_t NB, int slots, int kt, int tps, int nsplit, int nht,
                                                float qk_scale) {
  constexpr int KSTEPS = D / 32;
  constexpr int CPR = DV / 8;    // 16-byte chunks per value row
  constexpr int RPI = 64 / CPR;  // value rows per wave load
  constexpr int VL = 16 / RPI;   // value loads per 16-token tile
  static_assert(D % 32 == 0 && 64 % CPR == 0 && CPR <= 64, "unsupported shape");

  __shared__ float p_lds[4][16][16];  // [wave][token][head]
  __shared__ float c_lds[4][16];      // [wave][head] rescale factors
  __shared__ float ml_lds[4][16][2];  // [wave][head] (m, l)
  __shared__ float o_lds[HT * DV];

  const int split = blockIdx.x, ht = blockIdx.y, p = blockIdx.z;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int chunk = lane % CPR, rsub = lane / CPR;

  // Query fragments of this lane's MFMA row (head ht*HT + n): in registers,
  // or (for the wide MLA rows, which are not prefetched) in LDS.
  const int g_row = ht * HT + n;
  const bool row_ok = n < HT && g_row < G;
  __shared__ u32x4 q_lds[PRE ? 1 : KSTEPS][64];
  u32x4 qf[PRE ? KSTEPS : 1];
  {
    const uint16_t* qrow = q + ((int64_t)b * Hq + (int64_t)h * G + (row_ok ? g_row : 0)) * D;
    if constexpr (PRE) {
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) qf[k] = row_ok ? ld16(qrow + k * 32 + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
    } else {
      for (int k = wave; k < KSTEPS; k += 4) q_lds[k][lane] = row_ok ? ld16(qrow + k * 32 + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
  }

  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, kt);
  const int32_t* tix = token_idx + (int64_t)p * kt;
  const uint16_t* kvp = kv + (SMAP ? (int64_t)p * slots * bs : (int64_t)p * N) * row;
  const int32_t* smap = SMAP ? slot_map + (int64_t)p * NB : nullptr;

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  float acc[HT][8];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;

  // Each wave takes 64-token chunks of the split: lane l resolves token
  // chunk + l (index, then slot map) once; invalid tokens point at row 0 and
  // are masked afterwards, so every row load is unconditional.
  for (int c0 = t_begin + 64 * wave; c0 < t_end; c0 += 256) {
    int my_tok = -1, my_row = 0;
    {
      const int pos = c0 + lane;
      const int tok = pos < t_end ? tix[pos] : -1;
      if (tok >= 0 && tok < N) {
        if constexpr (SMAP) {
          const int slot = smap[tok / bs];
          if (slot >= 0 && slot < slots) {  // a block that is not resident is never read
            my_tok = tok;
            my_row = slot * bs + tok % bs;
          }
        } else {
          my_tok = tok;
          my_row = tok;
        }
      }
    }
    const int ntile = min(4, (t_end - c0 + 15) / 16);

    u32x4 kbuf[2][PRE ? KSTEPS : 1], vbuf[2][PRE ? VL : 1];
    int ktk[2] = {-1, -1};
    auto issue = [&](int j, int slot) {
      ktk[slot] = __shfl(my_tok, 16 * j + n, 64);
      if constexpr (PRE) {
        const uint16_t* kr = kvp + (int64_t)__shfl(my_row, 16 * j + n, 64) * row + 8 * kq;
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) kbuf[slot][k] = ld16(kr + k * 32);
#pragma unroll
        for (int v = 0; v < VL; ++v) {
          const int tt = 16 * j + v * RPI + rsub;
          vbuf[slot][v] = ld16(kvp + (int64_t)__shfl(my_row, tt, 64) * row + v_off + chunk * 8);
        }
      }
    };
    issue(0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= ntile) break;
      const int cur = j & 1;
      if (j + 1 < ntile) issue(j + 1, cur ^ 1);
      const bool tok_ok = ktk[cur] >= 0;
      // ---- scores of the 16 tokens (MFMA) ----
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = nullptr;
      if constexpr (!PRE) kr = kvp + (int64_t)__shfl(my_row, 16 * j + n, 64) * row + 8 * kq;
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        u32x4 kk, qq;
        if constexpr (PRE) {
          kk = kbuf[cur][k];
          qq = qf[k];
        } else {
          kk = ld16(kr + k * 32);
          qq = q_lds[k][lane];
        }
        z = mfma16x16x32(qq, kk, z);
      }
      // ---- online softmax (lane holds heads 4*kq+i of token n) ----
      float pr[4], corr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float zi = tok_ok ? z[i] * qk_scale : -INFINITY;
        const float tmax = max16(zi);
        const float m_new = fmaxf(m_run[i], tmax);
        const float ref = m_new == -INFINITY ? 0.0f : m_new;
        corr[i] = exp2f(m_run[i] - ref);
        pr[i] = exp2f(zi - ref);
        l_run[i] = l_run[i] * corr[i] + pr[i];
        m_run[i] = m_new;
      }
      *reinterpret_cast<f32x4*>(&p_lds[wave][n][4 * kq]) = f32x4{pr[0], pr[1], pr[2], pr[3]};
      if (n == 0) *reinterpret_cast<f32x4*>(&c_lds[wave][4 * kq]) = f32x4{corr[0], corr[1], corr[2], corr[3]};
      wave_lds_sync();
      // ---- P.V (vector ALU) ----
      // rescale only when some head's running max moved (wave-uniform test)
      if (__ballot(corr[0] != 1.0f || corr[1] != 1.0f || corr[2] != 1.0f || corr[3] != 1.0f)) {
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          const float c = c_lds[wave][hh];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] *= c;
        }
      }
#pragma unroll
      for (int v = 0; v < VL; ++v) {
        const int tt = v * RPI + rsub;
        const int vt = __shfl(my_tok, 16 * j + tt, 64);
        u32x4 w;
        if constexpr (PRE) w = vbuf[cur][v];
        else w = ld16(kvp + (int64_t)__shfl(my_row, 16 * j + tt, 64) * row + v_off + chunk * 8);
        if (vt < 0) w = u32x4{0u, 0u, 0u, 0u};  // masked token: its row may hold anything
        float vv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vv[2 * e] = bf_lo(w[e]);
          vv[2 * e + 1] = bf_hi(w[e]);
        }
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          const float ph = p_lds[wave][tt][hh];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(ph, vv[e], acc[hh][e]);
        }
      }
      wave_lds_sync();
    }
  }

  // ---- per-wave totals ----
  // l: sum over the 16 token columns; o: sum over the RPI row groups.
#pragma unroll
  for (int i = 0; i < 4; ++i) l_run[i] = sum16(l_run[i]);
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int hh = 0; hh < HT; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], o, 64);
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ml_lds[wave][4 * kq + i][0] = m_run[i];
      ml_lds[wave][4 * kq + i][1] = l_run[i];
    }
  }
  __syncthreads();
  // ---- merge the 4 waves ----
  float f[HT];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) ms = fmaxf(ms, ml_lds[w][hh][0]);
    const float mw = ml_lds[wave][hh][0];
    f[hh] = mw == -INFINITY ? 0.0f : exp2f(mw - ms);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w && rsub == 0) {
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float* dst = &o_lds[hh * DV + chunk * 8 + e];
          const float val = f[hh] * acc[hh][e];
          *dst = w == 0 ? val : *dst + val;
        }
    }
    __syncthreads();
  }
  // ---- the workgroup partial: per head (m, l, o[DV]) ----
  float* dst = part + (((int64_t)p * nht + ht) * nsplit + split) * HT * (DV + 2);
  for (int e = threadIdx.x; e < HT * (DV + 2); e += 256) {
    const int hh = e / (DV + 2), c = e % (DV + 2);
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) ms = fmaxf(ms, ml_lds[w][hh][0]);
    float val;
    if (c == 0) {
      val = ms;
    } else if (c == 1) {
      float l = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = ml_lds[w][hh][0];
        l += mw == -INFINITY ? 0.0f : ml_lds[w][hh][1] * exp2f(mw - ms);
      }
      val = l;
    } else {
      val = o_lds[hh * DV + c - 2];
    }
    dst[e] = val;
  }
}

// One workgroup per (pair, head tile): the split weights 2^(m_s - M) / L of
// every head are formed once in LDS, then each output channel is one pass of
// independent loads over the splits.
constexpr int kMaxSplits = 64;
template <int DV, int HT>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ part, float* __restrict__ out,
                                               float* __restrict__ lse, int Hq, int Hkv, int G, int nht, int nsplit) {
  __shared__ float m_lds[kMaxSplits][HT];
  __shared__ float w_lds[kMaxSplits][HT];
  const int ht = blockIdx.x, p = blockIdx.y;
  const int b = p / Hkv, h = p % Hkv;
  const float* base = part + ((int64_t)p * nht + ht) * nsplit * HT * (DV + 2);
  const int64_t sstride = (int64_t)HT * (DV + 2);
  for (int e = threadIdx.x; e < nsplit * HT; e += 256) {
    const int s = e / HT, hh = e % HT;
    m_lds[s][hh] = base[s * sstride + hh * (DV + 2)];
  }
  __syncthreads();
  if (threadIdx.x < HT) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, m_lds[s][hh]);
    float L = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = m_lds[s][hh];
      const float w = ms == -INFINITY ? 0.0f : exp2f(ms - M);
      L += base[s * sstride + hh * (DV + 2) + 1] * w;
      w_lds[s][hh] = w;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int s = 0; s < nsplit; ++s) w_lds[s][hh] *= inv;
    const int g = ht * HT + hh;
    if (lse && g < G) lse[(int64_t)b * Hq + (int64_t)h * G + g] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < HT * DV; e += 256) {
    const int hh = e / DV, c = e % DV;
    const int g = ht * HT + hh;
    if (g >= G) continue;
    const float* src = base + hh * (DV + 2) + 2 + c;
    float O = 0.0f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) O = fmaf(src[s * sstride], w_lds[s][hh], O);
    out[((int64_t)b * Hq + (int64_t)h * G + g) * DV + c] = O;
  }
}

// Launch shape: head tiles of HT <= 16 heads; a workgroup takes 256-token
// chunks (64 per wave); splits are sized for about 512 workgroups and capped
// at kMaxSplits. The 576-dim (MLA) rows are not prefetched.
static constexpr int head_tile(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16; }
static constexpr bool prefetch_rows(int D) { return D <= 256; }

bool plan_decode(int pairs, int G, int D, int DV, int kt, DecodePlan* plan) {
  const int HT = head_tile(G);
  const int nht = (G + HT - 1) / HT;
  const int units = pairs * nht;
  const int want = (512 + units - 1) / units;
  int tps = (kt + want - 1) / want;
  tps = ((tps + 255) / 256) * 256;
  const int min_tps = ((kt + kMaxSplits - 1) / kMaxSplits + 255) / 256 * 256;
  if (tps < min_tps) tps = min_tps;
  if (tps < 256) tps = 256;
  const int nsplit = (kt + tps - 1) / tps;
  plan->HT = HT;
  plan->nht = nht;
  plan->tps = tps;
  plan->nsplit = nsplit;
  plan->part_bytes = (size_t)pairs * nht * nsplit * HT * (DV + 2) * sizeof(float);
  (void)D;
  return true;
}

template <int D, int DV, int HT>
static hipError_t go_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  dim3 grid((unsigned)pl.nsplit, (unsigned)pl.nht, (unsigned)a.pairs);
  constexpr bool PRE = prefetch_rows(D);
  if (a.slot_map)
    hipLaunchKernelGGL((k_attend<D, DV, HT, PRE, true>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,
                       (float*)a.part, a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.bs, a.NB, a.slots, a.kt, pl.tps,
                       pl.nsplit, pl.nht, a.sm_scale * kLog2e);
  else
    hipLaunchKernelGGL((k_attend<D, DV, HT, PRE, false>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,
                       (float*)a.part, a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.bs, a.NB, a.slots, a.kt, pl.tps,
                       pl.nsplit, pl.nht, a.sm_scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid((unsigned)pl.nht, (unsigned)a.pairs);
  hipLaunchKernelGGL((k_merge<DV, HT>), mgrid, dim3(256), 0, st, (const float*)a.part, a.out, a.lse, a.Hq, a.Hkv, a.G,
                     pl.nht, pl.nsplit);
  return hipGetLastError();
}

template <int D, int DV>
static hipError_t go_decode_ht(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  switch (pl.HT) {
    case 1: return go_decode<D, DV, 1>(a, pl, st);
    case 2: return go_decode<D, DV, 2>(a, pl, st);
    case 4: return go_decode<D, DV, 4>(a, pl, st);
    case 8: return go_decode<D, DV, 8>(a, pl, st);
    case 16: return go_decode<D, DV, 16>(a, pl, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  if (a.D == 64 && a.DV == 64) return go_decode_ht<64, 64>(a, pl, st);
  if (a.D == 128 && a.DV == 128) return go_decode_ht<128, 128>(a, pl, st);
  if (a.D == 256 && a.DV == 256) return go_decode_ht<256, 256>(a, pl, st);
  if (a.D == 576 && a.DV == 512) return go_decode_ht<576, 512>(a, pl, st);
  return hipErrorInvalidValue;
}

}  // namespace tls

// k_decode.hip -- attention over the kept tokens, split over the token list,
// merged with log-sum-exp.
//
// AsyncTLS pages, section 2A: after the two selection stages, attention is
// computed only over the selected tokens. The G query heads of a pair share
// the gathered K/V rows, so each gathered row is read once per head tile.
//
// k_attend: workgroup = 4 wavefronts = one (pair, head tile, token split).
// Each wave takes 16-token tiles of the split in turn:
//   - q.K^T on MFMA (16x16x32 bf16): A = the tile's query heads (rows, zero
//     padded to 16), B = the 16 gathered key rows (columns); each lane loads
//     16-byte fragments of one token row;
//   - online softmax per head in the exp2 domain (scale folded with log2 e);
//   - P.V on the vector ALU: each lane owns 8 consecutive value channels of
//     one token per load (16 bytes), so a wave load covers 64/(DV/8) full rows;
//     the probabilities cross from the MFMA layout through LDS.
// The 4 waves merge their (m, l, o) in LDS; one partial per workgroup goes to
// the workspace. The last workgroup to finish a (pair, head tile) -- found
// with an atomic counter in the workspace, which it resets to zero -- merges
// the splits and writes out and lse, so one launch covers the whole call.
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {

template <int D, int DV, int HT>
__global__ __launch_bounds__(256) void k_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                const int32_t* __restrict__ slot_map,
                                                const int32_t* __restrict__ token_idx, float* __restrict__ part,
                                                int* __restrict__ counters, float* __restrict__ out,
                                                float* __restrict__ lse, int Hq, int Hkv, int G, int row, int v_off,
                                                int64_t N, int bs, int64_t NB, int slots, int kt, int tps,
                                                int nsplit, int nht, float qk_scale) {
  constexpr int KSTEPS = D / 32;
  constexpr int CPR = DV / 8;    // 16-byte chunks per value row
  constexpr int RPI = 64 / CPR;  // value rows per wave load
  static_assert(D % 32 == 0 && 64 % CPR == 0 && CPR <= 64, "unsupported head dims");

  __shared__ float p_lds[4][16][16];  // [wave][token][head]
  __shared__ float c_lds[4][16];      // [wave][head] rescale factors
  __shared__ float ml_lds[4][16][2];  // [wave][head] (m, l)
  __shared__ float o_lds[HT * DV];

  const int split = blockIdx.x, ht = blockIdx.y, p = blockIdx.z;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int chunk = lane % CPR, rsub = lane / CPR;

  // Query fragments of this lane's MFMA row (head ht*HT + n).
  const int g_row = ht * HT + n;
  const bool row_ok = n < HT && g_row < G;
  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = q + ((int64_t)b * Hq + (int64_t)h * G + (row_ok ? g_row : 0)) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) qf[k] = row_ok ? ld16(qrow + k * 32 + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
  }

  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, kt);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + 15) / 16 : 0;
  const int32_t* tix = token_idx + (int64_t)p * kt;
  const uint16_t* kvp = kv + (slot_map ? (int64_t)p * slots * bs : (int64_t)p * N) * row;
  const int32_t* smap = slot_map ? slot_map + (int64_t)p * NB : nullptr;

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

  for (int tile = wave; tile < ntiles; tile += 4) {
    const int t0 = t_begin + tile * 16;
    // ---- scores of the 16 tokens (MFMA) ----
    const int tq = t0 + n;
    int tok = tq < t_end ? tix[tq] : -1;
    int prow = 0;  // row of the token inside this pair's cache
    if (tok >= 0 && tok < N) {
      if (smap) {
        const int slot = smap[tok / bs];
        if (slot < 0 || slot >= slots) tok = -1;  // not resident: never read outside the cache
        else prow = slot * bs + tok % bs;
      } else {
        prow = tok;
      }
    } else {
      tok = -1;
    }
    const uint16_t* krow = kvp + (int64_t)prow * row;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      u32x4 kf = tok >= 0 ? ld16(krow + k * 32 + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
      z = mfma16x16x32(qf[k], kf, z);
    }
    // ---- online softmax (lane holds heads 4*kq+i of token n) ----
    float pr[4], corr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float zi = tok >= 0 ? z[i] * qk_scale : -INFINITY;
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
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
      const float c = c_lds[wave][hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= c;
    }
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RPI) {
      const int tt = r0 + rsub;
      const int tv = __shfl(tok, tt, 64);      // lane tt resolved this token above
      const int pv = __shfl(prow, tt, 64);
      if (tv >= 0) {
        const u32x4 w = ld16(kvp + (int64_t)pv * row + v_off + chunk * 8);
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf_lo(w[e]);
          v[2 * e + 1] = bf_hi(w[e]);
        }
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          const float ph = p_lds[wave][tt][hh];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(ph, v[e], acc[hh][e]);
        }
      }
    }
    wave_lds_sync();
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
  float mstar[HT];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) ms = fmaxf(ms, ml_lds[w][hh][0]);
    mstar[hh] = ms;
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
  // ---- write the workgroup partial: per head (m, l, o[DV]) ----
  float* dst = part + (((int64_t)p * nht + ht) * nsplit + split) * HT * (DV + 2);
  for (int e = threadIdx.x; e < HT * (DV + 2); e += 256) {
    const int hh = e / (DV + 2), c = e % (DV + 2);
    float val;
    if (c == 0) {
      val = mstar[hh];
    } else if (c == 1) {
      float l = 0.0f;
      for (int w = 0; w < 4; ++w) {
        const float mw = ml_lds[w][hh][0];
        l += mw == -INFINITY ? 0.0f : ml_lds[w][hh][1] * exp2f(mw - mstar[hh]);
      }
      val = l;
    } else {
      val = o_lds[hh * DV + c - 2];
    }
    dst[e] = val;
  }

  // ---- the last workgroup of this (pair, head tile) merges the splits ----
  __shared__ int last_flag;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last_flag = atomicAdd(&counters[p * nht + ht], 1) == nsplit - 1;
  __syncthreads();
  if (!last_flag) return;
  __threadfence();  // acquire: the other workgroups' partials are visible
  const float* base = part + ((int64_t)p * nht + ht) * nsplit * HT * (DV + 2);
  const int64_t sstride = (int64_t)HT * (DV + 2);
  for (int e = threadIdx.x; e < HT * DV; e += 256) {
    const int hh = e / DV, c = e % DV;
    const int g = ht * HT + hh;
    if (g >= G) continue;
    const float* ph = base + hh * (DV + 2);
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, ph[sp * sstride]);
    float L = 0.0f, O = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float ms = ph[sp * sstride];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - M);
      L += ph[sp * sstride + 1] * w;
      O += ph[sp * sstride + 2 + c] * w;
    }
    const int64_t oh = (int64_t)b * Hq + (int64_t)h * G + g;
    out[oh * DV + c] = L > 0.0f ? O / L : 0.0f;
    if (lse && c == 0) lse[oh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  if (threadIdx.x == 0) counters[p * nht + ht] = 0;  // ready for the next call
}

bool plan_decode(int pairs, int G, int D, int DV, int kt, DecodePlan* plan) {
  int HT = 1;
  while (HT < G && HT < 16) HT <<= 1;
  const int nht = (G + HT - 1) / HT;
  // Aim for about 1024 workgroups; splits are whole multiples of 64 tokens
  // (4 waves x 16-token tiles).
  const int units = pairs * nht;
  int want = (1024 + units - 1) / units;
  int tps = (kt + want - 1) / want;
  tps = ((tps + 63) / 64) * 64;
  if (tps < 64) tps = 64;
  const int nsplit = (kt + tps - 1) / tps;
  plan->HT = HT;
  plan->nht = nht;
  plan->tps = tps;
  plan->nsplit = nsplit;
  plan->cnt_bytes = (((size_t)pairs * nht * sizeof(int)) + 255) & ~(size_t)255;
  plan->part_bytes = plan->cnt_bytes + (size_t)pairs * nht * nsplit * HT * (DV + 2) * sizeof(float);
  (void)D;
  return true;
}

template <int D, int DV, int HT>
static hipError_t go_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  dim3 grid((unsigned)pl.nsplit, (unsigned)pl.nht, (unsigned)a.pairs);
  int* counters = reinterpret_cast<int*>(a.part);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(a.part) + pl.cnt_bytes);
  hipLaunchKernelGGL((k_attend<D, DV, HT>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx, part,
                     counters, a.out, a.lse, a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.bs, a.NB, a.slots, a.kt, pl.tps,
                     pl.nsplit, pl.nht, a.sm_scale * kLog2e);
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

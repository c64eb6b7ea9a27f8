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
// partial. k_merge then combines the splits of every head -- except after
// k_attend_pv launched as a single round of workgroups (at most two per CU),
// whose last workgroup of each (pair, head tile) merges the splits itself
// instead: every workgroup stores its partial with agent-scope atomic
// stores, waits for them and counts itself in with an agent-scope atomic add
// (a counter per group at the start of the workspace); the workgroup that
// completes the count loads the partials with agent-scope atomic loads,
// merges them and sets the counter back to zero. Those accesses are coherent
// across the XCDs' L2 caches without writing any of them back (an
// agent-scope release fence would write back the XCD's whole L2, which costs
// more than the second launch it saves).
#include <type_traits>

#include "tls_attn_dev.h"
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {


template <int D, int DV, int HT, bool PRE, bool SMAP>
__global__ __launch_bounds__(256) void k_attend(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                const int32_t* __restrict__ slot_map,
                                                const int32_t* __restrict__ token_idx, float* __restrict__ part,
                                                int Hq, int Hkv, int G, int row, int v_off, int64_t N, int64_t Ns, int bs,
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
  const uint16_t* kvp = kv + (SMAP ? (int64_t)p * slots * bs : (int64_t)p * Ns) * row;
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
  // ---- the workgroup partial: per head (m, l, -, -, o[DV]) ----
  float* dst = part + (((int64_t)p * nht + ht) * nsplit + split) * HT * (DV + kPartHdr);
  for (int e = threadIdx.x; e < HT * (DV + kPartHdr); e += 256) {
    const int hh = e / (DV + kPartHdr), c = e % (DV + kPartHdr);
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
    } else if (c < kPartHdr) {
      val = 0.0f;
    } else {
      val = o_lds[hh * DV + c - kPartHdr];
    }
    dst[e] = val;
  }
}

// k_attend_gqa: k_attend for rows of up to 128 channels, with the value
// product laid out so that every lane owns distinct outputs: lane l keeps
// channels CPL*l .. CPL*l+CPL-1 (CPL = DV/64) of every head of the tile, and
// reads, for each token, just those channels (one small load per token per
// lane, 256 bytes per wave for DV = 128). The accumulator is HT*CPL floats
// per lane instead of HT*8, which leaves room for two waves per SIMD with the
// 16-token tiles double-buffered; the probabilities are broadcast from LDS.
// Token validity and rows for the value loads are wave-uniform (readlane).
template <int D, int DV, int HT, bool SMAP>
__global__ __launch_bounds__(256, 2) void k_attend_gqa(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                       const int32_t* __restrict__ slot_map,
                                                       const int32_t* __restrict__ token_idx,
                                                       float* __restrict__ part, int Hq, int Hkv, int G, int row,
                                                       int v_off, int64_t N, int64_t Ns, int bs, int64_t NB, int slots, int kt,
                                                       int tps, int nsplit, int nht, float qk_scale) {
  constexpr int KSTEPS = D / 32;
  constexpr int CPL = DV / 64;  // value channels per lane
  static_assert(D % 32 == 0 && DV % 64 == 0 && (CPL == 1 || CPL == 2 || CPL == 4), "unsupported shape");
  using VT = typename std::conditional<CPL == 1, uint16_t, typename std::conditional<CPL == 2, uint32_t, u32x2>::type>::type;

  __shared__ __attribute__((aligned(16))) float p_lds[4][16][16];  // [wave][token][head]
  __shared__ __attribute__((aligned(16))) float c_lds[4][16];      // [wave][head] rescale factors
  __shared__ float ml_lds[4][16][2];                               // [wave][head] (m, l)
  __shared__ float o_lds[HT * DV];

  const int split = blockIdx.x, ht = blockIdx.y, p = blockIdx.z;
  const int b = p / Hkv, h = p % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;

  // query fragments of this lane's MFMA row (head ht*HT + n)
  const int g_row = ht * HT + n;
  const bool row_ok = n < HT && g_row < G;
  u32x4 qf[KSTEPS];
  {
    const uint16_t* qrow = q + ((int64_t)b * Hq + (int64_t)h * G + (row_ok ? g_row : 0)) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) qf[k] = ld16(qrow + k * 32 + 8 * kq);
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k)
      if (!row_ok) qf[k] = u32x4{0u, 0u, 0u, 0u};
  }

  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, kt);
  const int32_t* tix = token_idx + (int64_t)p * kt;
  const uint16_t* kvp = kv + (SMAP ? (int64_t)p * slots * bs : (int64_t)p * Ns) * row;
  const int32_t* smap = SMAP ? slot_map + (int64_t)p * NB : nullptr;

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  float acc[HT][CPL];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[hh][c] = 0.0f;

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

    u32x4 kbuf[2][KSTEPS];
    VT vbuf[2][16];
    int ktk[2] = {-1, -1};
    auto issue = [&](int j, int slot) {
      ktk[slot] = __shfl(my_tok, 16 * j + n, 64);
      const uint16_t* kr = kvp + (int64_t)__shfl(my_row, 16 * j + n, 64) * row + 8 * kq;
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) kbuf[slot][k] = ld16(kr + k * 32);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int r = __builtin_amdgcn_readlane(my_row, 16 * j + t);
        vbuf[slot][t] = *reinterpret_cast<const VT*>(kvp + (int64_t)r * row + v_off + CPL * lane);
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
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) z = mfma16x16x32(qf[k], kbuf[cur][k], z);
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
      // ---- P.V: this lane's channels of every head ----
      if (__ballot(corr[0] != 1.0f || corr[1] != 1.0f || corr[2] != 1.0f || corr[3] != 1.0f)) {
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          const float c = c_lds[wave][hh];
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[hh][e] *= c;
        }
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const bool vok = __builtin_amdgcn_readlane(my_tok, 16 * j + t) >= 0;
        float vv[CPL];
        if constexpr (CPL == 1) {
          vv[0] = bf2f(vbuf[cur][t]);
        } else if constexpr (CPL == 2) {
          vv[0] = bf_lo(vbuf[cur][t]);
          vv[1] = bf_hi(vbuf[cur][t]);
        } else {
          vv[0] = bf_lo(vbuf[cur][t][0]);
          vv[1] = bf_hi(vbuf[cur][t][0]);
          vv[2] = bf_lo(vbuf[cur][t][1]);
          vv[3] = bf_hi(vbuf[cur][t][1]);
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e)
          if (!vok) vv[e] = 0.0f;  // masked token: its row may hold anything
        float ph[HT];
        if constexpr (HT % 4 == 0) {
#pragma unroll
          for (int g4 = 0; g4 < HT / 4; ++g4) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(&p_lds[wave][t][4 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) ph[4 * g4 + i] = pv[i];
          }
        } else {
#pragma unroll
          for (int hh = 0; hh < HT; ++hh) ph[hh] = p_lds[wave][t][hh];
        }
#pragma unroll
        for (int hh = 0; hh < HT; ++hh)
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[hh][e] = fmaf(ph[hh], vv[e], acc[hh][e]);
      }
      wave_lds_sync();
    }
  }

  // ---- per-wave totals: l over the 16 token columns ----
#pragma unroll
  for (int i = 0; i < 4; ++i) l_run[i] = sum16(l_run[i]);
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
    if (wave == w) {
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          float* dst = &o_lds[hh * DV + CPL * lane + e];
          const float val = f[hh] * acc[hh][e];
          *dst = w == 0 ? val : *dst + val;
        }
    }
    __syncthreads();
  }
  // ---- the workgroup partial: per head (m, l, -, -, o[DV]) ----
  float* dst = part + (((int64_t)p * nht + ht) * nsplit + split) * HT * (DV + kPartHdr);
  for (int e = threadIdx.x; e < HT * (DV + kPartHdr); e += 256) {
    const int hh = e / (DV + kPartHdr), c = e % (DV + kPartHdr);
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
    } else if (c < kPartHdr) {
      val = 0.0f;
    } else {
      val = o_lds[hh * DV + c - kPartHdr];
    }
    dst[e] = val;
  }
}

constexpr int kMaxSplits = 64;      // split limit of the general attention kernels
constexpr int kMlaMaxSplits = 128;  // of the latent attention (512 tokens per split at most)
constexpr int kMergePre = 8;
// The log-sum-exp merge of one head's nsplit partials on value channels
// c .. c+3 (hd: the head in split 0; splits SP floats apart): M = max of the
// splits' m, L = sum of l_s 2^(m_s - M), o = sum of o_s 2^(m_s - M).
// kMergePre splits per round, all their loads in flight together; the running
// max and sums are rescaled when a round raises the max. COHERENT: the
// partials are read with agent-scope atomic loads (written in this launch).
template <bool COHERENT>
__device__ __forceinline__ void merge_splits(const float* hd, int64_t SP, int nsplit, int c, float& M, float& L,
                                             f32x4& o) {
  M = -INFINITY;
  L = 0.0f;
  o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += kMergePre) {
    float2 ml[kMergePre];
    f32x4 ov[kMergePre];
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) {
      const int64_t off = (int64_t)min(s0 + u, nsplit - 1) * SP;
      if constexpr (COHERENT) {
        ml[u] = load_agent2(hd + off);
        const float2 o01 = load_agent2(hd + off + kPartHdr + c), o23 = load_agent2(hd + off + kPartHdr + c + 2);
        ov[u] = f32x4{o01.x, o01.y, o23.x, o23.y};
      } else {
        ml[u] = *reinterpret_cast<const float2*>(hd + off);
        ov[u] = *reinterpret_cast<const f32x4*>(hd + off + kPartHdr + c);
      }
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < kMergePre; ++u) cm = fmaxf(cm, ml[u].x);  // clamped repeats leave the max as it is
    if (cm != M) {
      const float r = M == -INFINITY ? 0.0f : exp2f(M - cm);
      L *= r;
      o *= r;
      M = cm;
    }
#pragma unroll
    for (int u = 0; u < kMergePre; ++u)
      if (s0 + u < nsplit) {
        const float w = ml[u].x == -INFINITY ? 0.0f : exp2f(ml[u].x - M);
        L += ml[u].y * w;
        o += ov[u] * w;
      }
  }
}

// k_attend_pv: attend_pv_range over split blockIdx.x (tps tokens) of head tile
// blockIdx.y of pair blockIdx.z. FUSED: the last workgroup of each (pair,
// head tile) to finish merges the splits into out and lse (cnt: one counter
// per group, zero before the launch and again after it); otherwise k_merge
// does, in a launch of its own.
template <int HT, bool SMAP, bool FUSED>
__global__ __launch_bounds__(256, 2) void k_attend_pv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                      const int32_t* __restrict__ slot_map,
                                                      const int32_t* __restrict__ token_idx, float* __restrict__ part,
                                                      int* __restrict__ cnt, float* __restrict__ out,
                                                      float* __restrict__ lse, int Hq, int Hkv, int G, int64_t N,
                                                      int64_t Ns, int bs, int64_t NB, int slots, int kt, int tps,
                                                      int nsplit, int nht, float qk_scale) {
  __shared__ __attribute__((aligned(1024))) uint8_t tA[4][kPvTile * kPvRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t tB[4][kPvTile * kPvRowBytes];
  __shared__ int32_t rows[4][kPvMaxTps / 4];  // wave w: its tiles' rows, tile m at [16m, 16m+16)
  __shared__ float c_lds[4][16];
  __shared__ float ml_lds[4][16][2];
  const int split = blockIdx.x, ht = blockIdx.y, p = blockIdx.z;
  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, kt);
  constexpr int PS = 128 + kPartHdr, SP = HT * PS;
  float* grp = part + ((int64_t)p * nht + ht) * nsplit * SP;
  attend_pv_range<HT, SMAP, kPvMaxTps / 4, FUSED>(q, kv, slot_map, token_idx + (int64_t)p * kt + t_begin,
                                                  max(t_end - t_begin, 0), grp + (int64_t)split * SP, Hq, Hkv, G, N,
                                                  Ns, bs, NB, slots, p, ht, qk_scale, tA, tB, rows, c_lds, ml_lds);
  if constexpr (!FUSED) return;
  // count this workgroup in once all of its partial is stored
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int s_last;
  int* ctr = cnt + (int64_t)p * nht + ht;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  // the last one: merge the group's splits, as k_merge does
  const int b = p / Hkv, h = p % Hkv;
  for (int e = threadIdx.x; e < HT * 32; e += 256) {
    const int hh = e >> 5, c = (e & 31) * 4, g = ht * HT + hh;
    if (g >= G) continue;
    float M, L;
    f32x4 o;
    merge_splits<true>(grp + (int64_t)hh * PS, SP, nsplit, c, M, L, o);
    const int64_t row = (int64_t)b * Hq + (int64_t)h * G + g;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (lse && c == 0) lse[row] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    *reinterpret_cast<f32x4*>(out + row * 128 + c) = o * inv;
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// k_attend_mla: the latent-attention shape (K rows of 576, V = their first
// 512 channels, many query heads on one kv row), with both products on MFMA.
// Workgroup = 4 wavefronts = one (pair, group of 32 heads, token split).
//   - The split's token rows are resolved once into LDS. 32-token tiles of
//     whole rows go to LDS with direct global->LDS 16-byte loads, double-
//     buffered in two LDS objects (so the compiler sees that reading tile j
//     does not wait for the loads of tile j+1). Layout: 72 chunks of 512
//     bytes, one per 16-byte column piece cp, holding the 32 rows; row r of
//     chunk cp sits in slot r ^ (4 * (cp & 1)), which keeps both read
//     patterns below free of bank conflicts. A masked token loads the row of
//     the split's first valid token (finite data) and is masked in softmax.
//   - Wave w owns head tile w&1 (16 heads) and value channels 256*(w>>1) ..
//     +255. S^T = K q^T on MFMA (A = 16 staged key rows, B = query fragments
//     kept in registers), for both 16-token halves of the tile. The two waves
//     of a head tile split the contraction: each multiplies half of the key
//     steps, the second half hands its sums to the first through LDS, which
//     adds them and hands the totals back, so both continue from the same
//     scores. The lane holding head n then has tokens 4kq+i of each half,
//     which is exactly an A-operand row of P for the next product when the
//     k-slots of P.V are ordered (half, i) -- so P never leaves the registers.
//   - Online softmax per head in the exp2 domain; the running max is made
//     common across the lanes of a head with cross-row swaps.
//   - O += P V on MFMA. P is carried as two bf16 terms (hi + lo, each exact
//     in the product, together within about 2^-17 of the fp32 value), so the
//     product keeps fp32-level accuracy. V fragments (8 tokens of one channel
//     per lane) come from the staged rows with the LDS transpose read
//     (ds_read_b64_tr_b16): within a 16-lane group, lane j receives element
//     j%4 of the 4-element pieces addressed by lanes 4e + j/4, e = 0..3.
// The partial (m, l, o) of the 32 heads goes to the workspace for k_merge.
constexpr int kMlaHeads = 32;
constexpr int kMlaTile = 32;
constexpr int kMlaMaxTps = 512;

template <bool SMAP>
__global__ __launch_bounds__(256, 2) void k_attend_mla(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kv,
                                                       const int32_t* __restrict__ slot_map,
                                                       const int32_t* __restrict__ token_idx,
                                                       float* __restrict__ part, int Hq, int Hkv, int G, int64_t N,
                                                       int64_t Ns, int bs, int64_t NB, int slots, int kt, int tps, int nsplit,
                                                       int nhg, float qk_scale) {
  constexpr int D = 576, DV = 512, KS = D / 32;
  constexpr int CP = D / 8;           // 16-byte column pieces per row = LDS chunks per tile
  constexpr int CHUNK = kMlaTile * 16;  // bytes per chunk
  constexpr int NLOAD = CP / 2;       // 1 KB direct loads per tile (two chunks each)
  static_assert(NLOAD % 4 == 0 && kMlaTile == 32, "tile layout");
  __shared__ __attribute__((aligned(1024))) uint8_t tA[CP * CHUNK];
  __shared__ __attribute__((aligned(1024))) uint8_t tB[CP * CHUNK];
  __shared__ int32_t rows[kMlaMaxTps];
  __shared__ f32x4 sx[2][64][2];  // [head tile][lane][token half]: the score exchange
  __shared__ float c_lds[4][16];
  __shared__ uint32_t wfirst[4];

  const int split = blockIdx.x, hg = blockIdx.y, p = blockIdx.z;
  const int b = p / Hkv, h = p % Hkv;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15, kq = lane >> 4;
  const int mt = wave & 1, chh = wave >> 1;
  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, kt);
  const int ntok = max(t_end - t_begin, 0);
  const uint16_t* kvp = kv + (SMAP ? (int64_t)p * slots * bs : (int64_t)p * Ns) * D;

  // query fragments of the wave's 16 heads over its half of the key steps
  // (rows past G repeat row G-1), loaded together with the token lists below
  constexpr int KH = KS / 2;
  u32x4 qf[KH];
  {
    const int g = min(hg * kMlaHeads + mt * 16 + n, G - 1);
    const uint16_t* qr = q + ((int64_t)b * Hq + (int64_t)h * G + g) * D + 8 * kq + 32 * KH * chh;
#pragma unroll
    for (int k = 0; k < KH; ++k) qf[k] = ld16(qr + 32 * k);
  }
  // rows of the split's tokens (-1: masked), and the first valid one (the
  // smallest valid position over the waves)
  uint32_t kmin = 0xFFFFFFFFu;
  {
    const int32_t* tix = token_idx + (int64_t)p * kt + t_begin;
    const int32_t* smap = SMAP ? slot_map + (int64_t)p * NB : nullptr;
    for (int k = tid; k < tps; k += 256) {
      const int tok = k < ntok ? tix[k] : -1;
      int r = -1;
      if (tok >= 0 && tok < N) {
        if constexpr (SMAP) {
          const int slot = smap[tok / bs];
          if (slot >= 0 && slot < slots) r = slot * bs + tok % bs;
        } else {
          r = tok;
        }
      }
      rows[k] = r;
      if (r >= 0) kmin = min(kmin, (uint32_t)k);
    }
  }
  kmin = wave_umin(kmin);
  if (lane == 0) wfirst[wave] = kmin;
  __syncthreads();
  const uint32_t first_ok = min(min(wfirst[0], wfirst[1]), min(wfirst[2], wfirst[3]));
  const int fb = first_ok < (uint32_t)tps ? rows[first_ok] : -1;
  const int ntiles = fb < 0 ? 0 : (ntok + kMlaTile - 1) / kMlaTile;  // nothing valid: empty partial

  // direct loads of tile j into `dst`: wave w issues loads w, w+4, ..; lane L
  // of load i fills slot L&31 of chunk 2i + (L>>5)
  auto issue = [&](uint8_t* dst, int j) {
#pragma unroll
    for (int k = 0; k < NLOAD / 4; ++k) {
      const int i = wave + 4 * k;
      const int cp = 2 * i + (lane >> 5);
      const int r = (lane & 31) ^ (4 * (cp & 1));
      const int row = rows[j * kMlaTile + r];
      const uint16_t* src = kvp + (int64_t)(row >= 0 ? row : fb) * D + cp * 8;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + i * 2 * CHUNK), 16, 0, 0);
    }
  };

  float m_run = -INFINITY, l_part = 0.0f;  // head n of the wave's tile (common over kq after the swaps)
  f32x4 o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* tb, int j) {
    // ---- S^T for the two 16-token halves, this wave's half of the key steps ----
    // key fragments in groups of KG steps: all reads of a group are issued
    // before its MFMAs
    constexpr int KG = 3;
    static_assert(KH % KG == 0, "key step groups");
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kg = 0; kg < KH; kg += KG) {
      u32x4 k0[KG], k1[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const int cp = 4 * (KH * chh + kg + u) + kq;
        const uint8_t* cb = tb + cp * CHUNK;
        const int sw = 4 * (cp & 1);
        k0[u] = *reinterpret_cast<const u32x4*>(cb + (n ^ sw) * 16);
        k1[u] = *reinterpret_cast<const u32x4*>(cb + ((16 + n) ^ sw) * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        s0 = mfma16x16x32(k0[u], qf[kg + u], s0);
        s1 = mfma16x16x32(k1[u], qf[kg + u], s1);
      }
    }
    // the halves meet: the second hands its sums over, the first adds them
    // and hands the totals back (barriers without a memory fence, which would
    // also wait for the next tile's loads)
    if (chh == 1) {
      sx[mt][lane][0] = s0;
      sx[mt][lane][1] = s1;
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (chh == 0) {
      s0 += sx[mt][lane][0];
      s1 += sx[mt][lane][1];
      sx[mt][lane][0] = s0;
      sx[mt][lane][1] = s1;
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (chh == 1) {
      s0 = sx[mt][lane][0];
      s1 = sx[mt][lane][1];
    }
    // ---- online softmax: this lane has tokens 4kq+i and 16+4kq+i of head n ----
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok0 = rows[j * kMlaTile + 4 * kq + i] >= 0;
      const bool ok1 = rows[j * kMlaTile + 16 + 4 * kq + i] >= 0;
      z[i] = ok0 ? s0[i] * qk_scale : -INFINITY;
      z[4 + i] = ok1 ? s1[i] * qk_scale : -INFINITY;
    }
    float tmax = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, z[i]);
    tmax = max_rows(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float ref = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = exp2f(m_run - ref);
    float pr[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = exp2f(z[i] - ref);
      psum += pr[i];
    }
    l_part = l_part * corr + psum;
    m_run = m_new;
    // P as hi + lo bf16, k-slot order (half, i)
    u32x4 phi, plo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h0 = f32_to_bf16_rn(pr[2 * e]), h1 = f32_to_bf16_rn(pr[2 * e + 1]);
      const uint32_t l0 = f32_to_bf16_rn(pr[2 * e] - bf2f(h0)), l1 = f32_to_bf16_rn(pr[2 * e + 1] - bf2f(h1));
      phi[e] = h0 | (h1 << 16);
      plo[e] = l0 | (l1 << 16);
    }
    // rescale o (rows = heads 4kq+i) when a running max moved
    if (__ballot(corr != 1.0f)) {
      if (kq == 0) c_lds[wave][n] = corr;
      wave_lds_sync();
      const f32x4 cr = *reinterpret_cast<const f32x4*>(&c_lds[wave][4 * kq]);
#pragma unroll
      for (int t = 0; t < 16; ++t) o[t] *= cr;
    }
    // ---- O += P V over the wave's 16 channel tiles ----
    // lane n of a group addresses row 4kq + n/4 (+16), channels c0 + 4(n%4) ..
    // +3: chunk c0/8 + (n%4)/2, byte 8*(n&1) of the row's slot
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const int cpo = (n >> 1) & 1;
    const int r0 = (4 * kq + (n >> 2)) ^ (4 * cpo), r1 = (16 + 4 * kq + (n >> 2)) ^ (4 * cpo);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint8_t* cb = tb + (chh * 32 + 2 * t + cpo) * CHUNK + 8 * (n & 1);
      const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(cb + r0 * 16));
      const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(cb + r1 * 16));
      const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      const u32x4 vf = {w0[0], w0[1], w1[0], w1[1]};
      o[t] = mfma16x16x32(phi, vf, o[t]);
      o[t] = mfma16x16x32(plo, vf, o[t]);
    }
  };

  // Barrier without a memory fence (a fence would also wait for the loads of
  // the next tile); this wave's direct loads are complete before it.
  auto tile_barrier = [&]() {
    wait_vmcnt<0>();
    __asm__ volatile("s_barrier" ::: "memory");
  };
  if (ntiles > 0) issue(tA, 0);
  tile_barrier();
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles) issue(tB, j + 1);
    compute(tA, j);
    tile_barrier();  // tile j+1 landed; every wave is done with tA
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) issue(tA, j + 2);
    compute(tB, j + 1);
    tile_barrier();
  }

  // ---- the partial of the 32 heads: (m, l, -, -, o[DV]) ----
  const float l_tot = sum_rows(l_part);
  float* dst = part + (((int64_t)p * nhg + hg) * nsplit + split) * kMlaHeads * (DV + kPartHdr);
  if (chh == 0 && kq == 0) {
    float* hd = dst + (mt * 16 + n) * (DV + kPartHdr);
    hd[0] = m_run;
    hd[1] = l_tot;
  }
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[(mt * 16 + 4 * kq + i) * (DV + kPartHdr) + kPartHdr + chh * 256 + t * 16 + n] = o[t][i];
}

// Split merge. Workgroup = (256 float4 outputs, head tile, pair); every
// thread forms its head's split weights 2^(m_s - M) itself from the splits'
// (m, l), loaded together with its float4 of o, kMergePre splits per round:
// no LDS and no barrier.
template <int DV, int HT>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ part, float* __restrict__ out,
                                               float* __restrict__ lse, int Hq, int Hkv, int G, int nht, int nsplit) {
  const int ht = blockIdx.y, p = blockIdx.z, tid = threadIdx.x;
  const int b = p / Hkv, h = p % Hkv;
  constexpr int PS = DV + kPartHdr;  // floats per head in a partial
  constexpr int SP = HT * PS;        // floats per split
  const int e = blockIdx.x * 256 + tid;  // float4 index in [HT, DV/4]
  const int ee = min(e, HT * (DV / 4) - 1);
  const int hh = ee / (DV / 4), c = (ee % (DV / 4)) * 4;
  const int g = ht * HT + hh;
  const bool active = e < HT * (DV / 4) && g < G;
  // head hh of split 0: (m, l, -, -, o[DV])
  const float* hd = part + ((int64_t)p * nht + ht) * nsplit * SP + (int64_t)hh * PS;
  float M, L;
  f32x4 o;
  merge_splits<false>(hd, SP, nsplit, c, M, L, o);
  if (!active) return;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (lse && c == 0) lse[(int64_t)b * Hq + (int64_t)h * G + g] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
  *reinterpret_cast<f32x4*>(out + ((int64_t)b * Hq + (int64_t)h * G + g) * DV + c) = o * inv;
}

// Launch shape: head tiles of HT <= 16 heads; a workgroup takes 256-token
// chunks (64 per wave); splits are sized for about 512 workgroups and capped
// at kMaxSplits. The 576-dim (MLA) rows are not prefetched.
static constexpr int head_tile(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16; }
static constexpr bool prefetch_rows(int D) { return D <= 256; }

void plan_decode(int pairs, int G, int D, int DV, bool v_is_k_prefix, int kt, DecodePlan* plan) {
  if (D == 576 && DV == 512 && v_is_k_prefix && G > 16 && kt <= kMlaMaxSplits * kMlaMaxTps) {
    // latent attention: 32-head groups, 32-token tiles; about 512 workgroups
    // (two per CU, so that one's loads and barriers overlap the other's
    // MFMAs); the partials cost 2 KB per head and split
    const int nht = (G + kMlaHeads - 1) / kMlaHeads;
    const int units = pairs * nht;
    const int want = (512 + units - 1) / units;
    int tps = (kt + want - 1) / want;
    tps = ((tps + kMlaTile - 1) / kMlaTile) * kMlaTile;
    const int min_tps = ((kt + kMlaMaxSplits - 1) / kMlaMaxSplits + kMlaTile - 1) / kMlaTile * kMlaTile;
    if (tps < min_tps) tps = min_tps;
    if (tps < kMlaTile) tps = kMlaTile;
    if (tps > kMlaMaxTps) tps = kMlaMaxTps;  // kt <= kMlaMaxSplits * kMlaMaxTps keeps nsplit in range
    plan->mla = 1;
    plan->pv = 0;
    plan->fused = 0;
    plan->HT = kMlaHeads;
    plan->nht = nht;
    plan->tps = tps;
    plan->nsplit = (kt + tps - 1) / tps;
    plan->part_bytes = (size_t)pairs * nht * plan->nsplit * kMlaHeads * (DV + kPartHdr) * sizeof(float);
    return;
  }
  const int HT = head_tile(G);
  const int nht = (G + HT - 1) / HT;
  const int units = pairs * nht;
  const int want = (512 + units - 1) / units;
  if (D == 128 && DV == 128 && !v_is_k_prefix && kt <= kMaxSplits * kPvMaxTps) {
    // k_attend_pv: splits of a multiple of 64 tokens (a 16-token tile per
    // wave and round), about 256 workgroups: one per CU already keeps the
    // gather at its ceiling (128k: 30.9 µs per launch against 30.7 with 512),
    // and longer splits leave fewer partials to merge and fewer fixed costs
    // per token (32k: 38.5 against 39.8 µs per step)
    const int want_pv = (256 + units - 1) / units;
    int tps = (kt + want_pv - 1) / want_pv;
    const int min_tps = (kt + kMaxSplits - 1) / kMaxSplits;
    if (tps < min_tps) tps = min_tps;
    tps = ((tps + 63) / 64) * 64;
    if (tps > kPvMaxTps) tps = kPvMaxTps;  // kt <= kMaxSplits * kPvMaxTps keeps nsplit in range
    plan->mla = 0;
    plan->pv = 1;
    plan->HT = HT;
    plan->nht = nht;
    plan->tps = tps;
    plan->nsplit = (kt + tps - 1) / tps;
    // the split merge inside the launch pays when every workgroup is resident
    // at once (two per CU): with more, each workgroup's wait for its stores and
    // its count would recur round after round (the dense 128k launch, 4096
    // workgroups: 818 us fused against 734 with k_merge)
    plan->fused = (int64_t)units * plan->nsplit <= kFuseMaxWorkgroups;
    plan->part_bytes = (size_t)pairs * nht * plan->nsplit * HT * (DV + kPartHdr) * sizeof(float);
    return;
  }
  int tps = (kt + want - 1) / want;
  tps = ((tps + 255) / 256) * 256;
  const int min_tps = ((kt + kMaxSplits - 1) / kMaxSplits + 255) / 256 * 256;
  if (tps < min_tps) tps = min_tps;
  if (tps < 256) tps = 256;
  const int nsplit = (kt + tps - 1) / tps;
  plan->mla = 0;
  plan->pv = 0;
  plan->fused = 0;
  plan->HT = HT;
  plan->nht = nht;
  plan->tps = tps;
  plan->nsplit = nsplit;
  plan->part_bytes = (size_t)pairs * nht * nsplit * HT * (DV + kPartHdr) * sizeof(float);
  (void)D;
}

static void prof_mark(hipEvent_t ev, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev, st);
}

// The decode workspace: the group counters, then the partials.
static int* ws_counters(const DecodeArgs& a) { return reinterpret_cast<int*>(a.part); }
static float* ws_partials(const DecodeArgs& a) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(a.part) + kDecodeCntBytes);
}

template <int DV, int HT>
static hipError_t launch_merge(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  dim3 mgrid((unsigned)((HT * DV / 4 + 255) / 256), (unsigned)pl.nht, (unsigned)a.pairs);
  hipLaunchKernelGGL((k_merge<DV, HT>), mgrid, dim3(256), 0, st, (const float*)ws_partials(a), a.out, a.lse, a.Hq,
                     a.Hkv, a.G, pl.nht, pl.nsplit);
  return hipGetLastError();
}

template <int D, int DV, int HT>
static hipError_t go_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  dim3 grid((unsigned)pl.nsplit, (unsigned)pl.nht, (unsigned)a.pairs);
  constexpr bool PRE = prefetch_rows(D);
  prof_mark(a.prof_start, st);
  if constexpr (D == 128 && DV == 128) {
    if (pl.pv) {
#define TLS_PV(SM, FU)                                                                                          \
  hipLaunchKernelGGL((k_attend_pv<HT, SM, FU>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,       \
                     ws_partials(a), ws_counters(a), a.out, a.lse, a.Hq, a.Hkv, a.G, a.N, a.Ns, a.bs, a.NB, a.slots, \
                     a.kt, pl.tps, pl.nsplit, pl.nht, a.sm_scale * kLog2e)
      if (a.slot_map) {
        if (pl.fused) TLS_PV(true, true); else TLS_PV(true, false);
      } else {
        if (pl.fused) TLS_PV(false, true); else TLS_PV(false, false);
      }
#undef TLS_PV
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      prof_mark(a.prof_end, st);
      return pl.fused ? hipSuccess : launch_merge<DV, HT>(a, pl, st);  // (fused: merged inside the kernel)
    }
  }
  if constexpr (D <= 128) {  // wider rows: the per-lane buffers of k_attend_gqa would spill
    if (a.slot_map)
      hipLaunchKernelGGL((k_attend_gqa<D, DV, HT, true>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,
                         ws_partials(a), a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.Ns, a.bs, a.NB, a.slots, a.kt, pl.tps,
                         pl.nsplit, pl.nht, a.sm_scale * kLog2e);
    else
      hipLaunchKernelGGL((k_attend_gqa<D, DV, HT, false>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,
                         ws_partials(a), a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.Ns, a.bs, a.NB, a.slots, a.kt, pl.tps,
                         pl.nsplit, pl.nht, a.sm_scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_mark(a.prof_end, st);
    return launch_merge<DV, HT>(a, pl, st);
  }
  if (a.slot_map)
    hipLaunchKernelGGL((k_attend<D, DV, HT, PRE, true>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,
                       ws_partials(a), a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.Ns, a.bs, a.NB, a.slots, a.kt, pl.tps,
                       pl.nsplit, pl.nht, a.sm_scale * kLog2e);
  else
    hipLaunchKernelGGL((k_attend<D, DV, HT, PRE, false>), grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx,
                       ws_partials(a), a.Hq, a.Hkv, a.G, a.row, a.v_off, a.N, a.Ns, a.bs, a.NB, a.slots, a.kt, pl.tps,
                       pl.nsplit, pl.nht, a.sm_scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(a.prof_end, st);
  return launch_merge<DV, HT>(a, pl, st);
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

static hipError_t go_decode_mla(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  dim3 grid((unsigned)pl.nsplit, (unsigned)pl.nht, (unsigned)a.pairs);
  prof_mark(a.prof_start, st);
  if (a.slot_map)
    hipLaunchKernelGGL(k_attend_mla<true>, grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx, ws_partials(a),
                       a.Hq, a.Hkv, a.G, a.N, a.Ns, a.bs, a.NB, a.slots, a.kt, pl.tps, pl.nsplit, pl.nht,
                       a.sm_scale * kLog2e);
  else
    hipLaunchKernelGGL(k_attend_mla<false>, grid, dim3(256), 0, st, a.q, a.kv, a.slot_map, a.token_idx, ws_partials(a),
                       a.Hq, a.Hkv, a.G, a.N, a.Ns, a.bs, a.NB, a.slots, a.kt, pl.tps, pl.nsplit, pl.nht,
                       a.sm_scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(a.prof_end, st);
  return launch_merge<512, kMlaHeads>(a, pl, st);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t st) {
  if (pl.mla) return go_decode_mla(a, pl, st);
  if (a.D == 64 && a.DV == 64) return go_decode_ht<64, 64>(a, pl, st);
  if (a.D == 128 && a.DV == 128) return go_decode_ht<128, 128>(a, pl, st);
  if (a.D == 256 && a.DV == 256) return go_decode_ht<256, 256>(a, pl, st);
  if (a.D == 576 && a.DV == 512) return go_decode_ht<576, 512>(a, pl, st);
  return hipErrorInvalidValue;
}

}  // namespace tls

// tls_attn_dev.h -- the 128-channel attention body shared by k_attend_pv
// (k_decode.hip) and the attention items of the one-launch decode step
// (k_step.hip). (Internal to the HIP library; not part of the C ABI.)
#pragma once
#include "tls_dev.h"

namespace tls {

// A split's partial per head: m, l, two unused floats, then o[DV] (16-byte
// aligned for the merge's vector loads).
constexpr int kPartHdr = 4;

// attend_pv_range (the body of k_attend_pv and of the attention items of the
// one-launch decode step): 128-channel K and V in one 512-byte row (the GQA shape), with
// both products on MFMA. Workgroup = 4 wavefronts = one (pair, head tile of
// up to 16 heads, token split); every wave streams its own 16-token tiles
// (tiles w, w+4, ...) and keeps its own (m, l, o); the four meet in LDS.
//   - The split's token rows are resolved once into LDS. A tile's 16 whole
//     rows go to wave-private LDS with direct global->LDS 16-byte loads (two
//     512-byte rows per load), double-buffered. Row r keeps global 16-byte
//     piece c at position c ^ swz(r), which spreads both read patterns below
//     over the banks. A masked token loads the split's first valid row
//     (finite data) and is masked in softmax.
//   - S^T = K q^T on MFMA (16x16x32): A = the 16 key rows, B = the heads'
//     query fragments kept in registers. The lane of head n then holds tokens
//     4kq+i, which is exactly its A-operand row of P for a 16x16x16 product.
//   - Online softmax per head in the exp2 domain; the running max is made
//     common across the lanes of a head with cross-row swaps.
//   - O += P V on MFMA (16x16x16, 8 tiles of 16 channels), P as two bf16 terms
//     (hi + lo, together within about 2^-17 of the fp32 value); V fragments (4
//     tokens of one channel per lane) come from the staged rows with the LDS
//     transpose read (ds_read_b64_tr_b16).
// Against k_attend_gqa (P.V on the vector ALU, about 500 VALU instructions
// per 16-token tile) this leaves a tile 4 + 16 MFMAs and a few dozen VALU
// instructions, so the waves spend their time waiting on the gather instead.
constexpr int kPvTile = 16;
constexpr int kPvMaxTps = 2048;
constexpr int kPvRowBytes = 512;

__device__ __forceinline__ int pv_swz(int r) { return 2 * (r & 7) | ((r >> 3) & 1); }

// Attention of head tile `ht` of pair `p` over the ntok kept tokens tix[0 ..
// ntok) (ntok <= 4 * RPW; tix in global memory or LDS; entries -1 or >= N are
// skipped); writes the partial (m, l, -, -, o[128]) of each of the HT heads to
// dst. LDS (separate objects, so that reading one tile buffer does not wait
// for the loads into the other): tA and tB the wave-private tile buffers, rows
// the waves' token rows, c_lds and ml_lds the rescale factors and (m, l) of
// the four waves. COHERENT: the partial is stored with agent-scope atomic
// stores (store_agent), for a reader in another workgroup of the same launch.
// The rows of a wave's tiles (see attend_pv_range), lane L those of its tiles
// L/16, L/16 + 4, ..: every token (and slot) load of the lane is issued
// before the first is used, so the list costs one memory round trip, not one
// per group of four tiles. All MI groups are stored (-1 past the wave's
// tiles): with the stores under a condition, the compiler made every
// iteration of the tile loop after it wait for all loads in flight. Returns
// the lane's smallest valid row (0xFFFFFFFF: none).
template <bool SMAP, int MI>
__device__ __forceinline__ uint32_t pv_resolve_rows(int32_t* rw, const int32_t* tix, int ntok, int mt_w,
                                                 const int32_t* smap, int64_t N, int bs, int slots) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int tok[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = (lane >> 4) + 4 * i;
    const int k = (wave + 4 * m) * kPvTile + (lane & 15);
    tok[i] = m < mt_w && k < ntok ? tix[k] : -1;
  }
  int slot[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    slot[i] = 0;
    if constexpr (SMAP) slot[i] = tok[i] >= 0 && tok[i] < N ? smap[tok[i] / bs] : -1;
  }
  uint32_t vmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = (lane >> 4) + 4 * i;
    int r = -1;
    if (tok[i] >= 0 && tok[i] < N) {
      if constexpr (SMAP) {
        if (slot[i] >= 0 && slot[i] < slots) r = slot[i] * bs + tok[i] % bs;
      } else {
        r = tok[i];
      }
    }
    rw[m * kPvTile + (lane & 15)] = r;
    if (r >= 0) vmin = min(vmin, (uint32_t)r);
  }
  return vmin;
}

template <int HT, bool SMAP, int RPW, bool COHERENT = false>
__device__ __forceinline__ void attend_pv_range(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                                const int32_t* __restrict__ slot_map, const int32_t* tix, int ntok,
                                                float* __restrict__ dst, int Hq, int Hkv, int G, int64_t N,
                                                int64_t Ns, int bs, int64_t NB, int slots, int p, int ht,
                                                float qk_scale, uint8_t (*tA)[kPvTile * kPvRowBytes],
                                                uint8_t (*tB)[kPvTile * kPvRowBytes], int32_t (*rows)[RPW],
                                                float (*c_lds)[16], float (*ml_lds)[16][2]) {
  constexpr int D = 128, DV = 128, KS = D / 32, ROW = D + DV;  // elements per row
  constexpr int TB = kPvTile * kPvRowBytes;                     // bytes per tile buffer
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int b = p / Hkv, h = p % Hkv;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15, kq = lane >> 4;
  const uint16_t* kvp = kv + (SMAP ? (int64_t)p * slots * bs : (int64_t)p * Ns) * ROW;

  // query fragments (B of S^T): head ht*HT + n, rows past G repeat head G-1
  u32x4 qf[KS];
  {
    const int g = min(ht * HT + n, G - 1);
    const uint16_t* qr = q + ((int64_t)b * Hq + (int64_t)h * G + g) * D + 8 * kq;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = ld16(qr + 32 * k);
  }
  // Wave w takes tiles w, w+4, .. of the split (its m-th tile: tokens
  // 16(w+4m) ..). Each wave resolves the rows of its own tiles (-1: masked),
  // lane L those of tiles m = L/16 (mod 4), so that it starts loading without
  // waiting for the others; a masked token loads the wave's smallest valid
  // row. The rows stay in the wave's part of LDS.
  const int ntile_all = (ntok + kPvTile - 1) / kPvTile;
  const int mt_w = ntile_all > wave ? (ntile_all - wave + 3) / 4 : 0;  // this wave's tiles
  int32_t* rw = rows[wave];
  const uint32_t vmin = pv_resolve_rows<SMAP, RPW / kPvTile / 4>(rw, tix, ntok, mt_w, SMAP ? slot_map + (int64_t)p * NB : nullptr,
                                                                 N, bs, slots);
  const uint32_t fbu = wave_umin(vmin);
  const int fb = fbu == 0xFFFFFFFFu ? -1 : (int)fbu;
  const int ntw = fb < 0 ? 0 : mt_w;  // a wave without a valid row has nothing to add
  wait_vmcnt<0>();  // q and the token lists are in: the loop's only vector loads are the direct ones
  wave_lds_sync();

  // the wave's tile m into buffer `dst`: load i fills rows 2i, 2i+1 (lanes
  // 0-31, 32-63), lane L bringing global piece (L&31) ^ swz(row) to position L&31
  auto issue = [&](uint8_t* dst, int m) {
#pragma unroll
    for (int i = 0; i < kPvTile / 2; ++i) {
      const int r = 2 * i + (lane >> 5);
      const int row = rw[m * kPvTile + r];
      const int piece = (lane & 31) ^ pv_swz(r);
      const uint16_t* src = kvp + (int64_t)(row >= 0 ? row : fb) * ROW + piece * 8;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
    }
  };

  float m_run = -INFINITY, l_part = 0.0f;  // head n (m common over kq)
  f32x4 o[DV / 16];
#pragma unroll
  for (int t = 0; t < DV / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* tb, int j) {
    // ---- S^T: lane (head n, kq) gets tokens 4kq+i ----
    u32x4 kf[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k)
      kf[k] = *reinterpret_cast<const u32x4*>(tb + n * kPvRowBytes + (((4 * k + kq) ^ pv_swz(n)) * 16));
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) sc = mfma16x16x32(kf[k], qf[k], sc);
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = rw[j * kPvTile + 4 * kq + i] >= 0 ? sc[i] * qk_scale : -INFINITY;
    const float tmax = max_rows(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    const float m_new = fmaxf(m_run, tmax);
    const float ref = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = exp2f(m_run - ref);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2f(z[i] - ref);
    l_part = l_part * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m_run = m_new;
    // P as hi + lo bf16: A of the 16x16x16 product, k = token 4kq+i
    u32x2 phi, plo;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
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
      for (int t = 0; t < DV / 16; ++t) o[t] *= cr;
      wave_lds_sync();
    }
    // ---- O += P V: lane a of a 16-lane group addresses row 4kq + a/4,
    // channels 16t + 4(a%4) .. +3 (piece 16 + 2t + (a%4)/2, byte 8*(a&1)) ----
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const int vr = 4 * kq + (n >> 2);
    const uint8_t* vrow = tb + vr * kPvRowBytes + 8 * (n & 1);
    const int vsw = pv_swz(vr), vp = 16 + ((n >> 1) & 1);
    const s16x4 pa = __builtin_bit_cast(s16x4, phi), pb = __builtin_bit_cast(s16x4, plo);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t) {
      const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow + ((vp + 2 * t) ^ vsw) * 16));
      const s16x4 vb = __builtin_bit_cast(s16x4, v);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vb, o[t], 0, 0, 0);
    }
  };

  // wave-private double buffer: the wave's even tiles in tA, odd ones in tB.
  // Two tiles are in flight whenever the wave waits: a buffer is refilled
  // (tile m+2) as soon as tile m has been computed from it, and the wave then
  // waits only for tile m+1 (vmcnt <= 8: the 8 loads of tile m+2 are the
  // younger ones). The waits are the builtin's, which the compiler accounts
  // for, and the buffers are separate LDS objects, so reading one buffer does
  // not also wait for the loads into the other. Tile m's LDS reads have all
  // returned before its last MFMAs issue, so the refill cannot overtake them.
  static_assert(kPvTile / 2 == 8, "the waits below count 8 loads per tile");
  if (ntw > 0) issue(tA[wave], 0);
  if (ntw > 1) issue(tB[wave], 1);
  for (int m = 0; m < ntw; m += 2) {
    if (m + 1 < ntw) wait_vmcnt<8>(); else wait_vmcnt<0>();
    compute(tA[wave], m);
    if (m + 2 < ntw) issue(tA[wave], m + 2);
    if (m + 1 >= ntw) break;
    if (m + 2 < ntw) wait_vmcnt<8>(); else wait_vmcnt<0>();
    compute(tB[wave], m + 1);
    if (m + 3 < ntw) issue(tB[wave], m + 3);
  }
  wait_vmcnt<0>();
  // ---- the workgroup partial: per head (m, l, -, -, o[DV]) ----
  const float l_tot = sum_rows(l_part);
  if (kq == 0) {
    ml_lds[wave][n][0] = m_run;
    ml_lds[wave][n][1] = l_tot;
  }
  __syncthreads();
  // this wave's o scaled to the common max, into its own (now idle) buffer
  // as [channel][16 heads]: one 16-byte write per lane and channel tile
  {
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * kq + i;
      float ms = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) ms = fmaxf(ms, ml_lds[w][hh][0]);
      const float mw = ml_lds[wave][hh][0];
      f[i] = mw == -INFINITY ? 0.0f : exp2f(mw - ms);
    }
    f32x4* ow = reinterpret_cast<f32x4*>(tA[wave]);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
      ow[(16 * t + n) * 4 + kq] = f32x4{f[0] * o[t][0], f[1] * o[t][1], f[2] * o[t][2], f[3] * o[t][3]};
  }
  __syncthreads();
  if (tid < HT) {
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) ms = fmaxf(ms, ml_lds[w][tid][0]);
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = ml_lds[w][tid][0];
      l += mw == -INFINITY ? 0.0f : ml_lds[w][tid][1] * exp2f(mw - ms);
    }
    if constexpr (COHERENT)
      store_agent2(dst + tid * (DV + kPartHdr), ms, l);
    else
      *reinterpret_cast<f32x4*>(dst + tid * (DV + kPartHdr)) = f32x4{ms, l, 0.0f, 0.0f};
  }
  // thread (channel c, heads 8*(tid/128) ..): the sum over the four waves
  {
    const int c = tid & (DV - 1);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g4 = 2 * (tid >> 7) + gg;  // heads 4*g4 .. 4*g4+3
      if (4 * g4 >= HT) continue;
      f32x4 acc = reinterpret_cast<const f32x4*>(tA[0])[c * 4 + g4];
#pragma unroll
      for (int w = 1; w < 4; ++w) acc += reinterpret_cast<const f32x4*>(tA[w])[c * 4 + g4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g4 + i < HT) {
          float* d = &dst[(4 * g4 + i) * (DV + kPartHdr) + kPartHdr + c];
          if constexpr (COHERENT)
            store_agent(d, acc[i]);
          else
            *d = acc[i];
        }
    }
  }
}
}  // namespace tls

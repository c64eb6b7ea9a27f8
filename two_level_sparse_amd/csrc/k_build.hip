// k_build.hip -- block summaries and INT4 label cache (once per cache).
//
// AsyncTLS pages, section 2A: the cache is split into blocks, each indexed by
// a compressed key summary (per-channel maximum and minimum) for the coarse
// stage, and the keys are kept on a few label channels in INT4 for the fine
// stage. This kernel streams K once and writes both indices.
//
// Grid: (ceil(NB/4), pairs); 4 wavefronts per workgroup, one block per wave.
// Every key row of a block is read once: lane l holds channels 2l + 128k,
// 2l + 128k + 1 (k < ceil(D/128)) of each token as one 4-byte word, keeps the
// per-channel maximum and minimum in registers, and the lanes that hold a
// label channel leave its value in LDS; lane i then quantises token i (bs <= 64)
// from there, in double so that the codes are exactly those of the definition.
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {

// INT4 label codes of one token from its label-channel values v(0..r-1):
// symmetric absmax (a == 0: scale 0, codes 0; otherwise scale = float(a / 7)
// and code_i = clamp(rint(v_i / scale), -7, 7), both divisions in double),
// packed two per byte (channel i in byte i/2, low nibble for even i).
template <int RMAX, class Get>
__device__ __forceinline__ void quantize_vals(Get v_of, int r, uint8_t* cp, float* sc_out) {
  float v[RMAX];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < RMAX; ++i) {
    v[i] = i < r ? v_of(i) : 0.0f;
    a = fmaxf(a, fabsf(v[i]));
  }
  float sc = 0.0f;
  int code[RMAX];
  if (a == 0.0f) {
#pragma unroll
    for (int i = 0; i < RMAX; ++i) code[i] = 0;
  } else {
    sc = (float)((double)a / 7.0);
    const double dsc = (double)sc;
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
      double qv = rint((double)v[i] / dsc);
      qv = qv > 7.0 ? 7.0 : (qv < -7.0 ? -7.0 : qv);
      code[i] = (int)qv;
    }
  }
#pragma unroll
  for (int i = 0; i < RMAX; i += 2)
    if (i < r) cp[i / 2] = (uint8_t)((code[i] & 0xF) | ((code[i + 1] & 0xF) << 4));
  *sc_out = sc;
}

// The same for a token row in global memory and the head's label channels.
template <int RMAX>
__device__ __forceinline__ void quantize_row(const uint16_t* rowp, const int32_t* lab, int r, uint8_t* cp,
                                             float* sc_out) {
  quantize_vals<RMAX>([&](int i) { return bf2f(rowp[lab[i]]); }, r, cp, sc_out);
}

template <int RMAX, int KCH>
__global__ __launch_bounds__(256) void k_build(const uint16_t* __restrict__ kv, const int32_t* __restrict__ label_ch,
                                               uint16_t* __restrict__ summ, uint8_t* __restrict__ codes,
                                               float* __restrict__ scale, int Hkv, int D, int row, int64_t N, int bs,
                                               int r, int64_t NB, int64_t Ns, int64_t NBs, int64_t j_first) {
  constexpr int U = KCH == 1 ? 16 : (KCH == 2 ? 8 : 4);  // token rows in flight per wave
  constexpr int LS = RMAX + 2;  // LDS row of label values (bf16): an odd word count, so the
                                // quantiser's row reads fall in distinct banks
  __shared__ uint16_t lab_s[4][64 * LS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = j_first + (int64_t)blockIdx.x * 4 + wave;
  const int p = blockIdx.y;
  const bool live = j < NB;
  const int64_t t0 = j * bs;
  const int nt = live ? (int)((t0 + bs < N ? t0 + bs : N) - t0) : 0;  // valid tokens of block j (>= 1)
  uint16_t* ls = lab_s[wave];

  if (live) {
    const int32_t* lab = label_ch + (int64_t)(p % Hkv) * r;
    // Label slot of this lane's channels 2*lane + 128k + e, or -1.
    int li[KCH][2];
#pragma unroll
    for (int k = 0; k < KCH; ++k) li[k][0] = li[k][1] = -1;
    for (int i = 0; i < r; ++i) {
      const int ch = lab[i], cpair = ch >> 1;
      if ((cpair & 63) == lane) {
#pragma unroll
        for (int k = 0; k < KCH; ++k)
          if ((cpair >> 6) == k) {
            if (ch & 1)
              li[k][1] = i;
            else
              li[k][0] = i;
          }
      }
    }
    // Channel offset of word k; lanes past D in the last word read channel 0
    // instead (in bounds) and discard it.
    int off[KCH];
#pragma unroll
    for (int k = 0; k < KCH; ++k) off[k] = (2 * lane + 128 * k < D) ? 2 * lane + 128 * k : 0;
    const uint16_t* base = kv + ((int64_t)p * Ns + t0) * row;

    float mx[KCH][2], mn[KCH][2];
#pragma unroll
    for (int k = 0; k < KCH; ++k) mx[k][0] = mx[k][1] = -INFINITY, mn[k][0] = mn[k][1] = INFINITY;
    for (int u0 = 0; u0 < nt; u0 += U) {
      uint32_t w[U][KCH];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tt = u0 + u < nt ? u0 + u : nt - 1;  // past the block's end: its last row again
#pragma unroll
        for (int k = 0; k < KCH; ++k) w[u][k] = *reinterpret_cast<const uint32_t*>(base + tt * row + off[k]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = u0 + u < nt;
#pragma unroll
        for (int k = 0; k < KCH; ++k) {
          const float a = bf_lo(w[u][k]), b = bf_hi(w[u][k]);
          mx[k][0] = fmaxf(mx[k][0], in ? a : -INFINITY);
          mn[k][0] = fminf(mn[k][0], in ? a : INFINITY);
          mx[k][1] = fmaxf(mx[k][1], in ? b : -INFINITY);
          mn[k][1] = fminf(mn[k][1], in ? b : INFINITY);
          if (in && li[k][0] >= 0) ls[(u0 + u) * LS + li[k][0]] = (uint16_t)(w[u][k] & 0xFFFFu);
          if (in && li[k][1] >= 0) ls[(u0 + u) * LS + li[k][1]] = (uint16_t)(w[u][k] >> 16);
        }
      }
    }
    // Summaries in tile-fragment order (channels c, c+1 stay adjacent: one
    // 4-byte store each). Extremes of bf16 values are bf16 values: keep the
    // upper 16 bits.
    uint16_t* sp = summ + (int64_t)p * summ_pair_elems(NBs, D);
    const int KC = D / 32;
#pragma unroll
    for (int k = 0; k < KCH; ++k) {
      const int c = 2 * lane + 128 * k;
      if (c < D) {
        *reinterpret_cast<uint32_t*>(sp + summ_elem(j, c, 0, KC)) =
            (__float_as_uint(mx[k][0]) >> 16) | (__float_as_uint(mx[k][1]) & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(sp + summ_elem(j, c, 1, KC)) =
            (__float_as_uint(mn[k][0]) >> 16) | (__float_as_uint(mn[k][1]) & 0xFFFF0000u);
      }
    }
  }
  __syncthreads();  // label values of the wave's block are in LDS

  // INT4 label cache: symmetric absmax per token over the label channels.
  if (lane < nt) {
    const int64_t t = t0 + lane;
    const uint16_t* lv = ls + lane * LS;
    quantize_vals<RMAX>([&](int i) { return bf2f(lv[i]); }, r, codes + ((int64_t)p * Ns + t) * (r / 2),
                        scale + (int64_t)p * Ns + t);
  }
}

// Incremental index update for n new rows appended at N0 (rows [pairs, n,
// row] on the device): workgroup (i, p) = one wave for the i-th block that the
// new rows touch. A block's max / min over its valid tokens is the max / min
// of its previous summary (when it already held tokens) and of its new rows,
// exactly, so only the new rows are read -- in particular not the rows already
// offloaded to host memory. The new tokens are quantised as in k_build.
template <int RMAX>
__global__ __launch_bounds__(64) void k_append_index(const uint16_t* __restrict__ rows, int n,
                                                     const int32_t* __restrict__ label_ch, uint16_t* __restrict__ summ,
                                                     uint8_t* __restrict__ codes, float* __restrict__ scale, int Hkv,
                                                     int D, int row, int bs, int r, int64_t N0, int64_t Ns,
                                                     int64_t NBs) {
  const int lane = threadIdx.x, p = blockIdx.y;
  const int64_t j = N0 / bs + blockIdx.x;
  const int64_t t0 = j * bs, ta = t0 > N0 ? t0 : N0, tb = min(t0 + bs, N0 + n);  // new rows of block j
  const bool had = t0 < N0;                                                       // block held tokens before
  const uint16_t* src = rows + (int64_t)p * n * row;
  uint16_t* sp = summ + (int64_t)p * summ_pair_elems(NBs, D);
  const int KC = D / 32;
  for (int c = 2 * lane; c < D; c += 128) {
    uint32_t* pmx = reinterpret_cast<uint32_t*>(sp + summ_elem(j, c, 0, KC));
    uint32_t* pmn = reinterpret_cast<uint32_t*>(sp + summ_elem(j, c, 1, KC));
    float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY;
    if (had) {
      const uint32_t wx = *pmx, wn = *pmn;
      mx0 = bf_lo(wx);
      mx1 = bf_hi(wx);
      mn0 = bf_lo(wn);
      mn1 = bf_hi(wn);
    }
    for (int64_t t = ta; t < tb; ++t) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (t - N0) * row + c);
      const float a = bf_lo(w), b = bf_hi(w);
      mx0 = fmaxf(mx0, a);
      mn0 = fminf(mn0, a);
      mx1 = fmaxf(mx1, b);
      mn1 = fminf(mn1, b);
    }
    *pmx = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xFFFF0000u);
    *pmn = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xFFFF0000u);
  }
  const int64_t t = t0 + lane;
  if (lane < bs && t >= ta && t < tb)
    quantize_row<RMAX>(src + (t - N0) * row, label_ch + (int64_t)(p % Hkv) * r, r,
                       codes + ((int64_t)p * Ns + t) * (r / 2), scale + (int64_t)p * Ns + t);
}

hipError_t launch_append_index(const uint16_t* rows, int n, const int32_t* label_ch, uint16_t* summ, uint8_t* codes,
                               float* scale, int pairs, int Hkv, int D, int row, int bs, int r, int64_t N0,
                               int64_t Ns, int64_t NBs, hipStream_t st) {
  const int64_t nblk = (N0 + n - 1) / bs - N0 / bs + 1;
  dim3 grid((unsigned)nblk, (unsigned)pairs);
  if (r <= 16)
    hipLaunchKernelGGL(k_append_index<16>, grid, dim3(64), 0, st, rows, n, label_ch, summ, codes, scale, Hkv, D,
                       row, bs, r, N0, Ns, NBs);
  else
    hipLaunchKernelGGL(k_append_index<32>, grid, dim3(64), 0, st, rows, n, label_ch, summ, codes, scale, Hkv, D,
                       row, bs, r, N0, Ns, NBs);
  return hipGetLastError();
}

// Appended rows: workgroup (i, p) copies new row i of pair p (row*2 bytes, a
// multiple of 16) to position N0 + i of the pair's cache.
__global__ __launch_bounds__(64) void k_append_rows(const uint16_t* __restrict__ src, uint16_t* __restrict__ kv,
                                                    int n_new, int row, int64_t N0, int64_t Ns) {
  const int i = blockIdx.x, p = blockIdx.y;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + ((int64_t)p * n_new + i) * row);
  u32x4* d = reinterpret_cast<u32x4*>(kv + ((int64_t)p * Ns + N0 + i) * row);
  for (int k = threadIdx.x; k < row / 8; k += 64) d[k] = s[k];
}

hipError_t launch_append_rows(const uint16_t* src, uint16_t* kv, int pairs, int n_new, int row, int64_t N0,
                              int64_t Ns, hipStream_t st) {
  hipLaunchKernelGGL(k_append_rows, dim3((unsigned)n_new, (unsigned)pairs), dim3(64), 0, st, src, kv, n_new, row, N0,
                     Ns);
  return hipGetLastError();
}

template <int RMAX, int KCH>
static void launch_build_t(const BuildArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.NB - a.j_first + 3) / 4), (unsigned)a.pairs);
  hipLaunchKernelGGL((k_build<RMAX, KCH>), grid, dim3(256), 0, st, a.kv, a.label_ch, a.summ, a.codes, a.scale, a.Hkv,
                     a.D, a.row, a.N, a.bs, a.r, a.NB, a.Ns, a.NBs, a.j_first);
}

template <int RMAX>
static void launch_build_r(const BuildArgs& a, hipStream_t st) {
  switch ((a.D + 127) / 128) {
    case 1: launch_build_t<RMAX, 1>(a, st); break;
    case 2: launch_build_t<RMAX, 2>(a, st); break;
    case 3: launch_build_t<RMAX, 3>(a, st); break;
    case 4: launch_build_t<RMAX, 4>(a, st); break;
    default: launch_build_t<RMAX, 5>(a, st); break;  // D <= 576
  }
}

hipError_t launch_build(const BuildArgs& a, hipStream_t st) {
  if (a.r <= 16)
    launch_build_r<16>(a, st);
  else
    launch_build_r<32>(a, st);
  return hipGetLastError();
}

}  // namespace tls

// k_build.hip -- block summaries and INT4 label cache (once per cache).
//
// AsyncTLS pages, section 2A: the cache is split into blocks, each indexed by
// a compressed key summary (per-channel maximum and minimum) for the coarse
// stage, and the keys are kept on a few label channels in INT4 for the fine
// stage. This kernel streams K once and writes both indices.
//
// Grid: (ceil(NB/4), pairs); 4 wavefronts per workgroup, one block per wave.
//  - summaries: lane c owns channel pairs (2c, 2c+1), (2c+128, 2c+129), ...;
//    each token row is read as coalesced 4-byte words.
//  - label cache: lane i owns token i of the block (bs <= 64); the quantiser
//    runs in double so the codes are exactly those of the definition.
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {

template <int RMAX>
__global__ __launch_bounds__(256) void k_build(const uint16_t* __restrict__ kv, const int32_t* __restrict__ label_ch,
                                               uint16_t* __restrict__ summ, uint8_t* __restrict__ codes,
                                               float* __restrict__ scale, int Hkv, int D, int row, int64_t N, int bs,
                                               int r, int64_t NB, int64_t Ns, int64_t NBs, int64_t j_first) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = j_first + (int64_t)blockIdx.x * 4 + wave;
  const int p = blockIdx.y;
  if (j >= NB) return;
  const int h = p % Hkv;
  const uint16_t* base = kv + (int64_t)p * Ns * row;
  const int64_t t0 = j * bs;
  const int64_t t1 = t0 + bs < N ? t0 + bs : N;

  // Per-channel max / min over the valid tokens of block j.
  uint16_t* smax = summ + ((int64_t)p * NBs + j) * 2 * D;
  uint16_t* smin = smax + D;
  for (int c = 2 * lane; c < D; c += 128) {
    float mx0 = -INFINITY, mx1 = -INFINITY, mn0 = INFINITY, mn1 = INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(base + t * row + c);
      float a = bf_lo(w), b = bf_hi(w);
      mx0 = fmaxf(mx0, a);
      mn0 = fminf(mn0, a);
      mx1 = fmaxf(mx1, b);
      mn1 = fminf(mn1, b);
    }
    // Extremes of bf16 values are bf16 values: keep the upper 16 bits.
    *reinterpret_cast<uint32_t*>(smax + c) = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xFFFF0000u);
    *reinterpret_cast<uint32_t*>(smin + c) = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xFFFF0000u);
  }

  // INT4 label cache: symmetric absmax per token over the label channels.
  const int64_t t = t0 + lane;
  if (lane < bs && t < N) {
    const uint16_t* rowp = base + t * row;
    const int32_t* lab = label_ch + (int64_t)h * r;
    float v[RMAX];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
      v[i] = i < r ? bf2f(rowp[lab[i]]) : 0.0f;
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
    uint8_t* cp = codes + ((int64_t)p * Ns + t) * (r / 2);
#pragma unroll
    for (int i = 0; i < RMAX; i += 2)
      if (i < r) cp[i / 2] = (uint8_t)((code[i] & 0xF) | ((code[i + 1] & 0xF) << 4));
    scale[(int64_t)p * Ns + t] = sc;
  }
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

hipError_t launch_build(const BuildArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.NB - a.j_first + 3) / 4), (unsigned)a.pairs);
  if (a.r <= 16)
    hipLaunchKernelGGL(k_build<16>, grid, dim3(256), 0, st, a.kv, a.label_ch, a.summ, a.codes, a.scale, a.Hkv, a.D,
                       a.row, a.N, a.bs, a.r, a.NB, a.Ns, a.NBs, a.j_first);
  else
    hipLaunchKernelGGL(k_build<32>, grid, dim3(256), 0, st, a.kv, a.label_ch, a.summ, a.codes, a.scale, a.Hkv, a.D,
                       a.row, a.N, a.bs, a.r, a.NB, a.Ns, a.NBs, a.j_first);
  return hipGetLastError();
}

}  // namespace tls

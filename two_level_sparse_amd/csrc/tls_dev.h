// tls_dev.h -- device helpers shared by the gfx950 kernels of libtls.
// (Internal to the HIP library; not part of the C ABI.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tls {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bit pattern <-> float (exact widening).
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 16-byte global load (8 bf16 / 4 words); pointer must be 16-byte aligned.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Block summaries in tile-fragment order: per (batch, kv head) pair, tiles of
// 16 blocks; in tile T, 32-channel chunk c and m (0: Kmax, 1: Kmin) form one
// 512-element unit whose element (kq*16 + n)*8 + e holds channel 32c + 8kq + e
// of block 16T + n -- exactly the B fragment of a 16x16x32 MFMA with the tile's
// blocks as columns, so lane L of a fragment load reads elements 8L .. 8L+7
// and every load is 1 KB contiguous.
__host__ __device__ constexpr int64_t summ_tiles(int64_t nblocks) { return (nblocks + 15) / 16; }
// elements per pair for NBs blocks of capacity
__host__ __device__ constexpr int64_t summ_pair_elems(int64_t NBs, int D) { return summ_tiles(NBs) * 32 * D; }
// element offset, within a pair, of unit (tile T, chunk c, m); KC = D / 32
__host__ __device__ constexpr int64_t summ_unit(int64_t T, int c, int m, int KC) {
  return ((T * KC + c) * 2 + m) * 512;
}
// element offset, within a pair, of channel ch of block j's summary m
__host__ __device__ constexpr int64_t summ_elem(int64_t j, int ch, int m, int KC) {
  return summ_unit(j / 16, ch / 32, m, KC) + (((ch % 32) / 8) * 16 + j % 16) * 8 + ch % 8;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One 16x16x32 bf16 MFMA: acc[m][n] += sum_k a[m][k] * b[k][n].
// a: row m = lane%16; b: column n = lane%16; both carry the same 8 k-values
// per lane. Result: lane holds rows 4*(lane/16)+i (i=0..3) of column lane%16.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}

// Float -> 32-bit key whose unsigned order is the numeric order (-0 folded to +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rn(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Inverse of order_key for keys of finite floats.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- cross-lane helpers on DPP (data-parallel primitives: register moves
// between lanes of a 16-lane row, no LDS round trip) and readlane.
enum : int {
  kDppQuadXor1 = 0xB1,     // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,     // quad_perm [2,3,0,1]
  kDppRowShr1 = 0x111,     // row_shr:1 (lanes without a source read 0)
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowMirror = 0x140,
  kDppRowHalfMirror = 0x141,
};
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }

// Reductions across the 16 lanes of a row (lanes that share lane/16); every
// lane of the row receives the result.
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dppf<kDppQuadXor1>(v));
  v = fmaxf(v, dppf<kDppQuadXor2>(v));
  v = fmaxf(v, dppf<kDppRowHalfMirror>(v));
  v = fmaxf(v, dppf<kDppRowMirror>(v));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += dppf<kDppQuadXor1>(v);
  v += dppf<kDppQuadXor2>(v);
  v += dppf<kDppRowHalfMirror>(v);
  v += dppf<kDppRowMirror>(v);
  return v;
}
__device__ __forceinline__ uint32_t umin16(uint32_t v) {
  v = min(v, dpp<kDppQuadXor1>(v));
  v = min(v, dpp<kDppQuadXor2>(v));
  v = min(v, dpp<kDppRowHalfMirror>(v));
  return min(v, dpp<kDppRowMirror>(v));
}
__device__ __forceinline__ uint32_t umax16(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppRowHalfMirror>(v));
  return max(v, dpp<kDppRowMirror>(v));
}
__device__ __forceinline__ uint32_t usum16(uint32_t v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  return v + dpp<kDppRowMirror>(v);
}
// Whole-wave reductions (result uniform).
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = umin16(v);
  return min(min(readlane(v, 0), readlane(v, 16)), min(readlane(v, 32), readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = umax16(v);
  return max(max(readlane(v, 0), readlane(v, 16)), max(readlane(v, 32), readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_usum(uint32_t v) {
  v = usum16(v);
  return readlane(v, 0) + readlane(v, 16) + readlane(v, 32) + readlane(v, 48);
}
// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<kDppRowShr1>(v);
  v += dpp<kDppRowShr2>(v);
  v += dpp<kDppRowShr4>(v);
  v += dpp<kDppRowShr8>(v);
  const uint32_t r0 = readlane(v, 15), r1 = readlane(v, 31), r2 = readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t add = row == 0 ? 0u : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2;
  return v + add;
}

// Max / sum over the four 16-lane rows of the wave; every lane receives the
// result for its column (lane % 16). The swaps pair rows (l, l^32), then
// (l, l^16).
__device__ __forceinline__ float max_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Raw buffer resource over `bytes` bytes at `base`: loads beyond the range
// return 0 and stores beyond it are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// v[e] = row[first + e] for first + e < n, else 0, via bounded buffer loads
// (no branches, so all PER loads are in flight together). When n is a
// multiple of 4 and PER of 4, 16-byte loads (a group is wholly in or out).
template <int PER>
__device__ __forceinline__ void load_row_f32(const float* row, int n, int first, float (&v)[PER]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, n * 4);
  if (PER % 4 == 0 && (n & 3) == 0) {
#pragma unroll
    for (int e = 0; e < PER; e += 4) {
      const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (first + e) * 4, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) v[e + i] = __uint_as_float(w[i]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (first + e) * 4, 0, 0));
  }
}

// Relaxed atomic accesses at agent scope (global_store / global_load with
// sc1): coherent between the workgroups of one launch whatever XCDs they run
// on, without writing back or invalidating any L2. One workgroup publishes
// data this way, waits for its stores (s_waitcnt) and then counts with an
// agent-scope atomic; the workgroup that reads the final count loads the data
// the same way.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent2(float* p, float a, float b) {  // p 8-byte aligned
  const uint64_t w = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {  // p 8-byte aligned
  const uint64_t w = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32))};
}

// s_waitcnt vmcnt(N): at most N vector memory loads of this wave in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS traffic only: the fences are limited to
// the local address space, so vector memory loads still in flight (global
// data a thread fetched for later) are not waited for at the barrier.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders LDS traffic between lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace tls

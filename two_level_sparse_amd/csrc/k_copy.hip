// k_copy.hip -- one-launch incremental block transfer for the staggered
// offload (AsyncTLS pages, section 2B: only the blocks of T_t = M_t \ C_t
// cross the host link).
//
// k_gather_blocks: workgroup i copies block i of the step's transfer list
// from pinned host memory (read through its device mapping, over the host
// link) into its resident slot, 16 bytes per lane per access; workgroups past
// the block list apply the slot-map changes. The list itself also sits in
// pinned host memory, so a step costs one launch whatever the number of
// blocks.
#include "tls_dev.h"
#include "tls_launch.h"

namespace tls {

// One block of a transfer list, by one 256-thread workgroup: the loads of 8
// 16-byte pieces per thread are in flight together (each crosses the host
// link), then the stores.
__device__ __forceinline__ void copy_block(const uint16_t* __restrict__ host_kv, uint16_t* __restrict__ dev_cache,
                                           const CopyItem it, int64_t block_elems) {
  const u32x4* src = reinterpret_cast<const u32x4*>(host_kv + it.src_elem);
  u32x4* dst = reinterpret_cast<u32x4*>(dev_cache + it.dst_elem);
  const int64_t n16 = block_elems / 8;
  constexpr int U = 8;
  for (int64_t base = 0; base < n16; base += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = base + u * 256 + threadIdx.x;
      v[u] = src[k < n16 ? k : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = base + u * 256 + threadIdx.x;
      if (k < n16) dst[k] = v[u];
    }
  }
}

__global__ __launch_bounds__(256) void k_gather_blocks(const uint16_t* __restrict__ host_kv,
                                                       uint16_t* __restrict__ dev_cache,
                                                       const CopyItem* __restrict__ items, int nitems,
                                                       const MapItem* __restrict__ map_items, int nmap,
                                                       int32_t* __restrict__ slot_map, int64_t block_elems) {
  const int i = blockIdx.x;
  if (i < nitems) {
    copy_block(host_kv, dev_cache, items[i], block_elems);
    return;
  }
  for (int64_t k = (int64_t)(i - nitems) * blockDim.x + threadIdx.x; k < nmap; k += (int64_t)blockDim.x * 64) {
    const MapItem m = map_items[k];
    slot_map[m.index] = m.value;
  }
}

hipError_t launch_gather_blocks(const uint16_t* host_kv_dev, uint16_t* dev_cache, const CopyItem* items, int nitems,
                                const MapItem* map_items, int nmap, int32_t* slot_map, int64_t block_elems,
                                hipStream_t st) {
  const int map_wgs = nmap > 0 ? 64 : 0;
  if (nitems + map_wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_blocks, dim3(nitems + map_wgs), dim3(256), 0, st, host_kv_dev, dev_cache, items, nitems,
                     map_items, nmap, slot_map, block_elems);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Device-planned transfer (TLS_COPY_DEVICE): the same rules as the host
// engine, applied on the GPU so that a step never waits for the host.
// k_delta_plan, one workgroup per pair:
//   T_t = the blocks of M_t that are not resident (ascending, as M_t is);
//   free slots first; if they do not suffice, evict resident blocks outside
//   M_{t-1} u M_t in order of (last step selected, block number) -- a bitonic
//   sort of at most kDeltaMaxCap keys in LDS; T_t[i] goes to the i-th free slot
//   in ascending order; the slot map of step t+1 is map t with these changes.
// k_copy_listed then moves the listed blocks.

// The map of step t+1 starts as the map of step t: all loads of a round in
// flight before its stores (the two maps are distinct buffers).
__device__ __forceinline__ void copy_map(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int NB, int tid) {
  constexpr int R = 16;
  int base = 0;
  for (; base + 256 * R <= NB; base += 256 * R) {  // whole rounds, no per-element branches
    int32_t v[R];
#pragma unroll
    for (int u = 0; u < R; ++u) v[u] = src[base + u * 256 + tid];
#pragma unroll
    for (int u = 0; u < R; ++u) dst[base + u * 256 + tid] = v[u];
  }
  for (int i = base + tid; i < NB; i += 256) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_delta_plan(DeltaArgs a) {
  __shared__ uint32_t inm[kDeltaMaxNB / 32];      // M_{t-1} u M_t
  __shared__ uint32_t freeb[kDeltaMaxCap / 32];   // free slots
  __shared__ uint32_t wpre[kDeltaMaxCap / 32];    // free slots in the words before
  __shared__ unsigned long long cand[kDeltaMaxCap];
  __shared__ int32_t T[kDeltaMaxCap / 2];
  __shared__ uint32_t scan_sh[4];
  __shared__ uint32_t nfree_sh, bad_sh;
  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = a.NB, kb = a.kb, cap = a.cap;
  const int32_t step = *a.step_ctr;
  const int32_t* M = a.M + (int64_t)p * kb;
  int32_t* prev = a.prev + (int64_t)p * kb;
  int32_t* owner = a.owner + (int64_t)p * cap;
  int32_t* last = a.last + (int64_t)p * NB;
  const int32_t* map_cur = a.map_cur + (int64_t)p * NB;
  int32_t* map_next = a.map_next + (int64_t)p * NB;

  for (int i = tid; i < (NB + 31) / 32; i += 256) inm[i] = 0u;
  for (int i = tid; i < kDeltaMaxCap / 32; i += 256) freeb[i] = 0u;
  if (tid == 0) nfree_sh = bad_sh = 0u;
  copy_map(map_cur, map_next, NB, tid);
  __syncthreads();
  for (int i = tid; i < kb; i += 256) {
    const int b = M[i], bp = prev[i];
    if ((unsigned)b >= (unsigned)a.NBv) {
      bad_sh = 1u;
      continue;
    }
    atomicOr(&inm[b >> 5], 1u << (b & 31));
    atomicOr(&inm[bp >> 5], 1u << (bp & 31));
  }
  __syncthreads();
  if (bad_sh) {  // M_t holds a block number outside [0, NBv): nothing is changed
    if (tid == 0) {
      *a.err = 2;
      a.counts[p] = 0;
    }
    return;
  }
  uint32_t nf = 0u;
  for (int sl = tid; sl < cap; sl += 256)
    if (owner[sl] < 0) {
      atomicOr(&freeb[sl >> 5], 1u << (sl & 31));
      ++nf;
    }
  if (nf) atomicAdd(&nfree_sh, nf);
  // T_t in order: thread t looks at entries 2t and 2t+1 of M_t (kb <= 512)
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const bool f0 = i0 < kb && map_cur[M[i0]] < 0;
  const bool f1 = i1 < kb && map_cur[M[i1]] < 0;
  const uint32_t cnt = (uint32_t)f0 + (uint32_t)f1;
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == 63) scan_sh[wave] = incl;
  __syncthreads();
  uint32_t before = 0u, nT = 0u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? scan_sh[w] : 0u;
    nT += scan_sh[w];
  }
  const uint32_t pos = before + incl - cnt;
  if (f0) T[pos] = M[i0];
  if (f1) T[pos + (uint32_t)f0] = M[i1];
  const int need = (int)nT - (int)nfree_sh;
  if (need > 0) {
    int n2 = 1;
    while (n2 < cap) n2 <<= 1;
    for (int sl = tid; sl < n2; sl += 256) {
      unsigned long long key = ~0ull;
      if (sl < cap) {
        const int blk = owner[sl];
        if (blk >= 0 && !((inm[blk >> 5] >> (blk & 31)) & 1u))
          key = ((unsigned long long)(uint32_t)(last[blk] + 2) << 32) | ((unsigned long long)(uint32_t)blk << 10) |
                (unsigned long long)sl;
      }
      cand[sl] = key;
    }
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += 256) {
          const int ij = i ^ j;
          if (ij > i) {
            const unsigned long long x = cand[i], y = cand[ij];
            if ((x > y) == ((i & k) == 0)) {
              cand[i] = y;
              cand[ij] = x;
            }
          }
        }
        __syncthreads();
      }
    if (cand[need - 1] == ~0ull) {  // cannot happen with 2*Kb' slots; reported by the host queries
      if (tid == 0) {
        *a.err = 1;
        a.counts[p] = 0;
      }
      return;
    }
    for (int k = tid; k < need; k += 256) {
      const unsigned long long key = cand[k];
      const int sl = (int)(key & 1023u), blk = (int)((key >> 10) & 0x3FFFFFu);
      owner[sl] = -1;
      map_next[blk] = -1;
      atomicOr(&freeb[sl >> 5], 1u << (sl & 31));
    }
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t wcnt = lane < kDeltaMaxCap / 32 ? (uint32_t)__popc(freeb[lane]) : 0u;
    const uint32_t winc = wave_incl_scan(wcnt);
    if (lane < kDeltaMaxCap / 32) wpre[lane] = winc - wcnt;
  }
  __syncthreads();
  for (int sl = tid; sl < cap; sl += 256) {
    const uint32_t w = freeb[sl >> 5];
    if ((w >> (sl & 31)) & 1u) {
      const uint32_t rank = wpre[sl >> 5] + (uint32_t)__popc(w & ((1u << (sl & 31)) - 1u));
      if (rank < nT) {
        const int blk = T[rank];
        owner[sl] = blk;
        map_next[blk] = sl;
        a.items[(int64_t)p * kb + rank] =
            CopyItem{((int64_t)p * a.N + (int64_t)blk * a.bs) * a.row, ((int64_t)p * cap + sl) * a.block_elems};
      }
    }
  }
  for (int i = tid; i < kb; i += 256) {
    last[M[i]] = step;
    prev[i] = M[i];
    a.tblocks[(int64_t)p * kb + i] = i < (int)nT ? T[i] : -1;
  }
  if (tid == 0) {
    a.counts[p] = (int32_t)nT;
    atomicAdd(a.total, (unsigned long long)nT);
  }
}

// Full transfer (TLS_COPY_FULL, the baseline without reuse): every block of
// M_t is copied, block i into slot h*kb + i of the half h = (t+1)&1 of the
// resident cache -- the half the step reading M_{t-1} does not use (the
// prologue's M_{-1} sits in half 0) -- and the map of step t+1 holds exactly
// M_t.
__global__ __launch_bounds__(256) void k_full_plan(DeltaArgs a) {
  __shared__ uint32_t bad_sh;
  const int p = blockIdx.x, tid = threadIdx.x;
  const int NB = a.NB, kb = a.kb;
  const int32_t step = *a.step_ctr;
  const int h = (step + 1) & 1;
  const int32_t* M = a.M + (int64_t)p * kb;
  int32_t* prev = a.prev + (int64_t)p * kb;
  int32_t* map_next = a.map_next + (int64_t)p * NB;
  if (tid == 0) bad_sh = 0u;
  copy_map(a.map_cur + (int64_t)p * NB, map_next, NB, tid);
  __syncthreads();
  for (int i = tid; i < kb; i += 256)
    if ((unsigned)M[i] >= (unsigned)a.NBv) bad_sh = 1u;
  __syncthreads();
  if (bad_sh) {  // M_t holds a block number outside [0, NBv): the map stays that of M_{t-1}
    if (tid == 0) {
      *a.err = 2;
      a.counts[p] = 0;
    }
    return;
  }
  for (int i = tid; i < kb; i += 256) map_next[prev[i]] = -1;
  __syncthreads();
  for (int i = tid; i < kb; i += 256) {
    const int blk = M[i], sl = h * kb + i;
    map_next[blk] = sl;
    a.items[(int64_t)p * kb + i] =
        CopyItem{((int64_t)p * a.N + (int64_t)blk * a.bs) * a.row, ((int64_t)p * a.cap + sl) * a.block_elems};
    a.tblocks[(int64_t)p * kb + i] = blk;
    prev[i] = blk;
  }
  if (tid == 0) {
    a.counts[p] = kb;
    atomicAdd(a.total, (unsigned long long)kb);
  }
}

// The listed blocks of all pairs, taken in pair order as one list, by a small
// persistent grid: workgroup w moves list entries w, w+G, w+2G, ... . Reads of
// host memory wait on the host link for microseconds; a few workgroups already
// keep enough of them in flight to fill the link, while thousands of them
// would crowd the memory queues that concurrent kernels need.
__global__ __launch_bounds__(256) void k_copy_listed(const uint16_t* __restrict__ host_kv,
                                                     uint16_t* __restrict__ dev_cache,
                                                     const CopyItem* __restrict__ items,
                                                     const int32_t* __restrict__ counts, int pairs, int kb,
                                                     int64_t block_elems, int32_t* __restrict__ step_ctr) {
  __shared__ int32_t ex[256];
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, w = blockIdx.x;
  if (w == 0 && tid == 0) atomicAdd(step_ctr, 1);  // the planning kernel of this step has finished
  int base = 0;
  for (int p0 = 0; p0 < pairs; p0 += 256) {
    const uint32_t c = p0 + tid < pairs ? (uint32_t)counts[p0 + tid] : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0u, total = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      before += k < wave ? wsum[k] : 0u;
      total += wsum[k];
    }
    ex[tid] = (int32_t)(before + incl - c);
    __syncthreads();
    int j = base + (((w - base) % G) + G) % G;
    for (; j < base + (int)total; j += G) {
      // the pair holding entry j: last q with ex[q] <= j - base
      const int r = j - base;
      int lo = 0, hi = 255;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ex[mid] <= r) lo = mid; else hi = mid - 1;
      }
      // pairs past the end have count 0 and repeat ex; the search lands on the
      // last pair whose range holds r, which is a real one
      copy_block(host_kv, dev_cache, items[(int64_t)(p0 + lo) * kb + (r - ex[lo])], block_elems);
    }
    base += (int)total;
    __syncthreads();
  }
}

hipError_t launch_device_delta(const DeltaArgs& a, const uint16_t* host_kv_dev, uint16_t* dev_cache, hipStream_t st,
                               hipEvent_t prof_start, hipEvent_t prof_end) {
  if (a.full)
    hipLaunchKernelGGL(k_full_plan, dim3(a.pairs), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_delta_plan, dim3(a.pairs), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (prof_start) (void)hipEventRecord(prof_start, st);
  hipLaunchKernelGGL(k_copy_listed, dim3(a.copy_wgs), dim3(256), 0, st, host_kv_dev, dev_cache, a.items, a.counts,
                     a.pairs, a.kb, a.block_elems, a.step_ctr);
  e = hipGetLastError();
  if (prof_end) (void)hipEventRecord(prof_end, st);
  return e;
}

// Rows appended to an offloaded cache: workgroup (i, p) writes new row i of
// pair p (token N0 + i) into the resident slot of its block, when the block is
// resident in slot_map (the map the next attention uses); a block that is not
// resident is read from host memory, which holds the row, when it is next
// transferred.
__global__ __launch_bounds__(64) void k_patch_slots(const uint16_t* __restrict__ rows, int n, int64_t N0,
                                                    const int32_t* __restrict__ slot_map, int64_t NBs,
                                                    uint16_t* __restrict__ dev_cache, int cap, int bs, int row) {
  const int i = blockIdx.x, p = blockIdx.y;
  const int64_t t = N0 + i;
  const int slot = slot_map[(int64_t)p * NBs + t / bs];
  if (slot < 0 || slot >= cap) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(rows + ((int64_t)p * n + i) * row);
  u32x4* d = reinterpret_cast<u32x4*>(dev_cache + (((int64_t)p * cap + slot) * bs + t % bs) * row);
  for (int k = threadIdx.x; k < row / 8; k += 64) d[k] = s[k];
}

hipError_t launch_patch_slots(const uint16_t* rows, int n, int pairs, int64_t N0, const int32_t* slot_map,
                              int64_t NBs, uint16_t* dev_cache, int cap, int bs, int row, hipStream_t st) {
  hipLaunchKernelGGL(k_patch_slots, dim3((unsigned)n, (unsigned)pairs), dim3(64), 0, st, rows, n, N0, slot_map, NBs,
                     dev_cache, cap, bs, row);
  return hipGetLastError();
}

}  // namespace tls

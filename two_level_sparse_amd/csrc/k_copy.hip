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

__global__ __launch_bounds__(256) void k_gather_blocks(const uint16_t* __restrict__ host_kv,
                                                       uint16_t* __restrict__ dev_cache,
                                                       const CopyItem* __restrict__ items, int nitems,
                                                       const MapItem* __restrict__ map_items, int nmap,
                                                       int32_t* __restrict__ slot_map, int64_t block_elems) {
  const int i = blockIdx.x;
  if (i < nitems) {
    const CopyItem it = items[i];
    const u32x4* src = reinterpret_cast<const u32x4*>(host_kv + it.src_elem);
    u32x4* dst = reinterpret_cast<u32x4*>(dev_cache + it.dst_elem);
    const int64_t n16 = block_elems / 8;
    for (int64_t k = threadIdx.x; k < n16; k += blockDim.x) dst[k] = src[k];
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

}  // namespace tls

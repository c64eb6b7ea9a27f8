// offload.cpp -- staggered incremental prefetch of KV blocks from pinned host
// memory (AsyncTLS pages, section 2B "Asynchronous Offloading Engine").
//
// The device keeps, per (batch, kv head) pair, a resident cache of
// cap = 2*Kb' block slots and a slot map [NB] (-1 = not resident). The blocks
// chosen at step t-1 (M_{t-1}) are resident while step t runs; stage 1 for
// step t produces M_t on a side stream, and this engine then
//   1. copies M_t to the host and waits for it (the calling thread blocks),
//   2. forms T_t = M_t \ C_t (C_t: resident blocks),
//   3. if the free slots do not suffice, evicts resident blocks outside
//      M_{t-1} and M_t, least recently selected first (lower block first on
//      equal steps), so the blocks step t reads are never touched,
//   4. enqueues one host->device copy per block of T_t into its slot and the
//      slot map of step t+1 (double-buffered: step t reads map t%2, this call
//      writes map (t+1)%2), and records `copies_done` on the side stream.
// Capacity 2*Kb' is the least that always fits M_{t-1} u M_t.
//
// Copy modes: TLS_COPY_DEVICE (default when the pinned host cache has a
// device mapping and the shape fits the planning kernel) applies steps 2-4 on
// the GPU, so the call never waits: the planning kernel keeps the slot owners,
// the last-selected steps and M_{t-1} in device memory and writes the whole
// next slot map, and a copy kernel reads the listed blocks from host memory.
// TLS_COPY_GATHER plans on the host and moves the whole step's transfer with
// one kernel that reads the host blocks directly and patches the slot map with
// the changes of the last two steps; TLS_COPY_MEMCPY plans on the host and
// issues one hipMemcpyAsync per block plus a full slot-map upload.
//
// Ordering contract (the caller's streams): the side-stream work of step t
// (stage 1 and this call) must start after the main stream finished step
// t-1's attention, and step t+1's main-stream work must wait for
// `copies_done` of step t. Then no slot or map entry that a running kernel
// reads is ever written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/tls.h"
#include "tls_api_internal.h"
#include "tls_launch.h"

using namespace tls;

struct tls_offload {
  Derived d;                  // the shape at creation; per-block arrays are strided by d.NBs (capacity)
  int64_t cur_N = 0;          // tokens per sequence now (grows with tls_offload_append)
  const uint16_t* host_kv = nullptr;
  uint16_t* dev_cache = nullptr;
  int32_t* dev_map[2] = {nullptr, nullptr};
  int cap = 0;
  size_t block_elems = 0;
  std::vector<int32_t> slot_of;     // [pairs*NB] slot or -1
  std::vector<int64_t> last_sel;    // [pairs*NB] last step the block was selected (-1: prologue)
  std::vector<int32_t> slot_owner;  // [pairs*cap] block or -1
  std::vector<int32_t> prev;        // [pairs*kb] M_{t-1}
  std::vector<uint32_t> mark;       // [NB] scratch stamps
  uint32_t stamp = 0;
  int32_t* host_M = nullptr;        // pinned staging of M_t
  int32_t* host_map[2] = {nullptr, nullptr};  // pinned staging of the slot maps
  std::vector<int32_t> last_counts, last_blocks;
  int32_t next_step = 0;
  int copy_mode = TLS_COPY_MEMCPY;
  const uint16_t* host_kv_dev = nullptr;  // device mapping of host_kv (gather mode)
  tls::CopyItem* items = nullptr;          // pinned transfer list (host view)
  tls::MapItem* map_items = nullptr;       // pinned slot-map changes (host view)
  const tls::CopyItem* items_dev = nullptr;     // device views of the two lists
  const tls::MapItem* map_items_dev = nullptr;
  std::vector<tls::MapItem> prev_changes, cur_changes;  // reserved for 2*pairs*kb each
  std::vector<tls::MapItem> both;          // reserved for 4*pairs*kb: prev_changes + cur_changes
  std::vector<std::pair<int64_t, int32_t>> evict;  // reserved for cap: (last step selected, block)
  std::vector<int32_t> free_slots;         // reserved for cap
  std::vector<int32_t> last_pos;           // [pairs*NB] dedupe scratch, -1 when unused
  int64_t total_copied = 0;                // host-planned blocks moved since creation
  // device planning state (TLS_COPY_DEVICE), one allocation
  void* dev_state = nullptr;
  tls::DeltaArgs da{};
};

// TLS_COPY_DEVICE and TLS_COPY_FULL plan on the GPU; the others on the host.
static bool device_planned(int mode) { return mode == TLS_COPY_DEVICE || mode == TLS_COPY_FULL; }

static void free_ctx(tls_offload* c) {
  if (!c) return;
  if (c->dev_state) (void)hipFree(c->dev_state);
  if (c->items) (void)hipHostFree(c->items);
  if (c->map_items) (void)hipHostFree(c->map_items);
  if (c->host_M) (void)hipHostFree(c->host_M);
  for (int i = 0; i < 2; ++i)
    if (c->host_map[i]) (void)hipHostFree(c->host_map[i]);
  delete c;
}

// Workgroups of the device-planned copy: enough host reads in flight to fill
// the host link, few enough to leave the memory queues to concurrent kernels.
// TLS_OFFLOAD_COPY_WGS (1..1024) overrides it when the context is created.
constexpr int kCopyWorkgroups = 16;

// Device copy of the planning state after the prologue (TLS_COPY_DEVICE).
static hipError_t init_device_state(tls_offload* c) {
  const Derived& d = c->d;
  const size_t P = d.pairs, kb = d.kb, cap = c->cap, NB = d.NBs;
  auto up = [](size_t bytes) { return (bytes + 255) & ~(size_t)255; };
  const size_t o_items = 0, o_prev = o_items + up(P * kb * sizeof(CopyItem)), o_owner = o_prev + up(P * kb * 4),
               o_last = o_owner + up(P * cap * 4), o_counts = o_last + up(P * NB * 4),
               o_tblocks = o_counts + up(P * 4), o_total = o_tblocks + up(P * kb * 4), o_err = o_total + 256,
               o_step = o_err + 256, bytes = o_step + 256;
  hipError_t e = hipMalloc(&c->dev_state, bytes);
  if (e != hipSuccess) return e;
  char* base = (char*)c->dev_state;
  DeltaArgs& a = c->da;
  a.items = (CopyItem*)(base + o_items);
  a.prev = (int32_t*)(base + o_prev);
  a.owner = (int32_t*)(base + o_owner);
  a.last = (int32_t*)(base + o_last);
  a.counts = (int32_t*)(base + o_counts);
  a.tblocks = (int32_t*)(base + o_tblocks);
  a.total = (unsigned long long*)(base + o_total);
  a.err = (int32_t*)(base + o_err);
  a.step_ctr = (int32_t*)(base + o_step);
  a.pairs = d.pairs;
  a.NB = d.NBs;
  a.NBv = d.NB;
  a.kb = d.kb;
  a.cap = c->cap;
  a.bs = d.bs;
  a.row = d.row;
  a.N = d.Ns;
  a.block_elems = (int64_t)c->block_elems;
  a.copy_wgs = kCopyWorkgroups;
  if (const char* env = std::getenv("TLS_OFFLOAD_COPY_WGS")) {
    const int v = std::atoi(env);
    if (v >= 1 && v <= 1024) a.copy_wgs = v;
  }
  std::vector<int32_t> last32(c->last_sel.begin(), c->last_sel.end());
  std::vector<int32_t> zeros(P, 0);
  std::vector<int32_t> none(P * kb, -1);
  const uint64_t zero64 = 0;
  const int32_t zero32 = 0;
  if (e == hipSuccess) e = hipMemcpy(a.prev, c->prev.data(), P * kb * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.owner, c->slot_owner.data(), P * cap * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.last, last32.data(), P * NB * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.counts, zeros.data(), P * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.tblocks, none.data(), P * kb * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.total, &zero64, 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.err, &zero32, 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(a.step_ctr, &zero32, 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return e;
}

// Reads the device planning results after waiting for the device; reports a
// step the planning kernel could not apply.
static int device_state_check(const tls_offload* c) {
  hipError_t e = hipDeviceSynchronize();
  int32_t err = 0;
  if (e == hipSuccess) e = hipMemcpy(&err, c->da.err, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_error(e, "reading the offload state");
  if (err == 2) return set_error(TLS_ERR_STATE, "M_t held a block number outside [0, NB)");
  if (err) return set_error(TLS_ERR_STATE, "not enough evictable slots");
  return TLS_OK;
}

extern "C" {

int tls_offload_create(const tls_shape_t* shape, const void* host_kv, void* dev_cache, int32_t* dev_slot_map0,
                       int32_t* dev_slot_map1, const int32_t* initial_blocks, tls_offload_t** out) {
  clear_error();
  if (!out) return set_error(TLS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!host_kv || !dev_cache || !dev_slot_map0 || !dev_slot_map1 || !initial_blocks)
    return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  // blocks move whole: the host cache must hold every block of the capacity entirely
  if (d.Ns % d.bs != 0)
    return set_error(TLS_ERR_UNSUPPORTED, "offload needs ctx_capacity (ctx_len when 0) to be a multiple of block_size");
  // a cache that will grow keeps Kb' = Kb (and so its slot count) from the start
  if (d.Ns > d.N && d.NB < shape->top_kb)
    return set_error(TLS_ERR_UNSUPPORTED, "a growing offloaded cache needs at least top_kb blocks from the start");
  tls_offload* c = new tls_offload;
  c->d = d;
  c->cur_N = d.N;
  c->host_kv = (const uint16_t*)host_kv;
  c->dev_cache = (uint16_t*)dev_cache;
  c->dev_map[0] = dev_slot_map0;
  c->dev_map[1] = dev_slot_map1;
  c->cap = 2 * d.kb;
  c->block_elems = (size_t)d.bs * d.row;
  c->slot_of.assign((size_t)d.pairs * d.NBs, -1);
  c->last_sel.assign((size_t)d.pairs * d.NBs, -2);
  c->slot_owner.assign((size_t)d.pairs * c->cap, -1);
  c->prev.assign(initial_blocks, initial_blocks + (size_t)d.pairs * d.kb);
  c->mark.assign((size_t)d.NBs, 0u);
  c->last_counts.assign(d.pairs, 0);
  c->last_blocks.assign((size_t)d.pairs * d.kb, -1);
  // the host-planned steps only clear and refill these, so they never allocate:
  // a step changes at most kb evictions + kb copies per pair
  c->prev_changes.reserve((size_t)2 * d.pairs * d.kb);
  c->cur_changes.reserve((size_t)2 * d.pairs * d.kb);
  c->both.reserve((size_t)4 * d.pairs * d.kb);
  c->evict.reserve((size_t)c->cap);
  c->free_slots.reserve((size_t)c->cap);
  hipError_t e = hipHostMalloc((void**)&c->host_M, (size_t)d.pairs * d.kb * sizeof(int32_t), hipHostMallocDefault);
  for (int i = 0; i < 2 && e == hipSuccess; ++i)
    e = hipHostMalloc((void**)&c->host_map[i], (size_t)d.pairs * d.NBs * sizeof(int32_t), hipHostMallocDefault);
  if (e == hipSuccess)
    e = hipHostMalloc((void**)&c->items, (size_t)d.pairs * d.kb * sizeof(tls::CopyItem), hipHostMallocDefault);
  if (e == hipSuccess)
    e = hipHostMalloc((void**)&c->map_items, (size_t)d.pairs * d.kb * 4 * sizeof(tls::MapItem), hipHostMallocDefault);
  if (e != hipSuccess) {
    free_ctx(c);
    return hip_error(e, "hipHostMalloc(offload staging)");
  }
  {
    // Gather mode needs device views of the host cache and of both lists.
    void *dv = nullptr, *di = nullptr, *dm = nullptr;
    // (the copy kernels move 16-byte pieces: a block must be a whole number of them)
    if (c->block_elems % 8 == 0 && hipHostGetDevicePointer(&dv, const_cast<void*>(host_kv), 0) == hipSuccess && dv &&
        hipHostGetDevicePointer(&di, c->items, 0) == hipSuccess && di &&
        hipHostGetDevicePointer(&dm, c->map_items, 0) == hipSuccess && dm) {
      c->host_kv_dev = (const uint16_t*)dv;
      c->items_dev = (const tls::CopyItem*)di;
      c->map_items_dev = (const tls::MapItem*)dm;
      c->copy_mode = TLS_COPY_GATHER;
      c->last_pos.assign((size_t)d.pairs * d.NBs, -1);
    } else {
      (void)hipGetLastError();  // not device-mapped: per-block copies
    }
  }
  // Prologue: M_{-1} goes to slots 0..kb-1 of each pair, copied synchronously.
  for (int p = 0; p < d.pairs; ++p) {
    for (int i = 0; i < d.kb; ++i) {
      const int32_t blk = initial_blocks[(size_t)p * d.kb + i];
      if (blk < 0 || blk >= d.NB || (i > 0 && blk <= initial_blocks[(size_t)p * d.kb + i - 1])) {
        free_ctx(c);
        return set_error(TLS_ERR_INVALID_ARG, "initial_blocks must be ascending block numbers in [0, NB)");
      }
      c->slot_of[(size_t)p * d.NBs + blk] = i;
      c->slot_owner[(size_t)p * c->cap + i] = blk;
      c->last_sel[(size_t)p * d.NBs + blk] = -1;
      e = hipMemcpy(c->dev_cache + ((size_t)p * c->cap + i) * c->block_elems,
                    c->host_kv + ((size_t)p * d.Ns + (size_t)blk * d.bs) * d.row, c->block_elems * 2,
                    hipMemcpyHostToDevice);
      if (e != hipSuccess) {
        free_ctx(c);
        return hip_error(e, "hipMemcpy(initial blocks)");
      }
    }
  }
  std::memcpy(c->host_map[0], c->slot_of.data(), c->slot_of.size() * sizeof(int32_t));
  for (int i = 0; i < 2 && e == hipSuccess; ++i)
    e = hipMemcpy(c->dev_map[i], c->host_map[0], c->slot_of.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    free_ctx(c);
    return hip_error(e, "initial slot map upload");
  }
  if (c->host_kv_dev && c->cap <= kDeltaMaxCap && d.NBs <= kDeltaMaxNB) {
    e = init_device_state(c);
    if (e != hipSuccess) {
      free_ctx(c);
      return hip_error(e, "device planning state");
    }
    c->copy_mode = TLS_COPY_DEVICE;
  }
  *out = c;
  return TLS_OK;
}

const int32_t* tls_offload_slot_map(const tls_offload_t* ctx, int32_t step) {
  if (!ctx || step < 0) return nullptr;
  return ctx->dev_map[step & 1];
}

int tls_prefetch_delta(tls_offload_t* c, int32_t step, const int32_t* dev_block_idx, void* side, void* copies_done,
                       int64_t* n_copied_opt) {
  clear_error();
  if (!c || !dev_block_idx || !copies_done) return set_error(TLS_ERR_INVALID_ARG, "NULL argument");
  if (step != c->next_step)
    return set_error(TLS_ERR_STATE, "prefetch for step %d, expected step %d", step, c->next_step);
  const Derived& d = c->d;
  hipStream_t st = (hipStream_t)side;
  hipError_t e;
  if (device_planned(c->copy_mode)) {
    DeltaArgs a = c->da;
    a.full = c->copy_mode == TLS_COPY_FULL;
    a.M = dev_block_idx;
    a.map_cur = c->dev_map[step & 1];
    a.map_next = c->dev_map[(step + 1) & 1];
    hipEvent_t ps, pe;
    profile_events(TLS_PROFILE_HOST_COPY, &ps, &pe);
    e = launch_device_delta(a, c->host_kv_dev, c->dev_cache, st, ps, pe);
    if (e != hipSuccess) return hip_error(e, "delta launch");
    e = hipEventRecord((hipEvent_t)copies_done, st);
    if (e != hipSuccess) return hip_error(e, "event record");
    c->next_step = step + 1;
    if (n_copied_opt) *n_copied_opt = -1;
    return TLS_OK;
  }
  e = hipMemcpyAsync(c->host_M, dev_block_idx, (size_t)d.pairs * d.kb * sizeof(int32_t),
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_error(e, "copy of M_t to host");

  // every pair's M_t is checked before any state changes, so a rejected call
  // leaves the context as it was (and the same step can be retried)
  const int64_t nb_now = (c->cur_N + d.bs - 1) / d.bs;  // blocks of the cache as it is now
  for (int p = 0; p < d.pairs; ++p) {
    const int32_t* cur = c->host_M + (size_t)p * d.kb;
    for (int i = 0; i < d.kb; ++i)
      if (cur[i] < 0 || cur[i] >= nb_now || (i > 0 && cur[i] <= cur[i - 1]))
        return set_error(TLS_ERR_STATE, "M_t of pair %d is not ascending block numbers in [0, NB)", p);
  }

  int64_t total = 0;
  int nitems = 0;
  c->cur_changes.clear();
  std::vector<std::pair<int64_t, int32_t>>& evict = c->evict;
  std::vector<int32_t>& free_slots = c->free_slots;
  for (int p = 0; p < d.pairs; ++p) {
    const int32_t* cur = c->host_M + (size_t)p * d.kb;
    int32_t* prv = c->prev.data() + (size_t)p * d.kb;
    int32_t* slot_of = c->slot_of.data() + (size_t)p * d.NBs;
    int64_t* last = c->last_sel.data() + (size_t)p * d.NBs;
    int32_t* owner = c->slot_owner.data() + (size_t)p * c->cap;
    // mark M_{t-1} u M_t
    if (++c->stamp == 0) {
      std::fill(c->mark.begin(), c->mark.end(), 0u);
      c->stamp = 1;
    }
    const uint32_t s = c->stamp;
    for (int i = 0; i < d.kb; ++i) {
      c->mark[prv[i]] = s;
      c->mark[cur[i]] = s;
    }
    // T_t = M_t \ C_t (ascending, as M_t is)
    int32_t* T = c->last_blocks.data() + (size_t)p * d.kb;
    int nT = 0;
    for (int i = 0; i < d.kb; ++i)
      if (slot_of[cur[i]] < 0) T[nT++] = cur[i];
    for (int i = nT; i < d.kb; ++i) T[i] = -1;
    c->last_counts[p] = nT;
    total += nT;
    // free slots, then evictions if they do not suffice
    free_slots.clear();
    for (int sl = 0; sl < c->cap; ++sl)
      if (owner[sl] < 0) free_slots.push_back(sl);
    const int need = nT - (int)free_slots.size();
    if (need > 0) {
      evict.clear();
      for (int sl = 0; sl < c->cap; ++sl) {
        const int32_t blk = owner[sl];
        if (blk >= 0 && c->mark[blk] != s) evict.emplace_back(last[blk], blk);
      }
      // (cannot fail: cap = 2 kb slots hold M_{t-1} u M_t with room to spare)
      if ((int)evict.size() < need) return set_error(TLS_ERR_STATE, "not enough evictable slots");
      std::partial_sort(evict.begin(), evict.begin() + need, evict.end());
      for (int k = 0; k < need; ++k) {
        const int32_t blk = evict[k].second;
        const int32_t sl = slot_of[blk];
        slot_of[blk] = -1;
        owner[sl] = -1;
        free_slots.push_back(sl);
        c->cur_changes.push_back(tls::MapItem{(int64_t)p * d.NBs + blk, -1, 0});
      }
      std::sort(free_slots.begin(), free_slots.end());
    }
    // copies of T_t into the lowest free slots
    for (int i = 0; i < nT; ++i) {
      const int32_t blk = T[i], sl = free_slots[i];
      slot_of[blk] = sl;
      owner[sl] = blk;
      c->cur_changes.push_back(tls::MapItem{(int64_t)p * d.NBs + blk, sl, 0});
      const int64_t src = ((int64_t)p * d.Ns + (int64_t)blk * d.bs) * d.row;
      const int64_t dst = ((int64_t)p * c->cap + sl) * (int64_t)c->block_elems;
      if (c->copy_mode == TLS_COPY_GATHER) {
        c->items[nitems++] = tls::CopyItem{src, dst};
      } else {
        e = hipMemcpyAsync(c->dev_cache + dst, c->host_kv + src, c->block_elems * 2, hipMemcpyHostToDevice, st);
        if (e != hipSuccess) return hip_error(e, "block copy");
      }
    }
    for (int i = 0; i < d.kb; ++i) {
      last[cur[i]] = step;
      prv[i] = cur[i];
    }
  }
  const int nxt = (step + 1) & 1;
  if (c->copy_mode == TLS_COPY_GATHER) {
    // map (step+1)&1 holds the state of two prefetches ago: apply the changes
    // of the previous and of this prefetch (one entry per index, last wins).
    int nmap = 0;
    std::vector<tls::MapItem>& both = c->both;
    both.assign(c->prev_changes.begin(), c->prev_changes.end());
    both.insert(both.end(), c->cur_changes.begin(), c->cur_changes.end());
    for (size_t k = 0; k < both.size(); ++k) c->last_pos[both[k].index] = (int32_t)k;
    for (size_t k = 0; k < both.size(); ++k)
      if (c->last_pos[both[k].index] == (int32_t)k) c->map_items[nmap++] = both[k];
    for (size_t k = 0; k < both.size(); ++k) c->last_pos[both[k].index] = -1;
    hipEvent_t ps, pe;
    profile_events(TLS_PROFILE_HOST_COPY, &ps, &pe);
    if (ps) (void)hipEventRecord(ps, st);
    e = tls::launch_gather_blocks(c->host_kv_dev, c->dev_cache, c->items_dev, nitems, c->map_items_dev, nmap,
                                  c->dev_map[nxt], (int64_t)c->block_elems, st);
    if (pe) (void)hipEventRecord(pe, st);
    if (e != hipSuccess) return hip_error(e, "gather launch");
  } else {
    std::memcpy(c->host_map[nxt], c->slot_of.data(), c->slot_of.size() * sizeof(int32_t));
    e = hipMemcpyAsync(c->dev_map[nxt], c->host_map[nxt], c->slot_of.size() * sizeof(int32_t), hipMemcpyHostToDevice,
                       st);
    if (e != hipSuccess) return hip_error(e, "slot map upload");
  }
  c->prev_changes.swap(c->cur_changes);
  e = hipEventRecord((hipEvent_t)copies_done, st);
  if (e != hipSuccess) return hip_error(e, "event record");
  c->next_step = step + 1;
  c->total_copied += total;
  if (n_copied_opt) *n_copied_opt = total;
  return TLS_OK;
}

int tls_offload_append(tls_offload_t* c, const void* new_kv, int32_t n_new, const int32_t* label_ch, void* summ,
                       uint8_t* codes, float* scale, void* stream) {
  clear_error();
  if (!c || !new_kv || !label_ch || !summ || !codes || !scale) return set_error(TLS_ERR_INVALID_ARG, "NULL argument");
  const Derived& d = c->d;
  if (n_new < 1) return set_error(TLS_ERR_INVALID_ARG, "n_new must be >= 1");
  if (c->cur_N + n_new > d.Ns)
    return set_error(TLS_ERR_INVALID_ARG, "the cache length after the append (%lld) exceeds ctx_capacity (%lld)",
                     (long long)(c->cur_N + n_new), (long long)d.Ns);
  if (!aligned(new_kv, 16) || !aligned(summ, 4) || !aligned(scale, 4) || !aligned(label_ch, 4))
    return set_error(TLS_ERR_INVALID_ARG, "new_kv must be 16-byte aligned, summ, scale and label_ch 4-byte");
  if (!c->host_kv_dev)
    return set_error(TLS_ERR_UNSUPPORTED, "host_kv has no device mapping (allocate it with hipHostMalloc)");
  hipStream_t st = (hipStream_t)stream;
  const uint16_t* rows = (const uint16_t*)new_kv;
  // the rows into the host cache, written through its device mapping
  hipError_t e = launch_append_rows(rows, const_cast<uint16_t*>(c->host_kv_dev), d.pairs, n_new, d.row, c->cur_N,
                                    d.Ns, st);
  // the summaries of the blocks they fall in and their codes and scales
  if (e == hipSuccess)
    e = launch_append_index(rows, n_new, label_ch, (uint16_t*)summ, codes, scale, d.pairs, d.Hkv, d.D, d.row, d.bs,
                            d.r, c->cur_N, d.Ns, d.NBs, st);
  // the resident copies of those blocks, in the map the next attention reads
  if (e == hipSuccess)
    e = launch_patch_slots(rows, n_new, d.pairs, c->cur_N, c->dev_map[c->next_step & 1], d.NBs, c->dev_cache, c->cap,
                           d.bs, d.row, st);
  if (e != hipSuccess) return hip_error(e, "append launch");
  c->cur_N += n_new;
  c->da.NBv = (int)((c->cur_N + d.bs - 1) / d.bs);
  return TLS_OK;
}

int tls_offload_set_copy_mode(tls_offload_t* c, int mode) {
  clear_error();
  if (!c) return set_error(TLS_ERR_INVALID_ARG, "NULL context");
  if (mode != TLS_COPY_GATHER && mode != TLS_COPY_MEMCPY && mode != TLS_COPY_DEVICE && mode != TLS_COPY_FULL)
    return set_error(TLS_ERR_INVALID_ARG, "unknown copy mode");
  if (mode == TLS_COPY_GATHER && !c->host_kv_dev)
    return set_error(TLS_ERR_UNSUPPORTED, "host cache has no device mapping; only TLS_COPY_MEMCPY is available");
  if (device_planned(mode) && !c->dev_state)
    return set_error(TLS_ERR_UNSUPPORTED,
                     "device planning needs a device-mapped host cache, 2*Kb' <= %d slots and NB <= %d blocks",
                     kDeltaMaxCap, kDeltaMaxNB);
  if (mode != c->copy_mode && (device_planned(mode) || device_planned(c->copy_mode)) && c->next_step != 0)
    return set_error(TLS_ERR_STATE, "planning can move between host and device, or to or from full transfers, "
                                    "only before step 0");
  c->copy_mode = mode;
  return TLS_OK;
}

int tls_offload_get_copy_mode(const tls_offload_t* c) {
  if (!c) return set_error(TLS_ERR_INVALID_ARG, "NULL context");
  return c->copy_mode;
}

int tls_offload_last_delta(const tls_offload_t* c, int32_t* counts, int32_t* blocks) {
  clear_error();
  if (!c || !counts || !blocks) return set_error(TLS_ERR_INVALID_ARG, "NULL argument");
  if (device_planned(c->copy_mode)) {
    int rc = device_state_check(c);
    if (rc) return rc;
    hipError_t e = hipMemcpy(counts, c->da.counts, (size_t)c->d.pairs * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(blocks, c->da.tblocks, (size_t)c->d.pairs * c->d.kb * 4, hipMemcpyDeviceToHost);
    return e == hipSuccess ? TLS_OK : hip_error(e, "reading the last transfer");
  }
  std::memcpy(counts, c->last_counts.data(), c->last_counts.size() * sizeof(int32_t));
  std::memcpy(blocks, c->last_blocks.data(), c->last_blocks.size() * sizeof(int32_t));
  return TLS_OK;
}

int tls_offload_total_copied(const tls_offload_t* c, int64_t* total) {
  clear_error();
  if (!c || !total) return set_error(TLS_ERR_INVALID_ARG, "NULL argument");
  if (device_planned(c->copy_mode)) {
    int rc = device_state_check(c);
    if (rc) return rc;
    unsigned long long t = 0;
    hipError_t e = hipMemcpy(&t, c->da.total, 8, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_error(e, "reading the transfer count");
    *total = (int64_t)t;
    return TLS_OK;
  }
  *total = c->total_copied;
  return TLS_OK;
}

void tls_offload_destroy(tls_offload_t* c) {
  if (c) (void)hipDeviceSynchronize();
  free_ctx(c);
}

}  // extern "C"

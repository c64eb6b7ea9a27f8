// k_step.hip -- one whole decode step (both selection stages and the attention
// over the kept tokens, for every (batch, kv head) pair) in one launch, for the
// 128-channel GQA shape.
//
// AsyncTLS pages, section 2A: block filtering on the key max/min summaries,
// token selection inside the kept blocks on INT4 label channels, then exact
// attention over the kept tokens. The steps of one pair depend on each other,
// but the pairs do not: a pair's selection (a chain of small, latency-bound
// steps) can run while other pairs stream their summaries or gather their
// rows. Run as separate launches, every step waits for the slowest pair and
// the chip idles through each selection; here one persistent launch lets
// every workgroup take whatever work is ready.
//
// Work items of pair p (p runs on XCD x = p mod nx, so every hand-off between
// its items stays inside one XCD's L2):
//   A(p, c)  block scores of 128 blocks (16-block MFMA tiles; k_score_blocks'
//            product) -> S[p, ..]. The workgroup that completes the last A
//            item of p goes on with
//   B(p)     block top-Kb -> block_idx, then publishes p's T items.
//   T(p, u)  label-channel scores (folded MFMA form) of the 1024 candidates
//            of kept blocks 16u .. 16u+15, as order keys -> K[p, ..]. The
//            workgroup that completes the last T item of p goes on with
//   K(p)     the token top-Kt cut over all of p's keys (threshold key, how
//            many keys equal to it are kept) and, per chunk of 512
//            candidates, the number of kept keys before it and the number of
//            threshold-equal keys before it; then publishes p's C items.
//   C(p, v)  the kept tokens of candidate chunk v: their place in token_idx
//            follows from the chunk's counts, so the item writes them there
//            itself and attends over them (attend_pv_range) -> one partial
//            (m, l, o) per head. The workgroup that completes the last C
//            item of p goes on with
//   D(p)     the log-sum-exp merge of the partials -> out, lse.
// Each XCD has one queue: its A items (pair by pair), then its ring of T and
// C items in the order they were published. A workgroup reads its XCD from
// the hardware (HW_REG_XCC_ID), takes the next index of its XCD's queue, and
// for a ring entry waits until it has been published. Every item that waits
// was taken after every item it waits on had been taken by a running
// workgroup, and nothing waits on a later item, so the launch cannot deadlock
// whatever number of workgroups is resident; every wait is bounded all the
// same (a timeout sets an error word and abandons the item).
//
// Hand-offs: a producer's stores are complete in L2 once its s_waitcnt
// vmcnt(0) returns; it then counts or publishes with an agent-scope atomic.
// The consumer, on the same XCD (same L2), sees the atomic, invalidates its
// own L1 (buffer_inv sc0) and reads. No cache is written back: an agent-scope
// release would write back the whole L2 of the XCD every time.
//
// Every counter returns to zero within the launch (the last user of each
// resets it; the last workgroup to leave resets the queues), so the state
// words need clearing only once, before the first launch.
//
// Measured on the 128k GQA step (batch 8, 64/8 heads, 2048 blocks, Kb 128,
// Kt 4096): 77-79 us warm, against 68.7 us for the separate launches, which
// therefore stay the default. The step of one pair is a chain of dependent
// items (A, B, T, K, C, D: about 6 + 4.5 + 5.5 + 12 + 11 + 3.5 us, plus the
// hand-offs), about 50 us from its first A item to its merge; the overlap
// across pairs does not make up for that chain. Where the polling workgroups
// sleep 4, 16 or 64 cycles between polls the time does not change.
#include "tls_attn_dev.h"
#include "tls_dev.h"
#include "tls_launch.h"
#include "tls_select_dev.h"

namespace tls {

// ---------------------------------------------------------------- state --
// Words of the state area (int32), every counter on its own 256-byte line.
constexpr int kLine = 64;
constexpr int kStErr = 0;                         // error bits (sticky)
constexpr int kStExit = 1 * kLine;                // workgroups that left
constexpr int kStQueue = 2 * kLine;                  // [kMaxXcd] queue heads
constexpr int kStTail = kStQueue + kMaxXcd * kLine;  // [kMaxXcd] ring tails (entries reserved)
constexpr int kStPairs = kStTail + kMaxXcd * kLine;  // [pairs] A, then T, then C completion counts

__device__ __forceinline__ int xcc_id() {
  // HW_REG_XCC_ID (register 20), bits 0..15
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & 0xFFFF;
}
__device__ __forceinline__ int atomic_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_load(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The workgroup's stores are in L2 (every wave waited for its own).
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}
// Drop this CU's L1 lines, so that the loads after a hand-off read L2.
__device__ __forceinline__ void l1_invalidate() { asm volatile("buffer_inv sc0" ::: "memory"); }

constexpr int kStepBlocks = 128;  // blocks per A item: 4 waves x 2 tiles of 16
constexpr int kSpinLimit = 1 << 20;
enum { kItemT = 1, kItemC = 2 };  // ring entry types

// The launch's arguments, read by the item functions from the kernel-argument
// segment through a wave-uniform pointer (scalar loads).
typedef const __attribute__((address_space(4))) StepArgs* ArgsP;
__device__ __forceinline__ ArgsP uniform_args(ArgsP p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (ArgsP)(((uint64_t)hi << 32) | lo);
}

// LDS of the launch, at file scope so that the item functions (kept out of
// line, each with a register allocation of its own) address these objects
// directly: the attention's two tile buffers stay distinct objects, so that
// reading one does not wait for the loads into the other. The selection items
// use tB for their small arrays and tA for the block top-k's output staging.
__shared__ __attribute__((aligned(1024))) uint8_t s_tA[4][kPvTile * kPvRowBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_tB[4][kPvTile * kPvRowBytes];
__shared__ int32_t s_rows[4][kStepChunk / 4];
__shared__ int32_t s_tok[kStepChunk];  // the kept tokens of a C item's chunk
__shared__ float s_c[4][16];
__shared__ float s_ml[4][16][2];
__shared__ int s_ctl[4];  // the queue index taken; the ring entry; whether this workgroup completed a pair's last item; a count
__shared__ uint32_t s_scan[4];  // block scans: one word per wave

// -------------------------------------------------------- A: block scores --
// Blocks [j0, j0 + 128) of pair p: wave w scores tiles j0/16 + w and + w + 4
// (16 blocks each, both in flight), the channel loop in one group of four
// 32-channel chunks whose loads all go out before the MFMAs (as
// k_score_blocks with one head tile).
__device__ __attribute__((noinline)) void item_scores(ArgsP a0, int p, int64_t j0) {
  const ArgsP a = uniform_args(a0);
  const int b = p / a->Hkv, h = p % a->Hkv, G = a->G;
  const int64_t NB = a->NB;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, kq = lane >> 4;
  const uint16_t* qp = a->q + ((int64_t)b * a->Hq + (int64_t)h * G) * 128;
  const uint16_t* sp = a->summ + (int64_t)p * summ_pair_elems(a->NBs, 128);
  const uint16_t* brow[2];  // the two tiles in tile-fragment order (one past the last: the last again)
  int64_t jt[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    jt[s] = j0 + 16 * (wave + 4 * s);
    brow[s] = sp + summ_unit(min(jt[s] / 16, summ_tiles(NB) - 1), 0, 0, 4) + 8 * lane;
  }
  const uint16_t* qrow = qp + (int64_t)min(n, G - 1) * 128;
  u32x4 kmx[4][2], kmn[4][2], qr[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int off = c * 32 + 8 * kq;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      kmx[c][s] = ld16(brow[s] + summ_unit(0, c, 0, 4));
      kmn[c][s] = ld16(brow[s] + summ_unit(0, c, 1, 4));
    }
    qr[c] = ld16(qrow + off);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 pos, neg;
    split_sign(qr[c], pos, neg);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      acc[s] = mfma16x16x32(pos, kmx[c][s], acc[s]);
      acc[s] = mfma16x16x32(neg, kmn[c][s], acc[s]);
    }
  }
  float* S = a->S + (int64_t)p * NB;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float best = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * kq + i < G) best = fmaxf(best, acc[s][i]);
    best = max_rows(best);
    const int64_t j = jt[s] + n;
    if (kq == 0 && j < NB) S[j] = best;
  }
}

// ----------------------------------------------------- B: block top-Kb --
template <int PERB>
__device__ __attribute__((noinline)) void item_blocks(ArgsP a0, int p) {
  const ArgsP a = uniform_args(a0);
  TopkLds<256>& sh = *reinterpret_cast<TopkLds<256>*>(&s_tB[0][0]);
  uint32_t* stage = reinterpret_cast<uint32_t*>(&s_tA[0][0]);  // 256*PERB words
  const int tid = threadIdx.x, NB = (int)a->NB, kb = a->kb;
  const int per = (NB + 255) / 256;
  float v[PERB];
  load_row_f32<PERB>(a->S + (int64_t)p * NB, NB, tid * per, v);
  uint32_t key[PERB];
  int32_t id[PERB];
#pragma unroll
  for (int e = 0; e < PERB; ++e) {
    const int c = tid * per + e;
    id[e] = c;
    key[e] = (e < per && c < NB) ? order_key(v[e]) : 0u;
  }
  block_topk<PERB, 256>(key, id, (uint32_t)kb, a->block_idx + (int64_t)p * kb, kb, sh, stage);
}

// ------------------------------------------------- T: label-channel scores --
// Candidates of kept blocks 16u .. 16u+15 (wave w: blocks 16u + 4w .. +3), as
// order keys; candidates of no block, or past the cached tokens, get key 0.
// Each kept key is also counted in the pair's histogram of key >> kHistShift
// (the sign, exponent and top three mantissa bits of the score: bins in
// score order), first in LDS, then one atomic per non-empty bin.
constexpr int kHistShift = 20, kHistBins = 4096;
template <int RB>
__device__ __attribute__((noinline)) void item_tokens(ArgsP a0, int p, int u) {
  const ArgsP a = uniform_args(a0);
  uint16_t* sq = reinterpret_cast<uint16_t*>(&s_tB[0][0]);         // [16 * kLabRow]
  uint32_t* lh = reinterpret_cast<uint32_t*>(&s_tB[1][0]);         // [kHistBins]
  const int tid = threadIdx.x, wave = tid >> 6;
  const int b = p / a->Hkv, h = p % a->Hkv;
  const int kb = a->kb;
  const int32_t* bidx = a->block_idx + (int64_t)p * kb;
  uint32_t hl[2];
  label_q_issue<1>(hl, a->label_ch + (int64_t)h * a->r, a->q + ((int64_t)b * a->Hq + (int64_t)h * a->G) * 128, a->G,
                   128, a->r);
  const int c0 = (16 * u + 4 * wave) * 64;
  FoldLoads<4> L;
  fold_issue<RB, 4>(L, bidx, make_rsrc(a->codes + (int64_t)p * a->Ns * RB, (int)(a->Ns * RB)),
                    make_rsrc(a->scale + (int64_t)p * a->Ns, (int)(a->Ns * 4)), c0, kb);
  for (int i = tid; i < kHistBins; i += 256) lh[i] = 0u;
  u32x4 qa[1];
  label_q_finish<1, true>(qa, hl, sq, a->r);  // (its barrier also orders the histogram clear)
  float val[4];
  int cand[4];
  bool ok[4];
  fold_scores<4>(val, cand, ok, L, c0, kb, a->N, qa[0]);
  uint32_t* K = a->K + (int64_t)p * a->kstride;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t key = ok[g] ? order_key(val[g]) : 0u;
    K[cand[g]] = key;
    if (key) atomicAdd(&lh[key >> kHistShift], 1u);
  }
  lds_sync();
  uint32_t* gh = a->hist + (int64_t)p * kHistBins;
  for (int i = tid; i < kHistBins; i += 256)
    if (lh[i]) atomic_add(reinterpret_cast<int*>(&gh[i]), (int)lh[i]);
}

// -------------------------------------------------------- K: token cut --
// The token top-Kt cut: from the pair's histogram, the bin d holding the
// Kt-th largest key and the count of keys above it; the keys of bin d (a few
// hundred) are gathered in LDS and the exact threshold found among them by
// topk_cut. Then, per chunk of kStepChunk candidates, the kept keys before it
// and the threshold-equal keys before it. Pads token_idx with -1 past the
// kept count. (The C items clear the histogram for the next launch.)
// Keys in registers: thread t holds candidates [t*PERT, t*PERT + PERT).
template <int PERT>
__device__ __attribute__((noinline)) void item_cut(ArgsP a0, int p) {
  const ArgsP a = uniform_args(a0);
  TopkLds<256>& sh = *reinterpret_cast<TopkLds<256>*>(&s_tB[0][0]);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(&s_tB[1][0]);  // [2][chunks]: greater, equal
  uint32_t* bc = reinterpret_cast<uint32_t*>(&s_tB[2][0]);   // broadcast words
  uint32_t* list = reinterpret_cast<uint32_t*>(&s_tA[0][0]);  // the keys of bin d
  const int tid = threadIdx.x, kt = a->kt, ncand = a->kb * 64, nch = a->nsplit;
  const uint32_t* K = a->K + (int64_t)p * a->kstride;
  uint32_t* gh = a->hist + (int64_t)p * kHistBins;
  // thread t: histogram bins [16t, 16t + 16) (read as the atomics that
  // built them are performed: agent-scope loads) and its candidates' keys
  u32x4 hb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) hb[j][i] = (uint32_t)atomic_load(reinterpret_cast<const int*>(gh + 16 * tid + 4 * j + i));
  uint32_t kr[PERT];
#pragma unroll
  for (int j = 0; j < PERT / 4; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(K + tid * PERT + 4 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[4 * j + i] = tid * PERT + 4 * j + i < ncand ? v[i] : 0u;
  }
  for (int i = tid; i < 2 * nch; i += 256) cnt[i] = 0u;
  uint32_t mine = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) mine += hb[j][0] + hb[j][1] + hb[j][2] + hb[j][3];
  const uint32_t pre = block_exclusive_scan<4>(mine, s_scan);
  if (tid == 255) bc[0] = pre + mine;  // every kept-able key
  lds_sync();
  const uint32_t total = bc[0];
  TopkCut cut{0u, 0u, total};  // Kt >= the valid keys: keep them all
  if ((uint32_t)kt < total) {
    // bins descending: keys above thread t's bins = total - pre - mine
    uint32_t run = total - pre - mine;
    if (run < (uint32_t)kt && (uint32_t)kt <= run + mine) {
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        const uint32_t c = hb[i >> 2][i & 3];
        if (run < (uint32_t)kt && (uint32_t)kt <= run + c) {
          bc[1] = 16 * tid + i;  // bin d
          bc[2] = run;           // keys above bin d
        }
        run += c;
      }
    }
    if (tid == 0) bc[3] = 0xFFFFFFFFu;  // the smallest key of bin d
    lds_sync();
    const uint32_t d = bc[1], above = bc[2];
    // the keys of bin d, gathered in LDS at offsets from one block scan
    uint32_t nmine = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < PERT; ++e)
      if (kr[e] != 0u && (kr[e] >> kHistShift) == d) {
        ++nmine;
        kmin = min(kmin, kr[e]);
      }
    uint32_t at = block_exclusive_scan<4>(nmine, s_scan);
#pragma unroll
    for (int e = 0; e < PERT; ++e)
      if (kr[e] != 0u && (kr[e] >> kHistShift) == d) list[at++] = kr[e];
    kmin = wave_umin(kmin);
    if ((tid & 63) == 0) atomicMin(&bc[3], kmin);
    if (tid == 255) bc[4] = at;  // every key of bin d
    lds_sync();
    const int nd = (int)bc[4];
    const uint32_t kin = (uint32_t)kt - above;  // 1 <= kin <= nd
    TopkCut c;
    if (kin >= (uint32_t)nd) {
      c = TopkCut{bc[3], 0xFFFFFFFFu, kin};  // bin d is kept whole: every key from its smallest on
    } else if (nd <= 1024) {
      uint32_t lk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lk[e] = 4 * tid + e < nd ? list[4 * tid + e] : 0u;
      c = topk_cut<4, 256>(RegKeys<4>{lk}, kin, sh);
    } else {
      uint32_t lk[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) lk[e] = 32 * tid + e < nd ? list[32 * tid + e] : 0u;
      c = topk_cut<32, 256>(RegKeys<32>{lk}, kin, sh);
    }
    cut = TopkCut{c.thr, c.krem, (uint32_t)kt};
  }
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < PERT; ++e) {
    gt += kr[e] > cut.thr ? 1u : 0u;
    eq += (kr[e] == cut.thr && kr[e] != 0u) ? 1u : 0u;
  }
  const int ch = tid * PERT / kStepChunk;  // PERT divides kStepChunk
  if (gt) atomicAdd(&cnt[ch], gt);
  if (eq) atomicAdd(&cnt[nch + ch], eq);
  lds_sync();
  if (tid == 0) {
    int* info = a->chunk_info + (int64_t)p * 2 * nch;
    uint32_t g_before = 0u, e_before = 0u;
    for (int v = 0; v < nch; ++v) {
      info[2 * v] = (int)(g_before + min(e_before, cut.krem));
      info[2 * v + 1] = (int)e_before;
      g_before += cnt[v];
      e_before += cnt[nch + v];
    }
    int* ci = a->cut_info + (int64_t)p * 4;
    ci[0] = (int)cut.thr;
    ci[1] = (int)cut.krem;
    ci[2] = (int)cut.kk;
  }
  int32_t* ti = a->token_idx + (int64_t)p * kt;
  for (int i = (int)cut.kk + tid; i < kt; i += 256) ti[i] = -1;
}

// --------------------------------------------------------- C: attention --
// The kept tokens of candidate chunk v (two candidates per thread, placed in
// candidate order by one block scan, as topk_place places them), written to
// their place in token_idx and attended over.
__device__ __attribute__((noinline)) void item_attend(ArgsP a0, int p, int v) {
  const ArgsP a = uniform_args(a0);
  const int tid = threadIdx.x, kb = a->kb, ncand = kb * 64, kt = a->kt;
  const int* ci = a->cut_info + (int64_t)p * 4;
  const uint32_t thr = (uint32_t)ci[0], krem = (uint32_t)ci[1];
  const int* info = a->chunk_info + ((int64_t)p * a->nsplit + v) * 2;
  const int off = info[0];
  const uint32_t eqb = (uint32_t)info[1];
  const int c = v * kStepChunk + 2 * tid;
  const uint2 k2 = c < ncand ? *reinterpret_cast<const uint2*>(a->K + (int64_t)p * a->kstride + c) : uint2{0u, 0u};
  const int32_t* bidx = a->block_idx + (int64_t)p * kb;
  const int blk = bidx[min(c, ncand - 1) >> 6];
  const uint32_t k[2] = {k2.x, k2.y};
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    gt += k[e] > thr ? 1u : 0u;
    eq += (k[e] == thr && k[e] != 0u) ? 1u : 0u;
  }
  const uint32_t pre = block_exclusive_scan<4>(gt | (eq << 16), s_scan);
  uint32_t eq_before = eqb + (pre >> 16);
  uint32_t pos = (pre & 0xFFFFu) + min(eq_before, krem) - min(eqb, krem);
  int32_t* ti = a->token_idx + (int64_t)p * kt + off;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    bool take = k[e] > thr;
    if (k[e] == thr && k[e] != 0u) {
      take = eq_before < krem;
      ++eq_before;
    }
    if (take) {
      const int tok = blk * 64 + ((c + e) & 63);
      s_tok[pos] = tok;
      ti[pos] = tok;
      ++pos;
    }
  }
  // the chunk's count: the last thread's end position
  if (tid == 255) s_ctl[3] = (int)pos;
  __syncthreads();
  const int ntok = s_ctl[3];
  // the cut has read the pair's key histogram: the C items clear it for the
  // next launch, with atomic stores like the atomics that count into it (a
  // plain store may be held in this XCD's L2 while those counts are made
  // elsewhere)
  int* gh = reinterpret_cast<int*>(a->hist + (int64_t)p * kHistBins);
  for (int i = v * 256 + tid; i < kHistBins; i += a->nsplit * 256) atomic_store(&gh[i], 0);
  float* dst = a->part + ((int64_t)p * a->nsplit + v) * 8 * (128 + kPartHdr);
  attend_pv_range<8, false, kStepChunk / 4>(a->q, a->kv, nullptr, s_tok, ntok, dst, a->Hq, a->Hkv, a->G, a->N,
                                            a->Ns, 64, a->NB, 0, p, 0, a->qk_scale, s_tA, s_tB, s_rows, s_c, s_ml);
}

// ---------------------------------------------------------- D: the merge --
// The nsplit partials of pair p (8 heads each): thread (head tid/32, float4
// tid%32) forms the split weights itself, 8 splits per round.
__device__ __attribute__((noinline)) void item_merge(ArgsP a0, int p) {
  const ArgsP a = uniform_args(a0);
  constexpr int HT = 8, PS = 128 + kPartHdr, SP = HT * PS;
  const int tid = threadIdx.x, nsplit = a->nsplit;
  const int hh = tid >> 5, c = (tid & 31) * 4;
  const int b = p / a->Hkv, h = p % a->Hkv;
  const float* hd = a->part + (int64_t)p * nsplit * SP + (int64_t)hh * PS;
  float M = -INFINITY, L = 0.0f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float2 ml[8];
    f32x4 ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t off = (int64_t)min(s0 + u, nsplit - 1) * SP;
      ml[u] = *reinterpret_cast<const float2*>(hd + off);
      ov[u] = *reinterpret_cast<const f32x4*>(hd + off + kPartHdr + c);
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) cm = fmaxf(cm, ml[u].x);
    if (cm != M) {
      const float r = M == -INFINITY ? 0.0f : exp2f(M - cm);
      L *= r;
      o *= r;
      M = cm;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < nsplit) {
        const float w = ml[u].x == -INFINITY ? 0.0f : exp2f(ml[u].x - M);
        L += ml[u].y * w;
        o += ov[u] * w;
      }
  }
  if (hh >= a->G) return;
  const int64_t row = (int64_t)b * a->Hq + (int64_t)h * a->G + hh;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (a->lse && c == 0) a->lse[row] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
  *reinterpret_cast<f32x4*>(a->out + row * 128 + c) = o * inv;
}

// ---------------------------------------------------------- the launch --
// Publishes n ring entries (type, p, 0 .. n-1) on ring x (thread 0).
__device__ __forceinline__ void publish(int* st, int* ring, int x, int type, int p, int n) {
  const int base = atomic_add(&st[kStTail + x * kLine], n);
  for (int u = 0; u < n; ++u) atomic_store(&ring[base + u], ((type << 28) | (p << 12) | u) + 1);
}

template <int RB, int PERB, int PERT>
__global__ __launch_bounds__(256, 2) void k_step(StepArgs args) {
  const ArgsP a = (ArgsP)__builtin_amdgcn_kernarg_segment_ptr();  // `args` is the only argument
  const int tid = threadIdx.x;
  int* st = a->state;
  const int x = xcc_id(), nx = a->nx, pairs = a->pairs, nC_pp = a->nsplit, nA_pp = a->nA, nT_pp = a->nT;
  int* cntA = st + kStPairs;                       // [pairs] lines each
  int* cntT = st + kStPairs + pairs * kLine;
  int* cntC = st + kStPairs + 2 * pairs * kLine;
  if (x < nx) {
    const int npx = x < pairs ? (pairs - x + nx - 1) / nx : 0;  // pairs x, x + nx, ...
    const int nA = npx * nA_pp, nR = npx * (nT_pp + nC_pp);
    int* ring = a->ring + (int64_t)x * a->ring_cap;
    for (int guard = 0; guard <= nA + nR; ++guard) {
      __syncthreads();  // every thread has read the previous item's broadcast words
      if (tid == 0) s_ctl[0] = atomic_add(&st[kStQueue + x * kLine], 1);
      __syncthreads();
      const int it = s_ctl[0];
      if (it >= nA + nR) break;
      if (it < nA) {
        // ---- A(p, c); the last one of the pair goes on with B(p)
        const int p = x + (it / nA_pp) * nx;
        item_scores(a, p, (int64_t)(it % nA_pp) * kStepBlocks);
        stores_done();
        if (tid == 0) s_ctl[2] = atomic_add(&cntA[p * kLine], 1) == nA_pp - 1;
        __syncthreads();
        if (!s_ctl[2]) continue;
        l1_invalidate();
        item_blocks<PERB>(a, p);
        stores_done();
        if (tid == 0) {
          atomic_store(&cntA[p * kLine], 0);
          publish(st, ring, x, kItemT, p, nT_pp);
        }
        continue;
      }
      // ---- a ring entry: wait until it is published
      if (tid == 0) {
        int v = 0;
        int* e = &ring[it - nA];
        for (int spin = 0; spin < kSpinLimit; ++spin) {
          v = atomic_load(e);
          if (v != 0) break;
          __builtin_amdgcn_s_sleep(4);
        }
        if (v != 0)
          atomic_store(e, 0);
        else
          __hip_atomic_fetch_or(&st[kStErr], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_ctl[1] = v - 1;
      }
      __syncthreads();
      const int e = s_ctl[1];
      if (e < 0) continue;  // timed out (error word set)
      const int type = e >> 28, p = (e >> 12) & 0xFFFF, u = e & 0xFFF;
      l1_invalidate();
      if (type == kItemT) {
        // ---- T(p, u); the last one of the pair goes on with K(p)
        item_tokens<RB>(a, p, u);
        stores_done();
        if (tid == 0) s_ctl[2] = atomic_add(&cntT[p * kLine], 1) == nT_pp - 1;
        __syncthreads();
        if (!s_ctl[2]) continue;
        l1_invalidate();
        item_cut<PERT>(a, p);
        stores_done();
        if (tid == 0) {
          atomic_store(&cntT[p * kLine], 0);
          publish(st, ring, x, kItemC, p, nC_pp);
        }
      } else {
        // ---- C(p, v); the last one of the pair goes on with D(p)
        item_attend(a, p, u);
        stores_done();
        if (tid == 0) s_ctl[2] = atomic_add(&cntC[p * kLine], 1) == nC_pp - 1;
        __syncthreads();
        if (!s_ctl[2]) continue;
        l1_invalidate();
        item_merge(a, p);
        if (tid == 0) atomic_store(&cntC[p * kLine], 0);
      }
    }
  }
  // the last workgroup to leave checks that every queue was drained and
  // resets the queues for the next launch
  if (tid == 0) {
    if (atomic_add(&st[kStExit], 1) == (int)gridDim.x - 1) {
      for (int y = 0; y < nx; ++y) {
        const int npx = y < pairs ? (pairs - y + nx - 1) / nx : 0;
        if (atomic_load(&st[kStQueue + y * kLine]) < npx * (nA_pp + nT_pp + nC_pp))
          __hip_atomic_fetch_or(&st[kStErr], 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomic_store(&st[kStQueue + y * kLine], 0);
        atomic_store(&st[kStTail + y * kLine], 0);
      }
      atomic_store(&st[kStExit], 0);
    }
  }
}

// ------------------------------------------------------------- the host --
static int pow2_at_least(int v, int lo) {
  int p = lo;
  while (p < v) p *= 2;
  return p;
}

bool step_supported(int G, int D, int DV, bool v_is_k_prefix, int bs, int r, int64_t NB, int kb, int kt) {
  return D == 128 && DV == 128 && !v_is_k_prefix && G >= 1 && G <= 8 && bs == 64 && (r == 8 || r == 16) &&
         NB <= 4096 && NB < 65536 && kb >= 1 && kb <= 128 && kt >= 1;
}

void plan_step(int pairs, int nx, int64_t NB, int kb, StepPlan* pl) {
  pl->nx = nx;
  pl->nA = (int)((NB + kStepBlocks - 1) / kStepBlocks);
  pl->nT = (kb + 15) / 16;                       // 1024 candidates per T item
  pl->nC = (kb * 64 + kStepChunk - 1) / kStepChunk;
  pl->pert = kb <= 32 ? 8 : 32;                  // candidate keys per thread of the cut
  pl->kstride = 256 * pl->pert;
  const int npx = (pairs + nx - 1) / nx;
  pl->ring_cap = npx * (pl->nT + pl->nC);
  // the rings of nx XCDs hold at most (pairs + nx - 1) * (nT + nC) entries;
  // the area is sized for the most XCDs, so its size does not depend on the device
  pl->ring_off = kStPairs + 3 * pairs * kLine;
  pl->hist_off = (pl->ring_off + (size_t)(pairs + kMaxXcd) * (pl->nT + pl->nC) + kLine - 1) / kLine * kLine;
  pl->state_words = pl->hist_off + (size_t)pairs * kHistBins;
  pl->part_floats = (size_t)pairs * pl->nC * 8 * (128 + kPartHdr);
}

template <int RB, int PERB>
static hipError_t go_step_pert(const StepArgs& a, int pert, int grid, hipStream_t st) {
  static_assert(kStepChunk % 32 == 0, "a chunk is whole threads of the cut");
  switch (pert) {
    case 8: hipLaunchKernelGGL((k_step<RB, PERB, 8>), dim3(grid), dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((k_step<RB, PERB, 32>), dim3(grid), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int RB>
static hipError_t go_step_perb(const StepArgs& a, int perb, int pert, int grid, hipStream_t st) {
  switch (perb) {
    case 4: return go_step_pert<RB, 4>(a, pert, grid, st);
    case 8: return go_step_pert<RB, 8>(a, pert, grid, st);
    case 16: return go_step_pert<RB, 16>(a, pert, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step(const StepArgs& a, int grid, hipStream_t st) {
  const int perb = pow2_at_least((int)((a.NB + 255) / 256), 4);
  const int pert = a.kb <= 32 ? 8 : 32;
  return a.r == 8 ? go_step_perb<4>(a, perb, pert, grid, st) : go_step_perb<8>(a, perb, pert, grid, st);
}

}  // namespace tls

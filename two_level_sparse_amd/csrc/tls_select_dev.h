// tls_select_dev.h -- device functions of the selection stages shared by the
// selection kernels (k_select.hip) and the one-launch decode step
// (k_step.hip): sign split of the query fragments for the block-score GEMM,
// the exact block-wide radix top-k, and the INT4 label-channel token scores.
// (Internal to the HIP library; not part of the C ABI.)
#pragma once
#include "tls_dev.h"

namespace tls {

// q+ and q- of one A fragment: per 16-bit half, sign set -> negative part.
__device__ __forceinline__ void split_sign(u32x4 raw, u32x4& pos, u32x4& neg) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t mask = ((raw[e] >> 15) & 0x00010001u) * 0xFFFFu;
    neg[e] = raw[e] & mask;
    pos[e] = raw[e] & ~mask;
  }
}

// ------------------------------------------------------------------ top-k --
// Exact top-k of one row per workgroup of NT threads (256, 512 or 1024);
// keys in registers, thread t owning elements [t*PER, t*PER+PER). Invalid
// elements carry key 0, below every valid key.
constexpr int kTopkThreads = 1024;  // the largest workgroup: 16 keys per thread up to 16384
constexpr int kTopkChunk = 16384;   // the most keys one workgroup selects from

// Bins of the first (linear) pass: 1024 for the large rows of 512- and
// 1024-thread workgroups, so that the bin holding the cut keeps few keys.
template <int NT>
constexpr int topk_bins1() { return NT >= 512 ? 1024 : 256; }
constexpr int kTopkFew = 64;  // a cut bin of at most this many keys is gathered and resolved in LDS

template <int NT>
struct alignas(16) TopkLds {
  uint32_t hist0[topk_bins1<NT>()];  // first pass; later passes rotate hist0, hist[0], hist[1]
  uint32_t hist[2][256];
  uint32_t red[3][NT / 64];
  alignas(16) uint32_t scan[NT / 64];
  uint32_t few[kTopkFew];  // keys of a bin with few keys
  uint32_t nfew;
  __device__ __forceinline__ uint32_t* buf(int i) { return i == 0 ? hist0 : hist[i - 1]; }
};

// Block-wide exclusive scan of one uint32 per thread of NW waves; returns
// the prefix. Every wave reads all NW wave totals at once and adds those of
// the waves before it (a loop up to the wave's own index would make the last
// wave wait for NW-1 LDS round trips in turn).
template <int NW>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh /* one per wave */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sh[wave] = x;
  lds_sync();
  uint32_t tot[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) tot[w] = sh[w];
  uint32_t before = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) before += w < wave ? tot[w] : 0u;
  return before + x - v;
}

// The bin of an NBINS-bin histogram (NBINS = 256 or 1024) that holds the
// krem-th largest key: every wave reads the whole histogram and finds it on
// its own (wave-uniform results, no LDS round trip). Lane l holds the NBINS/64
// bins below NBINS - NBINS/64*l, so an exclusive prefix scan over lanes counts
// the keys in the bins above.
struct BinPick {
  uint32_t bin, above, count;
};
template <int NBINS = 256>
__device__ __forceinline__ BinPick pick_bin(const uint32_t* hist, uint32_t krem) {
  constexpr int PB = NBINS / 64;
  const int lane = threadIdx.x & 63;
  const int b0 = NBINS - PB * (lane + 1);
  uint32_t hb[PB];
#pragma unroll
  for (int i = 0; i < PB; i += 4) {
    const u32x4 h4 = *reinterpret_cast<const u32x4*>(&hist[b0 + i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) hb[i + e] = h4[e];
  }
  uint32_t mine = 0u;
#pragma unroll
  for (int i = 0; i < PB; ++i) mine += hb[i];
  const uint32_t above = wave_incl_scan(mine) - mine;
  const uint64_t hit = __ballot(above < krem && krem <= above + mine);
  const int L = __builtin_ctzll(hit);  // the lane whose bins hold it (one exists: krem <= keys in range)
  uint32_t bin = 0u, ab = 0u, cnt = 0u, run = above;
#pragma unroll
  for (int i = PB - 1; i >= 0; --i) {
    if (run < krem && krem <= run + hb[i]) {  // true for exactly one bin of lane L
      bin = (uint32_t)(b0 + i);
      ab = run;
      cnt = hb[i];
    }
    run += hb[i];
  }
  return BinPick{readlane(bin, L), readlane(ab, L), readlane(cnt, L)};
}

// Keys of the calling thread, four at a time: get4(j) returns its elements
// 4j .. 4j+3 (elements past PER read as 0, i.e. no element).
// RegKeys: keys in registers (fully unrolled uses keep the array there).
template <int PER>
struct RegKeys {
  const uint32_t (&k)[PER];
  __device__ __forceinline__ u32x4 get4(int j) const {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = 4 * j + i < PER ? k[4 * j + i] : 0u;
    return v;
  }
};
// LdsKeys: keys in LDS, thread t's element e (its element index t*PER + e)
// in 16-byte piece (e/4)*NT + t, word e%4: a thread reads its keys as PER/4
// pieces, and the lanes of a wave read consecutive pieces (no bank conflict).
template <int PER, int NT>
struct LdsKeys {
  const uint32_t* base;
  __device__ __forceinline__ u32x4 get4(int j) const {
    return *reinterpret_cast<const u32x4*>(base + 4 * (j * NT + (int)threadIdx.x));
  }
  // word of element c (0 <= c < NT*PER) in that layout
  static __device__ __forceinline__ int word(int c) {
    const int t = c / PER, e = c % PER;
    return 4 * ((e >> 2) * NT + t) + (e & 3);
  }
};

// Where the K largest keys end (ties: lower element index first): every key
// above thr is kept, and of the keys equal to thr the first krem in element
// order (krem = 0xFFFFFFFF: all of them); kk keys in all (K, or fewer when
// fewer are valid).
struct TopkCut {
  uint32_t thr, krem, kk;
};

// Radix select. The first pass bins the keys' float values linearly between
// the smallest and the largest (a monotone map, so a bin holds one interval
// of keys; binning the raw keys instead would put every float of one binade
// into a single bin). When the bin holding the cut has at most kTopkFew keys,
// one more pass gathers them into LDS, where the waves share out the search
// for the cut among them: for gathered key i, gt counts the keys above it and
// ge those not below it, and the key with gt < krem <= ge is the threshold.
// Otherwise the later passes histogram (key - lo) >> shift, the next 8 bits
// below the top set bit of (hi - lo), over the keys left in [lo, hi], and stop
// as soon as the chosen bin is taken whole, with the threshold at the bin's
// lower edge and every key equal to it kept. One barrier per pass: the
// histograms rotate over three buffers (a buffer is cleared two passes after
// its last read), and every wave picks the bin.
template <int PER, int NT, class Src>
__device__ TopkCut topk_cut(const Src& src, uint32_t K, TopkLds<NT>& sh) {
  constexpr int kWaves = NT / 64, NJ = (PER + 3) / 4, NB1 = topk_bins1<NT>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nval = 0u;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const u32x4 v = src.get4(j);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v[i] != 0u) {
        kmin = min(kmin, v[i]);
        kmax = max(kmax, v[i]);
        ++nval;
      }
  }
  kmin = wave_umin(kmin);
  kmax = wave_umax(kmax);
  nval = wave_usum(nval);
  if (lane == 0) {
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
    sh.red[2][wave] = nval;
  }
  for (int i = tid; i < NB1 + 256; i += NT) {  // buffers 0 and 1
    if (i < NB1) sh.hist0[i] = 0u;
    else sh.hist[0][i - NB1] = 0u;
  }
  if (tid == 0) sh.nfew = 0u;
  lds_sync();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, total = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    lo = min(lo, sh.red[0][w]);
    hi = max(hi, sh.red[1][w]);
    total += sh.red[2][w];
  }
  const uint32_t kk = K < total ? K : total;
  uint32_t thr = 0u, krem = 0u;  // kk == total: keep every valid element
  if (kk < total) {
    krem = kk;
    bool done = false;
    int pass = 0;  // histogram buffer = pass % 3; pass p clears buffer (p + 1) % 3
    const float vlo = key_float(lo), vhi = key_float(hi);
    const float sc = (float)NB1 / (vhi - vlo);
    if (hi > lo && sc > 0.0f && sc < INFINITY) {
      auto bin_of = [&](uint32_t k) { return min((uint32_t)((key_float(k) - vlo) * sc), (uint32_t)(NB1 - 1)); };
      uint32_t bn[NJ * 4];  // each key's first-pass bin (NB1: no key), kept for the gather below
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 v = src.get4(j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bn[4 * j + i] = v[i] != 0u ? bin_of(v[i]) : (uint32_t)NB1;
          if (v[i] != 0u) atomicAdd(&sh.hist0[bn[4 * j + i]], 1u);
        }
      }
      if (tid < 256) sh.hist[1][tid] = 0u;  // buffer 2 (buffer 1 was cleared at the start)
      lds_sync();
      const BinPick pk = pick_bin<NB1>(sh.hist0, krem);
      pass = 1;
      const uint32_t d = pk.bin;
      krem -= pk.above;
      if (pk.count <= (uint32_t)kTopkFew) {
        // gather the bin's keys (its count is known, so no slot overflows)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const u32x4 v = src.get4(j);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (bn[4 * j + i] == d) sh.few[atomicAdd(&sh.nfew, 1u)] = v[i];
        }
        lds_sync();
        // lane l holds gathered key l; wave w tests the keys w, w + kWaves, ..
        // against all of them with two ballots each, and the wave holding the
        // krem-th largest (1 <= krem <= c) publishes it
        const uint32_t c = pk.count;
        const uint32_t k = (uint32_t)lane < c ? sh.few[lane] : 0u;
        for (uint32_t i = (uint32_t)wave; i < c; i += kWaves) {
          const uint32_t ki = readlane(k, (int)i);
          const uint32_t gt = (uint32_t)__builtin_popcountll(__ballot(k > ki));  // empty lanes hold 0 < ki
          const uint32_t ge = (uint32_t)__builtin_popcountll(__ballot(k >= ki));
          if (gt < krem && krem <= ge && lane == 0) {  // keys equal to ki all pass and store the same
            sh.red[0][0] = ki;
            sh.red[1][0] = krem - gt;  // keys equal to thr to keep, first in element order
          }
        }
        lds_sync();
        thr = sh.red[0][0];
        krem = sh.red[1][0];
        done = true;
      } else {
        // keys of bin d: one interval [lo, hi] (a block reduction; its barrier
        // also orders this pass's histogram reads before buffer 0 is cleared)
        kmin = 0xFFFFFFFFu;
        kmax = 0u;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const u32x4 v = src.get4(j);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (bn[4 * j + i] == d) {
              kmin = min(kmin, v[i]);
              kmax = max(kmax, v[i]);
            }
        }
        kmin = wave_umin(kmin);
        kmax = wave_umax(kmax);
        if (lane == 0) {
          sh.red[0][wave] = kmin;
          sh.red[1][wave] = kmax;
        }
        lds_sync();
        lo = 0xFFFFFFFFu;
        hi = 0u;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          lo = min(lo, sh.red[0][w]);
          hi = max(hi, sh.red[1][w]);
        }
        if (krem == pk.count) {
          // the whole bin is taken: the threshold is its smallest key
          thr = lo;
          krem = 0xFFFFFFFFu;
          done = true;
        }
      }
    }
    while (!done && hi > lo) {
      const uint32_t diff = hi - lo;
      const int nbits = 32 - __clz(diff);
      const int shift = nbits > 8 ? nbits - 8 : 0;
      uint32_t* hcur = sh.buf(pass % 3);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 v = src.get4(j);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v[i] >= lo && v[i] <= hi) atomicAdd(&hcur[(v[i] - lo) >> shift], 1u);
      }
      if (tid < 256) sh.buf((pass + 1) % 3)[tid] = 0u;  // last read two barriers ago
      lds_sync();
      const BinPick pk = pick_bin(hcur, krem);
      ++pass;
      const uint32_t d = pk.bin;
      krem -= pk.above;
      const uint32_t nlo = lo + (d << shift);
      if (krem == pk.count) {
        // the whole bin is taken: every key in it is >= nlo and every key
        // of a lower bin is < nlo
        thr = nlo;
        krem = 0xFFFFFFFFu;
        done = true;
        break;
      }
      const uint32_t span = shift == 0 ? 0u : ((1u << shift) - 1u);
      hi = (hi - nlo) > span ? nlo + span : hi;
      lo = nlo;
    }
    if (!done) thr = lo;
  }
  return TopkCut{thr, krem, kk};
}

// Writes the ids of the kept elements (id(e): the id of the calling thread's
// element e) ascending in element order to out[0..kk), then -1 up to
// out_len; with out_key, their keys to out_key likewise (0 past kk). Kept
// elements are placed by one block-wide scan into `stage`, an LDS row of kk
// words or more, which goes out in coalesced stores (placing straight into
// global memory would scatter every store instruction over the wave's whole
// output range).
template <int PER, int NT, class Src, class Ids>
__device__ void topk_place(const Src& src, const TopkCut& cut, Ids id, int32_t* out, int out_len, TopkLds<NT>& sh,
                           uint32_t* stage, uint32_t* out_key = nullptr) {
  constexpr int NJ = (PER + 3) / 4;
  const int tid = threadIdx.x;
  const uint32_t thr = cut.thr, krem = cut.krem, kk = cut.kk;
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const u32x4 v = src.get4(j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gt += (v[i] > thr) ? 1u : 0u;
      eq += (v[i] == thr && v[i] != 0u) ? 1u : 0u;
    }
  }
  const uint32_t pre = block_exclusive_scan<NT / 64>(gt | (eq << 16), sh.scan);
  auto place = [&](bool ids) {
    uint32_t eq_before = pre >> 16;
    uint32_t pos = (pre & 0xFFFFu) + min(eq_before, krem);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const u32x4 v = src.get4(j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * j + i >= PER) continue;
        bool take = v[i] > thr;
        if (v[i] == thr && v[i] != 0u) {
          take = eq_before < krem;
          ++eq_before;
        }
        if (take) {
          if (pos < kk) stage[pos] = ids ? (uint32_t)id(4 * j + i) : v[i];  // never more than kk entries
          ++pos;
        }
      }
    }
  };
  place(true);
  lds_sync();
#pragma unroll 4
  for (int i = tid; i < out_len; i += NT) out[i] = i < (int)kk ? (int32_t)stage[i] : -1;
  if (out_key) {
    lds_sync();
    place(false);
    lds_sync();
    for (int i = tid; i < out_len; i += NT) out_key[i] = i < (int)kk ? stage[i] : 0u;  // key 0: no element
  }
}

// Selects the K largest of the keys in registers (thread t owning elements
// [t*PER, t*PER+PER), ids id[]) and writes their ids ascending to
// out[0..min(K, valid)), then -1 up to out_len (see topk_cut, topk_place).
// `stage`: an LDS row of NT*PER words.
template <int PER, int NT>
__device__ void block_topk(const uint32_t (&key)[PER], const int32_t (&id)[PER], uint32_t K, int32_t* out,
                           int out_len, TopkLds<NT>& sh, uint32_t* stage, uint32_t* out_key = nullptr) {
  const RegKeys<PER> src{key};
  const TopkCut cut = topk_cut<PER, NT>(src, K, sh);
  topk_place<PER, NT>(src, cut, [&](int e) { return id[e]; }, out, out_len, sh, stage, out_key);
}

// A fragments of q on the label channels, in two steps so that the gathers
// can be issued long before the fragments are needed. The workgroup of 256
// threads gathers the matrix of q on the label channels once (MT*16 rows x 32
// channel slots; rows past G repeat head G-1, so the maximum over all rows is
// the heads' maximum; slots past r are zero) and shares it through LDS: every
// wave needs all of it, and a wave gathering it alone makes MT*8 two-byte
// loads per lane at 64 scattered addresses each (for 128 heads the gathers
// alone kept a wave busy for about 6 us). Thread t gathers slot t%32 of rows
// t/32 + 8k (label_q_issue, into registers); label_q_finish writes them to
// LDS and reads the fragments back with one 16-byte read per tile from rows
// of 80 bytes (16 rows at distinct bank offsets).
// Plain form: lane (n, kq) of tile m holds head m*16 + n on channels 8kq ..
// 8kq+7. Folded form (G <= 8, one tile): lane (n, kq) holds head n&7 of half
// n>>3 on k = 8kq .. 8kq+7; half 0 takes channels 0-15 on k 0-15 and half 1
// the same channels on k 16-31, the other quarter of each row is zero.
constexpr int kLabRow = 40;  // uint16 per LDS row: 32 channels and 16 bytes of padding

template <int MT>
__device__ __forceinline__ void label_q_issue(uint32_t (&hl)[2 * MT], const int32_t* lab, const uint16_t* qp, int G,
                                              int D, int r) {
  const int t = threadIdx.x, i = t & 31;
  const int li = lab[min(i, r - 1)];
#pragma unroll
  for (int k = 0; k < 2 * MT; ++k) hl[k] = qp[(int64_t)min((t >> 5) + 8 * k, G - 1) * D + li];
}

template <int MT, bool FOLD>
__device__ __forceinline__ void label_q_finish(u32x4 (&qa)[MT], const uint32_t (&hl)[2 * MT], uint16_t* sq, int r) {
  const int t = threadIdx.x, i = t & 31;
  const int lane = t & 63, n = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int k = 0; k < 2 * MT; ++k) sq[((t >> 5) + 8 * k) * kLabRow + i] = i < r ? (uint16_t)hl[k] : (uint16_t)0;
  lds_sync();
  if constexpr (FOLD) {
    static_assert(MT == 1, "folded scores: one head tile");
    const u32x4 v = *reinterpret_cast<const u32x4*>(&sq[(n & 7) * kLabRow + 8 * (kq & 1)]);
    const bool mine = (kq >> 1) == (n >> 3);
    qa[0] = mine ? v : u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m) qa[m] = *reinterpret_cast<const u32x4*>(&sq[(m * 16 + n) * kLabRow + 8 * kq]);
  }
}

// Eight INT4 codes (one byte per channel pair, low nibble first) widened to
// bf16, exact: the B fragment of one lane.
__device__ __forceinline__ u32x4 codes_to_bf16(uint32_t w) {
  u32x4 bop;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int lo4 = (int)(w << (28 - 8 * e)) >> 28;  // channel 2e of the word
    const int hi4 = (int)(w << (24 - 8 * e)) >> 28;  // channel 2e + 1
    bop[e] = (__float_as_uint((float)lo4) >> 16) | (__float_as_uint((float)hi4) & 0xFFFF0000u);
  }
  return bop;
}

// ---- folded scores: up to 8 heads on 8 or 16 label channels, blocks of 64 ----
// One 16x16x32 MFMA carries two tiles of 16 candidates: rows 0-7 are the
// heads on k 0-15 (tile X's channels), rows 8-15 the same heads on k 16-31
// (tile Y's); B holds tile X's codes on k 0-15 and tile Y's on k 16-31.
// With G <= 8 and r <= 16 none of the product is padding, so every lane
// unpacks codes that count (a plain tile leaves half of k and half of the
// rows empty, and its lanes unpack zeros). A group of 64 candidates is one
// whole block: its codes and scales sit at a block-uniform offset (scalar)
// plus a per-lane constant, so the loads need no per-candidate address
// arithmetic. Rows past G repeat head G-1, which leaves every maximum as it is.
// NG groups of 64 candidates from candidate c0 (a multiple of 64): val[g] is
// the score of candidate cand[g] (0 if it does not exist). Lane (n, kq) ends
// with tile 2(kq&1) + (kq>>1) of its group: the MFMA of tiles 0/1 leaves
// tile 0 on rows 0-1 and tile 1 on rows 2-3, the one of tiles 2/3 likewise,
// and one 16-lane swap of the two (odd rows of the first with even rows of the
// second) pairs each tile's two row halves. `bidx` is the pair's block list.
// In two steps, so that the loads can go out before q's fragments are ready:
// fold_issue loads the codes and scales of the NG blocks, fold_scores forms
// the scores (ok[g]: candidate cand[g] exists).
template <int NG>
struct FoldLoads {
  uint32_t cwa[NG], cwb[NG];
  float tsc[NG];
  int tok0[NG];
};
template <int RB, int NG>
__device__ __forceinline__ void fold_issue(FoldLoads<NG>& L, const int32_t* bidx, __amdgpu_buffer_rsrc_t cr,
                                           __amdgpu_buffer_rsrc_t sr, int c0, int kb) {
  const int lane = threadIdx.x & 63, n = lane & 15, kq = lane >> 4;
  const int tile = 2 * (kq & 1) + (kq >> 1);
  const int voff = (n + 16 * (kq >> 1)) * RB + 4 * (kq & 1);  // tiles 0/1; +32 rows for tiles 2/3
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int blk = c0 / 64 + g;
    L.tok0[g] = __builtin_amdgcn_readfirstlane(blk < kb ? bidx[blk] : 0) * 64;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    L.cwa[g] = __builtin_amdgcn_raw_buffer_load_b32(cr, voff, L.tok0[g] * RB, 0);
    L.cwb[g] = __builtin_amdgcn_raw_buffer_load_b32(cr, voff + 32 * RB, L.tok0[g] * RB, 0);
    L.tsc[g] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, (16 * tile + n) * 4, L.tok0[g] * 4, 0));
  }
}
template <int NG>
__device__ __forceinline__ void fold_scores(float (&val)[NG], int (&cand)[NG], bool (&ok)[NG], const FoldLoads<NG>& L,
                                            int c0, int kb, int64_t N, u32x4 qa) {
  const int lane = threadIdx.x & 63, n = lane & 15, kq = lane >> 4;
  const int tile = 2 * (kq & 1) + (kq >> 1);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const f32x4 a = mfma16x16x32(qa, codes_to_bf16(L.cwa[g]), f32x4{0.f, 0.f, 0.f, 0.f});
    const f32x4 c = mfma16x16x32(qa, codes_to_bf16(L.cwb[g]), f32x4{0.f, 0.f, 0.f, 0.f});
    const float xa = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
    const float xc = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(xa), __float_as_uint(xc), false, false);
    const float best = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const int within = 16 * tile + n;
    ok[g] = c0 / 64 + g < kb && (int64_t)L.tok0[g] + within < N;
    val[g] = ok[g] ? L.tsc[g] * best : 0.0f;
    cand[g] = c0 + 64 * g + within;
  }
}
template <int RB, int NG>
__device__ __forceinline__ void fold_unit(float (&val)[NG], int (&cand)[NG], const int32_t* bidx,
                                          __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr, int c0, int kb,
                                          int64_t N, u32x4 qa) {
  FoldLoads<NG> L;
  fold_issue<RB, NG>(L, bidx, cr, sr, c0, kb);
  bool ok[NG];
  fold_scores<NG>(val, cand, ok, L, c0, kb, N, qa);
}

}  // namespace tls

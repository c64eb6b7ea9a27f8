// tls_launch.h -- host-side launchers of the gfx950 kernels (internal).
// The C ABI in include/tls.h validates arguments, then calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tls {

struct BuildArgs {
  const uint16_t* kv;
  const int32_t* label_ch;
  uint16_t* summ;
  uint8_t* codes;
  float* scale;
  int pairs, Hkv, D, row, bs, r;
  int64_t N, NB;     // tokens and blocks of every sequence
  int64_t Ns, NBs;   // per-sequence strides (allocated tokens, blocks)
  int64_t j_first;   // first block to build (blocks j_first .. NB-1)
};
hipError_t launch_build(const BuildArgs& a, hipStream_t st);
// Summaries, codes and scales after n new rows (rows [pairs, n, row]) were
// appended at N0, from the new rows and the previous summaries only.
hipError_t launch_append_index(const uint16_t* rows, int n, const int32_t* label_ch, uint16_t* summ, uint8_t* codes,
                               float* scale, int pairs, int Hkv, int D, int row, int bs, int r, int64_t N0,
                               int64_t Ns, int64_t NBs, hipStream_t st);
// Copies n_new rows per pair from src [pairs, n_new, row] to positions N0.. of kv (stride Ns tokens).
hipError_t launch_append_rows(const uint16_t* src, uint16_t* kv, int pairs, int n_new, int row, int64_t N0,
                              int64_t Ns, hipStream_t st);

struct BlockScoreArgs {
  const uint16_t* q;
  const uint16_t* summ;
  float* S;  // [pairs, NB]
  int pairs, Hq, Hkv, G, D;
  int64_t NB, NBs;  // blocks, and the summaries' per-sequence stride in blocks
};
hipError_t launch_score_blocks(const BlockScoreArgs& a, hipStream_t st);

// Stage 2 (token scores + top-k) for every pair.
struct TokenSelectArgs {
  const uint16_t* q;
  const int32_t* label_ch;
  const uint8_t* codes;
  const float* scale;
  const int32_t* block_idx;  // [pairs, kb]
  int32_t* token_idx;        // [pairs, kt], -1 padded
  int pairs, Hq, Hkv, G, D, bs, r, kb, kt;
  int64_t N, Ns;  // tokens, and the label cache's per-sequence stride
};
// Workspace of the token stage (0: unsupported): candidate scores; above
// 16384 candidates per pair also two lists for the top-k passes, which need
// Kt' <= 8192 and at most kMaxTokenCandidates candidates.
constexpr int64_t kMaxTokenCandidates = (int64_t)1 << 20;
size_t token_ws_bytes(int pairs, int64_t ncand, int kt);
hipError_t launch_select_tokens(const TokenSelectArgs& a, float* ws /* token_ws_bytes */, hipStream_t st);
// The token stage with the block top-k folded into its scoring kernel: reads
// the block scores S [pairs, NB], writes block_idx (= a.block_idx) and
// token_idx. Only where select_fused_ok(NB, kb).
bool select_fused_ok(int NB, int kb);
hipError_t launch_select_fused(const TokenSelectArgs& a, const float* S, int NB, int32_t* block_idx,
                               float* ws /* token_ws_bytes */, hipStream_t st);
// The same with the block scores computed by the token-scoring workgroups
// themselves from the summaries (the arithmetic of launch_score_blocks, so the
// same block sets): for few blocks per pair, where every workgroup reading its
// pair's summaries again costs less than a launch of the block scorer. Only
// where select_scores_inside_ok(G, D, NB, kb).
bool select_scores_inside_ok(int G, int D, int NB, int kb);
hipError_t launch_select_from_summaries(const TokenSelectArgs& a, const uint16_t* summ, int NB, int64_t NBs,
                                        int32_t* block_idx, float* ws /* token_ws_bytes */, hipStream_t st);

// Exact top-K per row of S ([rows, n] float); ids are column numbers.
hipError_t launch_topk_blocks(const float* S, int rows, int n, int K, int32_t* out, hipStream_t st);

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* slot_map;  // NULL = identity
  const int32_t* token_idx;
  void* part;               // workspace: group counters, then the partial results of the splits
  float* out;
  float* lse;               // may be NULL
  int pairs, B, Hq, Hkv, G, D, DV, row, v_off, bs, kt, slots;
  int64_t N, NB, Ns;  // Ns: per-sequence stride of kv in tokens (no slot map)
  float sm_scale;
  hipEvent_t prof_start, prof_end;  // recorded around the attention kernel when not null
};
// Decode workspace: kDecodeCntBytes of per-group counters (the fused merge
// of k_attend_pv; zero before a launch, zero after it), then the partials.
// The region has the same size and place for every shape, so calls of
// different shapes can share one workspace.
constexpr size_t kDecodeCntBytes = (size_t)64 << 10;
constexpr int kDecodeMaxGroups = (int)(kDecodeCntBytes / sizeof(int));
constexpr int64_t kFuseMaxWorkgroups = 512;  // the fused merge: one round of workgroups (two per CU)
struct DecodePlan {
  int HT, nht, tps, nsplit;
  int mla;            // 1: the MFMA latent-attention kernel (D 576, DV 512, HT 32)
  int pv;             // 1: the MFMA kernel for 128-channel K and V rows (k_attend_pv)
  int fused;          // 1: k_attend_pv merges the splits itself (at most kFuseMaxWorkgroups workgroups)
  size_t part_bytes;  // partial results (m, l, o) per split (after the counters)
};
// Always succeeds for the shapes the API accepts.
void plan_decode(int pairs, int G, int D, int DV, bool v_is_k_prefix, int kt, DecodePlan* plan);

// One transferred block (element offsets into the host cache and the resident
// cache) and one slot-map change.
struct CopyItem {
  int64_t src_elem;
  int64_t dst_elem;
};
struct MapItem {
  int64_t index;
  int32_t value;
  int32_t pad;
};
// Device-planned transfer of one step (see k_copy.hip).
constexpr int kDeltaMaxCap = 1024;    // resident slots per pair (2*Kb')
constexpr int kDeltaMaxNB = 16384;    // blocks per sequence
struct DeltaArgs {
  const int32_t* M;           // [pairs, kb] M_t, ascending
  int32_t* prev;              // [pairs, kb] M_{t-1}; becomes M_t
  int32_t* owner;             // [pairs, cap] block held by each slot, -1 free
  int32_t* last;              // [pairs, NB] last step each block was selected (-2 never, -1 prologue)
  const int32_t* map_cur;     // [pairs, NB] slot map of step t
  int32_t* map_next;          // [pairs, NB] slot map of step t+1 (written whole)
  CopyItem* items;            // [pairs, kb] transfers of the step
  int32_t* counts;            // [pairs] |T_t|
  int32_t* tblocks;           // [pairs, kb] T_t ascending, -1 padded
  unsigned long long* total;  // blocks moved since creation
  int32_t* err;               // set when a step cannot be planned
  int32_t* step_ctr;          // steps planned so far (the LRU clock), advanced by the copy kernel
  int pairs, NB, kb, cap, bs, row;  // NB: the per-pair stride of last and the maps (blocks of the capacity)
  int NBv;                    // blocks that exist now (a valid M_t holds block numbers below it)
  int copy_wgs;               // workgroups of the copy kernel
  int full;                   // 1: transfer every block of M_t (no reuse)
  int64_t N, block_elems;     // N: the per-pair stride of the host cache in tokens (the capacity)
};
// prof_start/prof_end (may be null) are recorded around the copy kernel.
hipError_t launch_device_delta(const DeltaArgs& a, const uint16_t* host_kv_dev, uint16_t* dev_cache, hipStream_t st,
                               hipEvent_t prof_start, hipEvent_t prof_end);

// New rows [pairs, n, row] of tokens N0.. into the resident slots of their
// blocks (where slot_map [pairs, NBs] has one).
hipError_t launch_patch_slots(const uint16_t* rows, int n, int pairs, int64_t N0, const int32_t* slot_map,
                              int64_t NBs, uint16_t* dev_cache, int cap, int bs, int row, hipStream_t st);

hipError_t launch_gather_blocks(const uint16_t* host_kv_dev, uint16_t* dev_cache, const CopyItem* items, int nitems,
                                const MapItem* map_items, int nmap, int32_t* slot_map, int64_t block_elems,
                                hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t st);

// One whole decode step in one launch (k_step.hip): 128-channel GQA rows,
// G <= 8, blocks of 64, 8 or 16 label channels, NB <= 4096, Kb' <= 128.
constexpr int kMaxXcd = 16;       // XCDs the state area has queues for
constexpr int kStepChunk = 512;   // candidates per attention item
struct StepArgs {
  const uint16_t* q;
  const uint16_t* summ;
  const int32_t* label_ch;
  const uint8_t* codes;
  const float* scale;
  const uint16_t* kv;
  int32_t* block_idx;  // [pairs, kb]
  int32_t* token_idx;  // [pairs, kt]
  float* out;
  float* lse;          // may be NULL
  float* S;            // [pairs, NB] block scores
  uint32_t* K;         // [pairs, kstride] candidate order keys
  uint32_t* hist;      // [pairs, 4096] histograms of the keys' top bits, inside the state area
  int* cut_info;       // [pairs, 4] threshold key, threshold-equal keys kept, kept count
  int* chunk_info;     // [pairs, nsplit, 2] kept and threshold-equal keys before each chunk
  float* part;         // [pairs, nsplit, 8, 132] partials
  int* state;          // zero at rest
  int* ring;           // [nx, ring_cap], inside the state area
  int pairs, Hq, Hkv, G, r, kb, kt;
  int64_t N, Ns, NB, NBs;
  float qk_scale;
  int nx, nA, nT, nsplit, ring_cap, kstride;
};
struct StepPlan {
  int nx, nA, nT, nC, pert, kstride, ring_cap;
  size_t ring_off;     // int32 words before the rings in the state area
  size_t hist_off;     // int32 words before the key histograms in the state area
  size_t state_words;  // int32 words of the state area (rings included; the same for any nx)
  size_t part_floats;
};
bool step_supported(int G, int D, int DV, bool v_is_k_prefix, int bs, int r, int64_t NB, int kb, int kt);
void plan_step(int pairs, int nx, int64_t NB, int kb, StepPlan* plan);
hipError_t launch_step(const StepArgs& a, int grid, hipStream_t st);

}  // namespace tls

// tls_api.cpp -- the C ABI of libtls (declared in include/tls.h): argument
// checks, workspace sizing and kernel dispatch. No allocation happens here;
// every buffer comes from the caller.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/tls.h"
#include "tls_api_internal.h"
#include "tls_launch.h"

namespace tls {

static thread_local char g_err[512] = "";
// events recorded around the profiled kernels (index: TLS_PROFILE_*)
static std::atomic<hipEvent_t> g_prof_start[3], g_prof_end[3];

void tls::profile_events(int which, hipEvent_t* start, hipEvent_t* end) {
  *start = g_prof_start[which].load(std::memory_order_relaxed);
  *end = g_prof_end[which].load(std::memory_order_relaxed);
}

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int hip_error(hipError_t e, const char* what) {
  return set_error(TLS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int derive(const tls_shape_t* s, Derived* d) {
  if (!s) return set_error(TLS_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->num_kv_heads < 1 || s->num_q_heads < 1)
    return set_error(TLS_ERR_INVALID_ARG, "batch and head counts must be >= 1");
  if (s->num_q_heads % s->num_kv_heads != 0)
    return set_error(TLS_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", s->num_q_heads,
                     s->num_kv_heads);
  if (s->head_dim_qk < 1 || s->head_dim_v < 1) return set_error(TLS_ERR_INVALID_ARG, "head dims must be >= 1");
  if (s->ctx_len < 1) return set_error(TLS_ERR_INVALID_ARG, "ctx_len must be >= 1");
  if (s->block_size < 1) return set_error(TLS_ERR_INVALID_ARG, "block_size must be >= 1");
  if (s->num_label_ch < 2 || s->num_label_ch % 2 != 0)
    return set_error(TLS_ERR_INVALID_ARG, "num_label_ch must be even and >= 2");
  if (s->top_kb < 1 || s->top_kt < 1) return set_error(TLS_ERR_INVALID_ARG, "top_kb and top_kt must be >= 1");
  if (!std::isfinite(s->sm_scale)) return set_error(TLS_ERR_INVALID_ARG, "sm_scale is not finite");
  if (s->v_is_k_prefix && s->head_dim_v > s->head_dim_qk)
    return set_error(TLS_ERR_INVALID_ARG, "v_is_k_prefix needs head_dim_v <= head_dim_qk");
  if (s->num_label_ch > s->head_dim_qk)
    return set_error(TLS_ERR_INVALID_ARG, "num_label_ch exceeds head_dim_qk");

  d->B = s->batch;
  d->Hq = s->num_q_heads;
  d->Hkv = s->num_kv_heads;
  d->G = d->Hq / d->Hkv;
  d->D = s->head_dim_qk;
  d->DV = s->head_dim_v;
  d->row = s->v_is_k_prefix ? d->D : d->D + d->DV;
  d->v_off = s->v_is_k_prefix ? 0 : d->D;
  d->N = s->ctx_len;
  d->bs = s->block_size;
  d->r = s->num_label_ch;
  d->NB = (d->N + d->bs - 1) / d->bs;
  if (s->ctx_capacity != 0 && s->ctx_capacity < s->ctx_len)
    return set_error(TLS_ERR_INVALID_ARG, "ctx_capacity (%lld) is below ctx_len (%lld)", (long long)s->ctx_capacity,
                     (long long)s->ctx_len);
  d->Ns = s->ctx_capacity ? s->ctx_capacity : d->N;
  d->NBs = (d->Ns + d->bs - 1) / d->bs;
  d->kb = (int)(s->top_kb < d->NB ? s->top_kb : d->NB);
  const int64_t cand = (int64_t)d->kb * d->bs;
  d->kt = (int)(s->top_kt < cand ? s->top_kt : cand);
  d->pairs = d->B * d->Hkv;
  d->sm = s->sm_scale;

  if (d->G > 128) return set_error(TLS_ERR_UNSUPPORTED, "more than 128 query heads per kv head");
  if (d->D % 32 != 0 || d->D > 576) return set_error(TLS_ERR_UNSUPPORTED, "head_dim_qk must be a multiple of 32, <= 576");
  if (d->DV % 8 != 0 || d->DV > 512) return set_error(TLS_ERR_UNSUPPORTED, "head_dim_v must be a multiple of 8, <= 512");
  if (d->bs > 64) return set_error(TLS_ERR_UNSUPPORTED, "block_size above 64");
  if (d->r > 32) return set_error(TLS_ERR_UNSUPPORTED, "more than 32 label channels");
  if (d->NB > 16384) return set_error(TLS_ERR_UNSUPPORTED, "more than 16384 blocks per sequence");
  if (d->Ns > (int64_t)0x7FFFFFFF) return set_error(TLS_ERR_UNSUPPORTED, "ctx_capacity above 2^31-1");
  return TLS_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ws_bytes(const Derived& d, int which) {
  switch (which) {
    case TLS_WS_BLOCKS: return round_up((size_t)d.pairs * d.NB * sizeof(float));
    case TLS_WS_TOKENS:
      return token_ws_bytes(d.pairs, (int64_t)d.kb * d.bs, d.kt);
    case TLS_WS_SELECT: {
      const size_t t = token_ws_bytes(d.pairs, (int64_t)d.kb * d.bs, d.kt);
      return t == 0 ? 0 : ws_bytes(d, TLS_WS_BLOCKS) + t;
    }
    case TLS_WS_DECODE: {
      DecodePlan pl;
      plan_decode(d.pairs, d.G, d.D, d.DV, d.v_off == 0, d.kt, &pl);
      return kDecodeCntBytes + round_up(pl.part_bytes);  // group counters, then the partials
    }
    case TLS_WS_STEP: {
      if (!step_supported(d.G, d.D, d.DV, d.v_off == 0, d.bs, d.r, d.NB, d.kb, d.kt)) return 0;
      StepPlan pl;
      plan_step(d.pairs, kMaxXcd, d.NB, d.kb, &pl);  // (the sizes do not depend on the XCD count)
      return round_up(pl.state_words * 4) + round_up((size_t)d.pairs * d.NB * 4) +
             round_up((size_t)d.pairs * pl.kstride * 4) + round_up((size_t)d.pairs * 4 * 4) +
             round_up((size_t)d.pairs * pl.nC * 2 * 4) + round_up(pl.part_floats * 4);
    }
    default: return 0;
  }
}

// XCDs (L2 domains) and compute units of the current device, queried once
// per device.
static void device_layout(int* nx, int* ncu) {
  static std::atomic<int> cache_nx[64], cache_cu[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int x = cache_nx[dev].load(std::memory_order_relaxed), c = cache_cu[dev].load(std::memory_order_relaxed);
  if (x == 0 || c == 0) {
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x < 1) x = 1;
    if (x > kMaxXcd) x = kMaxXcd;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 1;
    cache_nx[dev].store(x, std::memory_order_relaxed);
    cache_cu[dev].store(c, std::memory_order_relaxed);
  }
  *nx = x;
  *ncu = c;
}

}  // namespace tls

using namespace tls;

extern "C" {

const char* tls_last_error(void) { return g_err; }

const char* tls_version(void) { return "tls-gfx950 0.1"; }

int tls_profile_events(int which, void* start_event, void* end_event) {
  if (which != TLS_PROFILE_BLOCK_SCORES && which != TLS_PROFILE_ATTENTION && which != TLS_PROFILE_HOST_COPY)
    return set_error(TLS_ERR_INVALID_ARG, "unknown profiled kernel %d", which);
  if ((start_event == nullptr) != (end_event == nullptr))
    return set_error(TLS_ERR_INVALID_ARG, "pass both events or neither");
  g_prof_start[which].store((hipEvent_t)start_event, std::memory_order_relaxed);
  g_prof_end[which].store((hipEvent_t)end_event, std::memory_order_relaxed);
  return TLS_OK;
}

size_t tls_workspace_size(const tls_shape_t* shape, int which) {
  Derived d;
  if (derive(shape, &d) != TLS_OK) return 0;
  return ws_bytes(d, which);
}

int tls_build_summaries(const tls_shape_t* shape, const void* kv, const int32_t* label_ch, void* summ,
                        uint8_t* codes, float* scale, void* stream) {
  clear_error();
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!kv || !label_ch || !summ || !codes || !scale) return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(kv, 4) || !aligned(summ, 4) || !aligned(scale, 4) || !aligned(label_ch, 4))
    return set_error(TLS_ERR_INVALID_ARG, "kv, summ, scale and label_ch must be 4-byte aligned");
  BuildArgs a{(const uint16_t*)kv, label_ch, (uint16_t*)summ, codes, scale, d.pairs, d.Hkv, d.D, d.row, d.bs, d.r,
              d.N, d.NB, d.Ns, d.NBs, 0};
  hipError_t e = launch_build(a, (hipStream_t)stream);
  return e == hipSuccess ? TLS_OK : hip_error(e, "build_summaries launch");
}

int tls_append_kv(const tls_shape_t* shape, const void* new_kv, int32_t n_new, void* kv, const int32_t* label_ch,
                  void* summ, uint8_t* codes, float* scale, void* stream) {
  clear_error();
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!new_kv || !kv || !label_ch || !summ || !codes || !scale) return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (n_new < 1) return set_error(TLS_ERR_INVALID_ARG, "n_new must be >= 1");
  if (d.N + n_new > d.Ns)
    return set_error(TLS_ERR_INVALID_ARG, "ctx_len + n_new (%lld) exceeds ctx_capacity (%lld)",
                     (long long)(d.N + n_new), (long long)d.Ns);
  if (!aligned(new_kv, 16) || !aligned(kv, 16) || !aligned(summ, 4) || !aligned(scale, 4) || !aligned(label_ch, 4))
    return set_error(TLS_ERR_INVALID_ARG, "new_kv and kv must be 16-byte aligned, summ, scale and label_ch 4-byte");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_append_rows((const uint16_t*)new_kv, (uint16_t*)kv, d.pairs, n_new, d.row, d.N, d.Ns, st);
  if (e != hipSuccess) return hip_error(e, "append_rows launch");
  // the blocks holding the new tokens, built over all their tokens
  const int64_t N1 = d.N + n_new, NB1 = (N1 + d.bs - 1) / d.bs;
  BuildArgs a{(const uint16_t*)kv, label_ch, (uint16_t*)summ, codes, scale, d.pairs, d.Hkv, d.D, d.row, d.bs, d.r,
              N1, NB1, d.Ns, d.NBs, d.N / d.bs};
  e = launch_build(a, st);
  return e == hipSuccess ? TLS_OK : hip_error(e, "build_summaries launch (appended blocks)");
}

int tls_select_blocks(const tls_shape_t* shape, const void* q, const void* summ, int32_t* block_idx,
                      float* block_score_opt, void* ws, size_t ws_len, void* stream) {
  clear_error();
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!q || !summ || !block_idx) return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(q, 16) || !aligned(summ, 16))
    return set_error(TLS_ERR_INVALID_ARG, "q and summ must be 16-byte aligned");
  float* S = block_score_opt;
  if (!S) {
    if (!ws || ws_len < ws_bytes(d, TLS_WS_BLOCKS))
      return set_error(TLS_ERR_WORKSPACE, "workspace needs %zu bytes", ws_bytes(d, TLS_WS_BLOCKS));
    S = (float*)ws;
  }
  hipStream_t st = (hipStream_t)stream;
  BlockScoreArgs sa{(const uint16_t*)q, (const uint16_t*)summ, S, d.pairs, d.Hq, d.Hkv, d.G, d.D, d.NB, d.NBs};
  const hipEvent_t pb = g_prof_start[TLS_PROFILE_BLOCK_SCORES].load(std::memory_order_relaxed);
  const hipEvent_t pe = g_prof_end[TLS_PROFILE_BLOCK_SCORES].load(std::memory_order_relaxed);
  if (pb) (void)hipEventRecord(pb, st);
  hipError_t e = launch_score_blocks(sa, st);
  if (pe) (void)hipEventRecord(pe, st);
  if (e != hipSuccess) return hip_error(e, "score_blocks launch");
  e = launch_topk_blocks(S, d.pairs, (int)d.NB, d.kb, block_idx, st);
  return e == hipSuccess ? TLS_OK : hip_error(e, "topk(blocks) launch");
}

int tls_select_tokens(const tls_shape_t* shape, const void* q, const int32_t* label_ch, const uint8_t* codes,
                      const float* scale, const int32_t* block_idx, int32_t* token_idx, void* ws, size_t ws_len,
                      void* stream) {
  clear_error();
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!q || !label_ch || !codes || !scale || !block_idx || !token_idx)
    return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (token_ws_bytes(d.pairs, (int64_t)d.kb * d.bs, d.kt) == 0)
    return set_error(TLS_ERR_UNSUPPORTED,
                     "more than 16384 candidate tokens (Kb*bs) need Kt' <= 8192 and at most %lld candidates",
                     (long long)kMaxTokenCandidates);
  if (!ws || ws_len < ws_bytes(d, TLS_WS_TOKENS))
    return set_error(TLS_ERR_WORKSPACE, "workspace needs %zu bytes", ws_bytes(d, TLS_WS_TOKENS));
  TokenSelectArgs a{(const uint16_t*)q, label_ch, codes, scale, block_idx, token_idx, d.pairs, d.Hq, d.Hkv, d.G, d.D,
                    d.bs, d.r, d.kb, d.kt, d.N, d.Ns};
  hipError_t e = launch_select_tokens(a, (float*)ws, (hipStream_t)stream);
  return e == hipSuccess ? TLS_OK : hip_error(e, "select_tokens launch");
}

int tls_select(const tls_shape_t* shape, const void* q, const void* summ, const int32_t* label_ch,
               const uint8_t* codes, const float* scale, int32_t* block_idx, int32_t* token_idx, void* ws,
               size_t ws_len, void* stream) {
  clear_error();
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!q || !summ || !label_ch || !codes || !scale || !block_idx || !token_idx)
    return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(q, 16) || !aligned(summ, 16))
    return set_error(TLS_ERR_INVALID_ARG, "q and summ must be 16-byte aligned");
  const size_t need = ws_bytes(d, TLS_WS_SELECT);
  if (need == 0)
    return set_error(TLS_ERR_UNSUPPORTED,
                     "more than 16384 candidate tokens (Kb*bs) need Kt' <= 8192 and at most %lld candidates",
                     (long long)kMaxTokenCandidates);
  if (!ws || ws_len < need) return set_error(TLS_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return set_error(TLS_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  float* S = (float*)ws;
  float* A = (float*)((char*)ws + ws_bytes(d, TLS_WS_BLOCKS));
  TokenSelectArgs a{(const uint16_t*)q, label_ch, codes, scale, block_idx, token_idx, d.pairs, d.Hq, d.Hkv, d.G, d.D,
                    d.bs, d.r, d.kb, d.kt, d.N, d.Ns};
  hipError_t e;
  if (select_scores_inside_ok(d.G, d.D, (int)d.NB, d.kb)) {  // few blocks: no block-scorer launch
    e = launch_select_from_summaries(a, (const uint16_t*)summ, (int)d.NB, d.NBs, block_idx, A, st);
    return e == hipSuccess ? TLS_OK : hip_error(e, "select (block scores in the token stage) launch");
  }
  BlockScoreArgs sa{(const uint16_t*)q, (const uint16_t*)summ, S, d.pairs, d.Hq, d.Hkv, d.G, d.D, d.NB, d.NBs};
  const hipEvent_t pb = g_prof_start[TLS_PROFILE_BLOCK_SCORES].load(std::memory_order_relaxed);
  const hipEvent_t pe = g_prof_end[TLS_PROFILE_BLOCK_SCORES].load(std::memory_order_relaxed);
  if (pb) (void)hipEventRecord(pb, st);
  e = launch_score_blocks(sa, st);
  if (pe) (void)hipEventRecord(pe, st);
  if (e != hipSuccess) return hip_error(e, "score_blocks launch");
  if (select_fused_ok((int)d.NB, d.kb)) {
    e = launch_select_fused(a, S, (int)d.NB, block_idx, A, st);
    return e == hipSuccess ? TLS_OK : hip_error(e, "select (fused token stage) launch");
  }
  e = launch_topk_blocks(S, d.pairs, (int)d.NB, d.kb, block_idx, st);
  if (e != hipSuccess) return hip_error(e, "topk(blocks) launch");
  e = launch_select_tokens(a, A, st);
  return e == hipSuccess ? TLS_OK : hip_error(e, "select_tokens launch");
}

int tls_decode_step(const tls_shape_t* shape, const void* q, const void* summ, const int32_t* label_ch,
                    const uint8_t* codes, const float* scale, const void* kv, int32_t* block_idx, int32_t* token_idx,
                    float* out, float* lse_opt, void* ws, size_t ws_len, void* stream) {
  clear_error();
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!q || !summ || !label_ch || !codes || !scale || !kv || !block_idx || !token_idx || !out)
    return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(q, 16) || !aligned(summ, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(scale, 4) ||
      !aligned(codes, 4))
    return set_error(TLS_ERR_INVALID_ARG, "q, summ, kv and out must be 16-byte aligned, codes and scale 4-byte");
  if (!step_supported(d.G, d.D, d.DV, d.v_off == 0, d.bs, d.r, d.NB, d.kb, d.kt))
    return set_error(TLS_ERR_UNSUPPORTED,
                     "tls_decode_step covers D = DV = 128 with separate V, G <= 8, block size 64, 8 or 16 label "
                     "channels, NB <= 4096 and Kb' <= 128 (use tls_select and tls_sparse_decode)");
  if ((int64_t)d.Ns * (d.r / 2) > 0x7FFFFFFF)
    return set_error(TLS_ERR_UNSUPPORTED, "label cache of a sequence above 2 GiB");
  const size_t need = ws_bytes(d, TLS_WS_STEP);
  if (!ws || ws_len < need) return set_error(TLS_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return set_error(TLS_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  int nx = 1, ncu = 1;
  device_layout(&nx, &ncu);
  StepPlan pl;
  plan_step(d.pairs, nx, d.NB, d.kb, &pl);
  char* w = (char*)ws;
  StepArgs a;
  a.q = (const uint16_t*)q;
  a.summ = (const uint16_t*)summ;
  a.label_ch = label_ch;
  a.codes = codes;
  a.scale = scale;
  a.kv = (const uint16_t*)kv;
  a.block_idx = block_idx;
  a.token_idx = token_idx;
  a.out = out;
  a.lse = lse_opt;
  a.state = (int*)w;
  a.ring = a.state + pl.ring_off;
  a.hist = (uint32_t*)(a.state + pl.hist_off);
  w += round_up(pl.state_words * 4);
  a.S = (float*)w;
  w += round_up((size_t)d.pairs * d.NB * 4);
  a.K = (uint32_t*)w;
  w += round_up((size_t)d.pairs * pl.kstride * 4);
  a.cut_info = (int*)w;
  w += round_up((size_t)d.pairs * 4 * 4);
  a.chunk_info = (int*)w;
  w += round_up((size_t)d.pairs * pl.nC * 2 * 4);
  a.part = (float*)w;
  a.pairs = d.pairs;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.r = d.r;
  a.kb = d.kb;
  a.kt = d.kt;
  a.N = d.N;
  a.Ns = d.Ns;
  a.NB = d.NB;
  a.NBs = d.NBs;
  a.qk_scale = d.sm * 1.4426950408889634f;
  a.nx = pl.nx;
  a.nA = pl.nA;
  a.nT = pl.nT;
  a.nsplit = pl.nC;
  a.ring_cap = pl.ring_cap;
  a.kstride = pl.kstride;
  hipError_t e = launch_step(a, 2 * ncu, (hipStream_t)stream);
  return e == hipSuccess ? TLS_OK : hip_error(e, "decode_step launch");
}

int tls_decode_step_status(void* ws, void* stream) {
  clear_error();
  if (!ws) return set_error(TLS_ERR_INVALID_ARG, "NULL workspace");
  int err = 0;
  hipError_t e = hipMemcpyAsync(&err, ws, sizeof err, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_error(e, "decode_step status read");
  if (err & 1) return set_error(TLS_ERR_STATE, "an attention item was not published in time (error word %d)", err);
  if (err) return set_error(TLS_ERR_STATE, "a queue was left undrained (error word %d)", err);
  return TLS_OK;
}

}  // extern "C"

// ---- scratch of tls_sparse_decode_noalloc
// The library's own device array for the split partials of the attention, for
// callers that cannot allocate. Each GPU the library runs on holds its own
// copy (at its own address) until the process ends. In host code `scratch`
// names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept; only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[TLS_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];
static std::mutex g_scratch_mutex;

// The current device's address of `scratch`; nullptr (error message set) if
// the lookup fails.
static void* scratch_address() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_error(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error(TLS_ERR_UNSUPPORTED, "device %d: the scratch array is tracked for devices 0..%d", dev, kMaxDevices - 1);
    return nullptr;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    return nullptr;
  }
  g_scratch_addr[dev].store(p, std::memory_order_release);
  return p;
}

// The attention (tls_sparse_decode) with its split partials in `part`.
static int sparse_decode(const tls_shape_t* shape, const void* q, const void* kv_cache, const int32_t* slot_map,
                         int32_t slots_per_pair, const int32_t* token_idx, float* out, float* lse_opt, void* part,
                         size_t part_len, bool own_scratch, void* stream) {
  Derived d;
  int rc = derive(shape, &d);
  if (rc) return rc;
  if (!q || !kv_cache || !token_idx || !out) return set_error(TLS_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(q, 16) || !aligned(kv_cache, 16))
    return set_error(TLS_ERR_INVALID_ARG, "q and kv_cache must be 16-byte aligned");
  if (slot_map && slots_per_pair < 1) return set_error(TLS_ERR_INVALID_ARG, "slots_per_pair must be >= 1");
  const bool dims_ok = (d.D == 64 && d.DV == 64) || (d.D == 128 && d.DV == 128) || (d.D == 256 && d.DV == 256) ||
                       (d.D == 576 && d.DV == 512);
  if (!dims_ok)
    return set_error(TLS_ERR_UNSUPPORTED, "attention is compiled for (D,DV) in {(64,64),(128,128),(256,256),(576,512)}");
  DecodePlan pl;
  plan_decode(d.pairs, d.G, d.D, d.DV, d.v_off == 0, d.kt, &pl);
  const size_t need = ws_bytes(d, TLS_WS_DECODE);
  if (own_scratch) {
    if (need > TLS_NOALLOC_SCRATCH_BYTES)
      return set_error(TLS_ERR_WORKSPACE,
                       "the split partials of this shape need %zu bytes, above the %zu-byte scratch array of "
                       "tls_sparse_decode_noalloc (use tls_sparse_decode with a workspace)",
                       need, (size_t)TLS_NOALLOC_SCRATCH_BYTES);
    part = scratch_address();
    if (!part) return TLS_ERR_HIP;  // (message set by scratch_address)
  } else if (!part || part_len < need) {
    return set_error(TLS_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  }
  DecodeArgs a{(const uint16_t*)q, (const uint16_t*)kv_cache, slot_map, token_idx, part, out, lse_opt,
               d.pairs, d.B, d.Hq, d.Hkv, d.G, d.D, d.DV, d.row, d.v_off, d.bs, d.kt,
               slot_map ? slots_per_pair : 0, d.N, d.NBs, d.Ns, d.sm,  // (NBs: the slot map's per-pair stride)
               g_prof_start[TLS_PROFILE_ATTENTION].load(std::memory_order_relaxed),
               g_prof_end[TLS_PROFILE_ATTENTION].load(std::memory_order_relaxed)};
  hipError_t e = launch_decode(a, pl, (hipStream_t)stream);
  return e == hipSuccess ? TLS_OK : hip_error(e, "sparse_decode launch");
}

extern "C" {

int tls_sparse_decode(const tls_shape_t* shape, const void* q, const void* kv_cache, const int32_t* slot_map,
                      int32_t slots_per_pair, const int32_t* token_idx, float* out, float* lse_opt, void* ws,
                      size_t ws_len, void* stream) {
  clear_error();
  return sparse_decode(shape, q, kv_cache, slot_map, slots_per_pair, token_idx, out, lse_opt, ws, ws_len, false,
                       stream);
}

int tls_sparse_decode_noalloc(const tls_shape_t* shape, const void* q, const void* kv_cache, const int32_t* slot_map,
                              int32_t slots_per_pair, const int32_t* token_idx, float* out, float* lse_opt,
                              void* stream) {
  clear_error();
  return sparse_decode(shape, q, kv_cache, slot_map, slots_per_pair, token_idx, out, lse_opt, nullptr, 0, true,
                       stream);
}

}  // extern "C"

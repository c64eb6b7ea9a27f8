/*
 * tls_oracle.c -- plain fp64 CPU oracle for one decode step of two-level
 * sparse attention (AsyncTLS), and for the staggered offloaded schedule.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline of the benchmark may load this library. It shares no code, header,
 * table or helper with the HIP implementation, and the product path never
 * calls it.
 *
 * Source of the method: the AsyncTLS pages ("AsyncTLS: Efficient Generative
 * LLM Inference with Asynchronous Two-level Sparse Attention"), section 2
 * "Methodology" (A: hierarchical two-level sparse attention; B: asynchronous
 * offloading engine). The pages print no formulas; where they are silent the
 * readings below are taken (each is listed with its reason in the design
 * notes of the repository):
 *   - block summary = per-channel max and min of the keys of a block
 *     (the Italian page, section 2A, names the key maximum and minimum);
 *   - block score = Quest upper bound sum_c max(q_c*Kmax_c, q_c*Kmin_c), which
 *     equals [q+, q-] . [Kmax; Kmin] (the GEMM form of section 2A);
 *   - the G query heads that share a kv head are combined by max, for blocks
 *     and for tokens, and one selection is made per (batch, kv head);
 *   - INT4 label cache: per-token symmetric absmax over the label channels,
 *     codes in [-7, 7], fp32 scale a/7, quantizer evaluated in fp64;
 *   - ties in any top-k go to the lower index;
 *   - attention is exact softmax over the selected tokens only;
 *   - staggered schedule: tokens of step t come from the blocks selected at
 *     step t-1; the incremental transfer is T_t = M_t minus the resident set;
 *     capacity 2*Kb blocks per pair; least-recently-selected blocks outside
 *     M_{t-1} and M_t are evicted first (lower block index on ties).
 *
 * All arithmetic is in double. bf16 inputs arrive as uint16 bit patterns and
 * widen exactly. Products of two bf16 numbers are exact in double.
 *
 * Parity pins (tests/test_oracle_pins.py): dense attention when Kb and Kt
 * cover everything, the upper-bound property of block scores, brute-force
 * selection on tiny inputs with forced ties, block size 1, the Quest-only and
 * DS-only special cases, quantizer bounds, exact round trips and exact
 * half-way ties, log-sum-exp against a library routine, a zero-drift
 * staggered run, and drifting runs whose evictions are replayed by an
 * independent LRU.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t B, Hq, Hkv; /* batch, query heads, kv heads; G = Hq / Hkv        */
  int32_t D, DV;      /* query/key dimension, value dimension               */
  int32_t row;        /* elements per cached token row                      */
  int32_t v_off;      /* offset of V in a row (0: V is the key prefix)      */
  int64_t N;          /* tokens per sequence                                */
  int32_t bs;         /* tokens per block                                   */
  int32_t r;          /* label channels                                     */
  int32_t Kb, Kt;     /* blocks and tokens kept                             */
  double sm_scale;    /* softmax scale applied to q.k                       */
} orc_shape_t;

static double bf(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int64_t nblocks(const orc_shape_t *s) { return (s->N + s->bs - 1) / s->bs; }

/* ---------------------------------------------------------------- top-k --
 * Section 2A keeps the top-Kb blocks and then the top-Kt tokens. Order by score descending, lower index first on equal
 * scores, keep the first min(K, n), return them in ascending index order.  */
typedef struct {
  double s;
  int32_t i;
} orc_item;

static int by_score_then_index(const void *a, const void *b) {
  const orc_item *x = (const orc_item *)a, *y = (const orc_item *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->i > y->i) - (x->i < y->i);
}

static int by_index(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* scores[n], ids[n] (the index each score belongs to) -> out[0..k) ascending. */
int orc_topk(const double *scores, const int32_t *ids, int64_t n, int64_t K, int32_t *out) {
  if (n <= 0 || K <= 0) return 0;
  orc_item *it = (orc_item *)malloc((size_t)n * sizeof *it);
  if (!it) return -1;
  for (int64_t j = 0; j < n; ++j) {
    it[j].s = scores[j];
    it[j].i = ids ? ids[j] : (int32_t)j;
  }
  qsort(it, (size_t)n, sizeof *it, by_score_then_index);
  int64_t k = K < n ? K : n;
  for (int64_t j = 0; j < k; ++j) out[j] = it[j].i;
  qsort(out, (size_t)k, sizeof *out, by_index);
  free(it);
  return (int)k;
}

/* ------------------------------------------------- O1: block summaries --
 * Section 2A: the cache is partitioned into blocks, each with a compressed
 * key summary (its per-channel maximum and minimum). Block j holds tokens
 * [j*bs, min((j+1)*bs, N)).  kv_pair [N, row]; kmax/kmin [NB, D].          */
void orc_summaries_pair(const orc_shape_t *s, const uint16_t *kv_pair, double *kmax, double *kmin) {
  int64_t NB = nblocks(s);
  for (int64_t j = 0; j < NB; ++j) {
    int64_t t0 = j * s->bs, t1 = t0 + s->bs < s->N ? t0 + s->bs : s->N;
    for (int c = 0; c < s->D; ++c) {
      double mx = -INFINITY, mn = INFINITY;
      for (int64_t t = t0; t < t1; ++t) {
        double k = bf(kv_pair[t * s->row + c]);
        if (k > mx) mx = k;
        if (k < mn) mn = k;
      }
      kmax[j * s->D + c] = mx;
      kmin[j * s->D + c] = mn;
    }
  }
}

/* ----------------------------------------- O2: INT4 label-channel cache --
 * Section 2A (token stage): channel selection plus INT4 quantisation of the
 * key vectors. Per token t over its label channels c_0 < ... < c_{r-1}:
 *   a = max_i |K[t, c_i]|;  a == 0 -> scale 0 and all codes 0;
 *   otherwise scale = fp32(a / 7) and code_i = clamp(rint(K[t,c_i] / scale), -7, 7),
 * both divisions in double, rint rounding half to even.
 * codes [N, r] int8, scale [N] float.                                       */
void orc_quantize_pair(const orc_shape_t *s, const uint16_t *kv_pair, const int32_t *lab,
                       int8_t *codes, float *scale) {
  for (int64_t t = 0; t < s->N; ++t) {
    double a = 0.0;
    for (int i = 0; i < s->r; ++i) {
      double k = fabs(bf(kv_pair[t * s->row + lab[i]]));
      if (k > a) a = k;
    }
    if (a == 0.0) {
      scale[t] = 0.0f;
      for (int i = 0; i < s->r; ++i) codes[t * s->r + i] = 0;
      continue;
    }
    float sc = (float)(a / 7.0);
    scale[t] = sc;
    for (int i = 0; i < s->r; ++i) {
      double v = rint(bf(kv_pair[t * s->row + lab[i]]) / (double)sc);
      if (v > 7.0) v = 7.0;
      if (v < -7.0) v = -7.0;
      codes[t * s->r + i] = (int8_t)v;
    }
  }
}

/* Nibble packing of the codes: channel i goes to byte i/2, low nibble when i
 * is even, as the two's-complement low 4 bits of the code.  codes [n, r] ->
 * packed [n, r/2].                                                          */
void orc_pack_codes(const int8_t *codes, int64_t n, int r, uint8_t *packed) {
  for (int64_t t = 0; t < n; ++t)
    for (int i = 0; i < r; i += 2) {
      uint8_t lo = (uint8_t)(codes[t * r + i] & 0xF), hi = (uint8_t)(codes[t * r + i + 1] & 0xF);
      packed[t * (r / 2) + i / 2] = (uint8_t)(lo | (hi << 4));
    }
}

/* -------------------------------- O3 + O4 + O5: block filtering (stage 1) --
 * Section 2A: block importance from the summaries, computed in GEMM form,
 * then the top-Kb blocks form the candidate set M.
 *   s[g, j] = sum_c max(q_gc*Kmax_jc, q_gc*Kmin_jc)
 *           = sum_c ( max(q_gc,0)*Kmax_jc + min(q_gc,0)*Kmin_jc )
 * Both forms are evaluated, term by term in channel order; they must agree
 * exactly (each term of the second form has one exact zero summand).
 *   S[j] = max_g s[g, j];   M = top-Kb of S.
 * q_pair [G, D] bf16 bits; s_head [G, NB] (may be NULL); S [NB];
 * block_idx [min(Kb, NB)]. Returns the count, or -2 if the two forms differ. */
int orc_select_blocks_pair(const orc_shape_t *s, const uint16_t *q_pair, const double *kmax,
                           const double *kmin, double *s_head, double *S, int32_t *block_idx) {
  int G = s->Hq / s->Hkv;
  int64_t NB = nblocks(s);
  int bad = 0;
  for (int64_t j = 0; j < NB; ++j) {
    double best = -INFINITY;
    for (int g = 0; g < G; ++g) {
      double bound = 0.0, gemm = 0.0;
      for (int c = 0; c < s->D; ++c) {
        double q = bf(q_pair[g * s->D + c]);
        double hi = q * kmax[j * s->D + c], lo = q * kmin[j * s->D + c];
        bound += hi > lo ? hi : lo;
        gemm += (q > 0.0 ? q : 0.0) * kmax[j * s->D + c] + (q < 0.0 ? q : 0.0) * kmin[j * s->D + c];
      }
      if (bound != gemm) bad = 1;
      if (s_head) s_head[(int64_t)g * NB + j] = bound;
      if (bound > best) best = bound;
    }
    S[j] = best;
  }
  if (bad) return -2;
  return orc_topk(S, NULL, NB, s->Kb, block_idx);
}

/* -------------------------------- O6 + O7 + O8: token selection (stage 2) --
 * Section 2A: inside the selected blocks, Double-Sparsity style scores on the
 * label channels of the INT4 cache; the top-Kt tokens are kept.
 *   a[g, t] = scale_t * sum_i q[g, c_i] * code[t, i]   (q is not quantised)
 *   A[t]    = max_g a[g, t]
 * Candidates are the valid tokens (t < N) of the blocks in block_idx, in
 * ascending token order. cand_tok/cand_score (may be NULL) receive them.
 * Returns the number of selected tokens written to token_idx.              */
int orc_select_tokens_pair(const orc_shape_t *s, const uint16_t *q_pair, const int32_t *lab,
                           const int8_t *codes, const float *scale, const int32_t *block_idx,
                           int nblk, int32_t *token_idx, int32_t *cand_tok, double *cand_score,
                           int64_t *n_cand) {
  int G = s->Hq / s->Hkv;
  int64_t cap = (int64_t)nblk * s->bs;
  int32_t *ids = (int32_t *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof *ids);
  double *A = (double *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof *A);
  if (!ids || !A) {
    free(ids);
    free(A);
    return -1;
  }
  int64_t n = 0;
  for (int b = 0; b < nblk; ++b) {
    int64_t t0 = (int64_t)block_idx[b] * s->bs;
    for (int64_t t = t0; t < t0 + s->bs && t < s->N; ++t) {
      double best = -INFINITY;
      for (int g = 0; g < G; ++g) {
        double dot = 0.0;
        for (int i = 0; i < s->r; ++i) dot += bf(q_pair[g * s->D + lab[i]]) * (double)codes[t * s->r + i];
        double a = (double)scale[t] * dot;
        if (a > best) best = a;
      }
      ids[n] = (int32_t)t;
      A[n] = best;
      ++n;
    }
  }
  if (cand_tok) memcpy(cand_tok, ids, (size_t)n * sizeof *ids);
  if (cand_score) memcpy(cand_score, A, (size_t)n * sizeof *A);
  if (n_cand) *n_cand = n;
  int k = orc_topk(A, ids, n, s->Kt, token_idx);
  free(ids);
  free(A);
  return k;
}

/* ------------------------------------------- O9: attention over the set --
 * Section 2A: attention is computed only over the selected tokens. For each
 * query head g:  z_t = sm_scale * q_g . K[t],  m = max z,  l = sum exp(z - m),
 * o_g = sum exp(z_t - m) V[t] / l,  lse_g = m + ln l, in ascending t order.
 * V[t] is the DV entries at offset v_off of the token's row.
 * out [G, DV], lse [G] (may be NULL).                                       */
void orc_attend_pair(const orc_shape_t *s, const uint16_t *q_pair, const uint16_t *kv_pair,
                     const int32_t *tok, int n, double *out, double *lse) {
  int G = s->Hq / s->Hkv;
  double *z = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof *z);
  for (int g = 0; g < G; ++g) {
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      const uint16_t *k = kv_pair + (int64_t)tok[j] * s->row;
      double dot = 0.0;
      for (int c = 0; c < s->D; ++c) dot += bf(q_pair[g * s->D + c]) * bf(k[c]);
      z[j] = s->sm_scale * dot;
      if (z[j] > m) m = z[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) l += exp(z[j] - m);
    for (int c = 0; c < s->DV; ++c) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += exp(z[j] - m) * bf(kv_pair[(int64_t)tok[j] * s->row + s->v_off + c]);
      out[g * s->DV + c] = n > 0 ? acc / l : 0.0;
    }
    if (lse) lse[g] = n > 0 ? m + log(l) : -INFINITY;
  }
  free(z);
}

/* --------------------------------------------------------- whole step ----
 * The full pipeline for a list of (batch, kv head) pairs p = b*Hkv + h,
 * parallel over pairs. Buffers are indexed by the position in the list.
 *   q [B, Hq, D], kv [B, Hkv, N, row], label_ch [Hkv, r]
 *   kmax/kmin [np, NB, D], codes [np, N, r], scale [np, N]: built here when
 *     build != 0, otherwise taken as given (built by an earlier call).
 *   force_blocks [np, Kb] (may be NULL): use these block sets instead of
 *     stage 1 (to test later stages on identical selections).
 *   force_tokens [np, Kt] + force_ntok [np] (may be NULL): same for stage 2.
 *   S [np, NB], block_idx [np, Kb'], token_idx [np, Kt'], ntok [np],
 *   out [np, G, DV], lse [np, G]   (Kb' = min(Kb, NB), Kt' = min(Kt, Kb'*bs)).
 * Returns 0, or a negative value if a step failed.                          */
int orc_decode(const orc_shape_t *s, const uint16_t *q, const uint16_t *kv, const int32_t *label_ch,
               const int32_t *pairs, int np, int build, double *kmax, double *kmin, int8_t *codes,
               float *scale, const int32_t *force_blocks, const int32_t *force_tokens,
               const int32_t *force_ntok, double *S, int32_t *block_idx, int32_t *token_idx,
               int32_t *ntok, double *out, double *lse) {
  int G = s->Hq / s->Hkv;
  int64_t NB = nblocks(s);
  int kb = (int)(s->Kb < NB ? s->Kb : NB);
  int64_t ktc = (int64_t)kb * s->bs;
  int kt = (int)(s->Kt < ktc ? s->Kt : ktc);
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
  for (int i = 0; i < np; ++i) {
    int p = pairs[i], b = p / s->Hkv, h = p % s->Hkv;
    const uint16_t *qp = q + ((int64_t)b * s->Hq + (int64_t)h * G) * s->D;
    const uint16_t *kvp = kv + (int64_t)p * s->N * s->row;
    const int32_t *lab = label_ch + (int64_t)h * s->r;
    double *mx = kmax + (int64_t)i * NB * s->D, *mn = kmin + (int64_t)i * NB * s->D;
    int8_t *cd = codes + (int64_t)i * s->N * s->r;
    float *sc = scale + (int64_t)i * s->N;
    if (build) {
      orc_summaries_pair(s, kvp, mx, mn);
      orc_quantize_pair(s, kvp, lab, cd, sc);
    }
    int32_t *bi = block_idx + (int64_t)i * kb;
    int nb = orc_select_blocks_pair(s, qp, mx, mn, NULL, S + (int64_t)i * NB, bi);
    if (nb < 0) {
      err = nb;
      continue;
    }
    if (force_blocks) memcpy(bi, force_blocks + (int64_t)i * kb, (size_t)kb * sizeof *bi);
    int32_t *ti = token_idx + (int64_t)i * kt;
    int nt = orc_select_tokens_pair(s, qp, lab, cd, sc, bi, kb, ti, NULL, NULL, NULL);
    if (nt < 0) {
      err = nt;
      continue;
    }
    if (force_tokens) {
      nt = force_ntok[i];
      memcpy(ti, force_tokens + (int64_t)i * kt, (size_t)nt * sizeof *ti);
    }
    ntok[i] = nt;
    orc_attend_pair(s, qp, kvp, ti, nt, out + (int64_t)i * G * s->DV, lse ? lse + (int64_t)i * G : NULL);
  }
  return err;
}

/* Copies a given block set (ascending, distinct, in [0, NB)) into dst; -1 if
 * it is not one. */
static int orc_force_set(int32_t *dst, const int32_t *src, int kb, int64_t NB) {
  for (int j = 0; j < kb; ++j) {
    if (src[j] < 0 || src[j] >= NB || (j > 0 && src[j] <= src[j - 1])) return -1;
    dst[j] = src[j];
  }
  return 0;
}

/* ------------------------------------------- O10: staggered offloaded run --
 * Section 2B: block selections are stable across consecutive steps
 * (M_t ~ M_{t-1}); at step t the token stage runs inside M_{t-1} while M_t is
 * computed, and only T_t = M_t \ C_t (C_t: the blocks resident on the device)
 * is transferred.
 *   prologue: M_{-1} = top-Kb(q_0), loaded synchronously, C_0 = M_{-1};
 *   step t:   tokens = top-Kt over cand(M_{t-1}) scored with q_t,
 *             out_t  = attention(q_t, tokens);
 *             M_t    = top-Kb(q_t);  T_t = M_t \ C_t;
 *             if |C_t| + |T_t| > 2*Kb, evict the excess from
 *             C_t \ (M_{t-1} u M_t), least recently selected first (lower
 *             block index on equal steps);  C_{t+1} = (C_t - evicted) u T_t.
 * qs [steps, B, Hq, D]; kmax/kmin/codes/scale as built by orc_decode for ALL
 * pairs in order (np = B*Hkv).
 * force_prologue [np, Kb'] and force_M [steps, np, Kb'] (each may be NULL):
 *   block sets, ascending, used in place of the prologue's and step t's own
 *   stage 1 -- so that a run whose selections differ from these only among
 *   blocks of (nearly) equal score can be followed step by step.
 * lens [steps + 1] (may be NULL: every length is s->N): a cache that grows
 *   at decode time (pages, section 1: the cache grows with every generated
 *   token). s->N is then the allocated length (the stride of kv, codes and
 *   scale, which are given for all of it); the prologue sees the first
 *   lens[0] tokens and step t the first lens[t+1] (non-decreasing, each with
 *   at least Kb blocks): its token stage, attention and selection M_t all use
 *   that prefix, with block summaries built from it (the INT4 codes of a
 *   token depend on its own row only, so those of the whole length serve).
 *   Blocks that do not exist yet are never selected and never resident.
 * Outputs per step t and pair p:
 *   M [steps, np, Kb'] ; T [steps, np, Kb'] (first nT entries, ascending);
 *   nT [steps, np]; nevict [steps, np]; evicted [steps, np, 2*Kb'] (may be
 *   NULL: the first nevict entries, in eviction order); out [steps, np, G, DV];
 *   lse [steps, np, G].
 * Returns 0, or a negative value if the schedule was violated (-6: lens
 * invalid).                                                                 */
int orc_staggered(const orc_shape_t *s, int steps, const uint16_t *qs, const uint16_t *kv,
                  const int32_t *label_ch, const double *kmax, const double *kmin,
                  const int8_t *codes, const float *scale, const int32_t *force_prologue,
                  const int32_t *force_M, const int64_t *lens, int32_t *M, int32_t *T, int32_t *nT,
                  int32_t *nevict, int32_t *evicted, double *out, double *lse) {
  int G = s->Hq / s->Hkv;
  int np = s->B * s->Hkv;
  int64_t NB = nblocks(s); /* blocks of the whole (capacity) length */
  int kb = (int)(s->Kb < NB ? s->Kb : NB);
  /* A growing cache: every length must keep Kb' and Kt' unchanged, i.e. hold
   * at least Kb blocks from the first selection on, and never shrink. */
  if (lens) {
    for (int t = 0; t <= steps; ++t) {
      if (lens[t] < 1 || lens[t] > s->N || (t > 0 && lens[t] < lens[t - 1])) return -6;
      if ((lens[t] + s->bs - 1) / s->bs < s->Kb) return -6;
    }
  }
  int64_t ktc = (int64_t)kb * s->bs;
  int kt = (int)(s->Kt < ktc ? s->Kt : ktc);
  int cap = 2 * kb;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
  for (int p = 0; p < np; ++p) {
    int b = p / s->Hkv, h = p % s->Hkv;
    const uint16_t *kvp = kv + (int64_t)p * s->N * s->row;
    const int32_t *lab = label_ch + (int64_t)h * s->r;
    const double *mx = kmax + (int64_t)p * NB * s->D, *mn = kmin + (int64_t)p * NB * s->D;
    const int8_t *cd = codes + (int64_t)p * s->N * s->r;
    const float *sc = scale + (int64_t)p * s->N;
    double *Sbuf = (double *)malloc((size_t)NB * sizeof(double));
    int32_t *prev = (int32_t *)malloc((size_t)kb * sizeof(int32_t));
    int32_t *cur = (int32_t *)malloc((size_t)kb * sizeof(int32_t));
    int32_t *tok = (int32_t *)malloc((size_t)(kt > 0 ? kt : 1) * sizeof(int32_t));
    char *resident = (char *)calloc((size_t)NB, 1), *in_prev = (char *)calloc((size_t)NB, 1),
         *in_cur = (char *)calloc((size_t)NB, 1);
    int64_t *last = (int64_t *)malloc((size_t)NB * sizeof(int64_t));
    orc_item *ev = (orc_item *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(orc_item));
    int n_res = 0, perr = 0;
    /* the cache as it is when a selection or step runs: lens[0] tokens for
     * the prologue, lens[t+1] for step t (its token stage, its attention and
     * its own selection); the summaries of that prefix are built afresh */
    orc_shape_t cs = *s;
    double *gmx = NULL, *gmn = NULL;
    if (lens) {
      gmx = (double *)malloc((size_t)NB * s->D * sizeof(double));
      gmn = (double *)malloc((size_t)NB * s->D * sizeof(double));
      cs.N = lens[0];
      orc_summaries_pair(&cs, kvp, gmx, gmn);
      mx = gmx;
      mn = gmn;
    }
    const uint16_t *q0 = qs + ((int64_t)b * s->Hq + (int64_t)h * G) * s->D;
    if (orc_select_blocks_pair(&cs, q0, mx, mn, NULL, Sbuf, prev) < 0) perr = -2;
    if (force_prologue && orc_force_set(prev, force_prologue + (int64_t)p * kb, kb, nblocks(&cs)) != 0) perr = -5;
    for (int j = 0; j < kb; ++j) {
      resident[prev[j]] = 1;
      last[prev[j]] = -1;
    }
    n_res = kb;
    for (int t = 0; t < steps && perr == 0; ++t) {
      const uint16_t *qt = qs + (((int64_t)t * s->B + b) * s->Hq + (int64_t)h * G) * s->D;
      if (lens && lens[t + 1] != cs.N) { /* rows appended before step t */
        cs.N = lens[t + 1];
        orc_summaries_pair(&cs, kvp, gmx, gmn);
      }
      for (int j = 0; j < kb; ++j)
        if (!resident[prev[j]]) perr = -3; /* a block in use must be resident */
      int nt = orc_select_tokens_pair(&cs, qt, lab, cd, sc, prev, kb, tok, NULL, NULL, NULL);
      int64_t o = (int64_t)t * np + p;
      orc_attend_pair(&cs, qt, kvp, tok, nt, out + o * G * s->DV, lse + o * G);
      if (orc_select_blocks_pair(&cs, qt, mx, mn, NULL, Sbuf, cur) < 0) perr = -2;
      if (force_M && orc_force_set(cur, force_M + o * kb, kb, nblocks(&cs)) != 0) perr = -5;
      memset(in_prev, 0, (size_t)NB);
      memset(in_cur, 0, (size_t)NB);
      for (int j = 0; j < kb; ++j) {
        in_prev[prev[j]] = 1;
        in_cur[cur[j]] = 1;
      }
      int32_t *Tt = T + o * kb;
      int ntr = 0;
      for (int j = 0; j < kb; ++j)
        if (!resident[cur[j]]) Tt[ntr++] = cur[j];
      int need = n_res + ntr - cap, ne = 0;
      if (need > 0) {
        int nc = 0;
        for (int64_t j = 0; j < NB; ++j)
          if (resident[j] && !in_prev[j] && !in_cur[j]) {
            ev[nc].s = -(double)last[j]; /* larger -last = older; ties by index */
            ev[nc].i = (int32_t)j;
            ++nc;
          }
        qsort(ev, (size_t)nc, sizeof *ev, by_score_then_index);
        if (nc < need) perr = -4;
        for (int j = 0; j < need && j < nc; ++j) {
          resident[ev[j].i] = 0;
          if (evicted) evicted[o * cap + ne] = ev[j].i;
          ++ne;
        }
        n_res -= ne;
      }
      for (int j = 0; j < ntr; ++j) resident[Tt[j]] = 1;
      n_res += ntr;
      for (int j = 0; j < kb; ++j) last[cur[j]] = t;
      memcpy(M + o * kb, cur, (size_t)kb * sizeof *cur);
      nT[o] = ntr;
      nevict[o] = ne;
      int32_t *sw = prev;
      prev = cur;
      cur = sw;
    }
    if (perr < err) err = perr;
    free(gmx);
    free(gmn);
    free(Sbuf);
    free(prev);
    free(cur);
    free(tok);
    free(resident);
    free(in_prev);
    free(in_cur);
    free(last);
    free(ev);
  }
  return err;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

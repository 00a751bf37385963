/*
 * fp64 CPU oracle for paged Top-K decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * HIP path is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the library never does.  It
 * shares no code, header, table or helper with the HIP path.
 *
 * Every quantity is computed in double precision from exact float64 copies of
 * the (fp32 / fp16 / bf16) inputs, with plain loops in the order the
 * definitions state them.  OpenMP only splits independent rows
 * (a sequence, a head, a page) across threads; it never changes the order of
 * a sum.
 *
 * Sources (cited by page and section):
 *  - KVDrive paper (Chinese translation page), §2.2 "Sparse attention": Quest
 *    cuts the keys into blocks, estimates a block's importance by multiplying
 *    the query with the channel-wise minimum and maximum of its keys, and
 *    keeps only the Top-K blocks for each query.
 *  - KVDrive, §2.3 "KV cache offloading": spatial chunking uses min/max/mean
 *    keys of adjacent tokens as block representatives; a decode step selects
 *    critical entries through a GPU-resident index, fetches them, and runs
 *    sparse attention over them.
 *  - KVDrive, §4 "System overview": the index is built at prefill.
 *  - Dual-Blade page, "Background and key observations": every decode step
 *    loads all previous K/V pairs to compute the current token's attention.
 *  - DirectKV review page, "Core method" 3: the fused decode kernel computes
 *    scores and a streaming softmax in one pass over the KV.
 *
 * Readings where the pages are silent (also listed in the design notes):
 *  - block score  sigma = sum_c max(q_c*kmin_c, q_c*kmax_c), unscaled;
 *  - GQA: one selection per (sequence, KV head); its score is the max of the
 *    per-query-head scores of that group; query head h uses KV head h / G;
 *  - K_eff = min(K, N_b); ties go to the lower block index; the selected list
 *    is emitted in ascending block order;
 *  - attention logit z_t = scale * (q . k_t), softmax over the token set;
 *  - split s of a list of n blocks covers list positions
 *    [s*c, min((s+1)*c, n)) with c = ceil(n / S); an empty split has
 *    m = -inf, l = 0, o = 0;
 *  - mean-key index (KVDrive §2.3 spatial blocking, §4 overview: a page's
 *    average key as its representative): kmean = average of the valid keys,
 *    block score q . kmean, then the same group max and Top-K;
 *  - forced tokens (KVDrive §9.1 setup: the sparse systems always keep the
 *    first tokens and the most recent tokens): every block holding one of the
 *    first `sink` or the last `local` tokens of a sequence is selected and
 *    counts against the budget K; the other K_eff - |forced| places go to the
 *    best of the remaining blocks;
 *  - quantised cold pages (KVDrive §11 future work: cold blocks stored with
 *    aggressive quantisation, hot blocks in high precision; DirectKV review,
 *    "Assumption stress test": FP8/INT4 KV): K and V pages as FP8 E4M3 codes
 *    (the OCP 8-bit floating-point format: bias 7, 3 mantissa bits, no
 *    infinities, largest finite value 448) with one fp32 scale per (page, KV
 *    head) and tensor: s = amax / 448 over the valid slots (1 for an all-zero
 *    tile), code = round-to-nearest-even(x / s) saturated to +-448, code 0 for
 *    slots past the valid count; the value a code stands for is
 *    decode(code) * s.  The scale and the quotient are taken in fp32, the
 *    precision in which the quantiser decides the codes;
 *  - INT4 cold pages (the same passages name INT4; they fix no format, so the
 *    reading is the plain symmetric one): per (page, KV head) and tensor
 *    s = amax / 7 over the valid slots (1 for an all-zero tile), code n =
 *    round-half-even(x / s) clamped to [-7, 7], code 0 past the valid count;
 *    the value a code stands for is n * s.  Scale and quotient in fp32, as for
 *    FP8.  A code is stored as a 4-bit two's complement nibble, two per byte,
 *    the even channel in the low nibble;
 *  - GPU-resident block cache with lookahead eviction (KVDrive §5.1: a window
 *    of critical KV entries stays on the GPU; each step the new critical
 *    entries are fetched from host memory and the entries with the lowest
 *    attention in the step are the ones dropped): per (sequence, KV head) a
 *    cache of C >= K block slots.  A step's selected blocks that are resident
 *    keep their slots; for m missing blocks the reused slots are the first m
 *    of: the free slots in slot order, then the slots whose block is not
 *    selected, by increasing attention mass of the latest step (ties: lower
 *    slot first); the missing blocks, in list order, take the reused slots in
 *    increasing slot order.  The mass of a slot is the attention weight its block
 *    received in the latest step, summed over the block's tokens, max over
 *    the query heads of the group; 0 for a block the step did not attend;
 *  - tier plan (the tiered-offload blog, "page replacement": pages move to a
 *    slower tier when cold, and a hysteresis cooldown keeps a page just moved
 *    down from coming straight back; KVDrive §11: hot blocks keep high
 *    precision, cold blocks are quantised): each page in use has a heat
 *    h <- decay * h + (1 - decay) * hit, where hit = 1 when any KV head of its
 *    sequence selected its block in the step; a hot page that does not hold
 *    one of the sequence's last `recent` tokens turns cold when h < cold_below;
 *    a cold page turns hot when it holds a recent token, or when h > hot_above
 *    and at least `cooldown` steps have passed since it turned cold.  Heat is
 *    kept and compared in fp32, the precision in which the kernel decides.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static i64 ceil_div(i64 a, i64 b) { return (a + b - 1) / b; }

/* Element (page p, KV head j, slot s, channel c) of a [P, Hkv, bs, D] pool. */
static const double* pool_row(const double* pool, i64 p, i64 j, i64 s, int Hkv, int bs, int D) {
  return pool + (((p * Hkv + j) * bs + s) * (i64)D);
}

/*
 * O1 block meta (KVDrive §2.2 / §2.3: channel-wise min and max key of a block).
 * kmeta layout [P, Hkv, 2, D]; index 0 = min, 1 = max; only the listed pages
 * are written, over their first valid_tokens[i] slots.
 */
void oracle_block_meta(const double* k_pool, int Hkv, int bs, int D,
                       const int32_t* page_ids, const int32_t* valid_tokens, int n_ids,
                       double* kmeta) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_ids; ++i) {
    const i64 p = page_ids[i];
    const int nv = valid_tokens[i];
    for (int j = 0; j < Hkv; ++j) {
      double* mn = kmeta + ((p * Hkv + j) * 2 + 0) * (i64)D;
      double* mx = kmeta + ((p * Hkv + j) * 2 + 1) * (i64)D;
      for (int c = 0; c < D; ++c) {
        double lo = INFINITY, hi = -INFINITY;
        for (int s = 0; s < nv; ++s) {
          const double x = pool_row(k_pool, p, j, s, Hkv, bs, D)[c];
          if (x < lo) lo = x;
          if (x > hi) hi = x;
        }
        mn[c] = lo;
        mx[c] = hi;
      }
    }
  }
}

/*
 * O2 per-query-head Quest score of every logical block (KVDrive §2.2):
 *   sigma[b,h,n] = sum_c max(q[b,h,c]*kmin[p,j,c], q[b,h,c]*kmax[p,j,c])
 * with p = block_table[b,n] and j = h / G.  -inf for n >= N_b.
 */
void oracle_head_scores(const double* q, const double* kmeta, const int32_t* block_table,
                        const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int bs, int maxN,
                        double* head_scores) {
  const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const i64 nb = ceil_div(seq_lens[b], bs);
      const int j = h / G;
      const double* qh = q + ((i64)b * Hq + h) * D;
      double* out = head_scores + ((i64)b * Hq + h) * maxN;
      for (i64 n = 0; n < maxN; ++n) {
        if (n >= nb) { out[n] = -INFINITY; continue; }
        const i64 p = block_table[(i64)b * maxN + n];
        const double* mn = kmeta + ((p * Hkv + j) * 2 + 0) * (i64)D;
        const double* mx = kmeta + ((p * Hkv + j) * 2 + 1) * (i64)D;
        double acc = 0.0;
        for (int c = 0; c < D; ++c) {
          const double a = qh[c] * mn[c];
          const double e = qh[c] * mx[c];
          acc += (a > e) ? a : e;
        }
        out[n] = acc;
      }
    }
  }
}

/*
 * Mean-key representative (KVDrive §2.3, §4): kmean[p, j, c] is the average of
 * K[p, j, s, c] over the first valid_tokens[i] slots of each listed page.
 * kmean layout [P, Hkv, D].
 */
void oracle_block_mean(const double* k_pool, int Hkv, int bs, int D,
                       const int32_t* page_ids, const int32_t* valid_tokens, int n_ids,
                       double* kmean) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_ids; ++i) {
    const i64 p = page_ids[i];
    const int nv = valid_tokens[i];
    for (int j = 0; j < Hkv; ++j) {
      double* out = kmean + (p * Hkv + j) * (i64)D;
      for (int c = 0; c < D; ++c) {
        double sum = 0.0;
        for (int s = 0; s < nv; ++s) sum += pool_row(k_pool, p, j, s, Hkv, bs, D)[c];
        out[c] = sum / nv;
      }
    }
  }
}

/*
 * Per-query-head score against the mean-key index: sigma[b,h,n] = q[b,h] . kmean[p,j]
 * with p = block_table[b,n], j = h / G; -inf for n >= N_b.
 */
void oracle_head_scores_mean(const double* q, const double* kmean, const int32_t* block_table,
                             const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int bs,
                             int maxN, double* head_scores) {
  const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const i64 nb = ceil_div(seq_lens[b], bs);
      const int j = h / G;
      const double* qh = q + ((i64)b * Hq + h) * D;
      double* out = head_scores + ((i64)b * Hq + h) * maxN;
      for (i64 n = 0; n < maxN; ++n) {
        if (n >= nb) { out[n] = -INFINITY; continue; }
        const i64 p = block_table[(i64)b * maxN + n];
        const double* km = kmean + (p * Hkv + j) * (i64)D;
        double acc = 0.0;
        for (int c = 0; c < D; ++c) acc += qh[c] * km[c];
        out[n] = acc;
      }
    }
  }
}

/*
 * O3 group score: Sigma[b,j,n] = max over the G query heads h with h / G == j
 * of sigma[b,h,n].
 */
void oracle_group_scores(const double* head_scores, int B, int Hq, int Hkv, int maxN,
                         double* group_scores) {
  const int G = Hq / Hkv;
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < Hkv; ++j)
      for (i64 n = 0; n < maxN; ++n) {
        double best = -INFINITY;
        for (int g = 0; g < G; ++g) {
          const double s = head_scores[((i64)b * Hq + j * G + g) * maxN + n];
          if (s > best) best = s;
        }
        group_scores[((i64)b * Hkv + j) * maxN + n] = best;
      }
}

/*
 * O4 Top-K selection by rank count (KVDrive §2.2: keep the Top-K blocks):
 * block n < N_b is selected iff
 *   #{ m < N_b : S_m > S_n  or  (S_m == S_n and m < n) }  <  K_eff,
 * K_eff = min(K, N_b).  The selected blocks are written in ascending order,
 * the rest of the row is -1.
 */
void oracle_topk(const double* group_scores, const int32_t* seq_lens, int B, int Hkv, int maxN,
                 int bs, int K, int32_t* sel, int32_t* sel_count) {
  /* rank[b, j, n]: the number of blocks that come before block n; every
     block's count is independent, so the counts are spread over the threads
     by block (a 1M-token row alone has 65536 of them) */
  const i64 rows = (i64)B * Hkv;
  i64* ranks = (i64*)malloc((size_t)(rows * maxN > 0 ? rows * maxN : 1) * sizeof(i64));
#pragma omp parallel for schedule(dynamic, 64)
  for (i64 t = 0; t < rows * maxN; ++t) {
    const i64 u = t / maxN, n = t % maxN;
    const i64 nb = ceil_div(seq_lens[u / Hkv], bs);
    const double* s = group_scores + u * maxN;
    i64 rank = 0;
    if (n < nb)
      for (i64 m = 0; m < nb; ++m)
        if (s[m] > s[n] || (s[m] == s[n] && m < n)) ++rank;
    ranks[t] = rank;
  }
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < Hkv; ++j) {
      const i64 nb = ceil_div(seq_lens[b], bs);
      const i64 keff = (K < nb) ? K : nb;
      int32_t* out = sel + ((i64)b * Hkv + j) * K;
      i64 w = 0;
      for (i64 n = 0; n < nb; ++n) {
        const i64 rank = ranks[((i64)b * Hkv + j) * maxN + n];
        if (rank < keff) out[w++] = (int32_t)n;
      }
      for (i64 r = w; r < K; ++r) out[r] = -1;
      sel_count[(i64)b * Hkv + j] = (int32_t)w;
    }
  }
  free(ranks);
}

/*
 * Selection with forced tokens (KVDrive §9.1).  Block n < N_b covers tokens
 * [n*bs, min((n+1)*bs, L)); it is forced when it holds one of the first `sink`
 * tokens (n*bs < sink) or one of the last `local` tokens (local > 0 and
 * (n+1)*bs > L - local).  All forced blocks are selected; of the other blocks,
 * those whose rank among the non-forced blocks (score descending, lower index
 * first on ties) is below K_eff - #forced are selected too, K_eff = min(K, N_b).
 * Output ascending, -1 padded.  The caller keeps #forced <= K.  With
 * sink = local = 0 this is oracle_topk.
 */
static int is_forced(i64 n, i64 L, int bs, int sink, int local) {
  return n * bs < sink || (local > 0 && (n + 1) * bs > L - local);
}

void oracle_select(const double* group_scores, const int32_t* seq_lens, int B, int Hkv, int maxN,
                   int bs, int K, int sink, int local, int32_t* sel, int32_t* sel_count) {
  /* rank[b, j, n] of every block that is not forced, among the blocks that
     are not forced; counted in parallel by block as in oracle_topk */
  const i64 rows = (i64)B * Hkv;
  i64* ranks = (i64*)malloc((size_t)(rows * maxN > 0 ? rows * maxN : 1) * sizeof(i64));
#pragma omp parallel for schedule(dynamic, 64)
  for (i64 t = 0; t < rows * maxN; ++t) {
    const i64 u = t / maxN, n = t % maxN;
    const i64 L = seq_lens[u / Hkv];
    const i64 nb = ceil_div(L, bs);
    const double* s = group_scores + u * maxN;
    i64 rank = 0;
    if (n < nb && !is_forced(n, L, bs, sink, local)) {
      for (i64 m = 0; m < nb; ++m) {
        if (is_forced(m, L, bs, sink, local)) continue;
        if (s[m] > s[n] || (s[m] == s[n] && m < n)) ++rank;
      }
    }
    ranks[t] = rank;
  }
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < Hkv; ++j) {
      const i64 L = seq_lens[b];
      const i64 nb = ceil_div(L, bs);
      const i64 keff = (K < nb) ? K : nb;
      int32_t* out = sel + ((i64)b * Hkv + j) * K;
      i64 n_forced = 0;
      for (i64 n = 0; n < nb; ++n) n_forced += is_forced(n, L, bs, sink, local);
      const i64 free_slots = keff - n_forced;
      i64 w = 0;
      for (i64 n = 0; n < nb; ++n) {
        int take;
        if (is_forced(n, L, bs, sink, local)) {
          take = 1;
        } else {
          const i64 rank = ranks[((i64)b * Hkv + j) * maxN + n];
          take = rank < free_slots;
        }
        if (take) out[w++] = (int32_t)n;
      }
      for (i64 r = w; r < K; ++r) out[r] = -1;
      sel_count[(i64)b * Hkv + j] = (int32_t)w;
    }
  }
  free(ranks);
}

/*
 * FP8 E4M3 (OCP 8-bit floating point, E4M3 variant).  A code is s eeee mmm:
 * e = 0 encodes the subnormals m * 2^-9, e = 1..15 the normals
 * (1 + m/8) * 2^(e - 7); s eeee mmm = s 1111 111 is NaN (never produced here),
 * so the largest finite magnitude is 1.75 * 2^8 = 448.
 */
double oracle_fp8_decode(uint8_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return (code & 0x80) ? -mag : mag;
}

/*
 * Encode an fp32 value: round to the nearest E4M3 value, ties to the even
 * code (even mantissa), magnitudes that round past 448 saturate to 448.  The
 * representable magnitudes of exponent ex are multiples of 2^(ex - 3) for
 * 2^ex <= |y| < 2^(ex+1), ex >= -6; below 2^-6 they are multiples of 2^-9.
 */
uint8_t oracle_fp8_encode(float y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0x00;
  const double a = fabs((double)y);
  if (isnan(a)) return (uint8_t)(sign | 0x7F);
  int e2;
  frexp(a, &e2);                       /* a = f * 2^e2, f in [0.5, 1) */
  int ex = (a == 0.0) ? -6 : e2 - 1;   /* floor(log2 a) */
  if (ex < -6) ex = -6;
  const double step = ldexp(1.0, ex - 3);
  double r = nearbyint(a / step) * step; /* exact: a / step is a power-of-two scaling */
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return sign;
  frexp(r, &e2);
  int er = e2 - 1;
  if (er < -6) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));   /* subnormal */
  const int m = (int)((r / ldexp(1.0, er) - 1.0) * 8.0);
  return (uint8_t)(sign | ((er + 7) << 3) | m);
}

/*
 * Quantise the listed pages of one pool (K or V): for i < n_ids and KV head j,
 * p = page_ids[i], v = valid_tokens[i]:
 *   amax = max_{s < v, c} |X[p, j, s, c]|  (fp32 values of the stored dtype)
 *   scale[p, j] = amax / 448 in fp32, or 1 when amax == 0
 *   code[p, j, s, c] = encode(X / scale in fp32) for s < v, 0 for s >= v.
 * codes: uint8 [P, Hkv, bs, D]; scales: float [P, Hkv] (strided by
 * scale_stride floats, so K and V scales can interleave).
 */
void oracle_fp8_quantize(const double* pool, int Hkv, int bs, int D, const int32_t* page_ids,
                         const int32_t* valid_tokens, int n_ids, uint8_t* codes, float* scales,
                         int scale_stride) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_ids; ++i) {
    const i64 p = page_ids[i];
    const int nv = valid_tokens[i];
    for (int j = 0; j < Hkv; ++j) {
      float amax = 0.0f;
      for (int s = 0; s < nv; ++s) {
        const double* row = pool_row(pool, p, j, s, Hkv, bs, D);
        for (int c = 0; c < D; ++c) {
          const float x = fabsf((float)row[c]);
          if (x > amax) amax = x;
        }
      }
      const float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
      scales[(p * Hkv + j) * (i64)scale_stride] = sc;
      for (int s = 0; s < bs; ++s) {
        uint8_t* out = codes + ((p * Hkv + j) * bs + s) * (i64)D;
        if (s >= nv) {
          memset(out, 0, (size_t)D);
          continue;
        }
        const double* row = pool_row(pool, p, j, s, Hkv, bs, D);
        for (int c = 0; c < D; ++c) out[c] = oracle_fp8_encode((float)row[c] / sc);
      }
    }
  }
}

/*
 * INT4 (symmetric, one scale per tile).  Quantise the listed pages of one pool
 * (K or V): for i < n_ids and KV head j, p = page_ids[i], v = valid_tokens[i]:
 *   amax = max_{s < v, c} |X[p, j, s, c]|  (fp32 values of the stored dtype)
 *   scale[p, j] = amax / 7 in fp32, or 1 when amax == 0
 *   n = round-half-even(X / scale in fp32), clamped to [-7, 7], for s < v;
 *   n = 0 for s >= v.
 * codes: uint8 [P, Hkv, bs, D/2], byte c/2 of a row holding channel c (even c)
 * in bits 0..3 and channel c+1 in bits 4..7, each as two's complement.
 */
int oracle_int4_code(float y) {
  double r = nearbyint((double)y);     /* y is an fp32 value: exact in double */
  if (r > 7.0) r = 7.0;
  if (r < -7.0) r = -7.0;
  return (int)r;
}

void oracle_int4_quantize(const double* pool, int Hkv, int bs, int D, const int32_t* page_ids,
                          const int32_t* valid_tokens, int n_ids, uint8_t* codes, float* scales,
                          int scale_stride) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_ids; ++i) {
    const i64 p = page_ids[i];
    const int nv = valid_tokens[i];
    for (int j = 0; j < Hkv; ++j) {
      float amax = 0.0f;
      for (int s = 0; s < nv; ++s) {
        const double* row = pool_row(pool, p, j, s, Hkv, bs, D);
        for (int c = 0; c < D; ++c) {
          const float x = fabsf((float)row[c]);
          if (x > amax) amax = x;
        }
      }
      const float sc = (amax > 0.0f) ? amax / 7.0f : 1.0f;
      scales[(p * Hkv + j) * (i64)scale_stride] = sc;
      for (int s = 0; s < bs; ++s) {
        uint8_t* out = codes + ((p * Hkv + j) * bs + s) * (i64)(D / 2);
        memset(out, 0, (size_t)(D / 2));
        if (s >= nv) continue;
        const double* row = pool_row(pool, p, j, s, Hkv, bs, D);
        for (int c = 0; c < D; ++c) {
          const int n = oracle_int4_code((float)row[c] / sc);
          out[c / 2] |= (uint8_t)((n & 15) << (4 * (c & 1)));
        }
      }
    }
  }
}

/* The code of channel c in a packed row: the nibble, sign-extended. */
int oracle_int4_unpack(const uint8_t* row, int c) {
  const int nib = (row[c / 2] >> (4 * (c & 1))) & 15;
  return nib >= 8 ? nib - 16 : nib;
}

/*
 * The logical block list of (b, kv head j): all blocks 0..N_b-1 when sel is
 * NULL (dense decode, Dual-Blade background), else the selected list.
 */
static i64 block_list(const int32_t* sel, int sel_stride, int b, int j, int Hkv, i64 pos) {
  if (!sel) return pos;
  return sel[((i64)b * Hkv + j) * sel_stride + pos];
}

static i64 list_len(const int32_t* sel_count, int b, int j, int Hkv, i64 nb) {
  return sel_count ? sel_count[(i64)b * Hkv + j] : nb;
}

/*
 * Softmax attention of query (b, h) over the tokens of list positions
 * [pos0, pos1): z_t = scale * (q . k_t); m = max z; l = sum exp(z - m);
 * o = sum exp(z - m) v_t / l.  Token t of logical block n lives at page
 * block_table[b, n], slot t - n*bs, and only t < L_b count.
 * Writes o[D] and returns (m, l) through the pointers.  An empty range gives
 * m = -inf, l = 0, o = 0.
 */
static void attend_range(const double* q, const double* k_pool, const double* v_pool,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* sel, int sel_stride,
                         int Hq, int Hkv, int D, int bs, int maxN, double scale,
                         int b, int h, i64 pos0, i64 pos1,
                         double* z_buf, double* o, double* m_out, double* l_out) {
  const int G = Hq / Hkv;
  const int j = h / G;
  const i64 L = seq_lens[b];
  const double* qh = q + ((i64)b * Hq + h) * D;

  /* pass 1: logits of every token in the range */
  i64 nt = 0;
  double m = -INFINITY;
  for (i64 pos = pos0; pos < pos1; ++pos) {
    const i64 n = block_list(sel, sel_stride, b, j, Hkv, pos);
    const i64 p = block_table[(i64)b * maxN + n];
    for (int s = 0; s < bs; ++s) {
      const i64 t = n * bs + s;
      if (t >= L) break;
      const double* k = pool_row(k_pool, p, j, s, Hkv, bs, D);
      double dot = 0.0;
      for (int c = 0; c < D; ++c) dot += qh[c] * k[c];
      const double z = scale * dot;
      z_buf[nt++] = z;
      if (z > m) m = z;
    }
  }
  for (int c = 0; c < D; ++c) o[c] = 0.0;
  if (nt == 0) { *m_out = -INFINITY; *l_out = 0.0; return; }

  /* pass 2: l = sum exp(z - m), o = sum exp(z - m) v */
  double l = 0.0;
  i64 it = 0;
  for (i64 pos = pos0; pos < pos1; ++pos) {
    const i64 n = block_list(sel, sel_stride, b, j, Hkv, pos);
    const i64 p = block_table[(i64)b * maxN + n];
    for (int s = 0; s < bs; ++s) {
      const i64 t = n * bs + s;
      if (t >= L) break;
      const double e = exp(z_buf[it++] - m);
      const double* v = pool_row(v_pool, p, j, s, Hkv, bs, D);
      l += e;
      for (int c = 0; c < D; ++c) o[c] += e * v[c];
    }
  }
  for (int c = 0; c < D; ++c) o[c] /= l;
  *m_out = m;
  *l_out = l;
}

/*
 * O5 decode attention for every (b, h): dense over t < L_b when sel is NULL,
 * else over the tokens of the selected blocks of (b, h / G).
 * out [B, Hq, D]; lse [B, Hq] = m + ln l (may be NULL).
 */
void oracle_attention(const double* q, const double* k_pool, const double* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* sel, const int32_t* sel_count, int sel_stride,
                      int B, int Hq, int Hkv, int D, int bs, int maxN, double scale,
                      double* out, double* lse) {
  const int G = Hq / Hkv;
#pragma omp parallel
  {
    i64 maxL = 0;
    for (int b = 0; b < B; ++b) if (seq_lens[b] > maxL) maxL = seq_lens[b];
    double* z_buf = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
#pragma omp for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
      for (int h = 0; h < Hq; ++h) {
        const i64 nb = ceil_div(seq_lens[b], bs);
        const i64 n_list = list_len(sel_count, b, h / G, Hkv, nb);
        double m, l;
        double* o = out + ((i64)b * Hq + h) * D;
        attend_range(q, k_pool, v_pool, block_table, seq_lens, sel, sel_stride,
                     Hq, Hkv, D, bs, maxN, scale, b, h, 0, n_list, z_buf, o, &m, &l);
        if (lse) lse[(i64)b * Hq + h] = m + log(l);
      }
    }
    free(z_buf);
  }
}

/*
 * Block log-sum-exp of the attended list: for (b, h) and list position pos
 * (block n of the list of (b, h / G)),
 *   block_lse[b, h, pos] = ln sum_{t in block n, t < L_b} exp(scale * (q . k_t)),
 * so that exp(block_lse - lse) is the attention weight the block receives in
 * the step (KVDrive §5.1 ranks cached entries by it).  Positions past the list
 * are -inf.  block_lse [B, Hq, sel_stride] (dense: sel == NULL, stride maxN).
 */
void oracle_block_lse(const double* q, const double* k_pool, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* sel, const int32_t* sel_count,
                      int sel_stride, int B, int Hq, int Hkv, int D, int bs, int maxN,
                      double scale, double* block_lse) {
  const int G = Hq / Hkv;
  const int stride = sel ? sel_stride : maxN;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const int j = h / G;
      const i64 L = seq_lens[b];
      const i64 nb = ceil_div(L, bs);
      const i64 n_list = list_len(sel_count, b, j, Hkv, nb);
      const double* qh = q + ((i64)b * Hq + h) * D;
      double* out = block_lse + ((i64)b * Hq + h) * stride;
      for (i64 pos = 0; pos < stride; ++pos) {
        if (pos >= n_list) { out[pos] = -INFINITY; continue; }
        const i64 n = block_list(sel, sel_stride, b, j, Hkv, pos);
        const i64 p = block_table[(i64)b * maxN + n];
        double z[64];
        int nt = 0;
        double m = -INFINITY;
        for (int s = 0; s < bs && n * bs + s < L; ++s) {
          const double* k = pool_row(k_pool, p, j, s, Hkv, bs, D);
          double dot = 0.0;
          for (int c = 0; c < D; ++c) dot += qh[c] * k[c];
          z[nt] = scale * dot;
          if (z[nt] > m) m = z[nt];
          ++nt;
        }
        double l = 0.0;
        for (int t = 0; t < nt; ++t) l += exp(z[t] - m);
        out[pos] = m + log(l);
      }
    }
  }
}

/*
 * Eviction mass of every cache slot after a step (KVDrive §5.1): slot_mass is
 * set to 0 everywhere, then for each list position pos of (b, j) whose block
 * sits in slot sel_slots[b, j, pos]:
 *   slot_mass[b, j, slot] = max over the G query heads h of group j of
 *                           exp(block_lse[b, h, pos] - lse[b, h]).
 * block_lse [B, Hq, sel_stride]; lse [B, Hq]; slot_mass [B, Hkv, C].
 */
void oracle_slot_mass(const double* block_lse, const double* lse, const int32_t* sel_count,
                      const int32_t* sel_slots, int sel_stride, int B, int Hq, int Hkv, int C,
                      double* slot_mass) {
  const int G = Hq / Hkv;
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < Hkv; ++j) {
      double* out = slot_mass + ((i64)b * Hkv + j) * C;
      for (int c = 0; c < C; ++c) out[c] = 0.0;
      const i64 cnt = sel_count[(i64)b * Hkv + j];
      for (i64 pos = 0; pos < cnt; ++pos) {
        double best = 0.0;
        for (int g = 0; g < G; ++g) {
          const i64 h = (i64)j * G + g;
          const double w = exp(block_lse[((i64)b * Hq + h) * sel_stride + pos] - lse[(i64)b * Hq + h]);
          if (w > best) best = w;
        }
        out[sel_slots[((i64)b * Hkv + j) * sel_stride + pos]] = best;
      }
    }
  }
}

/*
 * One step of the block cache (KVDrive §5.1) for every (b, j).  In and out:
 * slot_block [B, Hkv, C] (block held by each slot, -1 free) and block_slot
 * [B, Hkv, maxN] (slot of each resident block, -1 otherwise).  In: the step's
 * list sel / sel_count (distinct blocks), slot_mass [B, Hkv, C] of the latest
 * step (compared as fp32, the precision the cache keeps it in).  Out:
 * sel_slots [B, Hkv, sel_stride] (slot of every list position, -1 past the
 * list), the fetch list fetch_block / fetch_slot [B, Hkv, sel_stride] of the
 * blocks that were not resident (-1 padded) and fetch_count [B, Hkv].
 * Requires C >= sel_count.
 */
void oracle_cache_plan(const int32_t* sel, const int32_t* sel_count, int sel_stride, int B,
                       int Hkv, int maxN, int C, int32_t* slot_block, int32_t* block_slot,
                       const float* slot_mass, int32_t* sel_slots, int32_t* fetch_block,
                       int32_t* fetch_slot, int32_t* fetch_count) {
  int* in_use = (int*)malloc(sizeof(int) * (size_t)C);
  int* cand = (int*)malloc(sizeof(int) * (size_t)C);
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < Hkv; ++j) {
      const i64 u = (i64)b * Hkv + j;
      int32_t* sb = slot_block + u * C;
      int32_t* bsl = block_slot + u * maxN;
      const float* mass = slot_mass + u * C;
      const int32_t* list = sel + u * sel_stride;
      int32_t* out_slots = sel_slots + u * sel_stride;
      int32_t* fb = fetch_block + u * sel_stride;
      int32_t* fs = fetch_slot + u * sel_stride;
      const int cnt = sel_count[u];
      for (int c = 0; c < C; ++c) in_use[c] = 0;
      for (int pos = 0; pos < sel_stride; ++pos) { out_slots[pos] = -1; fb[pos] = -1; fs[pos] = -1; }
      /* hits keep their slots */
      for (int pos = 0; pos < cnt; ++pos) {
        const int s = bsl[list[pos]];
        if (s >= 0) { out_slots[pos] = s; in_use[s] = 1; }
      }
      /* reuse order: free slots by index, then unselected resident blocks by
       * (mass, slot) -- a selection sort keeps the rule plain */
      int nc = 0;
      for (int c = 0; c < C; ++c) if (sb[c] < 0) cand[nc++] = c;
      const int n_free = nc;
      for (int c = 0; c < C; ++c) if (sb[c] >= 0 && !in_use[c]) cand[nc++] = c;
      for (int a = n_free; a < nc; ++a) {
        int best = a;
        for (int k = a + 1; k < nc; ++k) {
          const int ck = cand[k], cb = cand[best];
          if (mass[ck] < mass[cb] || (mass[ck] == mass[cb] && ck < cb)) best = k;
        }
        const int t = cand[a]; cand[a] = cand[best]; cand[best] = t;
      }
      /* the first m candidates are reused; misses take them in slot order */
      int m = 0;
      for (int pos = 0; pos < cnt; ++pos) if (out_slots[pos] < 0) ++m;
      for (int a = 0; a < m; ++a) {
        int lo = a;
        for (int k = a + 1; k < m; ++k) if (cand[k] < cand[lo]) lo = k;
        const int t = cand[a]; cand[a] = cand[lo]; cand[lo] = t;
      }
      int nf = 0;
      for (int pos = 0; pos < cnt; ++pos) {
        if (out_slots[pos] >= 0) continue;
        const int s = cand[nf];
        if (sb[s] >= 0) bsl[sb[s]] = -1;
        sb[s] = list[pos];
        bsl[list[pos]] = s;
        out_slots[pos] = s;
        fb[nf] = list[pos];
        fs[nf] = s;
        ++nf;
      }
      fetch_count[u] = nf;
    }
  }
  free(in_use);
  free(cand);
}

/*
 * Tier plan: one decode step's update of every page in use (see the reading
 * above).  Page p = block_table[b, n], n < N_b, is hit when block n is in
 * sel[b, j, 0..sel_count[b, j]) for some KV head j (row stride sel_stride),
 * and recent when it holds one of the last `recent` tokens of sequence b.
 * heat [P] (fp32), tier [P] (0 hot, 1 cold) and stamp [P] (the step at which
 * the page last turned cold) are updated in place; pages no sequence
 * references keep their state; each page is referenced by at most one
 * (sequence, block).  demote / promote [B, maxN] receive, per sequence and in
 * block order, the pages that turned cold / hot (-1 after the last), and
 * demote_count / promote_count [B] their numbers.
 */
void oracle_tier_plan(const int32_t* sel, const int32_t* sel_count, int sel_stride,
                      const int32_t* block_table, const int32_t* seq_lens, int B, int Hkv,
                      int maxN, int bs, float decay, float hot_above, float cold_below,
                      int recent, int cooldown, int step, float* heat, uint8_t* tier,
                      int32_t* stamp, int32_t* demote, int32_t* demote_count, int32_t* promote,
                      int32_t* promote_count) {
  for (int b = 0; b < B; ++b) {
    const i64 L = seq_lens[b];
    const i64 N = ceil_div(L, bs);
    int32_t* dem = demote + (i64)b * maxN;
    int32_t* pro = promote + (i64)b * maxN;
    for (int n = 0; n < maxN; ++n) { dem[n] = -1; pro[n] = -1; }
    int nd = 0, np = 0;
    for (i64 n = 0; n < N; ++n) {
      int hit = 0;
      for (int j = 0; j < Hkv && !hit; ++j) {
        const i64 u = (i64)b * Hkv + j;
        for (int pos = 0; pos < sel_count[u]; ++pos)
          if (sel[u * sel_stride + pos] == n) { hit = 1; break; }
      }
      /* the block holds tokens n*bs .. n*bs + bs - 1; the recent ones are L - recent .. L - 1 */
      const int is_recent = recent > 0 && n * bs + bs - 1 >= L - recent;
      const i64 p = block_table[(i64)b * maxN + n];
      const float h = hit ? fmaf(decay, heat[p], 1.0f - decay) : decay * heat[p];
      heat[p] = h;
      if (tier[p] == 0) {
        if (!is_recent && h < cold_below) {
          tier[p] = 1;
          stamp[p] = step;
          dem[nd++] = (int32_t)p;
        }
      } else if (is_recent || (h > hot_above && (i64)step - stamp[p] >= cooldown)) {
        tier[p] = 0;
        pro[np++] = (int32_t)p;
      }
    }
    demote_count[b] = nd;
    promote_count[b] = np;
  }
}

/*
 * O6 split partials: O5 restricted to each contiguous chunk of the block list.
 * part_o [B, Hq, S, D] (normalised per split), part_m / part_l [B, Hq, S].
 */
void oracle_attention_splits(const double* q, const double* k_pool, const double* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel, const int32_t* sel_count, int sel_stride,
                             int B, int Hq, int Hkv, int D, int bs, int maxN, double scale,
                             int num_splits, double* part_o, double* part_m, double* part_l) {
  const int G = Hq / Hkv;
  const int S = num_splits;
#pragma omp parallel
  {
    i64 maxL = 0;
    for (int b = 0; b < B; ++b) if (seq_lens[b] > maxL) maxL = seq_lens[b];
    double* z_buf = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
#pragma omp for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
      for (int h = 0; h < Hq; ++h) {
        const i64 nb = ceil_div(seq_lens[b], bs);
        const i64 n_list = list_len(sel_count, b, h / G, Hkv, nb);
        const i64 chunk = ceil_div(n_list, S);
        for (int s = 0; s < S; ++s) {
          i64 p0 = (i64)s * chunk, p1 = p0 + chunk;
          if (p0 > n_list) p0 = n_list;
          if (p1 > n_list) p1 = n_list;
          const i64 row = ((i64)b * Hq + h) * S + s;
          attend_range(q, k_pool, v_pool, block_table, seq_lens, sel, sel_stride,
                       Hq, Hkv, D, bs, maxN, scale, b, h, p0, p1, z_buf,
                       part_o + row * D, part_m + row, part_l + row);
        }
      }
    }
    free(z_buf);
  }
}

/*
 * Log-sum-exp merge of split partials:
 *   M = max_s m_s;  w_s = l_s * exp(m_s - M)  (0 for an empty split);
 *   out = sum_s w_s o_s / sum_s w_s;  lse = M + ln(sum_s w_s).
 */
void oracle_combine(int B, int Hq, int D, int num_splits, const double* part_o,
                    const double* part_m, const double* part_l, double* out, double* lse) {
  const int S = num_splits;
  for (i64 r = 0; r < (i64)B * Hq; ++r) {
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (part_m[r * S + s] > M) M = part_m[r * S + s];
    double wsum = 0.0;
    double* o = out + r * D;
    for (int c = 0; c < D; ++c) o[c] = 0.0;
    for (int s = 0; s < S; ++s) {
      const double ms = part_m[r * S + s];
      if (ms == -INFINITY) continue;
      const double w = part_l[r * S + s] * exp(ms - M);
      wsum += w;
      for (int c = 0; c < D; ++c) o[c] += w * part_o[(r * S + s) * D + c];
    }
    for (int c = 0; c < D; ++c) o[c] /= wsum;
    if (lse) lse[r] = M + log(wsum);
  }
}

/*
 * CPU oracle for the generation-logprob reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * GPU library; the two meet only on the seeded inputs.
 *
 * It is the plain definition, written out as directly as possible:
 * single-threaded, IEEE arithmetic, no blocking, no fusion, a full sort per
 * row.  Build with gcc without -ffast-math and with -ffp-contract=off.
 *
 * Sources (the Flare "generation logprobs" design page, hereafter GLP):
 *   - GLP, definition paragraph: a returned token's logprob is its logit
 *     minus the logsumexp of the whole vocabulary the sampler saw, formed in
 *     (at least) FP32 and before any sampling transform.
 *   - GLP, definition paragraph: K natural alternatives ordered by
 *     decreasing logprob, equal values by increasing token ID; or up to 128
 *     caller-selected IDs reported in caller order with the same
 *     normalization; the chosen token is stored on its own.
 *   - GLP, packed-position paragraph after the buffer table: word layout
 *     [chosen id, chosen bits, id0, bits0, ...]; IDs past the vocabulary are
 *     -1 when it has fewer than K entries.
 *   - GLP, gating paragraphs: only emitted positions are reduced; a zero
 *     request flag skips the row entirely (tiled-reduction paragraph and
 *     zero-flag paragraph).
 *   - GLP, tiled-reduction paragraph: the order is taken on the reported
 *     FP32 values (so equalities created by the subtraction are ties),
 *     signed zero is normalized, padded vocabulary lanes never take part,
 *     and selected IDs subtract the same normalization from their raw logit.
 *   - GLP, prompt-logprobs paragraphs (scored prefill): one row per prompt
 *     target with the target's logprob, its rank among strictly greater
 *     reported values and twenty alternatives in the generation order.
 *   - MTP design page, section "A speculative round is a state transaction":
 *     a slot's verify rows are emitted as a prefix of length 1..k+1.
 *
 * Readings where the pages leave a step open:
 *   R1  only lanes [0, V) are normalized or ranked; [V, V_pad) is padding.
 *   R2  the sum is taken in double, the normalization L is rounded to FP32
 *       once, and each reported value is one FP32 subtraction x - L.
 *   R4  a reported -0.0 is stored as +0.0.
 *   R5  unused pairs when V < K are (-1, 0x7FC00000).
 *   R6  cells that the rules do not write are left untouched.
 *   R7  a chosen or selected ID outside [0, V) is written as given with
 *       value bits 0x7FC00000 and is never dereferenced.
 *   R10 emitted counts are clamped to [0, T], ID counts to [0, 128]; a zero
 *       request flag wins over a nonzero ID count.
 *   R14 completion records: slot s's record is int64 [16 + T]; its emitted
 *       count is the field the caller names (the pages list the fields
 *       without their indices) and verify token t is field 16 + t.  A
 *       count outside [0, 2^31) reads as 0, a token outside the int32
 *       range as -1.  Without ID inputs every slot is natural and each
 *       position holds 2 + 2K words.
 *   R13 packed target rows: slot s's verify row t is logit row
 *       row_offsets[s] + t of P rows; a slot whose committed rows would leave
 *       [0, P) is treated as not emitting (nothing read or written).
 *
 * Parity pins: every function here is pinned by tests that do not reuse its
 * arithmetic (closed forms, brute-force ranks, designed tie rows, a library
 * logsumexp, poison invariants); see the test suite for the list.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_DTYPE_FP32 0
#define ORACLE_DTYPE_BF16 1
#define ORACLE_MAX_IDS 128
#define ORACLE_ROW_WORDS 258
#define ORACLE_MAX_K 20
#define ORACLE_NAN_BITS 0x7FC00000u
#define ORACLE_PROMPT_WORDS 43
#define ORACLE_PROMPT_ALTS 20

/* One vocabulary entry with its reported value, for sorting. */
typedef struct {
  float lp;
  int32_t id;
} oracle_entry;

/* Element i of a row as a double.  bf16 widens exactly: its 16 bits are
 * the top half of an FP32 word. */
static double oracle_widen(const void* row, int dtype, int64_t i) {
  if (dtype == ORACLE_DTYPE_BF16) {
    uint16_t h = ((const uint16_t*)row)[i];
    uint32_t w = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
  }
  return (double)((const float*)row)[i];
}

static uint32_t oracle_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* GLP definition paragraph: L = logsumexp over the unpadded vocabulary
 * (reading R1), computed as M + log(sum exp(x - M)) in double and rounded
 * to FP32 once (reading R2). */
float oracle_row_lse(const void* row, int dtype, int32_t V) {
  double M = -INFINITY;
  for (int32_t i = 0; i < V; ++i) {
    double x = oracle_widen(row, dtype, i);
    if (x > M) M = x;
  }
  if (M == -INFINITY) return -INFINITY; /* all lanes -inf: out of contract */
  double S = 0.0;
  for (int32_t i = 0; i < V; ++i) S += exp(oracle_widen(row, dtype, i) - M);
  return (float)(M + log(S));
}

/* The reported value of one lane: one FP32 subtraction, -0 stored as +0
 * (GLP tiled-reduction paragraph; readings R2 and R4). */
static float oracle_reported(const void* row, int dtype, int32_t i, float L) {
  float x = (float)oracle_widen(row, dtype, i);
  float lp = x - L;
  if (lp == 0.0f) lp = 0.0f;
  return lp;
}

/* Decreasing value, then increasing token ID (GLP definition paragraph). */
static int oracle_cmp_entry(const void* a, const void* b) {
  const oracle_entry* p = (const oracle_entry*)a;
  const oracle_entry* q = (const oracle_entry*)b;
  if (p->lp > q->lp) return -1;
  if (p->lp < q->lp) return 1;
  return (p->id < q->id) ? -1 : (p->id > q->id) ? 1 : 0;
}

/* A chosen or selected ID's pair (reading R7 for IDs outside [0, V)). */
static void oracle_pair(const void* row, int dtype, int32_t V, int32_t id,
                        float L, int32_t* w) {
  w[0] = id;
  if (id >= 0 && id < V)
    w[1] = (int32_t)oracle_bits(oracle_reported(row, dtype, id, L));
  else
    w[1] = (int32_t)ORACLE_NAN_BITS;
}

/*
 * The listing of one emitted position for a given normalization L: the
 * chosen pair, then the selected pairs or the K natural alternatives, all
 * reported as fl32(x - L) (GLP definition and tiled-reduction paragraphs).
 * It is the second half of oracle_row, callable with any L so that a test can
 * ask which listing a slightly different FP32 L would give.  Same return
 * values as oracle_row.
 */
int oracle_row_at_lse(const void* row, int dtype, int32_t V, int32_t token,
                      int32_t n_sel, const int32_t* sel, int32_t K, float L,
                      int32_t* words) {
  if (!row || !words || V < 1 || K < 0 || K > ORACLE_MAX_K) return -1;
  if (dtype != ORACLE_DTYPE_FP32 && dtype != ORACLE_DTYPE_BF16) return -1;
  if (n_sel < 0) n_sel = 0;
  if (n_sel > ORACLE_MAX_IDS) n_sel = ORACLE_MAX_IDS;
  if (n_sel > 0 && !sel) return -1;

  oracle_pair(row, dtype, V, token, L, words);
  if (n_sel > 0) {
    for (int32_t j = 0; j < n_sel; ++j)
      oracle_pair(row, dtype, V, sel[j], L, words + 2 + 2 * j);
    return 2 + 2 * n_sel;
  }
  if (K == 0) return 2;

  oracle_entry* all = (oracle_entry*)malloc((size_t)V * sizeof(oracle_entry));
  if (!all) return -1;
  for (int32_t i = 0; i < V; ++i) {
    all[i].lp = oracle_reported(row, dtype, i, L);
    all[i].id = i;
  }
  qsort(all, (size_t)V, sizeof(oracle_entry), oracle_cmp_entry);
  for (int32_t j = 0; j < K; ++j) {
    int32_t* w = words + 2 + 2 * j;
    if (j < V) {
      w[0] = all[j].id;
      w[1] = (int32_t)oracle_bits(all[j].lp);
    } else { /* GLP packed-position paragraph; reading R5 */
      w[0] = -1;
      w[1] = (int32_t)ORACLE_NAN_BITS;
    }
  }
  free(all);
  return 2 + 2 * K;
}

/*
 * One emitted position.  Writes words [0, 2 + 2W) of `words`, where W = n
 * (selected mode, n > 0) or K (natural mode), and returns that word count,
 * or -1 when the arguments are unusable.  `L_out` (may be NULL) gets the
 * row's normalization.
 */
int oracle_row(const void* row, int dtype, int32_t V, int32_t token,
               int32_t n_sel, const int32_t* sel, int32_t K, int32_t* words,
               float* L_out) {
  if (!row || !words || V < 1 || K < 0 || K > ORACLE_MAX_K) return -1;
  if (dtype != ORACLE_DTYPE_FP32 && dtype != ORACLE_DTYPE_BF16) return -1;
  float L = oracle_row_lse(row, dtype, V);
  if (L_out) *L_out = L;
  return oracle_row_at_lse(row, dtype, V, token, n_sel, sel, K, L, words);
}

/*
 * Prompt scoring (GLP, prompt-logprobs paragraphs): one scored row of a
 * prefill chunk, written as 43 words
 *     [target, bits(r_t), rank, id_0, bits_0, ..., id_19, bits_19]
 * with r_i the reported value of lane i (same L and subtraction as above),
 *     rank = 1 + #{ i in [0, V) : r_i > r_target }   (strictly greater:
 * lanes whose reported value equals r_target, ties the subtraction creates
 * included, do not count), and the twenty alternatives in the generation
 * order (oracle_row's natural listing with K = 20).
 * Readings: R11 a target outside [0, V) marks an invalid row, not only -1;
 * R12 an invalid row reads nothing and writes target -1, NaN bits, rank 0
 * and twenty (-1, 0x7FC00000) pairs (the page fixes the IDs, not the bits).
 * Returns 43, or -1 when the arguments are unusable.  `L_out` (may be NULL)
 * gets L, or NaN for an invalid row.
 */
int oracle_prompt_row(const void* row, int dtype, int32_t V, int32_t target,
                      int32_t* words, float* L_out) {
  if (!row || !words || V < 1) return -1;
  if (dtype != ORACLE_DTYPE_FP32 && dtype != ORACLE_DTYPE_BF16) return -1;
  if (target < 0 || target >= V) { /* readings R11, R12 */
    words[0] = -1;
    words[1] = (int32_t)ORACLE_NAN_BITS;
    words[2] = 0;
    for (int j = 0; j < ORACLE_PROMPT_ALTS; ++j) {
      words[3 + 2 * j] = -1;
      words[4 + 2 * j] = (int32_t)ORACLE_NAN_BITS;
    }
    if (L_out) *L_out = NAN;
    return ORACLE_PROMPT_WORDS;
  }
  int32_t listing[2 + 2 * ORACLE_MAX_K];
  float L;
  if (oracle_row(row, dtype, V, target, 0, NULL, ORACLE_PROMPT_ALTS, listing, &L) < 0)
    return -1;
  if (L_out) *L_out = L;
  float rt = oracle_reported(row, dtype, target, L);
  int32_t greater = 0;
  for (int32_t i = 0; i < V; ++i)
    if (oracle_reported(row, dtype, i, L) > rt) ++greater;
  words[0] = listing[0];
  words[1] = listing[1];
  words[2] = 1 + greater;
  memcpy(words + 3, listing + 2, sizeof(int32_t) * 2 * ORACLE_PROMPT_ALTS);
  return ORACLE_PROMPT_WORDS;
}

/*
 * A scored chunk: `rows` logit rows of stride V_pad and one target per row,
 * written to out [rows, 43] (GLP, prompt-logprobs paragraphs; the page
 * projects rows in blocks of at most 64, which changes nothing per row).
 * `lse_out` (may be NULL) gets each row's L (NaN for invalid rows).
 * Returns the number of valid rows, or -1 on unusable arguments.
 */
int64_t oracle_prompt(const void* logits, int dtype, int32_t rows, int32_t V,
                      int32_t V_pad, const int32_t* targets, int32_t* out,
                      float* lse_out) {
  if (!logits || !targets || !out || rows < 1 || V < 1 || V_pad < V) return -1;
  size_t esize = (dtype == ORACLE_DTYPE_BF16) ? 2 : 4;
  int64_t valid = 0;
  for (int32_t r = 0; r < rows; ++r) {
    const char* row = (const char*)logits + (size_t)r * (size_t)V_pad * esize;
    float L;
    if (oracle_prompt_row(row, dtype, V, targets[r],
                          out + (size_t)r * ORACLE_PROMPT_WORDS, &L) < 0)
      return -1;
    if (lse_out) lse_out[r] = L;
    if (targets[r] >= 0 && targets[r] < V) ++valid;
  }
  return valid;
}

/*
 * One frame [capacity, T, 258].  Row (s, t) of `logits` starts at element
 * (s * T + t) * V_pad.  Only active positions are written (GLP gating and
 * zero-flag paragraphs; MTP design page, round section):
 *   active(s, t)  <=>  requested[s] != 0  and  t < clamp(emitted[s], 0, T).
 * `lse_out` (may be NULL) is [capacity * T] and gets L for active rows only.
 * Returns the number of active rows, or -1 on unusable arguments.
 */
int64_t oracle_frame(const void* logits, int dtype, int32_t capacity,
                     int32_t T, int32_t V, int32_t V_pad,
                     const int32_t* requested, const int32_t* id_counts,
                     const int32_t* ids, const int32_t* emitted,
                     const int32_t* tokens, int32_t K, int32_t* out,
                     float* lse_out) {
  if (!logits || !requested || !id_counts || !ids || !emitted || !tokens ||
      !out)
    return -1;
  if (capacity < 1 || T < 1 || V < 1 || V_pad < V || K < 0 ||
      K > ORACLE_MAX_K)
    return -1;
  size_t esize = (dtype == ORACLE_DTYPE_BF16) ? 2 : 4;
  int64_t active = 0;
  for (int32_t s = 0; s < capacity; ++s) {
    if (requested[s] == 0) continue;
    int32_t e = emitted[s];
    if (e < 0) e = 0;
    if (e > T) e = T;
    int32_t n = id_counts[s];
    if (n < 0) n = 0;
    if (n > ORACLE_MAX_IDS) n = ORACLE_MAX_IDS;
    for (int32_t t = 0; t < e; ++t) {
      int64_t r = (int64_t)s * T + t;
      const char* row = (const char*)logits + (size_t)r * (size_t)V_pad * esize;
      float L;
      int rc = oracle_row(row, dtype, V, tokens[r], n,
                          ids + (size_t)s * ORACLE_MAX_IDS, K,
                          out + (size_t)r * ORACLE_ROW_WORDS, &L);
      if (rc < 0) return -1;
      if (lse_out) lse_out[r] = L;
      ++active;
    }
  }
  return active;
}

/*
 * One frame over packed target rows (MTP design page, graph catalog
 * paragraph: P physical target rows, possibly fewer than capacity * T; GLP
 * gating paragraph: a packed request's columns past its committed prefix are
 * never read).  As oracle_frame, except that position (s, t) reads logit row
 * row_offsets[s] + t of the P rows at `logits` (reading R13).  Output and
 * `lse_out` stay indexed by frame position s * T + t.
 */
int64_t oracle_frame_packed(const void* logits, int dtype, int32_t capacity,
                            int32_t T, int32_t P, int32_t V, int32_t V_pad,
                            const int32_t* requested, const int32_t* id_counts,
                            const int32_t* ids, const int32_t* emitted,
                            const int32_t* tokens, const int32_t* row_offsets,
                            int32_t K, int32_t* out, float* lse_out) {
  if (!logits || !requested || !id_counts || !ids || !emitted || !tokens ||
      !row_offsets || !out)
    return -1;
  if (capacity < 1 || T < 1 || P < 1 || V < 1 || V_pad < V || K < 0 ||
      K > ORACLE_MAX_K)
    return -1;
  size_t esize = (dtype == ORACLE_DTYPE_BF16) ? 2 : 4;
  int64_t active = 0;
  for (int32_t s = 0; s < capacity; ++s) {
    if (!requested[s]) continue;
    int32_t e = emitted[s] < 0 ? 0 : (emitted[s] > T ? T : emitted[s]);
    int64_t first = row_offsets[s];
    if (e > 0 && (first < 0 || first + e > P)) continue; /* reading R13 */
    int32_t n = id_counts[s] < 0 ? 0 : id_counts[s];
    if (n > ORACLE_MAX_IDS) n = ORACLE_MAX_IDS;
    for (int32_t t = 0; t < e; ++t) {
      int64_t pos = (int64_t)s * T + t; /* frame position */
      const char* row =
          (const char*)logits + (size_t)(first + t) * (size_t)V_pad * esize;
      float L;
      if (oracle_row(row, dtype, V, tokens[pos], n,
                     ids + (size_t)s * ORACLE_MAX_IDS, K,
                     out + (size_t)pos * ORACLE_ROW_WORDS, &L) < 0)
        return -1;
      if (lse_out) lse_out[pos] = L;
      ++active;
    }
  }
  return active;
}

/*
 * One frame whose emitted counts and chosen tokens are read from the int64
 * completion records [capacity, 16 + T] (GLP buffer table; MTP design page,
 * catalog paragraph; reading R14).  `id_counts` and `ids` may both be NULL
 * (a core without ID inputs, GLP declaration paragraph): then every slot is
 * natural and position (s, t) occupies `row_words` = 2 + 2K words of `out`;
 * otherwise row_words is 258.  Returns the active row count, or -1.
 */
int64_t oracle_frame_records(const void* logits, int dtype, int32_t capacity,
                             int32_t T, int32_t V, int32_t V_pad,
                             const int32_t* requested, const int32_t* id_counts,
                             const int32_t* ids, const int64_t* records,
                             int32_t emitted_field, int32_t K, int32_t row_words,
                             int32_t* out, float* lse_out) {
  if (!logits || !requested || !records || !out) return -1;
  if ((id_counts == NULL) != (ids == NULL)) return -1;
  if (emitted_field < 0 || emitted_field >= 16) return -1;
  if (capacity < 1 || T < 1 || V < 1 || V_pad < V || K < 0 || K > ORACLE_MAX_K)
    return -1;
  if (id_counts ? row_words != ORACLE_ROW_WORDS : (K < 1 || row_words != 2 + 2 * K))
    return -1;
  size_t esize = (dtype == ORACLE_DTYPE_BF16) ? 2 : 4;
  int32_t words[ORACLE_ROW_WORDS];
  int64_t active = 0;
  for (int32_t s = 0; s < capacity; ++s) {
    const int64_t* record = records + (size_t)s * (16 + (size_t)T);
    if (!requested[s]) continue;
    int64_t count = record[emitted_field];
    int32_t e = (count < 0 || count > 2147483647LL) ? 0 : (int32_t)count;
    if (e > T) e = T;
    int32_t n = 0;
    if (id_counts) n = id_counts[s] < 0 ? 0 : (id_counts[s] > ORACLE_MAX_IDS ? ORACLE_MAX_IDS : id_counts[s]);
    for (int32_t t = 0; t < e; ++t) {
      int64_t tok64 = record[16 + t];
      int32_t tok = (tok64 < -2147483648LL || tok64 > 2147483647LL) ? -1 : (int32_t)tok64;
      int64_t at = (int64_t)s * T + t;
      const char* row = (const char*)logits + (size_t)at * (size_t)V_pad * esize;
      float L;
      int used = oracle_row(row, dtype, V, tok, n, ids ? ids + (size_t)s * ORACLE_MAX_IDS : NULL,
                            K, words, &L);
      if (used < 0 || used > row_words) return -1;
      memcpy(out + (size_t)at * (size_t)row_words, words, sizeof(int32_t) * (size_t)used);
      if (lse_out) lse_out[at] = L;
      ++active;
    }
  }
  return active;
}


/*
 * Seeded synthetic inputs for the generation-logprob reduction.
 *
 * This module only makes inputs.  It holds none of the reduction's
 * arithmetic (no max, no logsumexp, no ranking) and is shared by the
 * oracle's tests, the GPU parity tests and the benchmark alike.
 *
 * Randomness is counter based: every value is a pure function of
 * (seed, stream tag, row, lane) through the SplitMix64 finalizer
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014), so any row can be regenerated on its own and
 * the threads that fill rows need no shared state.
 *
 *   row key  k = mix(mix(mix(seed) ^ tag) ^ row)
 *   lane     h = mix(k + (lane + 1) * 0x9E3779B97F4A7C15)
 *
 * Uniforms take the top 53 bits, (h >> 11 + 0.5) / 2^53, so they lie in
 * (0, 1).  Normals use the Box-Muller cosine branch with both halves of h.
 * Gumbel(0, 1) is -log(-log u).  bf16 values are FP32 values rounded to
 * nearest even.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_FP32 0
#define SYNTH_BF16 1

#define SYNTH_NORMAL 0 /* p0 * N(0,1) + optional spike p1 at one lane */
#define SYNTH_GUMBEL 1 /* Gumbel(0,1) + optional spike p1 at one lane */
#define SYNTH_GRID8 2  /* k/8 - 8, k uniform in 0..128; some rows one-hot */

#define SYNTH_PAD_ZERO 0
#define SYNTH_PAD_PINF 1
#define SYNTH_PAD_NAN 2

/* Stream tags, one per independent quantity. */
#define TAG_LOGITS 1u
#define TAG_SPIKE 6u
#define TAG_ONEHOT 7u

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

uint64_t synth_row_key(uint64_t seed, uint64_t tag, uint64_t row) {
  return mix64(mix64(mix64(seed) ^ tag) ^ row);
}

static inline uint64_t lane_hash(uint64_t key, uint64_t lane) {
  return mix64(key + (lane + 1) * GAMMA);
}

uint64_t synth_hash(uint64_t seed, uint64_t tag, uint64_t row, uint64_t lane) {
  return lane_hash(synth_row_key(seed, tag, row), lane);
}

/* out[i] = synth_hash(seed, tag, row, lane0 + i) */
void synth_hashes(uint64_t* out, int64_t n, uint64_t seed, uint64_t tag,
                  uint64_t row, uint64_t lane0) {
  uint64_t k = synth_row_key(seed, tag, row);
  for (int64_t i = 0; i < n; ++i) out[i] = lane_hash(k, lane0 + (uint64_t)i);
}

static inline double unif53(uint64_t h) {
  return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_bm(uint64_t h) {
  double u1 = ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(h & 0xffffffffu) + 0.5) * (1.0 / 4294967296.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t r = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + r) >> 16);
}

static inline void store(void* row, int dtype, int64_t i, float v) {
  if (dtype == SYNTH_BF16)
    ((uint16_t*)row)[i] = to_bf16(v);
  else
    ((float*)row)[i] = v;
}

static inline void store_bits(void* row, int dtype, int64_t i, uint32_t f32bits,
                              uint16_t bf16bits) {
  if (dtype == SYNTH_BF16)
    ((uint16_t*)row)[i] = bf16bits;
  else
    memcpy((char*)row + 4 * i, &f32bits, 4);
}

typedef struct {
  void* base;
  int dtype;
  int64_t r0, r1;        /* global row range filled by this job */
  int64_t row_offset;    /* global index of base's first row */
  int32_t V, V_pad;
  int recipe;
  double p0, p1;
  uint64_t seed;
  const uint8_t* garbage; /* per global row, may be NULL */
  int pad_kind;
} fill_job;

static void fill_one_row(const fill_job* j, int64_t r) {
  size_t esize = j->dtype == SYNTH_BF16 ? 2 : 4;
  void* row = (char*)j->base + (size_t)(r - j->row_offset) * j->V_pad * esize;
  if (j->garbage && j->garbage[r]) {
    /* Rows that must never be read: alternating NaN and +inf. */
    for (int64_t i = 0; i < j->V_pad; ++i) {
      if (i & 1)
        store_bits(row, j->dtype, i, 0x7F800000u, 0x7F80u);
      else
        store_bits(row, j->dtype, i, 0x7FC00000u, 0x7FC0u);
    }
    return;
  }
  uint64_t key = synth_row_key(j->seed, TAG_LOGITS, (uint64_t)r);
  int64_t spike = -1;
  if (j->p1 != 0.0 && j->recipe != SYNTH_GRID8)
    spike = (int64_t)(synth_hash(j->seed, TAG_SPIKE, (uint64_t)r, 0) % (uint64_t)j->V);

  if (j->recipe == SYNTH_GRID8) {
    uint64_t oh = synth_hash(j->seed, TAG_ONEHOT, (uint64_t)r, 0);
    int one_hot = (j->p0 > 0.0) && (oh % (uint64_t)j->p0 == 0);
    if (one_hot) {
      int64_t hot = (int64_t)(synth_hash(j->seed, TAG_ONEHOT, (uint64_t)r, 1) % (uint64_t)j->V);
      uint64_t kh = synth_hash(j->seed, TAG_ONEHOT, (uint64_t)r, 2);
      float hv = (float)((double)(kh % 129u) / 8.0 - 8.0);
      if (synth_hash(j->seed, TAG_ONEHOT, (uint64_t)r, 3) & 1u) hv = -0.0f;
      for (int64_t i = 0; i < j->V; ++i) store(row, j->dtype, i, -INFINITY);
      store(row, j->dtype, hot, hv);
    } else {
      for (int64_t i = 0; i < j->V; ++i) {
        uint64_t k = (uint64_t)(unif53(lane_hash(key, (uint64_t)i)) * 129.0);
        if (k > 128) k = 128;
        store(row, j->dtype, i, (float)((double)k / 8.0 - 8.0));
      }
    }
  } else {
    for (int64_t i = 0; i < j->V; ++i) {
      uint64_t h = lane_hash(key, (uint64_t)i);
      double v = (j->recipe == SYNTH_GUMBEL) ? -log(-log(unif53(h)))
                                             : j->p0 * normal_bm(h);
      if (i == spike) v += j->p1;
      store(row, j->dtype, i, (float)v);
    }
  }
  for (int64_t i = j->V; i < j->V_pad; ++i) {
    if (j->pad_kind == SYNTH_PAD_PINF)
      store_bits(row, j->dtype, i, 0x7F800000u, 0x7F80u);
    else if (j->pad_kind == SYNTH_PAD_NAN)
      store_bits(row, j->dtype, i, 0x7FC00000u, 0x7FC0u);
    else
      store_bits(row, j->dtype, i, 0u, 0u);
  }
}

static void* fill_worker(void* arg) {
  const fill_job* j = (const fill_job*)arg;
  for (int64_t r = j->r0; r < j->r1; ++r) fill_one_row(j, r);
  return NULL;
}

/*
 * Fill rows [row_begin, row_end) of a [*, V_pad] buffer whose first row is
 * global row `row_begin`.  `garbage` (may be NULL) marks global rows that
 * get the NaN/+inf pattern instead.  Returns 0 on success.
 */
int synth_fill(void* base, int dtype, int64_t row_begin, int64_t row_end,
               int32_t V, int32_t V_pad, int recipe, double p0, double p1,
               uint64_t seed, const uint8_t* garbage, int pad_kind,
               int nthreads) {
  if (!base || V < 1 || V_pad < V || row_end < row_begin) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  int64_t nrows = row_end - row_begin;
  if (nrows < nthreads) nthreads = nrows > 0 ? (int)nrows : 1;
  pthread_t th[64];
  int joinable[64];
  fill_job jobs[64];
  int64_t per = (nrows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    fill_job* j = &jobs[t];
    joinable[t] = 0;
    j->base = base;
    j->dtype = dtype;
    j->row_offset = row_begin;
    j->r0 = row_begin + t * per;
    j->r1 = j->r0 + per;
    if (j->r1 > row_end) j->r1 = row_end;
    if (j->r0 >= j->r1) continue;
    j->V = V;
    j->V_pad = V_pad;
    j->recipe = recipe;
    j->p0 = p0;
    j->p1 = p1;
    j->seed = seed;
    j->garbage = garbage;
    j->pad_kind = pad_kind;
    if (pthread_create(&th[t], NULL, fill_worker, j) == 0)
      joinable[t] = 1;
    else
      fill_worker(j);
  }
  for (int t = 0; t < nthreads; ++t)
    if (joinable[t]) pthread_join(th[t], NULL);
  return 0;
}

// CPU sanitizer leg: the oracle, the input generator and the host-only half
// of the C ABI (plans with device = -1 and every call's rejection paths),
// built with -fsanitize=address,undefined and run as one program.  Nothing
// here touches a GPU: the device-side entry points of the library and the few
// HIP runtime calls of the host code are stubbed, and every path exercised
// returns before it would reach them (a stub that is reached aborts).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "flare_logprobs.h"
#include "../full_vocab_logprob_amd/csrc/flp_internal.h"

// ---- stubs for what the exercised paths never reach
namespace flp {
int launch(const Params&, int, bool, bool, int, void*) { abort(); }
int reduce_occupancy(int, bool, bool, int, bool) { abort(); }
int launch_shard_finalize(const Params&, int, void*) { abort(); }
int launch_shard_merge(const Params&, int, bool, void*) { abort(); }
int scratch_address(int, void**) { abort(); }
}  // namespace flp
hipError_t hipGetDevice(int*) { abort(); }
hipError_t hipGetDeviceCount(int*) { abort(); }
hipError_t hipSetDevice(int) { abort(); }
hipError_t hipGetDeviceProperties(hipDeviceProp_t*, int) { abort(); }

// ---- the oracle and the generator (C, separate translation units)
extern "C" {
float oracle_row_lse(const void* row, int dtype, int32_t V);
int oracle_row(const void* row, int dtype, int32_t V, int32_t token, int32_t n_sel,
               const int32_t* sel, int32_t K, int32_t* words, float* L_out);
int oracle_row_at_lse(const void* row, int dtype, int32_t V, int32_t token, int32_t n_sel,
                      const int32_t* sel, int32_t K, float L, int32_t* words);
int oracle_prompt_row(const void* row, int dtype, int32_t V, int32_t target, int32_t* words,
                      float* L_out);
int64_t oracle_prompt(const void* logits, int dtype, int32_t rows, int32_t V, int32_t V_pad,
                      const int32_t* targets, int32_t* out, float* lse_out);
int64_t oracle_frame(const void* logits, int dtype, int32_t capacity, int32_t T, int32_t V,
                     int32_t V_pad, const int32_t* requested, const int32_t* id_counts,
                     const int32_t* ids, const int32_t* emitted, const int32_t* tokens, int32_t K,
                     int32_t* out, float* lse_out);
int64_t oracle_frame_packed(const void* logits, int dtype, int32_t capacity, int32_t T, int32_t P,
                            int32_t V, int32_t V_pad, const int32_t* requested,
                            const int32_t* id_counts, const int32_t* ids, const int32_t* emitted,
                            const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                            int32_t* out, float* lse_out);
int64_t oracle_frame_records(const void* logits, int dtype, int32_t capacity, int32_t T,
                             int32_t V, int32_t V_pad, const int32_t* requested,
                             const int32_t* id_counts, const int32_t* ids, const int64_t* records,
                             int32_t emitted_field, int32_t K, int32_t row_words, int32_t* out,
                             float* lse_out);
int synth_fill(void* base, int dtype, int64_t row_begin, int64_t row_end, int32_t V,
               int32_t V_pad, int recipe, double p0, double p1, uint64_t seed,
               const uint8_t* garbage, int pad_kind, int nthreads);
void synth_hashes(uint64_t* out, int64_t n, uint64_t seed, uint64_t tag, uint64_t row,
                  uint64_t lane0);
}

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);    \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}

// ------------------------------------------------------------- the oracle
static void oracle_rows() {
  const int Vs[] = {1, 5, 19, 20, 64, 1000};
  for (int dtype = 0; dtype < 2; ++dtype) {
    for (int V : Vs) {
      std::vector<float> f(V);
      std::vector<uint16_t> h(V);
      for (int i = 0; i < V; ++i) {
        const int k = (int)(rnd() % 17) - 8;
        f[i] = k == -8 ? -INFINITY : (k == 0 && (i & 1) ? -0.0f : 0.5f * k);
        uint32_t b;
        memcpy(&b, &f[i], 4);
        h[i] = (uint16_t)(b >> 16);
      }
      const void* row = dtype ? (const void*)h.data() : (const void*)f.data();
      const int32_t sel[6] = {0, V - 1, -1, V, 0x7FFFFFFF, V / 2};
      std::vector<int32_t> sel128(128);
      for (int j = 0; j < 128; ++j) sel128[j] = (int32_t)(rnd() % (uint64_t)(V + 2)) - 1;
      for (int K : {0, 1, 20}) {
        for (int tok : {-7, 0, V - 1, V}) {
          int32_t words[258];
          float L = 0.0f;
          const int n = oracle_row(row, dtype, V, tok, 0, nullptr, K, words, &L);
          CHECK(n == 2 + 2 * K);
          CHECK(words[0] == tok);
          for (int j = 0; j < K && j < V; ++j) CHECK(words[2 + 2 * j] >= 0 && words[2 + 2 * j] < V);
          for (int j = V; j < K; ++j) CHECK(words[2 + 2 * j] == -1);
          int32_t again[258];
          CHECK(oracle_row_at_lse(row, dtype, V, tok, 0, nullptr, K, L, again) == n);
          CHECK(memcmp(words, again, sizeof(int32_t) * (size_t)n) == 0);
          CHECK(oracle_row(row, dtype, V, tok, 6, sel, K, words, &L) == 14);
          CHECK(oracle_row(row, dtype, V, tok, 128, sel128.data(), K, words, nullptr) == 258);
          CHECK(oracle_row(row, dtype, V, tok, 300, sel128.data(), K, words, nullptr) == 258);
        }
      }
      int32_t pw[43];
      for (int tgt : {-1, 0, V - 1, V}) CHECK(oracle_prompt_row(row, dtype, V, tgt, pw, nullptr) == 43);
    }
  }
  // rejected arguments
  float one = 1.0f;
  int32_t w[258];
  CHECK(oracle_row(nullptr, 0, 1, 0, 0, nullptr, 1, w, nullptr) < 0);
  CHECK(oracle_row(&one, 0, 0, 0, 0, nullptr, 1, w, nullptr) < 0);
  CHECK(oracle_row(&one, 0, 1, 0, 0, nullptr, 21, w, nullptr) < 0);
  CHECK(oracle_row(&one, 2, 1, 0, 0, nullptr, 1, w, nullptr) < 0);
  CHECK(oracle_row(&one, 0, 1, 0, 3, nullptr, 1, w, nullptr) < 0);
  float ninf[3] = {-INFINITY, -INFINITY, -INFINITY};
  CHECK(std::isinf(oracle_row_lse(ninf, 0, 3)));
}

static void oracle_frames() {
  const int cap = 6, T = 3, V = 300, Vp = 304;
  std::vector<float> logits((size_t)cap * T * Vp);
  for (auto& x : logits) x = (float)((int)(rnd() % 2001) - 1000) / 100.0f;
  const int32_t req[cap] = {1, 0, 1, 1, 1, 1};
  const int32_t emi[cap] = {2, 3, 0, 9, -4, 3};
  const int32_t cnt[cap] = {-5, 4, 3, 0, 0, 300};
  std::vector<int32_t> ids(cap * 128), tok(cap * T);
  for (auto& i : ids) i = (int32_t)(rnd() % (V + 4)) - 2;
  for (auto& t : tok) t = (int32_t)(rnd() % (V + 4)) - 2;
  std::vector<int32_t> out((size_t)cap * T * 258, 0x5A5A5A5A);
  std::vector<float> lse(cap * T);
  CHECK(oracle_frame(logits.data(), 0, cap, T, V, Vp, req, cnt, ids.data(), emi, tok.data(), 20,
                     out.data(), lse.data()) == 2 + 3 + 3);
  // packed rows: slot 0 in range, slot 3 past P, slot 5 at a negative offset
  const int P = 7;
  const int32_t off[cap] = {0, 0, 0, 6, 0, -2};
  CHECK(oracle_frame_packed(logits.data(), 0, cap, T, P, V, Vp, req, cnt, ids.data(), emi,
                            tok.data(), off, 5, out.data(), lse.data()) == 2);
  // completion records, with and without ID inputs
  std::vector<int64_t> rec((size_t)cap * (16 + T));
  for (size_t i = 0; i < rec.size(); ++i) rec[i] = (int64_t)(rnd() % 600) - 50;
  rec[3] = 2;
  rec[(16 + T) + 3] = (int64_t)1 << 40;
  CHECK(oracle_frame_records(logits.data(), 0, cap, T, V, Vp, req, cnt, ids.data(), rec.data(), 3,
                             20, 258, out.data(), lse.data()) >= 0);
  std::vector<int32_t> compact((size_t)cap * T * (2 + 2 * 7));
  CHECK(oracle_frame_records(logits.data(), 0, cap, T, V, Vp, req, nullptr, nullptr, rec.data(),
                             3, 7, 2 + 2 * 7, compact.data(), nullptr) >= 0);
  CHECK(oracle_frame_records(logits.data(), 0, cap, T, V, Vp, req, cnt, nullptr, rec.data(), 3,
                             7, 258, out.data(), nullptr) < 0);
  CHECK(oracle_frame_records(logits.data(), 0, cap, T, V, Vp, req, nullptr, nullptr, rec.data(),
                             16, 7, 16, compact.data(), nullptr) < 0);
  // prompt chunk with invalid targets and a vocabulary below twenty
  std::vector<int32_t> tg(cap * T);
  for (size_t i = 0; i < tg.size(); ++i) tg[i] = (int32_t)(rnd() % 12) - 2;
  std::vector<int32_t> pout((size_t)cap * T * 43);
  CHECK(oracle_prompt(logits.data(), 0, cap * T, 9, Vp, tg.data(), pout.data(), lse.data()) >= 0);
  CHECK(oracle_frame(nullptr, 0, cap, T, V, Vp, req, cnt, ids.data(), emi, tok.data(), 20,
                     out.data(), nullptr) < 0);
}

// ---------------------------------------------------------- the generator
static void generator() {
  for (int dtype = 0; dtype < 2; ++dtype) {
    for (int recipe = 0; recipe < 3; ++recipe) {
      for (int pad = 0; pad < 3; ++pad) {
        const int rows = 5, V = 997, Vp = 1008;
        std::vector<uint8_t> buf((size_t)rows * Vp * (dtype ? 2 : 4));
        uint8_t garbage[12] = {0, 1, 0, 0, 1, 0, 0, 0, 0, 0, 0, 0};
        CHECK(synth_fill(buf.data(), dtype, 3, 3 + rows, V, Vp, recipe, recipe == 2 ? 3.0 : 2.5,
                         recipe == 2 ? 0.0 : 7.0, 11, garbage, pad, 1 + pad) == 0);
      }
    }
  }
  std::vector<uint64_t> h(1000);
  synth_hashes(h.data(), (int64_t)h.size(), 3, 1, 7, 0);
  CHECK(synth_fill(nullptr, 0, 0, 1, 1, 1, 0, 1.0, 0.0, 1, nullptr, 0, 1) < 0);
}

// ------------------------------------------------------- the host half
static void host_plans() {
  flare_logprobs_plan_t p;
  struct G { int cap, T, V, Vp, dt, K; };
  const G ok[] = {{8, 1, 32000, 32000, 0, 20},      {64, 1, 151936, 152064, 0, 20},
                  {128, 8, 248320, 248320, 1, 20},  {1024, 4, 262144, 262144, 0, 0},
                  {3, 4, 37, 41, 1, 5},             {8192, 1, 1, 1, 0, 20}};
  for (const G& g : ok) {
    CHECK(flare_logprobs_plan(&p, g.cap, g.T, g.V, g.Vp, g.dt, g.K, -1) == FLARE_OK);
    CHECK(p.workspace_bytes > 0 && p.grid == 1024 && p.shards == 0);
    CHECK(flare_logprobs_plan_packed(&p, g.cap, g.T, g.cap * g.T, g.V, g.Vp, g.dt, g.K, -1) ==
          FLARE_OK);
    CHECK(flare_logprobs_plan_sharded(&p, g.cap, g.T, g.V, g.Vp, g.dt, g.K, 1, -1) == FLARE_OK);
  }
  const G bad[] = {{0, 1, 10, 10, 0, 1},  {1, 0, 10, 10, 0, 1},  {1, 1, 0, 1, 0, 1},
                   {1, 1, 10, 9, 0, 1},   {1, 1, 10, 10, 0, -1}, {1, 1, 10, 10, 0, 21},
                   {1, 1, 10, 10, 2, 1},  {8193, 1, 10, 10, 0, 1}, {1, 1, 16384 * 64 + 1, 16384 * 64 + 1, 1, 1}};
  for (const G& g : bad) {
    CHECK(flare_logprobs_plan(&p, g.cap, g.T, g.V, g.Vp, g.dt, g.K, -1) != FLARE_OK);
    CHECK(p.abi_version == 0);
  }
  CHECK(flare_logprobs_plan(nullptr, 1, 1, 1, 1, 0, 0, -1) == FLARE_ERR_INVALID_ARGUMENT);
  CHECK(flare_logprobs_plan_packed(&p, 4, 2, 0, 100, 100, 0, 3, -1) == FLARE_ERR_INVALID_ARGUMENT);
  CHECK(flare_logprobs_plan_sharded(&p, 4, 2, 50, 56, 0, 3, 8, -1) == FLARE_ERR_INVALID_ARGUMENT);
  CHECK(flare_logprobs_plan_sharded(&p, 4, 2, 5000, 5000, 0, 3, 33, -1) == FLARE_ERR_INVALID_ARGUMENT);
  CHECK(flare_logprobs_plan_sharded(&p, 128, 8, 248320, 248320, 1, 20, 8, -1) == FLARE_OK);
  CHECK(p.shards == 8 && p.exchange_offset > 0);
  CHECK(flare_prompt_logprobs_plan(&p, 128, 248320, 248320, 1, -1) == FLARE_OK);
  CHECK(flare_prompt_logprobs_plan(&p, 8192, 16384 * 64 + 1, 16384 * 64 + 1, 1, -1) ==
        FLARE_ERR_UNSUPPORTED_SIZE);
  for (int s = -2; s < 10; ++s) CHECK(flare_status_string(s) != nullptr);
  CHECK(flare_logprobs_abi_version() == FLARE_LOGPROBS_ABI_VERSION);
}

static void host_rejections() {
  flare_logprobs_plan_t p, sp, pp, pr;
  CHECK(flare_logprobs_plan(&p, 16, 4, 5000, 5000, 1, 20, -1) == FLARE_OK);
  CHECK(flare_logprobs_plan_sharded(&sp, 16, 4, 5000, 5000, 1, 20, 4, -1) == FLARE_OK);
  CHECK(flare_logprobs_plan_packed(&pp, 16, 4, 30, 5000, 5000, 1, 20, -1) == FLARE_OK);
  CHECK(flare_prompt_logprobs_plan(&pr, 64, 5000, 5000, 1, -1) == FLARE_OK);
  int32_t* F = (int32_t*)(uintptr_t)0x10000;  // never dereferenced
  void* ws = (void*)(uintptr_t)0x20000;
  const int64_t rows = 64;
  // null pointers, mismatches, corrupted plans: every one fails before a launch
  CHECK(flare_logprobs_run(&p, nullptr, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 1);
  CHECK(flare_logprobs_run(&p, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, nullptr, nullptr) == 1);
  CHECK(flare_logprobs_run(&p, F, 0, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run(&p, F, 1, rows, 5001, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run(&p, F, 1, rows - 1, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run(&p, F, 1, rows, 5000, 5000, F, F, F, F, F, 19, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run(&p, F, 5, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 2);
  CHECK(flare_logprobs_run(&p, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, (char*)ws + 4, nullptr) == 1);
  flare_logprobs_plan_t bad = p;
  bad.abi_version = 99;
  CHECK(flare_logprobs_run(&bad, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  bad = p;
  bad.ranges = 3;
  CHECK(flare_logprobs_reduce(&bad, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  bad = p;
  bad.units = 65;
  CHECK(flare_logprobs_merge(&bad, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  // the other mode's, the packed and the sharded plans
  CHECK(flare_logprobs_run(&pr, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run(&sp, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run(&pp, F, 1, 30, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run_packed(&pp, F, 1, 30, 5000, 5000, F, F, F, F, F, nullptr, 20, F, ws, nullptr) == 1);
  CHECK(flare_logprobs_run_packed(&pp, F, 1, 31, 5000, 5000, F, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_run_sharded(&p, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_logprobs_shard_pass(&sp, 4, F, 1, rows, 5000, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 1);
  CHECK(flare_logprobs_shard_merge(&sp, F, 1, rows, 4999, 5000, F, F, F, F, F, 20, F, ws, nullptr) == 3);
  CHECK(flare_prompt_logprobs_run(&p, F, 1, 64, 5000, 5000, F, F, ws, nullptr) == 3);
  CHECK(flare_prompt_logprobs_run(&pr, F, 1, 63, 5000, 5000, F, F, ws, nullptr) == 3);
  // completion records: the field index, the compact extent, the ID inputs
  const int64_t* R = (const int64_t*)(uintptr_t)0x30000;
  CHECK(flare_logprobs_run_records(&p, F, 1, rows, 5000, 5000, F, F, F, R, 16, 20, F, 258, ws, nullptr) == 1);
  CHECK(flare_logprobs_run_records(&p, F, 1, rows, 5000, 5000, F, F, F, R, 3, 20, F, 42, ws, nullptr) == 1);
  CHECK(flare_logprobs_run_records(&p, F, 1, rows, 5000, 5000, F, F, nullptr, R, 3, 20, F, 258, ws, nullptr) == 1);
  CHECK(flare_logprobs_run_records(&p, F, 1, rows, 5000, 5000, F, F, F, nullptr, 3, 20, F, 258, ws, nullptr) == 1);
  // the no-allocation call: a null plan, and a plan beyond its scratch
  flare_logprobs_plan_t big;
  CHECK(flare_logprobs_plan(&big, 1024, 4, 262144, 262144, 0, 20, -1) == FLARE_OK);
  CHECK(flare_logprobs_run_noalloc(nullptr, F, 0, 4096, 262144, 262144, F, F, F, F, F, 20, F, nullptr) == 1);
  CHECK(flare_logprobs_run_noalloc(&big, F, 0, 4096, 262144, 262144, F, F, F, F, F, 20, F, nullptr) ==
        FLARE_ERR_SCRATCH_TOO_SMALL);
}

int main() {
  oracle_rows();
  oracle_frames();
  generator();
  host_plans();
  host_rejections();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("sanitizer leg: all checks passed\n");
  return 0;
}

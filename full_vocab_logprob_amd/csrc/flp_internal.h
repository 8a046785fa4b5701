// Internal layout shared by the host and device sources of libflare_logprobs.
#pragma once

#include <stdint.h>

namespace flp {

constexpr int kBlock = 256;      // threads per workgroup (4 wave64s)
constexpr int kWaves = kBlock / 64;
constexpr int kChunks = 8;       // 16-byte chunks held per thread
constexpr int kKeep = 32;        // raw keys a segment retains
constexpr int kMaxSegs = 64;     // segments per row the merge pool supports

// Vocabulary lanes per 16-byte chunk and per segment (= one workgroup).
constexpr int elems_per_chunk(int dtype) { return dtype == 1 ? 8 : 4; }
constexpr int seg_elems(int dtype) { return kBlock * kChunks * elems_per_chunk(dtype); }
constexpr int elem_bytes(int dtype) { return dtype == 1 ? 2 : 4; }

// One segment's contribution to a row: its max and exp-sum relative to that
// max, and its best raw keys (value, then smaller ID), sorted descending.
struct SegRecord {
  float m;
  float s;
  int32_t n;      // keys held (kKeep unless the segment has fewer lanes)
  int32_t flags;  // kRecComplete: every lane of the segment is held
  uint64_t keys[kKeep];
};
static_assert(sizeof(SegRecord) == 272, "record layout");
constexpr int32_t kRecComplete = 1;

struct Params {
  const void* logits;
  const int32_t* requested;
  const int32_t* id_counts;
  const int32_t* ids;
  const int32_t* emitted;
  const int32_t* tokens;
  int32_t* out;
  SegRecord* records;
  float* lse;
  uint32_t* tickets;
  int64_t V_pad;
  int32_t capacity;
  int32_t T;
  int32_t V;
  int32_t K;
  int32_t nseg;
  int32_t merge_pool;  // keys in the merge workgroup's LDS pool (power of 2)
};

// Launchers implemented in flp_kernels.hip; return a hipError_t as int.
int launch_reduce(const Params& p, int dtype, bool vector_rows, int merge_mode,
                  void* stream);
int launch_reset(uint32_t* tickets, int64_t n, void* stream);

}  // namespace flp

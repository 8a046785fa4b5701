// Internal layout shared by the host and device sources of libflare_logprobs.
#pragma once

#include <stdint.h>

namespace flp {

constexpr int kChunks = 8;          // 16-byte chunks each thread holds per unit
constexpr int kUnitThreads = 256;   // threads (4 wave64s) sharing one unit
constexpr int kBlock = kUnitThreads; // reduction workgroup
constexpr int kMergeBlock = 256;    // merge workgroup
constexpr int kKeep = 32;           // raw keys a part keeps
constexpr int kMaxUnits = 64;       // units per row (one merge lane per unit)
constexpr int kMaxCapacity = 8192;  // slots whose active-row prefix fits in LDS
constexpr int kPromptWords = 43;    // words of one scored prompt row
constexpr int kPromptAlts = 20;     // alternatives of a scored prompt row
constexpr int kMaxRangeRows = 64;   // rows one unit range may touch when scoring
constexpr int kRecordMeta = 16;     // metadata fields before a completion record's tokens

// Vocabulary lanes per 16-byte chunk, and per unit: the lanes one workgroup
// holds in registers at a time (16,384 bf16 or 8,192 FP32 lanes, 32 KiB).
constexpr int elems_per_chunk(int dtype) { return dtype == 1 ? 8 : 4; }
constexpr int unit_elems(int dtype) { return kUnitThreads * kChunks * elems_per_chunk(dtype); }
constexpr int elem_bytes(int dtype) { return dtype == 1 ? 2 : 4; }

// One part's contribution to a row: a part is the run of consecutive units
// of one row that one workgroup reduced.  m is the part's max, s the sum of
// exp(x - m) over its lanes, keys its best raw keys (value, then smaller ID)
// sorted descending, cut a bound on every key it dropped: each lane it did
// not keep has a raw key <= cut (0: the part kept every lane).  When a
// prompt row is scored, `above` counts the part's lanes whose raw logit
// exceeds the target's and `next_above` is the smallest such logit (+inf
// if none).  Stored at records[row * units + i] for the row's i-th part.
struct PartRecord {
  float m;
  float s;
  int32_t above;     // scoring only (0 otherwise)
  float next_above;  // scoring only
  uint64_t cut;
  uint64_t keys[kKeep];
};
static_assert(sizeof(PartRecord) == 280, "record layout");

// Vocabulary sharding (one GPU standing in for tensor-parallel ranks): shard
// r of `shards` owns vocabulary lanes [shard_lo(r), shard_lo(r + 1)), its
// boundaries rounded up to multiples of 8 lanes so that every shard's first
// lane is 16-byte aligned in bf16 and FP32 rows.
constexpr int kShardAlign = 8;
constexpr int kMaxShards = 32;
inline __host__ __device__ int shard_lo(int r, int V, int shards) {
  if (r >= shards) return V;
  const int64_t b = ((int64_t)r * V / shards + kShardAlign - 1) / kShardAlign * kShardAlign;
  return b < V ? (int)b : V;
}

// The record one shard would exchange per reduced position: its max and its
// exponential sum relative to it, the chosen token's raw logit when it owns
// the token, and either its best 32 raw keys (global token IDs) with a cut
// bounding every key it dropped, or the raw logits of the selected IDs it
// owns.  552 bytes.
struct ShardRecord {
  float m;
  float s;
  float chosen;      // raw logit of the chosen token (flags bit 0)
  int32_t flags;     // bit 0: this shard owns the chosen token
  uint64_t cut;      // every lane the shard dropped has a raw key <= cut (0: none)
  union {
    uint64_t keys[kKeep];  // natural: best raw keys, sorted descending
    float sel[128];        // selected: raw logit of ids[j] when owned
  };
  uint32_t owned[4];       // selected: bit j set iff this shard owns ids[j]
};
static_assert(sizeof(ShardRecord) == 552, "shard record layout");

struct Params {
  const void* logits;
  const int32_t* requested;
  const int32_t* id_counts;
  const int32_t* ids;
  const int32_t* emitted;
  const int32_t* tokens;
  int32_t* out;
  PartRecord* records;
  float* lse;
  int32_t* guard;       // [rows]: parts the merge read again (diagnostic)
  int32_t* slot_rows;   // [capacity + 1]: active rows before each slot, then their total
  float* xtok;          // [rows]: chosen raw logits captured by the reduction
  const int64_t* crecords;     // completion records [capacity, 16 + T] (or null): emitted
                               // count at field emitted_field, tokens at fields 16 + t
  int32_t emitted_field;
  int32_t row_words;           // output words per position: 258, or 2 + 2K without ID inputs
  const int32_t* row_offsets;  // packed target rows: logit row of (s, t) is row_offsets[s] + t
  int32_t packed_rows;         // rows of a packed logits buffer (0: rectangular, row s T + t)
  int64_t V_pad;
  int32_t capacity;
  int32_t T;
  int32_t V;
  int32_t K;
  int32_t units;    // units per row
  int32_t workers;  // workgroups of the persistent launch (one unit range each)
  // Vocabulary sharding: 0 shards for an unsharded call.  A shard pass runs
  // the reduction on shard `shard` (logits, V and units of that slice; token
  // IDs local to it) and the finalize writes xrec[row * shards + shard]; the
  // cross-shard merge takes the whole rows and the gathered records.
  int32_t shards;
  int32_t shard;
  int32_t shard_base;   // first vocabulary lane of `shard`
  int32_t full_V;       // the unsharded vocabulary
  ShardRecord* xrec;
};

// Launches of one call; `phases` is a mask of kPhaseReduce and kPhaseMerge.
constexpr int kPhaseReduce = 1;
constexpr int kPhaseMerge = 2;
// Launcher implemented in flp_kernels.hip; returns a hipError_t as int.
// `score` selects prompt scoring: one row per slot (T = 1), a row is active
// when its target (tokens[s]) is a vocabulary ID, K = 20, kPromptWords per row.
int launch(const Params& p, int dtype, bool vector_rows, bool score, int phases, void* stream);
// The static device scratch of flare_logprobs_run_noalloc: its size, and its
// address on `device` (the current device), looked up once per device.
constexpr uint64_t kScratchBytes = 16ull << 20;
constexpr int kMaxDevices = 64;
int scratch_address(int device, void** ptr);
// Shard pass tail and cross-shard merge (flp_kernels.hip); hipError_t as int.
int launch_shard_finalize(const Params& p, int dtype, void* stream);
int launch_shard_merge(const Params& p, int dtype, bool vector_rows, void* stream);
// Resident reduction workgroups per CU (0 on error).
int reduce_occupancy(int dtype, bool vector_rows, bool score, int capacity, bool packed);
// Dynamic LDS of the reduction: the slot table, and each slot's packed row offset (packed
// launches) or scored target (scoring: callers pass packed = true).
size_t prefix_lds_bytes(int capacity, bool packed);

}  // namespace flp

// Host side of the C ABI: argument validation, planning, workspace layout and
// launch.  Nothing here allocates device memory, synchronizes or compiles.
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../include/flare_logprobs.h"
#include "flp_internal.h"

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
// The chosen (or scored target) raw logits a reduction captures for its
// merge: float[capacity * T] after the guard counts.
uint64_t chosen_offset(const flare_logprobs_plan_t* plan) {
  return plan->guard_offset + align_up((uint64_t)plan->capacity * plan->T * sizeof(int32_t), kAlign);
}

bool geometry_ok(int32_t capacity, int32_t T, int32_t V, int32_t V_pad, int32_t K) {
  if (capacity < 1 || T < 1 || V < 1 || V_pad < V) return false;
  if (K < 0 || K > FLARE_LOGPROBS_MAX_K) return false;
  return true;
}

}  // namespace

extern "C" {

uint32_t flare_logprobs_abi_version(void) { return FLARE_LOGPROBS_ABI_VERSION; }

const char* flare_status_string(int status) {
  switch (status) {
    case FLARE_OK: return "ok";
    case FLARE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FLARE_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case FLARE_ERR_PLAN_MISMATCH: return "arguments do not match the plan";
    case FLARE_ERR_DEVICE: return "device query failed or device is not gfx950";
    case FLARE_ERR_LAUNCH: return "kernel launch failed";
    case FLARE_ERR_UNSUPPORTED_SIZE: return "vocabulary too large for the plan";
    case FLARE_ERR_SCRATCH_TOO_SMALL:
      return "the plan's workspace exceeds the 16 MiB static scratch of the no-allocation call";
    default: return "unknown status";
  }
}

}  // extern "C"

// Both plans: a generation frame (mode 0) or a scored prompt chunk (mode 1,
// capacity = rows, T = 1, K = 20).
static int make_plan(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T, int32_t V,
                     int32_t V_pad, int32_t dtype, int32_t K, int32_t device, int32_t mode,
                     int32_t packed_rows) {
  if (!plan) return FLARE_ERR_INVALID_ARGUMENT;
  memset(plan, 0, sizeof *plan);
  if (dtype != FLARE_DTYPE_FP32 && dtype != FLARE_DTYPE_BF16) return FLARE_ERR_UNSUPPORTED_DTYPE;
  if (!geometry_ok(capacity, T, V, V_pad, K)) return FLARE_ERR_INVALID_ARGUMENT;
  if (capacity > flp::kMaxCapacity) return FLARE_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)capacity * T;
  if (rows > (int64_t)1 << 30) return FLARE_ERR_INVALID_ARGUMENT;
  if (packed_rows < 0 || packed_rows > (1 << 30)) return FLARE_ERR_INVALID_ARGUMENT;
  const int unit = flp::unit_elems(dtype);
  const int64_t units = ((int64_t)V + unit - 1) / unit;
  if (units > flp::kMaxUnits) return FLARE_ERR_UNSUPPORTED_SIZE;
  if (rows * units > (int64_t)0x7FFFFFFF) return FLARE_ERR_UNSUPPORTED_SIZE;
  const bool vec = ((int64_t)V_pad * flp::elem_bytes(dtype)) % 16 == 0;
  // Row byte offsets inside a buffer resource are 32-bit.
  if ((int64_t)V_pad * flp::elem_bytes(dtype) > (int64_t)0x7FFFFFFF) return FLARE_ERR_UNSUPPORTED_SIZE;

  int32_t cus = 256, per_cu = 4;
  if (device >= 0) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return FLARE_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return FLARE_ERR_DEVICE;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return FLARE_ERR_DEVICE;
    cus = prop.multiProcessorCount;
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return FLARE_ERR_DEVICE;
    if (prev != device && hipSetDevice(device) != hipSuccess) return FLARE_ERR_DEVICE;
    per_cu = flp::reduce_occupancy(dtype, vec, mode == FLARE_MODE_PROMPT, capacity, packed_rows > 0);
    if (prev != device && hipSetDevice(prev) != hipSuccess) return FLARE_ERR_DEVICE;
    if (per_cu < 1) return FLARE_ERR_DEVICE;
  }

  plan->abi_version = FLARE_LOGPROBS_ABI_VERSION;
  plan->capacity = capacity;
  plan->T = T;
  plan->V = V;
  plan->V_pad = V_pad;
  plan->dtype = dtype;
  plan->K = K;
  plan->device = device;
  plan->unit_elems = unit;
  plan->units = (int32_t)units;
  plan->block = flp::kBlock;
  plan->grid = cus * per_cu;
  plan->vector_rows = vec ? 1 : 0;
  plan->cu_count = cus;
  plan->ranges = plan->grid;
  plan->mode = mode;
  plan->packed_rows = packed_rows;
  if (mode == FLARE_MODE_PROMPT) {
    // A unit range holds at most ceil(N / grid) units, so it touches at most
    // ceil((ceil(N / grid) - 1) / units) + 1 rows.
    const int64_t n = rows * units;
    const int64_t per = (n + plan->grid - 1) / plan->grid;
    if ((per - 1 + units - 1) / units + 1 > flp::kMaxRangeRows) {
      memset(plan, 0, sizeof *plan);
      return FLARE_ERR_UNSUPPORTED_SIZE;
    }
  }
  uint64_t off = 0;
  plan->record_offset = off;
  off = align_up(off + (uint64_t)rows * units * sizeof(flp::PartRecord), kAlign);
  plan->lse_offset = off;
  off = align_up(off + (uint64_t)rows * sizeof(float), kAlign);
  plan->slots_offset = off;
  off = align_up(off + ((uint64_t)capacity + 1) * sizeof(int32_t), kAlign);
  plan->guard_offset = off;
  off = align_up(off + (uint64_t)rows * sizeof(int32_t), kAlign);
  off = align_up(off + (uint64_t)rows * sizeof(float), kAlign);  // chosen raw logits
  plan->workspace_bytes = off;
  return FLARE_OK;
}

extern "C" {

int flare_logprobs_plan_sharded(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T,
                                int32_t V, int32_t V_pad, int32_t dtype, int32_t K,
                                int32_t shards, int32_t device) {
  if (!plan) return FLARE_ERR_INVALID_ARGUMENT;
  memset(plan, 0, sizeof *plan);
  if (shards < 1 || shards > flp::kMaxShards || V < 1) return FLARE_ERR_INVALID_ARGUMENT;
  for (int r = 0; r < shards; ++r)
    if (flp::shard_lo(r + 1, V, shards) <= flp::shard_lo(r, V, shards)) return FLARE_ERR_INVALID_ARGUMENT;
  const int rc = make_plan(plan, capacity, T, V, V_pad, dtype, K, device, FLARE_MODE_GENERATION, 0);
  if (rc != FLARE_OK) return rc;
  // Part records sized for the widest shard (the shard passes reuse them in
  // turn); then the gathered exchange records [rows, shards].
  const int unit = flp::unit_elems(dtype);
  int32_t units = 0;
  for (int r = 0; r < shards; ++r) {
    const int w = flp::shard_lo(r + 1, V, shards) - flp::shard_lo(r, V, shards);
    const int32_t u = (w + unit - 1) / unit;
    units = u > units ? u : units;
  }
  const uint64_t rows = (uint64_t)capacity * T;
  plan->units = units;
  plan->shards = shards;
  uint64_t off = plan->workspace_bytes;
  plan->exchange_offset = off;
  off = align_up(off + rows * shards * sizeof(flp::ShardRecord), kAlign);
  plan->workspace_bytes = off;
  return FLARE_OK;
}

int flare_logprobs_plan(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T, int32_t V,
                        int32_t V_pad, int32_t dtype, int32_t K, int32_t device) {
  return make_plan(plan, capacity, T, V, V_pad, dtype, K, device, FLARE_MODE_GENERATION, 0);
}

int flare_logprobs_plan_packed(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T,
                               int32_t packed_rows, int32_t V, int32_t V_pad, int32_t dtype,
                               int32_t K, int32_t device) {
  if (packed_rows < 1) {
    if (plan) memset(plan, 0, sizeof *plan);
    return FLARE_ERR_INVALID_ARGUMENT;
  }
  return make_plan(plan, capacity, T, V, V_pad, dtype, K, device, FLARE_MODE_GENERATION,
                   packed_rows);
}

int flare_prompt_logprobs_plan(flare_logprobs_plan_t* plan, int32_t rows, int32_t V,
                               int32_t V_pad, int32_t dtype, int32_t device) {
  return make_plan(plan, rows, 1, V, V_pad, dtype, FLARE_PROMPT_ALTERNATIVES, device,
                   FLARE_MODE_PROMPT, 0);
}

}  // extern "C"

// The `shard` argument of run_phases: an unsharded call, every shard pass then
// the cross-shard merge, the merge alone, or (>= 0) one shard's pass.
constexpr int32_t kNoShard = -1;
constexpr int32_t kAllShards = -2;
constexpr int32_t kShardMerge = -3;

// Validate one call's arguments against its plan and launch `phases`.
static int run_phases(const flare_logprobs_plan_t* plan, const void* logits, int32_t dtype,
                      int64_t rows, int32_t V, int32_t V_pad, const int32_t* requested,
                      const int32_t* id_counts, const int32_t* ids,
                      const int32_t* emitted_counts, const int32_t* tokens,
                      const int32_t* row_offsets, int32_t K, int32_t* out, void* workspace,
                      void* hip_stream, int phases, const int64_t* records = nullptr,
                      int32_t emitted_field = 0, int32_t row_words = FLARE_LOGPROBS_ROW_WORDS,
                      int32_t shard = kNoShard) {
  // Completion records replace emitted_counts and tokens; a frame without ID
  // inputs (both null) is natural-only with rows of 2 + 2K words.
  const bool rec = records != nullptr;
  if (!plan || !logits || !requested || !out || !workspace) return FLARE_ERR_INVALID_ARGUMENT;
  if (!rec && (!emitted_counts || !tokens || !id_counts || !ids)) return FLARE_ERR_INVALID_ARGUMENT;
  if ((id_counts == nullptr) != (ids == nullptr)) return FLARE_ERR_INVALID_ARGUMENT;
  if (rec && (emitted_field < 0 || emitted_field >= flp::kRecordMeta)) return FLARE_ERR_INVALID_ARGUMENT;
  if (row_words != FLARE_LOGPROBS_ROW_WORDS) {
    // The compact extent: only without ID inputs, 2 + 2K words, 1 <= K <= 20.
    if (id_counts || K < 1 || row_words != 2 + 2 * K) return FLARE_ERR_INVALID_ARGUMENT;
  }
  // A packed plan takes its row offsets and P logit rows; a rectangular one neither.
  if ((plan->packed_rows > 0) != (row_offsets != nullptr)) return FLARE_ERR_PLAN_MISMATCH;
  if (plan->abi_version != FLARE_LOGPROBS_ABI_VERSION) return FLARE_ERR_PLAN_MISMATCH;
  if (plan->mode != FLARE_MODE_GENERATION) return FLARE_ERR_PLAN_MISMATCH;
  if ((plan->shards > 0) != (shard != kNoShard)) return FLARE_ERR_PLAN_MISMATCH;
  if (dtype != FLARE_DTYPE_FP32 && dtype != FLARE_DTYPE_BF16) return FLARE_ERR_UNSUPPORTED_DTYPE;
  if (dtype != plan->dtype || V != plan->V || V_pad != plan->V_pad || K != plan->K)
    return FLARE_ERR_PLAN_MISMATCH;
  if (rows != (plan->packed_rows > 0 ? (int64_t)plan->packed_rows
                                      : (int64_t)plan->capacity * plan->T))
    return FLARE_ERR_PLAN_MISMATCH;
  if (plan->grid < 1 || plan->units < 1 || plan->units > flp::kMaxUnits ||
      plan->ranges != plan->grid || plan->block != flp::kBlock || plan->packed_rows < 0)
    return FLARE_ERR_PLAN_MISMATCH;
  if (((uintptr_t)workspace & 15u) != 0) return FLARE_ERR_INVALID_ARGUMENT;

  char* ws = (char*)workspace;
  flp::Params p;
  p.logits = logits;
  p.crecords = records;
  p.emitted_field = emitted_field;
  p.row_words = row_words;
  p.row_offsets = plan->packed_rows > 0 ? row_offsets : nullptr;
  p.packed_rows = plan->packed_rows;
  p.requested = requested;
  p.id_counts = id_counts;
  p.ids = ids;
  p.emitted = emitted_counts;
  p.tokens = tokens;
  p.out = out;
  p.records = (flp::PartRecord*)(ws + plan->record_offset);
  p.lse = (float*)(ws + plan->lse_offset);
  p.guard = (int32_t*)(ws + plan->guard_offset);
  p.xtok = (float*)(ws + chosen_offset(plan));
  p.slot_rows = (int32_t*)(ws + plan->slots_offset);
  p.V_pad = V_pad;
  p.capacity = plan->capacity;
  p.T = plan->T;
  p.V = V;
  p.K = K;
  p.units = plan->units;
  p.workers = plan->ranges;

  p.shards = 0;
  p.shard = 0;
  p.shard_base = 0;
  p.full_V = V;
  p.xrec = nullptr;

  const bool vec = plan->vector_rows && (((uintptr_t)logits & 15u) == 0);
  if (shard == kNoShard) {
    const int e = flp::launch(p, dtype, vec, false, phases, hip_stream);
    return e == 0 ? FLARE_OK : FLARE_ERR_LAUNCH;
  }
  // Vocabulary shards: a shard pass (the reduction on the shard's columns,
  // then its exchange records), or the cross-shard merge.
  p.shards = plan->shards;
  p.xrec = (flp::ShardRecord*)(ws + plan->exchange_offset);
  auto pass = [&](int r) -> int {
    flp::Params q = p;
    const int lo = flp::shard_lo(r, V, plan->shards), hi = flp::shard_lo(r + 1, V, plan->shards);
    q.shard = r;
    q.shard_base = lo;
    q.logits = (const char*)logits + (int64_t)lo * flp::elem_bytes(dtype);
    q.V = hi - lo;
    q.units = (q.V + flp::unit_elems(dtype) - 1) / flp::unit_elems(dtype);
    const bool qvec = plan->vector_rows && (((uintptr_t)q.logits & 15u) == 0);
    int e = flp::launch(q, dtype, qvec, false, flp::kPhaseReduce, hip_stream);
    if (e == 0) e = flp::launch_shard_finalize(q, dtype, hip_stream);
    return e;
  };
  int e = 0;
  if (shard >= 0) {
    e = pass(shard);
  } else {
    if (shard == kAllShards)
      for (int r = 0; r < plan->shards && e == 0; ++r) e = pass(r);
    if (e == 0) e = flp::launch_shard_merge(p, dtype, vec, hip_stream);
  }
  return e == 0 ? FLARE_OK : FLARE_ERR_LAUNCH;
}

// The same for a scored prompt chunk.
static int prompt_phases(const flare_logprobs_plan_t* plan, const void* logits, int32_t dtype,
                         int64_t rows, int32_t V, int32_t V_pad, const int32_t* targets,
                         int32_t* out, void* workspace, void* hip_stream, int phases) {
  if (!plan || !logits || !targets || !out || !workspace) return FLARE_ERR_INVALID_ARGUMENT;
  if (plan->abi_version != FLARE_LOGPROBS_ABI_VERSION) return FLARE_ERR_PLAN_MISMATCH;
  if (plan->mode != FLARE_MODE_PROMPT || plan->shards != 0) return FLARE_ERR_PLAN_MISMATCH;
  if (dtype != FLARE_DTYPE_FP32 && dtype != FLARE_DTYPE_BF16) return FLARE_ERR_UNSUPPORTED_DTYPE;
  if (dtype != plan->dtype || V != plan->V || V_pad != plan->V_pad) return FLARE_ERR_PLAN_MISMATCH;
  if (rows != (int64_t)plan->capacity || plan->T != 1 || plan->K != FLARE_PROMPT_ALTERNATIVES ||
      plan->packed_rows != 0)
    return FLARE_ERR_PLAN_MISMATCH;
  if (plan->grid < 1 || plan->units < 1 || plan->units > flp::kMaxUnits ||
      plan->ranges != plan->grid || plan->block != flp::kBlock)
    return FLARE_ERR_PLAN_MISMATCH;
  {
    const int64_t per = (rows * plan->units + plan->grid - 1) / plan->grid;
    if ((per - 1 + plan->units - 1) / plan->units + 1 > flp::kMaxRangeRows)
      return FLARE_ERR_PLAN_MISMATCH;
  }
  if (((uintptr_t)workspace & 15u) != 0) return FLARE_ERR_INVALID_ARGUMENT;

  char* ws = (char*)workspace;
  flp::Params p;
  p.logits = logits;
  p.crecords = nullptr;
  p.emitted_field = 0;
  p.row_words = FLARE_PROMPT_ROW_WORDS;
  p.row_offsets = nullptr;
  p.packed_rows = 0;
  p.requested = nullptr;
  p.id_counts = nullptr;
  p.ids = nullptr;
  p.emitted = nullptr;
  p.tokens = targets;
  p.out = out;
  p.records = (flp::PartRecord*)(ws + plan->record_offset);
  p.lse = (float*)(ws + plan->lse_offset);
  p.guard = (int32_t*)(ws + plan->guard_offset);
  p.xtok = (float*)(ws + chosen_offset(plan));
  p.slot_rows = (int32_t*)(ws + plan->slots_offset);
  p.V_pad = V_pad;
  p.capacity = plan->capacity;
  p.T = 1;
  p.V = V;
  p.K = FLARE_PROMPT_ALTERNATIVES;
  p.units = plan->units;
  p.workers = plan->ranges;
  p.shards = 0;
  p.shard = 0;
  p.shard_base = 0;
  p.full_V = V;
  p.xrec = nullptr;

  const bool vec = plan->vector_rows && (((uintptr_t)logits & 15u) == 0);
  const int e = flp::launch(p, dtype, vec, true, phases, hip_stream);
  return e == 0 ? FLARE_OK : FLARE_ERR_LAUNCH;
}

extern "C" {

int flare_logprobs_run(const flare_logprobs_plan_t* plan, const void* logits, int32_t dtype,
                       int64_t rows, int32_t V, int32_t V_pad, const int32_t* requested,
                       const int32_t* id_counts, const int32_t* ids,
                       const int32_t* emitted_counts, const int32_t* tokens, int32_t K,
                       int32_t* out, void* workspace, void* hip_stream) {
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, workspace, hip_stream,
                    flp::kPhaseReduce | flp::kPhaseMerge);
}

int flare_logprobs_run_packed(const flare_logprobs_plan_t* plan, const void* logits,
                              int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                              const int32_t* requested, const int32_t* id_counts,
                              const int32_t* ids, const int32_t* emitted_counts,
                              const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                              int32_t* out, void* workspace, void* hip_stream) {
  if (!row_offsets) return FLARE_ERR_INVALID_ARGUMENT;
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, row_offsets, K, out, workspace, hip_stream,
                    flp::kPhaseReduce | flp::kPhaseMerge);
}

int flare_logprobs_run_records(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int64_t* records, int32_t emitted_field,
                               int32_t K, int32_t* out, int32_t out_row_words, void* workspace,
                               void* hip_stream) {
  if (!records) return FLARE_ERR_INVALID_ARGUMENT;
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids, nullptr,
                    nullptr, nullptr, K, out, workspace, hip_stream,
                    flp::kPhaseReduce | flp::kPhaseMerge, records, emitted_field,
                    out_row_words);
}

int flare_logprobs_reduce_packed(const flare_logprobs_plan_t* plan, const void* logits,
                                 int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                 const int32_t* requested, const int32_t* id_counts,
                                 const int32_t* ids, const int32_t* emitted_counts,
                                 const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                                 int32_t* out, void* workspace, void* hip_stream) {
  if (!row_offsets) return FLARE_ERR_INVALID_ARGUMENT;
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, row_offsets, K, out, workspace, hip_stream,
                    flp::kPhaseReduce);
}

int flare_logprobs_merge_packed(const flare_logprobs_plan_t* plan, const void* logits,
                                int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                const int32_t* requested, const int32_t* id_counts,
                                const int32_t* ids, const int32_t* emitted_counts,
                                const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                                int32_t* out, void* workspace, void* hip_stream) {
  if (!row_offsets) return FLARE_ERR_INVALID_ARGUMENT;
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, row_offsets, K, out, workspace, hip_stream,
                    flp::kPhaseMerge);
}

int flare_logprobs_reduce(const flare_logprobs_plan_t* plan, const void* logits, int32_t dtype,
                          int64_t rows, int32_t V, int32_t V_pad, const int32_t* requested,
                          const int32_t* id_counts, const int32_t* ids,
                          const int32_t* emitted_counts, const int32_t* tokens, int32_t K,
                          int32_t* out, void* workspace, void* hip_stream) {
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, workspace, hip_stream, flp::kPhaseReduce);
}

int flare_logprobs_merge(const flare_logprobs_plan_t* plan, const void* logits, int32_t dtype,
                         int64_t rows, int32_t V, int32_t V_pad, const int32_t* requested,
                         const int32_t* id_counts, const int32_t* ids,
                         const int32_t* emitted_counts, const int32_t* tokens, int32_t K,
                         int32_t* out, void* workspace, void* hip_stream) {
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, workspace, hip_stream, flp::kPhaseMerge);
}

int flare_logprobs_run_noalloc(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int32_t* emitted_counts,
                               const int32_t* tokens, int32_t K, int32_t* out, void* hip_stream) {
  if (!plan) return FLARE_ERR_INVALID_ARGUMENT;
  if (plan->workspace_bytes > flp::kScratchBytes) return FLARE_ERR_SCRATCH_TOO_SMALL;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return FLARE_ERR_DEVICE;
  void* ws = nullptr;
  if (flp::scratch_address(device, &ws) != 0 || !ws) return FLARE_ERR_DEVICE;
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, ws, hip_stream,
                    flp::kPhaseReduce | flp::kPhaseMerge);
}

int flare_logprobs_run_sharded(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int32_t* emitted_counts,
                               const int32_t* tokens, int32_t K, int32_t* out, void* workspace,
                               void* hip_stream) {
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, workspace, hip_stream,
                    flp::kPhaseReduce | flp::kPhaseMerge, nullptr, 0, FLARE_LOGPROBS_ROW_WORDS,
                    kAllShards);
}

int flare_logprobs_shard_pass(const flare_logprobs_plan_t* plan, int32_t shard,
                              const void* logits, int32_t dtype, int64_t rows, int32_t V,
                              int32_t V_pad, const int32_t* requested, const int32_t* id_counts,
                              const int32_t* ids, const int32_t* emitted_counts,
                              const int32_t* tokens, int32_t K, int32_t* out, void* workspace,
                              void* hip_stream) {
  if (!plan || shard < 0 || shard >= plan->shards) return FLARE_ERR_INVALID_ARGUMENT;
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, workspace, hip_stream,
                    flp::kPhaseReduce, nullptr, 0, FLARE_LOGPROBS_ROW_WORDS, shard);
}

int flare_logprobs_shard_merge(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int32_t* emitted_counts,
                               const int32_t* tokens, int32_t K, int32_t* out, void* workspace,
                               void* hip_stream) {
  return run_phases(plan, logits, dtype, rows, V, V_pad, requested, id_counts, ids,
                    emitted_counts, tokens, nullptr, K, out, workspace, hip_stream,
                    flp::kPhaseMerge, nullptr, 0, FLARE_LOGPROBS_ROW_WORDS, kShardMerge);
}

int flare_prompt_logprobs_run(const flare_logprobs_plan_t* plan, const void* logits,
                              int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                              const int32_t* targets, int32_t* out, void* workspace,
                              void* hip_stream) {
  return prompt_phases(plan, logits, dtype, rows, V, V_pad, targets, out, workspace, hip_stream,
                       flp::kPhaseReduce | flp::kPhaseMerge);
}

int flare_prompt_logprobs_reduce(const flare_logprobs_plan_t* plan, const void* logits,
                                 int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                 const int32_t* targets, int32_t* out, void* workspace,
                                 void* hip_stream) {
  return prompt_phases(plan, logits, dtype, rows, V, V_pad, targets, out, workspace, hip_stream,
                       flp::kPhaseReduce);
}

int flare_prompt_logprobs_merge(const flare_logprobs_plan_t* plan, const void* logits,
                                int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                const int32_t* targets, int32_t* out, void* workspace,
                                void* hip_stream) {
  return prompt_phases(plan, logits, dtype, rows, V, V_pad, targets, out, workspace, hip_stream,
                       flp::kPhaseMerge);
}

}  // extern "C"

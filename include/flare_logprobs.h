/*
 * flare_logprobs.h -- C ABI of the MI355X (gfx950) generation-logprob
 * reduction.
 *
 * The operation (Flare generation-logprobs design page, definition paragraph
 * and tiled-reduction paragraph): for every emitted verify position of a
 * requesting slot, report
 *     lp(i) = fl32( x[i] - L ),   L = FP32 logsumexp of x over lanes [0, V),
 * where x is the raw target-logit row, before any sampling transform.  The
 * chosen token's pair is always written; then either the K natural
 * alternatives (decreasing lp, then increasing token ID, -0 reported as +0,
 * padded lanes [V, V_pad) never taking part) or the slot's selected IDs in
 * caller order with the same L.
 *
 * Output layout (design page, buffer table and packed-position paragraph):
 * one frame int32 [capacity, T, 258]; position (s, t) holds
 *     [chosen_id, chosen_bits, id_0, bits_0, ..., id_127, bits_127]
 * where bits are the FP32 value's bit pattern.  Only words [0, 2 + 2W) of
 * active positions are written, W = K (natural) or the slot's ID count
 * (selected).  When V < K the unused natural pairs are (-1, 0x7FC00000).
 *
 * Gating (design page, gating and zero-flag paragraphs; MTP design page,
 * round section):  position (s, t) is active iff requested[s] != 0 and
 * 0 <= t < min(max(emitted_counts[s], 0), T).  Inactive positions read no
 * logits and write nothing.  Logit row (s, t) is row s*T + t.
 *
 * Defined behaviour for device data that cannot be checked without a sync:
 * emitted counts are clamped to [0, T]; ID counts to [0, 128]; a zero flag
 * wins over a nonzero count; a chosen or selected ID outside [0, V) is
 * written as given with bits 0x7FC00000 and never dereferenced.  NaN or +inf
 * in lanes [0, V) and rows whose every lane is -inf are outside the contract.
 *
 * Threading and memory: every device buffer is owned by the caller.  The
 * library keeps no pointer after a call returns and never allocates, frees,
 * synchronizes or compiles at run time, and records no memset, so
 * flare_logprobs_run may be captured in a HIP graph.  Calls on one stream are ordered; concurrent calls need
 * distinct workspaces.  The inputs are only read.
 */
#ifndef FLARE_LOGPROBS_H
#define FLARE_LOGPROBS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLARE_LOGPROBS_ABI_VERSION 6u
#define FLARE_LOGPROBS_MAX_K 20
#define FLARE_LOGPROBS_MAX_IDS 128
#define FLARE_LOGPROBS_ROW_WORDS 258 /* 2 + 2 * 128 */
#define FLARE_LOGPROBS_NAN_BITS 0x7FC00000u
#define FLARE_PROMPT_ROW_WORDS 43     /* 3 + 2 * 20 */
#define FLARE_PROMPT_ALTERNATIVES 20

enum flare_mode {
  FLARE_MODE_GENERATION = 0, /* flare_logprobs_plan: emitted verify positions */
  FLARE_MODE_PROMPT = 1      /* flare_prompt_logprobs_plan: scored prompt rows */
};

enum flare_dtype {
  FLARE_DTYPE_FP32 = 0, /* IEEE binary32 logits */
  FLARE_DTYPE_BF16 = 1  /* bfloat16 logits, widened exactly to FP32 */
};

enum flare_status {
  FLARE_OK = 0,
  FLARE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad geometry or K */
  FLARE_ERR_UNSUPPORTED_DTYPE = 2,
  FLARE_ERR_PLAN_MISMATCH = 3,    /* run arguments differ from the plan */
  FLARE_ERR_DEVICE = 4,           /* device query failed or not gfx950 */
  FLARE_ERR_LAUNCH = 5,           /* a kernel launch reported an error */
  FLARE_ERR_UNSUPPORTED_SIZE = 6, /* V beyond what the plan can tile */
  FLARE_ERR_SCRATCH_TOO_SMALL = 7 /* flare_logprobs_run_noalloc: workspace_bytes > 16 MiB */
};

/*
 * A plan is a host value filled by flare_logprobs_plan.  It owns nothing and
 * needs no destruction.  Fields after `device` are chosen by the library and
 * are informational, except workspace_bytes, which the caller must allocate.
 * flare_logprobs_run rejects a plan whose fields were altered.
 */
typedef struct flare_logprobs_plan {
  uint32_t abi_version;
  int32_t capacity;      /* padded physical slot capacity */
  int32_t T;             /* verify rows per slot (k drafts + 1) */
  int32_t V;             /* vocabulary lanes that count */
  int32_t V_pad;         /* row stride in elements, V_pad >= V */
  int32_t dtype;         /* enum flare_dtype */
  int32_t K;             /* natural alternatives, 0..20 */
  int32_t device;        /* HIP device ordinal, or -1 for a host-only plan */
  int32_t unit_elems;    /* vocabulary lanes one workgroup holds at a time */
  int32_t units;         /* units per row, ceil(V / unit_elems), at most 64 */
  int32_t block;         /* threads per reduction workgroup */
  int32_t grid;          /* reduction workgroups of the persistent launch */
  int32_t vector_rows;   /* 1 if V_pad * element size is a multiple of 16 */
  int32_t cu_count;      /* compute units of `device` (256 if host-only) */
  int32_t ranges;        /* contiguous unit ranges of the launch (== grid) */
  int32_t mode;          /* enum flare_mode: which run entry points accept it */
  uint64_t workspace_bytes; /* bytes of device workspace the caller provides */
  uint64_t record_offset;   /* part records: units slots per row, part i in slot i */
  uint64_t lse_offset;      /* float[capacity * T]: L of each reduced row */
  uint64_t slots_offset;    /* int32[capacity + 1]: active rows before each slot, then all */
  uint64_t guard_offset;    /* int32[capacity * T]: parts of each reduced row that the
                               merge read again (diagnostic, see flare_logprobs_run) */
  int32_t packed_rows;      /* P of flare_logprobs_plan_packed; 0 for the rectangular layout */
  int32_t shards;           /* vocabulary shards of flare_logprobs_plan_sharded; 0 otherwise */
  uint64_t exchange_offset; /* sharded plans: the gathered shard records [rows, shards] */
  uint32_t reserved[2];
} flare_logprobs_plan_t;

/*
 * Validate a geometry and size a workspace.  Runs on the host only; with
 * device >= 0 it reads that device's attributes (CU count, architecture,
 * resident workgroups per CU) to size the persistent launch.
 *   1 <= capacity <= 8192, T >= 1, V >= 1, V_pad >= V, dtype a flare_dtype,
 *   0 <= K <= 20; V at most 64 units (1,048,576 bf16 or 524,288 FP32 lanes),
 *   else FLARE_ERR_UNSUPPORTED_SIZE.
 * Returns FLARE_OK and fills *plan, or an error and leaves *plan zeroed.
 */
int flare_logprobs_plan(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T,
                        int32_t V, int32_t V_pad, int32_t dtype, int32_t K,
                        int32_t device);

/*
 * Reduce one frame, asynchronously on `hip_stream` (a hipStream_t; NULL is
 * the null stream) of the current device.
 *   logits          device, [rows, V_pad] of `dtype`, row-major, read only
 *   dtype, V, V_pad, K   must equal the plan's (FLARE_ERR_PLAN_MISMATCH)
 *   rows            number of logit rows; must equal capacity * T
 *   requested       device int32 [capacity]: nonzero = slot requests logprobs
 *   id_counts       device int32 [capacity]: 0 = natural mode, n > 0 = n IDs
 *   ids             device int32 [capacity, 128]: selected IDs, caller order
 *   emitted_counts  device int32 [capacity]: committed prefix length per slot
 *   tokens          device int32 [capacity, T]: chosen token of each position
 *   out             device int32 [capacity, T, 258]: one output frame
 *   workspace       device, plan->workspace_bytes, 16-byte aligned; needs no
 *                   initialisation (every word whose value is used is written
 *                   first in the same call)
 * Two kernels run in order on the stream: the reduction, then the per-row
 * merge.  Host-checkable errors return before anything is launched.
 * Diagnostics left in the workspace for each active position (other entries
 * hold stale values): its L at lse_offset, and at guard_offset the number of
 * its parts that the merge's exactness guard streamed again because their
 * kept candidates could not settle the top K.
 */
int flare_logprobs_run(const flare_logprobs_plan_t* plan, const void* logits,
                       int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                       const int32_t* requested, const int32_t* id_counts,
                       const int32_t* ids, const int32_t* emitted_counts,
                       const int32_t* tokens, int32_t K, int32_t* out,
                       void* workspace, void* hip_stream);

/*
 * Packed target rows (MTP design page, graph catalog paragraph: a verify
 * descriptor's physical target capacity P may be below B x W; generation
 * design page, gating paragraph: a packed request's columns past its
 * committed prefix may hold another request's rows and are never read).
 * The logits hold P rows; slot s's verify row t is logit row
 * row_offsets[s] + t.  Everything else (gating, the [capacity, T, 258]
 * output frame indexed by slot and position, tokens, IDs) is as for
 * flare_logprobs_run.
 *   flare_logprobs_plan_packed: as flare_logprobs_plan, plus 1 <= packed_rows
 *     <= 2^30 (else FLARE_ERR_INVALID_ARGUMENT); the plan records P.
 *   flare_logprobs_run_packed: run's arguments with rows == P and
 *     row_offsets a device int32 [capacity] (NULL: FLARE_ERR_INVALID_ARGUMENT).
 *     A slot whose committed rows [row_offsets[s], row_offsets[s] + e) leave
 *     [0, P) reads and writes nothing (e the clamped emitted count).
 * A packed plan is rejected by flare_logprobs_run (and its two launches) and
 * a rectangular plan by the _packed entry points (FLARE_ERR_PLAN_MISMATCH).
 * flare_logprobs_reduce_packed and flare_logprobs_merge_packed are the two
 * launches of flare_logprobs_run_packed, as for the rectangular layout.
 */
int flare_logprobs_plan_packed(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T,
                               int32_t packed_rows, int32_t V, int32_t V_pad, int32_t dtype,
                               int32_t K, int32_t device);
int flare_logprobs_run_packed(const flare_logprobs_plan_t* plan, const void* logits,
                              int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                              const int32_t* requested, const int32_t* id_counts,
                              const int32_t* ids, const int32_t* emitted_counts,
                              const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                              int32_t* out, void* workspace, void* hip_stream);
int flare_logprobs_reduce_packed(const flare_logprobs_plan_t* plan, const void* logits,
                                 int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                 const int32_t* requested, const int32_t* id_counts,
                                 const int32_t* ids, const int32_t* emitted_counts,
                                 const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                                 int32_t* out, void* workspace, void* hip_stream);
int flare_logprobs_merge_packed(const flare_logprobs_plan_t* plan, const void* logits,
                                int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                const int32_t* requested, const int32_t* id_counts,
                                const int32_t* ids, const int32_t* emitted_counts,
                                const int32_t* tokens, const int32_t* row_offsets, int32_t K,
                                int32_t* out, void* workspace, void* hip_stream);

/*
 * Adapter for the completion records and for cores without ID inputs
 * (generation design page, buffer table: completion_records int64
 * [2, capacity, 16 + T], one record per slot with 16 metadata fields, the
 * emitted count among them, then T token IDs; declaration paragraph: a core
 * without the ID inputs has rows of 2 + 2K words, 1 <= K <= 20, and serves
 * natural alternatives only; MTP design page, catalog paragraph).
 *   records        device int64 [capacity, 16 + T]: one frame of records.
 *                  Slot s's emitted count is field emitted_field (0..15; the
 *                  pages do not fix its index), its verify token t is field
 *                  16 + t.  A count outside [0, 2^31) reads as 0, a token
 *                  outside the int32 range as -1 (then written with NaN bits).
 *   id_counts, ids both NULL (no ID inputs: every slot natural) or both given.
 *   out_row_words  258, or 2 + 2K (only without ID inputs): out is
 *                  int32 [capacity, T, out_row_words].
 * Everything else is as for flare_logprobs_run (rectangular plans only; a
 * packed plan is FLARE_ERR_PLAN_MISMATCH).  Host-checkable errors
 * (FLARE_ERR_INVALID_ARGUMENT): records NULL, emitted_field outside [0, 16),
 * one ID input NULL and not the other, an extent other than 258 or 2 + 2K, or
 * 2 + 2K with ID inputs or K = 0.
 */
int flare_logprobs_run_records(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int64_t* records, int32_t emitted_field,
                               int32_t K, int32_t* out, int32_t out_row_words, void* workspace,
                               void* hip_stream);

/*
 * The two launches of flare_logprobs_run, for callers that want to order
 * other work between them or time them apart (design page, tiled-reduction
 * paragraph: the per-tile statistics and best-key launches, then the final
 * merge launch).  flare_logprobs_reduce streams the logits once and writes
 * each part's statistics and best raw keys to the workspace (and, when it has
 * a workgroup with no logits to stream for every 256 positions, the chosen
 * tokens' raw logits);
 * flare_logprobs_merge reads them and writes `out` (and each row's L).  Both
 * take run's arguments and validate them the same way; a merge must follow
 * its reduce on the same stream with the same arguments and workspace, and
 * nothing else may use that workspace in between.  Reduce then merge gives
 * the same frame, bit for bit, as one run.
 */
int flare_logprobs_reduce(const flare_logprobs_plan_t* plan, const void* logits,
                          int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                          const int32_t* requested, const int32_t* id_counts,
                          const int32_t* ids, const int32_t* emitted_counts,
                          const int32_t* tokens, int32_t K, int32_t* out,
                          void* workspace, void* hip_stream);
int flare_logprobs_merge(const flare_logprobs_plan_t* plan, const void* logits,
                         int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                         const int32_t* requested, const int32_t* id_counts,
                         const int32_t* ids, const int32_t* emitted_counts,
                         const int32_t* tokens, int32_t K, int32_t* out,
                         void* workspace, void* hip_stream);

/*
 * Prompt scoring (Flare generation-logprobs design page, prompt-logprobs
 * paragraphs: scored prefill).  For each of `rows` prompt positions, with
 * x the raw logit row and t = targets[r] the prompt token that follows it:
 *     out[r] = [t, bits(lp(t)), rank, id_0, bits_0, ..., id_19, bits_19]
 * where lp is the same fl32(x - L) as above, rank = 1 + the number of lanes
 * in [0, V) whose lp is strictly greater than lp(t) (equal values, ties the
 * subtraction creates included, do not count), and the twenty alternatives
 * follow the generation order (decreasing lp, then increasing ID; when V < 20
 * the unused pairs are (-1, 0x7FC00000)).  A row whose target is outside
 * [0, V) (-1 at the prompt end and inside image spans) reads no logits and is
 * written as [-1, 0x7FC00000, 0, then (-1, 0x7FC00000) twenty times].
 *
 * flare_prompt_logprobs_plan validates 1 <= rows <= 8192 and the other
 * geometry as flare_logprobs_plan does (its plan has capacity = rows, T = 1,
 * K = 20 and mode FLARE_MODE_PROMPT; FLARE_ERR_UNSUPPORTED_SIZE also when a
 * launch range would touch more than 64 rows, which needs far more rows than
 * a GPU's workgroups) and sizes its workspace.
 *   logits     device, [rows, V_pad] of `dtype`, row-major, read only
 *   rows, dtype, V, V_pad   must equal the plan's (FLARE_ERR_PLAN_MISMATCH)
 *   targets    device int32 [rows]
 *   out        device int32 [rows, 43]; every row is written
 *   workspace  device, plan->workspace_bytes, 16-byte aligned, no initialisation
 * Ownership, errors, streams and graph capture are as for flare_logprobs_run;
 * a plan of one mode is rejected by the other mode's entry points.  _reduce
 * and _merge are the two launches of _run, with the same contract as
 * flare_logprobs_reduce and flare_logprobs_merge.  The diagnostics are
 * those of flare_logprobs_run for valid rows; a row's guard_offset entry
 * counts the parts whose lanes were counted again because the subtraction
 * tied a larger logit with the target.
 */
int flare_prompt_logprobs_plan(flare_logprobs_plan_t* plan, int32_t rows, int32_t V,
                               int32_t V_pad, int32_t dtype, int32_t device);
int flare_prompt_logprobs_run(const flare_logprobs_plan_t* plan, const void* logits,
                              int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                              const int32_t* targets, int32_t* out, void* workspace,
                              void* hip_stream);
int flare_prompt_logprobs_reduce(const flare_logprobs_plan_t* plan, const void* logits,
                                 int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                 const int32_t* targets, int32_t* out, void* workspace,
                                 void* hip_stream);
int flare_prompt_logprobs_merge(const flare_logprobs_plan_t* plan, const void* logits,
                                int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                                const int32_t* targets, int32_t* out, void* workspace,
                                void* hip_stream);

/*
 * flare_logprobs_run without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  It runs the same two kernels on a
 * file-scope static device array of the library, 16 MiB per GPU, held from
 * the library's first call on that GPU until the process ends; its address
 * is looked up once per device (hipGetSymbolAddress) with that device
 * current.  No allocation, free or memset happens here or in the kernels, and
 * nothing in the scratch needs clearing: every word a call reads is written
 * earlier in the same call.
 *   Arguments: those of flare_logprobs_run (rectangular and unsharded plans),
 *   minus `workspace`; the call runs on the current device.
 *   Errors: as flare_logprobs_run, plus FLARE_ERR_SCRATCH_TOO_SMALL, before
 *   anything is launched, when plan->workspace_bytes exceeds 16 MiB (e.g. a
 *   1,024-slot x T=4 frame of 262,144 FP32 lanes needs 37 MB), and
 *   FLARE_ERR_DEVICE when the scratch's address cannot be found.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap on one
 *   GPU (other streams, other threads) race and must be ordered by the
 *   caller.  The L and guard diagnostics of such a call are not readable.
 */
int flare_logprobs_run_noalloc(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int32_t* emitted_counts,
                               const int32_t* tokens, int32_t K, int32_t* out, void* hip_stream);

/*
 * Vocabulary-sharded reduction on one GPU (Flare generation-logprobs design
 * page, vocabulary-sharded paragraph: each tensor-parallel rank keeps its
 * target logits as a vocabulary shard; the ranks exchange, per position,
 * each shard's maximum and exponential mass, the chosen token's raw logit
 * from its owner, and each shard's best 32 sort keys or the selected IDs'
 * raw logits; a final launch merges them into the same packed output).
 *
 * Here the shards are column slices of one [rows, V_pad] logits buffer:
 * shard r owns lanes [lo(r), lo(r + 1)) with lo(r) = floor(r V / shards)
 * rounded up to a multiple of 8 and at most V (lo(shards) = V), so that each
 * slice starts on a 16-byte boundary.  The result is the frame flare_logprobs_run writes,
 * with the same gating, layout and defined behaviour; only the order in which
 * L's FP32 partial sums are combined differs (shard by shard).
 *
 * flare_logprobs_plan_sharded: as flare_logprobs_plan, plus 1 <= shards <= 32
 *   with every shard non-empty (else FLARE_ERR_INVALID_ARGUMENT).  The plan
 *   records the shard count and the exchange records in the workspace:
 *   plan->exchange_offset, [capacity * T, shards] records of 552 bytes
 *   (max and exponential sum as FP32, the chosen raw logit and an ownership
 *   flag, a 64-bit cut key, then either 32 raw 64-bit keys or 128 selected raw
 *   logits, and a 128-bit ownership mask) -- the message a rank would send.
 * flare_logprobs_shard_pass: what rank `shard` computes on its own: the
 *   reduction of its columns and its exchange records (two launches).  The
 *   arguments are those of flare_logprobs_run with the whole rows in `logits`;
 *   only the shard's columns are read.
 * flare_logprobs_shard_merge: the final launch over the gathered records:
 *   L from the shards' maxima and sums in shard order, chosen and selected
 *   values from their owners' raw logits, the natural top K over all shards'
 *   keys.  A shard whose cut could hide a lane of the top K (only when the
 *   subtraction of L ties values at the cutoff) has its columns streamed again
 *   here; across ranks that is a second exchange from that shard's owner.
 * flare_logprobs_run_sharded: every shard pass, then the merge.
 * The unsharded entry points reject a sharded plan and these reject an
 * unsharded one (FLARE_ERR_PLAN_MISMATCH).
 */
int flare_logprobs_plan_sharded(flare_logprobs_plan_t* plan, int32_t capacity, int32_t T,
                                int32_t V, int32_t V_pad, int32_t dtype, int32_t K,
                                int32_t shards, int32_t device);
int flare_logprobs_run_sharded(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int32_t* emitted_counts,
                               const int32_t* tokens, int32_t K, int32_t* out, void* workspace,
                               void* hip_stream);
int flare_logprobs_shard_pass(const flare_logprobs_plan_t* plan, int32_t shard,
                              const void* logits, int32_t dtype, int64_t rows, int32_t V,
                              int32_t V_pad, const int32_t* requested, const int32_t* id_counts,
                              const int32_t* ids, const int32_t* emitted_counts,
                              const int32_t* tokens, int32_t K, int32_t* out, void* workspace,
                              void* hip_stream);
int flare_logprobs_shard_merge(const flare_logprobs_plan_t* plan, const void* logits,
                               int32_t dtype, int64_t rows, int32_t V, int32_t V_pad,
                               const int32_t* requested, const int32_t* id_counts,
                               const int32_t* ids, const int32_t* emitted_counts,
                               const int32_t* tokens, int32_t K, int32_t* out, void* workspace,
                               void* hip_stream);

/* Human-readable name of a flare_status value (static storage). */
const char* flare_status_string(int status);

/* FLARE_LOGPROBS_ABI_VERSION of the loaded library. */
uint32_t flare_logprobs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLARE_LOGPROBS_H */

// gfx950 kernels of the generation-logprob reduction.
//
// What is computed (Flare generation-logprobs design page, definition and
// tiled-reduction paragraphs): for each emitted position, L = FP32 logsumexp
// of the raw logits over lanes [0, V); the chosen token's fl32(x - L); then
// either the K best lanes by (fl32(x - L) desc, ID asc), -0 read as +0, or
// the caller's selected IDs in caller order.
//
// How.  Every logit is read from HBM once; nothing here is a contraction, so
// there is no MFMA.  Two launches.
//
// reduce_kernel: a persistent launch of `grid` 256-thread workgroups (five
// per CU).  The work is the concatenation, over active rows, of each row's
// units (16,384 bf16 or 8,192 FP32 lanes, 32 KiB); workgroup g owns the
// contiguous unit range [g N / R, (g + 1) N / R), R = grid once N >= 2 grid
// (fewer units: one or two per range, see range_count), so every workgroup
// streams the same number of bytes and a range may cross rows; when the
// active rows are few enough, each range is instead one of p equal pieces
// of a row (see range_plan).  The units of one row inside one range form a
// part.
//   Per unit, each thread holds 8 x 16-byte chunks (coalesced dwordx4 loads)
//   in VGPRs and refills each chunk with the next unit as soon as it is
//   summed.  Each wave keeps a running (max, sum of exp2) for the part.
//   Natural-mode rows also feed a per-wave LDS pool of 64-bit raw keys
//   (value, then smaller ID) that always holds the wave's best 32: chunks
//   whose maximum passes the admission bar are copied to an LDS stash as they
//   stream by and expanded one lane per element afterwards.  In a part's first
//   unit each wave first takes the maxima of its registers and admits lanes
//   at or above its k-th largest lane maximum (k = ceil(K / waves)); later
//   the bar is the largest of that value, the wave's own K-th best key and
//   the smallest of the four waves' published ceil(K / 4)-th best keys.
//   Compaction sorts 64-key lists in registers.  At the end of a part the
//   waves fold their sorted best 32 into one as they arrive, and the last
//   one writes the part record (m, s, best 32 raw keys, and a cut bounding
//   every key the part dropped), staged in LDS and written when the stage
//   fills or the range ends.
//
// merge_kernel: one wave per row (four per row when the launch's ranges are
// short and rows hold many parts) merges the row's part records: L from the
// parts in part order, the chosen and selected gathers, and the natural top
// K re-keyed by the reported value fl32(x - L), with an exactness guard that
// rescans a part when the raw order it kept could differ from the final
// order.
//
// The pages' own scheme ranks normalized values in a second pass over the
// vocabulary; ranking raw values and re-keying only the survivors is what
// lets this path read the logits once.
//
// The same two kernels serve three variants of the input and output:
//   - prompt scoring (SCORE): one row per scored prompt position, active when
//     its target is an ID; the stream also counts, per part, the lanes above
//     the target's logit, and the merge turns the counts into the rank
//     (recounting a part only where the subtraction tied a larger logit with
//     the target) and writes 43-word rows;
//   - packed target rows: slot s's row t is logit row row_offsets[s] + t of P
//     rows, the offsets kept in the slot table in LDS;
//   - completion records: emitted counts and tokens read from int64 records,
//     with optional ID inputs and rows of 2 + 2K words.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "flp_internal.h"

namespace flp {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kNanBits = 0x7FC00000u;

// ------------------------------------------------------------------ keys
// Order-preserving map of an FP32 value (with -0 read as +0) to uint32.
__device__ __forceinline__ uint32_t ukey32(float x) {
  x = (x == 0.0f) ? 0.0f : x;
  const uint32_t b = __float_as_uint(x);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float unkey32(uint32_t u) {
  const uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}
// 64-bit key: larger value first, then smaller token ID.  Never 0 for a
// real lane (the key of -inf is 0x007FFFFF in the high word).
__device__ __forceinline__ uint64_t make_key(float x, uint32_t id) {
  return ((uint64_t)ukey32(x) << 32) | (uint64_t)(~id);
}
__device__ __forceinline__ float key_value(uint64_t k) { return unkey32((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return ~(uint32_t)k; }

__device__ __forceinline__ float canon0(float x) { return (x == 0.0f) ? 0.0f : x; }
// The reported value: one FP32 subtraction, never contracted.
__device__ __forceinline__ float reported(float x, float L) { return canon0(__fsub_rn(x, L)); }
__device__ __forceinline__ uint64_t final_key(uint64_t raw, float L) {
  return ((uint64_t)ukey32(reported(key_value(raw), L)) << 32) | (raw & 0xFFFFFFFFull);
}

// Sixteen bytes of one lane as a native vector, so that a chunk stays one
// register tuple (loads, LDS copies and the ordering asm below take it whole).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- dtype traits
template <int DT> struct Elem;
template <> struct Elem<1> {  // bf16
  static constexpr int kPer = 8;
  static constexpr int kBytes = 2;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  __device__ static __forceinline__ float get(const u32x4& r, int j) {
    const uint32_t w = r[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ static __forceinline__ uint32_t load_bits(const char* row, int64_t i) {
    return (uint32_t)(*(const uint16_t*)(row + 2 * i));
  }
  // Largest input value below x (skipping -0, equal to +0 after canon0).
  __device__ static __forceinline__ float pred(float x) {
    uint32_t v = (ukey32(x) >> 16) - 1;
    if (v == 0x7FFFu) v = 0x7FFEu;
    const uint32_t h = (v & 0x8000u) ? (v & 0x7FFFu) : (~v & 0xFFFFu);
    return __uint_as_float(h << 16);
  }
};
template <> struct Elem<0> {  // fp32
  static constexpr int kPer = 4;
  static constexpr int kBytes = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  __device__ static __forceinline__ float get(const u32x4& r, int j) {
    const uint32_t w = r[j];
    return __uint_as_float(w);
  }
  __device__ static __forceinline__ uint32_t load_bits(const char* row, int64_t i) {
    return *(const uint32_t*)(row + 4 * i);
  }
  __device__ static __forceinline__ float pred(float x) {
    uint32_t v = ukey32(x) - 1;
    if (v == 0x7FFFFFFFu) v = 0x7FFFFFFEu;
    return unkey32(v);
  }
};

// Smallest FP32 value whose order key has the 16-bit prefix k16 (for the
// prefix of a bf16 value, that value itself).
__device__ __forceinline__ float key_floor16(uint32_t k16) {
  uint32_t u = k16 << 16;
  if (!(u & 0x80000000u)) u |= 0xFFFFu;
  return unkey32(u);
}

// Chunk holding lanes [first, first + kPer) of a row; lanes >= V read -inf.
template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_chunk(const char* row, int64_t first, int V) {
  using E = Elem<DT>;
  u32x4 r = {E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord};
  if (first >= V) return r;
  if (VEC) {
    r = *(const u32x4*)(row + first * E::kBytes);
    if (first + E::kPer > V) {
      const int nv = (int)(V - first);
#pragma unroll
      for (int j = 0; j < E::kPer; ++j) {
        if (j >= nv) {
          if (DT == 1)
            r[j >> 1] = (j & 1) ? ((r[j >> 1] & 0x0000FFFFu) | 0xFF800000u)
                                : ((r[j >> 1] & 0xFFFF0000u) | 0xFF80u);
          else
            r[j] = 0xFF800000u;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < E::kPer; ++j) {
      const int64_t i = first + j;
      if (i < V) {
        const uint32_t b = E::load_bits(row, i);
        if (DT == 1)
          r[j >> 1] = (j & 1) ? ((r[j >> 1] & 0x0000FFFFu) | (b << 16)) : ((r[j >> 1] & 0xFFFF0000u) | b);
        else
          r[j] = b;
      }
    }
  }
  return r;
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int64_t i) {
  const uint32_t b = Elem<DT>::load_bits(row, i);
  return __uint_as_float(DT == 1 ? (b << 16) : b);
}

// ------------------------------------------------------ fast cross-lane ops
// All exchanges are VALU lane permutes (DPP and the gfx950 permlane swaps),
// never LDS round trips.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
// Value held by lane ^ X.
template <int X>
__device__ __forceinline__ uint32_t xlane(uint32_t v, int lane) {
  if constexpr (X == 1) {
    return dpp32<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (X == 2) {
    return dpp32<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (X == 4) {
    return dpp32<0x1B>(dpp32<0x141>(v));  // row_half_mirror, then quad_perm [3,2,1,0]
  } else if constexpr (X == 8) {
    return dpp32<0x128>(v);  // row_ror:8
  } else if constexpr (X == 15) {
    return dpp32<0x140>(v);  // row_mirror
  } else if constexpr (X == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(X == 32, "lane distance");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}
template <int X>
__device__ __forceinline__ uint64_t xlane64(uint64_t v, int lane) {
  const uint32_t lo = xlane<X>((uint32_t)v, lane);
  const uint32_t hi = xlane<X>((uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}
template <int X>
__device__ __forceinline__ float xlanef(float v, int lane) {
  return __uint_as_float(xlane<X>(__float_as_uint(v), lane));
}
// Value held by lane 63 - lane.
__device__ __forceinline__ uint64_t reverse64(uint64_t v, int lane) {
  return xlane64<32>(xlane64<16>(xlane64<15>(v, lane), lane), lane);
}
// Value held by lane - 1 (0 in lane 0).
__device__ __forceinline__ uint64_t wave_shr1_64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x138, 0xf, 0xf, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x138, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Butterfly reductions: every lane ends with the same value, and the
// order of the additions is fixed, so the sum is deterministic.
__device__ __forceinline__ float wave_max(float v, int lane) {
  v = fmaxf(v, xlanef<32>(v, lane));
  v = fmaxf(v, xlanef<16>(v, lane));
  v = fmaxf(v, xlanef<8>(v, lane));
  v = fmaxf(v, xlanef<4>(v, lane));
  v = fmaxf(v, xlanef<2>(v, lane));
  v = fmaxf(v, xlanef<1>(v, lane));
  return v;
}
__device__ __forceinline__ float wave_sum(float v, int lane) {
  v += xlanef<32>(v, lane);
  v += xlanef<16>(v, lane);
  v += xlanef<8>(v, lane);
  v += xlanef<4>(v, lane);
  v += xlanef<2>(v, lane);
  v += xlanef<1>(v, lane);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v, int lane) {
  v += (int)xlane<32>((uint32_t)v, lane);
  v += (int)xlane<16>((uint32_t)v, lane);
  v += (int)xlane<8>((uint32_t)v, lane);
  v += (int)xlane<4>((uint32_t)v, lane);
  v += (int)xlane<2>((uint32_t)v, lane);
  v += (int)xlane<1>((uint32_t)v, lane);
  return v;
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Order LDS accesses of one wave (no other wave is involved).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One compare-exchange step of a bitonic network: the lane keeps the larger
// key when `keep_max`.
template <int STRIDE>
__device__ __forceinline__ uint64_t cx(uint64_t k, int lane, bool keep_max) {
  const uint64_t o = xlane64<STRIDE>(k, lane);
  return keep_max ? (k > o ? k : o) : (k < o ? k : o);
}
// Sort one key per lane, descending by lane index.
__device__ __forceinline__ uint64_t sort64_desc(uint64_t k, int lane) {
#define FLP_STEP(SIZE, STRIDE) \
  k = cx<STRIDE>(k, lane, ((lane & (SIZE)) == 0) == ((lane & (STRIDE)) == 0));
  FLP_STEP(2, 1)
  FLP_STEP(4, 2) FLP_STEP(4, 1)
  FLP_STEP(8, 4) FLP_STEP(8, 2) FLP_STEP(8, 1)
  FLP_STEP(16, 8) FLP_STEP(16, 4) FLP_STEP(16, 2) FLP_STEP(16, 1)
  FLP_STEP(32, 16) FLP_STEP(32, 8) FLP_STEP(32, 4) FLP_STEP(32, 2) FLP_STEP(32, 1)
  FLP_STEP(64, 32) FLP_STEP(64, 16) FLP_STEP(64, 8) FLP_STEP(64, 4) FLP_STEP(64, 2)
  FLP_STEP(64, 1)
#undef FLP_STEP
  return k;
}
// Sort a bitonic sequence (one key per lane) descending.
__device__ __forceinline__ uint64_t bitonic_merge_desc(uint64_t k, int lane) {
  k = cx<32>(k, lane, (lane & 32) == 0);
  k = cx<16>(k, lane, (lane & 16) == 0);
  k = cx<8>(k, lane, (lane & 8) == 0);
  k = cx<4>(k, lane, (lane & 4) == 0);
  k = cx<2>(k, lane, (lane & 2) == 0);
  k = cx<1>(k, lane, (lane & 1) == 0);
  return k;
}
// Sort two lists held in lanes 0..31 and 32..63 descending.  Each list
// comes from a part record sorted by raw key; re-keying by the reported
// value keeps that order unless the subtraction ties distinct values, so
// the halves are checked first and, when both are in order, merged by one
// bitonic pass (the upper half mirrored to make the sequence bitonic).
__device__ __forceinline__ uint64_t sort_halves_desc(uint64_t k, int lane) {
  const uint64_t prev = wave_shr1_64(k);  // lane - 1
  const bool out_of_order = (lane & 31) != 0 && prev < k;
  if (__ballot(out_of_order) != 0ull) return sort64_desc(k, lane);
  const uint64_t mirrored = xlane64<16>(xlane64<15>(k, lane), lane);  // lane 31 - l within 32
  return bitonic_merge_desc(lane < 32 ? k : mirrored, lane);
}

// The same for two independent lists at once (one check of both, and the
// two networks' steps interleave).
__device__ __forceinline__ void sort_halves_desc2(uint64_t& ka, uint64_t& kb, int lane) {
  const uint64_t pa = wave_shr1_64(ka), pb = wave_shr1_64(kb);
  const bool out_of_order = (lane & 31) != 0 && (pa < ka || pb < kb);
  if (__ballot(out_of_order) != 0ull) {
    ka = sort64_desc(ka, lane);
    kb = sort64_desc(kb, lane);
    return;
  }
  const uint64_t ma = xlane64<16>(xlane64<15>(ka, lane), lane);
  const uint64_t mb = xlane64<16>(xlane64<15>(kb, lane), lane);
  ka = bitonic_merge_desc(lane < 32 ? ka : ma, lane);
  kb = bitonic_merge_desc(lane < 32 ? kb : mb, lane);
}

// Lanes 0..31 of the result hold the best 32 of {top[0..32), list[0..64)}
// sorted descending, given `top` sorted in lanes 0..31 and `list` sorted.
__device__ __forceinline__ uint64_t merge_top32(uint64_t top, uint64_t list, int lane) {
  const uint64_t rev = reverse64(list, lane);
  return bitonic_merge_desc(lane < 32 ? top : rev, lane);
}

// The q-th largest 16-bit key among the wave's voting lanes (ballot radix
// select; requires at least q voters).
__device__ __forceinline__ uint32_t wave_kth_largest16(uint32_t key, bool voter, int q) {
  uint32_t prefix = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t trial = prefix | (1u << b);
    const uint64_t m = __ballot(voter && key >= trial);
    if (__popcll(m) >= q) prefix = trial;
  }
  return prefix;
}

// ------------------------------------------------------ per-wave best 32
// Each wave keeps the best 32 raw keys of the part it is reducing as a list
// sorted descending across lanes 0..31 (0 marks an empty slot; lanes 32..63
// hold scratch).  A unit's new candidates are gathered in an LDS buffer and
// then inserted: a few one at a time (a ballot gives the position, a wave
// shift opens the slot), more by sorting them and merging.
constexpr int kCandBuf = 128;   // candidate slots per wave
constexpr int kInsertMax = 12;  // larger batches are sorted and merged

struct Best32 {
  uint64_t top;  // lane i < 32: the i-th best key
  int n;         // keys held (wave-uniform)
  int rank;      // the call's K: only the best K of a part can reach the top K
  uint64_t bar;  // the rank-th best key once n >= rank, else 0 (wave-uniform)
};


// Insert the wave-uniform key k if it ranks among the best 32: lanes past
// its position p take their lower neighbour's key (the shift's bound control
// feeds lane 0 a zero, which it never keeps) and lane p takes k.
__device__ __forceinline__ void best_insert(Best32& b, uint64_t k, int lane) {
  const int p = __popc((uint32_t)__ballot(b.top > k));  // better keys in lanes 0..31
  if (p >= kKeep) return;
  const uint32_t lo = (uint32_t)b.top, hi = (uint32_t)(b.top >> 32);
  const uint32_t slo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, 0x138, 0xf, 0xf, true);
  const uint32_t shi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, 0x138, 0xf, 0xf, true);
  const uint64_t shifted = ((uint64_t)shi << 32) | slo;
  b.top = lane < p ? b.top : (lane == p ? k : shifted);
  b.n = b.n < kKeep ? b.n + 1 : kKeep;
}

struct CandBuf {
  uint64_t* keys;  // this wave's kCandBuf slots in LDS
  int count;
};

// Move the buffered candidates into the list and empty the buffer.
__device__ __forceinline__ void cand_flush(CandBuf& cb, Best32& b, int lane) {
  if (cb.count == 0) return;
  wave_sync();
  if (cb.count <= kInsertMax) {
    const uint64_t mine = lane < cb.count ? cb.keys[lane] : 0ull;
    for (int i = 0; i < cb.count; ++i) best_insert(b, readlane64(mine, i), lane);
  } else {
    for (int base = 0; base < cb.count; base += 64) {
      const uint64_t v = base + lane < cb.count ? cb.keys[base + lane] : 0ull;
      b.top = merge_top32(b.top, sort64_desc(v, lane), lane);
    }
    b.n = __popc((uint32_t)__ballot(b.top != 0ull));
  }
  wave_sync();
  cb.count = 0;
  b.bar = b.n >= b.rank ? readlane64(b.top, b.rank - 1) : 0ull;
}

// Buffer one key per lane (0 = none).  A key at or below the list's bar (its
// K-th key) is dropped at once: it can no longer reach the top K (a run of equal values,
// -inf lanes say, then costs one flush instead of one per buffer).
__device__ __forceinline__ void cand_append(CandBuf& cb, Best32& b, uint64_t k, int lane) {
  if (k <= b.bar) k = 0ull;
  uint64_t m = __ballot(k != 0ull);
  if (m == 0ull) return;
  int n = __popcll(m);
  if (cb.count + n > kCandBuf) {
    cand_flush(cb, b, lane);
    if (k <= b.bar) k = 0ull;
    m = __ballot(k != 0ull);
    if (m == 0ull) return;
    n = __popcll(m);
  }
  if (k != 0ull) cb.keys[cb.count + lanes_below(m)] = k;
  cb.count += n;
}

// ------------------------------------------------------------ row mapping
// A prefix word holds the active rows of the slots before s in its low 31
// bits and, in bit 31, whether slot s selects IDs (its rows then keep no
// natural candidates).  Keeping that bit in LDS spares the stream a global
// load at each part end, whose wait would also wait for the next unit's
// loads already in flight.
constexpr int kSelBit = (int)0x80000000u;
constexpr int kRowsMask = 0x7FFFFFFF;

// Packed target rows: a slot whose committed rows [off, off + rows) would
// leave the P physical rows reads and writes nothing.
__device__ __forceinline__ int packed_rows_of(const Params& p, int s, int rows) {
  const int off = p.row_offsets[s];
  return rows > 0 && (off < 0 || (int64_t)off + rows > p.packed_rows) ? 0 : rows;
}

// A slot's emitted count and a position's chosen token, from the int32
// inputs or from the slot's int64 completion record (values outside the
// int32 range: a count reads as 0, a token as -1).
__device__ __forceinline__ int emitted_of(const Params& p, int s) {
  if (!p.crecords) return p.emitted[s];
  const int64_t v = p.crecords[(int64_t)s * (kRecordMeta + p.T) + p.emitted_field];
  return v < 0 || v > 0x7FFFFFFF ? 0 : (int)v;
}
__device__ __forceinline__ int token_of(const Params& p, int s, int t) {
  if (!p.crecords) return p.tokens[s * p.T + t];
  const int64_t v = p.crecords[(int64_t)s * (kRecordMeta + p.T) + kRecordMeta + t];
  return v < -0x80000000ll || v > 0x7FFFFFFF ? -1 : (int)v;
}

// A generation slot's active rows and whether it selects IDs.
__device__ __forceinline__ int slot_word(const Params& p, int s) {
  // The words are loaded together (one round trip).
  const int r = p.requested[s], e = emitted_of(p, s), n = p.id_counts ? p.id_counts[s] : 0;
  int rows = r == 0 ? 0 : (e < 0 ? 0 : (e > p.T ? p.T : e));
  if (p.row_offsets) rows = packed_rows_of(p, s, rows);
  return rows | (n > 0 ? kSelBit : 0);
}

// Inclusive sum over lanes 0..lane of the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31 into rows 2, 3
  return v;
}

// prefix[s] = active rows of slots before s (with slot s's selection bit);
// prefix[capacity] = total.  All NW waves of the workgroup take part; `scan`
// is NW ints of LDS.
template <int NW, bool SCORE>
__device__ int build_prefix(const Params& p, int* prefix, int* scan) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cap = p.capacity;
  const int per = (cap + NT - 1) / NT;
  const int s0 = tid * per;
  const int s1 = s0 + per < cap ? s0 + per : cap;
  int local = 0;
  // Packed row offsets (packed launches), or the scored rows' targets (scoring).
  int* phys = prefix + cap + 1;
  for (int s = s0; s < s1; ++s) {
    int c;
    if (SCORE) {
      // A scored prompt row (one per slot) is active when its target is an ID.
      const int tk = p.tokens[s];
      c = (tk >= 0 && tk < p.V) ? 1 : 0;
      phys[s] = tk;
    } else {
      c = slot_word(p, s);
      if (p.row_offsets) phys[s] = p.row_offsets[s];
    }
    prefix[s] = c;
    local += c & kRowsMask;
  }
  // exclusive scan of `local` over the block: within each wave an inclusive
  // scan by DPP (shifts by 1, 2, 4, 8 inside each row of 16 lanes, zeros
  // shifted in, then row 0's and row 1's last lanes broadcast into the rows
  // after them), no LDS round trips
  int incl = wave_incl_scan(local);
  if (lane == 63) scan[w] = incl;
  __syncthreads();
  int run = incl - local, total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    run += i < w ? scan[i] : 0;
    total += scan[i];
  }
  for (int s = s0; s < s1; ++s) {
    const int c = prefix[s];
    prefix[s] = run | (c & kSelBit);
    run += c & kRowsMask;
  }
  if (tid == 0) prefix[cap] = total;
  __syncthreads();
  return total;
}

// Slot of active row a: the largest s whose row count before it is <= a.
__device__ __forceinline__ int slot_of(const int* prefix, int cap, int a) {
  int lo = 0, hi = cap;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((prefix[mid] & kRowsMask) <= a) lo = mid; else hi = mid;
  }
  return lo;
}
// The same slot for a wave-uniform a, from lane-parallel compares instead of
// a chain of dependent reads: the counts are non-decreasing in s, so the
// slots whose count is at most a form a prefix.  Lane l tests slot
// l * stride (stride = ceil(cap / 64)); the last passing sample bounds the
// slot to the stride slots after it, which a second round tests.
__device__ __forceinline__ int slot_of_wave(const int* prefix, int cap, int a, int lane) {
  const int stride = (cap + 63) >> 6;
  const int sc = lane * stride;
  const int lo = (__popcll(__ballot(sc < cap && (prefix[sc] & kRowsMask) <= a)) - 1) * stride;
  int n = 0;
  for (int j = 1; j < stride; j += 64) {
    const int s = lo + j + lane;
    n += __popcll(__ballot(j + lane < stride && s < cap && (prefix[s] & kRowsMask) <= a));
  }
  return __builtin_amdgcn_readfirstlane(lo + n);
}

// ==================================================================== merge
// One wave per row, four rows per workgroup: L from the row's parts in part
// order, the chosen and selected gathers, and the natural top K.  The
// reduction left each slot's count of active rows before it, and their
// total, in the workspace: with them a row finds its index among the active
// rows, and its parts, from its first loads.
//
// Exactness guard.  Every lane a part did not keep has a raw key at most the
// part's cut c (value x_c): the part's K-th kept key, or a wave's first-unit
// bar, whichever is larger.  With F the final key (reported value, then
// smaller ID), F_K the K-th best final key among all kept candidates and v_K
// its value, such a lane e has either x_e == x_c and a larger ID (so
// F(e) <= F(c)) or x_e <= pred(x_c) (so its value is at most r(pred(x_c)),
// r(x) = fl32(x - L) being monotone).  Hence if F(c) <= F_K and
// r(pred(x_c)) < v_K no dropped lane can enter the top K.  A part that fails
// either test is rescanned lane by lane with final keys; F_K over a subset
// never exceeds the true K-th key, so the test stays sound.
constexpr int kMergeWaves = kMergeBlock / 64;
// A part record's statistics words, loaded one lane per part.
struct PartRecord0 {
  float m, s;
  int32_t above;
  float next_above;
  uint64_t cut;
};
constexpr int kLdsPairs = 14;  // part pairs after the first two staged in LDS (rows up to 32 parts)

// Whether unit x begins one of the `grid` ranges [floor(g n / grid),
// floor((g + 1) n / grid)) of n units: with g the smallest index whose range
// starts at or after x, ceil(x grid / n), it does iff floor(g n / grid) == x.
// Every product is below 2^53 and every quotient that is not an integer is
// at least 1/n (resp. 1/grid) away from one, so the double divisions round
// to the exact ceiling and floor.
// Unit ranges of a launch over n units with `grid` workgroups: one unit each
// up to grid units, then two units each (fewer, equally loaded workgroups
// rather than a mix of one- and two-unit ranges), then `grid` ranges.  The
// reduction and the merge derive it from the same n.
__device__ __forceinline__ int range_count(int64_t n, int grid) {
  if (n >= 2 * (int64_t)grid) return grid;
  if (n > grid) return (int)((n + 1) >> 1);
  return n < 1 ? 1 : (int)n;
}

__device__ __forceinline__ bool is_range_start(int x, int n, int grid) {
  const double g = __builtin_ceil((double)x * (double)grid / (double)n);
  return __builtin_floor(g * (double)n / (double)grid) == (double)x;
}

// Row-aligned ranges.  When the launch holds at least two units per
// workgroup and cutting every active row into p = grid / rows equal pieces
// makes no range more than one unit longer than the balanced split's
// longest, each range is one piece of one row: one part per range, so no
// range pays two part ends or ends on a one-unit part (the costliest unit,
// and at the end of a range nothing overlaps it).  Workgroup b takes piece
// b / rows of row b % rows: the pieces that hold a row's last (partial) unit
// go to the workgroups dispatched later, which get their first data later.
// When p pieces per row would leave at least a sixteenth of the grid idle
// (grid - p rows workgroups), the last grid - p rows rows are cut into p + 1
// pieces instead, the extra pieces going to the last workgroups: every
// workgroup streams, and the shorter pieces go to the workgroups dispatched
// last.  (A few idle workgroups are not worth the extra parts and merge
// work.)
constexpr int kRowAlignSlack = 1;
struct RangePlan {
  int count;   // ranges of the launch
  int pieces;  // pieces per row (0: the balanced split of all units)
  int extra;   // the last `extra` rows are cut into pieces + 1
};
__device__ __forceinline__ RangePlan range_plan(int rows, int U, int grid) {
  const uint32_t n = (uint32_t)rows * (uint32_t)U;  // below 2^31 (the host checks)
  if (n < 2u * (uint32_t)grid) return RangePlan{range_count(n, grid), 0, 0};
  const int p = grid / rows;
  const uint32_t longest = (n + (uint32_t)grid - 1u) / (uint32_t)grid;
  if (p >= 2 && (uint32_t)((U + p - 1) / p) <= longest + kRowAlignSlack) {
    const int idle = grid - rows * p;
    const int extra = U >= p + 1 && 16 * idle >= grid ? idle : 0;
    return RangePlan{rows * p + extra, p, extra};
  }
  return RangePlan{grid, 0, 0};
}
// Whether unit x of a launch over `rows` rows of U units begins a range.
__device__ __forceinline__ bool starts_range(int x, int rows, int U, const RangePlan& rp) {
  if (rp.pieces) {
    const int a = x / U;
    return is_range_start(x - a * U, U, rp.pieces + (a >= rows - rp.extra ? 1 : 0));
  }
  return is_range_start(x, rows * U, rp.count);
}

// Whether the reduction's idle workgroups capture every active position's
// chosen (or scored target) raw logit, one thread per position, for the
// merge of an unsharded call.
__device__ __forceinline__ bool chosen_captured(const Params& p, const RangePlan& rp) {
  return p.shards == 0 && (int64_t)(p.workers - rp.count) * kBlock >= (int64_t)p.capacity * p.T;
}

// Every lane [lo, hi) of a row whose final key reaches thr, merged into the
// sorted best 32 in `top`; thr rises to the K-th kept key as it fills.  One
// 16-byte chunk per lane per step, eight steps' chunks loaded at once.  Keys
// that reach thr are appended to the wave's LDS buffer `buf` (`cap` keys, a
// multiple of 64) and sorted into `top` only when it is full and at the end,
// so a step whose lanes hold candidates costs a ballot and one LDS store.
template <int DT, bool VEC>
__device__ __forceinline__ void rescan_lanes(uint64_t& top, uint64_t& thr, const char* rowp, int lo,
                                             int hi, float L, int Keff, int lane, uint64_t* buf,
                                             int cap) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  constexpr int kStep = 64 * kPer;
  constexpr int kBatch = 8;  // chunks per lane in flight at once
  int n = 0;                 // buffered keys (wave-uniform)
  auto flush = [&]() {
    wave_sync();
    for (int base = 0; base < n; base += 64) {
      const uint64_t v = base + lane < n ? buf[base + lane] : 0ull;
      top = merge_top32(top, sort64_desc(v, lane), lane);
    }
    n = 0;
    // The list only improves: its K-th key is a floor for the rest.
    const uint64_t kth = readlane64(top, Keff - 1);
    thr = kth > thr ? kth : thr;
    wave_sync();
  };
  for (int b = lo; b < hi; b += kBatch * kStep) {
    u32x4 cur[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const int first = b + c * kStep + lane * kPer;
      cur[c] = first < hi ? load_chunk<DT, VEC>(rowp, first, hi) : u32x4{0u, 0u, 0u, 0u};
    }
    const int steps = (hi - b + kStep - 1) / kStep < kBatch ? (hi - b + kStep - 1) / kStep : kBatch;
#pragma nounroll
    for (int c = 0; c < steps; ++c) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = b + c * kStep + lane * kPer + j;
        uint64_t f = i < hi ? make_key(reported(E::get(cur[0], j), L), (uint32_t)i) : 0ull;
        if (f < thr) f = 0ull;
        uint64_t m = __ballot(f != 0ull);
        if (m != 0ull) {
          if (n + __popcll(m) > cap) {
            flush();
            if (f < thr) f = 0ull;
            m = __ballot(f != 0ull);
          }
          if (f != 0ull) buf[n + lanes_below(m)] = f;
          n += __popcll(m);
        }
      }
#pragma unroll
      for (int c2 = 0; c2 + 1 < kBatch; ++c2) cur[c2] = cur[c2 + 1];
    }
  }
  flush();
}

// Lanes [lo, hi) of a row whose reported value exceeds rt, summed over the
// wave (every lane gets the total); eight 16-byte chunks per lane in flight.
template <int DT, bool VEC>
__device__ __forceinline__ int count_above(const char* rowp, int lo, int hi, float L, float rt,
                                           int lane) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  constexpr int kBatch = 8;  // chunks per lane in flight at once
  constexpr uint32_t w = E::kNegInfWord;
  int n = 0;
  for (int b = lo; b < hi; b += kBatch * 64 * kPer) {
    u32x4 r[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const int first = b + (c * 64 + lane) * kPer;
      r[c] = first < hi ? load_chunk<DT, VEC>(rowp, first, hi) : u32x4{w, w, w, w};
    }
#pragma unroll
    for (int c = 0; c < kBatch; ++c)
#pragma unroll
      for (int j = 0; j < kPer; ++j) n += reported(E::get(r[c], j), L) > rt ? 1 : 0;
  }
  return wave_sum_i32(n, lane);
}

// With SCORE the rows are the scored rows of a prompt chunk (T = 1): a row
// whose target is not an ID gets its fixed invalid record, the others the
// target's pair, its rank (one plus the count of lanes whose reported value
// exceeds the target's) and the top twenty, kPromptWords words in all.
//
// Rank.  The reduction counted, per part, the lanes whose raw logit exceeds
// the target's, x_t, and kept the smallest of them, x_n.  r(x) = fl32(x - L)
// is monotone, so no lane at or below x_t can report more than r(x_t), and a
// lane above x_t reports at least r(x_n) >= r(x_t); the raw count is exact
// unless r(x_n) == r(x_t) (the subtraction tied them).  FP32 parts also carry
// the number of lanes at x_n and the next larger value x_m: when r(x_m) >
// r(x_t) exactly those lanes tie and are taken off; otherwise (and for bf16,
// whose spacing makes such ties rare) the part is counted again lane by lane
// with reported values.
//
// WIDE: one row per workgroup, for launches whose rows hold many parts
// (short unit ranges).  The four waves read the row's words alike; wave w
// re-keys, sorts and merges the part pairs w, w + 4, ... and wave 0 merges
// the four lists and writes the row.  A row of at most four parts is merged
// by wave 0 alone, as in the one-wave layout.
template <int DT, bool VEC, bool SCORE, bool WIDE>
__global__ __launch_bounds__(kMergeBlock) void merge_kernel(Params p) {
  using E = Elem<DT>;
  constexpr int kUnitElems = kUnitThreads * kChunks * E::kPer;
  constexpr int kWidePairs = (kMaxUnits / 2 + kMergeWaves - 1) / kMergeWaves;  // pairs per wave
  __shared__ int16_t part_u0_all[kMergeWaves][kMaxUnits + 1];
  __shared__ uint64_t pair_keys[kMergeWaves][kLdsPairs][64];
  __shared__ uint64_t wide_lists[WIDE ? kMergeWaves : 1][kKeep];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = WIDE ? (int)blockIdx.x : (int)blockIdx.x * kMergeWaves + wv;
  // The wave that writes the row's words (every wave in the one-wave layout).
  const bool lead = !WIDE || wv == 0;
  {
    // The arguments the loads below take, all fetched before the first is
    // needed: one wait for the argument block instead of one per use.
    const void* a0 = p.records;
    const void* a1 = p.requested;
    const void* a2 = p.crecords;
    const void* a3 = p.emitted;
    const void* a4 = p.tokens;
    const void* a5 = p.id_counts;
    const void* a6 = p.row_offsets;
    const void* a7 = p.slot_rows;
    const void* a8 = p.xtok;
    const void* a9 = p.ids;
    asm volatile("" ::"s"(a0), "s"(a1), "s"(a2), "s"(a3), "s"(a4), "s"(a5), "s"(a6), "s"(a7), "s"(a8),
                 "s"(a9), "s"(p.capacity), "s"(p.T), "s"(p.units), "s"(p.shards), "s"(p.emitted_field));
  }
  if (row >= p.capacity * p.T) return;
  const int s = row / p.T, t = row - s * p.T;
  const int V = p.V, U = p.units;
  // Issued first, before the row's words and with nothing depending on them
  // (records are stored by part index): each part's statistics (lane i:
  // part i) and the first two parts' kept keys.
  const PartRecord* rec = p.records + (int64_t)row * U;
  PartRecord0 hdr{kNegInf, 0.0f, 0, __builtin_huge_valf(), 0ull};
  if (lane < U) hdr = PartRecord0{rec[lane].m, rec[lane].s, rec[lane].above, rec[lane].next_above, rec[lane].cut};
  uint64_t ex31 = 0ull;
  if (SCORE && DT == 0 && lane < U) ex31 = rec[lane].keys[kKeep - 1];
  const uint64_t spec0 = (lane >> 5) < U ? rec[lane >> 5].keys[lane & 31] : 0ull;
  // Every input word this row needs and the captured chosen logit, in one
  // round trip: the ten scalar loads are issued back to back and waited for
  // once.  (Scalar loads complete out of order, so compiled code waits for
  // all of them before it tests any pointer or word: a round trip per test.)
  // An input not given reads a stand-in word (the slot table's first, always
  // valid), ignored below; the row counts only mean something for an active
  // row.  The wait is in the same block as the loads.
  const int32_t* const w0 = p.slot_rows;
  const bool crec = !SCORE && p.crecords != nullptr;
  const int64_t* const cr = crec ? p.crecords + (int64_t)s * (kRecordMeta + p.T) : (const int64_t*)w0;
  const int64_t* const a_ce = crec ? cr + p.emitted_field : cr;
  const int64_t* const a_ct = crec ? cr + kRecordMeta + t : cr;
  const int32_t* const a_req = SCORE ? w0 : p.requested + s;
  const int32_t* const a_em = !SCORE && p.emitted ? p.emitted + s : w0;
  const int32_t* const a_tk = SCORE ? p.tokens + row : (p.tokens ? p.tokens + (s * p.T + t) : w0);
  const int32_t* const a_cnt = !SCORE && p.id_counts ? p.id_counts + s : w0;
  const int32_t* const a_off = !SCORE && p.row_offsets ? p.row_offsets + s : w0;
  const int32_t* const a_bef = p.slot_rows + s;
  const int32_t* const a_tot = p.slot_rows + p.capacity;
  const int32_t* const a_xt = p.shards == 0 ? (const int32_t*)p.xtok + row : w0;
  int w_req, w_em, w_tk, w_cnt, w_off, before, total, w_xt;
  int64_t w_ce, w_ct;
  asm volatile(
      "s_load_dword %0, %10, 0x0\n\t"
      "s_load_dword %1, %11, 0x0\n\t"
      "s_load_dword %2, %12, 0x0\n\t"
      "s_load_dword %3, %13, 0x0\n\t"
      "s_load_dword %4, %14, 0x0\n\t"
      "s_load_dword %5, %15, 0x0\n\t"
      "s_load_dword %6, %16, 0x0\n\t"
      "s_load_dword %7, %17, 0x0\n\t"
      "s_load_dwordx2 %8, %18, 0x0\n\t"
      "s_load_dwordx2 %9, %19, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(w_req), "=&s"(w_em), "=&s"(w_tk), "=&s"(w_cnt), "=&s"(w_off), "=&s"(before),
        "=&s"(total), "=&s"(w_xt), "=&s"(w_ce), "=&s"(w_ct)
      : "s"(a_req), "s"(a_em), "s"(a_tk), "s"(a_cnt), "s"(a_off), "s"(a_bef), "s"(a_tot), "s"(a_xt),
        "s"(a_ce), "s"(a_ct)
      : "memory");
  const float xt_spec = __int_as_float(w_xt);
  // Issued after the words and not waited for with the records above: the
  // third and fourth parts' keys and the selected IDs, which only some rows
  // use (and whose lines, unlike the records just written, may come from
  // HBM).
  // Unconditional loads (clamped part, stand-in word), so that the wait for
  // the records can count them as issued after the records on every path.
  const int part1 = 2 + (lane >> 5) < U ? 2 + (lane >> 5) : U - 1;
  const uint64_t spec1_raw = rec[part1].keys[lane & 31];
  const bool has_ids = !SCORE && p.ids != nullptr;
  const int32_t* const idb = has_ids ? p.ids + (int64_t)s * 128 : w0;
  const int ids_raw0 = idb[has_ids ? lane : 0], ids_raw1 = idb[has_ids ? 64 + lane : 0];
  const int req = SCORE ? 1 : w_req;
  const int emi = SCORE ? 1 : (crec ? (w_ce < 0 || w_ce > 0x7FFFFFFF ? 0 : (int)w_ce) : w_em);
  const int tok = crec ? (w_ct < -0x80000000ll || w_ct > 0x7FFFFFFF ? -1 : (int)w_ct) : w_tk;
  const int cnt = !SCORE && p.id_counts ? w_cnt : 0;
  const int off = !SCORE && p.row_offsets ? w_off : 0;
  // The record loads above are not sunk past the row's tests.
  asm volatile("" ::"v"(hdr.m), "v"(hdr.s), "v"(hdr.above), "v"(hdr.next_above), "v"(hdr.cut),
               "v"(ex31), "v"(spec0));
  const uint64_t spec1 = 2 + (lane >> 5) < U ? spec1_raw : 0ull;
  const int ids_spec[2] = {ids_raw0, ids_raw1};
  int32_t* out = p.out + (int64_t)row * (SCORE ? kPromptWords : p.row_words);
  if (SCORE && !(tok >= 0 && tok < V)) {
    // [-1, NaN, rank 0, then (-1, NaN) twenty times]
    if (lead && lane < kPromptWords)
      out[lane] = lane == 2 ? 0 : ((lane == 0 || (lane >= 3 && (lane & 1))) ? -1 : (int32_t)kNanBits);
    return;
  }
  int rows_s = req == 0 ? 0 : (emi < 0 ? 0 : (emi > p.T ? p.T : emi));
  if (!SCORE && p.row_offsets && rows_s > 0 && (off < 0 || (int64_t)off + rows_s > p.packed_rows))
    rows_s = 0;  // as packed_rows_of, with the offset already loaded
  if (t >= rows_s) return;
  const int n_sel = cnt < 0 ? 0 : (cnt > 128 ? 128 : cnt);
  const bool natural = p.K > 0 && n_sel == 0;
  const int lrow = !SCORE && p.row_offsets ? off + t : row;
  const char* rowp = (const char*)p.logits + (int64_t)lrow * p.V_pad * E::kBytes;
  int16_t* part_u0 = part_u0_all[wv];

  // ---- the row's parts (one lane per unit): a part starts at the row's
  // first unit and wherever a workgroup's unit range starts (the
  // reduction's partition, recomputed exactly: row pieces, or floor(g N / R)
  // of the N units of the active rows in double precision).
  const int a = before + t;
  const RangePlan rplan = range_plan(total, U, p.workers);
  int np;
  if (rplan.pieces) {
    // Row pieces: part i of q starts at unit floor(i U / q).
    np = rplan.pieces + (a >= total - rplan.extra ? 1 : 0);
    if (lane <= np) part_u0[lane] = (int16_t)(lane * U / np);
  } else {
    const bool start = lane < U && (lane == 0 || starts_range(a * U + lane, total, U, rplan));
    const uint64_t starts = __ballot(start);
    np = __popcll(starts);
    if (start) part_u0[lanes_below(starts)] = (int16_t)lane;
    if (lane == 0) part_u0[np] = (int16_t)U;
  }
  wave_sync();

  // ---- record and logit loads, issued together: the part statistics, the
  // first four parts' kept keys in registers, those of the next 2 kLdsPairs
  // parts (rows of many parts) staged in LDS, and each part's guard words
  float pm = kNegInf, ps = 0.0f;
  uint64_t c_key = 0ull;
  int p_above = 0, p_count = 0;
  float p_next = __builtin_huge_valf(), p_next2 = __builtin_huge_valf();
  if (lane < np) {
    pm = hdr.m;
    ps = hdr.s;
    c_key = hdr.cut;
    if (SCORE) {
      p_above = hdr.above;
      p_next = hdr.next_above;
      if (DT == 0) {
        p_count = (int)(uint32_t)ex31;
        p_next2 = __uint_as_float((uint32_t)(ex31 >> 32));
      }
    }
  }
  // FP32 scoring records use key slot 31 for the rank (read above), not a key.
  const bool extra_slot = SCORE && DT == 0 && (lane & 31) == kKeep - 1;
  const uint64_t raw0 = !extra_slot && (lane >> 5) < np ? spec0 : 0ull;
  const uint64_t raw1 = !extra_slot && 2 + (lane >> 5) < np ? spec1 : 0ull;
  // WIDE rows of more than four parts: this wave's pairs, loads all in flight.
  const bool wide = WIDE && natural && np > 4;
  uint64_t wraw[WIDE ? kWidePairs : 1];
#pragma unroll
  for (int i = 0; i < (WIDE ? kWidePairs : 1); ++i) {
    const int part = 2 * (wv + i * kMergeWaves) + (lane >> 5);
    wraw[i] = wide && !extra_slot && part < np ? rec[part].keys[lane & 31] : 0ull;
  }
  if (natural && np > 4 && !wide) {
    // All loads in flight at once: a row of many parts pays one round trip.
    uint64_t pre[kLdsPairs];
#pragma unroll
    for (int i = 0; i < kLdsPairs; ++i) {
      const int part = 4 + 2 * i + (lane >> 5);
      pre[i] = !extra_slot && part < np ? rec[part].keys[lane & 31] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < kLdsPairs; ++i) pair_keys[wv][i][lane] = pre[i];
    wave_sync();
  }
  // The chosen raw logit: captured by the reduction's idle workgroups when it
  // had some (see reduce_kernel), else read from the row.
  const bool xt_valid = chosen_captured(p, rplan);
  float x_tok = 0.0f;
  if (lane == 0 && tok >= 0 && tok < V) x_tok = xt_valid ? xt_spec : load_elem<DT>(rowp, tok);
  int sel_id[2] = {0, 0};
  float x_sel[2] = {0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    if (j < n_sel) {
      sel_id[h] = ids_spec[h];
      if (sel_id[h] >= 0 && sel_id[h] < V) x_sel[h] = load_elem<DT>(rowp, sel_id[h]);
    }
  }

  // ---- L, one lane per part
  const float M = wave_max(pm, lane);
  float term = 0.0f;
  if (lane < np && pm != kNegInf) term = ps * __builtin_amdgcn_exp2f((pm - M) * kLog2e);
  const float L = M + logf(wave_sum(term, lane));
  if (lead && lane == 0) {
    p.lse[row] = L;
    out[0] = tok;
    out[1] = (int32_t)(tok >= 0 && tok < V ? __float_as_uint(reported(x_tok, L)) : kNanBits);
  }
  if (SCORE) {
    const float rt = reported(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x_tok), 0)), L);
    bool tie = lane < np && p_next < __builtin_huge_valf() && reported(p_next, L) == rt;
    if (DT == 0 && tie && !(p_next2 < __builtin_huge_valf() && reported(p_next2, L) == rt)) {
      // Only the lanes at x_n tie with the target: the next larger value
      // already reports more, so the overcount is their number.
      p_above -= p_count;
      tie = false;
    }
    uint64_t ties = __ballot(tie);
    if (lead && lane == 0) p.guard[row] = __popcll(ties);
    while (ties != 0ull) {
      const int part = __builtin_ctzll(ties);
      ties &= ties - 1ull;
      const int lo = part_u0[part] * kUnitElems;
      int hi = part_u0[part + 1] * kUnitElems;
      hi = hi < V ? hi : V;
      const int exact = count_above<DT, VEC>(rowp, lo, hi, L, rt, lane);
      if (lane == part) p_above = exact;
    }
    const int greater = wave_sum_i32(lane < np ? p_above : 0, lane);
    if (lead && lane == 0) out[2] = 1 + greater;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    if (!SCORE && lead && j < n_sel) {
      const uint32_t bits = sel_id[h] >= 0 && sel_id[h] < V ? __float_as_uint(reported(x_sel[h], L))
                                                            : kNanBits;
      *(int2*)(out + 2 + 2 * j) = make_int2(sel_id[h], (int32_t)bits);
    }
  }
  if (!natural) {
    if (!SCORE && lead && lane == 0) p.guard[row] = 0;
    return;
  }

  // ---- kept candidates re-keyed by F, two parts (64 keys) per step
  const int K = p.K;
  const int Keff = K < V ? K : V;
  // Two independent chains (pairs 0, 2, 4, ... and 1, 3, 5, ...) merged at
  // the end, so that a row of many parts pays half the dependent steps.
  uint64_t top;
  if (wide) {
    uint64_t tw = 0ull;
#pragma unroll
    for (int i = 0; i < kWidePairs; ++i) {
      if (2 * (wv + i * kMergeWaves) >= np) break;
      const uint64_t sk = sort_halves_desc(wraw[i] != 0ull ? final_key(wraw[i], L) : 0ull, lane);
      tw = i == 0 ? sk : merge_top32(tw, sk, lane);
    }
    if (lane < kKeep) wide_lists[WIDE ? wv : 0][lane] = tw;
    __syncthreads();
    if (wv != 0) return;
    top = lane < kKeep ? wide_lists[0][lane] : 0ull;
#pragma unroll
    for (int i = 1; i < kMergeWaves; ++i)
      top = merge_top32(top, lane < kKeep ? wide_lists[WIDE ? i : 0][lane] : 0ull, lane);
  } else if (!lead) {
    return;
  } else if (np <= 2) {
    top = sort_halves_desc(raw0 != 0ull ? final_key(raw0, L) : 0ull, lane);
  } else {
    uint64_t ta = raw0 != 0ull ? final_key(raw0, L) : 0ull;
    uint64_t tb = raw1 != 0ull ? final_key(raw1, L) : 0ull;
    sort_halves_desc2(ta, tb, lane);
    for (int pb = 4; pb < np; pb += 4) {
      uint64_t r[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = pb + 2 * h;
        const int part = q + (lane >> 5);
        r[h] = 0ull;
        if (q < 4 + 2 * kLdsPairs) r[h] = q < np ? pair_keys[wv][(q - 4) >> 1][lane] : 0ull;
        else if (!extra_slot && part < np) r[h] = rec[part].keys[lane & 31];
      }
      uint64_t ka = r[0] != 0ull ? final_key(r[0], L) : 0ull;
      uint64_t kb = r[1] != 0ull ? final_key(r[1], L) : 0ull;
      sort_halves_desc2(ka, kb, lane);
      ta = merge_top32(ta, ka, lane);
      tb = merge_top32(tb, kb, lane);
    }
    top = merge_top32(ta, tb, lane);
  }
  // ---- guard, one lane per part
  const uint64_t FK = readlane64(top, Keff - 1);
  bool bad = false;
  if (lane < np && c_key != 0ull) {
    const float xc = key_value(c_key);
    bool ok = final_key(c_key, L) <= FK;
    if (ok && xc != kNegInf) ok = ukey32(reported(E::pred(xc), L)) < (uint32_t)(FK >> 32);
    bad = !ok;
  }
  const uint64_t unsafe = __ballot(bad);
  if (!SCORE && lane == 0) p.guard[row] = __popcll(unsafe);
  if (unsafe != 0ull) {
    // Rebuild from the safe parts' candidates plus every lane of each unsafe
    // part whose final key reaches FK.
    top = 0ull;
    for (int pb = 0; pb < np; pb += 2) {
      const int part = pb + (lane >> 5);
      uint64_t f = 0ull;
      if (!extra_slot && part < np && !((unsafe >> part) & 1ull)) {
        const uint64_t raw = rec[part].keys[lane & 31];
        if (raw != 0ull) f = final_key(raw, L);
      }
      top = merge_top32(top, sort64_desc(f, lane), lane);
    }
    uint64_t thr = FK;
    for (int part = 0; part < np; ++part) {
      if (!((unsafe >> part) & 1ull)) continue;
      const int lo = part_u0[part] * kUnitElems;
      int hi = part_u0[part + 1] * kUnitElems;
      hi = hi < V ? hi : V;
      rescan_lanes<DT, VEC>(top, thr, rowp, lo, hi, L, Keff, lane, &pair_keys[wv][0][0],
                            kLdsPairs * 64);
    }
  }
  if (lane < K) {
    int32_t id = -1;
    uint32_t bits = kNanBits;
    if (lane < Keff) {
      id = (int32_t)key_id(top);
      bits = __float_as_uint(unkey32((uint32_t)(top >> 32)));
    }
    if (SCORE) {  // after the rank word: pairs start at an odd word
      out[3 + 2 * lane] = id;
      out[4 + 2 * lane] = (int32_t)bits;
    } else {
      *(int2*)(out + 2 + 2 * lane) = make_int2(id, (int32_t)bits);
    }
  }
}

// ================================================================== reduce
constexpr int kWaves = kBlock / 64;  // 4 waves share each unit
constexpr int kStash = 128;          // hot chunks a wave can stash per unit
constexpr int kRecStage = 8;         // part records staged in LDS before they are written

// A finished part's record, held in LDS until the workgroup writes its
// records out: global stores issued while the stream's loads are in flight
// share the in-order memory counter with them and hold up the next waits.
struct StagedRec {
  PartRecord rec;
  int32_t dst;      // record index, row * units + the part's index in its row
  int32_t natural;  // whether the kept keys are meaningful
};

struct ReduceSmem {
  uint64_t pool[kWaves][kCandBuf];       // per-wave candidate buffers
  uint64_t chain_keys[2][kKeep];         // a part's best 32 over the waves arrived so far, by parity
  u32x4 stash[kWaves][kStash];           // hot chunks of the unit being reduced
  int16_t stash_off[kWaves][kStash];     // their chunk index c * 64 + lane
  uint64_t qbar[kWaves];                 // each wave's published ceil(K/4)-th key (see pub_key)
  uint64_t flush_cut[2][kWaves];         // a part's per-wave cut, by part parity
  float first_tau[2][kWaves];            // short ranges: the waves' first-unit thresholds, by parity
  float wm[2][kWaves];                   // a part's per-wave max and scaled sum
  float ws[2][kWaves];
  int wabove[2][kWaves];                 // scoring: a part's per-wave count above the target
  float wnext[2][kWaves];                // and smallest logit above it,
  int wcount[2][kWaves];                 // the lanes holding it (FP32)
  float wnext2[2][kWaves];               // and the next larger logit (FP32)
  int arrive[2];                         // waves that flushed the part of this parity
  int chain[2];                          // waves whose lists are folded into chain_keys
  int merged;                            // parts of the range merged into records
  int n_staged;                          // records staged in `staged`
  StagedRec staged[kRecStage];
  int scan[kWaves];
};

// A published key carries the number of the part it belongs to, so
// a wave never reads another part's bar: (value key << 32) | (part mod 4096)
// << 20 | ID, with IDs below 2^20 (at most 64 units of 16,384 lanes).
__device__ __forceinline__ uint64_t pub_key(uint64_t key, int part) {
  return (key & 0xFFFFFFFF00000000ull) | ((uint64_t)(part & 0xFFF) << 20) |
         (uint64_t)(key_id(key) & 0xFFFFFu);
}
// The key published for `part`, or 0.
__device__ __forceinline__ uint64_t pub_read(uint64_t pub, int part) {
  if (pub == 0ull || (int)((pub >> 20) & 0xFFF) != (part & 0xFFF)) return 0ull;
  return (pub & 0xFFFFFFFF00000000ull) | (uint64_t)(~(uint32_t)(pub & 0xFFFFFu));
}

// Where a unit sits: active row a, unit u of that row, slot s, frame
// position row = s T + t, and the logit row's address (packed or not).
struct UnitPos {
  int a, u, s, row;
  const char* rowp;
};

template <int DT>
__device__ __forceinline__ UnitPos locate(const Params& p, const int* prefix, int x, int lane) {
  UnitPos q;
  q.a = x / p.units;
  q.u = x - q.a * p.units;
  q.s = slot_of_wave(prefix, p.capacity, q.a, lane);
  const int t = q.a - (prefix[q.s] & kRowsMask);
  q.row = __builtin_amdgcn_readfirstlane(q.s * p.T + t);
  const int lrow =
      p.row_offsets ? __builtin_amdgcn_readfirstlane(prefix[p.capacity + 1 + q.s] + t) : q.row;
  q.rowp = (const char*)p.logits + (int64_t)lrow * p.V_pad * Elem<DT>::kBytes;
  return q;
}

// Chunk c of this lane in the wave's slice starting at wave_base; loff is
// the chunk's byte offset in the slice, (c * 64 + lane) * 16.  Row pointer
// and slice start are wave-uniform, so the interior load is an SGPR base plus
// a 32-bit lane offset.
template <int DT, bool VEC>
__device__ __forceinline__ u32x4 load_lane_chunk(const char* rowp, int64_t wave_base, uint32_t loff,
                                                 int c, int lane, int V, bool interior) {
  using E = Elem<DT>;
  if (VEC && interior) return *(const u32x4*)(rowp + wave_base * E::kBytes + loff);
  return load_chunk<DT, VEC>(rowp, wave_base + (int64_t)(c * 64 + lane) * E::kPer, V);
}

// Admission of a lane into a pool: by 64-bit key above a bar, or (a part's
// first unit) by value at or above a threshold.
struct Admit {
  bool by_key;
  uint64_t bar;
  float tau;
};
__device__ __forceinline__ bool admitted(const Admit& ad, float x, uint64_t key) {
  return ad.by_key ? key > ad.bar : x >= ad.tau;
}

// Hot chunks of the current unit, copied to the wave's LDS stash in
// compacted order (n may exceed kStash: then the stash is incomplete).
struct Stage {
  u32x4* stash;
  int16_t* off;
  int n;
};
__device__ __forceinline__ void stage_chunk(Stage& st, const u32x4& r, bool hot, int c, int lane) {
  const uint64_t m = __ballot(hot);
  if (m != 0ull) {
    const int n = __popcll(m);
    if (st.n + n <= kStash) {
      if (hot) {
        const int pos = st.n + lanes_below(m);
        st.stash[pos] = r;
        st.off[pos] = (int16_t)(c * 64 + lane);
      }
    }
    st.n += n;
  }
}

// Chunk test of the stash: a chunk is hot when its maximum exceeds `above`
// (the threshold itself when equality does not admit, else the float just
// below it), or, for a -inf threshold that admits equality, whenever it
// holds vocabulary (its first lane is below vlim, the slice's lane count).
struct HotTest {
  float above;
  bool every_lane;
  int vlim;
};
__device__ __forceinline__ HotTest hot_test(float tau, bool strict, int vlim) {
  HotTest h{tau, false, vlim};
  if (!strict) {
    if (tau == kNegInf) {
      h.every_lane = true;
    } else if (tau == 0.0f) {
      h.above = -__uint_as_float(1u);  // -0 and +0 both admit
    } else if (tau < __builtin_huge_valf()) {
      const uint32_t b = __float_as_uint(tau);
      h.above = __uint_as_float(tau > 0.0f ? b - 1u : b + 1u);
    } else {
      h.above = __uint_as_float(0x7F7FFFFFu);
    }
  }
  return h;
}
template <int kPer>
__device__ __forceinline__ bool is_hot(const HotTest& h, float mc, int c, int lane) {
  return h.every_lane ? (c * 64 + lane) * kPer < h.vlim : mc > h.above;
}

// Lanes at or past V of the chunk whose first lane is `first` read -inf.
template <int DT>
__device__ __forceinline__ u32x4 mask_tail(u32x4 r, int first, int V) {
#pragma unroll
  for (int j = 0; j < Elem<DT>::kPer; ++j) {
    if (first + j >= V) {
      if (DT == 1)
        r[j >> 1] = (j & 1) ? ((r[j >> 1] & 0x0000FFFFu) | 0xFF800000u)
                            : ((r[j >> 1] & 0xFFFF0000u) | 0xFF80u);
      else
        r[j] = 0xFF800000u;
    }
  }
  return r;
}

// Chunk c of a wave covers lanes [cbase, cbase + 64 kPer) of the row, lane l
// holding [cbase + l kPer, cbase + (l + 1) kPer).  Only the chunk that V
// falls in is masked lane by lane; a chunk wholly past V reads -inf and one
// wholly before it is left alone (both tests are wave-uniform).
template <int DT>
__device__ __forceinline__ u32x4 mask_chunk(u32x4 r, int cbase, int lane, int V) {
  constexpr int kPer = Elem<DT>::kPer;
  if (cbase + 64 * kPer <= V) return r;
  if (cbase >= V) {
    const uint32_t ninf = DT == 1 ? 0xFF80FF80u : 0xFF800000u;
    return u32x4{ninf, ninf, ninf, ninf};
  }
  return mask_tail<DT>(r, cbase + lane * kPer, V);
}

// A buffer resource over one logit row: loads past its `bytes` return zero
// without touching memory (the hardware range check covers the per-lane
// offset).  bytes = 0 makes every load a no-op.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const char* rowp, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)rowp, (short)0, bytes, 0x00020000);
}

// Cache policy of the stream's loads: streaming (each logit is read once).
constexpr int kSlc = 2;

// Refill chunk c of this lane with the next unit's slice at next_base.  With
// aligned rows every lane issues the same buffer load unconditionally, so the
// registers have one definition and the compiler's wait counts stay exact
// (no copies, no early waits); lanes past the row read zeros and are masked
// when the unit is reduced.  Unaligned rows read lane by lane.
template <int DT, bool VEC>
__device__ __forceinline__ void refill_chunk(u32x4& r, __amdgpu_buffer_rsrc_t rsrc,
                                             const char* next_rowp, int next_base, int c, int lane,
                                             int V, bool live) {
  using E = Elem<DT>;
  const int first = next_base + (c * 64 + lane) * E::kPer;
  if (VEC) {
    r = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, first * E::kBytes, 0, kSlc));
  } else if (live) {
    r = load_chunk<DT, false>(next_rowp, first, V);
  }
}

// One unit's statistics pass over a wave's registers: exp2 against the
// running max (or the unit's first chunk max), lane and chunk maxima on the
// side.  Each chunk's registers are refilled with the same chunk of the next
// unit as soon as they have been used, so a unit's loads are always in
// flight behind the current unit's arithmetic; with `stage` a chunk whose
// maximum passes the test is stashed first.
// Maximum of the eight chunk maxima in four instructions.  The maxima come
// out of v_max3 chains (never signalling NaNs), so the canonicalising moves
// the compiler would put before each fmaxf of a value it cannot trace (nine
// per unit) are not needed.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8(const float (&cm)[kChunks]) {
  static_assert(kChunks == 8, "eight chunks per lane");
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(cm[6]), "v"(cm[7]));
  return vmax3(vmax3(cm[0], cm[1], cm[2]), vmax3(cm[3], cm[4], cm[5]), r);
}

struct PassOut {
  float acc, lm, mref, nb;
  float tau;  // a first unit's threshold
};

// With `first` (a part's first unit, no bar yet) the pass sweeps the
// registers twice: the chunk maxima first, whose kq-th largest lane maximum
// (read from the 16-bit key prefix; -inf when fewer than kq lanes hold
// vocabulary) becomes the unit's threshold, then the statistics, staging
// the chunks that reach the threshold.  The first sweep waits for the whole
// unit, which only delays that unit's refills.  `ht`, `stage` and `o.tau`
// return the threshold and its test.
// With SCORE, a chunk whose maximum exceeds xa (the target's logit) also
// adds its lanes above xa to `above` and their minimum to `next_above`
// (FP32: with the count of lanes at that minimum and the next larger value).
template <int DT, bool VEC, bool SCORE>
__device__ __forceinline__ PassOut unit_pass(u32x4 (&raw)[kChunks], float (&cm)[kChunks],
                                             float m_l, bool tail, int wave_base,
                                             __amdgpu_buffer_rsrc_t next_rsrc,
                                             const char* next_rowp, int next_base, bool has_next,
                                             int V, int lane, bool& stage, HotTest& ht, Stage& st,
                                             bool first, int kq, float xa, int& above,
                                             float& next_above, int& next_count, float& next2,
                                             float* tau_base, int tau_off) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  PassOut o;
  o.tau = kNegInf;
  if (first) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (VEC && tail) raw[c] = mask_chunk<DT>(raw[c], wave_base + c * 64 * kPer, lane, V);
      float mc = E::get(raw[c], 0);
#pragma unroll
      for (int j = 1; j < kPer; ++j) mc = fmaxf(mc, E::get(raw[c], j));
      cm[c] = mc;
    }
    const float lm = max8(cm);
    const bool voter = wave_base + lane * kPer < V;
    const int nv = __popcll(__ballot(voter));
    o.tau = nv >= kq ? key_floor16(wave_kth_largest16(ukey32(lm) >> 16, voter, kq)) : kNegInf;
    if (!SCORE && tau_off >= 0) {
      // One- and two-unit ranges: every wave admits down to the smallest of
      // the waves' thresholds (waves without vocabulary left out).  Each
      // wave holding vocabulary has kq lanes at or above its own, so the part
      // keeps at least K lanes at or above that smallest one, and its cut
      // cannot sit above the row's K-th value, while the waves admit far
      // fewer lanes than K each.
      const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
      if (lane == 0) tau_base[tau_off + wv] = nv > 0 ? o.tau : __builtin_huge_valf();
      __syncthreads();
      float t = tau_base[tau_off];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) t = fminf(t, tau_base[tau_off + i]);
      o.tau = t;
    }
    ht = hot_test(o.tau, false, ht.vlim);
    stage = !ht.every_lane;
  }
  if (VEC && tail) raw[0] = mask_chunk<DT>(raw[0], wave_base, lane, V);
  float c0 = E::get(raw[0], 0);
#pragma unroll
  for (int j = 1; j < kPer; ++j) c0 = fmaxf(c0, E::get(raw[0], j));
  o.mref = fmaxf(m_l, c0);
  o.nb = -o.mref * kLog2e;
  o.acc = 0.0f;
  // Byte offsets of this lane's chunks 0 and 4 in the next unit's row (each
  // chunk of the wave is 64 lanes x 16 bytes further on).
  uint32_t vo_lo = (uint32_t)((next_base + lane * kPer) * E::kBytes);
  uint32_t vo_hi = vo_lo + 4u * 1024u;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    // Empty asm statements only add data dependencies: chunk c is not
    // unpacked before chunk c - 1 is summed, and its registers are refilled
    // only after their last use, so the refill lands in the same registers.
    if (c > 0) {
      asm volatile("" : "+v"(raw[c]) : "v"(o.acc), "v"(cm[c - 1]));
      if (VEC && tail) raw[c] = mask_chunk<DT>(raw[c], wave_base + c * 64 * kPer, lane, V);
    }
    float mc = kNegInf;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float xv = E::get(raw[c], j);
      mc = fmaxf(mc, xv);
      o.acc += __builtin_amdgcn_exp2f(__builtin_fmaf(xv, kLog2e, o.nb));
    }
    cm[c] = mc;
    if (SCORE && __ballot(mc > xa) != 0ull) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const float xv = E::get(raw[c], j);
        const bool gt = xv > xa;
        above += gt ? 1 : 0;
        if (DT == 0) {
          // FP32 also keeps how many lanes hold that smallest value and the
          // next larger value (see the merge's rank).
          const bool lt = gt && xv < next_above, eq = gt && xv == next_above;
          next2 = lt ? next_above : ((gt && !eq && xv < next2) ? xv : next2);
          next_count = lt ? 1 : (eq ? next_count + 1 : next_count);
          next_above = lt ? xv : next_above;
        } else {
          next_above = gt ? fminf(next_above, xv) : next_above;
        }
      }
    }
    if (stage) stage_chunk(st, raw[c], mc > ht.above, c, lane);
    if (VEC) {
      // The empty asm takes the offset register as rewritten after the
      // chunk's last use, so the refill cannot move above it; chunks 0-3
      // and 4-7 share one offset each (the rest is the immediate field).
      uint32_t& vo = c < 4 ? vo_lo : vo_hi;
      asm volatile("" : "+v"(vo) : "v"(o.acc), "v"(mc), "v"(raw[c]));
      raw[c] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(next_rsrc, vo + (uint32_t)(c & 3) * 1024u, 0, kSlc));
    } else {
      int lane_dep = lane;
      asm volatile("" : "+v"(lane_dep) : "v"(o.acc), "v"(mc), "v"(raw[c]));
      refill_chunk<DT, VEC>(raw[c], next_rsrc, next_rowp, next_base, c, lane_dep, V, has_next);
    }
  }
  o.lm = max8(cm);
  return o;
}

// Expand the stashed chunks one lane per element into the pool.
template <int DT>
__device__ __forceinline__ void expand_stash(CandBuf& cb, Best32& best, const Stage& st,
                                             int64_t wave_base, int V, int lane, const Admit& ad) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  constexpr int kPerRound = 64 / kPer;  // entries expanded per 64 lanes
  wave_sync();
  const int cnt = st.n;
  for (int s0 = 0; s0 < cnt; s0 += kPerRound) {
    const int i = s0 + lane / kPer, j = lane % kPer;
    uint64_t k = 0ull;
    if (i < cnt) {
      const int64_t id = wave_base + (int64_t)st.off[i] * kPer + j;
      const uint32_t bits = DT == 1 ? (uint32_t)((const uint16_t*)&st.stash[i])[j] << 16
                                    : ((const uint32_t*)&st.stash[i])[j];
      const float x = __uint_as_float(bits);
      const uint64_t key = make_key(x, (uint32_t)id);
      if (id < V && admitted(ad, x, key)) k = key;
    }
    cand_append(cb, best, k, lane);
  }
  wave_sync();  // the next unit may overwrite the stash
}

// Every chunk of the wave's slice, read again from memory (the stash
// overflowed: more hot chunks than it holds, e.g. a run of ties).  One key
// per lane per step keeps the register footprint small; the next chunk's
// load is in flight while a chunk is expanded.
template <int DT, bool VEC>
__device__ __forceinline__ void expand_global(CandBuf& cb, Best32& best, const char* rowp,
                                              int64_t wave_base, int V, int lane, const Admit& ad) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  u32x4 r = load_chunk<DT, VEC>(rowp, wave_base + (int64_t)lane * kPer, V);
  for (int c = 0; c < kChunks; ++c) {
    const int64_t first = wave_base + (int64_t)(c * 64 + lane) * kPer;
    const u32x4 cur = r;
    if (c + 1 < kChunks) r = load_chunk<DT, VEC>(rowp, first + 64 * kPer, V);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float x = E::get(cur, j);
      const uint64_t key = make_key(x, (uint32_t)(first + j));
      cand_append(cb, best, (first + j < V && admitted(ad, x, key)) ? key : 0ull, lane);
    }
  }
  // Leave no load outstanding, so that the stream's wait counts stay exact
  // where this rare path rejoins it.
  __builtin_amdgcn_s_waitcnt(0);
}

// The lane index as a value the compiler cannot prove loop-invariant: lane
// offsets derived from it are recomputed where used instead of being hoisted
// out of the round loop and spilled.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// Issue priority of a workgroup as it consumes its unit range.  The wave
// arbiter of a CU favours the oldest waves, so with equal priorities the
// workgroups dispatched first race through their ranges while the youngest
// lag and set the end of the launch; lowering the priority as a range is
// consumed hands issue slots to the workgroups that are behind.  A range of
// up to kShortRange units keeps priority 3 until its last three units and
// then steps down one level per unit (a short range's lag is a unit or two,
// settled at its end); a longer one steps down by quarters.  The step
// points are computed once per range (no division per unit).
constexpr int kShortRange = 16;
struct Quarters {
  int q1, q2, q3;
};
__device__ __forceinline__ Quarters range_quarters(int x0, int x1) {
  const int64_t n = x1 - x0;
  if (n <= kShortRange) return Quarters{x1 - 3, x1 - 2, x1 - 1};
  return Quarters{x0 + (int)((n + 3) >> 2), x0 + (int)((2 * n + 3) >> 2), x0 + (int)((3 * n + 3) >> 2)};
}
__device__ __forceinline__ void progress_priority(int x, const Quarters& q) {
  if (x < q.q1) __builtin_amdgcn_s_setprio(3);
  else if (x < q.q2) __builtin_amdgcn_s_setprio(2);
  else if (x < q.q3) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ uint64_t lds_load64(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store64(uint64_t* a, uint64_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Four waves per workgroup, five workgroups per CU: at most 96 VGPRs per lane.
template <int DT, bool VEC, bool SCORE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(5))) void reduce_kernel(
    Params p) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  constexpr int kWaveElems = 64 * kChunks * kPer;
  constexpr int kUnitElems = kWaves * kWaveElems;
  __shared__ ReduceSmem sh;
  extern __shared__ int prefix[];

  // The set-up runs at the priority of a range's first units: workgroups
  // dispatched later compete on equal terms with the earlier ones, which are
  // already streaming, to issue their first loads.
  __builtin_amdgcn_s_setprio(3);
  {
    // The arguments of the set-up, all fetched before the first is needed:
    // one wait for the argument block instead of one per use.
    const void* a0 = p.requested;
    const void* a1 = p.crecords;
    const void* a2 = p.emitted;
    const void* a3 = p.id_counts;
    const void* a4 = p.row_offsets;
    const void* a5 = p.tokens;
    const void* a6 = p.logits;
    const void* a7 = p.slot_rows;
    const void* a8 = p.records;
    asm volatile("" ::"s"(a0), "s"(a1), "s"(a2), "s"(a3), "s"(a4), "s"(a5), "s"(a6), "s"(a7), "s"(a8),
                 "s"(p.capacity), "s"(p.T), "s"(p.V), "s"(p.K), "s"(p.units), "s"(p.workers),
                 "s"(p.emitted_field), "s"(p.packed_rows), "s"(p.V_pad));
  }
  const int tid = threadIdx.x, lane_id = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = p.V, U = p.units;
  if (tid < kWaves) sh.qbar[tid] = 0ull;  // ordered by the barriers below
  if (tid < 2) sh.arrive[tid] = 0;
  if (tid < 2) sh.chain[tid] = 0;
  if (tid == 0) sh.merged = 0;
  if (tid == 0) sh.n_staged = 0;
  const int total = build_prefix<kWaves, SCORE>(p, prefix, sh.scan);
  // The slots' active-row counts before them, and the total, for the merge.
  if (blockIdx.x == 0)
    for (int s = tid; s <= p.capacity; s += kBlock) p.slot_rows[s] = prefix[s] & kRowsMask;
  // This workgroup's range of the N < 2^31 units (the host checks N).
  const int N = total * U;
  const RangePlan rplan = range_plan(total, U, p.workers);
  if ((int)blockIdx.x >= rplan.count) {
    // A workgroup with no units captures chosen raw logits for the merge,
    // one active position per thread, when the idle ones cover them all.
    if (chosen_captured(p, rplan)) {
      const int q = ((int)blockIdx.x - rplan.count) * kBlock + tid;
      if (q < p.capacity * p.T) {
        const int s = q / p.T, t = q - s * p.T;
        if (t < (prefix[s + 1] & kRowsMask) - (prefix[s] & kRowsMask)) {
          const int tok = token_of(p, s, t);
          const int lrow = p.row_offsets ? prefix[p.capacity + 1 + s] + t : q;
          if (tok >= 0 && tok < V)
            p.xtok[q] = load_elem<DT>((const char*)p.logits + (int64_t)lrow * p.V_pad * E::kBytes, tok);
        }
      }
    }
    return;
  }
  // The range, and the index of its first part among its row's parts (the
  // slot of the part's record): parts are numbered by where they start.
  int x0, x1, part_idx;
  if (rplan.pieces) {
    const int b = (int)blockIdx.x;
    int row, piece;
    if (b < total * rplan.pieces) {
      row = b % total;
      piece = b / total;
    } else {
      row = total - rplan.extra + (b - total * rplan.pieces);
      piece = rplan.pieces;
    }
    const int q = rplan.pieces + (row >= total - rplan.extra ? 1 : 0);
    x0 = row * U + piece * U / q;
    x1 = row * U + (piece + 1) * U / q;
    part_idx = piece;
  } else {
    // floor(b N / count) in double precision: b N < 2^53 is exact, and a
    // quotient that is not an integer lies at least 1 / count from one, far
    // beyond the division's rounding error, so the floor is exact.
    const double b = (double)blockIdx.x, n = (double)N, c = (double)rplan.count;
    x0 = (int)__builtin_floor(b * n / c);
    x1 = (int)__builtin_floor((b + 1.0) * n / c);
    // Ranges start at distinct units (count <= N), so ranges 0..b are the
    // ones starting at or before x0, and ceil((r + 1) count / N) of them
    // start at or before unit r: the row's first unit r = (x0 / U) U starts
    // part 0, and each range start after it one more part.
    const double r1 = (double)((x0 / U) * U + 1);
    part_idx = (int)blockIdx.x + 1 - (int)__builtin_ceil(r1 * c / n);
  }
  if (x0 >= x1) return;
  const bool short_ranges = N < 2 * p.workers;

  UnitPos cur = locate<DT>(p, prefix, x0, lane_id);
  // The current part's first unit (bits 0-7; U <= 64) and its index among
  // its row's parts (bits 8 up).
  int part_tag = cur.u | part_idx << 8;
  const int row_bytes = (int)(p.V_pad * E::kBytes);
  u32x4 raw[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    refill_chunk<DT, VEC>(raw[c], row_rsrc(cur.rowp, row_bytes), cur.rowp,
                          cur.u * kUnitElems + w * kWaveElems, c, lane_id, V, true);
  bool natural = p.K > 0 && (prefix[cur.s] & kSelBit) == 0;

  // Scoring: lane i holds the target logit of the range's i-th row (the
  // host keeps a range within kMaxRangeRows rows); each lane counts its
  // part's lanes above it.  The targets come from the slot table, so each
  // target logit's load follows the first unit's at once instead of after a
  // round trip for the target queued behind the whole unit.
  const int a_first = x0 / U;
  float xa_lane = 0.0f;
  if (SCORE) {
    const int a = a_first + lane_id;
    if (lane_id < kMaxRangeRows && (int64_t)a * U < x1) {
      const int s = slot_of(prefix, p.capacity, a);
      xa_lane = load_elem<DT>((const char*)p.logits + (int64_t)s * p.V_pad * E::kBytes,
                              prefix[p.capacity + 1 + s]);
    }
  }
  int above = 0;
  float next_above = __builtin_huge_valf();
  int next_count = 0;
  float next2 = __builtin_huge_valf();

  // Per lane: running max m_l and the sum, relative to m_l, of exp over the
  // lane's values except one occurrence of m_l (whose term is exactly 1 and
  // is added back when the lanes are combined).
  float m_l = kNegInf, s_l = 0.0f;
  // Bars rank by the call's K (K <= 32): a part's K-th key bounds what can
  // still enter the row's top K.
  const int K = p.K;
  const int kq = (K + kWaves - 1) / kWaves;  // published per-wave rank
  Best32 best{0ull, 0, K, 0ull};
  CandBuf cb{&sh.pool[w][0], 0};
  Stage st{&sh.stash[w][0], &sh.stash_off[w][0], 0};
  uint64_t published = 0ull;
  int part_seq = 0;  // parts of the range finished by this wave
  // The part's first-unit threshold as a key bar: a later lane passes it iff
  // its value is at least the threshold (0: none).
  uint64_t first_bar = 0ull;
  // Largest key this wave's share of the part may have dropped beyond the
  // part's K-th kept key (its first-unit bar).
  uint64_t cut = 0ull;

  const Quarters quarters = range_quarters(x0, x1);
  for (int x = x0; x < x1; ++x) {
    progress_priority(x, quarters);
    const int lane = opaque_lane(lane_id);
    const bool has_next = x + 1 < x1;
    UnitPos nxt = cur;
    if (has_next) {
      if (cur.u + 1 < U) nxt.u = cur.u + 1;
      else nxt = locate<DT>(p, prefix, x + 1, lane);
    }
    const bool part_ends = !has_next || nxt.a != cur.a;
    const bool part_starts = cur.u == (part_tag & 0xff);
    const int wave_base = cur.u * kUnitElems + w * kWaveElems;
    const int next_base = nxt.u * kUnitElems + w * kWaveElems;
    const bool tail = wave_base + kWaveElems > V;  // the slice reaches past V

    // ---- admission bar known before the pass: the wave's own K-th best
    // key, or the smallest of the four waves' published ceil(K/4)-th keys of
    // this part (K keys of the part lie at or above it), the larger.
    Admit ad{false, 0ull, kNegInf};
    float tau = kNegInf;
    bool strict = false;
    if (natural && !part_starts) {
      // Every lane reads the same words (all four loads in flight at once);
      // decode them as scalars.
      uint64_t qv[kWaves];
#pragma unroll
      for (int i = 0; i < kWaves; ++i) qv[i] = lds_load64(&sh.qbar[i]);
      uint64_t bq = pub_read(readlane64(qv[0], 0), part_seq);
#pragma unroll
      for (int i = 1; i < kWaves; ++i) {
        const uint64_t b = pub_read(readlane64(qv[i], 0), part_seq);
        bq = b < bq ? b : bq;
      }
      uint64_t bar = best.bar;
      bar = bq > bar ? bq : bar;
      bar = first_bar > bar ? first_bar : bar;
      if (bar != 0ull) {
        ad.by_key = true;
        ad.bar = bar;
        tau = key_value(bar);
        // A lane of this unit equal in value to the bar has a larger ID
        // whenever the bar's lane precedes the wave's slice.
        strict = key_id(bar) < (uint32_t)wave_base;
      }
    }
    const int vlim = V - wave_base <= 0 ? 0 : (V - wave_base < kWaveElems ? V - wave_base : kWaveElems);
    HotTest ht = hot_test(tau, strict, vlim);
    // Stash while streaming only with a bar that a chunk maximum can test; a
    // part's first unit finds its threshold in the pass itself.
    bool stage = natural && ad.by_key && !ht.every_lane;
    // Keys each wave admits in a part's first unit: ceil(K / waves holding
    // vocabulary), so that the part keeps at least K.  When the ranges are
    // one or two units long no later unit of the part can refine a wave's
    // threshold, and a wave holding several of the row's best lanes would
    // leave a cut above the row's K-th value: there the waves share the
    // smallest of their thresholds (unit_pass), or, in the scoring kernels
    // (whose registers are fuller), each wave admits K lanes.
    const int ubase = cur.u * kUnitElems;
    const int nw = V - ubase >= kUnitElems ? kWaves : (V - ubase + kWaveElems - 1) / kWaveElems;
    const int kfirst = SCORE && short_ranges ? K
                       : (nw == kWaves ? kq : (nw == 3 ? (K + 2) / 3 : (nw == 2 ? (K + 1) >> 1 : K)));

    st.n = 0;
    float cm[kChunks];
    const float xa =
        SCORE ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(xa_lane), cur.a - a_first))
              : 0.0f;
    const PassOut po = unit_pass<DT, VEC, SCORE>(
        raw, cm, m_l, tail, wave_base, row_rsrc(nxt.rowp, has_next ? row_bytes : 0), nxt.rowp,
        next_base, has_next, V, lane, stage, ht, st, natural && part_starts, kfirst, xa, above,
        next_above, next_count, next2, &sh.first_tau[0][0],
        short_ranges ? (part_seq & 1) * kWaves : -1);
    const float lm = po.lm;

    // ---- fold the unit into the lane's running (max, sum)
    {
      float mr = po.mref, nbr = po.nb, acc = po.acc;
      if (lm != kNegInf && !(acc < __builtin_huge_valf())) {
        // The reference was -inf or far below this unit's maximum: redo the
        // sum against the maximum, reading the lanes again.
        mr = lm;
        nbr = -lm * kLog2e;
        acc = 0.0f;
        for (int c = 0; c < kChunks; ++c) {
          const u32x4 r2 =
              load_chunk<DT, VEC>(cur.rowp, wave_base + (int64_t)(c * 64 + lane) * kPer, V);
#pragma unroll
          for (int j = 0; j < kPer; ++j)
            acc += __builtin_amdgcn_exp2f(__builtin_fmaf(E::get(r2, j), kLog2e, nbr));
        }
      }
      const bool any = lm != kNegInf;
      const bool up = lm > m_l;
      const float e_lm = __builtin_amdgcn_exp2f(__builtin_fmaf(lm, kLog2e, nbr));
      const float carry =
          m_l != kNegInf ? (1.0f + s_l) * __builtin_amdgcn_exp2f((m_l - mr) * kLog2e) : 0.0f;
      const float s_up = ((acc - e_lm) + carry) * __builtin_amdgcn_exp2f((mr - lm) * kLog2e);
      const float s_keep = s_l + acc;  // lm <= m_l implies mr == m_l
      s_l = any ? (up ? s_up : s_keep) : s_l;
      m_l = any && up ? lm : m_l;
    }

    // ---- candidates for this wave's pool
    if (natural) {
      if (part_starts) {
        // The part's first unit: admit lanes at or above the wave's k-th
        // largest lane maximum (lane maxima are distinct lanes, so at least
        // k lanes reach it; -inf when fewer than k lanes hold vocabulary),
        // which the pass found before staging against it.  Lanes below it
        // are covered by the wave's cut, which the merge's guard checks
        // against the row's K-th key.
        tau = po.tau;
        ad.by_key = false;
        ad.tau = tau;
        // As a key bar for the part's later units this admits values >= tau
        // (its low word ~ID = 0 belongs to no lane), so ties at tau stay.
        first_bar = tau == kNegInf ? 0ull : (uint64_t)ukey32(tau) << 32;
        cut = first_bar;
        if (!stage || st.n > kStash) expand_global<DT, VEC>(cb, best, cur.rowp, wave_base, V, lane, ad);
        else if (st.n > 0)
          expand_stash<DT>(cb, best, st, wave_base, V, lane, ad);
      } else if (!stage || st.n > kStash) {
        // No bar a chunk maximum can test, or more hot chunks than the stash
        // holds: every lane of the slice, read again.
        expand_global<DT, VEC>(cb, best, cur.rowp, wave_base, V, lane, ad);
      } else if (st.n > 0) {
        expand_stash<DT>(cb, best, st, wave_base, V, lane, ad);
      }
      cand_flush(cb, best, lane);
      const uint64_t b8 = best.n >= kq ? readlane64(best.top, kq - 1) : 0ull;
      if (b8 != published) {
        published = b8;
        if (lane == 0) lds_store64(&sh.qbar[w], pub_key(published, part_seq));
      }
    }

    if (part_ends) {
      // ---- this wave's share of the part record, in the buffers of the
      // part's parity once the part two back has been merged out of them
      const int b = part_seq & 1;
      if (part_seq >= 2) {
        while (__hip_atomic_load(&sh.merged, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
               part_seq - 1)
          __builtin_amdgcn_s_sleep(2);
      }
      {
        const float M = wave_max(m_l, lane);
        float term = 0.0f;
        if (m_l != kNegInf) term = (1.0f + s_l) * __builtin_amdgcn_exp2f((m_l - M) * kLog2e);
        const float S = wave_sum(term, lane);
        if (lane == 0) {
          sh.wm[b][w] = M;
          sh.ws[b][w] = S;
        }
        if (SCORE) {
          const int na = wave_sum_i32(above, lane);
          float nx = next_above;
          nx = fminf(nx, xlanef<32>(nx, lane));
          nx = fminf(nx, xlanef<16>(nx, lane));
          nx = fminf(nx, xlanef<8>(nx, lane));
          nx = fminf(nx, xlanef<4>(nx, lane));
          nx = fminf(nx, xlanef<2>(nx, lane));
          nx = fminf(nx, xlanef<1>(nx, lane));
          int nc = 0;
          float n2 = __builtin_huge_valf();
          if (DT == 0) {
            // lanes at the wave's minimum add their counts; the others offer
            // their minimum as a candidate for the next larger value
            nc = wave_sum_i32(next_above == nx ? next_count : 0, lane);
            n2 = next_above == nx ? next2 : next_above;
            n2 = fminf(n2, xlanef<32>(n2, lane));
            n2 = fminf(n2, xlanef<16>(n2, lane));
            n2 = fminf(n2, xlanef<8>(n2, lane));
            n2 = fminf(n2, xlanef<4>(n2, lane));
            n2 = fminf(n2, xlanef<2>(n2, lane));
            n2 = fminf(n2, xlanef<1>(n2, lane));
          }
          if (lane == 0) {
            sh.wabove[b][w] = na;
            sh.wnext[b][w] = nx;
            sh.wcount[b][w] = nc;
            sh.wnext2[b][w] = n2;
          }
        }
      }
      // Every key this wave kept is at or above its first-unit threshold, so
      // once it holds K of them the lanes below the threshold rank below its
      // K-th key, which the part's K-th kept key bounds: no cut of its own.
      if (lane == 0) sh.flush_cut[b][w] = natural && best.n < K ? cut : 0ull;
      // The last wave to arrive writes the record.
      int old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(&sh.arrive[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
      old = __builtin_amdgcn_readfirstlane(old);
      // The waves fold their lists into one in the order they arrive, each
      // merging its own into the fold of the earlier ones: the best 32 of a
      // set of distinct keys does not depend on the order, and the last wave
      // merges one list instead of all four.
      uint64_t top = 0ull;
      if (natural) {
        top = lane < kKeep ? best.top : 0ull;
        if (old > 0) {
          while (__hip_atomic_load(&sh.chain[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < old)
            __builtin_amdgcn_s_sleep(1);
          top = merge_top32(top, lane < kKeep ? sh.chain_keys[b][lane] : 0ull, lane);
        }
        if (old < kWaves - 1) {
          if (lane < kKeep) sh.chain_keys[b][lane] = top;
          if (lane == 0)
            __hip_atomic_store(&sh.chain[b], old + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      if (old == kWaves - 1) {
        const int slot = __builtin_amdgcn_readfirstlane(sh.n_staged);
        StagedRec* sr = &sh.staged[slot];
        PartRecord* rec = &sr->rec;
        // The range's last part is written straight from registers (nothing
        // streams after it); earlier parts are staged in LDS and written in
        // batches, so that no store sits among the stream's loads.
        const bool direct = !SCORE && !has_next;
        const int held = natural ? __popcll(__ballot(lane < kKeep && top != 0ull)) : 0;
        if (natural && lane < kKeep && !direct) rec->keys[lane] = top;
        // The waves' statistics, lane i < kWaves reading wave i's, all loads
        // at once; S adds the waves' terms in wave order as a sum in one lane
        // would.
        const float wmv = lane < kWaves ? sh.wm[b][lane] : kNegInf;
        const float wsv = lane < kWaves ? sh.ws[b][lane] : 0.0f;
        const uint64_t wcv = lane < kWaves ? sh.flush_cut[b][lane] : 0ull;
        float M = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wmv), 0));
#pragma unroll
        for (int i = 1; i < kWaves; ++i)
          M = fmaxf(M, __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wmv), i)));
        const float term =
            M != kNegInf && wmv != kNegInf ? wsv * __builtin_amdgcn_exp2f((wmv - M) * kLog2e) : 0.0f;
        float S = 0.0f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i)
          S += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(term), i));
        // Every lane the part dropped has a key at most the part's K-th kept
        // key or one of its waves' cuts.
        uint64_t pcut = held >= K ? readlane64(top, K - 1) : 0ull;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
          const uint64_t c = readlane64(wcv, i);
          pcut = c > pcut ? c : pcut;
        }
        if (lane == 0) {
          int na = 0, nc = 0;
          float nx = __builtin_huge_valf(), n2 = __builtin_huge_valf();
          if (SCORE) {
            for (int i = 0; i < kWaves; ++i) {
              na += sh.wabove[b][i];
              nx = fminf(nx, sh.wnext[b][i]);
            }
            for (int i = 0; i < kWaves; ++i) {
              nc += sh.wnext[b][i] == nx ? sh.wcount[b][i] : 0;
              n2 = fminf(n2, sh.wnext[b][i] == nx ? sh.wnext2[b][i] : sh.wnext[b][i]);
            }
            // FP32 scoring: key slot 31 (beyond the K = 20 the merge uses)
            // carries the next larger value and the count at the minimum.
            if (DT == 0) rec->keys[kKeep - 1] = ((uint64_t)__float_as_uint(n2) << 32) | (uint32_t)nc;
          }
          if (!direct) {
            rec->m = M;
            rec->s = S;
            rec->above = na;
            rec->next_above = nx;
            rec->cut = pcut;
            sr->dst = cur.row * U + (part_tag >> 8);
            sr->natural = natural;
          }
          sh.n_staged = (slot + 1 == kRecStage || !has_next) ? 0 : slot + 1;
          sh.arrive[b] = 0;
          sh.chain[b] = 0;
          __hip_atomic_store(&sh.merged, part_seq + 1, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // Write the staged records out once the stage is full, and at the end
        // of the range.
        if (slot + 1 == kRecStage || !has_next) {
          wave_sync();
          const int staged = direct ? slot : slot + 1;
          for (int r = 0; r < staged; ++r) {
            const StagedRec& s = sh.staged[r];
            const int words = __builtin_amdgcn_readfirstlane(s.natural) ? 3 + kKeep : 3;
            if (lane < words)
              ((uint64_t*)(p.records + __builtin_amdgcn_readfirstlane(s.dst)))[lane] =
                  ((const uint64_t*)&s.rec)[lane];
          }
        }
        if (direct) {
          // Header words (m, s), (above, next_above), cut; then the kept keys.
          uint64_t* g = (uint64_t*)(p.records + (cur.row * U + (part_tag >> 8)));
          const uint64_t hdr =
              lane == 0 ? ((uint64_t)__float_as_uint(S) << 32) | __float_as_uint(M)
                        : (lane == 1 ? (uint64_t)__float_as_uint(__builtin_huge_valf()) << 32 : pcut);
          if (lane < 3) g[lane] = hdr;
          if (natural && lane < kKeep) g[3 + lane] = top;
        }
      }
      ++part_seq;
      // ---- next part
      if (has_next) {
        m_l = kNegInf;
        s_l = 0.0f;
        best.top = 0ull;
        best.n = 0;
        best.bar = 0ull;
        published = 0ull;
        first_bar = 0ull;
        cut = 0ull;
        above = 0;
        next_above = __builtin_huge_valf();
        next_count = 0;
        next2 = __builtin_huge_valf();
        part_tag = nxt.u;  // a range's later parts start rows: index 0
        natural = p.K > 0 && (prefix[nxt.s] & kSelBit) == 0;
      }
    }
    cur = nxt;
  }
}

// =========================================================== vocabulary shards
// The pages' vocabulary-sharded variant keeps each tensor-parallel rank's
// logits as a vocabulary shard and exchanges, per position, each shard's max
// and exponential mass, the chosen token's raw logit from its owner, and each
// shard's best 32 sort keys or the selected IDs' raw logits; a final launch
// merges them into the same packed output (design page, vocabulary-sharded
// paragraph).  Here one GPU stands in for the ranks: a shard pass is the
// reduction on the shard's column slice followed by shard_finalize_kernel,
// which writes the record the rank would exchange; shard_merge_kernel reads
// the gathered records.  Keys rank raw logits (as in the unsharded path), so
// one exchange carries everything; only a shard that fails the exactness
// guard needs its lanes again (on one GPU the merge reads them directly).

// One wave per reduced position: the shard's parts combined into its record.
template <int DT>
__global__ __launch_bounds__(kMergeBlock) void shard_finalize_kernel(Params p) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = (int)blockIdx.x * kMergeWaves + wv;
  if (row >= p.capacity * p.T) return;
  const int s = row / p.T, t = row - s * p.T;
  const int req = p.requested[s], emi = emitted_of(p, s);
  const int cnt = p.id_counts ? p.id_counts[s] : 0;
  const int before = p.slot_rows[s], total = p.slot_rows[p.capacity];
  const int tok = token_of(p, s, t);
  const int rows_s = req == 0 ? 0 : (emi < 0 ? 0 : (emi > p.T ? p.T : emi));
  if (t >= rows_s) return;
  const int n_sel = cnt < 0 ? 0 : (cnt > 128 ? 128 : cnt);
  const bool natural = p.K > 0 && n_sel == 0;
  const int U = p.units, lo = p.shard_base, hi = p.shard_base + p.V;
  const PartRecord* rec = p.records + (int64_t)row * U;
  const char* rowp = (const char*)p.logits + (int64_t)row * p.V_pad * Elem<DT>::kBytes;
  ShardRecord* xr = p.xrec + (int64_t)row * p.shards + p.shard;

  // The row's parts in this shard's launch, as the merge finds them; part i's
  // record is the row's i-th.
  const int a = before + t;
  const RangePlan rplan = range_plan(total, U, p.workers);
  const bool start = lane < U && (lane == 0 || starts_range(a * U + lane, total, U, rplan));
  const int np = __popcll(__ballot(start));
  float pm = kNegInf, ps = 0.0f;
  uint64_t c_key = 0ull;
  if (lane < np) {
    pm = rec[lane].m;
    ps = rec[lane].s;
    c_key = rec[lane].cut;
  }
  const float M = wave_max(pm, lane);
  float term = 0.0f;
  if (lane < np && pm != kNegInf) term = ps * __builtin_amdgcn_exp2f((pm - M) * kLog2e);
  const float S = wave_sum(term, lane);

  // The shard's best 32 raw keys: every part's kept keys (sorted by raw key)
  // merged two parts at a time; keys that fall out bound what was dropped.
  uint64_t top = 0ull, cut = 0ull;
  int kept = 0;
  if (natural) {
    for (int pb = 0; pb < np; pb += 2) {
      const int part = pb + (lane >> 5);
      const uint64_t raw = part < np ? rec[part].keys[lane & 31] : 0ull;
      kept += __popcll(__ballot(raw != 0ull));
      top = merge_top32(top, sort_halves_desc(raw, lane), lane);
    }
    uint64_t c = c_key;
    c = xlane64<32>(c, lane) > c ? xlane64<32>(c, lane) : c;
    c = xlane64<16>(c, lane) > c ? xlane64<16>(c, lane) : c;
    c = xlane64<8>(c, lane) > c ? xlane64<8>(c, lane) : c;
    c = xlane64<4>(c, lane) > c ? xlane64<4>(c, lane) : c;
    c = xlane64<2>(c, lane) > c ? xlane64<2>(c, lane) : c;
    c = xlane64<1>(c, lane) > c ? xlane64<1>(c, lane) : c;
    cut = readlane64(c, 0);
    if (kept > kKeep) {
      const uint64_t k32 = readlane64(top, kKeep - 1);
      cut = k32 > cut ? k32 : cut;
    }
    // Global token IDs (the shard's lanes start at `lo`).
    if (top != 0ull) top = (top & 0xFFFFFFFF00000000ull) | (uint64_t)(~(key_id(top) + (uint32_t)lo));
    if (cut != 0ull && (uint32_t)cut != 0u)
      cut = (cut & 0xFFFFFFFF00000000ull) | (uint64_t)(~(key_id(cut) + (uint32_t)lo));
  }
  // The chosen token's and the owned selected IDs' raw logits.
  const bool own_tok = tok >= lo && tok < hi;
  float x_tok = 0.0f;
  if (lane == 0 && own_tok) x_tok = load_elem<DT>(rowp, tok - lo);
  uint32_t own_mask[2] = {0u, 0u};
  float x_sel[2] = {0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    bool own = false;
    if (j < n_sel) {
      const int id = p.ids[(int64_t)s * 128 + j];
      own = id >= lo && id < hi;
      if (own) x_sel[h] = load_elem<DT>(rowp, id - lo);
    }
    const uint64_t b = __ballot(own);
    own_mask[h] = 0u;
    if (lane == 0) own_mask[h] = 0u;
    if (lane < 2) own_mask[h] = (uint32_t)(b >> (32 * lane));
  }
  if (lane == 0) {
    xr->m = M;
    xr->s = S;
    xr->chosen = x_tok;
    xr->flags = own_tok ? 1 : 0;
    xr->cut = cut;
  }
  if (natural) {
    if (lane < kKeep) xr->keys[lane] = top;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = lane + 64 * h;
      if (j < n_sel) xr->sel[j] = x_sel[h];
      if (lane < 2) xr->owned[2 * h + lane] = own_mask[h];
    }
  }
}

// One wave per reduced position: L from the gathered shard records in shard
// order, the chosen and selected values from their owners' raw logits, and
// the natural top K over every shard's kept keys with the exactness guard
// per shard (an unsafe shard's lanes are streamed again).
template <int DT, bool VEC>
__global__ __launch_bounds__(kMergeBlock) void shard_merge_kernel(Params p) {
  __shared__ uint64_t buf[kMergeWaves][256];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = (int)blockIdx.x * kMergeWaves + wv;
  if (row >= p.capacity * p.T) return;
  const int s = row / p.T, t = row - s * p.T;
  const int req = p.requested[s], emi = emitted_of(p, s);
  const int cnt = p.id_counts ? p.id_counts[s] : 0;
  const int tok = token_of(p, s, t);
  const int rows_s = req == 0 ? 0 : (emi < 0 ? 0 : (emi > p.T ? p.T : emi));
  if (t >= rows_s) return;
  const int n_sel = cnt < 0 ? 0 : (cnt > 128 ? 128 : cnt);
  const bool natural = p.K > 0 && n_sel == 0;
  const int V = p.V, N = p.shards;
  const ShardRecord* xr = p.xrec + (int64_t)row * N;
  int32_t* out = p.out + (int64_t)row * p.row_words;
  const char* rowp = (const char*)p.logits + (int64_t)row * p.V_pad * Elem<DT>::kBytes;

  float pm = kNegInf, ps = 0.0f, pc = 0.0f;
  int pf = 0;
  uint64_t c_key = 0ull;
  if (lane < N) {
    pm = xr[lane].m;
    ps = xr[lane].s;
    pf = xr[lane].flags;
    pc = xr[lane].chosen;
    c_key = xr[lane].cut;
  }
  const float M = wave_max(pm, lane);
  float term = 0.0f;
  if (lane < N && pm != kNegInf) term = ps * __builtin_amdgcn_exp2f((pm - M) * kLog2e);
  const float L = M + logf(wave_sum(term, lane));
  const uint64_t owners = __ballot(lane < N && (pf & 1));
  if (lane == 0) {
    p.lse[row] = L;
    out[0] = tok;
    uint32_t bits = kNanBits;
    if (tok >= 0 && tok < V && owners != 0ull) {
      const float x = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pc), __builtin_ctzll(owners)));
      bits = __float_as_uint(reported(x, L));
    }
    out[1] = (int32_t)bits;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = lane + 64 * h;
    if (j < n_sel) {
      const int id = p.ids[(int64_t)s * 128 + j];
      uint32_t bits = kNanBits;
      if (id >= 0 && id < V) {
        // the owning shard, from the boundaries
        int r = (int)((int64_t)id * N / V);
        while (r + 1 < N && shard_lo(r + 1, V, N) <= id) ++r;
        while (r > 0 && shard_lo(r, V, N) > id) --r;
        if ((xr[r].owned[j >> 5] >> (j & 31)) & 1u) bits = __float_as_uint(reported(xr[r].sel[j], L));
      }
      *(int2*)(out + 2 + 2 * j) = make_int2(id, (int32_t)bits);
    }
  }
  if (!natural) {
    if (lane == 0) p.guard[row] = 0;
    return;
  }
  const int K = p.K;
  const int Keff = K < V ? K : V;
  uint64_t top = 0ull;
  for (int pb = 0; pb < N; pb += 2) {
    const int r = pb + (lane >> 5);
    const uint64_t raw = r < N ? xr[r].keys[lane & 31] : 0ull;
    top = merge_top32(top, sort_halves_desc(raw != 0ull ? final_key(raw, L) : 0ull, lane), lane);
  }
  const uint64_t FK = readlane64(top, Keff - 1);
  bool bad = false;
  if (lane < N && c_key != 0ull) {
    const float xc = key_value(c_key);
    bool ok = final_key(c_key, L) <= FK;
    if (ok && xc != kNegInf) ok = ukey32(reported(Elem<DT>::pred(xc), L)) < (uint32_t)(FK >> 32);
    bad = !ok;
  }
  const uint64_t unsafe = __ballot(bad);
  if (lane == 0) p.guard[row] = __popcll(unsafe);
  if (unsafe != 0ull) {
    top = 0ull;
    for (int pb = 0; pb < N; pb += 2) {
      const int r = pb + (lane >> 5);
      uint64_t f = 0ull;
      if (r < N && !((unsafe >> r) & 1ull)) {
        const uint64_t raw = xr[r].keys[lane & 31];
        if (raw != 0ull) f = final_key(raw, L);
      }
      top = merge_top32(top, sort64_desc(f, lane), lane);
    }
    uint64_t thr = FK;
    for (int r = 0; r < N; ++r) {
      if (!((unsafe >> r) & 1ull)) continue;
      rescan_lanes<DT, VEC>(top, thr, rowp, shard_lo(r, V, N), shard_lo(r + 1, V, N), L, Keff, lane,
                            &buf[wv][0], 256);
    }
  }
  if (lane < K) {
    int32_t id = -1;
    uint32_t bits = kNanBits;
    if (lane < Keff) {
      id = (int32_t)key_id(top);
      bits = __float_as_uint(unkey32((uint32_t)(top >> 32)));
    }
    *(int2*)(out + 2 + 2 * lane) = make_int2(id, (int32_t)bits);
  }
}

// Whether the merge takes four waves per row: when the launch's unit ranges
// are short enough that a row of the frame, every row active, could span
// more than four parts (ranges of at least n units start at most
// ceil((U - 1) / n) + 1 parts in a row of U units).  Fewer active rows only
// shorten the ranges further; the one-wave layout merges any row, only more
// slowly.
bool wide_merge(const Params& p) {
  const int64_t n = (int64_t)p.capacity * p.T * p.units;
  const int64_t per = n < 2 * (int64_t)p.workers ? (n > p.workers ? 2 : 1) : n / p.workers;
  return (p.units - 1 + per - 1) / per + 1 > 4;
}

template <int DT, bool VEC, bool SCORE>
hipError_t launch_typed(const Params& p, int phases, hipStream_t st) {
  if (phases & kPhaseReduce) {
    const size_t lds = prefix_lds_bytes(p.capacity, SCORE || p.row_offsets != nullptr);
    hipLaunchKernelGGL((reduce_kernel<DT, VEC, SCORE>), dim3((uint32_t)p.workers), dim3(kBlock), lds,
                       st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phases & kPhaseMerge)) return hipSuccess;
  const int64_t rows = (int64_t)p.capacity * p.T;
  if (wide_merge(p))
    hipLaunchKernelGGL((merge_kernel<DT, VEC, SCORE, true>), dim3((uint32_t)rows), dim3(kMergeBlock), 0, st, p);
  else
    hipLaunchKernelGGL((merge_kernel<DT, VEC, SCORE, false>),
                       dim3((uint32_t)((rows + kMergeWaves - 1) / kMergeWaves)), dim3(kMergeBlock), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// The workspace of flare_logprobs_run_noalloc: a file-scope device array that
// the library never allocates or frees (each GPU holds its own copy until the
// process ends).  Host code may not use its name as an address: the address
// on a device comes from hipGetSymbolAddress with that device current, looked
// up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_address(int device, void** ptr) {
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices || !ptr) return (int)hipErrorInvalidValue;
  std::lock_guard<std::mutex> hold(lock);
  if (!addr[device]) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[device] = a;
  }
  *ptr = addr[device];
  return 0;
}

int launch_shard_finalize(const Params& p, int dtype, void* stream) {
  const int64_t rows = (int64_t)p.capacity * p.T;
  const dim3 grid((uint32_t)((rows + kMergeWaves - 1) / kMergeWaves));
  if (dtype == 1)
    hipLaunchKernelGGL(shard_finalize_kernel<1>, grid, dim3(kMergeBlock), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(shard_finalize_kernel<0>, grid, dim3(kMergeBlock), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_shard_merge(const Params& p, int dtype, bool vector_rows, void* stream) {
  const int64_t rows = (int64_t)p.capacity * p.T;
  const dim3 grid((uint32_t)((rows + kMergeWaves - 1) / kMergeWaves));
  hipStream_t st = (hipStream_t)stream;
  if (dtype == 1) {
    if (vector_rows) hipLaunchKernelGGL((shard_merge_kernel<1, true>), grid, dim3(kMergeBlock), 0, st, p);
    else hipLaunchKernelGGL((shard_merge_kernel<1, false>), grid, dim3(kMergeBlock), 0, st, p);
  } else {
    if (vector_rows) hipLaunchKernelGGL((shard_merge_kernel<0, true>), grid, dim3(kMergeBlock), 0, st, p);
    else hipLaunchKernelGGL((shard_merge_kernel<0, false>), grid, dim3(kMergeBlock), 0, st, p);
  }
  return (int)hipGetLastError();
}

size_t prefix_lds_bytes(int capacity, bool packed) {
  return (size_t)(capacity + 1 + (packed ? capacity : 0)) * sizeof(int);
}

template <int DT, bool VEC, bool SCORE>
int occupancy_typed(size_t lds) {
  int n = 0;
  const hipError_t e =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reduce_kernel<DT, VEC, SCORE>, kBlock, lds);
  return e == hipSuccess ? n : 0;
}

int reduce_occupancy(int dtype, bool vector_rows, bool score, int capacity, bool packed) {
  const size_t lds = prefix_lds_bytes(capacity, packed || score);
  if (dtype == 1) {
    if (score) return vector_rows ? occupancy_typed<1, true, true>(lds) : occupancy_typed<1, false, true>(lds);
    return vector_rows ? occupancy_typed<1, true, false>(lds) : occupancy_typed<1, false, false>(lds);
  }
  if (score) return vector_rows ? occupancy_typed<0, true, true>(lds) : occupancy_typed<0, false, true>(lds);
  return vector_rows ? occupancy_typed<0, true, false>(lds) : occupancy_typed<0, false, false>(lds);
}

int launch(const Params& p, int dtype, bool vector_rows, bool score, int phases, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dtype == 1) {
    if (score)
      e = vector_rows ? launch_typed<1, true, true>(p, phases, st) : launch_typed<1, false, true>(p, phases, st);
    else
      e = vector_rows ? launch_typed<1, true, false>(p, phases, st) : launch_typed<1, false, false>(p, phases, st);
  } else {
    if (score)
      e = vector_rows ? launch_typed<0, true, true>(p, phases, st) : launch_typed<0, false, true>(p, phases, st);
    else
      e = vector_rows ? launch_typed<0, true, false>(p, phases, st) : launch_typed<0, false, false>(p, phases, st);
  }
  return (int)e;
}

}  // namespace flp

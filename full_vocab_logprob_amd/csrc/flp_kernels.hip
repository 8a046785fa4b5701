// gfx950 kernels of the generation-logprob reduction.
//
// What is computed (Flare generation-logprobs design page, definition and
// tiled-reduction paragraphs): for each emitted position, L = FP32 logsumexp
// of the raw logits over lanes [0, V); the chosen token's fl32(x - L); then
// either the K best lanes by (fl32(x - L) desc, ID asc) with -0 read as +0,
// or the caller's selected IDs in order.
//
// How (a single read of every logit; no MFMA, nothing here is a contraction):
//   segment pass, one workgroup per (active row, segment of 16K bf16 / 8K FP32
//   lanes): each thread loads 8 x 16-byte chunks with coalesced dwordx4 loads
//   and keeps them in VGPRs; per wave: max, then sum of exp2 against that
//   max; across the 4 waves an exact segment (m, s).  Natural-mode rows also
//   pick the segment's 32 best *raw* keys (value, then smaller ID) while the
//   data is still in registers: the 32nd-largest lane maximum is found by an
//   LDS radix select, only 16-byte chunks whose maximum reaches it are
//   staged to LDS, their qualifying lanes become 64-bit keys, and a bitonic
//   sort keeps the best 32.
//   merge, one workgroup per active row: combine the segment (m, s) in
//   segment order into L, re-key the retained candidates by the reported
//   value fl32(x - L), sort, and check an exactness guard per segment; a
//   segment that fails it is rescanned with final keys.  Then the chosen
//   and selected-ID gathers and the packed write.
//
// The pages' own scheme ranks normalized values in a second pass over the
// vocabulary; ranking raw values and re-keying only the survivors is what
// lets this path read the logits once.  The guard makes the two agree
// exactly (see merge_kernel).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flp_internal.h"

namespace flp {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kNanBits = 0x7FC00000u;
constexpr int kStageCap = 64;   // hot chunks staged per wave
constexpr int kPoolCap = 512;   // candidate keys per segment
constexpr int kRowWords = 258;

// ------------------------------------------------------------------ keys
// Order-preserving map of an FP32 value (with -0 read as +0) to uint32.
__device__ __forceinline__ uint32_t ukey32(float x) {
  x = (x == 0.0f) ? 0.0f : x;
  uint32_t b = __float_as_uint(x);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float unkey32(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}
// 64-bit key: larger value first, then smaller token ID.
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

// ------------------------------------------------------------- dtype traits
template <int DT> struct Elem;
template <> struct Elem<1> {  // bf16
  static constexpr int kPer = 8;
  static constexpr int kBytes = 2;
  static constexpr int kDigits = 2;  // a bf16 value's key has 16 bits
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  __device__ static __forceinline__ float get(const uint4& r, int j) {
    uint32_t w = (j >> 1) == 0 ? r.x : (j >> 1) == 1 ? r.y : (j >> 1) == 2 ? r.z : r.w;
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ static __forceinline__ uint32_t load_bits(const char* row, int64_t i) {
    return (uint32_t)(*(const uint16_t*)(row + 2 * i));
  }
  // Previous representable input value, for the merge guard.
  __device__ static __forceinline__ float pred(float x) {
    uint32_t u = ukey32(x) >> 16;  // 16-bit key of a bf16 value
    uint32_t v = u - 1;
    if (v == 0x7FFFu) v = 0x7FFEu;  // skip -0: it equals +0 after canon0
    uint32_t h = (v & 0x8000u) ? (v & 0x7FFFu) : (~v & 0xFFFFu);
    return __uint_as_float(h << 16);
  }
  __device__ static __forceinline__ float key_floor(uint32_t k16) {
    uint32_t h = (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
    return __uint_as_float(h << 16);
  }
};
template <> struct Elem<0> {  // fp32
  static constexpr int kPer = 4;
  static constexpr int kBytes = 4;
  static constexpr int kDigits = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  __device__ static __forceinline__ float get(const uint4& r, int j) {
    uint32_t w = j == 0 ? r.x : j == 1 ? r.y : j == 2 ? r.z : r.w;
    return __uint_as_float(w);
  }
  __device__ static __forceinline__ uint32_t load_bits(const char* row, int64_t i) {
    return *(const uint32_t*)(row + 4 * i);
  }
  __device__ static __forceinline__ float pred(float x) {
    uint32_t u = ukey32(x);
    uint32_t v = u - 1;
    if (v == 0x7FFFFFFFu) v = 0x7FFFFFFEu;  // skip -0
    return unkey32(v);
  }
  __device__ static __forceinline__ float key_floor(uint32_t k32) { return unkey32(k32); }
};

// Chunk holding lanes [first, first + kPer) of a row; lanes >= V read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ uint4 load_chunk(const char* row, int64_t first, int V) {
  using E = Elem<DT>;
  uint4 r;
  r.x = r.y = r.z = r.w = E::kNegInfWord;
  if (first >= V) return r;
  if (VEC) {
    r = *(const uint4*)(row + first * E::kBytes);
    if (first + E::kPer > V) {
      int nv = (int)(V - first);
      uint32_t* w = &r.x;
#pragma unroll
      for (int j = 0; j < E::kPer; ++j) {
        if (j >= nv) {
          if (DT == 1) {
            uint32_t& word = w[j >> 1];
            word = (j & 1) ? ((word & 0x0000FFFFu) | 0xFF800000u) : ((word & 0xFFFF0000u) | 0xFF80u);
          } else {
            w[j] = 0xFF800000u;
          }
        }
      }
    }
  } else {
    uint32_t* w = &r.x;
#pragma unroll
    for (int j = 0; j < E::kPer; ++j) {
      int64_t i = first + j;
      if (i < V) {
        uint32_t b = E::load_bits(row, i);
        if (DT == 1) {
          uint32_t& word = w[j >> 1];
          word = (j & 1) ? ((word & 0x0000FFFFu) | (b << 16)) : ((word & 0xFFFF0000u) | b);
        } else {
          w[j] = b;
        }
      }
    }
  }
  return r;
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int64_t i) {
  uint32_t b = Elem<DT>::load_bits(row, i);
  return __uint_as_float(DT == 1 ? (b << 16) : b);
}

// ------------------------------------------------------- wave / block helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Bitonic sort of pool[0, n) descending (n a power of two, all threads).
__device__ __forceinline__ void block_sort_desc(uint64_t* pool, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kBlock) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t a = pool[i], b = pool[ixj];
          bool first_half = (i & k) == 0;
          if (first_half ? (a < b) : (a > b)) {
            pool[i] = b;
            pool[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n, int lo) {
  int p = lo;
  while (p < n) p <<= 1;
  return p;
}

// The k-th largest of the voters' D-digit keys (one key per thread), by an
// LDS radix select over 8-bit digits.  Requires at least k voters.
template <int D>
__device__ uint32_t block_kth_largest(uint32_t key, bool voter, int k, uint32_t* hist,
                                      int* bcast) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0;
  int need = k;
#pragma unroll
  for (int d = D - 1; d >= 0; --d) {
    hist[tid] = 0;
    __syncthreads();
    bool match = voter && (d == D - 1 || (key >> (8 * (d + 1))) == prefix);
    if (match) atomicAdd(&hist[(key >> (8 * d)) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
          h3 = hist[4 * lane + 3];
      int own = h0 + h1 + h2 + h3;
      int suf = own;  // inclusive suffix sum over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += t;
      }
      int above = suf - own;  // count in bins of higher lanes
      int c3 = above + h3, c2 = c3 + h2, c1 = c2 + h1, c0 = c1 + h0;
      int b = -1, gt = 0;
      if (c3 >= need) { b = 4 * lane + 3; gt = above; }
      else if (c2 >= need) { b = 4 * lane + 2; gt = c3; }
      else if (c1 >= need) { b = 4 * lane + 1; gt = c2; }
      else if (c0 >= need) { b = 4 * lane; gt = c1; }
      // cnt_ge is non-increasing in the bin, so the highest qualifying bin
      // lies in the highest lane that found one.
      uint64_t found = __ballot(b >= 0);
      int top = 63 - __builtin_clzll(found);
      if (lane == top) {
        bcast[0] = b;
        bcast[1] = gt;
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | (uint32_t)bcast[0];
    need -= bcast[1];
    __syncthreads();
  }
  return prefix;
}

// ============================================================ segment pass
struct SegShared {
  uint32_t hist[256];
  int bcast[4];
  float wm[kWaves];
  float ws[kWaves];
  int wcount[kWaves];
  int pool_count;
  int overflow;
  uint4 stage[kWaves][kStageCap];
  int32_t stage_off[kWaves][kStageCap];
  uint64_t pool[kPoolCap];
};

__device__ __forceinline__ bool row_active(const Params& p, int row, int* n_sel) {
  int s = row / p.T;
  int t = row - s * p.T;
  if (p.requested[s] == 0) return false;
  int e = p.emitted[s];
  e = e < 0 ? 0 : (e > p.T ? p.T : e);
  if (t >= e) return false;
  int n = p.id_counts[s];
  *n_sel = n < 0 ? 0 : (n > 128 ? 128 : n);
  return true;
}

// Keep the best kKeep keys of pool[0, count): sort, zero the rest.
__device__ void pool_compact(uint64_t* pool, int count, int cap) {
  for (int i = count + threadIdx.x; i < cap; i += kBlock) pool[i] = 0;
  __syncthreads();
  block_sort_desc(pool, pow2_at_least(count, 64));
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void segment_kernel(Params p) {
  using E = Elem<DT>;
  constexpr int kPer = E::kPer;
  constexpr int kWaveElems = 64 * kChunks * kPer;
  constexpr int kSegElems = kWaves * kWaveElems;
  __shared__ SegShared sh;

  const int row = blockIdx.x / p.nseg;
  const int seg = blockIdx.x - row * p.nseg;
  int n_sel = 0;
  if (!row_active(p, row, &n_sel)) return;
  const bool need_cand = (p.K > 0) && (n_sel == 0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int V = p.V;
  const int64_t seg_base = (int64_t)seg * kSegElems;
  const int64_t wave_base = seg_base + (int64_t)w * kWaveElems;
  const char* rowp = (const char*)p.logits + (int64_t)row * p.V_pad * E::kBytes;

  uint4 raw[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    raw[c] = load_chunk<DT, VEC>(rowp, wave_base + (int64_t)(c * 64 + lane) * kPer, V);

  // ---- statistics: wave max, then sum of exp2 relative to it
  float cm[kChunks];
  float lm = kNegInf;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    float m = E::get(raw[c], 0);
#pragma unroll
    for (int j = 1; j < kPer; ++j) m = fmaxf(m, E::get(raw[c], j));
    cm[c] = m;
    lm = fmaxf(lm, m);
  }
  const float mw = wave_max(lm);
  float sum = 0.0f;
  if (mw != kNegInf) {
    // exp2((x - m) * log2 e): the maximum's own term is exactly 1, so a row
    // with one finite lane gets L equal to that lane and a logprob of +0.
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        sum += __builtin_amdgcn_exp2f((E::get(raw[c], j) - mw) * kLog2e);
  }
  sum = wave_sum(sum);
  if (lane == 0) {
    sh.wm[w] = mw;
    sh.ws[w] = sum;
  }
  if (tid == 0) {
    sh.pool_count = 0;
    sh.overflow = 0;
  }
  __syncthreads();
  SegRecord* rec = p.records + (int64_t)row * p.nseg + seg;
  if (tid == 0) {
    float M = sh.wm[0];
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sh.wm[i]);
    float S = 0.0f;
    if (M != kNegInf) {
      for (int i = 0; i < kWaves; ++i)
        if (sh.wm[i] != kNegInf)
          S += sh.ws[i] * __builtin_amdgcn_exp2f((sh.wm[i] - M) * kLog2e);
    }
    rec->m = M;
    rec->s = S;
    if (!need_cand) {
      rec->n = 0;
      rec->flags = 0;
    }
  }
  if (!need_cand) return;

  // ---- candidates: threshold = 32nd-largest lane maximum over valid lanes
  const int64_t nvalid64 = (int64_t)V - seg_base;
  const int nvalid = nvalid64 > kSegElems ? kSegElems : (int)nvalid64;
  int valid_lanes = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    int rem = nvalid - i * kWaveElems;
    int vl = rem <= 0 ? 0 : (rem + kPer - 1) / kPer;
    valid_lanes += vl > 64 ? 64 : vl;
  }
  const bool lane_valid = (wave_base + (int64_t)lane * kPer) < V;
  const bool take_all = valid_lanes < kKeep;
  float tau = kNegInf;
  if (!take_all) {
    uint32_t k = ukey32(lm) >> (32 - 8 * E::kDigits);
    uint32_t kth = block_kth_largest<E::kDigits>(k, lane_valid, kKeep, sh.hist, sh.bcast);
    tau = E::key_floor(kth);
  }

  // ---- stage hot chunks (max reaches tau) into LDS in (chunk, lane) order
  int nh = 0;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t first = wave_base + (int64_t)(c * 64 + lane) * kPer;
    const bool hot = first < V && cm[c] >= tau;
    const uint64_t m = __ballot(hot);
    const int slot = nh + lanes_below(m);
    if (hot && slot < kStageCap) {
      sh.stage[w][slot] = raw[c];
      sh.stage_off[w][slot] = (int32_t)(first - seg_base);
    }
    nh += __popcll(m);
  }
  if (nh > kStageCap && lane == 0) sh.overflow = 1;
  __syncthreads();
  const bool overflow_stage = sh.overflow != 0;

  if (!overflow_stage) {
    // Lane i expands staged chunk i into keys of qualifying lanes.
    uint64_t keys[kPer];
    int cnt = 0;
    if (lane < nh) {
      const uint4 r = sh.stage[w][lane];
      const int64_t off = seg_base + sh.stage_off[w][lane];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const float x = E::get(r, j);
        const int64_t id = off + j;
        keys[j] = 0;
        if (id < V && x >= tau) keys[j] = make_key(x, (uint32_t)id);
        cnt += keys[j] != 0;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) keys[j] = 0;
    }
    const int incl = wave_incl_scan(cnt, lane);
    if (lane == 63) sh.wcount[w] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      base += (i < w) ? sh.wcount[i] : 0;
      total += sh.wcount[i];
    }
    if (total <= kPoolCap) {
      int pos = base + incl - cnt;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (keys[j] != 0) sh.pool[pos++] = keys[j];
      __syncthreads();
      pool_compact(sh.pool, total, kPoolCap);
      if (tid == 0) sh.pool_count = total;
      __syncthreads();
    } else {
      __syncthreads();
      if (tid == 0) sh.overflow = 1;
      __syncthreads();
    }
  }

  if (sh.overflow != 0) {
    // Exact fallback for tie-heavy segments: stream every qualifying lane
    // through the pool, compacting to the best kKeep whenever it fills; the
    // admission threshold rises to the kKeep-th key after each compaction.
    __syncthreads();
    if (tid == 0) sh.pool_count = 0;
    __syncthreads();
    uint64_t thr = take_all ? 0ull : ((uint64_t)ukey32(tau) << 32);
    // The lanes are read again (from cache) so that no register array is
    // indexed dynamically here.
#pragma unroll 1
    for (int c = 0; c < kChunks; ++c) {
      const int64_t first = wave_base + (int64_t)(c * 64 + lane) * kPer;
#pragma unroll 1
      for (int j = 0; j < kPer; ++j) {
        const int64_t id = first + j;
        if (id < V) {
          const uint64_t key = make_key(load_elem<DT>(rowp, id), (uint32_t)id);
          if (key >= thr) {
            int at = atomicAdd(&sh.pool_count, 1);
            sh.pool[at] = key;
          }
        }
        __syncthreads();
        const int count = sh.pool_count;
        if (count > kPoolCap - kBlock) {
          pool_compact(sh.pool, count, kPoolCap);
          thr = sh.pool[kKeep - 1];
          __syncthreads();
          if (tid == 0) sh.pool_count = kKeep;
          __syncthreads();
        }
      }
    }
    const int count = sh.pool_count;
    pool_compact(sh.pool, count, kPoolCap);
    __syncthreads();
  }

  const int held = sh.pool_count < kKeep ? sh.pool_count : kKeep;
  if (tid < kKeep) rec->keys[tid] = tid < held ? sh.pool[tid] : 0ull;
  if (tid == 0) {
    rec->n = held;
    rec->flags = (nvalid <= kKeep) ? kRecComplete : 0;
  }
}

// ================================================================== merge
// Per row: L from the segment records; chosen and selected gathers; natural
// top-K from the retained raw candidates re-keyed by the reported value.
//
// Exactness guard.  Segment j holds its best 32 raw keys; let c be the 32nd,
// with value x_c.  With F the final key (reported value, then smaller ID),
// F_K the K-th best final key among all held candidates and v_K its value,
// every lane e that segment j dropped has either x_e == x_c and a larger ID
// (so F(e) < F(c)) or x_e <= pred(x_c) (so its value is at most
// r(pred(x_c)), r(x) = fl32(x - L) being monotone).  Hence if F(c) <= F_K
// and r(pred(x_c)) < v_K no dropped lane can enter the top K.  A segment
// failing either test is rescanned lane by lane with final keys; F_K over a
// subset never exceeds the true K-th key, so the test stays sound.
struct MergeShared {
  float red[kBlock];
  int count;
  int unsafe_any;
  uint8_t unsafe[kMaxSegs];
};

__device__ float block_max_all(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Deterministic block sum: a fixed tree over thread slots.
__device__ float block_sum_fixed(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kBlock / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  float r = red[0];
  __syncthreads();
  return r;
}

template <int DT>
__device__ void merge_row(const Params& p, int row, int n_sel, MergeShared& sh,
                          uint64_t* pool) {
  using E = Elem<DT>;
  constexpr int kSegElems = kBlock * kChunks * E::kPer;
  const int tid = threadIdx.x;
  const int V = p.V;
  const int nseg = p.nseg;
  const SegRecord* rec = p.records + (int64_t)row * nseg;
  const char* rowp = (const char*)p.logits + (int64_t)row * p.V_pad * E::kBytes;
  int32_t* out = p.out + (int64_t)row * kRowWords;

  // ---- normalization, combined in segment order
  float M = kNegInf;
  for (int j = tid; j < nseg; j += kBlock) M = fmaxf(M, rec[j].m);
  M = block_max_all(M, sh.red);
  float part = 0.0f;
  if (M != kNegInf)
    for (int j = tid; j < nseg; j += kBlock) {
      float mj = rec[j].m;
      if (mj != kNegInf) part += rec[j].s * __builtin_amdgcn_exp2f((mj - M) * kLog2e);
    }
  const float S = block_sum_fixed(part, sh.red);
  const float L = M + logf(S);
  if (tid == 0) p.lse[row] = L;

  // ---- chosen token
  if (tid == 0) {
    const int tok = p.tokens[row];
    uint32_t bits = kNanBits;
    if (tok >= 0 && tok < V) bits = __float_as_uint(reported(load_elem<DT>(rowp, tok), L));
    out[0] = tok;
    out[1] = (int32_t)bits;
  }

  // ---- selected IDs, caller order
  if (n_sel > 0) {
    const int s = row / p.T;
    for (int j = tid; j < n_sel; j += kBlock) {
      const int id = p.ids[(int64_t)s * 128 + j];
      uint32_t bits = kNanBits;
      if (id >= 0 && id < V) bits = __float_as_uint(reported(load_elem<DT>(rowp, id), L));
      out[2 + 2 * j] = id;
      out[3 + 2 * j] = (int32_t)bits;
    }
    return;
  }
  const int K = p.K;
  if (K == 0) return;

  // ---- natural top-K from the held candidates
  const int cap = p.merge_pool;
  const int held_slots = nseg * kKeep;
  for (int i = tid; i < cap; i += kBlock) {
    uint64_t f = 0;
    if (i < held_slots) {
      const int j = i / kKeep, k = i - j * kKeep;
      if (k < rec[j].n) f = final_key(rec[j].keys[k], L);
    }
    pool[i] = f;
  }
  if (tid == 0) sh.unsafe_any = 0;
  __syncthreads();
  block_sort_desc(pool, pow2_at_least(held_slots, 64));
  const int Keff = K < V ? K : V;
  const uint64_t FK = pool[Keff - 1];
  const uint32_t vK = (uint32_t)(FK >> 32);
  for (int j = tid; j < nseg; j += kBlock) {
    bool bad = false;
    if (!(rec[j].flags & kRecComplete)) {
      const uint64_t c = rec[j].keys[kKeep - 1];
      const float xc = key_value(c);
      bool ok = final_key(c, L) <= FK;
      if (ok && xc != kNegInf) ok = ukey32(reported(E::pred(xc), L)) < vK;
      bad = !ok;
    }
    sh.unsafe[j] = bad ? 1 : 0;
    if (bad) atomicOr(&sh.unsafe_any, 1);
  }
  __syncthreads();

  if (sh.unsafe_any) {
    // Rebuild: held candidates of safe segments, then every lane of each
    // unsafe segment whose final key reaches the bound FK.
    if (tid == 0) sh.count = 0;
    __syncthreads();
    for (int i = tid; i < held_slots; i += kBlock) {
      const int j = i / kKeep, k = i - j * kKeep;
      if (!sh.unsafe[j] && k < rec[j].n) {
        const int at = atomicAdd(&sh.count, 1);
        pool[at] = final_key(rec[j].keys[k], L);
      }
    }
    __syncthreads();
    uint64_t thr = FK;
    for (int j = 0; j < nseg; ++j) {
      if (!sh.unsafe[j]) continue;
      const int64_t lo = (int64_t)j * kSegElems;
      const int64_t hi = lo + kSegElems < V ? lo + kSegElems : V;
      for (int64_t b = lo; b < hi; b += kBlock) {
        const int64_t i = b + tid;
        if (i < hi) {
          const uint64_t f = make_key(reported(load_elem<DT>(rowp, i), L), (uint32_t)i);
          if (f >= thr) {
            const int at = atomicAdd(&sh.count, 1);
            pool[at] = f;
          }
        }
        __syncthreads();
        const int count = sh.count;
        if (count > cap - kBlock) {
          for (int q = count + tid; q < cap; q += kBlock) pool[q] = 0;
          __syncthreads();
          block_sort_desc(pool, cap);
          thr = pool[Keff - 1];
          __syncthreads();
          if (tid == 0) sh.count = Keff;
          __syncthreads();
        }
      }
    }
    const int count = sh.count;
    for (int q = count + tid; q < cap; q += kBlock) pool[q] = 0;
    __syncthreads();
    block_sort_desc(pool, cap);
  }

  for (int j = tid; j < K; j += kBlock) {
    int32_t id = -1;
    uint32_t bits = kNanBits;
    if (j < Keff) {
      const uint64_t f = pool[j];
      id = (int32_t)key_id(f);
      bits = __float_as_uint(unkey32((uint32_t)(f >> 32)));
    }
    out[2 + 2 * j] = id;
    out[3 + 2 * j] = (int32_t)bits;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void merge_kernel(Params p) {
  __shared__ MergeShared sh;
  extern __shared__ uint64_t pool[];
  const int row = blockIdx.x;
  int n_sel = 0;
  if (!row_active(p, row, &n_sel)) return;
  merge_row<DT>(p, row, n_sel, sh, pool);
}

__global__ void reset_kernel(uint32_t* t, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    t[i] = 0u;
}

template <int DT, bool VEC>
hipError_t launch_typed(const Params& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.capacity * p.T;
  hipLaunchKernelGGL((segment_kernel<DT, VEC>), dim3((uint32_t)(rows * p.nseg)), dim3(kBlock),
                     0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<DT>), dim3((uint32_t)rows), dim3(kBlock),
                     (size_t)p.merge_pool * sizeof(uint64_t), st, p);
  return hipGetLastError();
}

}  // namespace

int launch_reduce(const Params& p, int dtype, bool vector_rows, int merge_mode,
                  void* stream) {
  (void)merge_mode;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dtype == 1)
    e = vector_rows ? launch_typed<1, true>(p, st) : launch_typed<1, false>(p, st);
  else
    e = vector_rows ? launch_typed<0, true>(p, st) : launch_typed<0, false>(p, st);
  return (int)e;
}

int launch_reset(uint32_t* tickets, int64_t n, void* stream) {
  if (n <= 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(reset_kernel, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                     tickets, n);
  return (int)hipGetLastError();
}

}  // namespace flp

// Device code of the decode step for gfx950 (MI355X): LM head with a fused
// softmax-statistics epilogue, cross-workgroup merge, and the three commit
// policies on one wavefront per sequence.
//
// Method (dInfer explainer, 91haoming.cn, summary of arXiv 2510.08666):
//   decoding-strategy component -- candidates and confidences per position,
//   then threshold / hierarchical / credit decoding; diffusion-iteration
//   manager -- one fixed-size block per step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dlm.h"

namespace dlm {

constexpr int kWaves = 8;             // wavefronts per workgroup
constexpr int kThreads = kWaves * 64; // workgroup size
constexpr int kTileRows = 16;         // vocabulary rows per MFMA tile
constexpr int kPrefetch = 8;          // 16-byte W fragments in flight per lane (measured: 8 beats 16 and 32)
constexpr int kRowsPerStage = 1024;   // finalize: rows staged in LDS at a time
constexpr int kMaxVocabGroups = 256;  // vocabulary ranges (records per row) at most
constexpr int kGroup = 16;            // records per first-level group of the cross-workgroup merge
constexpr unsigned kFlagCommit = 1u << 16;  // internal: run the commit policies
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Rule {
  int kind;
  float thr;
  float decay;
  int depth;
  int eos;   // end token for early stop, -1 = none (also when the call has no state array)
};

// Everything the commit policies touch.
struct CommitArgs {
  uint8_t* mask;
  dlm_credit_slot* credit;
  int32_t* out_tokens;
  uint8_t* out_commit;
  float* out_conf;
  float* out_gap;
  uint8_t* seq_done;   // [B] early-stop state (DLM_SEQ_*), or null
  int32_t* out_topk_tokens;  // [B*L][topk] top-k export, or null (topk == 0)
  float* out_topk_prob;      // [B*L][topk] or null
  int topk;
  float4* out_records;       // vocabulary shard: [B*L] merged records (global ids) instead of conf / token
  int v_begin;               // first global token id of the shard
  int B, L;
  unsigned flags;
  Rule rules[DLM_MAX_RULES];
  uint8_t rule_of[DLM_MAX_SEQS];
};

// LDS of the step kernel for NMB 16-row blocks: two buffers of per-wavefront partial logits
// (8 waves x NMB x 1 KB each), reused for the per-slot statistics and the finalize stage.
__host__ __device__ constexpr size_t lds_bytes(int NMB) {
  return (size_t)2 * kWaves * NMB * 1024 > (size_t)kRowsPerStage * 12 ? (size_t)2 * kWaves * NMB * 1024
                                                                       : (size_t)kRowsPerStage * 12;
}

// With the top-k fold the per-slot statistics (16 bytes) are followed by the per-slot lists
// (DLM_MAX_TOPK entries of 8 bytes) of the 256 * NMB logit slots of a tile.
__host__ __device__ constexpr size_t lds_bytes_topk(int NMB) {
  return lds_bytes(NMB) > (size_t)256 * NMB * (16 + DLM_MAX_TOPK * 8) ? lds_bytes(NMB)
                                                                        : (size_t)256 * NMB * (16 + DLM_MAX_TOPK * 8);
}
static_assert(lds_bytes_topk(1) >= (size_t)kRowsPerStage * 20, "the finalize stage with top-k lists fits");

struct StepArgs {
  const void* hidden;  // [M][H]
  const void* W;       // [V][H]
  float4* partials;    // [n_rg * 16 * NMB][G_v] statistics record of each (row, vocabulary range)
  unsigned* ticket;    // completion counter, zero between calls
  int H, V, M;
  int n_rg;            // row groups of 16 * NMB rows
  int G_v;             // vocabulary ranges (multiple of 8)
  int ntiles;          // ceil(V / 16)
  float4* topk_records;  // top-k fold only: [n_rg * 16 * NMB][G_v] lists of kTopK (logit, id)
  unsigned* group_tickets;  // [n_rg][nq] completion counters of the groups of kGroup ranges
  float4* level2;        // [n_rg * 16 * NMB][nq] merged record of each (row, group of ranges)
  float4* topk_level2;   // top-k fold only: [n_rg * 16 * NMB][nq] merged lists of each (row, group)
  int nq;                // groups of ranges: ceil(G_v / kGroup)
  CommitArgs c;
};

// ----------------------------------------------------------------------------------------------
// Online softmax statistics of a set of logits: running max m1, sum s of exp(z - m1), lowest
// arg-max id, and the second-largest logit m2 (counted with multiplicity).  s == 0 marks "empty".
// ----------------------------------------------------------------------------------------------
struct Stats {
  float m1, s, m2;
  int id;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work-item and work-group ids read straight from the hardware-initialised registers: the device
// library's accessors behind threadIdx / blockIdx are not inlined into kernels built without IEEE
// mode and would be real calls.
__device__ __forceinline__ int lid() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int gid() { return (int)__builtin_amdgcn_workgroup_id_x(); }

// ---- cross-lane exchange on a 64-lane wavefront -------------------------------------------------
// Within a row of 16 lanes: DPP quad permutes and row mirrors.  Across rows: the gfx950 row-swap
// permutes, which hand each lane its own value and its partner row's value; applying a symmetric
// operation to the pair gives every lane the combined result.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, x)));
}

// (value of this lane's row pair partner) for rows 16 (W = 16) or 32 (W = 32) apart, as a pair
// (lower row's value, upper row's value) identical in both rows
template <int W>
__device__ __forceinline__ void row_swap(int x, int& lo, int& hi) {
  const auto r = W == 16 ? __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false)
                         : __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  lo = (int)r[0];
  hi = (int)r[1];
}

template <class Op>
__device__ __forceinline__ float wave_allreduce(float x, Op op) {
  x = op(x, dpp<kDppXor1>(x));
  x = op(x, dpp<kDppXor2>(x));
  x = op(x, dpp<kDppHalfMirror>(x));
  x = op(x, dpp<kDppMirror>(x));
  int lo, hi;
  row_swap<16>(__builtin_bit_cast(int, x), lo, hi);
  x = op(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
  row_swap<32>(__builtin_bit_cast(int, x), lo, hi);
  return op(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

__device__ __forceinline__ int wave_allreduce_min(int x) {
  x = min(x, dpp<kDppXor1>(x));
  x = min(x, dpp<kDppXor2>(x));
  x = min(x, dpp<kDppHalfMirror>(x));
  x = min(x, dpp<kDppMirror>(x));
  int lo, hi;
  row_swap<16>(x, lo, hi);
  x = min(lo, hi);
  row_swap<32>(x, lo, hi);
  return min(lo, hi);
}

__device__ __forceinline__ float wave_max(float x) {
  return wave_allreduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_allreduce(x, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ Stats stats_empty() {
  Stats t;
  t.m1 = -INFINITY;
  t.s = 0.f;
  t.m2 = -INFINITY;
  t.id = 0x7fffffff;
  return t;
}

// Symmetric in its operands, bit for bit (every operation in it is), and an empty operand leaves
// the other unchanged: any grouping of records that follows the same tree gives the same bits.
// The larger maximum's sum is rescaled by exp(0) = 1 exactly, so only the other sum needs an
// exponential (the sum of zero stays zero, also for two empty operands).
__device__ __forceinline__ Stats stats_merge(const Stats& a, const Stats& b) {
  Stats r;
  r.m1 = fmaxf(a.m1, b.m1);
  const float lo = fminf(a.m1, b.m1);
  const bool a_hi = a.m1 >= b.m1;
  const float s_hi = a_hi ? a.s : b.s, s_lo = a_hi ? b.s : a.s;
  r.s = s_hi + (s_lo == 0.f ? 0.f : s_lo * ex2((lo - r.m1) * kLog2e));
  r.id = a.m1 > b.m1 ? a.id : (b.m1 > a.m1 ? b.id : min(a.id, b.id));
  r.m2 = fmaxf(fmaxf(a.m2, b.m2), lo);
  return r;
}

// Balanced binary tree over v[0..N) in index order, ((v0 v1)(v2 v3))((v4 v5)(v6 v7))..., held in
// one lane's registers: the tree stats_row16_merge builds across the 16 lanes of a row.
template <int N>
__device__ __forceinline__ Stats stats_tree(Stats (&v)[N]) {
  static_assert((N & (N - 1)) == 0, "a power of two");
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int i = 0; i < N; i += 2 * w) v[i] = stats_merge(v[i], v[i + w]);
  return v[0];
}

template <int CTRL>
__device__ __forceinline__ Stats stats_dpp(const Stats& a) {
  Stats r;
  r.m1 = dpp<CTRL>(a.m1);
  r.s = dpp<CTRL>(a.s);
  r.m2 = dpp<CTRL>(a.m2);
  r.id = dpp<CTRL>(a.id);
  return r;
}

// Every lane of a 16-lane row ends with the merge of the row's 16 statistics (fixed order).
__device__ __forceinline__ Stats stats_row16_merge(Stats t) {
  t = stats_merge(t, stats_dpp<kDppXor1>(t));
  t = stats_merge(t, stats_dpp<kDppXor2>(t));
  t = stats_merge(t, stats_dpp<kDppHalfMirror>(t));
  t = stats_merge(t, stats_dpp<kDppMirror>(t));
  return t;
}

// Every lane gets the merge of its value with the same lane's value in the row W lanes away
// (W = 16: rows 0+1 and 2+3; W = 32: rows 0+2 and 1+3).
template <int W>
__device__ __forceinline__ Stats stats_merge_rows(const Stats& t) {
  Stats a, b;
  int lo, hi;
  row_swap<W>(__builtin_bit_cast(int, t.m1), lo, hi);
  a.m1 = __builtin_bit_cast(float, lo);
  b.m1 = __builtin_bit_cast(float, hi);
  row_swap<W>(__builtin_bit_cast(int, t.s), lo, hi);
  a.s = __builtin_bit_cast(float, lo);
  b.s = __builtin_bit_cast(float, hi);
  row_swap<W>(__builtin_bit_cast(int, t.m2), lo, hi);
  a.m2 = __builtin_bit_cast(float, lo);
  b.m2 = __builtin_bit_cast(float, hi);
  row_swap<W>(t.id, lo, hi);
  a.id = lo;
  b.id = hi;
  return stats_merge(a, b);
}

// ----------------------------------------------------------------------------------------------
// Top-k candidates: a best-first list of (logit, token id).  Larger logits first; among equal
// logits the lower id first.  An empty entry is (-inf, kNoToken).
// ----------------------------------------------------------------------------------------------
constexpr int kTopK = DLM_MAX_TOPK;
constexpr int kNoToken = 0x7fffffff;

struct TopK {
  float z[kTopK];
  int id[kTopK];
};

__device__ __forceinline__ void topk_clear(TopK& t) {
#pragma unroll
  for (int i = 0; i < kTopK; ++i) {
    t.z[i] = -INFINITY;
    t.id[i] = kNoToken;
  }
}

// Insert logit z of token v, where v is larger than every id already in the list (a thread meets
// its tokens in ascending order), so v goes behind equal logits.  Branch-free: from the bottom
// up, entry i takes entry i - 1, the new value, or keeps its own.
__device__ __forceinline__ void topk_push_ascending(TopK& t, float z, int v) {
#pragma unroll
  for (int i = kTopK - 1; i > 0; --i) {
    const bool up = z > t.z[i - 1];
    const bool here = z > t.z[i];
    t.id[i] = up ? t.id[i - 1] : here ? v : t.id[i];
    t.z[i] = up ? t.z[i - 1] : here ? z : t.z[i];
  }
  if (z > t.z[0]) {
    t.id[0] = v;
    t.z[0] = z;
  }
}

// Drop the head of the list where `pop` holds (an empty entry enters at the bottom).
__device__ __forceinline__ void topk_pop_if(TopK& t, bool pop) {
#pragma unroll
  for (int i = 0; i < kTopK - 1; ++i) {
    t.z[i] = pop ? t.z[i + 1] : t.z[i];
    t.id[i] = pop ? t.id[i + 1] : t.id[i];
  }
  t.z[kTopK - 1] = pop ? -INFINITY : t.z[kTopK - 1];
  t.id[kTopK - 1] = pop ? kNoToken : t.id[kTopK - 1];
}

// Every lane of a 16-lane row ends with the kTopK best entries of the row's 16 lists: each round
// takes the best head (largest logit, then lowest id) and pops it from the list that held it.
// Token ids are distinct across the lists, so exactly one list pops (or only empty heads).
__device__ __forceinline__ void topk_row16_merge(TopK& t, TopK& out) {
#pragma unroll
  for (int r = 0; r < kTopK; ++r) {
    const float hz = t.z[0];
    const int hi = t.id[0];
    float m = fmaxf(hz, dpp<kDppXor1>(hz));
    m = fmaxf(m, dpp<kDppXor2>(m));
    m = fmaxf(m, dpp<kDppHalfMirror>(m));
    m = fmaxf(m, dpp<kDppMirror>(m));
    int id = hz == m ? hi : kNoToken;
    id = min(id, dpp<kDppXor1>(id));
    id = min(id, dpp<kDppXor2>(id));
    id = min(id, dpp<kDppHalfMirror>(id));
    id = min(id, dpp<kDppMirror>(id));
    out.z[r] = m;
    out.id[r] = id;
    topk_pop_if(t, hz == m && hi == id);
  }
}

// A best-first list travels as four 16-byte records: (z0, id0, z1, id1), (z2, id2, z3, id3), ...
__device__ __forceinline__ void topk_from_records(TopK& t, const float4 (&e)[kTopK / 2]) {
#pragma unroll
  for (int q = 0; q < kTopK / 2; ++q) {
    t.z[2 * q] = e[q].x;
    t.id[2 * q] = __float_as_int(e[q].y);
    t.z[2 * q + 1] = e[q].z;
    t.id[2 * q + 1] = __float_as_int(e[q].w);
  }
}

__device__ __forceinline__ float4 topk_record(const TopK& t, int q) {
  return make_float4(t.z[2 * q], __int_as_float(t.id[2 * q]), t.z[2 * q + 1], __int_as_float(t.id[2 * q + 1]));
}

// The export of one row from its merged list, which every lane of the row's 16-lane row holds:
// lane j of that row writes rank j (readings T1-T3).  A rank's probability is
// 2^((z - M) log2 e) / S with the row's maximum M and sum S, so rank 0 equals the confidence
// min(1/S, 1) bit for bit; ranks past the vocabulary are token -1 with probability 0.
__device__ __forceinline__ void topk_write_row(const CommitArgs& c, const TopK& best, int row, int j, float M,
                                               float inv_s) {
  float z = best.z[0];
  int id = best.id[0];
#pragma unroll
  for (int i = 1; i < kTopK; ++i) {
    z = j == i ? best.z[i] : z;
    id = j == i ? best.id[i] : id;
  }
  if (j < c.topk) {
    const bool real = id != kNoToken;
    const size_t o = (size_t)row * c.topk + j;
    c.out_topk_tokens[o] = real ? id : -1;
    if (c.out_topk_prob) c.out_topk_prob[o] = real ? fminf(ex2((z - M) * kLog2e) * inv_s, 1.f) : 0.f;
  }
}

// Statistics records are exchanged between workgroups with 16-byte buffer accesses carrying the
// device-scope coherence bit (the cache policy the compiler gives device-scope atomics): stores
// are written through to the device coherence point and loads read from it, so no cache
// write-back or invalidation is needed around the completion counter.
constexpr int kDeviceCoherent = 16;   // cache-policy operand: device scope

__device__ __forceinline__ void record_store(__amdgpu_buffer_rsrc_t r, unsigned off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDeviceCoherent);
}

__device__ __forceinline__ float4 record_load(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceCoherent));
}

// Records written by an earlier kernel on the stream: the kernel boundary already makes them
// visible to every compute unit, so an ordinary load serves, and neighbouring records come in
// whole cache lines through L2 instead of one 16-byte device-scope read each.
__device__ __forceinline__ float4 record_load_after_kernel(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float4 stats_pack(const Stats& a) {
  return make_float4(a.m1, a.s, __int_as_float(a.id), a.m2);
}

__device__ __forceinline__ Stats stats_unpack(const float4& v) {
  Stats t;
  t.m1 = v.x;
  t.s = v.y;
  t.id = __float_as_int(v.z);
  t.m2 = v.w;
  return t;
}

// The record, or the empty statistics where `in` is false, by one select per field: a select of
// whole structs became a branch around the record's use, the compiler then moved the load into
// that branch, and a load issued on a branch makes every later wait a wait for all loads.
__device__ __forceinline__ Stats stats_unpack_if(const float4& v, bool in) {
  Stats t;
  t.m1 = in ? v.x : -INFINITY;
  t.s = in ? v.y : 0.f;
  t.id = in ? __float_as_int(v.z) : 0x7fffffff;
  t.m2 = in ? v.w : -INFINITY;
  return t;
}

// Fold one logit z of id v (ids arrive in ascending order per thread) into the running stats.
__device__ __forceinline__ void stats_fold1(Stats& st, float z, int v) {
  const float mnew = fmaxf(st.m1, z);
  const float nb = mnew * kLog2e;
  st.s = st.s * ex2(fmaf(st.m1, kLog2e, -nb)) + ex2(fmaf(z, kLog2e, -nb));
  st.m2 = fmaxf(st.m2, fminf(z, st.m1));
  if (z > st.m1) st.id = v;
  st.m1 = mnew;
}

// Every path that merges a row's per-range records follows one fixed two-level tree: the groups
// of kGroup consecutive records first (a balanced binary tree over each group, in index order),
// then the group results, in group order, as one more such tree.  The distributed merge at the
// end of step_kernel takes the two levels in separate workgroups (16-lane DPP trees), the
// finalizers in one (finalize_sequences), so they produce the same bits.  Merging with an empty
// record gives the other operand exactly, so records past G are empty ones and skipped work
// changes no bits.
static_assert(kMaxVocabGroups == kGroup * kGroup, "two levels of 16 cover every range");

// ----------------------------------------------------------------------------------------------
// Element-type traits: one 16-byte fragment per lane feeds one bf16 MFMA (16x16x32) or four
// fp32 MFMAs (16x16x4).  Lane l holds row (l % 16) and K-chunk (l / 16) of its operand; both
// operands use the same K assignment, so any permutation of K inside a fragment is harmless.
// ----------------------------------------------------------------------------------------------
template <class T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bfloat16 bit patterns
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ----------------------------------------------------------------------------------------------
// Wavefront helpers for the commit policies (lane = position, L <= 64).
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Lane holding the largest value; the lowest lane wins a tie.
__device__ __forceinline__ int argmax_lane(float v) {
  const float m = wave_max(v);
  return wave_allreduce_min(v == m ? (int)__lane_id() : 64);
}

// Hierarchical decoding on the 64-bit mask U: the maximal masked runs are the top-level regions;
// every region whose centre (s+e)/2 reaches tau commits that centre and splits in two, the others
// wait for a later step.  Regions of one level are disjoint, so a level-by-level sweep commits
// the same set as any worklist order.  Returns the commit bits and the top-level centre bits.
__device__ __forceinline__ uint64_t hierarchical_commit(uint64_t U, float conf, float tau, int max_depth,
                                                        uint64_t* top_centres) {
  const int l = __lane_id();
  const bool masked = (U >> l) & 1ull;
  int s = 0, e = 63;
  if (masked) {
    const uint64_t holes = ~U;
    const uint64_t below = holes & ((1ull << l) - 1ull);
    const uint64_t above = holes & ~((2ull << l) - 1ull);
    s = below ? 64 - __clzll((long long)below) : 0;
    e = above ? __ffsll((long long)above) - 2 : 63;
  }
  bool active = masked;
  uint64_t committed = 0, top = 0;
  for (int depth = 1; max_depth == 0 || depth <= max_depth; ++depth) {
    if (ballot(active) == 0ull) break;
    const int c = (s + e) >> 1;
    const bool is_c = active && c == l;
    const uint64_t pass = ballot(is_c && conf >= tau);
    if (depth == 1) top = ballot(is_c);
    committed |= pass;
    if (active) {
      if ((pass >> c) & 1ull) {
        if (l < c) e = c - 1;
        else if (l > c) s = c + 1;
        else active = false;
      } else {
        active = false;
      }
    }
  }
  *top_centres = top;
  return committed;
}

// State of one position of a sequence as the commit reads it (lane = position), with the
// sequence's rule and early-stop state: loading them here lets a caller prefetch all of it while
// it waits for something else (the rule lookup is two dependent reads of the argument block).
struct SeqState {
  int mask;   // the position's mask byte as loaded (0 past L), tested only when the commit needs it
  int st[DLM_CREDIT_SLOTS];
  float sc[DLM_CREDIT_SLOTS];
  Rule rule;
  int done;   // early-stop state on entry (DLM_SEQ_RUNNING without a state array)
};

__device__ __forceinline__ SeqState load_seq_state(const CommitArgs& a, int b) {
  const int l = __lane_id();
  const size_t row = (size_t)b * a.L + l;
  SeqState s;
  // The rule index is a byte of the argument block (4-byte aligned array): reading its whole
  // word lets a wavefront-uniform b go through scalar loads, so the rule costs no vector-memory
  // round trip ahead of the sequence's own state.
  unsigned ro;
  __builtin_memcpy(&ro, __builtin_assume_aligned(a.rule_of + 4 * (b >> 2), 4), 4);
  s.rule = a.rules[(ro >> (8 * (b & 3))) & 0xffu];
  s.done = a.seq_done ? (int)a.seq_done[b] : DLM_SEQ_RUNNING;
  s.mask = l < a.L ? (int)a.mask[row] : 0;
#pragma unroll
  for (int i = 0; i < DLM_CREDIT_SLOTS; ++i) {
    s.st[i] = -1;
    s.sc[i] = 0.f;
  }
  if (a.credit != nullptr && l < a.L) {
#pragma unroll
    for (int i = 0; i < DLM_CREDIT_SLOTS; ++i) {
      const dlm_credit_slot cs = a.credit[row * DLM_CREDIT_SLOTS + i];
      s.st[i] = cs.token;
      s.sc[i] = cs.credit;
    }
  }
  return s;
}

// One sequence on one wavefront: policy, outputs and state update.
__device__ void commit_sequence(const CommitArgs& a, int b, float conf, int tok, const SeqState& in_state) {
  const int l = __lane_id();
  const bool in = l < a.L;
  const size_t row = (size_t)b * a.L + l;
  // the rule and the early-stop state are the same in every lane: scalar registers, so the
  // policy branches are uniform jumps
  Rule R;
  R.kind = __builtin_amdgcn_readfirstlane(in_state.rule.kind);
  R.thr = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in_state.rule.thr)));
  R.decay = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, in_state.rule.decay)));
  R.depth = __builtin_amdgcn_readfirstlane(in_state.rule.depth);
  R.eos = __builtin_amdgcn_readfirstlane(in_state.rule.eos);
  if (!in) conf = -INFINITY;

  // early stop: a finished sequence only reports its candidates (its state stays as it is)
  const bool stopping = R.eos >= 0;
  int done = stopping ? __builtin_amdgcn_readfirstlane(in_state.done) : DLM_SEQ_RUNNING;
  if (done == DLM_SEQ_FINISHED) {
    if (in) {
      if (a.out_tokens) a.out_tokens[row] = tok;
      a.out_commit[row] = 0;
    }
    return;
  }

  bool masked = in_state.mask != 0;
  uint64_t U = ballot(masked);
  const bool advance = U == 0ull && (a.flags & DLM_AUTO_ADVANCE);
  if (advance) {
    masked = in;
    U = ballot(masked);
    done = DLM_SEQ_RUNNING;
  }

  // credit slots of this position (cleared when a new block starts)
  int st[DLM_CREDIT_SLOTS];
  float sc[DLM_CREDIT_SLOTS];
  const bool has_credit = a.credit != nullptr;
#pragma unroll
  for (int i = 0; i < DLM_CREDIT_SLOTS; ++i) {
    st[i] = advance ? -1 : in_state.st[i];
    sc[i] = advance ? 0.f : in_state.sc[i];
  }

  uint64_t C = 0;
  if (R.kind == DLM_THRESHOLD) {
    C = ballot(masked && conf >= R.thr);
    if (C == 0ull && U != 0ull) C = 1ull << argmax_lane(masked ? conf : -INFINITY);
  } else if (R.kind == DLM_HIERARCHICAL) {
    uint64_t top = 0;
    C = hierarchical_commit(U, conf, R.thr, R.depth, &top);
    if (C == 0ull && U != 0ull) C = 1ull << argmax_lane(((top >> l) & 1ull) ? conf : -INFINITY);
  } else {  // DLM_CREDIT: decay, then credit the current candidate, then test conf * (1 + credit)
    float score = -INFINITY;
    if (masked) {
#pragma unroll
      for (int i = 0; i < DLM_CREDIT_SLOTS; ++i) sc[i] = __fmul_rn(sc[i], R.decay);
      int hit = -1;
#pragma unroll
      for (int i = DLM_CREDIT_SLOTS - 1; i >= 0; --i)
        if (st[i] == tok) hit = i;
      if (hit < 0) {  // first empty slot, else smallest credit (lowest slot on ties)
        int victim = -1;
#pragma unroll
        for (int i = DLM_CREDIT_SLOTS - 1; i >= 0; --i)
          if (st[i] == -1) victim = i;
        if (victim < 0) {
          victim = 0;
#pragma unroll
          for (int i = 1; i < DLM_CREDIT_SLOTS; ++i)
            if (sc[i] < sc[victim]) victim = i;
        }
#pragma unroll
        for (int i = 0; i < DLM_CREDIT_SLOTS; ++i)
          if (i == victim) {
            st[i] = tok;
            sc[i] = 0.f;
          }
        hit = victim;
      }
      float cr = 0.f;
#pragma unroll
      for (int i = 0; i < DLM_CREDIT_SLOTS; ++i)
        if (i == hit) {
          sc[i] = __fadd_rn(sc[i], conf);
          cr = sc[i];
        }
      score = __fmul_rn(conf, __fadd_rn(1.f, cr));
    }
    C = ballot(masked && score >= R.thr);
    if (C == 0ull && U != 0ull) C = 1ull << argmax_lane(masked ? score : -INFINITY);
  }

  // early stop: when the end token commits, the text ends at its first position e; every
  // position after e still masked commits too, and every position after e committed now
  // carries the end token.  The block that completes after it finishes the sequence.
  uint64_t pad = 0;
  if (stopping) {
    const uint64_t E = ballot(((C >> l) & 1ull) && tok == R.eos);
    if (E != 0ull) {
      const int e = __builtin_ctzll(E);
      const uint64_t after = e >= 63 ? 0ull : (~0ull << (e + 1));
      C |= U & after;
      pad = C & after;
      done = DLM_SEQ_EOS_IN_BLOCK;
    }
    if (done == DLM_SEQ_EOS_IN_BLOCK && (U & ~C) == 0ull) done = DLM_SEQ_FINISHED;
    if (l == 0) a.seq_done[b] = (uint8_t)done;
  }

  if (in) {
    const bool c = (C >> l) & 1ull;
    if (a.out_tokens) a.out_tokens[row] = ((pad >> l) & 1ull) ? R.eos : tok;
    a.out_commit[row] = c ? 1 : 0;
    a.mask[row] = (masked && !c) ? 1 : 0;
    if (has_credit && (advance || (masked && R.kind == DLM_CREDIT))) {
#pragma unroll
      for (int i = 0; i < DLM_CREDIT_SLOTS; ++i) {
        dlm_credit_slot cs;
        cs.token = st[i];
        cs.credit = sc[i];
        a.credit[row * DLM_CREDIT_SLOTS + i] = cs;
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// Final merge + commit of sequences [b_begin, b_end).
//   GROUPED = false: record g of row r sits at index r*rs_row + g*rs_g of `rec` (rs_row = G,
//     rs_g = 1 for the records of one head's workgroups; rs_row = 1, rs_g = B*L for gathered
//     vocabulary shards), G <= kMaxVocabGroups.  One 16-lane row per row of the block: lane j
//     loads group j's records and merges them in registers, then the 16 lanes merge the groups
//     (the two-level tree, four rows per wavefront at once).
//   GROUPED = true: `rec` holds the second-level records of the distributed merge, G <= kGroup per
//     row at r*rs_row + g; one 16-lane row per row of the block (the second level of the same tree).
// IN_KERNEL: `rec` may have been written by other workgroups of the running kernel (or outside
// this library's kernels): device-scope loads; otherwise an earlier kernel of this library on the
// stream wrote it and ordinary loads serve.
// conf / token go to LDS, then one wavefront per sequence commits.  With c.out_records the merged
// record itself is written instead (ids offset by c.v_begin) and nothing commits.
// `pre` is the state this wavefront already fetched for sequence `pre_b` (or pre_b = -1).
// The per-row outputs (confidence, gap, and the candidates without a commit) are written after the
// commits: a wavefront's vector-memory counter also counts its stores, so a store issued before a
// commit would make the commit's wait for its loaded state wait for the store's acknowledgement.
// TK (GROUPED only): each row's 16 lanes also merge the groups' top-k lists and write the export.
// A wavefront that commits a sequence merges its rows' lists before the commits; the others merge
// theirs after the barrier, while the commits run (each row's maximum and 1/sum wait in LDS).
// Called by a whole workgroup; `smem` needs kRowsPerStage * 12 bytes (20 with TK).
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ void finalize_row(const CommitArgs& c, const Stats& t, int row, int rr, float* s_conf,
                                             int* s_tok, float* s_gap) {
  if (c.out_records) {
    Stats o = t;
    o.id = t.id + c.v_begin;
    c.out_records[row] = stats_pack(o);
    return;
  }
  // S >= 1 in exact arithmetic (the top logit's own term is 1); the exponent of that term
  // carries the rounding of m*log2(e), so 1/S may land a few ulps above 1
  s_conf[rr] = fminf(1.f / t.s, 1.f);
  s_tok[rr] = t.id;
  s_gap[rr] = t.m1 - t.m2;
}

template <bool GROUPED, bool IN_KERNEL, bool TK = false>
__device__ void finalize_sequences(const CommitArgs& c, __amdgpu_buffer_rsrc_t rec, int G, int rs_row, int rs_g,
                                   int b_begin, int b_end, uint4* smem, const SeqState& pre, int pre_b,
                                   __amdgpu_buffer_rsrc_t trec) {
  const int tid = lid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool do_commit = (c.flags & kFlagCommit) != 0;
  float* s_conf = reinterpret_cast<float*>(smem);
  int* s_tok = reinterpret_cast<int*>(smem) + kRowsPerStage;
  float* s_gap = reinterpret_cast<float*>(smem) + 2 * kRowsPerStage;
  float* s_m1 = reinterpret_cast<float*>(smem) + 3 * kRowsPerStage;     // TK: each row's maximum
  float* s_inv_s = reinterpret_cast<float*>(smem) + 4 * kRowsPerStage;  // TK: each row's 1/sum
  const int seq_per_stage = max(1, kRowsPerStage / c.L);
  auto rec_off = [&](int r_first, int nrows, int rr, int j) {
    const unsigned src = (unsigned)((size_t)(r_first + (rr < nrows ? rr : 0)) * rs_row * 16);
    return j < G && rr < nrows ? src + 16u * (unsigned)(j * rs_g) : 0x80000000u;
  };
  auto list_off = [](unsigned o, int q) { return o == 0x80000000u ? o : o * (unsigned)(kTopK / 2) + 16u * q; };
  for (int b0 = b_begin; b0 < b_end; b0 += seq_per_stage) {
    const int b1 = min(b_end, b0 + seq_per_stage);
    const int r_first = b0 * c.L, nrows = (b1 - b0) * c.L;
    // GROUPED: one record per lane, two passes of 4 rows per iteration (rows rr0 + 32h + lane/16,
    // lane j taking group j), both passes' loads issued before the first merge, so up to 64 rows
    // cost one round trip
    const bool commits = do_commit && !c.out_records && wave < b1 - b0;   // (uniform)
    float4 tl[TK ? 2 : 1][kTopK / 2];                     // TK: the iteration's top-k lists
    auto stats_load = [&](int rr0, float4 (&v)[2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned o = rec_off(r_first, nrows, rr0 + h * kWaves * 4 + (lane >> 4), lane & 15);
        v[h] = IN_KERNEL ? record_load(rec, o) : record_load_after_kernel(rec, o);
      }
    };
    auto lists_load = [&](int rr0) {                      // (64 bytes at [row][group] in trec)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned o = rec_off(r_first, nrows, rr0 + h * kWaves * 4 + (lane >> 4), lane & 15);
#pragma unroll
        for (int q = 0; q < kTopK / 2; ++q) tl[h][q] = record_load(trec, list_off(o, q));
      }
    };
    auto merge_lists = [&](int rr0, int h, float m1, float inv_s) {   // the row's 16 lanes; the export
      const int rr = rr0 + h * kWaves * 4 + (lane >> 4), j = lane & 15;
      TopK mine, best;
      if (j < G) {
        topk_from_records(mine, tl[h]);
      } else {
        topk_clear(mine);
      }
      topk_row16_merge(mine, best);
      if (rr < nrows) topk_write_row(c, best, r_first + rr, j, m1, inv_s);
    };
    if constexpr (GROUPED) {
      auto stats_pass = [&](int rr0, const float4 (&v)[2]) {
        const int j = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = rr0 + h * kWaves * 4 + (lane >> 4);
          if (rr0 + h * kWaves * 4 >= nrows) break;   // (uniform: no row of this pass exists)
          const Stats t = stats_row16_merge(stats_unpack(j < G ? v[h] : stats_pack(stats_empty())));
          if (rr < nrows && j == 0) {
            finalize_row(c, t, r_first + rr, rr, s_conf, s_tok, s_gap);
            if constexpr (TK) {
              s_m1[rr] = t.m1;
              s_inv_s[rr] = 1.f / t.s;
            }
          }
          if constexpr (TK) {
            if (commits) merge_lists(rr0, h, t.m1, 1.f / t.s);
          }
        }
      };
      int rr0 = wave * 4;
      if constexpr (TK) {
        // The first iteration is straight-line code: its lists are loaded right behind its
        // statistics records, and since loads return in order, the statistics merge waits for
        // the records only.  (A branch between the two would leave the compiler's wait counts
        // assuming the worst, so the merge would wait for the lists too.)
        float4 v[2];
        stats_load(rr0, v);
        __builtin_amdgcn_sched_barrier(0);
        lists_load(rr0);
        __builtin_amdgcn_sched_barrier(0);
        if (rr0 < nrows) stats_pass(rr0, v);
        rr0 += 2 * kWaves * 4;
      }
      for (; rr0 < nrows; rr0 += 2 * kWaves * 4) {
        float4 v[2];
        stats_load(rr0, v);
        if constexpr (TK) {
          if (commits) lists_load(rr0);
        }
        stats_pass(rr0, v);
      }
    } else
    for (int rr0 = wave * 4; rr0 < nrows; rr0 += kWaves * 4) {   // 4 rows per pass, one per 16-lane row
      const int rr = rr0 + (lane >> 4), j = lane & 15;
      const bool rin = rr < nrows;
      const unsigned src = (unsigned)((size_t)(r_first + (rin ? rr : 0)) * rs_row * 16);
      Stats t;
      if (GROUPED || G <= kGroup) {
        // at most one group: record j in lane j, one 16-lane tree
        const unsigned o = j < G ? src + 16u * (unsigned)(j * rs_g) : 0x80000000u;
        float4 v = IN_KERNEL ? record_load(rec, o) : record_load_after_kernel(rec, o);
        v = j < G ? v : stats_pack(stats_empty());
        t = stats_row16_merge(stats_unpack(v));
      } else {
        // group j's records in lane j's registers (its tree in registers), then the groups
        float4 v[kGroup];
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
          const int g = kGroup * j + k;
          const unsigned o = g < G ? src + 16u * (unsigned)(g * rs_g) : 0x80000000u;
          v[k] = IN_KERNEL ? record_load(rec, o) : record_load_after_kernel(rec, o);
        }
        Stats q[kGroup];
#pragma unroll
        for (int k = 0; k < kGroup; ++k) q[k] = stats_unpack_if(v[k], kGroup * j + k < G);
        t = stats_row16_merge(stats_tree(q));
      }
      if (rin && j == 0) finalize_row(c, t, r_first + rr, rr, s_conf, s_tok, s_gap);
    }
    __syncthreads();
    if (do_commit) {
      for (int b = b0 + wave; b < b1; b += kWaves) {
        const int off = (b - b0) * c.L + lane;
        const bool in = lane < c.L;
        const SeqState sq = b == pre_b ? pre : load_seq_state(c, b);
        commit_sequence(c, b, in ? s_conf[off] : 0.f, in ? s_tok[off] : 0, sq);
      }
    }
    if constexpr (GROUPED && TK) {
      // the wavefronts that commit nothing merge their rows' lists now, beside the commits
      if (!commits) {
        for (int rr0 = wave * 4; rr0 < nrows; rr0 += 2 * kWaves * 4) {
          if (rr0 != wave * 4) lists_load(rr0);           // (the first iteration's are loaded)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rr = rr0 + h * kWaves * 4 + (lane >> 4);
            if (rr0 + h * kWaves * 4 >= nrows) break;   // (uniform)
            const int rc = rr < nrows ? rr : nrows - 1;
            merge_lists(rr0, h, s_m1[rc], s_inv_s[rc]);
          }
        }
      }
    }
    if (!c.out_records) {
      for (int rr = tid; rr < nrows; rr += kThreads) {
        const int row = r_first + rr;
        if (c.out_conf) c.out_conf[row] = s_conf[rr];
        if (c.out_gap) c.out_gap[row] = s_gap[rr];
        if (!do_commit) c.out_tokens[row] = s_tok[rr];
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------------------
// The fused step kernel.
//
// Grid: G_v vocabulary ranges x n_rg row groups of MR = 16*NMB hidden rows, one workgroup of 8
// wavefronts each.  Workgroup ids are dealt round-robin over the 8 XCDs; the row groups of one
// vocabulary range sit on the same XCD back to back, so repeated W reads of a range hit its L2.
//
// Streaming: the 8 wavefronts share every 16-row vocabulary tile.  Wavefront w owns the 64-byte K
// fragment pairs (2w, 2w+1), (16+2w, 16+2w+1), ... of each row (whole 128-byte lines; together
// the wavefronts sweep each row left to right) and keeps the matching hidden-state fragments in
// registers for the whole kernel.  W fragments go
// straight from HBM into a ring of registers (RING loads in flight per lane) and through the
// matrix cores.  At the end of a tile each wavefront leaves its partial logits in LDS; after one
// barrier every thread sums the 8 partials of its (row, vocabulary slot) and folds the logit into
// its own online-softmax statistics (double-buffered LDS, one barrier per tile).
//
// Then the statistics of each row are merged inside the workgroup and one record per row goes to
// the device coherence point; the last workgroup to finish (completion counter) merges the
// records of every row in a fixed order, derives conf / token / gap and runs each sequence's
// commit policy on one wavefront.
//
// With TK (top-k export) every thread also keeps the DLM_MAX_TOPK best logits of its slot, the
// workgroup merges them per row into a second record (a best-first list), and the two merge
// levels merge the lists next to the statistics: 16 ranges' lists per row by the group's last
// workgroup, then the groups' lists by the last group, which writes the export.
// ----------------------------------------------------------------------------------------------
template <class T, int NMB, int KFWM, bool TK>
__global__ __launch_bounds__(kThreads) void step_kernel(const StepArgs a) {
  extern __shared__ uint4 smem[];
  using E = Elem<T>;
  constexpr int MR = 16 * NMB;                           // hidden rows of the row group
  constexpr int RING = KFWM > (NMB * KFWM >= 32 ? 8 : kPrefetch) ? KFWM : (NMB * KFWM >= 32 ? 8 : kPrefetch);  // in flight per lane
  constexpr int G = RING / KFWM;                         // tiles per unrolled ring pass
  constexpr int LOGITS = kTileRows * MR;                 // logits of one tile
  constexpr int P = (LOGITS + kThreads - 1) / kThreads;  // logit slots per thread
  static_assert(RING % KFWM == 0, "ring must hold whole tiles");
  const int tid = lid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the loop scalar

  const int bid = gid();
  const int xcd = bid & 7, slot = bid >> 3;
  const int rg = slot % a.n_rg;
  const int gv = (slot / a.n_rg) * 8 + xcd;

  const int H = a.H;
  const int F = H / (4 * (16 / E::kBytes));              // 64-byte fragments per row
  const unsigned row_bytes = (unsigned)H * E::kBytes;
  const unsigned kOOB = 0x80000000u;                     // beyond any range: loads return 0
  const unsigned lane_off = (lane & 15) * row_bytes + (lane >> 4) * 16u;

  // ---- this workgroup's tiles and its W range ----------------------------------------------
  // range index q: each XCD owns a contiguous eighth of the ranges, so the short ranges of the
  // even split spread evenly over the XCDs
  const int q = (gv & 7) * (a.G_v >> 3) + (gv >> 3);
  const int t_begin = (int)((long long)q * a.ntiles / a.G_v);
  const int t_end = (int)((long long)(q + 1) * a.ntiles / a.G_v);
  const int nloc = t_end - t_begin;
  const int nloc_p = (nloc + G - 1) / G * G;
  const long long row0 = (long long)t_begin * kTileRows;
  const long long row_end = min((long long)a.V, (long long)t_end * kTileRows);
  const long long nbytes = row_end > row0 ? (row_end - row0) * row_bytes : 0;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(a.W) + row0 * row_bytes), 0, (int)nbytes, 0x00020000);

  // K fragment j of this wavefront: the wavefronts take adjacent pairs of 64-byte fragments,
  // (2w, 2w+1), (16+2w, 16+2w+1), ..., so fragments j and j+1 (j even) are the two halves of the
  // same 128-byte lines and every line a wavefront touches is used whole.  KFWM is even.
  static_assert(KFWM % 2 == 0, "fragments go in pairs");
  auto frag = [&](int j) -> int { return (j >> 1) * (2 * kWaves) + 2 * wave + (j & 1); };

  // byte offset of fragment j of tile t (zero-filled past the range or the row)
  auto w_off = [&](int t, int j) -> unsigned {
    const int kf = frag(j);
    return (t < nloc && kf < F) ? (unsigned)t * kTileRows * row_bytes + lane_off + (unsigned)kf * 64u : kOOB;
  };

  // ---- hidden fragments of this wavefront's K positions, in registers ------------------------
  // Every workgroup reads all hidden rows before its first tile completes, so their loads use
  // whole 128-byte lines: for the fragment pair (2q, 2q+1) of a 16-row block, lane l loads chunk
  // l%8 of the pair's 128 bytes of row l/8 (rows 0-7), then of row 8 + l/8.  The two loads go
  // through this wavefront's 2 KB of LDS per block (chunk c of row r at slot c ^ ((r/2)%8): 16
  // lanes hit 16 distinct 16-byte bank groups) and come back in the MFMA layout: row l%16, chunk
  // l/16 of fragment 2q or 2q+1.  (Loads of the MFMA layout itself cover 16 half lines each and
  // arrived at about two thirds of the rate.)  Rows past M and fragments past F read as zero.
  // Hidden pair q goes out just before W fragments 2q, 2q+1 of the first tile.
  uint4 hreg[KFWM][NMB];
  // ring slot u*KFWM + j always holds fragment j of a tile congruent to u modulo G
  uint4 ring[RING];
  {
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.hidden), 0, a.M * (int)row_bytes, 0x00020000);
    constexpr int NQ = KFWM / 2;
    uint4 hl[NQ][NMB][2];                                  // [pair][block][rows 0-7 | rows 8-15]
    const int c_ld = lane & 7, r_ld = lane >> 3;           // loading layout
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int kf = frag(2 * q);                          // even: the pair's first fragment
      const bool in = kf + (c_ld >> 2) < F;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned row = (unsigned)(rg * MR + mb * 16 + 8 * h + r_ld);
          hl[q][mb][h] = buffer_load16(hrs, in ? row * row_bytes + (unsigned)kf * 64u + (unsigned)c_ld * 16u : kOOB);
        }
#pragma unroll
      for (int j = 2 * q; j < 2 * q + 2; ++j) {
        ring[j] = buffer_load16(wrs, w_off(0, j));
        __builtin_amdgcn_sched_barrier(0);  // slot order = issue order
      }
    }
    static_assert((size_t)kWaves * NMB * 2048 <= lds_bytes(NMB), "the areas fit the kernel's LDS");
    uint4* area = smem + wave * (NMB * 128);               // 2 KB per 16-row block
    auto slot = [](int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); };
    const int r_mf = lane & 15, c_mf = lane >> 4;          // MFMA layout
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h) area[mb * 128 + slot(8 * h + r_ld, c_ld)] = hl[q][mb][h];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        hreg[2 * q][mb] = area[mb * 128 + slot(r_mf, c_mf)];
        hreg[2 * q + 1][mb] = area[mb * 128 + slot(r_mf, 4 + c_mf)];
      }
    }
    __syncthreads();   // the areas overlap the reduction buffers of the first tile
  }
#pragma unroll
  for (int u = 1; u < G; ++u)
#pragma unroll
    for (int j = 0; j < KFWM; ++j) {
      ring[u * KFWM + j] = buffer_load16(wrs, w_off(u, j));
      __builtin_amdgcn_sched_barrier(0);
    }

  // ---- stream the tiles -------------------------------------------------------------------------
  float* red = reinterpret_cast<float*>(smem);           // [2][kWaves][NMB][64 lanes][4] partials
  Stats st[P];
  TopK tk[TK ? P : 1];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    st[p] = stats_empty();
    if constexpr (TK) topk_clear(tk[p]);
  }
  f32x4 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mma_frag = [&](const uint4& w, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) acc[mb] = E::mma(w, hreg[j][mb], acc[mb]);
  };
  // tile r done: partials to LDS, one barrier, every thread folds its logit slots
  auto tile_end = [&](int r) __attribute__((always_inline)) {
    float* buf = red + (r & 1) * (kWaves * NMB * 256);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      *reinterpret_cast<f32x4*>(buf + ((wave * NMB + mb) * 64 + lane) * 4) = acc[mb];
      acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    if (r < nloc) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int f = tid + p * kThreads;          // slot: (mb, lane, component) of the tile
        if (f < LOGITS) {
          const int mb = f >> 8, rest = f & 255;
          float z = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) z += buf[(w * NMB + mb) * 256 + rest];
          const int v = (t_begin + r) * kTileRows + 4 * (rest >> 6) + (rest & 3);
          if (v < a.V) {
            stats_fold1(st[p], z, v);
            if constexpr (TK) topk_push_ascending(tk[p], z, v);
          }
        }
      }
    }
  };

  for (int r0 = 0; r0 < nloc_p; r0 += G) {
#pragma unroll
    for (int u = 0; u < G; ++u) {
#pragma unroll
      for (int j = 0; j < KFWM; ++j) {
        mma_frag(ring[u * KFWM + j], j);
        ring[u * KFWM + j] = buffer_load16(wrs, w_off(r0 + u + G, j));
        __builtin_amdgcn_sched_barrier(0);  // keep consume-then-refill order: the wait stays RING-1 deep
      }
      tile_end(r0 + u);
    }
  }

  // ---- merge each row's 16 slots inside the workgroup; one record per row -----------------------
  __syncthreads();
  float4* slots = reinterpret_cast<float4*>(smem);       // [LOGITS] statistics, by slot
  float2* lists = reinterpret_cast<float2*>(slots + LOGITS);   // [kTopK][LOGITS] (logit, id)
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int f = tid + p * kThreads;
    if (f < LOGITS) {
      slots[f] = stats_pack(st[p]);
      if constexpr (TK) {
#pragma unroll
        for (int i = 0; i < kTopK; ++i) lists[i * LOGITS + f] = make_float2(tk[p].z[i], __int_as_float(tk[p].id[i]));
      }
    }
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rec = __builtin_amdgcn_make_buffer_rsrc(
      a.partials, 0, a.n_rg * MR * a.G_v * 16, 0x00020000);
  for (int rr = wave * 4 + (lane >> 4); rr < MR; rr += kWaves * 4) {   // 4 rows per wavefront pass
    // slot of contributor k = lane%16 of row rr: vocabulary sub-row 4*(k/4) + k%4 of the tile
    const int k = lane & 15;
    const int f = (rr >> 4) * 256 + 64 * (k >> 2) + 4 * (rr & 15) + (k & 3);
    const Stats t = stats_row16_merge(stats_unpack(slots[f]));
    if (k == 0) record_store(rec, (unsigned)((((size_t)rg * MR + rr) * a.G_v + gv) * 16), stats_pack(t));
    if constexpr (TK) {
      TopK mine, best;
#pragma unroll
      for (int i = 0; i < kTopK; ++i) {
        const float2 e = lists[i * LOGITS + f];
        mine.z[i] = e.x;
        mine.id[i] = __float_as_int(e.y);
      }
      topk_row16_merge(mine, best);
      if (k == 0) {
        const __amdgpu_buffer_rsrc_t trec = __builtin_amdgcn_make_buffer_rsrc(
            a.topk_records, 0, a.n_rg * MR * a.G_v * (kTopK * 8), 0x00020000);
        const unsigned off = (unsigned)((((size_t)rg * MR + rr) * a.G_v + gv) * (kTopK * 8));
#pragma unroll
        for (int j = 0; j < kTopK / 2; ++j) record_store(trec, off + 16u * j, topk_record(best, j));
      }
    }
  }
  // The records must be complete before this workgroup is counted; device-scope stores need no
  // cache write-back, only the wait for their acknowledgement.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- two-level merge across workgroups --------------------------------------------------------
  // The records of each group of kGroup consecutive vocabulary ranges are merged, row by row, by
  // the group's last workgroup to finish; the last group to finish then merges the groups'
  // records of every row and commits (the two levels of the merge tree).  Each counter is
  // incremented with wrap-around: it runs 0 .. n-1 and its last arrival puts it back to 0, so a
  // workspace that starts zeroed is zero again between calls.
  __shared__ int s_last;
  const int grp = gv / kGroup;
  const int gsize = min(kGroup, a.G_v - kGroup * grp);
  if (tid == 0) {
    const unsigned prev = __builtin_amdgcn_atomic_inc32(a.group_tickets + rg * a.nq + grp, (unsigned)(gsize - 1),
                                                        __ATOMIC_RELAXED, "agent");
    s_last = prev == (unsigned)(gsize - 1);
  }
  __syncthreads();
  if (!s_last) return;
  const __amdgpu_buffer_rsrc_t l2 = __builtin_amdgcn_make_buffer_rsrc(a.level2, 0, a.n_rg * MR * a.nq * 16, 0x00020000);
  // 4 rows per wavefront pass; every pass's load is issued before the first merge, so the
  // passes (two at 64 rows) share one round trip to the coherence point
  constexpr int kPasses = (MR + kWaves * 4 - 1) / (kWaves * 4);
  float4 gv_rec[kPasses];
  float4 gv_list[TK ? kPasses : 1][kTopK / 2];            // with TK: the ranges' top-k lists
  const __amdgpu_buffer_rsrc_t trec = __builtin_amdgcn_make_buffer_rsrc(
      TK ? a.topk_records : a.partials, 0, TK ? a.n_rg * MR * a.G_v * (kTopK * 8) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t tl2 = __builtin_amdgcn_make_buffer_rsrc(
      TK ? a.topk_level2 : a.level2, 0, TK ? a.n_rg * MR * a.nq * (kTopK * 8) : 0, 0x00020000);
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int rr = pass * kWaves * 4 + wave * 4 + (lane >> 4);
    const int j = lane & 15, g = kGroup * grp + j;
    const unsigned row = (unsigned)(rg * MR + rr);
    const bool in = g < a.G_v && rr < MR;
    gv_rec[pass] = record_load(rec, in ? (row * (unsigned)a.G_v + (unsigned)g) * 16u : 0x80000000u);
    if constexpr (TK) {
#pragma unroll
      for (int q = 0; q < kTopK / 2; ++q)
        gv_list[pass][q] =
            record_load(trec, in ? (row * (unsigned)a.G_v + (unsigned)g) * (kTopK * 8u) + 16u * q : 0x80000000u);
    }
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int rr = pass * kWaves * 4 + wave * 4 + (lane >> 4);
    if (rr >= MR) continue;                   // (uniform over the row's 16 lanes)
    const int j = lane & 15, g = kGroup * grp + j;
    const unsigned row = (unsigned)(rg * MR + rr);
    const float4 v = g < a.G_v ? gv_rec[pass] : stats_pack(stats_empty());
    const Stats t = stats_row16_merge(stats_unpack(v));
    if (j == 0) record_store(l2, (row * (unsigned)a.nq + (unsigned)grp) * 16u, stats_pack(t));
    if constexpr (TK) {
      TopK mine, best;
      if (g < a.G_v) {
        topk_from_records(mine, gv_list[pass]);
      } else {
        topk_clear(mine);
      }
      topk_row16_merge(mine, best);
      if (j == 0) {
#pragma unroll
        for (int q = 0; q < kTopK / 2; ++q)
          record_store(tl2, (row * (unsigned)a.nq + (unsigned)grp) * (kTopK * 8u) + 16u * q, topk_record(best, q));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);              // the group's records are out before it is counted
  __syncthreads();
  const CommitArgs& c = a.c;
  const bool do_commit = (c.flags & kFlagCommit) != 0;
  // While the counter answers, each wavefront fetches the state of the sequence it would commit
  // first (only the last workgroup uses it; the others drop it): the loads go out after the
  // counter's increment and before the wait for its answer.
  const unsigned total = (unsigned)(a.n_rg * a.nq);
  unsigned prev = 0;
  if (tid == 0) prev = __builtin_amdgcn_atomic_inc32(a.ticket, total - 1, __ATOMIC_RELAXED, "agent");
  SeqState pre;
  if (do_commit && wave < c.B) pre = load_seq_state(c, wave);
  if (tid == 0) s_last = prev == total - 1;
  __syncthreads();
  if (!s_last) return;

  if constexpr (TK) {
    const __amdgpu_buffer_rsrc_t tl2 =
        __builtin_amdgcn_make_buffer_rsrc(a.topk_level2, 0, a.n_rg * MR * a.nq * (kTopK * 8), 0x00020000);
    finalize_sequences<true, true, true>(c, l2, a.nq, a.nq, 1, 0, c.B, smem, pre, wave < c.B ? wave : -1, tl2);
  } else {
    finalize_sequences<true, true>(c, l2, a.nq, a.nq, 1, 0, c.B, smem, pre, wave < c.B ? wave : -1, l2);
  }
}

// ----------------------------------------------------------------------------------------------
// GEMM-shaped LM head for many rows (B*L > 64, bf16): the work crosses the MFMA ridge, so W must
// be reused across all rows instead of being re-streamed per row group.
//
// A work unit is a vocabulary tile against all rows of a row group.  Four wavefronts (one per SIMD,
// so each may hold 256 accumulator registers) own the group's hidden rows in equal parts and share
// every W tile through LDS (tile shapes: GemmShape).  Per 64-element K stage:
//   * W moves HBM -> LDS by direct-to-LDS buffer loads, never through registers: each wavefront
//     instruction brings 8 whole 128-byte row segments (fully used cache lines) into a ring of
//     four stage buffers, issued three stages before their use.  Inside a row the 16-byte
//     chunks are permuted (chunk c of tile row r sits at slot c ^ swz(r)) so that the MFMA
//     fragment reads hit 16 distinct bank groups per 16 lanes;
//   * hidden rows are packed beforehand (pack_hidden_kernel) into MFMA fragment order, so each
//     fragment is one contiguous 1 KB load from L2; they run G::HDepth stages ahead in registers;
//   * VB x HB v_mfma_f32_32x32x16_bf16 per K16 step: acc[vb][hb] = W[32 vocab] x h[32 rows]^T.
// Vector-memory loads retire in issue order, so a wait for a hidden fragment also waits for
// every W load issued before it: the hidden fragments' lead bounds the W loads' latency cover.
// One barrier per stage, after the second K16 step.  Before it each wavefront waits until its
// own W loads for the next stage have landed (a counted wait: at least G::VmAfterW
// vector-memory instructions are issued after them in program order); after it the wavefront
// issues the W loads three stages ahead, into the buffer that every wavefront finished reading a
// stage earlier.
// With several row groups, the workgroups that share a vocabulary tile run on one XCD (block
// indices 8 apart) at the same pace, so W is fetched from HBM once and re-read from that L2.
// Lane l of acc[vb][hb] register r holds vocabulary row 32vb + 8(r/4) + 4(l/32) + r%4 of the tile
// against hidden row 32hb + l%32 of the wavefront: 16 VB logits of one row per lane and tile, in
// ascending vocabulary order, folded into that row's running statistics at the end of the tile.
// Each workgroup ends with one record per row; finalize_parts_kernel merges them and commits.
// ----------------------------------------------------------------------------------------------
constexpr int kGemmBK = 64;                               // K per stage
constexpr int kGemmRing = 4;                              // W stage buffers in LDS

// Tile shape: WAVES wavefronts, each owning VB 32-row vocabulary blocks x HB 32-row hidden blocks
// (VB * HB * WAVES = 64 accumulator blocks: every accumulator register of the CU's four SIMDs).
// Two shapes are built, both with 64 hidden rows per wavefront (few hidden rows make its hidden
// fragments a small register cost per stage of lead; 4 x 4 blocks, which read each W fragment
// for 4 products instead of 2, measured as fast at 512 rows and slower at 256):
//   * GemmR256: 4 wavefronts (one per SIMD, 256 accumulator registers each) x 8 x 2 blocks:
//     256 vocabulary rows per tile against a 256-row group;
//   * GemmR512: 8 wavefronts (two per SIMD, 128 accumulator registers each) x 4 x 2 blocks: 128
//     vocabulary rows per tile against a 512-row group.  While one wavefront of a SIMD folds its
//     statistics or waits, the other keeps the matrix core busy; each hidden fragment is read
//     for half as many products.  Used above 256 rows (below, most of a 512-row group is
//     padding).
template <int VB_, int HB_, int WAVES_>
struct GemmShape {
  static constexpr int VB = VB_, HB = HB_, Waves = WAVES_, Threads = 64 * WAVES_;
  static constexpr int BN = 32 * VB;                      // vocabulary rows per tile
  static constexpr int RowsPerWave = 32 * HB;
  static constexpr int Rows = Waves * RowsPerWave;        // hidden rows per row group
  static constexpr int Slot = BN * 8;                     // 16-byte slots per W stage buffer
  static constexpr int WDma = BN / 8 / Waves;             // W load instructions per wavefront per stage
  static constexpr int HDepth = 4 / HB;                   // stages of hidden fragments in flight (64 VGPRs)
  // vector-memory instructions issued after a stage's W loads and before the wait that must cover
  // them: the rest of that stage (2 K16 steps of hidden loads), one whole stage (4 K16 steps of
  // hidden loads + the next W loads) and the first half of the following one
  static constexpr int VmAfterW = 2 * HB + (4 * HB + WDma) + 2 * HB;
  static_assert(VB * HB * Waves == 64, "every accumulator register of the SIMDs");
  static_assert(VmAfterW <= 63, "vmcnt holds at most 63");
  // the prologue's first W stage has the other two prologue stages and every prologue hidden
  // load behind it, at least as many as the steady-state wait counts on
  static_assert(2 * WDma + HDepth * 4 * HB >= VmAfterW, "prologue wait covers W stage 0");
};
using GemmR256 = GemmShape<8, 2, 4>;
using GemmR512 = GemmShape<4, 2, 8>;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const void* hidden_packed;  // fragment-ordered hidden rows (pack_hidden_kernel), zero-padded to 32 rows
  const void* W;              // [V][H] bf16
  float4* records;            // [G_t][n_rg * rows per group]: each workgroup's records in one run
  int H, V, M;
  int n_rg;                   // row groups
  int G_t;                    // workgroups per row group
  int ntiles;                 // ceil(V / tile rows)
  unsigned packed_bytes;      // bytes of hidden_packed
  unsigned fold_gate;         // all ones (see fold_tile)
  uint4* topk_records;        // top-k fold only: [G_t][n_rg * rows per group] chunk lists, 64 bytes each
  int id_bits;                // top-k fold only: bit length of V (chunk entries)
};

// ---- top-k on the GEMM-shaped head: lists of chunk maxima ---------------------------------------
// A lane's 16 logits of one 32-row vocabulary block of a tile (ids 32vb + 8q + 4h + r, q, r < 4,
// h = lane / 32) form a chunk.  The fold already finds each chunk's maximum, its lowest arg-max
// and its second-largest value; with the top-k export each lane also keeps, per hidden row, the
// best kTopK chunks by (maximum desc, arg-max id asc), in LDS.  The row's k best tokens lie in the
// k best chunks (each of those has its maximum at or above the k-th best chunk maximum T, and any
// token outside them is at or below T and loses to all k maxima, ties by id), and inside such a
// chunk a token other than its maximum can only qualify when the chunk's second value reaches T;
// those few chunks are recomputed exactly in the finalizer.
// An entry is (maximum, id | gap code << id_bits), id_bits = bit length of V (so the all-ones id
// is no token).  The code is a lower bound on the gap g = maximum - second in a small float format
// (4 exponent bits for g in [2^-7, 2^8), the remaining 28 - id_bits bits of mantissa, truncated
// and then lowered by one unit; 0 = below 2^-7, all ones = 2^8 or more), so maximum - bound(code)
// bounds the second value from above.
constexpr int kMaxGemmTopkV = 1 << 22;                    // id_bits <= 22: at least 6 mantissa bits

__device__ __forceinline__ unsigned chunk_gap_code(float m, float m2, int id_bits) {
  const int mb = 28 - id_bits;                            // mantissa bits of the code
  const float g = m - m2;                                 // +inf when the chunk has one valid logit
  if (!(g >= 0.0078125f)) return 0u;                      // below 2^-7 (or no second value: never here)
  const unsigned bits = __float_as_uint(g);
  const int e = (int)(bits >> 23) - 127;
  if (e >= 8) return (1u << (32 - id_bits)) - 1u;         // 2^8 or more (and +inf)
  const unsigned c = ((unsigned)(e + 8) << mb) | ((bits & 0x7FFFFFu) >> (23 - mb));
  return c > (1u << mb) ? c - 1u : 0u;
}

__device__ __forceinline__ float chunk_gap_bound(unsigned code, int id_bits) {
  const int mb = 28 - id_bits;
  const unsigned e = code >> mb;
  if (e == 0) return 0.f;
  return __uint_as_float(((e + 119u) << 23) | ((code & ((1u << mb) - 1u)) << (23 - mb)));
}

// (z, id) of entry a before entry b: larger maximum first, lower id on ties (bitwise, so that the
// compiler emits selects rather than a branch per operand)
__device__ __forceinline__ bool chunk_before(uint2 a, uint2 b, unsigned id_mask) {
  const float za = __uint_as_float(a.x), zb = __uint_as_float(b.x);
  return (za > zb) | ((za == zb) & ((a.y & id_mask) < (b.y & id_mask)));
}

__device__ __forceinline__ uint2 chunk_empty(unsigned id_mask) { return make_uint2(__float_as_uint(-INFINITY), id_mask); }

// Hidden rows -> MFMA fragment order.  Fragment (rb, kg) of the packed rows is 1 KB: lane l's
// 16 bytes are K elements 16kg + 8(l/32) .. +7 of row 32rb + l%32 (zeros past M), at
// (rb * H/16 + kg) * 1 KB.  One wavefront packs four consecutive
// fragments of one 32-row block: each of its four loads covers 8 rows x 128 contiguous bytes, and
// each store writes 8 whole 128-byte lines of the output (lanes l%8 == u, 8 rows apart).
// ceil(M/32) * H/64 wavefronts in all (H % 64 == 0); wavefront w of them packs its four fragments.
__device__ __forceinline__ void pack_hidden_wave(const uint4* h, uint4* hp, int M, int H, int w, int lane) {
  const int KG = H / 16;
  const int quads = KG / 4;
  if (w >= ((M + 31) / 32) * quads) return;
  const int rb = w / quads, kg0 = 4 * (w % quads);
  const int u = lane & 7;                                 // 16-byte unit of the row's 128 bytes
  uint4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * rb + 8 * j + (lane >> 3);
    v[j] = row < M ? h[(unsigned)row * (unsigned)(H / 8) + (unsigned)(2 * kg0 + u)] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 8 * j + (lane >> 3);
    hp[((unsigned)(rb * KG + kg0 + (u >> 1)) << 6) + (unsigned)(i + 32 * (u & 1))] = v[j];
  }
}

// Grid: the pack's wavefronts, four per workgroup.
__global__ __launch_bounds__(256) void pack_hidden_kernel(const uint4* h, uint4* hp, int M, int H) {
  pack_hidden_wave(h, hp, M, H, gid() * 4 + (lid() >> 6), lid() & 63);
}

// The next step's pack riding on a finalizer launch (several steps per call): workgroups from
// first_block on pack, two wavefronts each.  The packed rows are free once the step's GEMM kernel
// has ended, which the finalizer's launch follows; the next GEMM kernel follows the finalizer.
struct PackArgs {
  const uint4* h;               // the next step's hidden rows, [M][H] bf16
  uint4* hp;                    // the packed copy in the workspace
  int M, H;
  int first_block;              // the finalizer's own workgroups come first; past the grid: no pack
};

__device__ __forceinline__ f32x16 mma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, export count 6:4 and LDS/scalar count 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Fold the 16 VB logits of hidden block HB held by this lane (ids ascending with (vb, r)) into st.
// Four interleaved sub-chains (r % 4) keep the top-2 / arg-max tracking and the sums independent;
// one maximum per 16 logits sets the exponent base.  With the chain maximum c1 >= second c2, the
// new second maximum after seeing z is the median of (c1, c2, z).  With TAIL, logits at offsets
// >= lim from v0 (ids >= V, last tile) become -inf first.
// Each 16-logit chunk sits behind its own bit of `gate` (all ones at run time): separate basic
// blocks keep the compiler from interleaving chunks, which would hold every logit in registers.
template <class G, int HB, bool TAIL, bool TK>
__device__ __forceinline__ void fold_tile(Stats& st, const f32x16 (&acc)[G::VB][G::HB], int v0, int lim,
                                          unsigned gate, uint2* list, int id_bits) {
#pragma unroll
  for (int vb = 0; vb < G::VB; ++vb) {
    if (!((gate >> (G::VB * HB + vb)) & 1u)) continue;
    float z[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = acc[vb][HB][r];
    if constexpr (TAIL) {
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 32 * vb + 8 * (r >> 2) + (r & 3) < lim ? z[r] : -INFINITY;
    }
    float c1[4], c2[4];
    int ci[4];                                            // offset of the chain maximum in the chunk
#pragma unroll
    for (int j = 0; j < 4; ++j) {                         // sub-chain j: r = j, j+4, j+8, j+12
      c1[j] = z[j];
      c2[j] = -INFINITY;
      ci[j] = j;
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const int r = j + 4 * q;
        c2[j] = __builtin_amdgcn_fmed3f(c1[j], c2[j], z[r]);
        ci[j] = z[r] > c1[j] ? 8 * q + j : ci[j];
        c1[j] = fmaxf(c1[j], z[r]);
      }
    }
    // merge the sub-chains (ids interleave, so ties go to the lower id explicitly)
    float m = c1[0], m2 = c2[0];
    int id = ci[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      m2 = fmaxf(fmaxf(m2, c2[j]), fminf(m, c1[j]));
      const bool better = (c1[j] > m) | ((c1[j] == m) & (ci[j] < id));
      id = better ? ci[j] : id;
      m = fmaxf(m, c1[j]);
    }
    const float mnew = fmaxf(st.m1, m);
    const float nb = mnew == -INFINITY ? 0.f : mnew * kLog2e;   // nothing valid yet: every term is 0
    float ps[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ps[j] = ex2(fmaf(z[j], kLog2e, -nb));
#pragma unroll
      for (int q = 1; q < 4; ++q) ps[j] += ex2(fmaf(z[j + 4 * q], kLog2e, -nb));
    }
    st.s = st.s * ex2(fmaf(st.m1, kLog2e, -nb)) + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    st.m2 = fmaxf(fmaxf(st.m2, m2), fminf(st.m1, m));
    st.id = m > st.m1 ? v0 + 32 * vb + id : st.id;        // ids of this chunk exceed earlier ones
    st.m1 = mnew;
    if constexpr (TK) {
      // the chunk enters this lane's list (entries [i * 64], best first) where it beats the last
      // entry.  A lane meets its chunks in ascending id order, so the new chunk goes in front of
      // the first entry with a smaller maximum (behind equal maxima: their ids are lower; empty
      // entries hold -inf), and every entry from there on moves down one place.
      const bool enter = m > __uint_as_float(list[(kTopK - 1) * 64].x);
      if (__builtin_amdgcn_ballot_w64(enter)) {
        if (enter) {
          uint2 carry = make_uint2(__float_as_uint(m),
                                   (unsigned)(v0 + 32 * vb + id) | (chunk_gap_code(m, m2, id_bits) << id_bits));
          bool shift = false;
#pragma unroll
          for (int i = 0; i < kTopK; ++i) {
            const uint2 e = list[i * 64];
            shift = shift | (m > __uint_as_float(e.x));
            list[i * 64] = make_uint2(shift ? carry.x : e.x, shift ? carry.y : e.y);
            carry = make_uint2(shift ? e.x : carry.x, shift ? e.y : carry.y);
          }
        }
      }
    }
  }
}

// The running statistics live in LDS between folds (st[hb * 64 + lane]): they are touched once
// per tile, and registers are what the streaming loop needs.
template <class G, int HB, bool TAIL, bool TK>
__device__ __forceinline__ void fold_all(float4* st, const f32x16 (&acc)[G::VB][G::HB], int v0, int lim,
                                         unsigned gate, uint2* lists, int id_bits) {
  Stats t = stats_unpack(st[HB * 64]);
  fold_tile<G, HB, TAIL, TK>(t, acc, v0, lim, gate, lists + HB * kTopK * 64, id_bits);
  st[HB * 64] = stats_pack(t);
  if constexpr (HB + 1 < G::HB) fold_all<G, HB + 1, TAIL, TK>(st, acc, v0, lim, gate, lists, id_bits);
}

// TAIL: V is not a multiple of the tile, so the last tile's padding ids are masked in the fold (a
// separate instantiation keeps that code out of the common case).
template <class G, bool TAIL, bool TK = false>
__device__ __forceinline__ void gemm_stats(const GemmArgs& a) {
  // W stage buffers [row * 8 + permuted chunk], one array each so that the compiler can tell a
  // buffer being filled from the one being read (it would otherwise wait for every fill)
  __shared__ uint4 wring0[G::Slot], wring1[G::Slot], wring2[G::Slot], wring3[G::Slot];
  auto ring = [&](int slot) -> uint4* { return slot == 0 ? wring0 : slot == 1 ? wring1 : slot == 2 ? wring2 : wring3; };
  __shared__ float4 st_lds[G::Waves * G::HB * 64];    // running statistics, [wave][hb][lane]
  // top-k: [wave][hb][entry][lane] chunk lists (kTopK entries of 8 bytes per lane and hidden row)
  __shared__ uint2 tk_lds[TK ? G::Waves * G::HB * kTopK * 64 : 1];
  const int tid = lid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroups of one vocabulary range (one per row group) sit 8 block indices apart: one XCD
  int rg, gi;
  if ((a.G_t & 7) == 0) {
    const int q = gid() >> 3;
    rg = q % a.n_rg;
    gi = (q / a.n_rg) * 8 + (gid() & 7);
  } else {
    rg = gid() % a.n_rg;
    gi = gid() / a.n_rg;
  }
  rg = __builtin_amdgcn_readfirstlane(rg);                // (uniform; keeps the stage logic scalar)
  gi = __builtin_amdgcn_readfirstlane(gi);
  const int nt = a.ntiles > gi ? (a.ntiles - gi + a.G_t - 1) / a.G_t : 0;   // tiles gi, gi+G_t, ...
  const int S = a.H / kGemmBK;                            // stages per tile (multiple of 4)
  const int KG = a.H / 16;
  const int total = __builtin_amdgcn_readfirstlane(nt * S);
  const unsigned row_bytes = (unsigned)a.H * 2u;
  const unsigned kOOB = 0x80000000u;                      // beyond any range: loads return 0
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.W), 0, (int)((unsigned)a.V * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.hidden_packed), 0, (int)a.packed_bytes, 0x00020000);

  // Addresses split into a per-lane constant (voffset) and a per-stage, wavefront-uniform part
  // (soffset, kOOB past the last stage so the loads return zeros without touching memory).
  // W load instruction i of this wavefront: tile rows 64w + 8i + l/8, lane l bringing chunk
  // (l%8) ^ swz(row) of the stage's 128-byte segment, landing at LDS slot row * 8 + l%8, with
  // swz(r) = (r ^ (r >> 3)) & 7.
  unsigned w_voff[G::WDma];
#pragma unroll
  for (int i = 0; i < G::WDma; ++i) {
    const int r = 8 * G::WDma * wave + 8 * i + (lane >> 3);
    w_voff[i] = (unsigned)r * row_bytes + 16u * (unsigned)((lane & 7) ^ ((r ^ (r >> 3)) & 7));
  }
  // stage (tile index ti, K block kk) of this workgroup
  // (readfirstlane: these are wavefront-uniform by construction, and the buffer instructions take
  // them in scalar registers)
  auto w_soff = [&](int ti, int kk) -> unsigned {
    const int s = ti * S + kk;
    return __builtin_amdgcn_readfirstlane(
        s < total ? (unsigned)((gi + ti * a.G_t) * G::BN) * row_bytes + (unsigned)(kk * kGemmBK * 2) : kOOB);
  };
  // W is read once: the loads carry the non-temporal policy (cache policy bit 1, nt), so W lines
  // leave the L2 first and the packed hidden rows, which every workgroup of the XCD re-reads per
  // tile, stay (HBM fetch 1.13x -> 1.05x the algorithmic bytes)
  auto w_issue = [&](int slot, unsigned soff) {
#pragma unroll
    for (int i = 0; i < G::WDma; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (__attribute__((address_space(3))) void*)(ring(slot) + (8 * G::WDma * wave + 8 * i) * 8), 16,
          w_voff[i], soff, 0, 2);
  };
  // fragment reads: lane l, block vb, K16 step ks reads tile row r = 32vb + l%32, chunk
  // c = 2ks + l/32, at slot r*8 + (c ^ swz(r)) = 256vb + 8(l%32) + (x_l ^ 2(ks ^ 2(vb&1))) with
  // x_l = (l/32) ^ (l%8) ^ ((l/8)%4)
  const int x_l = (lane >> 5) ^ (lane & 7) ^ ((lane >> 3) & 3);
  int rd_base[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) rd_base[k] = 8 * (lane & 31) + (x_l ^ (2 * k));
  auto w_frag = [&](int slot, int vb, int ks) -> uint4 {
    return ring(slot)[rd_base[ks ^ (2 * (vb & 1))] + 256 * vb];
  };
  // hidden fragment (block hb, K16 step 4kk + ks) of this wavefront
  const unsigned h_voff = ((unsigned)((G::Rows / 32) * rg + G::HB * wave) * (unsigned)KG) * 1024u + 16u * lane;
  const unsigned hb_stride = (unsigned)KG * 1024u;        // bytes between 32-row blocks
  auto h_soff = [&](int ti, int kk) -> unsigned {
    return __builtin_amdgcn_readfirstlane(ti * S + kk < total ? (unsigned)(kk * 4) * 1024u : kOOB);
  };
  auto h_load = [&](unsigned soff, int ks, int hb) -> uint4 {
    return __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(hrs, h_voff + (unsigned)(ks * 1024), soff + hb * hb_stride, 0));
  };

  uint4 hr[G::HDepth][4][G::HB], af[2][G::VB];
  f32x16 acc[G::VB][G::HB];
  float4* const st = st_lds + wave * (G::HB * 64) + lane;
#pragma unroll
  for (int hb = 0; hb < G::HB; ++hb) st[hb * 64] = stats_pack(stats_empty());
  uint2* const lists = tk_lds + (TK ? wave * (G::HB * kTopK * 64) + lane : 0);
  const int id_bits = TK ? __builtin_amdgcn_readfirstlane(a.id_bits) : 0;
  const unsigned id_mask = (1u << id_bits) - 1u;
  if constexpr (TK) {
#pragma unroll
    for (int i = 0; i < G::HB * kTopK; ++i) lists[i * 64] = chunk_empty(id_mask);
  }

  // prologue: W stages 0..2, hidden stages 0 .. depth-1, then the barrier that opens stage 0.
  // Every W load of the prologue has at least G::VmAfterW vector-memory instructions behind it
  // by the barrier that needs it, as in the steady state.  (S >= 4, so stages 0..2 are in tile 0.)
#pragma unroll
  for (int p = 0; p < 3; ++p) w_issue(p, w_soff(0, p));
#pragma unroll
  for (int p = 0; p < G::HDepth; ++p) {
    const unsigned so = h_soff(0, p);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int hb = 0; hb < G::HB; ++hb) hr[p][ks][hb] = h_load(so, ks, hb);
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<G::VmAfterW>();                            // W stage 0 landed
  __builtin_amdgcn_s_waitcnt(0xc07f);                     // and no LDS access pending
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int vb = 0; vb < G::VB; ++vb) af[0][vb] = w_frag(0, vb, 0);

  // four stages kk0 .. kk0+3 of tile ti; FIRST: the tile's first group, whose first K16 step
  // starts the accumulators from zero
  auto group = [&](int ti, int kk0, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    const bool last4 = kk0 + 4 == S;                      // stages kk0+u+depth / +3 may wrap to tile ti+1
#pragma unroll
    for (int u = 0; u < 4; ++u) {                         // stage kk0+u: buffer u, hidden set u % depth
      const int hp = u % G::HDepth;
      const bool hw = last4 && u + G::HDepth >= 4, ww = last4 && u + 3 >= 4;
      const unsigned hso = h_soff(ti + hw, kk0 + u + G::HDepth - (hw ? S : 0));
      const unsigned wso = w_soff(ti + ww, kk0 + u + 3 - (ww ? S : 0));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        // fragments of the next K16 step: this stage's buffer, or at ks == 3 the next stage's,
        // which the barrier at ks == 1 opened
#pragma unroll
        for (int vb = 0; vb < G::VB; ++vb) af[nxt][vb] = ks < 3 ? w_frag(u, vb, ks + 1) : w_frag((u + 1) & 3, vb, 0);
#pragma unroll
        for (int vb = 0; vb < G::VB; ++vb)
#pragma unroll
          for (int hb = 0; hb < G::HB; ++hb)
            acc[vb][hb] = mma32(af[cur][vb], hr[hp][ks][hb], (FIRST && u == 0 && ks == 0) ? f32x16{} : acc[vb][hb]);
#pragma unroll
        for (int hb = 0; hb < G::HB; ++hb) hr[hp][ks][hb] = h_load(hso, ks, hb);   // G::HDepth stages ahead
        // the fragment reads go out between the first MFMAs (into registers of their own), so
        // their latency is covered by the rest of the step; the hidden loads reuse the
        // registers the step's MFMAs read, so they come last
#pragma unroll
        for (int i = 0; i < G::VB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, G::VB * G::HB - G::VB, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, G::HB, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 1) {
          // open the next stage: its W landed for every wavefront; buffer (u+3)&3 was last read
          // in the previous stage, so the W loads three stages ahead may overwrite it
          wait_vmcnt<G::VmAfterW>();
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          w_issue((u + 3) & 3, wso);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  for (int ti = 0; ti < nt; ++ti) {
    group(ti, 0, std::true_type{});
    for (int kk0 = 4; kk0 < S; kk0 += 4) group(ti, kk0, std::false_type{});
    // tile done: fold its logits (the next tile's loads are in flight)
    const int t0 = (gi + ti * a.G_t) * G::BN;
    const int v0 = t0 + 4 * (lane >> 5);
    fold_all<G, 0, TAIL, TK>(st, acc, v0, a.V - v0, a.fold_gate, lists, id_bits);  // ids >= V are skipped
  }
  __builtin_amdgcn_s_waitcnt(0);                          // no load into LDS may outlive the workgroup

  // lanes l and l+32 hold the same rows over different vocabulary ids: merge the pair, then
  // lanes 0..31 write one record per row
  const unsigned h_row0 = (unsigned)(rg * G::Rows + wave * G::RowsPerWave + (lane & 31));
#pragma unroll
  for (int hb = 0; hb < G::HB; ++hb) {
    Stats lo, hi;
    int x0, x1;
    const Stats sh = stats_unpack(st[hb * 64]);
    row_swap<32>(__float_as_int(sh.m1), x0, x1); lo.m1 = __int_as_float(x0); hi.m1 = __int_as_float(x1);
    row_swap<32>(__float_as_int(sh.s), x0, x1);  lo.s = __int_as_float(x0);  hi.s = __int_as_float(x1);
    row_swap<32>(__float_as_int(sh.m2), x0, x1); lo.m2 = __int_as_float(x0); hi.m2 = __int_as_float(x1);
    row_swap<32>(sh.id, x0, x1);                 lo.id = x0;                 hi.id = x1;
    const Stats t = stats_merge(lo, hi);
    const unsigned row = h_row0 + 32u * hb;
    if (lane < 32 && (int)row < a.M) a.records[(size_t)gi * (a.n_rg * G::Rows) + row] = stats_pack(t);
    if constexpr (TK) {
      // the two lanes' chunk lists of the row -> its k best chunks (a bitonic merge: the better
      // of A[i] and B[k-1-i] for every i, then three compare-exchange stages)
      uint2 A[kTopK], B[kTopK], C[kTopK];
#pragma unroll
      for (int i = 0; i < kTopK; ++i) {
        const uint2 e = lists[(hb * kTopK + i) * 64];
        int x0, x1, y0, y1;
        row_swap<32>((int)e.x, x0, x1);
        row_swap<32>((int)e.y, y0, y1);
        A[i] = make_uint2((unsigned)x0, (unsigned)y0);
        B[i] = make_uint2((unsigned)x1, (unsigned)y1);
      }
#pragma unroll
      for (int i = 0; i < kTopK; ++i) {
        const bool a = chunk_before(A[i], B[kTopK - 1 - i], id_mask);  // (selects per component: no indexing)
        C[i].x = a ? A[i].x : B[kTopK - 1 - i].x;
        C[i].y = a ? A[i].y : B[kTopK - 1 - i].y;
      }
#pragma unroll
      for (int d = kTopK / 2; d >= 1; d /= 2)
#pragma unroll
        for (int i = 0; i < kTopK; ++i)
          if ((i & d) == 0) {
            const bool keep = chunk_before(C[i], C[i + d], id_mask);
            const unsigned x0 = C[i].x, x1 = C[i].y, y0 = C[i + d].x, y1 = C[i + d].y;
            C[i].x = keep ? x0 : y0;
            C[i].y = keep ? x1 : y1;
            C[i + d].x = keep ? y0 : x0;
            C[i + d].y = keep ? y1 : x1;
          }
      if (lane < 32 && (int)row < a.M) {
        uint4* dst = a.topk_records + ((size_t)gi * (a.n_rg * G::Rows) + row) * (kTopK / 2);
#pragma unroll
        for (int q = 0; q < kTopK / 2; ++q) dst[q] = make_uint4(C[2 * q].x, C[2 * q].y, C[2 * q + 1].x, C[2 * q + 1].y);
      }
    }
  }
}

// One kernel per tail handling (plain kernels, so both compilation passes see them)
__global__ __launch_bounds__(GemmR256::Threads) void gemm_r256_kernel(const GemmArgs a) { gemm_stats<GemmR256, false>(a); }
__global__ __launch_bounds__(GemmR256::Threads) void gemm_r256_tail_kernel(const GemmArgs a) { gemm_stats<GemmR256, true>(a); }
__global__ __launch_bounds__(GemmR512::Threads) void gemm_r512_kernel(const GemmArgs a) { gemm_stats<GemmR512, false>(a); }
__global__ __launch_bounds__(GemmR512::Threads) void gemm_r512_tail_kernel(const GemmArgs a) { gemm_stats<GemmR512, true>(a); }
__global__ __launch_bounds__(GemmR512::Threads) void gemm_r512_topk_kernel(const GemmArgs a) {
  gemm_stats<GemmR512, false, true>(a);
}
__global__ __launch_bounds__(GemmR512::Threads) void gemm_r512_topk_tail_kernel(const GemmArgs a) {
  gemm_stats<GemmR512, true, true>(a);
}

// Merge + commit after the GEMM-path kernel, spread over more compute units: workgroup
// (b, part) merges rows kFinRows*part .. +kFinRows-1 of sequence b (two wavefronts of four rows,
// one 16-lane row each, the tree of finalize_sequences: the same bits), then
//   * without a commit, writes those rows' outputs (or, for a vocabulary shard, their merged
//     records with global ids) and ends;
//   * with one, publishes conf / token / gap of its rows at device scope, and the last part of the
//     sequence to finish (a wrapping counter per sequence, so a zeroed workspace is zero again
//     after every call) commits the sequence from the published values.
// records: [G][nrows_total] (the GEMM kernels' layout).  Grid: B x ceil(L / kFinRows) workgroups of
// 128 threads, then the pack workgroups of PackArgs, if any.  tickets: [B] counters; row_out:
// [B*L] 16-byte values.
// With TK (top-k export after gemm_r512_topk_kernel) a workgroup takes kFinRowsTopk rows, one per
// wavefront (lane j + 16q merges records 16j + 4q .. +3, the same tree), and each wavefront also
// writes its row's export (gemm_topk_row).
constexpr int kFinRows = 8;
constexpr int kFinRowsTopk = 2;   // with the top-k export: one row per wavefront, two per workgroup

// Exact logits of one chunk (vocabulary rows base32 + 8q + 4h + r, q, r < 4) against hidden row
// `row`, by the same v_mfma_f32_32x32x16_bf16 sequence as the GEMM kernels (the same operands for
// the row's column, K order and zero start), so every value is bit-identical to the one the GEMM
// folded.  An output element depends only on its A row, its B column and its own accumulator, so
// the other elements may hold anything: A row i takes chunk row slot 4(i/8) + i%4 (the rows with
// (i/4)%2 == h are the chunk's, in the GEMM's order) and every B column takes the hidden row.
// The operands are staged in this wavefront's LDS area (kRcLdsBytes), K segment by K segment, with
// direct-to-LDS loads, all in flight at once: slot s = 4q + r holds the chunk row's segment, slot
// 16 the hidden row's, kRcSlotBytes apart (16 bytes of padding put the A reads of the 16 slots on
// distinct banks).  (The compiler cannot tell which direct-to-LDS load an LDS read depends on, so
// it waits for all of them before the first read anyway.)  The operand reads of the next eight
// MFMAs go out before the current eight.  Lane l gets the 16 logits of lane (row % 32) + 32h:
// register r is vocabulary row base32 + 8(r/4) + 4h + r%4.
constexpr int kRcPieceK = 512;                            // K elements of one row per direct-to-LDS load
constexpr int kRcSegK = 2048;                             // K elements staged at a time
constexpr int kRcSegBytes = kRcSegK * 2;
constexpr int kRcSlotBytes = kRcSegBytes + 16;
constexpr int kRcLdsBytes = 17 * kRcSlotBytes;            // 16 chunk rows + the hidden row

__device__ void gemm_chunk_logits(__amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t hrs, int base32, int h, int row,
                                  int H, uint4* area, float (&zr)[16]) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int lane = __lane_id();
  const int i = lane & 31, hk = lane >> 5;
  const int slot = 4 * (i >> 3) + (i & 3);
  const unsigned row_bytes = (unsigned)H * 2u;
  const uint4* a_src = area + (slot * kRcSlotBytes + 16 * hk) / 16;
  const uint4* b_src = area + (16 * kRcSlotBytes + 16 * hk) / 16;
  f32x16 acc = f32x16{};
  uint4 a0[8], b0[8], a1[8], b1[8];
  auto lds8 = [&](int kg, uint4 (&a)[8], uint4 (&b)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = a_src[2 * (kg + u)];
      b[u] = b_src[2 * (kg + u)];
    }
  };
  auto mma8 = [&](const uint4 (&a)[8], const uint4 (&b)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = mma32(a[u], b[u], acc);   // (the very first adds to zeros)
  };
  for (int seg0 = 0; seg0 < H; seg0 += kRcSegK) {        // (uniform)
    const int seg_bytes = min(kRcSegK, H - seg0) * 2;     // multiple of 512
    const int np = (seg_bytes + kRcPieceK * 2 - 1) / (kRcPieceK * 2);
    __builtin_amdgcn_s_waitcnt(0xc07f);                   // the previous segment's LDS reads are done
#pragma unroll 1
    for (int sl = 0; sl < 17; ++sl) {
      const unsigned r = sl < 16 ? (unsigned)(base32 + 8 * (sl >> 2) + 4 * h + (sl & 3)) : (unsigned)row;
#pragma unroll 1
      for (int c = 0; c < np; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sl < 16 ? wrs : hrs,
                                                 (lds_ptr)((char*)area + sl * kRcSlotBytes + c * kRcPieceK * 2), 16,
                                                 r * row_bytes + (unsigned)(seg0 + c * kRcPieceK) * 2u + 16u * (unsigned)lane,
                                                 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);                        // (vmcnt: the direct-to-LDS loads have landed)
    const int kgs = seg_bytes / 32;                       // K16 steps: a multiple of 16
    lds8(0, a0, b0);
    for (int kg = 0; kg < kgs; kg += 16) {
      lds8(kg + 8, a1, b1);
      mma8(a0, b0);
      if (kg + 16 < kgs) lds8(kg + 16, a0, b0);
      mma8(a1, b1);
    }
  }
  const int src_lane = __builtin_amdgcn_readfirstlane((row & 31) + 32 * h);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const float v = acc[rr];
    zr[rr] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
  }
}

// The top-k export of one row from its workgroups' chunk lists (one wavefront):
//   1. the k best chunks of the row: lane l holds lists l, l+64, ... (one per GEMM workgroup), and
//      kTopK rounds take the best head across the wavefront;
//   2. the candidates are those chunks' maxima, plus every other token of a chunk whose second
//      value can reach the k-th chunk maximum T (maximum - bound(gap code) >= T), recomputed
//      exactly, best first; a recomputed token enters only above the current k-th candidate;
//   3. lanes i < topk write rank i with probability 2^((z - M) log2 e) / S.
constexpr int kTopkListsPerLane = kMaxVocabGroups / 64;

// This lane's chunk lists of the row (lists lane, lane + 64, ...; past G: out of range, zeros).
// Issued beside the row's statistics records, so both arrive in one round trip.
__device__ __forceinline__ void gemm_topk_load(__amdgpu_buffer_rsrc_t tk, int G, int nrows_total, int row, bool rin,
                                               uint4 (&e)[kTopkListsPerLane][kTopK / 2]) {
  const int lane = __lane_id();
#pragma unroll
  for (int n = 0; n < kTopkListsPerLane; ++n) {
    const int g = lane + 64 * n;
    const unsigned off = g < G && rin ? (unsigned)(g * nrows_total + row) * (kTopK * 8u) : 0x80000000u;
#pragma unroll
    for (int q = 0; q < kTopK / 2; ++q) e[n][q] = buffer_load16(tk, off == 0x80000000u ? off : off + 16u * q);
  }
}

__device__ void gemm_topk_row(const CommitArgs& c, const uint4 (&e)[kTopkListsPerLane][kTopK / 2], int G, int row,
                              bool rin, __amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t hrs, int H, int V,
                              int id_bits, float M, float inv_s, uint4* area) {
  constexpr int N = kTopkListsPerLane;
  const int lane = __lane_id();
  const unsigned id_mask = (1u << id_bits) - 1u;
  uint2 Lst[N][kTopK];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const bool in = lane + 64 * n < G && rin;
#pragma unroll
    for (int q = 0; q < kTopK / 2; ++q) {
      Lst[n][2 * q] = in ? make_uint2(e[n][q].x, e[n][q].y) : chunk_empty(id_mask);
      Lst[n][2 * q + 1] = in ? make_uint2(e[n][q].z, e[n][q].w) : chunk_empty(id_mask);
    }
  }
  // 1. the k best chunks, in order (every lane ends with them)
  uint2 C[kTopK];
#pragma unroll
  for (int r = 0; r < kTopK; ++r) {
    uint2 bh = Lst[0][0];
    int bn = 0;
#pragma unroll
    for (int n = 1; n < N; ++n) {
      const bool better = chunk_before(Lst[n][0], bh, id_mask);
      bh = make_uint2(better ? Lst[n][0].x : bh.x, better ? Lst[n][0].y : bh.y);
      bn = better ? n : bn;
    }
    // the best head: the largest maximum, then the lowest id.  Entries are real chunks (finite
    // maxima) or empty (-inf, the all-ones id), and no chunk sits in two lists, so the winner is
    // unique; the lowest-id reduction runs only when several heads share the maximum.
    const float m = wave_max(__uint_as_float(bh.x));
    const bool top = __uint_as_float(bh.x) == m && (bh.y & id_mask) != id_mask;
    uint64_t wl = __builtin_amdgcn_ballot_w64(top);
    if (__builtin_popcountll(wl) > 1) {                   // (uniform)
      const int id = wave_allreduce_min(top ? (int)(bh.y & id_mask) : (int)id_mask);
      wl = __builtin_amdgcn_ballot_w64(top && (int)(bh.y & id_mask) == id);
    }
    const bool win = (wl >> lane) & 1ull;
    C[r] = chunk_empty(id_mask);
    if (wl) {
      const int w = __builtin_ctzll(wl);
      C[r] = make_uint2(__float_as_uint(m), (unsigned)__builtin_amdgcn_readlane((int)bh.y, w));
    }
    if (win) {
#pragma unroll
      for (int n = 0; n < N; ++n)
        if (n == bn) {
#pragma unroll
          for (int i = 0; i < kTopK - 1; ++i) Lst[n][i] = Lst[n][i + 1];
          Lst[n][kTopK - 1] = chunk_empty(id_mask);
        }
    }
  }
  // 2. the candidates: the chunk maxima, best first, then the recomputed chunks' other tokens
  uint2 F[kTopK];
#pragma unroll
  for (int i = 0; i < kTopK; ++i) F[i] = make_uint2(C[i].x, C[i].y & id_mask);
  const float T = __uint_as_float(C[kTopK - 1].x);
  for (int i = 0; i < kTopK; ++i) {
    uint2 ci = C[0];                                      // (selects: no indexing by a variable)
#pragma unroll
    for (int k = 1; k < kTopK; ++k) ci = make_uint2(i == k ? C[k].x : ci.x, i == k ? C[k].y : ci.y);
    const float zc = __uint_as_float((unsigned)__builtin_amdgcn_readfirstlane((int)ci.x));
    const unsigned idc = (unsigned)__builtin_amdgcn_readfirstlane((int)ci.y);
    const bool recompute = zc > -INFINITY && zc - chunk_gap_bound(idc >> id_bits, id_bits) >= T;
    if (!recompute) continue;                             // (uniform)
    const int id1 = (int)(idc & id_mask);
    const int base32 = id1 & ~31, h = (id1 >> 2) & 1;
    float zr[16];                                         // the chunk's 16 logits, in every lane
    gemm_chunk_logits(wrs, hrs, base32, h, row, H, area, zr);
#pragma unroll 1
    for (int rr = 0; rr < 16; ++rr) {
      const int v = base32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
      float zv = zr[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) zv = rr == q ? zr[q] : zv;
      uint2 carry = make_uint2(__float_as_uint(zv), (unsigned)v);
      if (v >= V || v == id1 || !chunk_before(carry, F[kTopK - 1], id_mask)) continue;   // (uniform)
#pragma unroll
      for (int k = 0; k < kTopK; ++k) {
        const bool b = chunk_before(carry, F[k], id_mask);
        const uint2 e = F[k];
        F[k] = make_uint2(b ? carry.x : e.x, b ? carry.y : e.y);
        carry = make_uint2(b ? e.x : carry.x, b ? e.y : carry.y);
      }
    }
  }
  // 3. the export: lane i writes rank i
  if (rin && lane < c.topk) {
    uint2 e = F[0];
#pragma unroll
    for (int i = 1; i < kTopK; ++i) e = make_uint2(lane == i ? F[i].x : e.x, lane == i ? F[i].y : e.y);
    const bool real = e.y != id_mask;
    const size_t o = (size_t)row * c.topk + lane;
    c.out_topk_tokens[o] = real ? (int)e.y : -1;
    if (c.out_topk_prob) c.out_topk_prob[o] = real ? fminf(ex2((__uint_as_float(e.x) - M) * kLog2e) * inv_s, 1.f) : 0.f;
  }
}

struct GemmTopkArgs {           // the export's inputs on the GEMM path (TK finalizer only)
  const uint4* lists;           // [G][nrows_total] chunk lists of gemm_r512_topk_kernel
  const void* W;                // [V][H] bf16
  const void* hidden;           // [M][H] bf16, the step's hidden rows
  int H, V;
  int id_bits;                  // bit length of V (the chunk entries' id field)
};

template <bool TK>
__global__ __launch_bounds__(128) void finalize_parts_kernel(const CommitArgs c, const float4* records, int G,
                                                             int nrows_total, unsigned* tickets, float4* row_out,
                                                             const GemmTopkArgs tka, const PackArgs pk) {
  if (gid() >= pk.first_block) {                          // (uniform) a pack workgroup
    pack_hidden_wave(pk.h, pk.hp, pk.M, pk.H, (gid() - pk.first_block) * 2 + (lid() >> 6), lid() & 63);
    return;
  }
  constexpr unsigned kOOB = 0x80000000u;
  constexpr int kRows = TK ? kFinRowsTopk : kFinRows;
  const int parts = (c.L + kRows - 1) / kRows;
  const int b = gid() / parts, part = gid() % parts;
  const int tid = lid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool do_commit = (c.flags & kFlagCommit) != 0;
  const __amdgpu_buffer_rsrc_t rec =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float4*>(records), 0, nrows_total * G * 16, 0x00020000);
  const int r = part * kRows + (TK ? wave : wave * 4 + (lane >> 4));   // row within the sequence
  const bool rin = r < c.L;
  const int row = b * c.L + (rin ? r : 0);
  const int j = lane & 15;
  const bool writer = TK ? lane == 0 : j == 0;              // one lane per row writes its outputs
  Stats t;
  // with TK: the row's chunk lists, loaded right behind the statistics records
  uint4 tl[TK ? kTopkListsPerLane : 1][kTopK / 2];
  const __amdgpu_buffer_rsrc_t tk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(tka.lists), 0, TK ? nrows_total * G * (kTopK * 8) : 0, 0x00020000);
  if (G <= kGroup) {
    const float4 v = record_load_after_kernel(rec, j < G && rin ? 16u * (unsigned)(row + j * nrows_total) : kOOB);
    if constexpr (TK) gemm_topk_load(tk, G, nrows_total, row, rin, tl);
    t = stats_row16_merge(stats_unpack_if(v, j < G));
  } else if constexpr (TK) {
    // one row per wavefront: lane j + 16qq merges records 16j + 4qq .. +3 in registers, the
    // quarters of each group pairwise across the 16-lane rows, then the groups: the same tree as
    // one lane per group (stats_merge is symmetric), with four records per lane instead of 16
    const int qq = lane >> 4;
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int g = kGroup * j + 4 * qq + k;
      v[k] = record_load_after_kernel(rec, g < G && rin ? 16u * (unsigned)(row + g * nrows_total) : kOOB);
    }
    if constexpr (TK) gemm_topk_load(tk, G, nrows_total, row, rin, tl);
    Stats q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = stats_unpack_if(v[k], kGroup * j + 4 * qq + k < G);
    t = stats_row16_merge(stats_merge_rows<32>(stats_merge_rows<16>(stats_tree(q))));
  } else {
    float4 v[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int g = kGroup * j + k;
      v[k] = record_load_after_kernel(rec, g < G && rin ? 16u * (unsigned)(row + g * nrows_total) : kOOB);
    }
    Stats q[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) q[k] = stats_unpack_if(v[k], kGroup * j + k < G);
    t = stats_row16_merge(stats_tree(q));
  }
  // S >= 1 in exact arithmetic; the rounding of m*log2(e) may put 1/S a few ulps above 1
  const float conf = fminf(1.f / t.s, 1.f), gap = t.m1 - t.m2;
  if constexpr (TK) {
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(tka.W), 0, (int)((unsigned)tka.V * (unsigned)tka.H * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(tka.hidden), 0, (int)((unsigned)(c.B * c.L) * (unsigned)tka.H * 2u), 0x00020000);
    __shared__ uint4 rc_area[TK ? kFinRowsTopk * kRcLdsBytes / 16 : 1];   // a recompute area per wavefront
    gemm_topk_row(c, tl, G, row, rin, wrs, hrs, tka.H, tka.V, tka.id_bits, t.m1, 1.f / t.s,
                  rc_area + (TK ? wave * (kRcLdsBytes / 16) : 0));
  }
  if (!do_commit) {
    if (rin && writer) {
      if (c.out_records) {                                // vocabulary shard: the merged record
        Stats o = t;
        o.id = t.id + c.v_begin;
        c.out_records[row] = stats_pack(o);
      } else {
        c.out_tokens[row] = t.id;
        if (c.out_conf) c.out_conf[row] = conf;
        if (c.out_gap) c.out_gap[row] = gap;
      }
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(row_out, 0, c.B * c.L * 16, 0x00020000);
  if (rin && writer) record_store(out, 16u * (unsigned)row, make_float4(conf, __int_as_float(t.id), gap, 0.f));
  __builtin_amdgcn_s_waitcnt(0);                          // published before this part is counted
  __syncthreads();
  __shared__ int s_last;
  // the sequence's state is fetched while the counter answers (used by the last part only)
  unsigned prev = 0;
  if (tid == 0) prev = __builtin_amdgcn_atomic_inc32(tickets + b, (unsigned)(parts - 1), __ATOMIC_RELAXED, "agent");
  SeqState pre;
  if (wave == 0) pre = load_seq_state(c, b);
  if (tid == 0) s_last = prev == (unsigned)(parts - 1);
  __syncthreads();
  if (!s_last || wave != 0) return;
  const bool in = lane < c.L;
  const float4 v = record_load(out, in ? 16u * (unsigned)(b * c.L + lane) : kOOB);
  commit_sequence(c, b, in ? v.x : 0.f, in ? __float_as_int(v.y) : 0, pre);
  if (in) {
    if (c.out_conf) c.out_conf[b * c.L + lane] = v.x;
    if (c.out_gap) c.out_gap[b * c.L + lane] = v.z;
  }
}

// Merge + commit of gathered vocabulary shards (records [G][B*L], shards in vocabulary order):
// the same merge and commit as the single-GPU head's, one workgroup per sequence.
__global__ __launch_bounds__(kThreads) void merge_commit_kernel(const CommitArgs c, const float4* records, int G) {
  __shared__ uint4 stage[kRowsPerStage * 12 / 16];
  const int b = gid();
  const int M = c.B * c.L;
  const int wave = __builtin_amdgcn_readfirstlane(lid() >> 6);
  const __amdgpu_buffer_rsrc_t rec =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float4*>(records), 0, G * M * 16, 0x00020000);
  SeqState pre;
  if (wave == 0) pre = load_seq_state(c, b);
  // (the gathered records may have been written by a copy or by another device: device-scope
  // loads, as in the in-kernel merge)
  finalize_sequences<false, true>(c, rec, G, 1, M, b, b + 1, stage, pre, wave == 0 ? b : -1, rec);
}

// dlm_commit: conf / tokens given, one wavefront per sequence.
__global__ __launch_bounds__(kThreads) void commit_kernel(const CommitArgs a, const float* conf, const int32_t* tok) {
  const int b = gid() * kWaves + (lid() >> 6);
  if (b >= a.B) return;
  const int l = lid() & 63;
  const bool in = l < a.L;
  const size_t row = (size_t)b * a.L + l;
  commit_sequence(a, b, in ? conf[row] : 0.f, in ? tok[row] : 0, load_seq_state(a, b));
}

// dlm_workspace_init: zero fill.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* p, size_t n, int nthreads) {
  const size_t stride = (size_t)nthreads;
  const size_t nvec = n / 16;
  uint4* p4 = reinterpret_cast<uint4*>(p);
  for (size_t i = (size_t)gid() * 256 + lid(); i < nvec; i += stride) p4[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = nvec * 16 + (size_t)gid() * 256 + lid(); i < n; i += stride) p[i] = 0;
}

}  // namespace dlm

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

#include "dlm.h"

namespace dlm {

constexpr int kWaves = 8;             // wavefronts per workgroup
constexpr int kThreads = kWaves * 64; // workgroup size
constexpr int kTileRows = 16;         // vocabulary rows per MFMA tile
constexpr int kPrefetch = 16;         // 16-byte W fragments in flight per lane
constexpr int kRowsPerStage = 1024;   // finalize: rows staged in LDS at a time
constexpr int kMergeLanes = 16;       // finalize: lanes merging one row
constexpr int kMaxVocabGroups = kMergeLanes * 16;
constexpr unsigned kFlagCommit = 1u << 16;  // internal: run the commit policies
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Rule {
  int kind;
  float thr;
  float decay;
  int depth;
};

// Everything the commit policies touch.
struct CommitArgs {
  uint8_t* mask;
  dlm_credit_slot* credit;
  int32_t* out_tokens;
  uint8_t* out_commit;
  float* out_conf;
  float* out_gap;
  int B, L;
  unsigned flags;
  Rule rules[DLM_MAX_RULES];
  uint8_t rule_of[DLM_MAX_SEQS];
};

// LDS: area A holds the hidden rows (phases 1-2) and later the finalize stage (conf + token of
// kRowsPerStage rows); area B the per-wavefront statistics of phase 3.  Sizes in 16-byte units.
__host__ __device__ constexpr size_t lds_area_a(size_t h_vec) {
  return h_vec > (size_t)kRowsPerStage / 2 ? h_vec : (size_t)kRowsPerStage / 2;
}
__host__ __device__ constexpr size_t lds_bytes(size_t h_vec, int MR) {
  return (lds_area_a(h_vec) + (size_t)kWaves * MR) * 16;
}

struct StepArgs {
  const void* hidden;  // [M][H]
  const void* W;       // [V][H]
  float4* partials;    // [n_rg][G_v][MR] statistics of each vocabulary range
  unsigned* ticket;    // completion counter, zero between calls
  int H, V, M;
  int n_rg;            // row groups of MR rows
  int G_v;             // vocabulary ranges (multiple of 8)
  int ntiles;          // ceil(V / 16)
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

__device__ __forceinline__ Stats stats_empty() {
  Stats t;
  t.m1 = -INFINITY;
  t.s = 0.f;
  t.m2 = -INFINITY;
  t.id = 0x7fffffff;
  return t;
}

__device__ __forceinline__ Stats stats_merge(const Stats& a, const Stats& b) {
  Stats r;
  r.m1 = fmaxf(a.m1, b.m1);
  const float sa = a.s == 0.f ? 0.f : a.s * ex2((a.m1 - r.m1) * kLog2e);
  const float sb = b.s == 0.f ? 0.f : b.s * ex2((b.m1 - r.m1) * kLog2e);
  r.s = sa + sb;
  r.id = a.m1 > b.m1 ? a.id : (b.m1 > a.m1 ? b.id : min(a.id, b.id));
  r.m2 = fmaxf(fmaxf(a.m2, b.m2), fminf(a.m1, b.m1));
  return r;
}

__device__ __forceinline__ Stats stats_shfl_xor(const Stats& a, int off) {
  Stats r;
  r.m1 = __shfl_xor(a.m1, off);
  r.s = __shfl_xor(a.s, off);
  r.m2 = __shfl_xor(a.m2, off);
  r.id = __shfl_xor(a.id, off);
  return r;
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

// Fold four logits of ascending ids v0..v0+3 (ids >= V are padding) into the running stats.
__device__ __forceinline__ void stats_fold4(Stats& st, f32x4 z, int v0, int V) {
#pragma unroll
  for (int r = 0; r < 4; ++r) z[r] = (v0 + r < V) ? z[r] : -INFINITY;
  const float mnew = fmaxf(st.m1, fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
  if (mnew == -INFINITY) return;  // nothing valid seen yet
  const float nb = mnew * kLog2e;
  float s = st.s * ex2(fmaf(st.m1, kLog2e, -nb));
#pragma unroll
  for (int r = 0; r < 4; ++r) s += ex2(fmaf(z[r], kLog2e, -nb));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    st.m2 = fmaxf(st.m2, fminf(z[r], st.m1));
    if (z[r] > st.m1) {
      st.m1 = z[r];
      st.id = v0 + r;
    }
  }
  st.s = s;
}

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
  int idx = __lane_id();
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(idx, off);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  }
  return idx;
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

// One sequence on one wavefront: policy, outputs and state update.
__device__ void commit_sequence(const CommitArgs& a, int b, float conf, int tok) {
  const int l = __lane_id();
  const bool in = l < a.L;
  const size_t row = (size_t)b * a.L + l;
  const Rule R = a.rules[a.rule_of[b]];
  if (!in) conf = -INFINITY;

  bool masked = in && a.mask[row] != 0;
  uint64_t U = ballot(masked);
  const bool advance = U == 0ull && (a.flags & DLM_AUTO_ADVANCE);
  if (advance) {
    masked = in;
    U = ballot(masked);
  }

  // credit slots of this position (cleared when a new block starts)
  int st[DLM_CREDIT_SLOTS];
  float sc[DLM_CREDIT_SLOTS];
  const bool has_credit = a.credit != nullptr;
  if (has_credit && in) {
#pragma unroll
    for (int i = 0; i < DLM_CREDIT_SLOTS; ++i) {
      const dlm_credit_slot cs = a.credit[row * DLM_CREDIT_SLOTS + i];
      st[i] = advance ? -1 : cs.token;
      sc[i] = advance ? 0.f : cs.credit;
    }
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

  if (in) {
    const bool c = (C >> l) & 1ull;
    if (a.out_tokens) a.out_tokens[row] = tok;
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
// The fused step kernel.
//
// Grid: G_v vocabulary ranges x n_rg row groups, one workgroup each, 8 wavefronts.  Workgroup
// ids are dealt round-robin over the 8 XCDs; the row groups of one vocabulary range are placed
// on the same XCD back to back so the repeated W reads of a range hit that XCD's L2.
//
// Phase 1: the row group's hidden rows go to LDS in MFMA fragment order.
// Phase 2: each wavefront streams the W tiles (16 vocab rows) of its share of the range straight
//          from HBM into registers (kPrefetch fragments in flight), multiplies them with the
//          hidden fragments on the matrix cores and folds every finished tile into per-lane
//          online-softmax statistics.
// Phase 3: lanes, then wavefronts merge their statistics; one record per row goes to memory.
// Phase 4: the last workgroup to finish (completion counter) merges the records of every row in
//          a fixed order, derives conf / token / gap and runs each sequence's commit policy.
// ----------------------------------------------------------------------------------------------
template <class T, int MR>
__global__ __launch_bounds__(kThreads) void step_kernel(const StepArgs a) {
  extern __shared__ uint4 smem[];
  using E = Elem<T>;
  constexpr int NMB = MR / 16;                  // 16-row blocks of hidden rows
  constexpr int CH = 16 / E::kBytes;            // elements per 16-byte chunk
  constexpr int KF = 4 * CH;                    // K covered by one fragment
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the loop scalar

  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int rg = slot % a.n_rg;
  const int gv = (slot / a.n_rg) * 8 + xcd;

  const int H = a.H;
  const int F = H / KF;                          // fragments per row
  const int hchunks = H / CH;                    // 16-byte chunks per hidden row
  uint4* lds_h = smem;                           // [F][NMB][64] fragments
  const size_t h_vec = (size_t)MR * hchunks;     // hidden-state area, in 16-byte units
  float4* red = reinterpret_cast<float4*>(smem + lds_area_a(h_vec));  // [kWaves][MR] statistics

  // ---- phase 1: hidden rows of this group -> LDS, straight from memory (no registers) -------
  // One wavefront instruction fills one 1 KB fragment block (kf, mb): lane l brings row
  // mb*16 + l%16, 16-byte chunk kf*4 + l/16.  Rows past M fall outside the buffer range and
  // arrive as zeros.
  {
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.hidden), 0, a.M * hchunks * 16, 0x00020000);
    const int nblk = F * NMB;
    for (int p = wave; p < nblk; p += kWaves) {
      const int kf = p / NMB, mb = p - kf * NMB;
      const unsigned r = (unsigned)(rg * MR + mb * 16 + (lane & 15));
      const unsigned off = (r * (unsigned)hchunks + (unsigned)(kf * 4 + (lane >> 4))) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          hrs, (__attribute__((address_space(3))) void*)(lds_h + (size_t)p * 64), 16, off, 0, 0, 0);
    }
  }

  // ---- phase 2 set-up; the first W loads overlap the hidden-state fill -----------------------
  const int t_begin = (int)((long long)gv * a.ntiles / a.G_v);
  const int t_end = (int)((long long)(gv + 1) * a.ntiles / a.G_v);
  const int nloc = t_end - t_begin;
  const int ntw = nloc > wave ? (nloc - wave + kWaves - 1) / kWaves : 0;
  const int Q = ntw * F;
  const int Qp = (Q + kPrefetch - 1) / kPrefetch * kPrefetch;
  const long long row0 = (long long)t_begin * kTileRows;
  const long long row_end = min((long long)a.V, (long long)t_end * kTileRows);
  const long long nbytes = row_end > row0 ? (row_end - row0) * H * E::kBytes : 0;
  const char* wbase = static_cast<const char*>(a.W) + row0 * H * E::kBytes;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wbase), 0, (int)nbytes, 0x00020000);
  const unsigned row_bytes = (unsigned)H * E::kBytes;
  const unsigned tile_stride = (unsigned)kWaves * kTileRows * row_bytes;
  const unsigned frag_bytes = KF * E::kBytes;
  const unsigned kOOB = 0x80000000u;             // beyond any range: loads return 0, no traffic
  unsigned ld_off = (unsigned)(wave * kTileRows + (lane & 15)) * row_bytes + (lane >> 4) * 16u;
  int ld_q = 0, ld_kf = 0;
  auto next_off = [&]() -> unsigned {
    const unsigned o = ld_q < Q ? ld_off + (unsigned)ld_kf * frag_bytes : kOOB;
    ++ld_q;
    if (++ld_kf == F) {
      ld_kf = 0;
      ld_off += tile_stride;
    }
    return o;
  };
  uint4 ring[kPrefetch];
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) ring[j] = buffer_load16(rsrc, next_off());

  __syncthreads();

  // ---- phase 2: stream W ----------------------------------------------------------------------
  Stats st[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) st[mb] = stats_empty();
  f32x4 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  int kf = 0, tile_j = 0;
  for (int q0 = 0; q0 < Qp; q0 += kPrefetch) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      // consume slot j, then refill it: the slot keeps its registers across iterations
      const uint4* hp = lds_h + (size_t)kf * NMB * 64 + lane;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acc[mb] = E::mma(ring[j], hp[mb * 64], acc[mb]);
      ring[j] = buffer_load16(rsrc, next_off());
      if (++kf == F) {
        kf = 0;
        if (tile_j < ntw) {
          const int v0 = (t_begin + wave + kWaves * tile_j) * kTileRows + 4 * (lane >> 4);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) stats_fold4(st[mb], acc[mb], v0, a.V);
        }
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        ++tile_j;
      }
    }
  }

  // ---- phase 3: lanes -> wavefront -> workgroup ------------------------------------------------
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    st[mb] = stats_merge(st[mb], stats_shfl_xor(st[mb], 16));
    st[mb] = stats_merge(st[mb], stats_shfl_xor(st[mb], 32));
  }
  if (lane < 16) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) red[wave * MR + mb * 16 + lane] = stats_pack(st[mb]);
  }
  __syncthreads();
  if (tid < MR) {
    Stats t = stats_unpack(red[tid]);
    for (int w = 1; w < kWaves; ++w) t = stats_merge(t, stats_unpack(red[w * MR + tid]));
    a.partials[((size_t)rg * a.G_v + gv) * MR + tid] = stats_pack(t);
    __threadfence();
  }
  __syncthreads();

  // ---- phase 4: the last workgroup merges every row and commits -------------------------------
  // Wrapping increment: the counter runs 0 .. gridDim.x-1 and the last arrival puts it back to 0,
  // so a workspace that starts zeroed is zero again between calls.
  __shared__ int s_last;
  if (tid == 0) {
    const unsigned prev = __builtin_amdgcn_atomic_inc32(a.ticket, gridDim.x - 1, __ATOMIC_ACQ_REL, "agent");
    s_last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  float* s_conf = reinterpret_cast<float*>(smem);            // reuses the hidden-state area
  int* s_tok = reinterpret_cast<int*>(smem) + kRowsPerStage;
  const CommitArgs& c = a.c;
  const bool do_commit = (c.flags & kFlagCommit) != 0;
  const int seq_per_stage = max(1, kRowsPerStage / c.L);
  const int sub = tid % kMergeLanes;
  for (int b0 = 0; b0 < c.B; b0 += seq_per_stage) {
    const int b1 = min(c.B, b0 + seq_per_stage);
    const int r_first = b0 * c.L, nrows = (b1 - b0) * c.L;
    for (int rr0 = 0; rr0 < nrows; rr0 += kThreads / kMergeLanes) {  // same trip count for all
      const int rr = rr0 + tid / kMergeLanes;
      const bool valid = rr < nrows;
      const int row = r_first + (valid ? rr : 0);
      const int g_rg = row / MR, ri = row % MR;
      const float4* src = a.partials + (size_t)g_rg * a.G_v * MR + ri;
      float4 buf[kMaxVocabGroups / kMergeLanes];
#pragma unroll
      for (int i = 0; i < kMaxVocabGroups / kMergeLanes; ++i) {
        const int g = sub + i * kMergeLanes;
        buf[i] = g < a.G_v ? src[(size_t)g * MR] : stats_pack(stats_empty());
      }
      Stats t = stats_unpack(buf[0]);
#pragma unroll
      for (int i = 1; i < kMaxVocabGroups / kMergeLanes; ++i) t = stats_merge(t, stats_unpack(buf[i]));
#pragma unroll
      for (int off = kMergeLanes / 2; off >= 1; off >>= 1) t = stats_merge(t, stats_shfl_xor(t, off));
      if (valid && sub == 0) {
        const float conf = 1.f / t.s;
        const float gap = t.m1 - t.m2;
        s_conf[rr] = conf;
        s_tok[rr] = t.id;
        if (c.out_conf) c.out_conf[row] = conf;
        if (c.out_gap) c.out_gap[row] = gap;
        if (!do_commit) c.out_tokens[row] = t.id;
      }
    }
    __syncthreads();
    if (do_commit) {
      for (int b = b0 + wave; b < b1; b += kWaves) {
        const int off = (b - b0) * c.L + lane;
        const bool in = lane < c.L;
        commit_sequence(c, b, in ? s_conf[off] : 0.f, in ? s_tok[off] : 0);
      }
    }
    __syncthreads();
  }
}

// dlm_commit: conf / tokens given, one wavefront per sequence.
__global__ __launch_bounds__(kThreads) void commit_kernel(const CommitArgs a, const float* conf, const int32_t* tok) {
  const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (b >= a.B) return;
  const int l = threadIdx.x & 63;
  const bool in = l < a.L;
  const size_t row = (size_t)b * a.L + l;
  commit_sequence(a, b, in ? conf[row] : 0.f, in ? tok[row] : 0);
}

// dlm_workspace_init: zero fill.
__global__ void fill_zero_kernel(uint8_t* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t nvec = n / 16;
  uint4* p4 = reinterpret_cast<uint4*>(p);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) p4[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = nvec * 16 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

}  // namespace dlm

// Host side of the C ABI declared in include/dlm.h: argument validation (before any HIP call),
// launch planning, workspace layout and the launches themselves.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <algorithm>
#include <mutex>

#include "dlm.h"
#include "dlm_device.hpp"

static_assert(sizeof(dlm_shard_record) == 16, "a shard record is one 16-byte statistics record");
static_assert(sizeof(dlm_seq_policy) == 20 && sizeof(dlm_policy) == 136 && sizeof(dlm_credit_slot) == 8,
              "C ABI struct layout (the Python binding mirrors it)");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DLM_OK;
}

constexpr size_t kTicketBytes = 256;     // completion counter, padded to a cache line
constexpr int kTargetWorkgroups = 256;   // one per compute unit on MI355X

// Launch geometry of one step, a pure function of the shapes (so the workspace size is too).
struct Plan {
  int gemm = 0;      // many rows: GEMM-shaped head + separate finalize kernel (256 or 512: rows per group)
  int NMB = 0;       // 16-row blocks of hidden rows per workgroup (1, 2 or 4)
  int KFWM = 0;      // K fragments per wavefront per tile, rounded up (2, 8 or 16)
  int n_rg = 0;      // row groups
  int G_v = 0;       // vocabulary ranges, multiple of 8
  int ntiles = 0;    // 16-row vocabulary tiles
  size_t lds = 0;    // dynamic LDS bytes
  size_t ws = 0;     // workspace bytes
  size_t packed_off = 0, packed_bytes = 0;  // GEMM path: fragment-ordered hidden rows in the workspace
  size_t rowout_off = 0;                    // GEMM path: published per-row conf / token / gap [B*L]
  int topk = 0;      // kernels with the top-k fold
  size_t topk_off = 0;                      // top-k records in the workspace
  size_t topk_l2_off = 0;                   // second-level top-k records [rows][nq] x 64 bytes
  int nq = 0;        // streaming kernel: groups of dlm::kGroup vocabulary ranges (two-level merge)
  size_t ticket_bytes = kTicketBytes;       // completion counters: global, then [n_rg][nq] groups
  size_t level2_off = 0;                    // second-level records [n_rg * rows][nq]
};

int elem_bytes(int32_t dtype) { return dtype == DLM_BF16 ? 2 : dtype == DLM_F32 ? 4 : 0; }

// topk > 0 selects the kernels with the top-k fold (the 512-row GEMM-shaped head beyond 64 bf16
// rows, else the streaming kernel) and appends their lists to the workspace; the caller validates
// topk's range.
// fixed_ticket_bytes > 0 places the counters in a region of that size at the start of the
// workspace whatever the shapes (the records follow it), so that calls of different shapes
// sharing one workspace never find another shape's records where their counters are.
int make_plan(int64_t B, int64_t L, int64_t H, int64_t V, int32_t dtype, int topk, Plan* p,
              size_t fixed_ticket_bytes = 0) {
  const int es = elem_bytes(dtype);
  if (!es) return fail(DLM_ERR_DTYPE, "dtype %d is neither DLM_F32 (0) nor DLM_BF16 (1)", (int)dtype);
  if (B < 1 || B > DLM_MAX_SEQS) return fail(DLM_ERR_SHAPE, "B=%lld outside [1, %d]", (long long)B, DLM_MAX_SEQS);
  if (L < 1 || L > DLM_MAX_L) return fail(DLM_ERR_SHAPE, "L=%lld outside [1, %d]", (long long)L, DLM_MAX_L);
  if (H < 32 || H % 32) return fail(DLM_ERR_SHAPE, "H=%lld must be a positive multiple of 32", (long long)H);
  if (V < 1) return fail(DLM_ERR_SHAPE, "V=%lld must be >= 1", (long long)V);
  const int64_t M = B * L;
  const int64_t ntiles = (V + dlm::kTileRows - 1) / dlm::kTileRows;
  if (ntiles > (1ll << 26)) return fail(DLM_ERR_SHAPE, "V=%lld too large", (long long)V);
  const int64_t m_pad = (M + 31) / 32 * 32;
  if (dtype == DLM_BF16 && M > 64 && H % 256 == 0 && V * H * 2 < (1ll << 31) - 64 && m_pad * H * 2 < (1ll << 31) &&
      (!topk || V < dlm::kMaxGemmTopkV)) {
    // GEMM-shaped path: 256-row vocabulary tiles against 256-row groups up to 256 rows, 128-row
    // tiles against 512-row groups beyond; workgroups per row group a multiple of 8 where
    // possible (so the groups of one tile can share an XCD).  The top-k fold exists for the
    // 512-row shape only (its chunk lists need LDS the 256-row shape's ring leaves no room for).
    const bool r512 = M > dlm::GemmR256::Rows || topk;
    const int64_t BN = r512 ? dlm::GemmR512::BN : dlm::GemmR256::BN;
    const int64_t rows = r512 ? dlm::GemmR512::Rows : dlm::GemmR256::Rows;
    const int64_t nt = (V + BN - 1) / BN;
    const int64_t n_rg = (M + rows - 1) / rows;
    int64_t G_t = kTargetWorkgroups / n_rg;
    if (G_t >= 8) G_t = G_t / 8 * 8;
    if (G_t < 1) G_t = 1;
    if (G_t > nt) G_t = nt;
    if (G_t > dlm::kMaxVocabGroups) G_t = dlm::kMaxVocabGroups;
    if (n_rg * rows * G_t * 16 >= (1ll << 31)) return fail(DLM_ERR_SHAPE, "B*L too large");
    p->gemm = (int)rows;
    p->n_rg = (int)n_rg;
    p->G_v = (int)G_t;
    p->ntiles = (int)nt;
    p->lds = 0;
    // per-sequence counters [B] (padded to 256 bytes) | records [G_t][n_rg * rows] | hidden rows
    // in fragment order, padded to 32 rows | published per-row values [B*L] x 16 bytes
    p->ticket_bytes = (size_t)((4 * B + 255) / 256 * 256);
    if (fixed_ticket_bytes) {
      if (p->ticket_bytes > fixed_ticket_bytes) return fail(DLM_ERR_SHAPE, "B=%lld: too many counters", (long long)B);
      p->ticket_bytes = fixed_ticket_bytes;
    }
    p->packed_off = p->ticket_bytes + (size_t)n_rg * rows * G_t * 16;
    p->packed_bytes = (size_t)m_pad * H * 2;
    p->rowout_off = p->packed_off + p->packed_bytes;
    p->ws = p->rowout_off + (size_t)M * 16;
    if (topk) {
      // ... | chunk lists [G_t][n_rg * rows] x DLM_MAX_TOPK x 8 bytes
      if (n_rg * rows * G_t * (DLM_MAX_TOPK * 8) >= (1ll << 31)) return fail(DLM_ERR_SHAPE, "B*L too large for top-k");
      p->topk = 1;
      p->topk_off = p->ws;
      p->ws += (size_t)n_rg * rows * G_t * (DLM_MAX_TOPK * 8);
    }
    return DLM_OK;
  }
  // each wavefront holds ceil(F / 8) hidden fragments per 16-row block in registers
  const int64_t F = H * es / 64;                        // 64-byte fragments per row
  const int64_t kfw = (F + dlm::kWaves - 1) / dlm::kWaves;
  const int KFWM = kfw <= 2 ? 2 : kfw <= 8 ? 8 : kfw <= 16 ? 16 : 0;
  if (!KFWM)
    return fail(DLM_ERR_SHAPE, "H=%lld too large: at most %d for this dtype", (long long)H, 16 * 8 * 64 / es);
  int NMB = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  if (NMB == 4 && KFWM == 16) NMB = 2;                  // register budget of the hidden fragments
  const int MR = 16 * NMB;
  const int64_t n_rg = (M + MR - 1) / MR;
  int64_t G_v = (kTargetWorkgroups / n_rg) / 8 * 8;
  if (G_v < 8) G_v = 8;
  const int64_t need = (ntiles + 7) / 8 * 8;            // no more ranges than tiles (rounded to 8)
  if (G_v > need) G_v = need;
  if (G_v > dlm::kMaxVocabGroups) G_v = dlm::kMaxVocabGroups;
  // buffer ranges are addressed with 31-bit offsets
  const int64_t range_bytes = ((ntiles + G_v - 1) / G_v) * dlm::kTileRows * H * es;
  if (range_bytes >= (1ll << 31) - 64)
    return fail(DLM_ERR_SHAPE, "V*H too large: %lld bytes of W per workgroup", (long long)range_bytes);
  if ((n_rg * MR) * H * es >= (1ll << 31) || n_rg * MR * G_v * 16 >= (1ll << 31))
    return fail(DLM_ERR_SHAPE, "B*L*H too large");
  p->NMB = NMB;
  p->KFWM = KFWM;
  p->n_rg = (int)n_rg;
  p->G_v = (int)G_v;
  p->ntiles = (int)ntiles;
  p->lds = dlm::lds_bytes(NMB);
  // counters (global + one per group, padded to 256 bytes) | records [n_rg * MR][G_v] |
  // second-level records [n_rg * MR][nq]
  const int64_t nq = (G_v + dlm::kGroup - 1) / dlm::kGroup;
  p->nq = (int)nq;
  p->ticket_bytes = (size_t)((4 * (1 + n_rg * nq) + 255) / 256 * 256);
  if (fixed_ticket_bytes) {
    if (p->ticket_bytes > fixed_ticket_bytes) return fail(DLM_ERR_SHAPE, "B*L=%lld: too many counters", (long long)M);
    p->ticket_bytes = fixed_ticket_bytes;
  }
  p->level2_off = p->ticket_bytes + (size_t)n_rg * MR * G_v * 16;
  p->ws = p->level2_off + (size_t)n_rg * MR * nq * 16;
  if (topk) {
    // ... | top-k lists [n_rg * MR][G_v] x DLM_MAX_TOPK x 8 bytes | second-level lists [n_rg * MR][nq] x 64
    if (n_rg * MR * G_v * (DLM_MAX_TOPK * 8) >= (1ll << 31)) return fail(DLM_ERR_SHAPE, "B*L too large for top-k");
    p->topk = 1;
    p->topk_off = p->ws;
    p->ws += (size_t)n_rg * MR * G_v * (DLM_MAX_TOPK * 8);
    p->topk_l2_off = p->ws;
    p->ws += (size_t)n_rg * MR * nq * (DLM_MAX_TOPK * 8);
    p->lds = dlm::lds_bytes_topk(NMB);
  }
  return DLM_OK;
}

bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Validate the per-sequence rules and pack them (distinct rules + index per sequence).
// vocab: the vocabulary size the end tokens must fall in (0: not known to this call).
int pack_rules(const dlm_policy* pol, bool need_credit_state, const void* credit, int64_t vocab, dlm::CommitArgs* c) {
  if (!pol->seq) return fail(DLM_ERR_NULL, "policy->seq is NULL");
  c->seq_done = pol->seq_done;
  int n = 0;
  bool any_credit = false;
  for (int64_t b = 0; b < pol->B; ++b) {
    const dlm_seq_policy& s = pol->seq[b];
    if (s.kind != DLM_THRESHOLD && s.kind != DLM_HIERARCHICAL && s.kind != DLM_CREDIT)
      return fail(DLM_ERR_POLICY, "seq[%lld].kind=%d is not a known policy", (long long)b, (int)s.kind);
    if (!std::isfinite(s.threshold))
      return fail(DLM_ERR_POLICY, "seq[%lld].threshold is not finite", (long long)b);
    if (s.kind == DLM_CREDIT && !(s.decay >= 0.f && s.decay < 1.f))
      return fail(DLM_ERR_POLICY, "seq[%lld].decay=%g outside [0, 1)", (long long)b, (double)s.decay);
    if (s.kind == DLM_HIERARCHICAL && s.max_depth < 0)
      return fail(DLM_ERR_POLICY, "seq[%lld].max_depth=%d is negative", (long long)b, (int)s.max_depth);
    if (s.eos_token < -1 || (vocab > 0 && s.eos_token >= vocab))
      return fail(DLM_ERR_POLICY, "seq[%lld].eos_token=%d is neither -1 nor a token id", (long long)b,
                  (int)s.eos_token);
    any_credit |= s.kind == DLM_CREDIT;
    dlm::Rule r;
    r.kind = s.kind;
    r.thr = s.threshold;
    r.decay = s.kind == DLM_CREDIT ? s.decay : 0.f;
    r.depth = s.kind == DLM_HIERARCHICAL ? s.max_depth : 0;
    r.eos = pol->seq_done ? s.eos_token : -1;
    int k = 0;
    for (; k < n; ++k)
      if (std::memcmp(&c->rules[k], &r, sizeof r) == 0) break;
    if (k == n) {
      if (n == DLM_MAX_RULES)
        return fail(DLM_ERR_POLICY, "more than %d distinct per-sequence rules in one call", DLM_MAX_RULES);
      c->rules[n++] = r;
    }
    c->rule_of[b] = (uint8_t)k;
  }
  if (need_credit_state && any_credit && !credit)
    return fail(DLM_ERR_NULL, "credit_state is NULL but a sequence uses DLM_CREDIT");
  return DLM_OK;
}

template <class T, int NMB, int KFWM, bool TK>
int launch_step(const dlm::StepArgs& a, const Plan& p, hipStream_t stream) {
  hipLaunchKernelGGL((dlm::step_kernel<T, NMB, KFWM, TK>), dim3(p.n_rg * p.G_v), dim3(dlm::kThreads), p.lds, stream,
                     a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DLM_ERR_HIP, "step kernel launch: %s", hipGetErrorString(e));
  return ok();
}

template <class T, bool TK>
int launch_step_for(const dlm::StepArgs& a, const Plan& p, hipStream_t stream) {
  switch (p.NMB * 100 + p.KFWM) {
    case 102: return launch_step<T, 1, 2, TK>(a, p, stream);
    case 108: return launch_step<T, 1, 8, TK>(a, p, stream);
    case 116: return launch_step<T, 1, 16, TK>(a, p, stream);
    case 202: return launch_step<T, 2, 2, TK>(a, p, stream);
    case 208: return launch_step<T, 2, 8, TK>(a, p, stream);
    case 216: return launch_step<T, 2, 16, TK>(a, p, stream);
    case 402: return launch_step<T, 4, 2, TK>(a, p, stream);
    case 408: return launch_step<T, 4, 8, TK>(a, p, stream);
    default: return fail(DLM_ERR_SHAPE, "no kernel for NMB=%d KFWM=%d", p.NMB, p.KFWM);
  }
}

// Top-k fields of the policy: range and output pointer (before any launch).
int check_topk(const dlm_policy* pol, dlm::CommitArgs* c) {
  if (pol->topk < 0 || pol->topk > DLM_MAX_TOPK)
    return fail(DLM_ERR_POLICY, "topk=%d outside [0, %d]", (int)pol->topk, DLM_MAX_TOPK);
  if (pol->topk > 0 && !pol->out_topk_tokens) return fail(DLM_ERR_NULL, "topk > 0 but out_topk_tokens is NULL");
  c->topk = pol->topk;
  c->out_topk_tokens = pol->topk > 0 ? pol->out_topk_tokens : nullptr;
  c->out_topk_prob = pol->topk > 0 ? pol->out_topk_prob : nullptr;
  return DLM_OK;
}

// Records policy->head_events[i] (if set) on the stream: i = 0 before the kernel that streams W,
// i = 1 after it.  Only for calls that time the head (time_head).
int head_event(const dlm_policy* pol, bool time_head, int i, hipStream_t stream) {
  if (!time_head || !pol->head_events[i]) return DLM_OK;
  const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(pol->head_events[i]), stream);
  if (e != hipSuccess) return fail(DLM_ERR_HIP, "head_events[%d] record: %s", i, hipGetErrorString(e));
  return DLM_OK;
}

// next_hidden (GEMM path without top-k, several steps per call): the finalizer launch also packs
// the next step's hidden rows; prepacked: this step's were packed that way, so no pack launch.
int run_step(const void* hidden, const void* W, const dlm_policy* pol, dlm::CommitArgs c, bool commit,
             bool time_head, size_t fixed_ticket_bytes = 0, const void* next_hidden = nullptr, bool prepacked = false) {
  Plan p;
  int rc = make_plan(pol->B, pol->L, pol->H, pol->V, pol->dtype, c.topk, &p, fixed_ticket_bytes);
  if (rc) return rc;
  if (!pol->workspace) return fail(DLM_ERR_NULL, "policy->workspace is NULL");
  if (pol->workspace_bytes < p.ws)
    return fail(DLM_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", pol->workspace_bytes, p.ws);
  if (misaligned(hidden, 16) || misaligned(W, 16) || misaligned(pol->workspace, 256))
    return fail(DLM_ERR_SHAPE, "hidden and W_vocab must be 16-byte aligned, the workspace 256-byte aligned");
  dlm::StepArgs a;
  a.hidden = hidden;
  a.W = W;
  a.ticket = static_cast<unsigned*>(pol->workspace);
  a.group_tickets = a.ticket + 1;
  a.partials = reinterpret_cast<float4*>(static_cast<char*>(pol->workspace) + p.ticket_bytes);
  a.level2 = reinterpret_cast<float4*>(static_cast<char*>(pol->workspace) + p.level2_off);
  a.nq = p.nq;
  a.H = (int)pol->H;
  a.V = (int)pol->V;
  a.M = (int)(pol->B * pol->L);
  a.n_rg = p.n_rg;
  a.G_v = p.G_v;
  a.ntiles = p.ntiles;
  a.topk_records = p.topk ? reinterpret_cast<float4*>(static_cast<char*>(pol->workspace) + p.topk_off) : nullptr;
  a.topk_level2 = p.topk ? reinterpret_cast<float4*>(static_cast<char*>(pol->workspace) + p.topk_l2_off) : nullptr;
  c.B = (int)pol->B;
  c.L = (int)pol->L;
  c.flags = (commit ? dlm::kFlagCommit : 0u) | (commit ? (pol->flags & DLM_AUTO_ADVANCE) : 0u);
  a.c = c;
  hipStream_t stream = static_cast<hipStream_t>(pol->stream);
  if (p.gemm) {
    void* packed = static_cast<char*>(pol->workspace) + p.packed_off;
    const int pack_waves = (a.M + 31) / 32 * (a.H / 64);   // (H % 256 == 0 on this path)
    hipError_t e = hipSuccess;
    if (!prepacked) {
      hipLaunchKernelGGL(dlm::pack_hidden_kernel, dim3((pack_waves + 3) / 4), dim3(256), 0, stream,
                         static_cast<const uint4*>(hidden), static_cast<uint4*>(packed), a.M, a.H);
      e = hipGetLastError();
      if (e != hipSuccess) return fail(DLM_ERR_HIP, "pack kernel launch: %s", hipGetErrorString(e));
    }
    dlm::GemmArgs g;
    g.hidden_packed = packed;
    g.packed_bytes = (unsigned)p.packed_bytes;
    g.fold_gate = 0xffffffffu;
    g.W = W;
    g.records = a.partials;
    g.H = a.H;
    g.V = a.V;
    g.M = a.M;
    g.n_rg = p.n_rg;
    g.G_t = p.G_v;
    g.ntiles = p.ntiles;
    g.topk_records = p.topk ? reinterpret_cast<uint4*>(static_cast<char*>(pol->workspace) + p.topk_off) : nullptr;
    g.id_bits = 1;
    while ((1ll << g.id_bits) <= (long long)a.V) ++g.id_bits;   // bit length of V: all ones is no token
    const bool r512 = p.gemm == dlm::GemmR512::Rows;
    const dim3 grid(p.n_rg * p.G_v), block(r512 ? dlm::GemmR512::Threads : dlm::GemmR256::Threads);
    const int rows = p.gemm;
    const bool tail = a.V % (r512 ? dlm::GemmR512::BN : dlm::GemmR256::BN) != 0;
    if ((rc = head_event(pol, time_head, 0, stream))) return rc;
    if (p.topk)
      hipLaunchKernelGGL(tail ? dlm::gemm_r512_topk_tail_kernel : dlm::gemm_r512_topk_kernel, grid, block, 0, stream, g);
    else if (r512)
      hipLaunchKernelGGL(tail ? dlm::gemm_r512_tail_kernel : dlm::gemm_r512_kernel, grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL(tail ? dlm::gemm_r256_tail_kernel : dlm::gemm_r256_kernel, grid, block, 0, stream, g);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(DLM_ERR_HIP, "gemm kernel launch: %s", hipGetErrorString(e));
    if ((rc = head_event(pol, time_head, 1, stream))) return rc;
    const int fin_rows = p.topk ? dlm::kFinRowsTopk : dlm::kFinRows;
    const int parts = (c.L + fin_rows - 1) / fin_rows;
    dlm::GemmTopkArgs tka;
    tka.lists = g.topk_records;
    tka.W = W;
    tka.hidden = hidden;
    tka.H = a.H;
    tka.V = a.V;
    tka.id_bits = g.id_bits;
    float4* const row_out = reinterpret_cast<float4*>(static_cast<char*>(pol->workspace) + p.rowout_off);
    dlm::PackArgs pk;                                     // the next step's pack, if any, after the parts
    pk.h = static_cast<const uint4*>(next_hidden);
    pk.hp = static_cast<uint4*>(packed);
    pk.M = a.M;
    pk.H = a.H;
    pk.first_block = c.B * parts;
    const int pack_blocks = next_hidden && !p.topk ? (pack_waves + 1) / 2 : 0;
    if (p.topk)
      hipLaunchKernelGGL(dlm::finalize_parts_kernel<true>, dim3(c.B * parts), dim3(64 * dlm::kFinRowsTopk), 0, stream,
                         a.c, a.partials, p.G_v, p.n_rg * rows, a.ticket, row_out, tka, pk);
    else
      hipLaunchKernelGGL(dlm::finalize_parts_kernel<false>, dim3(c.B * parts + pack_blocks), dim3(128), 0, stream,
                         a.c, a.partials, p.G_v, p.n_rg * rows, a.ticket, row_out, tka, pk);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(DLM_ERR_HIP, "finalize kernel launch: %s", hipGetErrorString(e));
    return ok();
  }
  if ((rc = head_event(pol, time_head, 0, stream))) return rc;
  if (p.topk)
    rc = pol->dtype == DLM_BF16 ? launch_step_for<uint16_t, true>(a, p, stream) : launch_step_for<float, true>(a, p, stream);
  else
    rc = pol->dtype == DLM_BF16 ? launch_step_for<uint16_t, false>(a, p, stream) : launch_step_for<float, false>(a, p, stream);
  if (rc) return rc;
  return head_event(pol, time_head, 1, stream);
}

// ---- the workspace of dlm_decode_step_noalloc --------------------------------------------------
// One static array per GPU the library runs on (each device holds its own copy of it until the
// process ends).  In host code `scratch` names a host-side stand-in, not the device memory: host
// code uses only the per-device address that hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = DLM_NOALLOC_SCRATCH_BYTES;
// Counter region at the start of the array, large enough for every shape that fits the array
// (at most 4 * (1 + 1024) bytes on the streaming path, 4 * DLM_MAX_SEQS on the GEMM-shaped one).
constexpr size_t kScratchTicketBytes = 8192;

}  // namespace

static __device__ __align__(256) uint8_t scratch[DLM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch`.  On the first call on a device: its address, then a fill
// kernel on `stream` that zeroes the counter region (the counters must start at zero; every call
// leaves them at zero again).  The records and staging areas need no clearing.
int scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DLM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DLM_ERR_HIP, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(DLM_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int blocks = (int)((kScratchTicketBytes / 16 + 255) / 256);
    hipLaunchKernelGGL(dlm::fill_zero_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint8_t*>(ptr),
                       kScratchTicketBytes, blocks * 256);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(DLM_ERR_HIP, "scratch counter clear: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DLM_OK;
}

}  // namespace

extern "C" {

int dlm_decode_step(const void* hidden, const void* W_vocab, uint8_t* mask_state, dlm_credit_slot* credit_state,
                    const dlm_policy* policy, int32_t* out_tokens, uint8_t* out_commit) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!hidden || !W_vocab || !mask_state || !out_tokens || !out_commit)
    return fail(DLM_ERR_NULL, "hidden, W_vocab, mask_state, out_tokens and out_commit must be non-NULL");
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  int rc = check_topk(policy, &c);
  if (rc) return rc;
  Plan p;
  rc = make_plan(policy->B, policy->L, policy->H, policy->V, policy->dtype, c.topk, &p);
  if (rc) return rc;
  rc = pack_rules(policy, true, credit_state, policy->V, &c);
  if (rc) return rc;
  c.mask = mask_state;
  c.credit = credit_state;
  c.out_tokens = out_tokens;
  c.out_commit = out_commit;
  c.out_conf = policy->out_conf;
  c.out_gap = policy->out_gap;
  return run_step(hidden, W_vocab, policy, c, true, true);
}

int dlm_decode_step_noalloc(const void* hidden, const void* W_vocab, uint8_t* mask_state,
                            dlm_credit_slot* credit_state, const dlm_policy* policy, int32_t* out_tokens,
                            uint8_t* out_commit) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!hidden || !W_vocab || !mask_state || !out_tokens || !out_commit)
    return fail(DLM_ERR_NULL, "hidden, W_vocab, mask_state, out_tokens and out_commit must be non-NULL");
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  int rc = check_topk(policy, &c);
  if (rc) return rc;
  Plan p;
  rc = make_plan(policy->B, policy->L, policy->H, policy->V, policy->dtype, c.topk, &p, kScratchTicketBytes);
  if (rc) return rc;
  if (p.ws > kScratchBytes)
    return fail(DLM_ERR_WORKSPACE, "these shapes need %zu bytes of workspace; the static scratch of "
                "dlm_decode_step_noalloc holds %zu (DLM_NOALLOC_SCRATCH_BYTES): use dlm_decode_step", p.ws,
                kScratchBytes);
  rc = pack_rules(policy, true, credit_state, policy->V, &c);
  if (rc) return rc;
  if (misaligned(hidden, 16) || misaligned(W_vocab, 16))   // (before the first call's clear is enqueued)
    return fail(DLM_ERR_SHAPE, "hidden and W_vocab must be 16-byte aligned");
  c.mask = mask_state;
  c.credit = credit_state;
  c.out_tokens = out_tokens;
  c.out_commit = out_commit;
  c.out_conf = policy->out_conf;
  c.out_gap = policy->out_gap;
  void* ws = nullptr;
  rc = scratch_of_current_device(static_cast<hipStream_t>(policy->stream), &ws);
  if (rc) return rc;
  dlm_policy pol = *policy;
  pol.workspace = ws;
  pol.workspace_bytes = kScratchBytes;
  return run_step(hidden, W_vocab, &pol, c, true, true, kScratchTicketBytes);
}

int dlm_decode_steps(const void* hidden_steps, const void* W_vocab, uint8_t* mask_state,
                     dlm_credit_slot* credit_state, const dlm_policy* policy, int64_t n_steps,
                     int32_t* out_tokens_steps, uint8_t* out_commit_steps) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!hidden_steps || !W_vocab || !mask_state || !out_tokens_steps || !out_commit_steps)
    return fail(DLM_ERR_NULL, "hidden_steps, W_vocab, mask_state, out_tokens_steps and out_commit_steps must be non-NULL");
  if (n_steps < 1) return fail(DLM_ERR_SHAPE, "n_steps=%lld must be >= 1", (long long)n_steps);
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  int rc = check_topk(policy, &c);
  if (rc) return rc;
  Plan p;
  rc = make_plan(policy->B, policy->L, policy->H, policy->V, policy->dtype, c.topk, &p);
  if (rc) return rc;
  rc = pack_rules(policy, true, credit_state, policy->V, &c);
  if (rc) return rc;
  const size_t rows = (size_t)(policy->B * policy->L);
  const size_t step_bytes = rows * (size_t)policy->H * (size_t)elem_bytes(policy->dtype);
  if (misaligned(hidden_steps, 16) || step_bytes % 16)
    return fail(DLM_ERR_SHAPE, "hidden_steps must be 16-byte aligned (and so every step's slice)");
  c.mask = mask_state;
  c.credit = credit_state;
  c.out_conf = policy->out_conf;
  c.out_gap = policy->out_gap;
  int32_t* const topk_tokens0 = c.out_topk_tokens;
  float* const topk_prob0 = c.out_topk_prob;
  // on the GEMM path without top-k, each step's finalizer also packs the next step's hidden rows
  const bool chain_pack = p.gemm && !p.topk;
  const char* const h0 = static_cast<const char*>(hidden_steps);
  for (int64_t n = 0; n < n_steps; ++n) {
    c.out_tokens = out_tokens_steps + n * rows;
    c.out_commit = out_commit_steps + n * rows;
    if (c.topk) {
      c.out_topk_tokens = topk_tokens0 + (size_t)n * rows * c.topk;
      c.out_topk_prob = topk_prob0 ? topk_prob0 + (size_t)n * rows * c.topk : nullptr;
    }
    const void* next = chain_pack && n + 1 < n_steps ? h0 + (n + 1) * step_bytes : nullptr;
    rc = run_step(h0 + n * step_bytes, W_vocab, policy, c, true, false, 0, next, chain_pack && n > 0);
    if (rc) return rc;  // only a failed launch can get here, after validation passed
  }
  return ok();
}

int dlm_token_stats(const void* hidden, const void* W_vocab, const dlm_policy* policy, float* out_conf,
                    int32_t* out_tokens, float* out_gap) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!hidden || !W_vocab || !out_conf || !out_tokens)
    return fail(DLM_ERR_NULL, "hidden, W_vocab, out_conf and out_tokens must be non-NULL");
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  const int rc = check_topk(policy, &c);
  if (rc) return rc;
  c.out_tokens = out_tokens;
  c.out_conf = out_conf;
  c.out_gap = out_gap;
  return run_step(hidden, W_vocab, policy, c, false, true);
}

int dlm_shard_stats(const void* hidden, const void* W_shard, int64_t v_begin, const dlm_policy* policy,
                    dlm_shard_record* out_records) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!hidden || !W_shard || !out_records)
    return fail(DLM_ERR_NULL, "hidden, W_shard and out_records must be non-NULL");
  if (policy->topk != 0) return fail(DLM_ERR_POLICY, "topk=%d: the shard call has no top-k export", (int)policy->topk);
  if (v_begin < 0 || v_begin + policy->V > 0x7fffffffll)
    return fail(DLM_ERR_SHAPE, "v_begin=%lld: the shard's tokens must lie in [0, 2^31 - 1)", (long long)v_begin);
  if (misaligned(out_records, 16)) return fail(DLM_ERR_SHAPE, "out_records must be 16-byte aligned");
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  c.out_records = reinterpret_cast<float4*>(out_records);
  c.v_begin = (int)v_begin;
  return run_step(hidden, W_shard, policy, c, false, false);
}

int dlm_merge_commit(const dlm_shard_record* records, int64_t n_shards, uint8_t* mask_state,
                     dlm_credit_slot* credit_state, const dlm_policy* policy, int32_t* out_tokens,
                     uint8_t* out_commit) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!records || !mask_state || !out_tokens || !out_commit)
    return fail(DLM_ERR_NULL, "records, mask_state, out_tokens and out_commit must be non-NULL");
  if (policy->B < 1 || policy->B > DLM_MAX_SEQS)
    return fail(DLM_ERR_SHAPE, "B=%lld outside [1, %d]", (long long)policy->B, DLM_MAX_SEQS);
  if (policy->L < 1 || policy->L > DLM_MAX_L)
    return fail(DLM_ERR_SHAPE, "L=%lld outside [1, %d]", (long long)policy->L, DLM_MAX_L);
  if (policy->V < 1) return fail(DLM_ERR_SHAPE, "V=%lld must be >= 1 (the full vocabulary)", (long long)policy->V);
  if (n_shards < 1 || n_shards > DLM_MAX_SHARDS)
    return fail(DLM_ERR_SHAPE, "n_shards=%lld outside [1, %d]", (long long)n_shards, DLM_MAX_SHARDS);
  if (misaligned(records, 16)) return fail(DLM_ERR_SHAPE, "records must be 16-byte aligned");
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  int rc = pack_rules(policy, true, credit_state, policy->V, &c);
  if (rc) return rc;
  c.mask = mask_state;
  c.credit = credit_state;
  c.out_tokens = out_tokens;
  c.out_commit = out_commit;
  c.out_conf = policy->out_conf;
  c.out_gap = policy->out_gap;
  c.B = (int)policy->B;
  c.L = (int)policy->L;
  c.flags = dlm::kFlagCommit | (policy->flags & DLM_AUTO_ADVANCE);
  hipLaunchKernelGGL(dlm::merge_commit_kernel, dim3(c.B), dim3(dlm::kThreads), 0, static_cast<hipStream_t>(policy->stream),
                     c, reinterpret_cast<const float4*>(records), (int)n_shards);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DLM_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int dlm_commit(const float* conf, const int32_t* tokens, uint8_t* mask_state, dlm_credit_slot* credit_state,
               const dlm_policy* policy, uint8_t* out_commit) {
  if (!policy) return fail(DLM_ERR_NULL, "policy is NULL");
  if (!conf || !tokens || !mask_state || !out_commit)
    return fail(DLM_ERR_NULL, "conf, tokens, mask_state and out_commit must be non-NULL");
  if (policy->B < 1 || policy->B > DLM_MAX_SEQS)
    return fail(DLM_ERR_SHAPE, "B=%lld outside [1, %d]", (long long)policy->B, DLM_MAX_SEQS);
  if (policy->L < 1 || policy->L > DLM_MAX_L)
    return fail(DLM_ERR_SHAPE, "L=%lld outside [1, %d]", (long long)policy->L, DLM_MAX_L);
  dlm::CommitArgs c;
  std::memset(&c, 0, sizeof c);
  int rc = pack_rules(policy, true, credit_state, 0, &c);
  if (rc) return rc;
  c.mask = mask_state;
  c.credit = credit_state;
  c.out_tokens = nullptr;  // the candidates are the caller's input here
  c.out_commit = out_commit;
  c.B = (int)policy->B;
  c.L = (int)policy->L;
  c.flags = policy->flags & DLM_AUTO_ADVANCE;
  const int grid = (c.B + dlm::kWaves - 1) / dlm::kWaves;
  hipLaunchKernelGGL(dlm::commit_kernel, dim3(grid), dim3(dlm::kThreads), 0, static_cast<hipStream_t>(policy->stream),
                     c, conf, tokens);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DLM_ERR_HIP, "commit kernel launch: %s", hipGetErrorString(e));
  return ok();
}

size_t dlm_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t V, int32_t dtype) {
  return dlm_workspace_bytes_topk(B, L, H, V, dtype, 0);
}

size_t dlm_workspace_bytes_topk(int64_t B, int64_t L, int64_t H, int64_t V, int32_t dtype, int32_t topk) {
  if (topk < 0 || topk > DLM_MAX_TOPK) return 0;
  Plan p;
  const std::string saved = g_last_error;
  const int rc = make_plan(B, L, H, V, dtype, topk, &p);
  g_last_error = saved;
  return rc ? 0 : p.ws;
}

int dlm_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(DLM_ERR_NULL, "workspace is NULL");
  if (workspace_bytes == 0) return ok();
  const size_t blocks = std::min<size_t>(1024, (workspace_bytes + 16 * 256 - 1) / (16 * 256));
  hipLaunchKernelGGL(dlm::fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint8_t*>(workspace), workspace_bytes, (int)blocks * 256);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DLM_ERR_HIP, "fill kernel launch: %s", hipGetErrorString(e));
  return ok();
}

const char* dlm_last_error(void) { return g_last_error.c_str(); }

const char* dlm_version(void) { return DLM_VERSION_STRING; }

}  // extern "C"

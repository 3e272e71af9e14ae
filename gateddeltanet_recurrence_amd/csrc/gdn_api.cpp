// C ABI of libgdn.so: argument validation, plan resolution and dispatch.
//
// Every check runs on the host before any launch, so an error status other
// than GDN_ERR_HIP leaves device memory untouched (validation and preparation
// before the publication boundary: "Replay compact fixed state for hybrid
// decoding", Key Changes). The library allocates nothing and keeps no state.
#include "../../include/gdn.h"
#include "../../include/gdn_conv.h"
#include "../../include/gdn_pool.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <utility>
#include <vector>

#include "gdn_kernels.h"

namespace {

constexpr int kRecurrentMaxLenForAuto = 32;

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t io_bytes(int dtype) { return dtype == GDN_F16 ? 2 : 4; }

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
  Span() = default;
  Span(const void* p, size_t bytes) : lo(reinterpret_cast<uintptr_t>(p)), hi(lo + (p ? bytes : 0)) {}
  bool empty() const { return lo == hi; }
  bool overlaps(const Span& o) const { return !empty() && !o.empty() && lo < o.hi && o.lo < hi; }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every forward entry point; fills the resolved values.
struct Resolved {
  int64_t N, R, Hk, Hv, Dk, Dv;
  int cap;
  float scale;
  int plan;
  int64_t chunk_slots;  // chunk slots the CHUNK workspace holds
};

int check_params(const gdn_params* p, Resolved* out) {
  if (p == nullptr) return GDN_ERR_NULL;
  if (p->update_rule != GDN_RULE_GATED_DELTA && p->update_rule != GDN_RULE_DELTA &&
      p->update_rule != GDN_RULE_GATED && p->update_rule != GDN_RULE_LINEAR)
    return GDN_ERR_RULE;
  if (p->gate_activation != GDN_GATE_RAW && p->gate_activation != GDN_GATE_NONE) return GDN_ERR_RULE;
  if (p->state_layout != GDN_STATE_V_MAJOR && p->state_layout != GDN_STATE_K_MAJOR) return GDN_ERR_SHAPE;
  if (p->io_dtype != GDN_F32 && p->io_dtype != GDN_F16) return GDN_ERR_DTYPE;
  if (p->num_tokens < 0 || p->num_reqs < 0 || p->num_k_heads <= 0 || p->num_v_heads <= 0)
    return GDN_ERR_SHAPE;
  if (p->num_v_heads % p->num_k_heads != 0) return GDN_ERR_SHAPE;
  if (!supported_dim(p->head_k_dim) || !supported_dim(p->head_v_dim)) return GDN_ERR_SHAPE;
  if (std::isnan(p->scale) || std::isinf(p->scale)) return GDN_ERR_SHAPE;
  if (p->state_update_capacity < 0) return GDN_ERR_CAPACITY;
  if (p->chunk != 0 && p->chunk != gdn::kChunk) return GDN_ERR_SHAPE;
  if (p->plan != GDN_PLAN_AUTO && p->plan != GDN_PLAN_RECURRENT && p->plan != GDN_PLAN_CHUNK)
    return GDN_ERR_PLAN;
  out->N = p->num_tokens;
  out->R = p->num_reqs;
  out->Hk = p->num_k_heads;
  out->Hv = p->num_v_heads;
  out->Dk = p->head_k_dim;
  out->Dv = p->head_v_dim;
  out->cap = p->state_update_capacity;
  out->scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt(static_cast<float>(p->head_k_dim));
  // capsule rows of one request must be addressable with 32-bit row offsets in-kernel
  const int64_t W = out->Hv + out->Hk * out->Dk + out->Hv * out->Dv;
  if (W > std::numeric_limits<int32_t>::max()) return GDN_ERR_SHAPE;
  return GDN_OK;
}

int check_cu_host(const int32_t* cu, int64_t R, int64_t N, int64_t* max_len, int64_t* slots) {
  if (cu[0] != 0) return GDN_ERR_SHAPE;
  int64_t mx = 0, nch = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t len = static_cast<int64_t>(cu[r + 1]) - cu[r];
    if (len < 0) return GDN_ERR_SHAPE;
    if (len > mx) mx = len;
    nch += (len + gdn::kChunk - 1) / gdn::kChunk;
  }
  if (cu[R] != N) return GDN_ERR_SHAPE;
  *max_len = mx;
  *slots = nch;
  return GDN_OK;
}

// Resolves the plan and the chunk-slot count. `capsule` says a capsule is written;
// `dense` says every request holds N / R tokens (no cu_seqlens).
int resolve_plan(const gdn_params* p, const int32_t* cu_host, bool capsule, Resolved* rv,
                 bool dense = false) {
  int64_t max_len = 0, slots = 0;
  if (dense) {
    max_len = rv->R > 0 ? rv->N / rv->R : 0;
    slots = rv->R * ((max_len + gdn::kChunk - 1) / gdn::kChunk);
  } else if (cu_host != nullptr) {
    int st = check_cu_host(cu_host, rv->R, rv->N, &max_len, &slots);
    if (st != GDN_OK) return st;
  } else {
    // upper bound valid for any split of N tokens into R requests
    max_len = rv->R > 0 ? (rv->N + rv->R - 1) / rv->R : 0;  // mean, for planning only
    slots = rv->R > 0 ? (rv->N + rv->R * (gdn::kChunk - 1)) / gdn::kChunk : 0;
  }
  // the MFMA chunk path takes fp16 operands: it serves fp16 I/O at Dk = Dv = 128
  const bool chunk_shape = rv->Dk == 128 && rv->Dv == 128 && p->io_dtype == GDN_F16;
  int plan = p->plan;
  if (plan == GDN_PLAN_CHUNK) {
    if (capsule || !chunk_shape) return GDN_ERR_PLAN;
  } else if (plan == GDN_PLAN_AUTO) {
    plan = (capsule || !chunk_shape || max_len <= kRecurrentMaxLenForAuto) ? GDN_PLAN_RECURRENT
                                                                            : GDN_PLAN_CHUNK;
  }
  rv->plan = plan;
  rv->chunk_slots = slots;
  return GDN_OK;
}

bool conv_shape_ok(int64_t C, int64_t K) { return C >= 4 && C % 4 == 0 && K >= 2 && K <= 8; }

// Tokens one convolution workgroup walks: enough workgroups to fill the chip
// several times over, and at most 64 tokens so the K - 1 re-read inputs at each
// workgroup's start stay a small fraction of the traffic.
int conv_tokens_per_block(int64_t N, int64_t C) {
  const int64_t tb = (N * gdn::conv_channel_groups(C) + 8191) / 8192;
  return (int)(tb < 1 ? 1 : tb > 64 ? 64 : tb);
}

// Slots of one call: P = 0 for states indexed by request.
struct SlotPlan {
  int64_t P = 0;
  const int32_t* rd = nullptr;
  const int32_t* wr = nullptr;
};

// Validates a slot description for R requests (gdn_pool.h, slot rules).
// `same_pool`: the read and write pools are one buffer. Collisions are checked
// where the host knows the slots (a mirror, or the identity of a NULL array).
int plan_slots(const gdn_slots* s, int64_t R, bool same_pool, SlotPlan* out) {
  *out = SlotPlan{};
  if (s == nullptr) return GDN_OK;
  const int64_t P = s->num_slots;
  if (P < 1) return GDN_ERR_SHAPE;
  if ((s->read_slots == nullptr && s->read_slots_host != nullptr) ||
      (s->write_slots == nullptr && s->write_slots_host != nullptr))
    return GDN_ERR_SHAPE;
  if ((s->read_slots == nullptr || s->write_slots == nullptr) && R > P) return GDN_ERR_SHAPE;
  const bool rd_known = s->read_slots == nullptr || s->read_slots_host != nullptr;
  const bool wr_known = s->write_slots == nullptr || s->write_slots_host != nullptr;
  auto rd = [&](int64_t r) -> int64_t { return s->read_slots == nullptr ? r : s->read_slots_host[r]; };
  auto wr = [&](int64_t r) -> int64_t { return s->write_slots == nullptr ? r : s->write_slots_host[r]; };
  for (int64_t r = 0; r < R; ++r) {
    if (rd_known && (rd(r) < -1 || rd(r) >= P)) return GDN_ERR_SHAPE;
    if (wr_known && (wr(r) < -1 || wr(r) >= P)) return GDN_ERR_SHAPE;
  }
  if (wr_known) {
    // (slot, request) of every write, sorted: equal neighbours are a double write
    std::vector<std::pair<int64_t, int64_t>> writes;
    writes.reserve((size_t)R);
    for (int64_t r = 0; r < R; ++r)
      if (wr(r) >= 0) writes.emplace_back(wr(r), r);
    std::sort(writes.begin(), writes.end());
    for (size_t i = 1; i < writes.size(); ++i)
      if (writes[i].first == writes[i - 1].first) return GDN_ERR_ALIAS;
    if (same_pool && rd_known) {
      // a slot written by one request and read by another
      std::vector<std::pair<int64_t, int64_t>> reads;
      reads.reserve((size_t)R);
      for (int64_t r = 0; r < R; ++r)
        if (rd(r) >= 0) reads.emplace_back(rd(r), r);
      std::sort(reads.begin(), reads.end());
      for (const auto& w : writes) {
        auto it = std::lower_bound(reads.begin(), reads.end(), std::make_pair(w.first, int64_t{-1}));
        for (; it != reads.end() && it->first == w.first; ++it)
          if (it->second != w.second) return GDN_ERR_ALIAS;
      }
    }
  }
  out->P = P;
  out->rd = s->read_slots;
  out->wr = s->write_slots;
  return GDN_OK;
}

size_t workspace_for(const Resolved& rv) {
  if (rv.plan != GDN_PLAN_CHUNK) return 0;
  return gdn::chunk_workspace_bytes(rv.chunk_slots, (int)rv.R, (int)rv.Hk, (int)rv.Hv);
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_strerror(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "unsupported size, malformed cu_seqlens or misaligned pointer";
    case GDN_ERR_DTYPE: return "io dtype must be FP16 or FP32 (BF16 is not supported)";
    case GDN_ERR_ALIAS: return "buffers overlap in a way the call does not allow";
    case GDN_ERR_CAPACITY: return "capacity is negative or an accepted/captured count exceeds it";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_PLAN: return "the forced plan cannot run these arguments";
    case GDN_ERR_RULE: return "unknown update rule (gdn_rule) or gate activation";
    case GDN_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case GDN_ERR_SCRATCH:
      return "the call needs more scratch than the static array of gdn_forward_no_alloc holds "
             "(GDN_NO_ALLOC_SCRATCH_BYTES); use gdn_forward with a workspace";
    default: return "unknown status";
  }
}

int gdn_resolve_plan(const gdn_params* p, const int32_t* cu_host, int32_t* plan) {
  Resolved rv;
  int st = check_params(p, &rv);
  if (st != GDN_OK) return st;
  if (plan == nullptr) return GDN_ERR_NULL;
  st = resolve_plan(p, cu_host, rv.cap > 0, &rv);
  if (st != GDN_OK) return st;
  *plan = rv.plan;
  return GDN_OK;
}

int gdn_forward_workspace_bytes(const gdn_params* p, const int32_t* cu_host, size_t* bytes) {
  Resolved rv;
  int st = check_params(p, &rv);
  if (st != GDN_OK) return st;
  if (bytes == nullptr) return GDN_ERR_NULL;
  st = resolve_plan(p, cu_host, rv.cap > 0, &rv);
  if (st != GDN_OK) return st;
  *bytes = workspace_for(rv);
  return GDN_OK;
}

// The previous step's capsule, accepted counts and inactive bank of gdn_replay_forward.
struct FusedReplay {
  const float* capsule;
  const int32_t* accepted;
  const int32_t* accepted_host;
  float* state;
};

static int forward_impl(const gdn_params* p, const gdn_tensors* t, const gdn_slots* slots,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const FusedReplay* rp = nullptr, const gdn_conv_fused* cv = nullptr) {
  Resolved rv;
  int st = check_params(p, &rv);
  if (st != GDN_OK) return st;
  if (t == nullptr) return GDN_ERR_NULL;
  const bool capsule = t->state_update != nullptr;
  if (capsule && rv.cap == 0) return GDN_ERR_CAPACITY;   // a capsule needs rows
  if (cv != nullptr) {
    // the fused convolution: q, k, v come from it; V-major decode, no capsule
    if (cv->activation != GDN_CONV_SILU && cv->activation != GDN_CONV_NONE) return GDN_ERR_RULE;
    if (cv->kernel_size != gdn::kConvFusedK) return GDN_ERR_SHAPE;
    if (t->q != nullptr || t->k != nullptr || t->v != nullptr) return GDN_ERR_SHAPE;
    if (capsule || p->state_layout != GDN_STATE_V_MAJOR) return GDN_ERR_SHAPE;
    if (p->plan == GDN_PLAN_CHUNK) return GDN_ERR_PLAN;
  }
  if (rp != nullptr) {
    // the fused step: a verify (capsule) from the replayed committed V-major bank
    if (!capsule || t->initial_state == nullptr || rp->capsule == nullptr || rp->accepted == nullptr ||
        rp->state == nullptr)
      return GDN_ERR_NULL;
    if (p->state_layout != GDN_STATE_V_MAJOR) return GDN_ERR_SHAPE;
    if (!aligned16(rp->state)) return GDN_ERR_SHAPE;
    // with pools the write slots address the replayed state; no final state then
    if (slots != nullptr && t->final_state != nullptr) return GDN_ERR_SHAPE;
    if (rp->accepted_host != nullptr)
      for (int64_t r = 0; r < rv.R; ++r)
        if (rp->accepted_host[r] < 0 || rp->accepted_host[r] > rv.cap) return GDN_ERR_CAPACITY;
  }
  if (rv.R == 0) return rv.N == 0 ? GDN_OK : GDN_ERR_SHAPE;

  // required pointers; without cu_seqlens every request holds N / R tokens (dense
  // rank-4 layout), and the effective gates need no A_log, dt_bias
  const bool dense = t->cu_seqlens == nullptr;
  if (dense && (t->cu_seqlens_host != nullptr || rv.N % rv.R != 0)) return GDN_ERR_SHAPE;
  const bool gate_none = p->gate_activation == GDN_GATE_NONE;
  // the decay input is read by the gated rules, beta by the rules with the delta correction
  const bool gated = p->update_rule == GDN_RULE_GATED_DELTA || p->update_rule == GDN_RULE_GATED;
  const bool delta = p->update_rule == GDN_RULE_GATED_DELTA || p->update_rule == GDN_RULE_DELTA;
  if (gated && !gate_none && (t->A_log == nullptr || t->dt_bias == nullptr)) return GDN_ERR_NULL;
  const bool qkv_given = cv == nullptr;
  if (rv.N > 0 && ((qkv_given && (t->q == nullptr || t->k == nullptr || t->v == nullptr)) ||
                   (gated && t->a == nullptr) || (delta && t->b == nullptr) || t->output == nullptr))
    return GDN_ERR_NULL;
  if (cv != nullptr && rv.N > 0 && (cv->mixed == nullptr || cv->weight == nullptr)) return GDN_ERR_NULL;

  // alignment of vector-accessed buffers (the K-major kernels move v and the
  // output in 4-column vectors)
  const bool k_major = p->state_layout == GDN_STATE_K_MAJOR;
  const void* vec_ptrs[] = {t->q, t->k, t->initial_state, t->final_state, k_major ? t->v : nullptr,
                            k_major ? t->output : nullptr};
  for (const void* ptr : vec_ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDN_ERR_SHAPE;
  if (cv != nullptr) {
    const void* conv_vec[] = {cv->mixed, cv->weight, cv->initial_state, cv->final_state};
    for (const void* ptr : conv_vec)
      if (ptr != nullptr && !aligned16(ptr)) return GDN_ERR_SHAPE;
  }

  // the fused convolution runs with the token-recurrent kernel only
  st = resolve_plan(p, t->cu_seqlens_host, capsule || cv != nullptr, &rv, dense);
  if (st != GDN_OK) return st;
  const int32_t dense_len = dense ? (int32_t)(rv.N / rv.R) : 0;

  // overlap rules
  const size_t io = io_bytes(p->io_dtype);
  const size_t N = (size_t)rv.N, R = (size_t)rv.R, Hk = (size_t)rv.Hk, Hv = (size_t)rv.Hv;
  const size_t Dk = (size_t)rv.Dk, Dv = (size_t)rv.Dv;
  const size_t W = Hv + Hk * Dk + Hv * Dv;
  SlotPlan sp;
  // the pool written (the final state, or the replayed state of a fused step) may be
  // the pool read
  const float* write_pool = rp != nullptr ? rp->state : t->final_state;
  st = plan_slots(slots, rv.R, t->initial_state != nullptr && t->initial_state == write_pool, &sp);
  if (st != GDN_OK) return st;
  const size_t state_bytes = (sp.P > 0 ? (size_t)sp.P : R) * Hv * Dv * Dk * 4;
  const Span inputs[] = {
      Span(t->q, N * Hk * Dk * io), Span(t->k, N * Hk * Dk * io), Span(t->v, N * Hv * Dv * io),
      Span(t->a, N * Hv * 4),       Span(t->b, N * Hv * 4),       Span(t->A_log, Hv * 4),
      Span(t->dt_bias, Hv * 4),     Span(t->cu_seqlens, (R + 1) * 4),
      Span(t->capture_count, capsule ? R * 4 : 0), Span(sp.rd, sp.rd ? R * 4 : 0),
      Span(sp.wr, sp.wr ? R * 4 : 0)};
  const Span init(t->initial_state, state_bytes);
  const Span fin(t->final_state, state_bytes);
  const Span out(t->output, N * Hv * Dv * io);
  const Span cap(t->state_update, capsule ? R * (size_t)rv.cap * W * 4 : 0);
  // the workspace size is checked before the overlap rules, which read need_ws bytes of it
  const size_t need_ws = workspace_for(rv);
  if (need_ws > 0 && (workspace == nullptr || workspace_bytes < need_ws)) return GDN_ERR_WORKSPACE;
  if (need_ws > 0 && !aligned16(workspace)) return GDN_ERR_WORKSPACE;
  const Span ws(workspace, need_ws);
  const Span outputs[] = {out, fin, cap, ws};
  for (const Span& o : outputs) {
    for (const Span& i : inputs)
      if (o.overlaps(i)) return GDN_ERR_ALIAS;
  }
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (outputs[i].overlaps(outputs[j])) return GDN_ERR_ALIAS;
  if (out.overlaps(init) || cap.overlaps(init) || ws.overlaps(init)) return GDN_ERR_ALIAS;
  // final_state may be the very same buffer as initial_state (in-place update)
  if (fin.overlaps(init) && t->final_state != t->initial_state) return GDN_ERR_ALIAS;
  if (rp != nullptr) {
    // the committed bank is read only; the previous capsule and the accepted
    // counts are inputs; the inactive bank overlaps nothing
    const Span prev(rp->capsule, R * (size_t)rv.cap * W * 4);
    const Span acc(rp->accepted, R * 4);
    const Span dst(rp->state, state_bytes);
    if (fin.overlaps(init)) return GDN_ERR_ALIAS;
    for (const Span& o : {out, fin, cap, dst})
      if (o.overlaps(prev) || o.overlaps(acc)) return GDN_ERR_ALIAS;
    for (const Span& o : {out, fin, cap})
      if (o.overlaps(dst)) return GDN_ERR_ALIAS;
    // one pool for the committed and the inactive slots (distinct slots), or disjoint banks
    if (init.overlaps(dst) && !(sp.P > 0 && rp->state == t->initial_state)) return GDN_ERR_ALIAS;
    for (const Span& i : inputs)
      if (dst.overlaps(i)) return GDN_ERR_ALIAS;
  }
  const size_t Cm = 2 * Hk * Dk + Hv * Dv;         // channels of the fused convolution
  if (cv != nullptr) {
    // its carried inputs are read by every workgroup of a key head and written by
    // one, so the new ones go to another buffer; nothing else overlaps them
    const size_t K = (size_t)cv->kernel_size;
    const Span c_in[] = {Span(cv->mixed, N * Cm * io), Span(cv->weight, Cm * K * 4), Span(cv->bias, Cm * 4),
                         Span(cv->initial_state, R * Cm * (K - 1) * 4)};
    const Span c_fin(cv->final_state, R * Cm * (K - 1) * 4);
    for (const Span& o : {out, fin, cap, ws, c_fin})
      for (const Span& i : c_in)
        if (o.overlaps(i)) return GDN_ERR_ALIAS;
    for (const Span& o : {out, fin, cap, ws, init})
      if (c_fin.overlaps(o)) return GDN_ERR_ALIAS;
    for (const Span& i : inputs)
      if (c_fin.overlaps(i)) return GDN_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (rv.plan == GDN_PLAN_RECURRENT) {
    gdn::RecurrentArgs a{};
    a.q = t->q; a.k = t->k; a.v = t->v; a.a = t->a; a.b = t->b;
    a.A_log = t->A_log; a.dt_bias = t->dt_bias; a.cu_seqlens = t->cu_seqlens;
    a.initial_state = t->initial_state; a.final_state = t->final_state; a.output = t->output;
    a.state_update = t->state_update; a.capture_count = t->capture_count;
    a.N = (int32_t)rv.N; a.R = (int32_t)rv.R; a.Hk = (int32_t)rv.Hk; a.Hv = (int32_t)rv.Hv;
    a.Dk = (int32_t)rv.Dk; a.Dv = (int32_t)rv.Dv; a.group = (int32_t)(rv.Hv / rv.Hk);
    a.capacity = rv.cap; a.capsule_width = (int32_t)W; a.scale = rv.scale;
    a.dense_len = dense_len; a.gate_none = gate_none ? 1 : 0;
    a.initial_slots = sp.rd; a.final_slots = sp.wr; a.num_slots = (int32_t)sp.P;
    a.k_major = k_major ? 1 : 0;
    a.gated = gated ? 1 : 0; a.delta = delta ? 1 : 0;
    if (rp != nullptr) {
      a.replay_capsule = rp->capsule; a.accepted = rp->accepted; a.replay_state = rp->state;
    }
    if (cv != nullptr) {
      a.mixed = cv->mixed; a.conv_weight = cv->weight; a.conv_bias = cv->bias;
      a.conv_init = cv->initial_state; a.conv_final = cv->final_state;
      a.conv_channels = (int32_t)Cm; a.conv_silu = cv->activation == GDN_CONV_SILU ? 1 : 0;
    }
    err = k_major ? gdn::launch_recurrent_kmajor(a, p->io_dtype, s) : gdn::launch_recurrent(a, p->io_dtype, s);
  } else {
    gdn::ChunkArgs a{};
    a.q = t->q; a.k = t->k; a.v = t->v; a.a = t->a; a.b = t->b;
    a.A_log = t->A_log; a.dt_bias = t->dt_bias; a.cu_seqlens = t->cu_seqlens;
    a.initial_state = t->initial_state; a.final_state = t->final_state; a.output = t->output;
    a.workspace = workspace;
    a.N = (int32_t)rv.N; a.R = (int32_t)rv.R; a.Hk = (int32_t)rv.Hk; a.Hv = (int32_t)rv.Hv;
    a.group = (int32_t)(rv.Hv / rv.Hk); a.max_chunks = (int32_t)rv.chunk_slots; a.scale = rv.scale;
    a.dense_len = dense_len; a.gate_none = gate_none ? 1 : 0;
    a.initial_slots = sp.rd; a.final_slots = sp.wr; a.num_slots = (int32_t)sp.P;
    a.k_major = k_major ? 1 : 0;
    a.gated = gated ? 1 : 0; a.delta = delta ? 1 : 0;
    err = gdn::launch_chunk(a, p->io_dtype, s);
  }
  return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

static int replay_impl(int32_t R, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, int32_t capacity,
                       const float* src, const float* capsule, const int32_t* accepted,
                       const int32_t* accepted_host, float* dst, const gdn_slots* slots, bool k_major,
                       void* stream) {
  if (R < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0) return GDN_ERR_SHAPE;
  if (!supported_dim(Dk) || !supported_dim(Dv)) return GDN_ERR_SHAPE;
  if (capacity < 0) return GDN_ERR_CAPACITY;
  if (R == 0) return GDN_OK;
  if (src == nullptr || dst == nullptr || accepted == nullptr) return GDN_ERR_NULL;
  if (capacity > 0 && capsule == nullptr) return GDN_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return GDN_ERR_SHAPE;
  const int64_t W64 = (int64_t)Hv + (int64_t)Hk * Dk + (int64_t)Hv * Dv;
  if (W64 > std::numeric_limits<int32_t>::max()) return GDN_ERR_SHAPE;
  if (accepted_host != nullptr) {
    for (int32_t r = 0; r < R; ++r)
      if (accepted_host[r] < 0 || accepted_host[r] > capacity) return GDN_ERR_CAPACITY;
  }
  SlotPlan sp;
  const int sst = plan_slots(slots, R, src == dst, &sp);
  if (sst != GDN_OK) return sst;
  const size_t state_bytes = (sp.P > 0 ? (size_t)sp.P : (size_t)R) * Hv * Dv * Dk * 4;
  const Span d(dst, state_bytes);
  // a pooled replay may read and write one pool (distinct slots); otherwise the banks are disjoint
  if ((d.overlaps(Span(src, state_bytes)) && !(sp.P > 0 && src == dst)) ||
      d.overlaps(Span(capsule, (size_t)R * capacity * W64 * 4)) || d.overlaps(Span(accepted, (size_t)R * 4)) ||
      d.overlaps(Span(sp.rd, sp.rd ? (size_t)R * 4 : 0)) || d.overlaps(Span(sp.wr, sp.wr ? (size_t)R * 4 : 0)))
    return GDN_ERR_ALIAS;
  gdn::ReplayArgs a{};
  a.src = src; a.capsule = capsule; a.accepted = accepted; a.dst = dst;
  a.src_slots = sp.rd; a.dst_slots = sp.wr; a.num_slots = (int32_t)sp.P;
  a.R = R; a.Hk = Hk; a.Hv = Hv; a.Dk = Dk; a.Dv = Dv; a.group = Hv / Hk;
  a.capacity = capacity; a.capsule_width = (int32_t)W64;
  a.k_major = k_major ? 1 : 0;
  hipError_t err = gdn::launch_replay(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

static int conv_forward_impl(const gdn_conv_params* p, const gdn_conv_tensors* t, const gdn_slots* slots,
                             void* stream) {
  if (p == nullptr || t == nullptr) return GDN_ERR_NULL;
  if (p->activation != GDN_CONV_SILU && p->activation != GDN_CONV_NONE) return GDN_ERR_RULE;
  if (p->io_dtype != GDN_F32 && p->io_dtype != GDN_F16) return GDN_ERR_DTYPE;
  const int64_t N = p->num_tokens, R = p->num_reqs, C = p->channels, K = p->kernel_size;
  if (N < 0 || R < 0 || !conv_shape_ok(C, K)) return GDN_ERR_SHAPE;
  const int64_t cap = p->state_update_capacity;
  if (cap < 0) return GDN_ERR_CAPACITY;
  const bool capture = t->state_update != nullptr;
  if (capture && cap == 0) return GDN_ERR_CAPACITY;
  if (R == 0) return N == 0 ? GDN_OK : GDN_ERR_SHAPE;
  const bool dense = t->cu_seqlens == nullptr;
  if (dense && (t->cu_seqlens_host != nullptr || N % R != 0)) return GDN_ERR_SHAPE;
  if (N > 0 && (t->x == nullptr || t->weight == nullptr || t->output == nullptr)) return GDN_ERR_NULL;
  const void* vec_ptrs[] = {t->x, t->weight, t->initial_state, t->final_state, t->output, t->state_update};
  for (const void* ptr : vec_ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return GDN_ERR_SHAPE;
  if (!dense && t->cu_seqlens_host != nullptr) {
    int64_t max_len = 0, slots = 0;
    const int st = check_cu_host(t->cu_seqlens_host, R, N, &max_len, &slots);
    if (st != GDN_OK) return st;
  }

  SlotPlan sp;
  const int sst = plan_slots(slots, R, t->initial_state != nullptr && t->initial_state == t->final_state, &sp);
  if (sst != GDN_OK) return sst;
  const size_t io = io_bytes(p->io_dtype);
  const size_t state_bytes = (size_t)((sp.P > 0 ? sp.P : R) * C * (K - 1)) * 4;
  const Span inputs[] = {Span(t->x, (size_t)(N * C) * io), Span(t->weight, (size_t)(C * K) * 4),
                         Span(t->bias, (size_t)C * 4), Span(t->cu_seqlens, (size_t)(R + 1) * 4),
                         Span(t->capture_count, capture ? (size_t)R * 4 : 0),
                         Span(sp.rd, sp.rd ? (size_t)R * 4 : 0), Span(sp.wr, sp.wr ? (size_t)R * 4 : 0)};
  const Span init(t->initial_state, state_bytes);
  const Span fin(t->final_state, state_bytes);
  const Span out(t->output, (size_t)(N * C) * io);
  const Span cap_rows(t->state_update, capture ? (size_t)(R * cap * C) * 4 : 0);
  const Span outputs[] = {out, fin, cap_rows};
  for (const Span& o : outputs)
    for (const Span& i : inputs)
      if (o.overlaps(i)) return GDN_ERR_ALIAS;
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (outputs[i].overlaps(outputs[j])) return GDN_ERR_ALIAS;
  if (out.overlaps(init) || cap_rows.overlaps(init)) return GDN_ERR_ALIAS;
  // final_state may be the very same buffer as initial_state (in-place update)
  if (fin.overlaps(init) && t->final_state != t->initial_state) return GDN_ERR_ALIAS;

  // packed requests of one common length, as the host mirror shows, are indexed
  // like the dense layout (cu[r] = r L), which spares the kernel its search
  int64_t uniform_len = dense ? (N / R) : -1;
  if (!dense && t->cu_seqlens_host != nullptr && N > 0 && N % R == 0) {
    uniform_len = N / R;
    for (int64_t r = 0; r <= R && uniform_len >= 0; ++r)
      if (t->cu_seqlens_host[r] != r * (N / R)) uniform_len = -1;
  }

  gdn::ConvArgs a{};
  a.x = t->x; a.weight = t->weight; a.bias = t->bias;
  a.cu_seqlens = uniform_len >= 0 ? nullptr : t->cu_seqlens;
  a.initial_state = t->initial_state; a.final_state = t->final_state; a.output = t->output;
  a.state_update = capture ? t->state_update : nullptr;
  a.capture_count = capture ? t->capture_count : nullptr;
  a.N = (int32_t)N; a.R = (int32_t)R; a.C = (int32_t)C; a.K = (int32_t)K;
  a.dense_len = uniform_len >= 0 ? (int32_t)uniform_len : 0;
  a.silu = p->activation == GDN_CONV_SILU ? 1 : 0;
  a.capacity = (int32_t)cap;
  a.initial_slots = sp.rd; a.final_slots = sp.wr; a.num_slots = (int32_t)sp.P;
  a.tokens_per_block = conv_tokens_per_block(N, C);
  // one-dimensional grids of (token blocks or requests) x channel groups
  const int64_t groups = gdn::conv_channel_groups(C);
  if (((N + a.tokens_per_block - 1) / a.tokens_per_block) * groups > std::numeric_limits<int32_t>::max() ||
      R * groups > std::numeric_limits<int32_t>::max())
    return GDN_ERR_SHAPE;
  // the final-state kernel is launched unless the host can see that the forward
  // kernel writes every request's final state
  a.final_in_place = t->final_state != nullptr && t->final_state == t->initial_state;
  const bool in_place = a.final_in_place != 0;
  a.final_pending = 1;
  if (uniform_len >= 0) {
    bool all = true;
    for (int64_t r = 0; r < R && all; ++r)
      all = gdn::final_in_forward((int)(r * uniform_len), (int)((r + 1) * uniform_len), a.tokens_per_block,
                                  in_place);
    a.final_pending = all ? 0 : 1;
  } else if (t->cu_seqlens_host != nullptr) {
    bool all = true;
    for (int64_t r = 0; r < R && all; ++r)
      all = gdn::final_in_forward(t->cu_seqlens_host[r], t->cu_seqlens_host[r + 1], a.tokens_per_block,
                                  in_place);
    a.final_pending = all ? 0 : 1;
  }
  const hipError_t err = gdn::launch_conv(a, p->io_dtype, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

static int conv_replay_impl(int32_t R, int32_t C, int32_t K, int32_t capacity, const float* src,
                            const float* capture, const int32_t* accepted, const int32_t* accepted_host,
                            float* dst, const gdn_slots* slots, void* stream) {
  if (R < 0 || !conv_shape_ok(C, K)) return GDN_ERR_SHAPE;
  if (capacity < 0) return GDN_ERR_CAPACITY;
  if (R == 0) return GDN_OK;
  if (src == nullptr || dst == nullptr || accepted == nullptr) return GDN_ERR_NULL;
  if (capacity > 0 && capture == nullptr) return GDN_ERR_NULL;
  if ((int64_t)R * gdn::conv_channel_groups(C) > std::numeric_limits<int32_t>::max()) return GDN_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst) || (capture != nullptr && !aligned16(capture))) return GDN_ERR_SHAPE;
  if (accepted_host != nullptr) {
    for (int32_t r = 0; r < R; ++r)
      if (accepted_host[r] < 0 || accepted_host[r] > capacity) return GDN_ERR_CAPACITY;
  }
  SlotPlan sp;
  const int sst = plan_slots(slots, R, src == dst, &sp);
  if (sst != GDN_OK) return sst;
  const size_t state_bytes = (sp.P > 0 ? (size_t)sp.P : (size_t)R) * C * (K - 1) * 4;
  const Span d(dst, state_bytes);
  if ((d.overlaps(Span(src, state_bytes)) && !(sp.P > 0 && src == dst)) ||
      d.overlaps(Span(capture, (size_t)R * capacity * C * 4)) || d.overlaps(Span(accepted, (size_t)R * 4)) ||
      d.overlaps(Span(sp.rd, sp.rd ? (size_t)R * 4 : 0)) || d.overlaps(Span(sp.wr, sp.wr ? (size_t)R * 4 : 0)))
    return GDN_ERR_ALIAS;
  gdn::ConvReplayArgs a{};
  a.src = src; a.capture = capture; a.accepted = accepted; a.dst = dst;
  a.src_slots = sp.rd; a.dst_slots = sp.wr; a.num_slots = (int32_t)sp.P;
  a.R = R; a.C = C; a.K = K; a.capacity = capacity;
  const hipError_t err = gdn::launch_conv_replay(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_forward(const gdn_params* p, const gdn_tensors* t, void* workspace, size_t workspace_bytes,
                void* stream) {
  return forward_impl(p, t, nullptr, workspace, workspace_bytes, stream);
}

int gdn_forward_pooled(const gdn_params* p, const gdn_tensors* t, const gdn_slots* slots, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (slots == nullptr) return GDN_ERR_NULL;
  return forward_impl(p, t, slots, workspace, workspace_bytes, stream);
}

int gdn_replay_forward(const gdn_params* p, const gdn_tensors* t, const float* prev_state_update,
                       const int32_t* accepted, const int32_t* accepted_host, float* replay_state,
                       void* stream) {
  const FusedReplay rp{prev_state_update, accepted, accepted_host, replay_state};
  return forward_impl(p, t, nullptr, nullptr, 0, stream, &rp);
}

int gdn_replay_forward_pooled(const gdn_params* p, const gdn_tensors* t, const gdn_slots* slots,
                              const float* prev_state_update, const int32_t* accepted,
                              const int32_t* accepted_host, float* replay_pool, void* stream) {
  if (slots == nullptr) return GDN_ERR_NULL;
  const FusedReplay rp{prev_state_update, accepted, accepted_host, replay_pool};
  return forward_impl(p, t, slots, nullptr, 0, stream, &rp);
}

int gdn_replay(int32_t R, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, int32_t capacity,
               const float* src, const float* capsule, const int32_t* accepted,
               const int32_t* accepted_host, float* dst, void* stream) {
  return replay_impl(R, Hk, Hv, Dk, Dv, capacity, src, capsule, accepted, accepted_host, dst, nullptr, false,
                     stream);
}

int gdn_replay_pooled(const gdn_params* p, const float* src_pool, const float* capsule, const int32_t* accepted,
                      const int32_t* accepted_host, float* dst_pool, const gdn_slots* slots, void* stream) {
  if (p == nullptr) return GDN_ERR_NULL;
  if (p->state_layout != GDN_STATE_V_MAJOR && p->state_layout != GDN_STATE_K_MAJOR) return GDN_ERR_SHAPE;
  return replay_impl(p->num_reqs, p->num_k_heads, p->num_v_heads, p->head_k_dim, p->head_v_dim,
                     p->state_update_capacity, src_pool, capsule, accepted, accepted_host, dst_pool, slots,
                     p->state_layout == GDN_STATE_K_MAJOR, stream);
}

int gdn_conv_decode_forward(const gdn_params* p, const gdn_tensors* t, const gdn_conv_fused* conv, void* stream) {
  if (conv == nullptr) return GDN_ERR_NULL;
  return forward_impl(p, t, nullptr, nullptr, 0, stream, nullptr, conv);
}

int gdn_conv_forward(const gdn_conv_params* p, const gdn_conv_tensors* t, void* stream) {
  return conv_forward_impl(p, t, nullptr, stream);
}

int gdn_conv_forward_pooled(const gdn_conv_params* p, const gdn_conv_tensors* t, const gdn_slots* slots,
                            void* stream) {
  if (slots == nullptr) return GDN_ERR_NULL;
  return conv_forward_impl(p, t, slots, stream);
}

int gdn_conv_replay(int32_t R, int32_t C, int32_t K, int32_t capacity, const float* src,
                    const float* capture, const int32_t* accepted, const int32_t* accepted_host,
                    float* dst, void* stream) {
  return conv_replay_impl(R, C, K, capacity, src, capture, accepted, accepted_host, dst, nullptr, stream);
}

int gdn_conv_replay_pooled(int32_t R, int32_t C, int32_t K, int32_t capacity, const float* src_pool,
                           const float* capture, const int32_t* accepted, const int32_t* accepted_host,
                           float* dst_pool, const gdn_slots* slots, void* stream) {
  if (slots == nullptr) return GDN_ERR_NULL;
  return conv_replay_impl(R, C, K, capacity, src_pool, capture, accepted, accepted_host, dst_pool, slots,
                          stream);
}

int gdn_publish_slots(int32_t R, int32_t* committed, int32_t* inactive, void* stream) {
  if (R < 0) return GDN_ERR_SHAPE;
  if (R == 0) return GDN_OK;
  if (committed == nullptr || inactive == nullptr) return GDN_ERR_NULL;
  if (Span(committed, (size_t)R * 4).overlaps(Span(inactive, (size_t)R * 4))) return GDN_ERR_ALIAS;
  const hipError_t err = gdn::launch_publish(R, committed, inactive, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"

// The forward call with a workspace the caller does not own (gdn_noalloc.hip).
namespace gdn {
int forward_entry(const gdn_params* p, const gdn_tensors* t, const gdn_slots* slots, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return forward_impl(p, t, slots, workspace, workspace_bytes, stream);
}
}  // namespace gdn

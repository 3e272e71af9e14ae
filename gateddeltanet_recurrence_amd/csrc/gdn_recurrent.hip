// Token-recurrent GatedDeltaNet kernels: gdn_decode, gdn_capsule, the fused
// speculative step gdn_replay_verify and the decode with the causal convolution
// fused in, gdn_conv_decode.
//
// The recurrent decode path of the operator ("[CUDA] Add compact GatedDeltaNet
// operator", Description) and, with a capsule, the compact state-update capture
// of the same page: for every captured token the FP32 decay alpha, the shared
// unit key k^ and the delta u = beta (v - alpha S k^) are written so that
// S_t = alpha_t S_{t-1} + u_t k^_t^T can be replayed later.
//
// Work decomposition (CDNA4, wave64). A workgroup owns a block of state rows
// of one (request, value head); each wavefront owns RW = RI * NI rows and keeps
// them in registers for the whole segment, so the FP32 state is read once and
// written once whatever the segment length. A state row (Dk floats, V-major,
// contiguous) is spread over LPR adjacent lanes holding E = Dk/LPR floats each,
// loaded as 16-byte vectors: one wave instruction covers RI full rows, i.e. RI
// fully used 128-byte lines for Dk = 128. Row dot products (S k^ and S q^) are
// in-lane FMAs followed by a DPP reduction over the LPR lanes; the decode uses no
// LDS (the capsule kernels stage their tokens in LDS, and gdn_conv_decode its
// convolution's output).
//
// Per token, with the old state S:
//   pk = S k^, pq = S q^  (one pass over the registers, reduced together)
//   u  = beta (v - alpha pk)
//   o  = alpha pq + u (k^ . q^)      ( = S_new q^ )
//   S  = alpha S + u k^^T
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

// Launch shape of the Dk = 128 instantiation: state rows per lane group (NI) and
// waves per workgroup; state streams may use nontemporal loads/stores.
#ifndef GDN_REC_NI128
#define GDN_REC_NI128 2
#endif
#ifndef GDN_REC_WAVES
#define GDN_REC_WAVES 4
#endif
#ifndef GDN_STATE_NT
#define GDN_STATE_NT 1
#endif
// Rows per lane group of the Dk = 128 capsule (verify) instantiation.
#ifndef GDN_CAP_NI128
#define GDN_CAP_NI128 4
#endif

namespace gdn {

__device__ __forceinline__ float4_t load_state4(const float* p) {
#if GDN_STATE_NT
  return __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(p));
#else
  return *reinterpret_cast<const float4_t*>(p);
#endif
}

__device__ __forceinline__ void store_state4(float* p, float4_t x) {
#if GDN_STATE_NT
  __builtin_nontemporal_store(x, reinterpret_cast<float4_t*>(p));
#else
  *reinterpret_cast<float4_t*>(p) = x;
#endif
}

template <int DK>
struct RecLayout {
  static constexpr int LPR = DK >= 32 ? 8 : 4;   // lanes per state row
  static constexpr int E = DK / LPR;              // floats per lane per row
  static constexpr int V4 = E / 4;                // 16-byte vectors per lane per row
  static constexpr int RI = 64 / LPR;             // rows per wave instruction
  static_assert(E % 4 == 0, "row slice must be whole float4 vectors");
};

// The NI state rows of a lane group (rows row_base + i RI + rg, this lane's E
// floats of each) into registers, zero without an initial state. Raw buffer
// loads with a range check do it without a single branch: the range is the
// head's Dv x Dk floats, or empty when there is no initial state, and a load
// outside it returns zero (rows at or past Dv included). Branches around the
// loads had compiled to waits for the first loads before the later ones were
// issued, and to waits that also covered the state where only later loads
// were needed.
template <int DK, int NI, int I0 = 0, int NL = NI>
__device__ __forceinline__ void load_state_rows(const float* init, const void* any_base, int row_base, int rg,
                                                int c, int Dv, float (&S)[NI][RecLayout<DK>::E],
                                                bool (&valid)[NI]) {
  using L = RecLayout<DK>;
  constexpr int LPR = L::LPR, V4 = L::V4, RI = L::RI;
  const rsrc_t rs = make_rsrc(init != nullptr ? static_cast<const void*>(init) : any_base,
                              init != nullptr ? Dv * DK * 4 : 0);
#pragma unroll
  for (int i = I0; i < I0 + NL; ++i) {
    const int row = row_base + i * RI + rg;
    valid[i] = row < Dv;
#pragma unroll
    for (int j = 0; j < V4; ++j) {
      const float4_t x = __builtin_bit_cast(
          float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (row * DK + 4 * c + 4 * LPR * j) * 4, 0,
                                                          kBufferNontemporal));
      S[i][4 * j + 0] = x.x;
      S[i][4 * j + 1] = x.y;
      S[i][4 * j + 2] = x.z;
      S[i][4 * j + 3] = x.w;
    }
  }
}

// ---- The causal convolution fused into the decode (RecurrentArgs::mixed).
// A workgroup of (request r, value head h, state rows rb0 .. rb0 + nrow - 1)
// convolves, per token, the channels it reads: the q and k channels of key
// head g (DK each) and the v channels of its rows, in groups of 4 adjacent
// channels; group i lands at floats 4 i .. 4 i + 3 of the token's LDS slot,
// which is [q (DK) | k (DK) | v rows].
template <int DK>
__device__ __forceinline__ int conv_channel(const RecurrentArgs& p, int g, int h, int rb0, int gi) {
  if (gi < DK / 4) return g * DK + 4 * gi;
  if (gi < DK / 2) return p.Hk * DK + g * DK + 4 * (gi - DK / 4);
  return 2 * p.Hk * DK + h * p.Dv + rb0 + 4 * (gi - DK / 2);
}

// Entry idx of e = [carried inputs (K - 1), x of the request's tokens] for the
// 4 channels c .. c + 3: from the carried state below K - 1 (an empty range
// without one reads zeros), else from packed token t0 + idx - (K - 1).
template <typename IO>
__device__ __forceinline__ float4_t conv_entry(const RecurrentArgs& p, rsrc_t rs, int c, int t0, int idx) {
  constexpr int K = kConvFusedK;
  if (idx < K - 1) {
    float4_t v;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) v[ch] = buf_load_f32(rs, ((c + ch) * (K - 1) + idx) * 4);
    return v;
  }
  return IoOps<IO>::load4(static_cast<const IO*>(p.mixed) + (size_t)(t0 + idx - (K - 1)) * p.conv_channels + c);
}

__device__ __forceinline__ rsrc_t conv_state_rsrc(const RecurrentArgs& p, int r) {
  constexpr int K = kConvFusedK;
  const int bytes = p.conv_channels * (K - 1) * 4;
  return p.conv_init != nullptr ? make_rsrc(p.conv_init + (size_t)r * p.conv_channels * (K - 1), bytes)
                                : make_rsrc(p.mixed, 0);
}

// Token j of the request: y = act(bias + sum_{m<K} w[m] e[j + m]), the
// multiply-adds in the convolution kernel's order (oldest entry first), rounded
// to the I/O type as the convolution's stored output is, into dst.
template <typename IO, int DK>
__device__ __forceinline__ void conv_token(const RecurrentArgs& p, int r, int g, int h, int rb0, int nrow,
                                           int t0, int j, int nthreads, float* dst, int gi0) {
  constexpr int K = kConvFusedK;
  const int ngroups = DK / 2 + nrow / 4;
  const rsrc_t rs = conv_state_rsrc(p, r);
  const rsrc_t rb = make_rsrc(p.conv_bias != nullptr ? static_cast<const void*>(p.conv_bias) : p.mixed,
                              p.conv_bias != nullptr ? p.conv_channels * 4 : 0);
  for (int gi = gi0; gi < ngroups; gi += nthreads) {
    const int c = conv_channel<DK>(p, g, h, rb0, gi);
    // weights [C, K]: 4 K consecutive floats, channel-major
    float wf[4 * K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float4_t x = *reinterpret_cast<const float4_t*>(p.conv_weight + (size_t)c * K + 4 * i);
      wf[4 * i + 0] = x.x; wf[4 * i + 1] = x.y; wf[4 * i + 2] = x.z; wf[4 * i + 3] = x.w;
    }
    float4_t e[K];
#pragma unroll
    for (int m = 0; m < K; ++m) e[m] = conv_entry<IO>(p, rs, c, t0, j + m);
    float y[4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      float z = buf_load_f32(rb, (c + ch) * 4);
#pragma unroll
      for (int m = 0; m < K; ++m) z = fmaf(wf[ch * K + m], e[m][ch], z);
      y[ch] = (float)(IO)(p.conv_silu ? silu(z) : z);
    }
    *reinterpret_cast<float4_t*>(dst + 4 * gi) = float4_t{y[0], y[1], y[2], y[3]};
  }
}

// The inputs of the first token for the thread's first channel group (group
// threadIdx.x), loaded before the state rows so that they arrive first (loads
// complete in issue order) and the convolution runs while the state is in
// flight; the carried inputs also serve the final write. Range-checked buffer
// loads with no branch: a thread without a group reads past the ranges, i.e.
// zeros (unused), and without a token the input row's range is empty.
struct ConvFirst {
  float4_t w[kConvFusedK];        // the 4 K weights of channels c .. c + 3, [C, K] order
  float4_t st[kConvFusedK - 1];   // their 4 (K - 1) carried inputs, [C, K - 1] order
  float4_t x;                     // their inputs at the first token
  float4_t bias;
};

template <typename IO, int DK>
__device__ __forceinline__ ConvFirst conv_first_load(const RecurrentArgs& p, int r, int g, int h, int rb0,
                                                     int nrow, int t0, bool has_token) {
  constexpr int K = kConvFusedK;
  const int C = p.conv_channels;
  const int gi = threadIdx.x;
  const bool on = gi < DK / 2 + nrow / 4;
  const int c = on ? conv_channel<DK>(p, g, h, rb0, gi) : 0;
  ConvFirst f;
  const rsrc_t rw = make_rsrc(p.conv_weight != nullptr ? static_cast<const void*>(p.conv_weight) : p.mixed,
                              p.conv_weight != nullptr ? C * K * 4 : 0);
#pragma unroll
  for (int i = 0; i < K; ++i)
    f.w[i] = __builtin_bit_cast(float4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(rw, on ? c * K * 4 + 16 * i : C * K * 4, 0, 0));
  const rsrc_t rs = conv_state_rsrc(p, r);
#pragma unroll
  for (int i = 0; i < K - 1; ++i)
    f.st[i] = __builtin_bit_cast(
        float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, on ? c * (K - 1) * 4 + 16 * i : C * (K - 1) * 4, 0, 0));
  const int io = (int)sizeof(IO);
  const rsrc_t rx = make_rsrc(p.mixed != nullptr ? static_cast<const IO*>(p.mixed) + (size_t)t0 * C : nullptr,
                              (p.mixed != nullptr && has_token) ? C * io : 0);
  if constexpr (sizeof(IO) == 2) {
    const half4_t hx = buf_load_h4(rx, on ? c * io : C * io);
    f.x = float4_t{(float)hx.x, (float)hx.y, (float)hx.z, (float)hx.w};
  } else {
    f.x = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, on ? c * io : C * io, 0, 0));
  }
  const rsrc_t rb = make_rsrc(p.conv_bias != nullptr ? static_cast<const void*>(p.conv_bias) : p.mixed,
                              p.conv_bias != nullptr ? C * 4 : 0);
  f.bias = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, on ? c * 4 : C * 4, 0, 0));
  return f;
}

// The first token's output of the thread's first group from f: the window is
// the carried inputs then the token's input, the arithmetic that of conv_token.
template <typename IO, int DK>
__device__ __forceinline__ void conv_first_compute(const RecurrentArgs& p, const ConvFirst& f, int nrow,
                                                   float* dst) {
  constexpr int K = kConvFusedK;
  const int gi = threadIdx.x;
  if (gi >= DK / 2 + nrow / 4) return;
  float wf[4 * K], sf[4 * (K - 1)];
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wf[4 * i + jj] = f.w[i][jj];
#pragma unroll
  for (int i = 0; i < K - 1; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sf[4 * i + jj] = f.st[i][jj];
  float y[4];
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    float z = f.bias[ch];
#pragma unroll
    for (int m = 0; m < K - 1; ++m) z = fmaf(wf[ch * K + m], sf[ch * (K - 1) + m], z);
    z = fmaf(wf[ch * K + K - 1], f.x[ch], z);
    y[ch] = (float)(IO)(p.conv_silu ? silu(z) : z);
  }
  *reinterpret_cast<float4_t*>(dst + 4 * gi) = float4_t{y[0], y[1], y[2], y[3]};
}

// The request's new carried inputs, e[L .. L + K - 2] (L tokens), for the
// channels this workgroup owns: its v rows, and the q and k channels of g when
// own_qk (one workgroup per key head and request). With at most one token the
// thread's first group takes them from the inputs fetched for that token.
template <typename IO, int DK>
__device__ __forceinline__ void conv_final_write(const RecurrentArgs& p, int r, int g, int h, int rb0, int nrow,
                                                 int t0, int L, bool own_qk, int nthreads, const ConvFirst& cf) {
  constexpr int K = kConvFusedK;
  const int ngroups = DK / 2 + nrow / 4;
  const rsrc_t rs = conv_state_rsrc(p, r);
  float* fin = p.conv_final + (size_t)r * p.conv_channels * (K - 1);
  for (int gi = threadIdx.x; gi < ngroups; gi += nthreads) {
    if (gi < DK / 2 && !own_qk) continue;
    const int c = conv_channel<DK>(p, g, h, rb0, gi);
    float f[4 * (K - 1)];                          // channel-major: f[ch (K - 1) + m]
    if (gi == (int)threadIdx.x && L <= 1) {
      // cf.st holds the carried inputs in this order already; one token shifts them
      float sf[4 * (K - 1)];
#pragma unroll
      for (int i = 0; i < K - 1; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sf[4 * i + jj] = cf.st[i][jj];
#pragma unroll
      for (int ch = 0; ch < 4; ++ch)
#pragma unroll
        for (int m = 0; m < K - 1; ++m)
          f[ch * (K - 1) + m] = L == 0 ? sf[ch * (K - 1) + m]
                                       : (m + 1 < K - 1 ? sf[ch * (K - 1) + m + 1] : cf.x[ch]);
    } else {
#pragma unroll
      for (int m = 0; m < K - 1; ++m) {
        const float4_t v = conv_entry<IO>(p, rs, c, t0, L + m);
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) f[ch * (K - 1) + m] = v[ch];
      }
    }
#pragma unroll
    for (int i = 0; i < K - 1; ++i)
      *reinterpret_cast<float4_t*>(fin + (size_t)c * (K - 1) + 4 * i) =
          float4_t{f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]};
  }
}

template <typename IO, int DK, int NI, bool CAPTURE, bool CONV = false>
__device__ __forceinline__ void recurrent_body(const RecurrentArgs& p, int waves_per_block,
                                               int blocks_per_head) {
  using L = RecLayout<DK>;
  constexpr int LPR = L::LPR, E = L::E, V4 = L::V4, RI = L::RI, RW = RI * NI;
  static_assert(NI <= LPR, "a lane group writes its NI rows with one lane each");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = lane / LPR;
  const int c = lane % LPR;

  int r, h, blk;
  if constexpr (CONV) {
    // The workgroups of one (request, key head) convolve the same q and k
    // channels: they are dealt to one XCD (workgroups go to the 8 XCDs round-robin
    // by index), so the convolution's inputs are fetched into one L2 rather than
    // into each of four (the grid is padded to whole rounds of 8 units).
    const int per_unit = p.group * blocks_per_head;
    const int xcd = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
    const int unit = xcd + 8 * (j / per_unit), m = j % per_unit;
    if (unit >= p.R * p.Hk) return;                  // padding: uniform, before any barrier
    r = unit / p.Hk;
    h = (unit % p.Hk) * p.group + m / blocks_per_head;
    blk = m % blocks_per_head;
  } else {
    int item = blockIdx.x;
    blk = item % blocks_per_head;
    item /= blocks_per_head;
    h = item % p.Hv;
    r = item / p.Hv;
  }
  const int g = h / p.group;
  const int Dv = p.Dv;
  const int row_base = (blk * waves_per_block + wave) * RW;

  // segment of this request; clamped so a malformed device array cannot index out of range
  const int t0 = seq_start(p, r);
  const int t1 = max(seq_start(p, r + 1), t0);

  const float* init = state_head(p.initial_state, state_slot(p.initial_slots, r, p.num_slots), p.Hv, h,
                                (size_t)Dv * DK);
  float* fin = state_head(p.final_state, state_slot(p.final_slots, r, p.num_slots), p.Hv, h, (size_t)Dv * DK);

  // fused convolution: the first token's inputs are requested before the state
  const int rb0 = blk * waves_per_block * RW;
  const int nrow = min(waves_per_block * RW, Dv - rb0);
  ConvFirst cfirst;
  if constexpr (CONV) cfirst = conv_first_load<IO, DK>(p, r, g, h, rb0, nrow, t0, t1 > t0);

  // ---- state rows into registers
  float S[NI][E];
  bool valid[NI];
  load_state_rows<DK, NI>(init, p.q, row_base, rg, c, Dv, S, valid);

  const bool gnone = p.gate_none != 0;             // A_log, dt_bias may be null then
  const bool gated = p.gated != 0, delta = p.delta != 0;
  const float expA = (gnone || !gated) ? 0.f : expf(p.A_log[h]);
  const float dtb = (gnone || !gated) ? 0.f : p.dt_bias[h];
  const IO* __restrict__ qp = static_cast<const IO*>(p.q);
  const IO* __restrict__ kp = static_cast<const IO*>(p.k);
  const IO* __restrict__ vp = static_cast<const IO*>(p.v);
  IO* __restrict__ op = static_cast<IO*>(p.output);

  int ncap = 0;
  if constexpr (CAPTURE) {
    int cmax = p.capacity;
    if (p.capture_count != nullptr) cmax = min(max(p.capture_count[r], 0), p.capacity);
    ncap = min(t1 - t0, cmax);
  }

  // fused convolution: a slot per token parity (one barrier per token: a slot is
  // rewritten two tokens later, after every wave has passed the barrier of the
  // token in between)
  constexpr int kConvSlot = CONV ? 2 * DK + GDN_REC_WAVES * RW : 1;
  __shared__ __attribute__((aligned(16))) float conv_slot[CONV ? 2 : 1][kConvSlot];

  // one token; `first` (a constant at each call) marks the first token of the
  // segment, whose convolution inputs were fetched ahead of the state
  auto step = [&](const int t, const bool first) __attribute__((always_inline)) {
    float kv[E], qv[E];
    float vv[NI];
    if constexpr (CONV) {
      float* cs = conv_slot[(t - t0) & 1];
      const int nthreads = 64 * waves_per_block;
      if (first) {
        conv_first_compute<IO, DK>(p, cfirst, nrow, cs);
        conv_token<IO, DK>(p, r, g, h, rb0, nrow, t0, 0, nthreads, cs, threadIdx.x + nthreads);
      } else {
        conv_token<IO, DK>(p, r, g, h, rb0, nrow, t0, t - t0, nthreads, cs, threadIdx.x);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < V4; ++j) {
        const float4_t qx = *reinterpret_cast<const float4_t*>(cs + 4 * c + 4 * LPR * j);
        const float4_t kx = *reinterpret_cast<const float4_t*>(cs + DK + 4 * c + 4 * LPR * j);
        kv[4 * j + 0] = kx.x; kv[4 * j + 1] = kx.y; kv[4 * j + 2] = kx.z; kv[4 * j + 3] = kx.w;
        qv[4 * j + 0] = qx.x; qv[4 * j + 1] = qx.y; qv[4 * j + 2] = qx.z; qv[4 * j + 3] = qx.w;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) vv[i] = cs[2 * DK + wave * RW + i * RI + rg];   // unused past Dv
    } else {
      const IO* krow = kp + ((size_t)t * p.Hk + g) * DK;
      const IO* qrow = qp + ((size_t)t * p.Hk + g) * DK;
#pragma unroll
      for (int j = 0; j < V4; ++j) {
        const float4_t kx = IoOps<IO>::load4(krow + 4 * c + 4 * LPR * j);
        const float4_t qx = IoOps<IO>::load4(qrow + 4 * c + 4 * LPR * j);
        kv[4 * j + 0] = kx.x; kv[4 * j + 1] = kx.y; kv[4 * j + 2] = kx.z; kv[4 * j + 3] = kx.w;
        qv[4 * j + 0] = qx.x; qv[4 * j + 1] = qx.y; qv[4 * j + 2] = qx.z; qv[4 * j + 3] = qx.w;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = min(row_base + i * RI + rg, Dv - 1);     // in bounds; unused past Dv
        vv[i] = IoOps<IO>::load1(vp + ((size_t)t * p.Hv + h) * Dv + row);
      }
    }
    const float at = gated ? p.a[(size_t)t * p.Hv + h] : 0.f;
    const float bt = delta ? p.b[(size_t)t * p.Hv + h] : 0.f;

    float ssk = 0.f, ssq = 0.f, skq = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ssk = fmaf(kv[e], kv[e], ssk);
      ssq = fmaf(qv[e], qv[e], ssq);
      skq = fmaf(kv[e], qv[e], skq);
    }
    ssk = group_sum<LPR>(ssk);
    ssq = group_sum<LPR>(ssq);
    skq = group_sum<LPR>(skq);
    const float rk = rsqrtf(ssk + kNormEps);
    const float rq = rsqrtf(ssq + kNormEps) * p.scale;
    // the rule: alpha = 1 without the gate; u = v (beta 1, no correction) without the delta
    const float alpha = gated ? gate_alpha(at, gnone, expA, dtb) : 1.f;
    const float beta = delta ? gate_beta(bt, gnone) : 1.f;
    const float kd = delta ? alpha : 0.f;         // weight of the correction alpha S k^
    const float kq = skq * rk * rq;               // k^ . q^
#pragma unroll
    for (int e = 0; e < E; ++e) kv[e] *= rk;      // k^

    float pk[NI], pq[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        sk = fmaf(S[i][e], kv[e], sk);
        sq = fmaf(S[i][e], qv[e], sq);
      }
      pk[i] = sk;
      pq[i] = sq;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      pk[i] = group_sum<LPR>(pk[i]);
      pq[i] = group_sum<LPR>(pq[i]);
    }

    const int jcap = t - t0;
    float* caprow = nullptr;
    if constexpr (CAPTURE) {
      if (jcap < ncap) caprow = p.state_update + ((size_t)r * p.capacity + jcap) * p.capsule_width;
    }
    // one range-checked store per token for the lane group's NI rows: lane c < NI
    // writes row c (as in recurrent_body_staged)
    float o_c = 0.f, u_c = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float u = beta * (vv[i] - kd * pk[i]);
      const float o = fmaf(alpha * rq, pq[i], u * kq);
#pragma unroll
      for (int e = 0; e < E; ++e) S[i][e] = fmaf(alpha, S[i][e], u * kv[e]);
      o_c = c == i ? o : o_c;
      u_c = c == i ? u : u_c;
    }
    {
      const int row_c = c < NI ? row_base + c * RI + rg : Dv;
      const rsrc_t ro = make_rsrc(op + ((size_t)t * p.Hv + h) * Dv, Dv * (int)sizeof(IO));
      if constexpr (sizeof(IO) == 2)
        buf_store_h1((_Float16)o_c, ro, row_c * 2);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, o_c), ro, row_c * 4, 0, 0);
      if constexpr (CAPTURE) {
        if (caprow != nullptr)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(unsigned, u_c), make_rsrc(caprow + p.Hv + p.Hk * DK + h * Dv, Dv * 4),
              row_c * 4, 0, 0);
      }
    }
    if constexpr (CAPTURE) {
      if (caprow != nullptr && blk == 0 && wave == 0) {
        if (lane == 0) caprow[h] = alpha;
        // the shared key is written once per key head, by its first value head
        if (h % p.group == 0 && rg == 0) {
#pragma unroll
          for (int j = 0; j < V4; ++j)
#pragma unroll
            for (int x = 0; x < 4; ++x)
              caprow[p.Hv + g * DK + 4 * c + 4 * LPR * j + x] = kv[4 * j + x];
        }
      }
    }
  };
  if constexpr (CONV) {
    if (t0 < t1) step(t0, true);
    for (int t = t0 + 1; t < t1; ++t) step(t, false);
  } else {
    for (int t = t0; t < t1; ++t) step(t, false);
  }

  if (fin != nullptr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!valid[i]) continue;
      const int row = row_base + i * RI + rg;
#pragma unroll
      for (int j = 0; j < V4; ++j) {
        float4_t x = {S[i][4 * j + 0], S[i][4 * j + 1], S[i][4 * j + 2], S[i][4 * j + 3]};
        store_state4(fin + (size_t)row * DK + 4 * c + 4 * LPR * j, x);
      }
    }
  }
  if constexpr (CONV) {
    if (p.conv_final != nullptr)
      conv_final_write<IO, DK>(p, r, g, h, rb0, nrow, t0, t1 - t0, h % p.group == 0 && blk == 0,
                               64 * waves_per_block, cfirst);
  }
}

// Token-staged variant: the workgroup stages groups of up to kStageTokens tokens
// into LDS before its waves walk them (raw k, q and v loaded once per workgroup;
// unit key, scaled unit query, k^.q^, alpha and beta computed once per token). The
// waves' state loads are issued before the staging, so a short segment (the
// speculative verify) pays one memory latency instead of one per token.
constexpr int kStageTokens = 16;
// Smallest decay product the staged recurrence keeps factored out of its
// registers; below it the product is applied to the state and reset to one.
constexpr float kMinStateScale = 0x1p-40f;

template <int DK>
struct __attribute__((aligned(16))) StageSmem {
  // 16-byte aligned so that a lane's four consecutive floats of kh / qh are one
  // ds_read_b128 (the compiler split them into pairs of 4-byte reads without it)
  float kh[kStageTokens][DK];      // unit keys
  float qh[kStageTokens][DK];      // unit queries times the scale
  float v[kStageTokens][256];      // this block's value rows (at most 4 waves x 64 rows)
  float alpha[kStageTokens], beta[kStageTokens], kq[kStageTokens];
};

// For the verify with fp16 I/O at Dk = 128 a token group's raw inputs come into
// LDS by direct loads that one wave issues before its state loads: k, q (a
// 256-byte row each), the block's value rows (a 256-byte window) and the raw
// gates. They complete ahead of the state, so the normalisation runs while the
// state is in flight and no register holds a staged value across the state loads
// (verify 18.1 -> 17.1 us).
template <int DK>
struct StageSmemDma : StageSmem<DK> {
  _Float16 rawk[kStageTokens][128];
  _Float16 rawq[kStageTokens][128];
  _Float16 rawv[kStageTokens][128];
  float rawa[64], rawb[64];
};
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void lds_dma16(rsrc_t r, void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4(rsrc_t r, void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voffset, 0, 0, 0);
}

template <typename IO, int DK, int NI, bool CAPTURE, bool REPLAY>
__device__ __forceinline__ void recurrent_body_staged(const RecurrentArgs& p, int waves_per_block,
                                                      int blocks_per_head) {
  using L = RecLayout<DK>;
  constexpr int LPR = L::LPR, E = L::E, V4 = L::V4, RI = L::RI, RW = RI * NI;
  static_assert(NI <= LPR, "a lane group writes its NI rows with one lane each");
  constexpr int TPT = 16;                 // threads per staged token
  constexpr int EPT = DK / TPT;           // elements per staging thread
  // (the fused replay keeps the plain staging: with both its registers exceed
  // three waves per SIMD, and capped there it was no faster)
  constexpr bool kDma = std::is_same<IO, _Float16>::value && DK == 128 && !REPLAY;
  __shared__ std::conditional_t<kDma, StageSmemDma<DK>, StageSmem<DK>> sm;

  const int tid = threadIdx.x;
  // the workgroup size from the argument: blockDim.x is a load from the dispatch
  // packet, and its wait would also wait for the state loads in flight
  const int nthreads = 64 * waves_per_block;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPR;
  const int c = lane % LPR;

  int item = blockIdx.x;
  const int blk = item % blocks_per_head;
  item /= blocks_per_head;
  const int h = item % p.Hv;
  const int r = item / p.Hv;
  const int g = h / p.group;
  const int Dv = p.Dv;
  const int block_row0 = blk * waves_per_block * RW;
  const int block_rows = waves_per_block * RW;
  const int row_base = block_row0 + wave * RW;

  const int t0 = seq_start(p, r);
  const int t1 = max(seq_start(p, r + 1), t0);
  const float* init = state_head(p.initial_state, state_slot(p.initial_slots, r, p.num_slots), p.Hv, h,
                                (size_t)Dv * DK);
  float* fin = state_head(p.final_state, state_slot(p.final_slots, r, p.num_slots), p.Hv, h, (size_t)Dv * DK);

  const bool gated = p.gated != 0, delta = p.delta != 0;
  // raw inputs of the group of tokens ts .. ts + nt - 1 into LDS (wave 0; tokens
  // past nt read zero, past the ranges)
  auto issue_dma = [&](int ts, int nt) {
    if constexpr (kDma) {
      if (wave != 0 || nt <= 0) return;
      const int kbytes = ((nt - 1) * p.Hk * DK + DK) * 2;
      const rsrc_t rk = make_rsrc(static_cast<const _Float16*>(p.k) + ((size_t)ts * p.Hk + g) * DK, kbytes);
      const rsrc_t rq = make_rsrc(static_cast<const _Float16*>(p.q) + ((size_t)ts * p.Hk + g) * DK, kbytes);
      const rsrc_t rv = make_rsrc(static_cast<const _Float16*>(p.v) + ((size_t)ts * p.Hv + h) * Dv + block_row0,
                                  ((nt - 1) * p.Hv * Dv + (Dv - block_row0)) * 2);
      // four tokens per load: lane l takes 16 bytes of token 4 i + l / 16
      for (int i = 0; i < (nt + 3) / 4; ++i) {
        const int j = 4 * i + (lane >> 4);
        lds_dma16(rk, &sm.rawk[4 * i][0], j * p.Hk * DK * 2 + 16 * (lane & 15));
        lds_dma16(rq, &sm.rawq[4 * i][0], j * p.Hk * DK * 2 + 16 * (lane & 15));
        lds_dma16(rv, &sm.rawv[4 * i][0], j * p.Hv * Dv * 2 + 16 * (lane & 15));
      }
      if (gated) lds_dma4(make_rsrc(p.a + (size_t)ts * p.Hv + h, ((nt - 1) * p.Hv + 1) * 4), sm.rawa, lane * p.Hv * 4);
      if (delta) lds_dma4(make_rsrc(p.b + (size_t)ts * p.Hv + h, ((nt - 1) * p.Hv + 1) * 4), sm.rawb, lane * p.Hv * 4);
    }
  };
  issue_dma(t0, min(kStageTokens, t1 - t0));
  int m_rep = 0;
  if constexpr (REPLAY) m_rep = min(max(p.accepted[r], 0), p.capacity);
  // the state loads stay behind the direct loads (the waits below count on it)
  if constexpr (kDma) __builtin_amdgcn_sched_barrier(0);

  // ---- state rows into registers (issued before any other staging)
  float S[NI][E];
  bool valid[NI];
  // The verify walks a lane group's rows in NP passes of NH rows. Only the
  // first pass's state is loaded here; the second pass's loads go out once the
  // first token group is staged and land while the first pass computes (the
  // whole grid is resident at once, so without this every wave would wait for
  // all of its state before its first token). The replaying kernel keeps one
  // pass: its replay and the replayed-state stores need every row first.
  constexpr int NP = (!REPLAY && NI % 2 == 0 && NI >= 4) ? 2 : 1;
  constexpr int NH = NI / NP;
  load_state_rows<DK, NI, 0, NH>(init, p.q, row_base, rg, c, Dv, S, valid);
  if constexpr (kDma) __builtin_amdgcn_sched_barrier(0);

  // the previous step's accepted capsule prefix, applied in registers with the
  // arithmetic of gdn_replay (S = alpha S + u k^, one fused multiply-add of
  // alpha S onto the product u k^ per element), then the result to the inactive
  // bank: replay_state equals what gdn_replay writes, bit for bit. With the
  // direct-load staging it runs after the normalisation, which it would
  // otherwise hold behind the state loads.
  // the previous step's accepted capsule prefix, applied in registers with the
  // arithmetic of gdn_replay (S = alpha S + u k^, one fused multiply-add of
  // alpha S onto the product u k^ per element): replay_state equals what
  // gdn_replay writes, bit for bit. Its loads follow the state loads, and it
  // runs as soon as they land (the staged tokens are then in LDS already).
  if constexpr (REPLAY) {
    const float* caprow = p.replay_capsule + (size_t)r * p.capacity * p.capsule_width;
    for (int j = 0; j < m_rep; ++j, caprow += p.capsule_width) {
      const float alpha = caprow[h];
      float kv[E];
#pragma unroll
      for (int jj = 0; jj < V4; ++jj)
#pragma unroll
        for (int x = 0; x < 4; ++x) kv[4 * jj + x] = caprow[p.Hv + g * DK + 4 * c + 4 * LPR * jj + x];  // rows of W floats need not be 16-byte aligned
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = row_base + i * RI + rg;
        const float u = valid[i] ? caprow[p.Hv + p.Hk * DK + h * Dv + row] : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) S[i][e] = fmaf(alpha, S[i][e], u * kv[e]);
      }
    }
  }
  // The replayed state goes to the inactive bank once the first token group is
  // staged: stores count with the loads in the wave's memory counter, so stores
  // issued before the staging loads would make the staging wait for them.
  auto store_replayed = [&]() {
    // the replayed state's slot: the write slot with pools (none: not written)
    float* dst = state_head(p.replay_state, state_slot(p.final_slots, r, p.num_slots), p.Hv, h,
                            (size_t)Dv * DK);
    if (dst == nullptr) return;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!valid[i]) continue;
      const int row = row_base + i * RI + rg;
#pragma unroll
      for (int j = 0; j < V4; ++j)
        store_state4(dst + (size_t)row * DK + 4 * c + 4 * LPR * j,
                     float4_t{S[i][4 * j + 0], S[i][4 * j + 1], S[i][4 * j + 2], S[i][4 * j + 3]});
    }
  };

  const bool gnone = p.gate_none != 0;             // A_log, dt_bias may be null then
  const float expA = (gnone || !gated) ? 0.f : expf(p.A_log[h]);
  const float dtb = (gnone || !gated) ? 0.f : p.dt_bias[h];
  const IO* __restrict__ qp = static_cast<const IO*>(p.q);
  const IO* __restrict__ kp = static_cast<const IO*>(p.k);
  const IO* __restrict__ vp = static_cast<const IO*>(p.v);
  IO* __restrict__ op = static_cast<IO*>(p.output);
  float* __restrict__ cap = p.state_update;

  int ncap = 0;
  if constexpr (CAPTURE) {
    int cmax = p.capacity;
    if (p.capture_count != nullptr) cmax = min(max(p.capture_count[r], 0), p.capacity);
    ncap = min(t1 - t0, cmax);
  }

  // The registers hold S / gam: a token's decay then folds into gam and the
  // update is one fused multiply-add per element, S/gam += (u/gam) k^. Each pass
  // keeps its own gam (both see the same gates, so they agree).
  float gam_p[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) gam_p[q] = 1.f;
  // One token group; the first is called outside the loop, so that the compiler's
  // flush of the memory counter at the entry of a loop that reads the state comes
  // only after that group's staging.
  auto group = [&](int ts) {
    const int nt = min(kStageTokens, t1 - ts);
    if constexpr (kDma) {
      // the group's raw inputs are in LDS once wave 0's direct loads land: for the
      // first group they precede exactly NH V4 state loads (the first pass's), so
      // waiting until no more than those are pending leaves the state in flight
      if (ts != t0) issue_dma(ts, nt);
      if (ts == t0) {
        constexpr int kState = NH * V4;
        static_assert(kState < 64, "vmcnt holds 6 bits");
        __builtin_amdgcn_s_waitcnt((kState & 15) | (7 << 4) | (15 << 8) | ((kState >> 4) << 14));
      } else {
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));      // vmcnt(0)
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    // ---- stage: 16 threads per token normalise k and q and form the gates (a
    // workgroup of fewer than four waves takes several passes)
    for (int j = tid / TPT; j < nt; j += nthreads / TPT) {
      const int part = tid % TPT;
      {
        const int t = ts + j;
        float kv[EPT], qv[EPT];
        if constexpr (kDma) {
          static_assert(EPT == 8, "one 16-byte LDS read per thread");
          const half8_t k8 = *reinterpret_cast<const half8_t*>(&sm.rawk[j][part * EPT]);
          const half8_t q8 = *reinterpret_cast<const half8_t*>(&sm.rawq[j][part * EPT]);
#pragma unroll
          for (int e = 0; e < EPT; ++e) {
            kv[e] = (float)k8[e];
            qv[e] = (float)q8[e];
          }
        } else {
          const IO* krow = kp + ((size_t)t * p.Hk + g) * DK + part * EPT;
          const IO* qrow = qp + ((size_t)t * p.Hk + g) * DK + part * EPT;
#pragma unroll
          for (int e = 0; e < EPT; ++e) {
            kv[e] = IoOps<IO>::load1(krow + e);
            qv[e] = IoOps<IO>::load1(qrow + e);
          }
        }
        float ssk = 0.f, ssq = 0.f, skq = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          ssk = fmaf(kv[e], kv[e], ssk);
          ssq = fmaf(qv[e], qv[e], ssq);
          skq = fmaf(kv[e], qv[e], skq);
        }
        ssk = group_sum<TPT>(ssk);
        ssq = group_sum<TPT>(ssq);
        skq = group_sum<TPT>(skq);
        const float rk = rsqrtf(ssk + kNormEps);
        const float rq = rsqrtf(ssq + kNormEps) * p.scale;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          sm.kh[j][part * EPT + e] = kv[e] * rk;
          sm.qh[j][part * EPT + e] = qv[e] * rq;
        }
        if (part == 0) {
          float ra = 0.f, rb = 0.f;
          if constexpr (kDma) {
            ra = sm.rawa[j];
            rb = sm.rawb[j];
          } else {
            if (gated) ra = p.a[(size_t)t * p.Hv + h];
            if (delta) rb = p.b[(size_t)t * p.Hv + h];
          }
          sm.alpha[j] = gated ? gate_alpha(ra, gnone, expA, dtb) : 1.f;
          sm.beta[j] = delta ? gate_beta(rb, gnone) : 1.f;
          sm.kq[j] = skq * rk * rq;
        }
      }   // a token's 16 lanes are one aligned DPP row group: active or idle together
    }
    // this block's value rows of every staged token
    for (int idx = tid; idx < nt * block_rows; idx += nthreads) {
      const int jj = idx / block_rows, rr = idx % block_rows;
      const int row = block_row0 + rr;
      if constexpr (kDma)
        sm.v[jj][rr] = row < Dv ? (float)sm.rawv[jj][rr] : 0.f;
      else
        sm.v[jj][rr] = row < Dv ? IoOps<IO>::load1(vp + ((size_t)(ts + jj) * p.Hv + h) * Dv + row) : 0.f;
    }
    __syncthreads();
    if constexpr (REPLAY) {
      if (ts == t0) store_replayed();              // the registers hold the replayed state
    }

    // one pass over the group's tokens for the rows I0 .. I1 - 1 of each lane group
    auto walk = [&](auto pc) {
      constexpr int PASS = decltype(pc)::value, I0 = PASS * NH, I1 = I0 + NH;
      float& gam = gam_p[PASS];
      for (int j = 0; j < nt; ++j) {
        const int t = ts + j;
        float kv[E], qv[E];
#pragma unroll
        for (int jj = 0; jj < V4; ++jj) {
          const float4_t kx = *reinterpret_cast<const float4_t*>(&sm.kh[j][4 * c + 4 * LPR * jj]);
          const float4_t qx = *reinterpret_cast<const float4_t*>(&sm.qh[j][4 * c + 4 * LPR * jj]);
          kv[4 * jj + 0] = kx.x; kv[4 * jj + 1] = kx.y; kv[4 * jj + 2] = kx.z; kv[4 * jj + 3] = kx.w;
          qv[4 * jj + 0] = qx.x; qv[4 * jj + 1] = qx.y; qv[4 * jj + 2] = qx.z; qv[4 * jj + 3] = qx.w;
        }
        const float beta = sm.beta[j], kq = sm.kq[j];
        // decay of the held state up to and including this token
        const float gn = gam * sm.alpha[j];
        const bool keep_scaled = gn >= kMinStateScale;   // uniform over the workgroup
        float pk[NI], pq[NI];
#pragma unroll
        for (int i = I0; i < I1; ++i) {
          float sk = 0.f, sq = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            sk = fmaf(S[i][e], kv[e], sk);
            sq = fmaf(S[i][e], qv[e], sq);
          }
          pk[i] = sk;
          pq[i] = sq;
        }
#pragma unroll
        for (int i = I0; i < I1; ++i) {
          pk[i] = group_sum<LPR>(pk[i]);
          pq[i] = group_sum<LPR>(pq[i]);
        }
        const int jcap = t - t0;
        float* caprow = nullptr;
        if constexpr (CAPTURE) {
          if (jcap < ncap) caprow = cap + ((size_t)r * p.capacity + jcap) * p.capsule_width;
        }
        // the state's scale is reset (one in-place multiply) only when the
        // product would leave the range where 1/gam is safe
        const float rgn = keep_scaled ? __builtin_amdgcn_rcpf(gn) : 1.f;
        // u = beta (v - alpha S k^) with the delta correction, v without it
        const float gk = delta ? gn : 0.f;
        float u[NI];
#pragma unroll
        for (int i = I0; i < I1; ++i) {
          const float vv = sm.v[j][row_base + i * RI + rg - block_row0];   // zero past Dv
          u[i] = beta * (vv - gk * pk[i]);
        }
        // the state after the segment's last token is used only as a final state
        // (the verify asks for none)
        if (t + 1 < t1 || fin != nullptr) {          // uniform over the workgroup
          if (!keep_scaled) {
#pragma unroll
            for (int i = I0; i < I1; ++i)
#pragma unroll
              for (int e = 0; e < E; ++e) S[i][e] *= gn;
          }
#pragma unroll
          for (int i = I0; i < I1; ++i) {
            const float w = u[i] * rgn;
#pragma unroll
            for (int e = 0; e < E; ++e) S[i][e] = fmaf(w, kv[e], S[i][e]);
          }
        }
        // One store per token for the NI rows of a lane group: every lane of the group
        // holds every row's total, and lane c < NI writes row c. The stores are range
        // checked against the head's Dv rows, so lanes c >= NI (sent past the range)
        // and rows past Dv write nothing, without a branch per row.
        {
          float o_c = 0.f, u_c = 0.f;
#pragma unroll
          for (int i = I0; i < I1; ++i) {
            const float o = fmaf(gn, pq[i], u[i] * kq);
            o_c = c == i ? o : o_c;
            u_c = c == i ? u[i] : u_c;
          }
          const int row_c = (c >= I0 && c < I1) ? row_base + c * RI + rg : Dv;
          const rsrc_t ro = make_rsrc(op + ((size_t)t * p.Hv + h) * Dv, Dv * (int)sizeof(IO));
          if constexpr (sizeof(IO) == 2)
            buf_store_h1((_Float16)o_c, ro, row_c * 2);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, o_c), ro, row_c * 4, 0, 0);
          if constexpr (CAPTURE) {
            if (caprow != nullptr)                   // uniform over the workgroup
              __builtin_amdgcn_raw_buffer_store_b32(
                  __builtin_bit_cast(unsigned, u_c), make_rsrc(caprow + p.Hv + p.Hk * DK + h * Dv, Dv * 4),
                  row_c * 4, 0, 0);
          }
        }
        if constexpr (CAPTURE && PASS == 0) {
          if (caprow != nullptr && blk == 0 && wave == 0) {
            if (lane == 0) caprow[h] = sm.alpha[j];
            // the shared key is written once per key head, by its first value head
            if (h % p.group == 0 && rg == 0) {
#pragma unroll
              for (int jj = 0; jj < V4; ++jj)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                  caprow[p.Hv + g * DK + 4 * c + 4 * LPR * jj + x] = kv[4 * jj + x];
            }
          }
        }
        gam = keep_scaled ? gn : 1.f;
      }
    };
    if constexpr (NP == 2) {
      if (ts == t0) {
        __builtin_amdgcn_sched_barrier(0);
        load_state_rows<DK, NI, NH, NH>(init, p.q, row_base, rg, c, Dv, S, valid);
        // wait for everything but these loads: the first pass's loop then reads
        // no register with a load in flight, and the compiler does not drain the
        // memory counter (the second pass's loads with it) at its entry
        constexpr int kB = NH * V4;
        static_assert(kB < 64, "vmcnt holds 6 bits");
        __builtin_amdgcn_s_waitcnt((kB & 15) | (7 << 4) | (15 << 8) | ((kB >> 4) << 14));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    walk(std::integral_constant<int, 0>());
    if constexpr (NP == 2) walk(std::integral_constant<int, 1>());
    __syncthreads();   // the next group's staging overwrites the staged tokens
  };
  if (t1 > t0) group(t0);
  for (int ts = t0 + kStageTokens; ts < t1; ts += kStageTokens) group(ts);
  if constexpr (NP == 2) {
    // no tokens: the second half is loaded only here, for the final state
    if (t1 == t0) load_state_rows<DK, NI, NH, NH>(init, p.q, row_base, rg, c, Dv, S, valid);
  }
  if constexpr (REPLAY) {
    if (t1 == t0) store_replayed();                // no tokens: the replayed state as it is
  }

  if (fin != nullptr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!valid[i]) continue;
      const int row = row_base + i * RI + rg;
      const float gam = gam_p[i / NH];
#pragma unroll
      for (int j = 0; j < V4; ++j) {
        float4_t x = {gam * S[i][4 * j + 0], gam * S[i][4 * j + 1], gam * S[i][4 * j + 2],
                      gam * S[i][4 * j + 3]};
        store_state4(fin + (size_t)row * DK + 4 * c + 4 * LPR * j, x);
      }
    }
  }
}

// Distinct kernel names for the profiler: gdn_decode (no capture), gdn_conv_decode
// (the causal convolution fused in), gdn_capsule.
template <typename IO, int DK, int NI>
__global__ void __launch_bounds__(64 * GDN_REC_WAVES) gdn_decode(RecurrentArgs p, int wpb, int bph) {
  recurrent_body<IO, DK, NI, false>(p, wpb, bph);
}
template <typename IO, int DK, int NI>
__global__ void __launch_bounds__(64 * GDN_REC_WAVES) gdn_conv_decode(RecurrentArgs p, int wpb, int bph) {
  recurrent_body<IO, DK, NI, false, true>(p, wpb, bph);
}
template <typename IO, int DK, int NI>
__global__ void __launch_bounds__(64 * GDN_REC_WAVES) gdn_capsule(RecurrentArgs p, int wpb, int bph) {
  recurrent_body_staged<IO, DK, NI, true, false>(p, wpb, bph);
}
// gdn_capsule preceded by the replay of the previous step's accepted prefix
// (gdn_replay_forward): one read of the committed state for both.
template <typename IO, int DK, int NI>
__global__ void __launch_bounds__(64 * GDN_REC_WAVES) gdn_replay_verify(RecurrentArgs p, int wpb, int bph) {
  recurrent_body_staged<IO, DK, NI, true, true>(p, wpb, bph);
}

template <int DK, int NI>
static void launch_shape(int Dv, int* wpb, int* bph) {
  constexpr int RW = RecLayout<DK>::RI * NI;
  const int waves_needed = (Dv + RW - 1) / RW;
  *wpb = waves_needed < GDN_REC_WAVES ? waves_needed : GDN_REC_WAVES;
  *bph = (Dv + *wpb * RW - 1) / (*wpb * RW);
}

template <typename IO, int DK, int NI, int NI_CAP>
static hipError_t launch_dk(const RecurrentArgs& p, hipStream_t stream) {
  int wpb, bph;
  if (p.state_update != nullptr) {
    launch_shape<DK, NI_CAP>(p.Dv, &wpb, &bph);
    if (p.replay_capsule != nullptr)
      hipLaunchKernelGGL((gdn_replay_verify<IO, DK, NI_CAP>), dim3((unsigned)((size_t)p.R * p.Hv * bph)),
                         dim3((unsigned)(64 * wpb)), 0, stream, p, wpb, bph);
    else
      hipLaunchKernelGGL((gdn_capsule<IO, DK, NI_CAP>), dim3((unsigned)((size_t)p.R * p.Hv * bph)),
                         dim3((unsigned)(64 * wpb)), 0, stream, p, wpb, bph);
  } else {
    launch_shape<DK, NI>(p.Dv, &wpb, &bph);
    if (p.conv_channels > 0) {
      // whole rounds of 8 (request, key head) units, see recurrent_body
      const size_t units = 8 * (((size_t)p.R * p.Hk + 7) / 8);
      hipLaunchKernelGGL((gdn_conv_decode<IO, DK, NI>), dim3((unsigned)(units * p.group * bph)),
                         dim3((unsigned)(64 * wpb)), 0, stream, p, wpb, bph);
    }
    else
      hipLaunchKernelGGL((gdn_decode<IO, DK, NI>), dim3((unsigned)((size_t)p.R * p.Hv * bph)),
                         dim3((unsigned)(64 * wpb)), 0, stream, p, wpb, bph);
  }
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_io(const RecurrentArgs& p, hipStream_t stream) {
  switch (p.Dk) {
    case 16: return launch_dk<IO, 16, 1, 1>(p, stream);
    case 32: return launch_dk<IO, 32, 2, 2>(p, stream);
    case 64: return launch_dk<IO, 64, 2, 2>(p, stream);
    case 128: return launch_dk<IO, 128, GDN_REC_NI128, GDN_CAP_NI128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_recurrent(const RecurrentArgs& p, int io_dtype, hipStream_t stream) {
  if (p.R == 0) return hipSuccess;
  return io_dtype == 1 ? launch_io<_Float16>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace gdn

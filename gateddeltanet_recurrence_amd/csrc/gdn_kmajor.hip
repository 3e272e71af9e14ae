// Token-recurrent GatedDeltaNet kernels for the K-major state layout:
// gdn_decode_kmajor and gdn_capsule_kmajor.
//
// The dense LinearAttention path keeps its recurrent state K-major,
// [B, heads, key_dim, value_dim], where the packed GatedDeltaNet path keeps it
// V-major (first page, Copilot review of the builder). The matrix per head is
// M = S^T (Dk rows of Dv contiguous floats), and the gated delta rule reads
//   pk = M^T k^, pq = M^T q^,  u = beta (v - alpha pk),  o = alpha pq + u (k^ . q^),
//   M = alpha M + k^ u^T.
//
// Work decomposition (CDNA4, wave64). A slice of 4 LK value columns of one
// (request, value head) is held in registers for the whole segment by DKS
// wavefronts, each with Dk / DKS of its rows: lane l holds the 4 columns
// 4 (l mod LK) .. +3 (one 16-byte vector, so LK adjacent lanes read a 16 LK-byte
// run of a row) in the NR consecutive rows dk = dk0 + NR (l / LK) + i, so that
// the lane's k and q values are one vector load each. The contraction over dk
// is an in-lane sum over the lane's rows, a sum over the lanes of equal
// l mod LK (DPP rotations within each row of 16 lanes, two cross-row
// exchanges), and with DKS = 2 the partner wavefront's partial sums through
// LDS; the update M = alpha M + k^ u^T is lane-local. LK = 8 (full 128-byte
// lines per row segment) took the batched decode from 69 us (LK = 4, 64-byte
// segments) to 51 us; DKS = 2 at Dk = 128 (104 VGPRs, four waves per SIMD,
// against 150 and three) to 49.5 us; range-checked loads with no branch around
// them (every load issued before the first wait) to 48.1 us.
#include "gdn_common.h"
#include "gdn_kernels.h"

#ifndef GDN_KMAJ_WAVES
#define GDN_KMAJ_WAVES 4
#endif
// Lanes per state row segment: a wavefront owns 4 * GDN_KMAJ_LANES value columns.
#ifndef GDN_KMAJ_LANES
#define GDN_KMAJ_LANES 8
#endif

namespace gdn {

namespace {

constexpr int kDppRowRor4 = 0x124;    // row_ror:4 within a row of 16 lanes
constexpr int kDppRowRor8 = 0x128;    // row_ror:8

// x[l] + x[l ^ 16] and x[l] + x[l ^ 32] on the VALU: v_permlane16_swap exchanges
// the odd 16-lane rows of one register with the even rows of another, and
// v_permlane32_swap the upper half of one with the lower half of the other. With
// x in both, every lane holds the two values of its pair, one in each result;
// their sum is the pair's sum in every lane (a + b = b + a exactly).
__device__ __forceinline__ float swap16_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the lanes of each class l mod LK (LK = 4 or 8 lanes per row
// segment); every lane gets its class total. All 64 lanes must be active. Only
// DPP and lane swaps: no LDS permutes.
template <int LK>
__device__ __forceinline__ float column_sum(float x) {
  if constexpr (LK == 4) x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  x = swap16_sum(x);
  return swap32_sum(x);
}

__device__ __forceinline__ void store_state4_nt(float* p, float4_t x) {
  __builtin_nontemporal_store(x, reinterpret_cast<float4_t*>(p));
}

// Four consecutive values of a row as floats through a range-checked buffer
// load: past the range they read as zero, so lanes past Dv need no branch.
template <typename IO> struct Io4Buf;
template <> struct Io4Buf<float> {
  static __device__ __forceinline__ float4_t load(rsrc_t r, int byte_off) {
    return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
  }
};
template <> struct Io4Buf<_Float16> {
  static __device__ __forceinline__ float4_t load(rsrc_t r, int byte_off) {
    const half4_t h = buf_load_h4(r, byte_off);
    return float4_t{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
  }
};

template <typename IO> struct Io4Store;
template <> struct Io4Store<float> {
  static __device__ __forceinline__ void store(float* p, float4_t v) { *reinterpret_cast<float4_t*>(p) = v; }
};
template <> struct Io4Store<_Float16> {
  static __device__ __forceinline__ void store(_Float16* p, float4_t v) {
    *reinterpret_cast<half4_t*>(p) = half4_t{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
  }
};

// N consecutive values of a k or q row as floats: 16-byte loads where the run is
// whole 16-byte vectors (q and k are 16-byte aligned and every run starts at a
// multiple of its length), single loads otherwise.
template <typename IO, int N>
__device__ __forceinline__ void load_run(const IO* src, float (&dst)[N]) {
  constexpr int PER16 = 16 / (int)sizeof(IO);
  if constexpr (N % PER16 == 0) {
#pragma unroll
    for (int v = 0; v < N / PER16; ++v) {
      if constexpr (PER16 == 8) {
        const half8_t x = *reinterpret_cast<const half8_t*>(src + 8 * v);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[8 * v + e] = (float)x[e];
      } else {
        const float4_t x = *reinterpret_cast<const float4_t*>(src + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * v + e] = x[e];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = IoOps<IO>::load1(src + i);
  }
}

// Dk rows of a column slice are split over DKS wavefronts (DKS = 2 at Dk = 128:
// 32 state floats per lane instead of 64, five waves per SIMD instead of three).
// The contractions over dk then add the DKS partial sums through LDS, one
// barrier per token; every wave of a slice forms the same totals (the partner's
// sum is added to its own, and a + b = b + a exactly).
template <int DK>
struct KmajSplit {
  static constexpr int DKS = DK == 128 ? 2 : 1;
};

template <typename IO, int DK, bool CAPTURE>
__device__ __forceinline__ void kmajor_body(const RecurrentArgs& p, int waves_per_block, int blocks_per_head) {
  constexpr int LK = GDN_KMAJ_LANES;               // lanes per row segment
  constexpr int WD = 4 * LK;                       // value columns per wavefront
  constexpr int RG = 64 / LK;                      // row groups
  constexpr int DKS = KmajSplit<DK>::DKS;          // wavefronts per column slice
  constexpr int NR = DK / DKS / RG;                // rows per lane
  constexpr int SPB = GDN_KMAJ_WAVES / DKS;        // column slices per workgroup (at most)
  static_assert(NR >= 1, "Dk must cover the row groups");
  // partial sums pk (4), pq (4), |k|^2, |q|^2, k.q (padded to 12), two token buffers
  __shared__ float xsum[DKS > 1 ? 2 : 1][SPB][DKS][LK][12];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cl = lane % LK;                        // column quad within the slice
  const int rg = lane / LK;                        // row group: rows NR rg .. NR rg + NR - 1 of this part
  const int part = wave % DKS;                     // which dk part of the slice
  const int sl = wave / DKS;                       // slice within the workgroup
  const int dk0 = part * (DK / DKS);

  int item = blockIdx.x;
  const int blk = item % blocks_per_head;
  item /= blocks_per_head;
  const int h = item % p.Hv;
  const int r = item / p.Hv;
  const int g = h / p.group;
  const int Dv = p.Dv;
  const int slices_per_block = waves_per_block / DKS;
  const int slice = blk * slices_per_block + sl;
  const bool sactive = slice * WD < Dv;            // idle slices still take part in the barriers
  if constexpr (DKS == 1) {
    if (!sactive) return;                          // no barrier below: idle waves may leave
  }
  const int col = slice * WD + 4 * cl;             // first of this lane's 4 columns
  const bool cvalid = sactive && col < Dv;         // Dv is a multiple of 16, maybe not of WD

  const int t0 = seq_start(p, r);
  const int t1 = max(seq_start(p, r + 1), t0);

  const size_t head_elems = (size_t)Dv * DK;
  const float* init = state_head(p.initial_state, state_slot(p.initial_slots, r, p.num_slots), p.Hv, h, head_elems);
  float* fin = state_head(p.final_state, state_slot(p.final_slots, r, p.num_slots), p.Hv, h, head_elems);

  const int row0 = dk0 + NR * rg;                  // this lane's first state row
  // The state rows come in through range-checked buffer loads over the head's
  // Dk x Dv floats (an empty range without an initial state); a lane past Dv
  // reads from the end of the range, i.e. zeros. With no branch around them the
  // k, q, v and gate loads that follow are issued before any of them is waited
  // for; a branch on the lane's validity had compiled to a wait for every load
  // (the state included) before the gates were even requested.
  const int head_bytes = (int)(head_elems * 4);
  float4_t M[NR];
  {
    const rsrc_t rs = make_rsrc(init != nullptr ? static_cast<const void*>(init) : p.q,
                                init != nullptr ? head_bytes : 0);
    const int lane_off = cvalid ? (row0 * Dv + col) * 4 : head_bytes;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      M[i] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + i * Dv * 4, 0,
                                                                                kBufferNontemporal));
  }

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

  for (int t = t0; t < t1; ++t) {
    float kv[NR], qv[NR];
    load_run<IO, NR>(kp + ((size_t)t * p.Hk + g) * DK + row0, kv);
    load_run<IO, NR>(qp + ((size_t)t * p.Hk + g) * DK + row0, qv);
    const int io = (int)sizeof(IO);
    const float4_t vv = Io4Buf<IO>::load(make_rsrc(vp + ((size_t)t * p.Hv + h) * Dv, Dv * io),
                                         cvalid ? col * io : Dv * io);
    // the gates of an absent rule term read as zero from an empty range
    const size_t gi = (size_t)t * p.Hv + h;
    const float at = buf_load_f32(make_rsrc(gated ? static_cast<const void*>(p.a + gi) : p.q, gated ? 4 : 0), 0);
    const float bt = buf_load_f32(make_rsrc(delta ? static_cast<const void*>(p.b + gi) : p.q, delta ? 4 : 0), 0);

    float ssk = 0.f, ssq = 0.f, skq = 0.f;
    float4_t pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      ssk = fmaf(kv[i], kv[i], ssk);
      ssq = fmaf(qv[i], qv[i], ssq);
      skq = fmaf(kv[i], qv[i], skq);
      pk.x = fmaf(M[i].x, kv[i], pk.x); pk.y = fmaf(M[i].y, kv[i], pk.y);
      pk.z = fmaf(M[i].z, kv[i], pk.z); pk.w = fmaf(M[i].w, kv[i], pk.w);
      pq.x = fmaf(M[i].x, qv[i], pq.x); pq.y = fmaf(M[i].y, qv[i], pq.y);
      pq.z = fmaf(M[i].z, qv[i], pq.z); pq.w = fmaf(M[i].w, qv[i], pq.w);
    }
    // with the raw k and q: pk = M^T k = |k| M^T k^, so the norms scale afterwards
    ssk = column_sum<LK>(ssk);
    ssq = column_sum<LK>(ssq);
    skq = column_sum<LK>(skq);
    pk.x = column_sum<LK>(pk.x); pk.y = column_sum<LK>(pk.y); pk.z = column_sum<LK>(pk.z); pk.w = column_sum<LK>(pk.w);
    pq.x = column_sum<LK>(pq.x); pq.y = column_sum<LK>(pq.y); pq.z = column_sum<LK>(pq.z); pq.w = column_sum<LK>(pq.w);
    if constexpr (DKS > 1) {
      static_assert(DKS == 2, "two dk parts");
      const int buf = (t - t0) & 1;                // the other buffer may still be read by the partner
      if (rg == 0) {
        float* d = xsum[buf][sl][part][cl];
        d[0] = pk.x; d[1] = pk.y; d[2] = pk.z; d[3] = pk.w;
        d[4] = pq.x; d[5] = pq.y; d[6] = pq.z; d[7] = pq.w;
        d[8] = ssk; d[9] = ssq; d[10] = skq;
      }
      __syncthreads();
      const float* o = xsum[buf][sl][part ^ 1][cl];
      pk.x += o[0]; pk.y += o[1]; pk.z += o[2]; pk.w += o[3];
      pq.x += o[4]; pq.y += o[5]; pq.z += o[6]; pq.w += o[7];
      ssk += o[8]; ssq += o[9]; skq += o[10];
    }
    const float rk = rsqrtf(ssk + kNormEps);
    const float rq = rsqrtf(ssq + kNormEps) * p.scale;
    // the rule: alpha = 1 without the gate; u = v (beta 1, no correction) without the delta
    const float alpha = gated ? gate_alpha(at, gnone, expA, dtb) : 1.f;
    const float beta = delta ? gate_beta(bt, gnone) : 1.f;
    const float kq = skq * rk * rq;                // k^ . q^
    const float ak = (delta ? alpha : 0.f) * rk, aq = alpha * rq;

    float4_t u, o;
    u.x = beta * fmaf(-ak, pk.x, vv.x); u.y = beta * fmaf(-ak, pk.y, vv.y);
    u.z = beta * fmaf(-ak, pk.z, vv.z); u.w = beta * fmaf(-ak, pk.w, vv.w);
    o.x = fmaf(aq, pq.x, u.x * kq); o.y = fmaf(aq, pq.y, u.y * kq);
    o.z = fmaf(aq, pq.z, u.z * kq); o.w = fmaf(aq, pq.w, u.w * kq);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float kh = kv[i] * rk;
      M[i].x = fmaf(alpha, M[i].x, kh * u.x); M[i].y = fmaf(alpha, M[i].y, kh * u.y);
      M[i].z = fmaf(alpha, M[i].z, kh * u.z); M[i].w = fmaf(alpha, M[i].w, kh * u.w);
    }
    if (part == 0 && rg == 0 && cvalid) Io4Store<IO>::store(op + ((size_t)t * p.Hv + h) * Dv + col, o);

    if constexpr (CAPTURE) {
      const int jcap = t - t0;
      if (jcap < ncap) {
        float* caprow = p.state_update + ((size_t)r * p.capacity + jcap) * p.capsule_width;
        if (part == 0 && rg == 0 && cvalid) {
          float* d = caprow + p.Hv + p.Hk * DK + h * Dv + col;
          d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
        }
        if (slice == 0) {
          if (part == 0 && lane == 0) caprow[h] = alpha;
          // the shared key is written once per key head, by its first value head
          if (h % p.group == 0 && cl == 0) {
#pragma unroll
            for (int i = 0; i < NR; ++i) caprow[p.Hv + g * DK + row0 + i] = kv[i] * rk;
          }
        }
      }
    }
  }

  if (fin != nullptr && cvalid) {
#pragma unroll
    for (int i = 0; i < NR; ++i) store_state4_nt(fin + (size_t)(row0 + i) * Dv + col, M[i]);
  }
}

}  // namespace

template <typename IO, int DK>
__global__ void __launch_bounds__(64 * GDN_KMAJ_WAVES) gdn_decode_kmajor(RecurrentArgs p, int wpb, int bph) {
  kmajor_body<IO, DK, false>(p, wpb, bph);
}
template <typename IO, int DK>
__global__ void __launch_bounds__(64 * GDN_KMAJ_WAVES) gdn_capsule_kmajor(RecurrentArgs p, int wpb, int bph) {
  kmajor_body<IO, DK, true>(p, wpb, bph);
}

template <typename IO, int DK>
static hipError_t launch_kmajor_dk(const RecurrentArgs& p, hipStream_t stream) {
  constexpr int DKS = KmajSplit<DK>::DKS;
  constexpr int SPB = GDN_KMAJ_WAVES / DKS;
  const int slices = (p.Dv + 4 * GDN_KMAJ_LANES - 1) / (4 * GDN_KMAJ_LANES);
  const int spb = slices < SPB ? slices : SPB;
  const int wpb = spb * DKS;
  const int bph = (slices + spb - 1) / spb;
  const dim3 grid((unsigned)((size_t)p.R * p.Hv * bph)), block((unsigned)(64 * wpb));
  if (p.state_update != nullptr)
    hipLaunchKernelGGL((gdn_capsule_kmajor<IO, DK>), grid, block, 0, stream, p, wpb, bph);
  else
    hipLaunchKernelGGL((gdn_decode_kmajor<IO, DK>), grid, block, 0, stream, p, wpb, bph);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_kmajor_io(const RecurrentArgs& p, hipStream_t stream) {
  switch (p.Dk) {
    case 16: return launch_kmajor_dk<IO, 16>(p, stream);
    case 32: return launch_kmajor_dk<IO, 32>(p, stream);
    case 64: return launch_kmajor_dk<IO, 64>(p, stream);
    case 128: return launch_kmajor_dk<IO, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_recurrent_kmajor(const RecurrentArgs& p, int io_dtype, hipStream_t stream) {
  if (p.R == 0) return hipSuccess;
  return io_dtype == 1 ? launch_kmajor_io<_Float16>(p, stream) : launch_kmajor_io<float>(p, stream);
}

}  // namespace gdn

// Chunked prefill of the gated delta rule on fp16 MFMA (gfx950): gdn_chunk_prefill.
//
// The tensor-core chunked prefill path of "[CUDA] Add compact GatedDeltaNet
// operator" (Description), rebuilt for CDNA4: chunk C = 64, an intra-chunk
// UT/WY transform and the state passing on v_mfma_f32_16x16x32_f16 with FP32
// accumulation; the inter-chunk state is carried in FP32.
//
// Per sequence, chunks start at the sequence's first token (the last one may be
// short, length L <= 64). For one chunk and value head h (key head g = h / G),
// with k^ = rk k, q^ = rq q (rq includes the query scale), g_t the in-chunk
// cumulative log decay and S0 the state entering the chunk:
//   A[r,i] = beta_r e^{g_r - g_i} k^_r.k^_i  (i < r),   T = (I + A)^-1
//   P[r,i] = e^{g_r - g_i} q^_r.k^_i         (i <= r)
//   X = K S0^T,  Y = Q S0^T                              (raw fp16 k, q)
//   Z = diag(beta) (V - diag(e^g rk) X),   U = T Z       (U rows: the deltas u_t)
//   O = diag(e^g rq) Y + P U
//   S = e^{g_L} S0 + (diag(e^{g_L - g} rk) U)^T K
// Everything that does not depend on S0 (Gram matrices, T, P, gates, norms) is
// chunk-parallel and done first by gdn_chunk_prep; gdn_chunk_scan then walks
// the chunks of each sequence in order. The rows of S evolve independently,
// so the scan splits every head's state into Dv tiles of TV rows, one
// workgroup each: the serial chain is spread over heads x tiles workgroups.
//
// Kernels: gdn_chunk_index (chunk offsets per sequence), gdn_chunk_prep,
// gdn_chunk_scan. Dk = Dv = 128, fp16 I/O only.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C = kChunk;     // 64 tokens per chunk
constexpr int D = 128;        // Dk = Dv
constexpr int KS = D + 8;     // LDS row stride (halves) of 128-wide fp16 tiles
constexpr int TS = C + 8;     // LDS row stride (halves) of 64-wide fp16 tiles
constexpr int AS = C + 4;     // LDS row stride (floats) of the fp32 A matrix
constexpr int kThreads = 256;

__device__ __forceinline__ float4_t mfma_f16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// e^x on the hardware exp2 (about 1 ulp); used where the result is stored at
// fp16 or enters a product already rounded to fp16.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ half8_t lds8(const _Float16* p) {
  return *reinterpret_cast<const half8_t*>(p);
}

// Workspace layout: chunk offsets, then per (slot, value head) T and P (fp16
// 64x64 row-major) and the per-token factors the scan applies (fp32 rows of 64):
//   kVecZ  e^{g_t} rk_t            kVecBeta beta_t
//   kVecO  e^{g_t} rq_t            kVecU    e^{g_L - g_t} rk_t
//   kVecGamma  element 0: e^{g_L}, the decay of the whole chunk
constexpr int kVecZ = 0, kVecBeta = 1, kVecO = 2, kVecU = 3, kVecGamma = 4, kVecRows = 5;

struct Ws {
  int32_t* chunk_start;
  _Float16* T;
  _Float16* P;
  float* vec;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Ws ws_layout(void* base, int64_t slots, int R, int Hk, int Hv) {
  char* p = static_cast<char*>(base);
  Ws w;
  size_t off = 0;
  w.chunk_start = reinterpret_cast<int32_t*>(p + off);
  off += align256((size_t)(R + 1) * 4);
  w.T = reinterpret_cast<_Float16*>(p + off);
  off += align256((size_t)slots * Hv * C * C * 2);
  w.P = reinterpret_cast<_Float16*>(p + off);
  off += align256((size_t)slots * Hv * C * C * 2);
  w.vec = reinterpret_cast<float*>(p + off);
  return w;
}

__host__ inline size_t ws_bytes(int64_t slots, int R, int Hk, int Hv) {
  (void)Hk;
  return align256((size_t)(R + 1) * 4) + 2 * align256((size_t)slots * Hv * C * C * 2) +
         align256((size_t)slots * Hv * kVecRows * C * 4);
}

__device__ __forceinline__ int clamp_cu(const int32_t* cu, int i, int N) {
  return min(max(cu[i], 0), N);
}

}  // namespace

// ----------------------------------------------------------------------------
// chunk offsets: chunk_start[r] = sum_{i<r} ceil(len_i / 64), chunk_start[R] = total
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) gdn_chunk_index(ChunkArgs p, Ws w) {
  __shared__ int part[kThreads];
  const int tid = threadIdx.x;
  const int per = (p.R + kThreads - 1) / kThreads;
  const int r0 = min(tid * per, p.R), r1 = min(r0 + per, p.R);
  int prev = clamp_cu(p.cu_seqlens, r0, p.N);
  int sum = 0;
  for (int r = r0; r < r1; ++r) {
    const int nxt = max(clamp_cu(p.cu_seqlens, r + 1, p.N), prev);
    sum += (nxt - prev + C - 1) / C;
    prev = nxt;
  }
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 256 partial sums (Hillis-Steele)
  for (int d = 1; d < kThreads; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  prev = clamp_cu(p.cu_seqlens, r0, p.N);
  for (int r = r0; r < r1; ++r) {
    w.chunk_start[r] = run;
    const int nxt = max(clamp_cu(p.cu_seqlens, r + 1, p.N), prev);
    run += (nxt - prev + C - 1) / C;
    prev = nxt;
  }
  if (tid == kThreads - 1) w.chunk_start[p.R] = part[kThreads - 1];
}

// Locates (request, first token, length) of a chunk slot; false past the end.
__device__ __forceinline__ bool locate_chunk(const ChunkArgs& p, const Ws& w, int slot, int* req,
                                             int* t0, int* len) {
  const int total = min(w.chunk_start[p.R], p.max_chunks);
  if (slot >= total) return false;
  int lo = 0, hi = p.R - 1;                 // last r with chunk_start[r] <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (w.chunk_start[mid] <= slot) lo = mid; else hi = mid - 1;
  }
  const int beg = clamp_cu(p.cu_seqlens, lo, p.N);
  const int end = max(clamp_cu(p.cu_seqlens, lo + 1, p.N), beg);
  *req = lo;
  *t0 = beg + C * (slot - w.chunk_start[lo]);
  *len = min(C, end - *t0);
  return *len > 0;
}

// ----------------------------------------------------------------------------
// gdn_chunk_prep: one workgroup per (chunk slot, key head)
//
// T = (I + A)^-1 of every value head is built blockwise from 16x16 blocks:
// the four diagonal blocks by forward substitution (one lane per column), then
// the blocks below the diagonal column by column,
//   T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj,
// on fp32 MFMA into a buffer of its own (A stays intact). Block columns are
// independent of each other, so two waves share a head: one sweeps column 0,
// the other columns 1 and 2; two heads are in flight at once.
// ----------------------------------------------------------------------------
constexpr int kHeadsPerPass = 2;

struct PrepSmem {
  union {
    struct {
      _Float16 K[C * KS];
      _Float16 Q[C * KS];
    } in;
    struct {
      float A[kHeadsPerPass][C * AS];   // A of the heads of one pass
      float T[kHeadsPerPass][C * AS];   // their T (blocks on and below the diagonal)
    } m;
  } u;
  float wtmp[4][16 * 17];             // per-wave 16x16 staging for MFMA operands
  float rk[C], rq[C];
  float g[kHeadsPerPass][C], beta[kHeadsPerPass][C];
};

__device__ __forceinline__ float4_t mfma_f32(float a, float b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Block (ib, jb) below the diagonal of T; T already holds column jb's blocks
// above ib and the diagonal blocks.
__device__ __forceinline__ void t_offdiag_block(const float* A, float* T, float* wt, int ib, int jb,
                                                int lane) {
  const int m = lane & 15, kq = lane >> 4;
  float4_t W = {0.f, 0.f, 0.f, 0.f};
  for (int kb = jb; kb < ib; ++kb) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float a = A[(16 * ib + m) * AS + 16 * kb + 4 * s4 + kq];
      const float b = T[(16 * kb + 4 * s4 + kq) * AS + 16 * jb + m];
      W = mfma_f32(a, b, W);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) wt[(4 * kq + e) * 17 + m] = W[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  float4_t Tb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const float a = T[(16 * ib + m) * AS + 16 * ib + 4 * s4 + kq];
    const float b = wt[(4 * s4 + kq) * 17 + m];
    Tb = mfma_f32(a, b, Tb);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) T[(16 * ib + 4 * kq + e) * AS + 16 * jb + m] = -Tb[e];
}

__global__ void __launch_bounds__(kThreads) gdn_chunk_prep(ChunkArgs p, Ws w) {
  __shared__ PrepSmem sm;
  const int slot = blockIdx.x;
  const int g = blockIdx.y;
  int req, t0, L;
  if (!locate_chunk(p, w, slot, &req, &t0, &L)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const _Float16* kp = static_cast<const _Float16*>(p.k);
  const _Float16* qp = static_cast<const _Float16*>(p.q);

  // gate inputs of the first pass, loaded early (wave w < heads of the pass: head g*G + w);
  // tokens >= L and heads past the group read as zero
  const int gate_bytes = ((L - 1) * p.Hv + 1) * 4;
  float a_pf, b_pf;
  {
    const bool on = wave < min(kHeadsPerPass, p.group);
    const int h = g * p.group + (on ? wave : 0);
    a_pf = buf_load_f32(make_rsrc(p.a + (size_t)t0 * p.Hv + h, on ? gate_bytes : 0), lane * p.Hv * 4);
    b_pf = buf_load_f32(make_rsrc(p.b + (size_t)t0 * p.Hv + h, on ? gate_bytes : 0), lane * p.Hv * 4);
  }

  // ---- K, Q chunk tiles into LDS (rows >= L zero); 16 lanes per row, so the
  // per-token sums of squares reduce across those 16 lanes
  float ssk[4], ssq[4];
  const int krow = p.Hk * D;
  const rsrc_t rk = make_rsrc(kp + ((size_t)t0 * p.Hk + g) * D, ((L - 1) * krow + D) * 2);
  const rsrc_t rq = make_rsrc(qp + ((size_t)t0 * p.Hk + g) * D, ((L - 1) * krow + D) * 2);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + kThreads * it;    // 1024 16-byte pieces per tile
    const int row = idx >> 4, c8 = (idx & 15) * 8;
    const half8_t kv = buf_load_h8(rk, (row * krow + c8) * 2);   // rows >= L read as zero
    const half8_t qv = buf_load_h8(rq, (row * krow + c8) * 2);
    *reinterpret_cast<half8_t*>(&sm.u.in.K[row * KS + c8]) = kv;
    *reinterpret_cast<half8_t*>(&sm.u.in.Q[row * KS + c8]) = qv;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sk = fmaf((float)kv[j], (float)kv[j], sk);
      sq = fmaf((float)qv[j], (float)qv[j], sq);
    }
    ssk[it] = group_sum<16>(sk);
    ssq[it] = group_sum<16>(sq);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + kThreads * it;
    if ((idx & 15) == 0) {
      const int row = idx >> 4;
      const float rk = rsqrtf(ssk[it] + kNormEps);
      const float rq = rsqrtf(ssq[it] + kNormEps) * p.scale;
      sm.rk[row] = rk;
      sm.rq[row] = rq;
    }
  }
  lds_barrier();

  // ---- Gram matrices K K^T and Q K^T, rows 16*wave .. +15, column blocks <= wave
  float4_t kk[4], qk[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    kk[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    qk[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (nb <= wave) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int col = 32 * ks + 8 * (lane >> 4);
        const half8_t ak = lds8(&sm.u.in.K[(16 * wave + (lane & 15)) * KS + col]);
        const half8_t aq = lds8(&sm.u.in.Q[(16 * wave + (lane & 15)) * KS + col]);
        const half8_t bk = lds8(&sm.u.in.K[(16 * nb + (lane & 15)) * KS + col]);
        kk[nb] = mfma_f16(ak, bk, kk[nb]);
        qk[nb] = mfma_f16(aq, bk, qk[nb]);
      }
    }
  }
  lds_barrier();   // K, Q tiles are dead from here; their LDS becomes A

  for (int base = 0; base < p.group; base += kHeadsPerPass) {
    const int nb_heads = min(kHeadsPerPass, p.group - base);
    // ---- gates and in-chunk cumulative log decay: wave hv handles head base + hv
    if (wave < nb_heads) {
      const int h = g * p.group + base + wave;
      const int t = lane;
      float la = 0.f, be = 0.f;
      if (t < L) {
        la = -expf(p.A_log[h]) * softplus_f(a_pf + p.dt_bias[h]);
        be = sigmoid_f(b_pf);
      }
      // the next pass's gate inputs, in flight while this pass computes
      const bool on = base + kHeadsPerPass + wave < p.group;
      const int hn = on ? h + kHeadsPerPass : h;
      a_pf = buf_load_f32(make_rsrc(p.a + (size_t)t0 * p.Hv + hn, on ? gate_bytes : 0), t * p.Hv * 4);
      b_pf = buf_load_f32(make_rsrc(p.b + (size_t)t0 * p.Hv + hn, on ? gate_bytes : 0), t * p.Hv * 4);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {      // inclusive prefix sum over the 64 lanes
        const float y = __shfl_up(la, d, 64);
        if (t >= d) la += y;
      }
      sm.g[wave][t] = la;
      sm.beta[wave][t] = be;
      const float gL = __shfl(la, C - 1, 64);
      float* vec = w.vec + ((size_t)slot * p.Hv + h) * kVecRows * C;
      vec[kVecZ * C + t] = expf(la) * sm.rk[t];
      vec[kVecBeta * C + t] = be;
      vec[kVecO * C + t] = expf(la) * sm.rq[t];
      vec[kVecU * C + t] = expf(gL - la) * sm.rk[t];
      vec[kVecGamma * C + t] = expf(gL);
    }
    lds_barrier();

    // ---- A (fp32, LDS) and P (fp16, kept in registers until T is out) from the Gram
    half4_t pk[kHeadsPerPass][4];
#pragma unroll
    for (int hv = 0; hv < kHeadsPerPass; ++hv) {
      if (hv >= nb_heads) break;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int i = 16 * nb + (lane & 15);            // column (earlier token)
        const float gi = sm.g[hv][i], rki = sm.rk[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * wave + 4 * (lane >> 4) + e;  // row (later token)
          const float gr = sm.g[hv][r];
          float av = 0.f, pv = 0.f;
          if (nb <= wave) {
            const float dec = fast_exp(fminf(gr - gi, 0.f));
            if (i < r) av = sm.beta[hv][r] * dec * sm.rk[r] * rki * kk[nb][e];
            if (i <= r) pv = dec * sm.rq[r] * rki * qk[nb][e];
          }
          sm.u.m.A[hv][r * AS + i] = av;
          pk[hv][nb][e] = (_Float16)pv;
        }
      }
    }
    lds_barrier();

    // ---- T, step 1: the four diagonal 16x16 blocks (wave 2*hv, lane = 16*block + column)
    const int hv = wave >> 1, half_w = wave & 1;
    if (hv < nb_heads && half_w == 0) {
      const float* A = sm.u.m.A[hv];
      float* T = sm.u.m.T[hv];
      const int blk = lane >> 4, j = lane & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* arow = &A[(16 * blk + r) * AS + 16 * blk];
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int i = 0; i < r; i += 4) {
          const float4_t a4 = *reinterpret_cast<const float4_t*>(&arow[i]);
          s0 = fmaf(a4.x, x[i], s0);
          s1 = fmaf(a4.y, x[i + 1], s1);
          s2 = fmaf(a4.z, x[i + 2], s2);
          s3 = fmaf(a4.w, x[i + 3], s3);
        }
        x[r] = (r == j ? 1.f : 0.f) - ((s0 + s1) + (s2 + s3));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) T[(16 * blk + r) * AS + 16 * blk + j] = x[r];
    }
    lds_barrier();

    // ---- T, step 2: blocks below the diagonal; wave 2*hv: column 0, wave 2*hv+1: columns 1, 2
    if (hv < nb_heads) {
      const float* A = sm.u.m.A[hv];
      float* T = sm.u.m.T[hv];
      float* wt = sm.wtmp[wave];
      if (half_w == 0) {
        for (int ib = 1; ib < 4; ++ib) t_offdiag_block(A, T, wt, ib, 0, lane);
      } else {
        for (int ib = 2; ib < 4; ++ib) t_offdiag_block(A, T, wt, ib, 1, lane);
        t_offdiag_block(A, T, wt, 3, 2, lane);
      }
    }
    lds_barrier();

    // ---- T (fp16) to the workspace: the two waves of a head write 32 rows each
    if (hv < nb_heads) {
      const int h = g * p.group + base + hv;
      const float* T = sm.u.m.T[hv];
      _Float16* Tw = w.T + ((size_t)slot * p.Hv + h) * C * C;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = 64 * (4 * half_w + it) + lane;   // 512 pieces of 8 per head
        const int row = idx >> 3, c8 = (idx & 7) * 8;
        half8_t hv8 = {};                                // blocks above the diagonal are 0
        if ((c8 >> 4) <= (row >> 4)) {
          const float4_t lo = *reinterpret_cast<const float4_t*>(&T[row * AS + c8]);
          const float4_t hi = *reinterpret_cast<const float4_t*>(&T[row * AS + c8 + 4]);
          hv8 = half8_t{(_Float16)lo.x, (_Float16)lo.y, (_Float16)lo.z, (_Float16)lo.w,
                        (_Float16)hi.x, (_Float16)hi.y, (_Float16)hi.z, (_Float16)hi.w};
        }
        *reinterpret_cast<half8_t*>(Tw + row * C + c8) = hv8;
      }
    }
    lds_barrier();

    // ---- P (fp16) through LDS (the T buffers are free now) to the workspace
#pragma unroll
    for (int hvp = 0; hvp < kHeadsPerPass; ++hvp) {
      if (hvp >= nb_heads) break;
      _Float16* Ps = reinterpret_cast<_Float16*>(sm.u.m.T[hvp]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Ps[(16 * wave + 4 * (lane >> 4) + e) * TS + 16 * nb + (lane & 15)] = pk[hvp][nb][e];
    }
    lds_barrier();
    if (hv < nb_heads) {
      const int h = g * p.group + base + hv;
      const _Float16* Ps = reinterpret_cast<const _Float16*>(sm.u.m.T[hv]);
      _Float16* Pw = w.P + ((size_t)slot * p.Hv + h) * C * C;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = 64 * (4 * half_w + it) + lane;
        const int row = idx >> 3, c8 = (idx & 7) * 8;
        *reinterpret_cast<half8_t*>(Pw + row * C + c8) = lds8(&Ps[row * TS + c8]);
      }
    }
    lds_barrier();
  }
}

// ----------------------------------------------------------------------------
// gdn_chunk_scan: one workgroup per (request, value head, Dv tile of TV rows)
//
// The state tile is held transposed, S^T [dk][dv], in MFMA accumulators: wave w
// owns dk rows 32w .. 32w+31 for all TV dv columns. X, Y, Z, U and O are split
// by token rows: wave w computes tokens 16w .. 16w+15. K and Q of the chunk are
// staged once, row-major; the update S^T += K^T (uf o U) takes its K^T operand
// from the row-major tile with transposing LDS reads (ds_read_b64_tr_b16).
// ----------------------------------------------------------------------------
constexpr int VS_PAD = 4;           // V tile row padding (halves)

template <int TV>
struct ScanSmem {
  _Float16 K[C * KS];      // k of the chunk, [token][dk]
  _Float16 Q[C * KS];      // q of the chunk, [token][dk]
  _Float16 T[C * TS];
  _Float16 P[C * TS];
  _Float16 V[C * (TV + VS_PAD)];
  _Float16 S16[TV * KS];   // fp16 copy of the state tile, [dv][dk]
  _Float16 Zt[TV * TS];    // Z^T  [dv][token]
  _Float16 Ut[TV * TS];    // U^T  [dv][token]
  _Float16 Uk[TV * TS];    // (diag(uf) U)^T
  float zf[C], beta[C], of[C], uf[C];
  float gamma;
};

// Registers holding the next chunk's inputs while the current one computes.
template <int TV>
struct Prefetch {
  static constexpr int VH = TV / 4;   // halves of the V tile per thread (64 rows x TV)
  half8_t k[4], q[4];                 // row-major pieces of K and Q
  half8_t t[2], pm[2];
  _Float16 v[VH];
  float vec;
  float gamma;
};

// Loads of the chunk that starts at token t0 with L tokens (L = 0: all loads
// return zeros and touch no memory). Every load is a range-checked buffer load.
template <int TV>
__device__ __forceinline__ void prefetch_chunk(const ChunkArgs& p, const Ws& w, int slot, int t0, int L,
                                               int h, int g, int d0, Prefetch<TV>& f) {
  const int tid = threadIdx.x;
  const int krow = p.Hk * D;                   // elements between consecutive tokens of k, q
  const int vrow = p.Hv * D;
  const size_t kq_base = ((size_t)t0 * p.Hk + g) * D;
  const int kq_bytes = L > 0 ? ((L - 1) * krow + D) * 2 : 0;
  const rsrc_t rk = make_rsrc(static_cast<const _Float16*>(p.k) + kq_base, kq_bytes);
  const rsrc_t rq = make_rsrc(static_cast<const _Float16*>(p.q) + kq_base, kq_bytes);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + kThreads * it;       // 64 rows x 16 pieces of 8
    const int row = idx >> 4, c8 = (idx & 15) * 8;
    f.k[it] = buf_load_h8(rk, (row * krow + c8) * 2);
    f.q[it] = buf_load_h8(rq, (row * krow + c8) * 2);
  }
  const int wsz = L > 0 ? C * C * 2 : 0;
  const rsrc_t rt = make_rsrc(w.T + ((size_t)slot * p.Hv + h) * C * C, wsz);
  const rsrc_t rp = make_rsrc(w.P + ((size_t)slot * p.Hv + h) * C * C, wsz);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = tid + kThreads * it;       // 512 pieces of 8 halves
    f.t[it] = buf_load_h8(rt, idx * 16);
    f.pm[it] = buf_load_h8(rp, idx * 16);
  }
  {
    const rsrc_t rv = make_rsrc(static_cast<const _Float16*>(p.v) + ((size_t)t0 * p.Hv + h) * D + d0,
                                L > 0 ? ((L - 1) * vrow + TV) * 2 : 0);
    constexpr int VH = Prefetch<TV>::VH, PER_ROW = TV / VH;
    const int row = tid / PER_ROW, cc = (tid % PER_ROW) * VH;
    if constexpr (VH == 8) {
      const half8_t x = buf_load_h8(rv, (row * vrow + cc) * 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    } else {
      const half4_t x = buf_load_h4(rv, (row * vrow + cc) * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.v[j] = x[j];
    }
  }
  {
    const rsrc_t rvec = make_rsrc(w.vec + ((size_t)slot * p.Hv + h) * kVecRows * C,
                                  L > 0 ? kVecRows * C * 4 : 0);
    f.vec = buf_load_f32(rvec, tid * 4);       // rows kVecZ .. kVecU, 64 floats each
    f.gamma = buf_load_f32(rvec, kVecGamma * C * 4);
  }
}

// Waits here for the prefetched registers (an empty asm that reads them), so the
// wait lands at the end of an iteration and the loop header inherits nothing
// outstanding.
template <typename V>
__device__ __forceinline__ void settle(const V& x) {
  asm volatile("" ::"v"(x));
}

template <int TV>
__device__ __forceinline__ void settle_prefetch(const Prefetch<TV>& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    settle(f.k[i]);
    settle(f.q[i]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    settle(f.t[i]);
    settle(f.pm[i]);
  }
#pragma unroll
  for (int j = 0; j < Prefetch<TV>::VH; ++j) settle(f.v[j]);
  settle(f.vec);
  settle(f.gamma);
}

template <int TV>
__device__ __forceinline__ void stage_chunk(ScanSmem<TV>& sm, const Prefetch<TV>& f) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + kThreads * it;
    const int row = idx >> 4, c8 = (idx & 15) * 8;
    *reinterpret_cast<half8_t*>(&sm.K[row * KS + c8]) = f.k[it];
    *reinterpret_cast<half8_t*>(&sm.Q[row * KS + c8]) = f.q[it];
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = tid + kThreads * it;
    const int row = idx >> 3, c8 = (idx & 7) * 8;
    *reinterpret_cast<half8_t*>(&sm.T[row * TS + c8]) = f.t[it];
    *reinterpret_cast<half8_t*>(&sm.P[row * TS + c8]) = f.pm[it];
  }
  {
    constexpr int VH = Prefetch<TV>::VH, PER_ROW = TV / VH;
    const int row = tid / PER_ROW, cc = (tid % PER_ROW) * VH;
#pragma unroll
    for (int j = 0; j < VH; ++j) sm.V[row * (TV + VS_PAD) + cc + j] = f.v[j];
  }
  {
    const int which = tid >> 6, t = tid & 63;
    float* dst = which == kVecZ ? sm.zf : which == kVecBeta ? sm.beta : which == kVecO ? sm.of : sm.uf;
    dst[t] = f.vec;
    if (tid == 0) sm.gamma = f.gamma;
  }
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// MFMA operand holding, for lane (n = lane % 16, q = lane / 16), the eight values
// X[t0 + 8q + j][n0 + n] (j = 0..7) of a row-major fp16 LDS tile X with row
// stride `ld` halves: two transposing 64-bit LDS reads. Within each 16-lane group
// the read hands lane n element e of lane 4e + n/4's 4-element row segment, so
// lane i addresses row t0 + 8q + 4h + i/4, columns n0 + 4 (i % 4) .. +3.
// The halves are reinterpreted as whole vectors: element-wise casts of the read's
// result were folded into a broadcast of element 0 by the compiler.
__device__ __forceinline__ half8_t lds_col8(const _Float16* X, int ld, int t0, int n0) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, q = lane >> 4;
  const _Float16* a0 = X + (t0 + 8 * q + (i >> 2)) * ld + n0 + 4 * (i & 3);
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(a0));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(a0 + 4 * ld));
  const half4_t l4 = __builtin_bit_cast(half4_t, lo), h4 = __builtin_bit_cast(half4_t, hi);
  return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int TV>
__global__ void __launch_bounds__(kThreads) gdn_chunk_scan(ChunkArgs p, Ws w, int n_items) {
  constexpr int NT = D / TV;        // Dv tiles per head
  constexpr int MB = TV / 16;       // 16-column dv blocks of the tile
  __shared__ ScanSmem<TV> sm;

  // XCD-aware order: consecutive items (same request and key head) share an XCD's L2
  const int per_xcd = (int)(gridDim.x / 8);
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= n_items) return;
  const int tile = item % NT;
  int rest = item / NT;
  const int hv = rest % p.group;
  rest /= p.group;
  const int g = rest % p.Hk;
  const int req = rest / p.Hk;
  const int h = g * p.group + hv;
  const int d0 = tile * TV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;

  const int beg = clamp_cu(p.cu_seqlens, req, p.N);
  const int end = max(clamp_cu(p.cu_seqlens, req + 1, p.N), beg);
  const int slot0 = w.chunk_start[req];
  int nch = (end - beg + C - 1) / C;
  nch = max(0, min(nch, p.max_chunks - slot0));

  // ---- state tile, transposed: ST[i][nb] holds S[dv = d0+16nb+l16][dk = 32*wave+16i+4q4+e]
  float4_t ST[2][MB];
  const size_t head_off = ((size_t)req * p.Hv + h) * D * D;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      const int dv = d0 + 16 * nb + l16, dk = 32 * wave + 16 * i + 4 * q4;
      ST[i][nb] = float4_t{0.f, 0.f, 0.f, 0.f};
      if (p.initial_state != nullptr)
        ST[i][nb] = *reinterpret_cast<const float4_t*>(p.initial_state + head_off + (size_t)dv * D + dk);
    }

  Prefetch<TV> f;
  prefetch_chunk<TV>(p, w, slot0, beg, nch > 0 ? min(C, end - beg) : 0, h, g, d0, f);
  settle_prefetch<TV>(f);

  _Float16* op = static_cast<_Float16*>(p.output);
  for (int c = 0; c < nch; ++c) {
    const int t0 = beg + C * c;
    const int L = min(C, end - t0);
    const bool more = c + 1 < nch;
    const int tn = t0 + C;
    const int Ln = more ? min(C, end - tn) : 0;       // 0: the prefetch below loads nothing
    const int slot_n = more ? slot0 + c + 1 : slot0 + c;
    // ---- chunk inputs and the fp16 state copy into LDS
    stage_chunk<TV>(sm, f);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < MB; ++nb) {
        half4_t s4 = {(_Float16)ST[i][nb][0], (_Float16)ST[i][nb][1], (_Float16)ST[i][nb][2],
                      (_Float16)ST[i][nb][3]};
        *reinterpret_cast<half4_t*>(&sm.S16[(16 * nb + l16) * KS + 32 * wave + 16 * i + 4 * q4]) = s4;
      }
    lds_barrier();
    prefetch_chunk<TV>(p, w, slot_n, tn, Ln, h, g, d0, f);

    // ---- X = K S0^T and Y = Q S0^T for tokens 16*wave .. +15
    float4_t X[MB], Y[MB];
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      X[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
      Y[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int col = 32 * ks + 8 * q4;
      const half8_t ak = lds8(&sm.K[(16 * wave + l16) * KS + col]);
      const half8_t aq = lds8(&sm.Q[(16 * wave + l16) * KS + col]);
#pragma unroll
      for (int nb = 0; nb < MB; ++nb) {
        const half8_t bs = lds8(&sm.S16[(16 * nb + l16) * KS + col]);
        X[nb] = mfma_f16(ak, bs, X[nb]);
        Y[nb] = mfma_f16(aq, bs, Y[nb]);
      }
    }
    // ---- Z = beta (V - zf X) -> Zt[dv][token]
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      half4_t z4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * wave + 4 * q4 + e;
        const float vv = (float)sm.V[t * (TV + VS_PAD) + 16 * nb + l16];
        z4[e] = (_Float16)(sm.beta[t] * (vv - sm.zf[t] * X[nb][e]));
      }
      *reinterpret_cast<half4_t*>(&sm.Zt[(16 * nb + l16) * TS + 16 * wave + 4 * q4]) = z4;
    }
    lds_barrier();

    // ---- U = T Z (T is lower triangular: tokens beyond this row block add nothing)
    float4_t U[MB];
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) U[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks <= 16 * wave + 15) {
        const int col = 32 * ks + 8 * q4;
        const half8_t at = lds8(&sm.T[(16 * wave + l16) * TS + col]);
#pragma unroll
        for (int nb = 0; nb < MB; ++nb) {
          const half8_t bz = lds8(&sm.Zt[(16 * nb + l16) * TS + col]);
          U[nb] = mfma_f16(at, bz, U[nb]);
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      half4_t u4, w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * wave + 4 * q4 + e;
        u4[e] = (_Float16)U[nb][e];
        w4[e] = (_Float16)(sm.uf[t] * U[nb][e]);
      }
      *reinterpret_cast<half4_t*>(&sm.Ut[(16 * nb + l16) * TS + 16 * wave + 4 * q4]) = u4;
      *reinterpret_cast<half4_t*>(&sm.Uk[(16 * nb + l16) * TS + 16 * wave + 4 * q4]) = w4;
    }
    lds_barrier();

    // ---- O = diag(of) Y + P U  -> output rows < L
    float4_t O[MB];
#pragma unroll
    for (int nb = 0; nb < MB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) O[nb][e] = sm.of[16 * wave + 4 * q4 + e] * Y[nb][e];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks <= 16 * wave + 15) {
        const int col = 32 * ks + 8 * q4;
        const half8_t ap = lds8(&sm.P[(16 * wave + l16) * TS + col]);
#pragma unroll
        for (int nb = 0; nb < MB; ++nb) {
          const half8_t bu = lds8(&sm.Ut[(16 * nb + l16) * TS + col]);
          O[nb] = mfma_f16(ap, bu, O[nb]);
        }
      }
    }
    {
      const int vrow = p.Hv * D;
      const rsrc_t ro = make_rsrc(op + ((size_t)t0 * p.Hv + h) * D + d0, ((L - 1) * vrow + TV) * 2);
#pragma unroll
      for (int nb = 0; nb < MB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * wave + 4 * q4 + e;   // rows t >= L fall outside the range: dropped
          buf_store_h1((_Float16)O[nb][e], ro, (t * vrow + 16 * nb + l16) * 2);
        }
    }

    // ---- S^T = gamma S^T + K^T (uf o U)   (wave: dk rows 32*wave .. +31)
    const float decay_L = sm.gamma;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < MB; ++nb) ST[i][nb] *= decay_L;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int col = 32 * ks + 8 * q4;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const half8_t ak = lds_col8(sm.K, KS, 32 * ks, 32 * wave + 16 * i);
#pragma unroll
        for (int nb = 0; nb < MB; ++nb) {
          const half8_t bu = lds8(&sm.Uk[(16 * nb + l16) * TS + col]);
          ST[i][nb] = mfma_f16(ak, bu, ST[i][nb]);
        }
      }
    }
    settle_prefetch<TV>(f);
    lds_barrier();   // all LDS reads of this chunk are done before the next stage
  }

  if (p.final_state != nullptr) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nb = 0; nb < MB; ++nb) {
        const int dv = d0 + 16 * nb + l16, dk = 32 * wave + 16 * i + 4 * q4;
        *reinterpret_cast<float4_t*>(p.final_state + head_off + (size_t)dv * D + dk) = ST[i][nb];
      }
  }
}

constexpr int kScanTile = 32;

size_t chunk_workspace_bytes(int64_t chunk_slots, int R, int Hk, int Hv) {
  return ws_bytes(chunk_slots, R, Hk, Hv);
}

hipError_t launch_chunk(const ChunkArgs& p, int io_dtype, hipStream_t stream) {
  if (io_dtype != 1) return hipErrorInvalidValue;     // fp16 I/O only
  if (p.R == 0) return hipSuccess;
  const Ws w = ws_layout(p.workspace, p.max_chunks, p.R, p.Hk, p.Hv);
  hipLaunchKernelGGL(gdn_chunk_index, dim3(1), dim3(kThreads), 0, stream, p, w);
  if (p.max_chunks > 0)
    hipLaunchKernelGGL(gdn_chunk_prep, dim3((unsigned)p.max_chunks, (unsigned)p.Hk), dim3(kThreads),
                       0, stream, p, w);
  const int n_items = p.R * p.Hv * (D / kScanTile);
  const int grid = (n_items + 7) / 8 * 8;
  hipLaunchKernelGGL(gdn_chunk_scan<kScanTile>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p, w,
                     n_items);
  return hipGetLastError();
}

}  // namespace gdn

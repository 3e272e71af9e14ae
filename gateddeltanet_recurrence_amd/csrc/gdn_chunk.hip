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
//   A[r,i] = beta_r e^{g_r - g_i} k^_r.k^_i  (i < r),   T' = (I + A)^-1 diag(beta)
//   P[r,i] = e^{g_r - g_i} q^_r.k^_i         (i <= r)
//   X = K S0^T,  Y = Q S0^T                              (raw fp16 k, q)
//   U = T' (V - diag(e^g rk) X)                          (U rows: the deltas u_t)
//   O = diag(e^g rq) Y + P U
//   S = e^{g_L} S0 + (diag(e^{g_L - g} rk) U)^T K
// Everything that does not depend on S0 (Gram matrices, T', P, gates, norms) is
// chunk-parallel and done first by gdn_chunk_prep; gdn_chunk_scan then walks
// the chunks of each sequence in order. The rows of S evolve independently,
// so the scan splits every head's state into Dv tiles, one workgroup each, and
// every wave of a workgroup runs the whole chain for 16 state rows of its own.
//
// Kernels: gdn_chunk_index (chunk offsets per sequence), gdn_chunk_prep,
// gdn_chunk_scan. Dk = Dv = 128, fp16 I/O only.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C = kChunk;     // 64 tokens per chunk
constexpr int D = 128;        // Dk = Dv
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


// T' and P reach the scan as MFMA operand fragments of v_mfma_f32_16x16x32_f16:
// the six 16x32 blocks on and below the diagonal (row block rb, column step s),
// 64 lanes x 8 halves each. Lane (l16 = lane % 16, q = lane / 16) of block f
// holds row 16 rb + l16 at columns
//   32 s + 4 q + j        (j = 0..3)
//   32 s + 16 + 4 q + j-4 (j = 4..7),
// the column order in which a 16x16 accumulator tile (rows 4q .. 4q+3 in lane
// group q) of two adjacent row blocks serves as the other operand.
constexpr int kFrags = 6;
constexpr int kFragHalves = kFrags * 64 * 8;     // 3072 halves = 6 KiB per (chunk, head)
__device__ constexpr int kFragRow[kFrags] = {0, 1, 2, 2, 3, 3};
__device__ constexpr int kFragStep[kFrags] = {0, 0, 0, 1, 0, 1};

__host__ __device__ constexpr int frag_col(int s, int q, int j) {
  return 32 * s + (j < 4 ? 4 * q + j : 16 + 4 * q + (j - 4));
}

// Workspace layout: chunk offsets, then per (slot, value head) the T' and P
// fragments and the per-token factors the scan applies (fp32 rows of 64):
//   kVecZ  e^{g_t} rk_t            kVecO  e^{g_t} rq_t
//   kVecU  e^{g_L - g_t} rk_t      kVecGamma  element 0: e^{g_L}, the decay of the whole chunk
constexpr int kVecZ = 0, kVecO = 1, kVecU = 2, kVecGamma = 3, kVecRows = 4;

struct Ws {
  int32_t* chunk_start;
  int32_t* order;       // requests by decreasing chunk count (ties: lower index first)
  _Float16* T;
  _Float16* P;
  float* vec;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Ws ws_layout(void* base, int64_t slots, int R, int Hk, int Hv) {
  (void)Hk;
  char* p = static_cast<char*>(base);
  Ws w;
  size_t off = 0;
  w.chunk_start = reinterpret_cast<int32_t*>(p + off);
  off += align256((size_t)(R + 1) * 4);
  w.order = reinterpret_cast<int32_t*>(p + off);
  off += align256((size_t)R * 4);
  w.T = reinterpret_cast<_Float16*>(p + off);
  off += align256((size_t)slots * Hv * kFragHalves * 2);
  w.P = reinterpret_cast<_Float16*>(p + off);
  off += align256((size_t)slots * Hv * kFragHalves * 2);
  w.vec = reinterpret_cast<float*>(p + off);
  return w;
}

__host__ inline size_t ws_bytes(int64_t slots, int R, int Hk, int Hv) {
  (void)Hk;
  return align256((size_t)(R + 1) * 4) + align256((size_t)R * 4) + 2 * align256((size_t)slots * Hv * kFragHalves * 2) +
         align256((size_t)slots * Hv * kVecRows * C * 4);
}

}  // namespace

// ----------------------------------------------------------------------------
// chunk offsets: chunk_start[r] = sum_{i<r} ceil(len_i / 64), chunk_start[R] = total;
// order: the requests sorted by decreasing chunk count (ties by index), so that the
// scan starts the longest sequences first (identity beyond kMaxSortRequests)
// ----------------------------------------------------------------------------
constexpr int kMaxSortRequests = 1024;

__global__ void __launch_bounds__(kThreads) gdn_chunk_index(ChunkArgs p, Ws w) {
  __shared__ int part[kThreads];
  const int tid = threadIdx.x;
  const int per = (p.R + kThreads - 1) / kThreads;
  const int r0 = min(tid * per, p.R), r1 = min(r0 + per, p.R);
  int prev = seq_start(p, r0);
  int sum = 0;
  for (int r = r0; r < r1; ++r) {
    const int nxt = max(seq_start(p, r + 1), prev);
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
  prev = seq_start(p, r0);
  for (int r = r0; r < r1; ++r) {
    w.chunk_start[r] = run;
    const int nxt = max(seq_start(p, r + 1), prev);
    run += (nxt - prev + C - 1) / C;
    prev = nxt;
  }
  if (tid == kThreads - 1) w.chunk_start[p.R] = part[kThreads - 1];
  __syncthreads();
  for (int r = r0; r < r1; ++r) {
    int rank = r;
    if (p.R <= kMaxSortRequests) {
      const int nr = w.chunk_start[r + 1] - w.chunk_start[r];
      rank = 0;
      for (int o = 0; o < p.R; ++o) {
        const int no = w.chunk_start[o + 1] - w.chunk_start[o];
        rank += (no > nr) || (no == nr && o < r);
      }
    }
    w.order[rank] = r;
  }
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
  const int beg = seq_start(p, lo);
  const int end = max(seq_start(p, lo + 1), beg);
  *req = lo;
  *t0 = beg + C * (slot - w.chunk_start[lo]);
  *len = min(C, end - *t0);
  return *len > 0;
}

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

// ----------------------------------------------------------------------------
// gdn_chunk_scan: one workgroup per (request, value head, tile of 32 state rows);
// each of its two waves owns 16 rows dv of the state and runs the whole chain
// for them, with no data exchanged between the waves:
//   X  = K S0^T        (tokens x dv)      A: K rows (LDS)      B: fp16 copy of S0
//   Y^T = S0 Q^T       (dv x tokens)      A: the same S0 copy  B: Q rows (LDS)
//   U  = T' (V - zf X)                    A: T' fragments      B: Z, straight from X's accumulators
//   O^T = of Y^T + U^T P^T                A: U, from accumulators  B: P fragments
//   S^T = gamma S^T + K^T (uf U)          A: K^T (transposing LDS reads)  B: uf U, from accumulators
// An accumulator tile (rows 4q .. 4q+3 in lane group q) of two adjacent 16-row
// blocks is an operand whose 32 contraction indices run in the order of
// frag_col, which is why T' and P are stored in that order.
//
// K, Q and V of a chunk are copied into LDS by buffer loads that write LDS
// directly, one chunk ahead, into two alternating buffers; one barrier per
// chunk. K and Q rows are stored without padding, their 16-byte units permuted
// by an XOR of the row (kv_swizzle) so that the row-fragment reads and the
// transposing column reads are both free of bank conflicts.
// ----------------------------------------------------------------------------
// Tile configurations: NW compute waves own 16 state rows each (tile TV = 16 NW
// rows); two loader waves copy the chunks. NW = 2 keeps more workgroups in flight
// for few, long sequences (three LDS buffers); NW = 4 halves the k, q, T', P bytes
// each CU pulls per state row when there are workgroups enough (two buffers).
constexpr int kLoaderWaves = 2;
constexpr int kRowsPerWave = 16;

template <int NW>
struct ScanCfg {
  static constexpr int TV = kRowsPerWave * NW;          // state rows per workgroup
  static constexpr int NT = D / TV;                     // tiles per head
  static constexpr int NBUF = NW == 2 ? 3 : 2;          // LDS buffers (chunks in flight)
  static constexpr int THREADS = 64 * (NW + kLoaderWaves);
  static constexpr int VROW = TV * 2;                   // bytes of a V tile row
  static constexpr int VROWS_PER_LOAD = 1024 / VROW;
  static constexpr int VLOADS = C / VROWS_PER_LOAD;     // 1 KiB loads of the V tile (4 or 8)
  // direct loads per loader wave and chunk: half of K, Q (8 + 8), T', P (3 + 3), V,
  // and the factors (both loaders write the same bytes)
  static constexpr int STAGE_LOADS = 8 + 8 + 3 + 3 + VLOADS / 2 + 1;
};

// 16-byte unit u of row r of a K or Q tile is stored at unit u ^ kv_swizzle(r).
__device__ __forceinline__ int kv_swizzle(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// 16-byte unit u of row r of a V tile is stored at unit u ^ v_swizzle<NW>(r): the
// 8 rows that a transposing read of one wave's 32-byte slice touches then fall in
// distinct banks (64-byte rows: alternate the halves every 4 rows; 128-byte rows:
// rotate the slice among the four pairs every 2 rows).
template <int NW>
__device__ __forceinline__ int v_swizzle(int r) {
  if constexpr (NW == 2) return ((r >> 2) & 1) << 1;
  else return ((r >> 1) & 3) << 1;
}

// Operands of NBUF chunks in LDS (buffer b = chunk index mod NBUF). Each piece is
// an LDS object of its own: the compiler then knows that the direct-to-LDS loads
// into one buffer do not alias the reads of another, and does not wait for the
// loads of a later chunk before reading the current one.
#define GDN_SCAN_LDS3(type, name, count) \
  __shared__ __attribute__((aligned(16))) type name##0[count]; \
  __shared__ __attribute__((aligned(16))) type name##1[count]; \
  __shared__ __attribute__((aligned(16))) type name##2[count];
#define GDN_SCAN_LDS2(type, name, count) \
  __shared__ __attribute__((aligned(16))) type name##0[count]; \
  __shared__ __attribute__((aligned(16))) type name##1[count];
// NW = 2
GDN_SCAN_LDS3(_Float16, lds2_K, C * D)           // [token][dk], units permuted by kv_swizzle
GDN_SCAN_LDS3(_Float16, lds2_Q, C * D)
GDN_SCAN_LDS3(_Float16, lds2_T, kFragHalves)     // T' fragments as stored by gdn_chunk_prep
GDN_SCAN_LDS3(_Float16, lds2_P, kFragHalves)
GDN_SCAN_LDS3(_Float16, lds2_V, C * 32)          // [token][dv of the tile], units permuted by v_swizzle
GDN_SCAN_LDS3(float, lds2_vec, kVecRows * C)
__shared__ __attribute__((aligned(16))) unsigned lds2_touch[kLoaderWaves][64];  // discarded prefetch data
// NW = 4
GDN_SCAN_LDS2(_Float16, lds4_K, C * D)
GDN_SCAN_LDS2(_Float16, lds4_Q, C * D)
GDN_SCAN_LDS2(_Float16, lds4_T, kFragHalves)
GDN_SCAN_LDS2(_Float16, lds4_P, kFragHalves)
GDN_SCAN_LDS2(_Float16, lds4_V, C * 64)
GDN_SCAN_LDS2(float, lds4_vec, kVecRows * C)
__shared__ __attribute__((aligned(16))) unsigned lds4_touch[kLoaderWaves][64];
#undef GDN_SCAN_LDS3
#undef GDN_SCAN_LDS2

template <int NW, int B> struct ScanBuf;
template <int B> struct ScanBuf<2, B> {
  static __device__ __forceinline__ _Float16* K() { return B == 0 ? lds2_K0 : B == 1 ? lds2_K1 : lds2_K2; }
  static __device__ __forceinline__ _Float16* Q() { return B == 0 ? lds2_Q0 : B == 1 ? lds2_Q1 : lds2_Q2; }
  static __device__ __forceinline__ _Float16* T() { return B == 0 ? lds2_T0 : B == 1 ? lds2_T1 : lds2_T2; }
  static __device__ __forceinline__ _Float16* P() { return B == 0 ? lds2_P0 : B == 1 ? lds2_P1 : lds2_P2; }
  static __device__ __forceinline__ _Float16* V() { return B == 0 ? lds2_V0 : B == 1 ? lds2_V1 : lds2_V2; }
  static __device__ __forceinline__ float* vec() { return B == 0 ? lds2_vec0 : B == 1 ? lds2_vec1 : lds2_vec2; }
  static __device__ __forceinline__ unsigned* touch(int loader) { return lds2_touch[loader]; }
};
template <int B> struct ScanBuf<4, B> {
  static __device__ __forceinline__ _Float16* K() { return B == 0 ? lds4_K0 : lds4_K1; }
  static __device__ __forceinline__ _Float16* Q() { return B == 0 ? lds4_Q0 : lds4_Q1; }
  static __device__ __forceinline__ _Float16* T() { return B == 0 ? lds4_T0 : lds4_T1; }
  static __device__ __forceinline__ _Float16* P() { return B == 0 ? lds4_P0 : lds4_P1; }
  static __device__ __forceinline__ _Float16* V() { return B == 0 ? lds4_V0 : lds4_V1; }
  static __device__ __forceinline__ float* vec() { return B == 0 ? lds4_vec0 : lds4_vec1; }
  static __device__ __forceinline__ unsigned* touch(int loader) { return lds4_touch[loader]; }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Lane l of a direct load fills LDS bytes 16 l .. 16 l + 15 of the load's 1 KiB destination.
__device__ __forceinline__ void load_lds16(rsrc_t r, void* lds, int byte_off, int uniform_off = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, byte_off, uniform_off, 0, 0);
}

constexpr int kTouchLoads = 3;     // L2 prefetch loads per loader wave and chunk
// Prefetched this many chunks ahead of the direct loads. Further ahead, the lines in
// flight per XCD approach its 4 MB L2 when every CU runs a workgroup, and some are
// evicted before their direct loads: one chunk ahead took the ragged prefill from
// 223-229 to 214-218 us (three ahead), the long one unchanged; without the prefetch
// the long prefill took 904 us.
constexpr int kTouchAhead = 1;

// Copies chunk (slot, t0, L) into LDS buffer B; rows >= L read as zero (L = 0: no
// memory is read, the buffer fills with zeros). Loader wave w copies rows
// 32 w .. 32 w + 31 of K, Q and V and fragments 3 w .. 3 w + 2 of T' and P; both
// write the 1 KiB of factors (the same bytes): STAGE_LOADS loads each.
template <int NW, int B>
struct Stage {
  typedef ScanCfg<NW> Cfg;
  typedef ScanBuf<NW, B> Buf;
  rsrc_t rk, rq, rt, rp, rv, rvec;
  int krow, vrow, wave, lane;

  __device__ __forceinline__ Stage(const ChunkArgs& p, const Ws& w, int slot, int t0, int L, int h, int g,
                                   int d0, int wave_, int lane_)
      : krow(p.Hk * D), vrow(p.Hv * D), wave(wave_), lane(lane_) {
    const size_t kq_base = ((size_t)t0 * p.Hk + g) * D;
    const int kq_bytes = L > 0 ? ((L - 1) * krow + D) * 2 : 0;
    rk = make_rsrc(static_cast<const _Float16*>(p.k) + kq_base, kq_bytes);
    rq = make_rsrc(static_cast<const _Float16*>(p.q) + kq_base, kq_bytes);
    const size_t fo = ((size_t)slot * p.Hv + h) * kFragHalves;
    const int f_bytes = L > 0 ? kFragHalves * 2 : 0;
    rt = make_rsrc(w.T + fo, f_bytes);
    rp = make_rsrc(w.P + fo, f_bytes);
    rv = make_rsrc(static_cast<const _Float16*>(p.v) + ((size_t)t0 * p.Hv + h) * D + d0,
                   L > 0 ? ((L - 1) * vrow + Cfg::TV) * 2 : 0);
    rvec = make_rsrc(w.vec + ((size_t)slot * p.Hv + h) * kVecRows * C, L > 0 ? kVecRows * C * 4 : 0);
  }

  // K or Q rows 32 wave .. +31: 4 rows of 256 bytes per load; kv_swizzle repeats
  // every 16 rows, so four per-lane offsets serve all loads and the row block
  // goes in the uniform offset (8 loads)
  __device__ __forceinline__ void kq(rsrc_t r, _Float16* dst) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * j + (lane >> 4);
      const int off = row * krow * 2 + 16 * ((lane & 15) ^ kv_swizzle(row));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int blk = 8 * wave + 4 * i + j;          // rows 4 blk .. 4 blk + 3
        load_lds16(r, dst + 4 * blk * D, off, (32 * wave + 16 * i) * krow * 2);
      }
    }
  }
  // T' and P fragments 3 wave .. +2 (6 loads)
  __device__ __forceinline__ void tp() const {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = 3 * wave + i;
      load_lds16(rt, Buf::T() + f * 512, lane * 16, f * 1024);
      load_lds16(rp, Buf::P() + f * 512, lane * 16, f * 1024);
    }
  }
  // V rows 32 wave .. +31, VROWS_PER_LOAD rows per load (v_swizzle repeats within
  // that many rows), and the factors
  __device__ __forceinline__ void v() const {
    constexpr int UNITS = Cfg::VROW / 16;
    const int vr = lane / UNITS;
    const int voff = vr * vrow * 2 + 16 * ((lane % UNITS) ^ v_swizzle<NW>(vr));
#pragma unroll
    for (int i = 0; i < Cfg::VLOADS / 2; ++i) {
      const int blk = (Cfg::VLOADS / 2) * wave + i;
      load_lds16(rv, Buf::V() + Cfg::VROWS_PER_LOAD * blk * Cfg::TV, voff, Cfg::VROWS_PER_LOAD * blk * vrow * 2);
    }
    load_lds16(rvec, Buf::vec(), lane * 16);
  }
  __device__ __forceinline__ void all() const {
    kq(rk, Buf::K());
    kq(rq, Buf::Q());
    tp();
    v();
  }
};

__device__ __forceinline__ half8_t lds_b128(const _Float16* base, int byte_off) {
  return *reinterpret_cast<const half8_t*>(reinterpret_cast<const char*>(base) + byte_off);
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef unsigned int uint2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half4_t lds_tr4(const _Float16* base, int byte_off) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t*)(reinterpret_cast<const char*>(base) + byte_off));
  return __builtin_bit_cast(half4_t, v);
}

__device__ __forceinline__ half4_t to_half4(float4_t x) {
  return half4_t{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}

__device__ __forceinline__ half8_t cat8(half4_t lo, half4_t hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Loader waves: wait until this wave has at most LIMIT vector memory operations
// in flight, then the workgroup barrier. Per chunk a loader issues STAGE_LOADS
// direct loads into the buffer that is NBUF - 1 chunks ahead, then kTouchLoads
// prefetches; loads complete in issue order, and after the last direct load of
// the chunk the barrier releases come at least (NBUF - 2) STAGE_LOADS +
// (NBUF - 1) kTouchLoads more, so once no more than that many are pending the
// chunk is in LDS. No release fence: one would wait for every direct load still
// in flight (they write LDS).
template <int NW>
__device__ __forceinline__ void loader_barrier() {
  typedef ScanCfg<NW> Cfg;
  constexpr int kLimit = (Cfg::NBUF - 2) * Cfg::STAGE_LOADS + (Cfg::NBUF - 1) * kTouchLoads;
  static_assert(kLimit < 64, "vmcnt holds 6 bits");
  // s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in [15:14]
  constexpr int kWait = (kLimit & 15) | (7 << 4) | (15 << 8) | ((kLimit >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(kWait);
  __builtin_amdgcn_s_barrier();
}

// Compute waves: the same barrier. The release fence makes this wave's reads of
// the previous chunk (whose buffer the loaders refill next) complete before it:
// the compiler may otherwise leave the last of them in flight across the barrier.
// The acquire fence keeps this chunk's reads below it.
__device__ __forceinline__ void compute_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct ScanCtx {
  const ChunkArgs& p;
  const Ws& w;
  int h, g, d0, dvw, wave, lane, beg, end, slot0, nch;
};

// Output rows (t0 .. t0 + L - 1) of O^T tiles: lane (l16, q) holds dv 4q .. 4q+3 of
// token 16 nb + l16; rows >= L fall outside the range and are dropped.
__device__ __forceinline__ void store_out(const ScanCtx& x, const float4_t (&O)[4], int t0, int L) {
  const int vrow = x.p.Hv * D;
  const int l16 = x.lane & 15, q = x.lane >> 4;
  const rsrc_t ro = make_rsrc(static_cast<_Float16*>(x.p.output) + ((size_t)t0 * x.p.Hv + x.h) * D + x.dvw,
                              L > 0 ? ((L - 1) * vrow + kRowsPerWave) * 2 : 0);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const half4_t o4 = to_half4(O[nb]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2_t, o4), ro,
                                          ((16 * nb + l16) * vrow + 4 * q) * 2, 0, 0);
  }
}

// State tiles. The wave's 16 x 128 state slice is kept transposed in 8 MFMA
// accumulator tiles ST[mb]; lane (l16, q) element e of tile mb holds
// S[dv = l16][dk_tile(mb, q) + e]. Tiles 2 ks and 2 ks + 1 thus hold, in lane
// group q, dk 32 ks + 8 q .. 32 ks + 8 q + 7: converted to fp16 and concatenated
// they are the state operand of the 32-wide k step ks, in the plain fragment
// order, with no trip through LDS. The row order is set by the transposing reads
// of K^T in the state update, whose output row j = 4 m + i is dk_tile(mb, m) + i.
__device__ __forceinline__ constexpr int dk_tile(int mb, int m) { return 32 * (mb >> 1) + 8 * m + 4 * (mb & 1); }

// Per-lane LDS byte offsets that do not change from chunk to chunk; every
// access adds only compile-time constants to one of them.
struct LaneOffsets {
  int row[4];     // K / Q row-fragment reads, per 32-wide k step: row l16, unit (4 ks + q) ^ sw
  int tr[8];      // K^T transposing reads, per state tile mb (token 4q + l16/4 of the first block)
  int v;          // V transposing reads
  int frag;       // T' / P fragment reads
};

template <int NW>
__device__ __forceinline__ LaneOffsets lane_offsets(int wave, int lane) {
  LaneOffsets o;
  const int l16 = lane & 15, q = lane >> 4;
  const int sw = kv_swizzle(l16);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.row[ks] = l16 * (D * 2) + 16 * ((4 * ks + q) ^ sw);
  // token r0 = 32 s + 4 q + l16 / 4 (+16): kv_swizzle depends on r0 % 16 = 4 q + l16 / 4 only.
  // The lane reads dk_tile(mb, l16 & 3) .. +3, the four state rows that its transposed
  // data becomes (see dk_tile)
  const int r0 = 4 * q + (l16 >> 2), swt = kv_swizzle(r0);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int dk = dk_tile(mb, l16 & 3);
    o.tr[mb] = r0 * (D * 2) + 16 * ((dk >> 3) ^ swt) + 2 * (dk & 7);
  }
  // V: row 16 mb + rv, rv = 4 q + l16 / 4; v_swizzle depends on the row mod 8 only
  const int rv = 4 * q + (l16 >> 2);
  const int col8 = kRowsPerWave * 2 * wave + 8 * (l16 & 3);
  o.v = rv * (ScanCfg<NW>::TV * 2) + 16 * ((col8 >> 4) ^ v_swizzle<NW>(rv)) + (col8 & 15);
  o.frag = lane * 16;
  return o;
}

// L2 prefetch of chunk (slot, t0, L) for the direct loads a few chunks later:
// one 4-byte load per 128-byte line into a discarded LDS area. Lines shared by
// several workgroups are split between them: K and Q of a key head among its
// nshare = group x tiles workgroups (share index sub), T', P and the factors of
// a head among its tiles, and a V line (128 bytes of a row: one or two tiles) goes to
// the tile that starts it. Loader 0 takes K, Q and the factors, loader 1 T', P and V:
// kTouchLoads loads each; a lane without a line gets an offset past the range.
template <int NW>
__device__ __forceinline__ void touch_chunk(const ScanCtx& x, int slot, int t0, int L, int loader, int sub,
                                            int nshare, int tile) {
  constexpr int kNone = 0x7FFFFFF0;                // past every range below
  typedef ScanCfg<NW> Cfg;
  const int lane = x.lane;
  lds_void_t* dst = (lds_void_t*)ScanBuf<NW, 0>::touch(loader);
  const size_t fo = ((size_t)slot * x.p.Hv + x.h) * kFragHalves;
  const int f_bytes = L > 0 ? kFragHalves * 2 : 0;
  if (loader == 0) {
    const int krow = x.p.Hk * D;
    const size_t kq_base = ((size_t)t0 * x.p.Hk + x.g) * D;
    const int kq_bytes = L > 0 ? ((L - 1) * krow + D) * 2 : 0;
    const int i = sub + nshare * lane;             // line i: row i / 2, half i % 2 of the 256-byte row
    const int off = i < 2 * C ? (i >> 1) * krow * 2 + (i & 1) * 128 : kNone;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(static_cast<const _Float16*>(x.p.k) + kq_base, kq_bytes),
                                             dst, 4, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(static_cast<const _Float16*>(x.p.q) + kq_base, kq_bytes),
                                             dst, 4, off, 0, 0, 0);
    const rsrc_t rvec = make_rsrc(x.w.vec + ((size_t)slot * x.p.Hv + x.h) * kVecRows * C,
                                  (L > 0 && tile == 0) ? kVecRows * C * 4 : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rvec, dst, 4, lane < 8 ? 128 * lane : kNone, 0, 0, 0);
  } else {
    const int m = tile + Cfg::NT * lane;           // fragment line m of 48
    const int off = m < kFragHalves * 2 / 128 ? 128 * m : kNone;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(x.w.T + fo, f_bytes), dst, 4, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(x.w.P + fo, f_bytes), dst, 4, off, 0, 0, 0);
    const int vrow = x.p.Hv * D;
    const int dline = x.d0 & ~63;                  // first dv of the 128-byte line
    const rsrc_t rv = make_rsrc(static_cast<const _Float16*>(x.p.v) + ((size_t)t0 * x.p.Hv + x.h) * D + dline,
                                (L > 0 && dline == x.d0) ? ((L - 1) * vrow + 64) * 2 : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 4, lane * vrow * 2, 0, 0, 0);
  }
}

// Loader step: chunk c is in LDS buffer B once the barrier passes; then the loads
// of chunk c + NBUF - 1 into the buffer that chunk c - 1 used (the compute waves
// are past it) and the L2 prefetch of the chunk kTouchAhead after that.
template <int NW, int B>
__device__ __forceinline__ void loader_step(const ScanCtx& x, int c, int loader, int sub, int nshare, int tile) {
  constexpr int NBUF = ScanCfg<NW>::NBUF, LEAD = NBUF - 1;
  const bool more = c + LEAD < x.nch;
  const int t0 = x.beg + C * (c + LEAD);
  loader_barrier<NW>();
  Stage<NW, (B + LEAD) % NBUF>(x.p, x.w, more ? x.slot0 + c + LEAD : x.slot0 + c, t0,
                               more ? min(C, x.end - t0) : 0, x.h, x.g, x.d0, loader, x.lane)
      .all();
  const int ca = c + LEAD + kTouchAhead;
  const bool ahead = ca < x.nch;
  const int ta = x.beg + C * ca;
  touch_chunk<NW>(x, ahead ? x.slot0 + ca : x.slot0, ta, ahead ? min(C, x.end - ta) : 0, loader, sub, nshare,
                  tile);
}

// Compute step: chunk c from LDS buffer B = c mod NBUF; stores the output of chunk c - 1.
template <int NW, int B>
__device__ __forceinline__ void scan_step(const ScanCtx& x, const LaneOffsets& lo_in, int c, float4_t (&ST)[8],
                                          float4_t (&O)[4], int& o_t0, int& o_L) {
  const int lane = x.lane, l16 = lane & 15, q = lane >> 4;
  const int t0 = x.beg + C * c;
  const LaneOffsets& lo = lo_in;
  typedef ScanBuf<NW, B> Buf;
  const float* vec = Buf::vec();
  compute_barrier();                                   // chunk c is in LDS buffer B
  store_out(x, O, o_t0, o_L);

  // ---- X = K S0^T (X[mb]: tokens 16 mb + 4q + e, column dv = l16) and Y^T = S0 Q^T
  // (Yt[nb]: dv 4q + e, token 16 nb + l16); operands of step ks + 1 are read
  // while the products of step ks run
  float4_t X[4], Yt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    X[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    Yt[i] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  half8_t s8[2], k8[2][4], q8[2][4];
  auto load_xy = [&](int ks, int slot) {
    s8[slot] = cat8(to_half4(ST[2 * ks]), to_half4(ST[2 * ks + 1]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k8[slot][i] = lds_b128(Buf::K(), lo.row[ks] + 16 * D * 2 * i);
      q8[slot][i] = lds_b128(Buf::Q(), lo.row[ks] + 16 * D * 2 * i);
    }
  };
  load_xy(0, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks < 3) load_xy(ks + 1, (ks + 1) & 1);
    const int sl = ks & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      X[i] = mfma_f16(k8[sl][i], s8[sl], X[i]);
      Yt[i] = mfma_f16(s8[sl], q8[sl][i], Yt[i]);
    }
  }

  // ---- Z = V - zf X (fp16); V rows 16 mb + 4q + e at column l16 by transposing reads
  half4_t v4[4];
  float4_t zf[4];
  half8_t tf[kFrags];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    v4[mb] = lds_tr4(Buf::V(), lo.v + 16 * mb * (ScanCfg<NW>::TV * 2));
    zf[mb] = *reinterpret_cast<const float4_t*>(&vec[kVecZ * C + 16 * mb + 4 * q]);
  }
#pragma unroll
  for (int f = 0; f < kFrags; ++f) tf[f] = lds_b128(Buf::T(), lo.frag + f * 1024);
  half4_t Zh[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float4_t z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = (float)v4[mb][e] - zf[mb][e] * X[mb][e];
    Zh[mb] = to_half4(z);
  }

  // ---- U = T' Z
  float4_t U[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) U[i] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    const int s2 = 2 * kFragStep[f];
    U[kFragRow[f]] = mfma_f16(tf[f], cat8(Zh[s2], Zh[s2 + 1]), U[kFragRow[f]]);
  }

  // ---- O^T = of Y^T + U^T P^T (stored at the next step)
  half8_t pf[kFrags];
  float4_t uf[4];
  float of[4];
#pragma unroll
  for (int f = 0; f < kFrags; ++f) pf[f] = lds_b128(Buf::P(), lo.frag + f * 1024);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uf[i] = *reinterpret_cast<const float4_t*>(&vec[kVecU * C + 16 * i + 4 * q]);
    of[i] = vec[kVecO * C + 16 * i + l16];
  }
  half4_t Uh[4], Wh[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    Uh[mb] = to_half4(U[mb]);
    Wh[mb] = to_half4(uf[mb] * U[mb]);
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) O[nb] = of[nb] * Yt[nb];
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    const int s2 = 2 * kFragStep[f];
    O[kFragRow[f]] = mfma_f16(cat8(Uh[s2], Uh[s2 + 1]), pf[f], O[kFragRow[f]]);
  }
  o_t0 = t0;
  o_L = min(C, x.end - t0);

  // ---- S^T = gamma S^T + K^T W, W = uf U; K^T rows dk = dk_tile(mb, i / 4) + i % 4 by
  // transposing reads of tokens 32 s + 4 q + i / 4 (first half) and 16 tokens later
  // (second half)
  const float gamma = vec[kVecGamma * C];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) ST[mb] *= gamma;
  // 16 products (s, mb) in groups of four; the transposing reads of group j + 1
  // are issued before the products of group j
  half8_t kt[2][4];
  auto load_kt = [&](int grp, int slot) {
    const int s = grp >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mb = 4 * (grp & 1) + i;
      const half4_t a0 = lds_tr4(Buf::K(), lo.tr[mb] + 32 * s * (D * 2));
      const half4_t a1 = lds_tr4(Buf::K(), lo.tr[mb] + (32 * s + 16) * (D * 2));
      kt[slot][i] = cat8(a0, a1);
    }
  };
  const half8_t w8[2] = {cat8(Wh[0], Wh[1]), cat8(Wh[2], Wh[3])};
  load_kt(0, 0);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    if (grp < 3) load_kt(grp + 1, (grp + 1) & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mb = 4 * (grp & 1) + i;
      ST[mb] = mfma_f16(kt[grp & 1][i], w8[grp >> 1], ST[mb]);
    }
  }
}

template <int NW>
__global__ void __launch_bounds__(ScanCfg<NW>::THREADS) gdn_chunk_scan(ChunkArgs p, Ws w, int n_units) {
  typedef ScanCfg<NW> Cfg;
  constexpr int NT = Cfg::NT, NBUF = Cfg::NBUF, LEAD = NBUF - 1;

  // Work units are (request, key head) pairs, group x NT workgroups each, which
  // share the unit's k and q in L2. Workgroups are dealt to the 8 XCDs round-robin
  // by block index, so unit u goes to XCD u % 8: every XCD gets an equal share of
  // every request, and within an XCD the units run longest request first.
  const int per_unit = p.group * NT;
  const int xcd = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
  const int unit = xcd + 8 * (j / per_unit), m = j % per_unit;
  if (unit >= n_units) return;
  const int req = w.order[unit / p.Hk];
  const int g = unit % p.Hk;
  const int hv = m / NT, tile = m % NT;
  const int h = g * p.group + hv;
  const int d0 = tile * Cfg::TV;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, q = lane >> 4;

  const int beg = seq_start(p, req);
  const int end = max(seq_start(p, req + 1), beg);
  const int slot0 = w.chunk_start[req];
  int nch = (end - beg + C - 1) / C;
  nch = max(0, min(nch, p.max_chunks - slot0));

  if (wave >= NW) {
    // ---- loader waves: chunks 0 .. LEAD - 1 (a missing chunk has length 0: its
    // loads read nothing), then chunk c + LEAD after the barrier of chunk c
    const int loader = wave - NW;
    ScanCtx x{p, w, h, g, d0, 0, loader, lane, beg, end, slot0, nch};
    auto stage_first = [&](auto bc) {
      constexpr int b = decltype(bc)::value;
      Stage<NW, b>(p, w, nch > b ? slot0 + b : slot0, beg + C * b, nch > b ? min(C, end - beg - C * b) : 0, h, g,
                   d0, loader, lane)
          .all();
    };
    stage_first(std::integral_constant<int, 0>());
    if constexpr (LEAD > 1) stage_first(std::integral_constant<int, 1>());
    // L2 prefetch of chunks LEAD .. LEAD + kTouchAhead - 1 (the later ones go with the loader steps)
    const int sub = hv * NT + tile, nshare = p.group * NT;
#pragma unroll
    for (int ca = LEAD; ca < LEAD + kTouchAhead; ++ca) {
      const bool ahead = ca < nch;
      const int ta = beg + C * ca;
      touch_chunk<NW>(x, ahead ? slot0 + ca : slot0, ta, ahead ? min(C, end - ta) : 0, loader, sub, nshare, tile);
    }
    int c = 0;
    if constexpr (NBUF == 3) {
      for (; c + 2 < nch; c += 3) {
        loader_step<NW, 0>(x, c, loader, sub, nshare, tile);
        loader_step<NW, 1>(x, c + 1, loader, sub, nshare, tile);
        loader_step<NW, 2>(x, c + 2, loader, sub, nshare, tile);
      }
      if (c < nch) loader_step<NW, 0>(x, c, loader, sub, nshare, tile);
      if (c + 1 < nch) loader_step<NW, 1>(x, c + 1, loader, sub, nshare, tile);
    } else {
      for (; c + 1 < nch; c += 2) {
        loader_step<NW, 0>(x, c, loader, sub, nshare, tile);
        loader_step<NW, 1>(x, c + 1, loader, sub, nshare, tile);
      }
      if (c < nch) loader_step<NW, 0>(x, c, loader, sub, nshare, tile);
    }
    // the last loads fill buffers that no one reads; let them land before the
    // wave ends
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // ---- state rows of this wave, transposed: ST[mb] = S[dv][dk = dk_tile(mb, q) + e], dv = dvw + l16
  const int dvw = d0 + kRowsPerWave * wave;
  float4_t ST[8];
  const float* init = state_head(p.initial_state, state_slot(p.initial_slots, req, p.num_slots), p.Hv, h,
                                (size_t)D * D);
  float* fin = state_head(p.final_state, state_slot(p.final_slots, req, p.num_slots), p.Hv, h, (size_t)D * D);
  // V-major: S[dv][dk .. dk+3] is one 16-byte vector; K-major (the transpose,
  // [Dk, Dv]): four scalars a row apart. Once per workgroup either way.
  const bool kmaj = p.k_major != 0;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    ST[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (init != nullptr && !kmaj)
      ST[mb] = *reinterpret_cast<const float4_t*>(init + (size_t)(dvw + l16) * D + dk_tile(mb, q));
    if (init != nullptr && kmaj) {
      const float* c0 = init + (size_t)dk_tile(mb, q) * D + dvw + l16;
      ST[mb] = float4_t{c0[0], c0[D], c0[2 * D], c0[3 * D]};
    }
  }

  ScanCtx x{p, w, h, g, d0, dvw, wave, lane, beg, end, slot0, nch};
  const LaneOffsets lo = lane_offsets<NW>(wave, lane);
  float4_t O[4];
  int o_t0 = beg, o_L = 0;                 // output rows of the previous chunk, stored one step late
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) O[nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // NBUF chunks per iteration, one LDS buffer each (one barrier per chunk, as the loaders)
  int c = 0;
  if constexpr (NBUF == 3) {
    for (; c + 2 < nch; c += 3) {
      scan_step<NW, 0>(x, lo, c, ST, O, o_t0, o_L);
      scan_step<NW, 1>(x, lo, c + 1, ST, O, o_t0, o_L);
      scan_step<NW, 2>(x, lo, c + 2, ST, O, o_t0, o_L);
    }
    if (c < nch) scan_step<NW, 0>(x, lo, c, ST, O, o_t0, o_L);
    if (c + 1 < nch) scan_step<NW, 1>(x, lo, c + 1, ST, O, o_t0, o_L);
  } else {
    for (; c + 1 < nch; c += 2) {
      scan_step<NW, 0>(x, lo, c, ST, O, o_t0, o_L);
      scan_step<NW, 1>(x, lo, c + 1, ST, O, o_t0, o_L);
    }
    if (c < nch) scan_step<NW, 0>(x, lo, c, ST, O, o_t0, o_L);
  }

  // ---- output of the last chunk, final state
  __builtin_amdgcn_s_waitcnt(0);
  store_out(x, O, o_t0, o_L);
  if (fin != nullptr && !kmaj) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      *reinterpret_cast<float4_t*>(fin + (size_t)(dvw + l16) * D + dk_tile(mb, q)) = ST[mb];
  }
  if (fin != nullptr && kmaj) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      float* c0 = fin + (size_t)dk_tile(mb, q) * D + dvw + l16;
      c0[0] = ST[mb].x; c0[D] = ST[mb].y; c0[2 * D] = ST[mb].z; c0[3 * D] = ST[mb].w;
    }
  }
}

// ----------------------------------------------------------------------------
// gdn_chunk_prep: one workgroup per (chunk slot, key head g), for the G value
// heads h = g G .. g G + G - 1 that share g's keys and queries
//
//   K, Q tiles -> LDS (direct loads, the scan's swizzled layout); the raw gates of
//   up to four heads are loaded meanwhile (wave w: head w of each batch of four)
//   Gram tiles on fp16 MFMA, once for all G heads; wave w = row block w, taken
//   transposed:
//     K_nb K_w^T and K_nb Q_w^T (nb <= w), Q_w Q_w^T
//   so that lane (l16, q) of tile nb holds row r = 16 w + l16, columns
//   i = 16 nb + 4 q + e of K K^T and Q K^T: P's MFMA fragment layout (frag_col),
//   and one decay factor e^{g_r - g_i} serves both A and P
//   norms from the Gram diagonals: rk_t = (k_t.k_t + eps)^-1/2, rq_t likewise times
//   the scale; the normalized, masked Gram values stay in registers:
//     kn = rk_r rk_i (K K^T)_ri (i < r),  pn = rq_r rk_i (Q K^T)_ri (i <= r)
//   per value head h:
//     cumulative log decay g and beta of h; the per-token factors
//     P = e^{g_r - g_i} pn (MFMA fragments, straight from registers)
//     A = beta_r e^{g_r - g_i} kn
//     T = (I + A)^-1 blockwise from 16x16 blocks: the diagonal blocks by forward
//     substitution, the blocks below the diagonal column by column,
//       T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj,
//     on fp32 MFMA (waves 0, 1, 2 take block columns 0, 1, 2); T' = T diag(beta).
// The K, Q tiles are dead once the Gram tiles are in registers; A and T reuse
// their LDS, which keeps a workgroup at 40 KiB (four per CU).
// ----------------------------------------------------------------------------
constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / 64;

struct PrepSmem {
  union {
    _Float16 kq[2][C * D];        // K, Q tiles, units permuted by kv_swizzle
    struct {
      float A[C * AS];
      float T[C * AS];            // blocks on and below the diagonal
    } m;
  } u;
  float wtmp[4][16 * 17];         // per-wave 16x16 staging for MFMA operands
  float g[2][C], beta[2][C];      // gates of the current head (alternate buffers)
  float rk[C], rq[C];
};

// row block of the Gram/P tiles -> fragment indices (kFragRow / kFragStep order)
__device__ __forceinline__ int frag_index(int rb, int s) { return rb == 3 ? 4 + s : rb == 2 ? 2 + s : rb; }

// Raw gates of head h at token t (rows >= L read as zero).
struct RawGates {
  float a, b;
};
// An input the update rule does not read gets an empty range (it reads as zero).
__device__ __forceinline__ RawGates load_gates(const ChunkArgs& p, int t0, int L, int h, int t) {
  const int gate_bytes = ((L - 1) * p.Hv + 1) * 4;
  const size_t off = (size_t)t0 * p.Hv + h;
  RawGates r;
  r.a = buf_load_f32(make_rsrc(p.gated ? p.a + off : nullptr, p.gated ? gate_bytes : 0), t * p.Hv * 4);
  r.b = buf_load_f32(make_rsrc(p.delta ? p.b + off : nullptr, p.delta ? gate_bytes : 0), t * p.Hv * 4);
  return r;
}

// Cumulative log decay (inclusive prefix sum over the 64 lanes = tokens) and beta
// of head h; tokens >= L get log decay 0 and beta 0. Without the rule's gate the
// log decay is 0; without its delta correction beta is 1 (T' = I; A and the
// correction factor are zeroed where they are formed).
__device__ __forceinline__ void gates_of(const ChunkArgs& p, int h, int L, int t, RawGates r, float* g,
                                         float* beta) {
  float la = 0.f, be = 0.f;
  if (t < L) {
    const bool gnone = p.gate_none != 0;           // A_log, dt_bias may be null then
    if (p.gated)
      la = gate_log_alpha(r.a, gnone, gnone ? 0.f : expf(p.A_log[h]), gnone ? 0.f : p.dt_bias[h]);
    be = p.delta ? gate_beta(r.b, gnone) : 1.f;
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(la, d, 64);
    if (t >= d) la += y;
  }
  *g = la;
  *beta = be;
}

__global__ void __launch_bounds__(kPrepThreads) gdn_chunk_prep(ChunkArgs p, Ws w, int n_items) {
  __shared__ PrepSmem sm;
  const int item = (int)blockIdx.x;
  if (item >= n_items) return;
  const int slot = item / p.Hk, g = item % p.Hk;
  int req, t0, L;
  if (!locate_chunk(p, w, slot, &req, &t0, &L)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int G = p.group, h0 = g * G;

  // ---- K, Q tiles into LDS (rows >= L read as zero): wave w copies rows 16 w .. 16 w + 15
  {
    const int krow = p.Hk * D;
    const size_t kq_base = ((size_t)t0 * p.Hk + g) * D;
    const int kq_bytes = ((L - 1) * krow + D) * 2;
    const rsrc_t rk = make_rsrc(static_cast<const _Float16*>(p.k) + kq_base, kq_bytes);
    const rsrc_t rq = make_rsrc(static_cast<const _Float16*>(p.q) + kq_base, kq_bytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * j + (lane >> 4);
      const int off = row * krow * 2 + 16 * ((lane & 15) ^ kv_swizzle(row));
      const int blk = 4 * wave + j;                       // rows 4 blk .. 4 blk + 3
      load_lds16(rk, sm.u.kq[0] + 4 * blk * D, off, 16 * wave * krow * 2);
      load_lds16(rq, sm.u.kq[1] + 4 * blk * D, off, 16 * wave * krow * 2);
    }
  }
  // gates of the first batch of heads (wave w: head h0 + w) while the tiles are in flight
  float gw = 0.f, bw = 0.f;
  if (wave < G) gates_of(p, h0 + wave, L, lane, load_gates(p, t0, L, h0 + wave, lane), &gw, &bw);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  // ---- Gram tiles of row block wave
  float4_t kk[4], kq[4], qq = float4_t{0.f, 0.f, 0.f, 0.f};
  {
    const _Float16* Kt = sm.u.kq[0];
    const _Float16* Qt = sm.u.kq[1];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      kk[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
      kq[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int sw = kv_swizzle(l16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int uoff = 16 * ((4 * ks + q) ^ sw);
      const half8_t kw = lds_b128(Kt, (16 * wave + l16) * (D * 2) + uoff);
      const half8_t qw = lds_b128(Qt, (16 * wave + l16) * (D * 2) + uoff);
      half8_t kn[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) kn[nb] = lds_b128(Kt, (16 * nb + l16) * (D * 2) + uoff);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (nb <= wave) {
          kk[nb] = mfma_f16(kn[nb], kw, kk[nb]);    // KK[16 w + l16][16 nb + 4q + e]
          kq[nb] = mfma_f16(kn[nb], qw, kq[nb]);    // QK[16 w + l16][16 nb + 4q + e]
        }
      }
      qq = mfma_f16(qw, qw, qq);
    }
  }
  // norms: the diagonal element of row 16 w + l16 sits in lane group q = l16 / 4, element e = l16 % 4
  {
    float4_t kd = kk[0];
#pragma unroll
    for (int nb = 1; nb < 4; ++nb)
      if (nb == wave) kd = kk[nb];
    const int e = l16 & 3;
    const float kdiag = e == 0 ? kd[0] : e == 1 ? kd[1] : e == 2 ? kd[2] : kd[3];
    const float qdiag = e == 0 ? qq[0] : e == 1 ? qq[1] : e == 2 ? qq[2] : qq[3];
    if (q == (l16 >> 2)) {
      sm.rk[16 * wave + l16] = rsqrtf(kdiag + kNormEps);
      sm.rq[16 * wave + l16] = rsqrtf(qdiag + kNormEps) * p.scale;
    }
  }
  lds_barrier();                                   // K, Q tiles dead from here; their LDS becomes A, T

  // ---- normalized, masked Gram values of row r = 16 w + l16, columns i = 16 nb + 4 q + e
  const int r = 16 * wave + l16;
  {
    const float rkr = sm.rk[r], rqr = sm.rq[r];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const float4_t ki = *reinterpret_cast<const float4_t*>(&sm.rk[16 * nb + 4 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * nb + 4 * q + e;
        kk[nb][e] = i < r ? rkr * ki[e] * kk[nb][e] : 0.f;
        kq[nb][e] = i <= r ? rqr * ki[e] * kq[nb][e] : 0.f;
      }
    }
  }
  float* const A = sm.u.m.A;
  float* const T = sm.u.m.T;

  for (int hb = 0; hb < G; hb += kPrepWaves) {
    if (hb > 0 && wave < G - hb) gates_of(p, h0 + hb + wave, L, lane, load_gates(p, t0, L, h0 + hb + wave, lane), &gw, &bw);
    for (int hh = 0; hh < min(kPrepWaves, G - hb); ++hh) {
      const int h = h0 + hb + hh;
      const int gb = (hb + hh) & 1;                // gate buffer of this head
      float* const gs = sm.g[gb];
      float* const bs = sm.beta[gb];
      if (wave == hh) {
        gs[lane] = gw;
        bs[lane] = bw;
      }
      lds_barrier();

      // ---- per-token factors, one row per wave:
      //   kVecZ e^{g_t} rk_t, kVecO e^{g_t} rq_t, kVecU e^{g_L - g_t} rk_t, kVecGamma e^{g_L}
      {
        const int t = lane;
        const float gt = gs[t], gL = gs[C - 1];
        const float v = wave == kVecZ ? (p.delta ? expf(gt) * sm.rk[t] : 0.f)
                      : wave == kVecO ? expf(gt) * sm.rq[t]
                      : wave == kVecU ? expf(gL - gt) * sm.rk[t]
                                      : expf(gL);
        w.vec[((size_t)slot * p.Hv + h) * kVecRows * C + wave * C + t] = v;
      }

      // ---- A (rows 16 w + l16 of the fp32 LDS matrix; the blocks above the diagonal
      // are never read) and the P fragments of row block w, from one decay factor
      // per element. T' and P go out by nontemporal stores: the scan reads them
      // once, well after this workgroup (long prefill 790 -> 778 us)
      {
        const float gr = gs[r], br = p.delta ? bs[r] : 0.f;   // A = 0 without the delta correction
        half4_t ph[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          ph[nb] = half4_t{0, 0, 0, 0};                 // blocks above the diagonal
          if (nb <= wave) {
            const float4_t gi = *reinterpret_cast<const float4_t*>(&gs[16 * nb + 4 * q]);
            float4_t av;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float dec = fast_exp(fminf(gr - gi[e], 0.f));
              av[e] = br * dec * kk[nb][e];
              ph[nb][e] = (_Float16)(dec * kq[nb][e]);
            }
            *reinterpret_cast<float4_t*>(&A[r * AS + 16 * nb + 4 * q]) = av;
          }
        }
        _Float16* Pw = w.P + ((size_t)slot * p.Hv + h) * kFragHalves;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (2 * s <= wave)
            __builtin_nontemporal_store(cat8(ph[2 * s], ph[2 * s + 1]), reinterpret_cast<half8_t*>(Pw + frag_index(wave, s) * 512 + lane * 8));
      }
      lds_barrier();

      // ---- T, step 1: the four diagonal 16x16 blocks (wave 0, lane = 16 block + column)
      if (wave == 0) {
        const int blk = lane >> 4, j = lane & 15;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) x[rr] = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float* arow = &A[(16 * blk + rr) * AS + 16 * blk];
          float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
          for (int i = 0; i < rr; i += 4) {
            const float4_t a4 = *reinterpret_cast<const float4_t*>(&arow[i]);
            s0 = fmaf(a4.x, x[i], s0);
            s1 = fmaf(a4.y, x[i + 1], s1);
            s2 = fmaf(a4.z, x[i + 2], s2);
            s3 = fmaf(a4.w, x[i + 3], s3);
          }
          x[rr] = (rr == j ? 1.f : 0.f) - ((s0 + s1) + (s2 + s3));
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) T[(16 * blk + rr) * AS + 16 * blk + j] = x[rr];
      }
      lds_barrier();

      // ---- T, step 2: blocks below the diagonal; wave j sweeps block column j
      if (wave < 3) {
        float* wt = sm.wtmp[wave];
        for (int ib = wave + 1; ib < 4; ++ib) t_offdiag_block(A, T, wt, ib, wave, lane);
      }
      lds_barrier();

      // ---- T' = T diag(beta) fragments of row block w (blocks above the diagonal are zero)
      {
        _Float16* Tw = w.T + ((size_t)slot * p.Hv + h) * kFragHalves;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (2 * s <= wave) {
            half8_t x;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int c = frag_col(s, q, j);
              x[j] = (c >> 4) <= wave ? (_Float16)(T[r * AS + c] * bs[c]) : (_Float16)0.f;
            }
            __builtin_nontemporal_store(x, reinterpret_cast<half8_t*>(Tw + frag_index(wave, s) * 512 + lane * 8));
          }
        }
      }
      // the next head's gates go to the other buffer, and its first LDS writes
      // come after one more barrier
    }
  }
}

size_t chunk_workspace_bytes(int64_t chunk_slots, int R, int Hk, int Hv) {
  return ws_bytes(chunk_slots, R, Hk, Hv);
}

hipError_t launch_chunk(const ChunkArgs& p, int io_dtype, hipStream_t stream) {
  if (io_dtype != 1) return hipErrorInvalidValue;     // fp16 I/O only
  if (p.R == 0) return hipSuccess;
  const Ws w = ws_layout(p.workspace, p.max_chunks, p.R, p.Hk, p.Hv);
  hipLaunchKernelGGL(gdn_chunk_index, dim3(1), dim3(kThreads), 0, stream, p, w);
  if (p.max_chunks > 0) {
    const int n_prep = p.max_chunks * p.Hk;
    hipLaunchKernelGGL(gdn_chunk_prep, dim3((unsigned)n_prep), dim3(kPrepThreads), 0, stream, p, w, n_prep);
  }
  // Both scan configurations hold one workgroup per CU. 64-row tiles move half the
  // k, q, T', P bytes per state row; they are taken when their workgroups fill
  // every CU at least once, else 32-row tiles keep twice as many CUs busy.
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int n_units = p.R * p.Hk;
  const int units_padded = 8 * ((n_units + 7) / 8);
  if ((int64_t)n_units * p.group * ScanCfg<4>::NT >= n_cu) {
    const int grid = units_padded * p.group * ScanCfg<4>::NT;
    hipLaunchKernelGGL(gdn_chunk_scan<4>, dim3((unsigned)grid), dim3(ScanCfg<4>::THREADS), 0, stream, p, w, n_units);
  } else {
    const int grid = units_padded * p.group * ScanCfg<2>::NT;
    hipLaunchKernelGGL(gdn_chunk_scan<2>, dim3((unsigned)grid), dim3(ScanCfg<2>::THREADS), 0, stream, p, w, n_units);
  }
  return hipGetLastError();
}

}  // namespace gdn

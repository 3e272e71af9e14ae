// gdn_replay: advance the committed state by an accepted capsule prefix and
// write the result into an inactive state bank ("Replay compact fixed state
// for hybrid decoding", Summary and Key Changes: compact prefix replay into
// double-buffered banks).
//
//   dst[r,h] = src[r,h];  for j < m_r:  dst[r,h] = alpha_j * dst[r,h] + u_j k^_j^T
//
// A pure stream: every state element is read once from the committed bank and
// written once to the inactive bank (nontemporal, so the streams do not evict
// cached data); the m_r rank-1 updates run in registers.
// A workgroup owns one (request, value head) slice of Dv x Dk floats, in either
// state layout; the capsule values it needs per row are read through the cache
// (the capsule is small and shared by a head's threads).
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

// ROW is the length of a stored state row: Dk for the V-major layout (rows are
// dv), Dv for the K-major one (rows are dk). A thread owns one 16-byte group of
// 4 row elements in rows t / (ROW/4) + (256/(ROW/4)) i. Per capsule row it needs
// a 4-vector and one scalar per row: V-major the key k^[4 dk] and u[dv = row],
// K-major u[4 dv] and k^[dk = row].
template <int ROW, bool KMAJOR>
__global__ void __launch_bounds__(256) gdn_replay(ReplayArgs p) {
  constexpr int C4 = ROW / 4;         // 16-byte groups per row
  constexpr int RPP = 256 / C4;       // rows per pass of the block
  constexpr int ITERS = 128 / RPP;    // passes: the block covers up to 128 rows
  const int tid = threadIdx.x;
  const int c4 = tid % C4;
  const int rsub = tid / C4;

  const int h = blockIdx.x % p.Hv;
  const int r = blockIdx.x / p.Hv;
  const int g = h / p.group;
  const int rows = KMAJOR ? p.Dk : p.Dv;
  const size_t head_elems = (size_t)p.Dv * p.Dk;
  const float* src = state_head(p.src, state_slot(p.src_slots, r, p.num_slots), p.Hv, h, head_elems);
  float* dst = state_head(p.dst, state_slot(p.dst_slots, r, p.num_slots), p.Hv, h, head_elems);
  if (dst == nullptr) return;                      // no slot to write

  float4_t S[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = rsub + RPP * it;
    S[it] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (row < rows && src != nullptr)
      S[it] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(src + (size_t)row * ROW + 4 * c4));
  }

  const int m = min(max(p.accepted[r], 0), p.capacity);
  const float* caprow = p.capsule + (size_t)r * p.capacity * p.capsule_width;
  const int key_off = p.Hv + g * p.Dk;
  const int delta_off = p.Hv + p.Hk * p.Dk + h * p.Dv;
  const int vec_off = (KMAJOR ? delta_off : key_off) + 4 * c4;     // the 4-vector of this thread
  const int row_off = KMAJOR ? key_off : delta_off;                // the per-row scalars
  for (int j = 0; j < m; ++j, caprow += p.capsule_width) {
    const float alpha = caprow[h];
    const float4_t w = {caprow[vec_off], caprow[vec_off + 1], caprow[vec_off + 2], caprow[vec_off + 3]};
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int row = rsub + RPP * it;
      const float s = row < rows ? caprow[row_off + row] : 0.f;
      S[it].x = fmaf(alpha, S[it].x, s * w.x);
      S[it].y = fmaf(alpha, S[it].y, s * w.y);
      S[it].z = fmaf(alpha, S[it].z, s * w.z);
      S[it].w = fmaf(alpha, S[it].w, s * w.w);
    }
  }

#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int row = rsub + RPP * it;
    if (row < rows)
      __builtin_nontemporal_store(S[it], reinterpret_cast<float4_t*>(dst + (size_t)row * ROW + 4 * c4));
  }
}

// Double-buffered publication: after a replay has written every request's
// inactive slot, the two slot arrays trade places, so the slot just written
// becomes the committed one and the old committed slot the next inactive one.
__global__ void __launch_bounds__(256) gdn_publish(int32_t R, int32_t* committed, int32_t* inactive) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const int32_t c = committed[r];
  committed[r] = inactive[r];
  inactive[r] = c;
}

hipError_t launch_publish(int32_t R, int32_t* committed, int32_t* inactive, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(gdn_publish, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, stream, R, committed, inactive);
  return hipGetLastError();
}

hipError_t launch_replay(const ReplayArgs& p, hipStream_t stream) {
  if (p.R == 0) return hipSuccess;
  const dim3 grid((unsigned)((size_t)p.R * p.Hv));
  const dim3 block(256);
  const int row = p.k_major ? p.Dv : p.Dk;
  switch (row * 2 + (p.k_major ? 1 : 0)) {
    case 32: hipLaunchKernelGGL((gdn_replay<16, false>), grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL((gdn_replay<32, false>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((gdn_replay<64, false>), grid, block, 0, stream, p); break;
    case 256: hipLaunchKernelGGL((gdn_replay<128, false>), grid, block, 0, stream, p); break;
    case 33: hipLaunchKernelGGL((gdn_replay<16, true>), grid, block, 0, stream, p); break;
    case 65: hipLaunchKernelGGL((gdn_replay<32, true>), grid, block, 0, stream, p); break;
    case 129: hipLaunchKernelGGL((gdn_replay<64, true>), grid, block, 0, stream, p); break;
    case 257: hipLaunchKernelGGL((gdn_replay<128, true>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn

// Compact causal convolution: gdn_conv_forward, gdn_conv_final, gdn_conv_replay.
//
// The depthwise causal conv1d + SiLU with a carried state upstream of the
// GatedDeltaNet operator ("[CUDA] Add compact GatedDeltaNet operator", the
// embedded VarlenCausalConv commit): per request and channel, with the K - 1
// carried inputs s (oldest first) and the request's inputs x_0 .. x_{L-1},
//   e = [s, x],  out_j = act(bias + sum_{i<K} w[i] e[j + i]),  final = e[L .. L+K-2],
// and the inputs of the leading n_r tokens captured for prefix replay.
//
// The operator moves each input and output once and does K multiply-adds per
// element, so it is bound by HBM. A thread owns 4 adjacent channels (one 8- or
// 16-byte vector per token, coalesced across the workgroup) and walks a block of
// packed tokens with the last K - 1 inputs of each channel in registers; a block
// may cross request boundaries, where the window restarts from the next
// request's carried state. Blocks are independent, so long sequences spread
// over the whole chip. The workgroup that convolves a request's last token
// writes that request's final state from its window. An in-place update
// (final_state == initial_state) is race-free that way only when the request's
// tokens all fall in that one workgroup; in-place requests that span
// workgroups, and empty requests, are written by a small final-state kernel
// that runs after the convolution.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kConvThreads = kConvBlockThreads;
constexpr int kConvChannelsPerBlock = 4 * kConvThreads;
// Tokens whose inputs a thread loads before using any (the loop's unroll): one
// round for a whole block of up to kConvUnrollLong tokens, so that a thread keeps
// all of its loads in flight at once (ragged prefill, 15 tokens per block: 92 ->
// 88 us against two rounds of 8); blocks of a few tokens (decode) take the short
// loop, which issues fewer redundant loads past their last token.
constexpr int kConvUnrollLong = 16, kConvUnrollShort = 4;

// The output is a stream written once: nontemporal stores (ragged prefill
// 103 -> 83..90 us). Nontemporal loads of x were slower: a block re-reads the K - 1
// rows before its first token, which the previous block has just read.
template <typename IO> struct Io4;
template <> struct Io4<float> {
  static __device__ __forceinline__ float4_t load(const float* p) { return *reinterpret_cast<const float4_t*>(p); }
  static __device__ __forceinline__ void store_stream(float* p, float4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<float4_t*>(p));
  }
};
template <> struct Io4<_Float16> {
  static __device__ __forceinline__ float4_t load(const _Float16* p) {
    const half4_t h = *reinterpret_cast<const half4_t*>(p);
    return float4_t{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
  }
  static __device__ __forceinline__ void store_stream(_Float16* p, float4_t v) {
    const half4_t h = half4_t{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    __builtin_nontemporal_store(h, reinterpret_cast<half4_t*>(p));
  }
};

// Request that holds packed token t (t < N, the same t in every thread of the
// workgroup): the last r with seq_start(r) <= t, which skips empty requests.
// The workgroup searches cooperatively: each round, its threads test evenly
// spaced candidates at once and the count of those at or before t narrows the
// range by the workgroup size, so R <= 256 takes a single round of loads. Every
// thread of the workgroup must call it. The result lies in [0, R) whatever
// cu_seqlens holds.
__device__ __forceinline__ int request_of_block(const ConvArgs& p, int t) {
  if (p.cu_seqlens == nullptr) return t / p.dense_len;
  __shared__ int counts[2][kConvThreads / 64];
  int lo = 0, n = p.R, round = 0;
  while (n > 1) {
    const int stride = (n + kConvThreads - 1) / kConvThreads;
    const int off = threadIdx.x * stride;
    const bool at_or_before = off < n && seq_start(p, lo + off) <= t;
    const unsigned long long ballot = __ballot(at_or_before);
    if ((threadIdx.x & 63) == 0) counts[round & 1][threadIdx.x >> 6] = __popcll(ballot);
    __syncthreads();
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kConvThreads / 64; ++w) cnt += counts[round & 1][w];
    cnt = max(cnt, 1);
    lo += (cnt - 1) * stride;
    n = min(stride, n - (cnt - 1) * stride);
    ++round;
  }
  return lo;
}

// Captured rows of request r of length L.
__device__ __forceinline__ int capture_rows(const ConvArgs& p, int r, int L) {
  int n = p.capacity;
  if (p.capture_count != nullptr) n = min(max(p.capture_count[r], 0), p.capacity);
  return min(L, n);
}

// n floats of a thread's 4 channels, stored channel-major ([channel][n]) and
// 16-byte aligned, as v[n][channel].
template <int n>
__device__ __forceinline__ void load_channel_major(const float* base, float (&v)[n][4]) {
  float f[4 * n];
#pragma unroll
  for (int i = 0; i < n; ++i) {
    const float4_t x = *reinterpret_cast<const float4_t*>(base + 4 * i);
    f[4 * i + 0] = x.x; f[4 * i + 1] = x.y; f[4 * i + 2] = x.z; f[4 * i + 3] = x.w;
  }
#pragma unroll
  for (int ch = 0; ch < 4; ++ch)
#pragma unroll
    for (int m = 0; m < n; ++m) v[m][ch] = f[ch * n + m];
}

template <int n>
__device__ __forceinline__ void store_channel_major(float* base, const float (&v)[n][4]) {
#pragma unroll
  for (int i = 0; i < n; ++i)
    *reinterpret_cast<float4_t*>(base + 4 * i) =
        float4_t{v[(4 * i + 0) % n][(4 * i + 0) / n], v[(4 * i + 1) % n][(4 * i + 1) / n],
                 v[(4 * i + 2) % n][(4 * i + 2) / n], v[(4 * i + 3) % n][(4 * i + 3) / n]};
}

template <typename IO>
__device__ __forceinline__ void load_io4(const IO* p, float (&dst)[4]) {
  const float4_t v = Io4<IO>::load(p);
  dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}

// The carried inputs of one request's state slot, seen through a raw buffer
// resource with a range check: the slot's C x (K - 1) floats, or an empty range
// when there is no state array or no slot, so that every load from it is
// unconditional and reads zero in the empty case. `off` is this thread's byte
// offset (its 4 channels' K - 1 entries each, channel-major).
struct StateRef {
  rsrc_t rs;
  int off;
};

template <typename T>
__device__ __forceinline__ StateRef state_ref(T* s, int slot, int C, int c, int K) {
  const bool any = s != nullptr && slot >= 0;
  return StateRef{make_rsrc(any ? static_cast<const void*>(s + (size_t)slot * C * (K - 1)) : nullptr,
                            any ? C * (K - 1) * 4 : 0),
                  c * (K - 1) * 4};
}

// e[idx .. idx + K - 2] of one request for 4 channels (e = [carried state, the
// inputs from token `start` on], idx >= 0). idx is uniform across the
// workgroup. The two common cases, all from the state (idx = 0) and all from
// the inputs (idx >= K - 1), issue their loads back to back; the mixed case
// reads entry by entry. No register array is indexed at run time.
template <typename IO, int K>
__device__ __forceinline__ void window_at(const IO* x, int C, int c, int start, int idx, StateRef st,
                                          float (&win)[K - 1][4]) {
  if (idx == 0) {
    // float 4 i + j of the thread's run is entry m = (4 i + j) mod (K - 1) of
    // channel (4 i + j) / (K - 1)
#pragma unroll
    for (int i = 0; i < K - 1; ++i) {
      const float4_t v = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(st.rs, st.off + 16 * i, 0, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) win[(4 * i + j) % (K - 1)][(4 * i + j) / (K - 1)] = v[j];
    }
  } else if (idx >= K - 1) {
    const IO* row = x + (size_t)(start + idx - (K - 1)) * C + c;
#pragma unroll
    for (int m = 0; m < K - 1; ++m) {
      const float4_t v = Io4<IO>::load(row + (size_t)m * C);
      win[m][0] = v.x; win[m][1] = v.y; win[m][2] = v.z; win[m][3] = v.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < K - 1; ++m) {
      const int e = idx + m;
      if (e >= K - 1) {
        const float4_t v = Io4<IO>::load(x + (size_t)(start + e - (K - 1)) * C + c);
        win[m][0] = v.x; win[m][1] = v.y; win[m][2] = v.z; win[m][3] = v.w;
      } else {
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) win[m][ch] = buf_load_f32(st.rs, st.off + (ch * (K - 1) + e) * 4);
      }
    }
  }
}

// This thread's K - 1 entries of 4 channels in the state of `slot` (see
// state_slot), or null when there is no state array or no slot.
template <typename T>
__device__ __forceinline__ T* state_of(T* s, int slot, int C, int c, int K) {
  return (s != nullptr && slot >= 0) ? s + ((size_t)slot * C + c) * (K - 1) : nullptr;
}

// Workgroups are numbered channel group fastest (token block = blockIdx.x /
// groups): the workgroups running together cover whole rows of x and output
// rather than one column slice of many rows, and the workgroup that continues a
// channel group's tokens runs on the same XCD as the one before it, whose rows
// its window re-reads.
template <typename IO, int K, int U>
__global__ void __launch_bounds__(kConvThreads) gdn_conv_forward_k(ConvArgs p) {
  const int groups = (p.C + kConvChannelsPerBlock - 1) / kConvChannelsPerBlock;
  const int c = 4 * ((int)(blockIdx.x % groups) * kConvThreads + threadIdx.x);
  const int tb = p.tokens_per_block;
  const int t_begin = (int)(blockIdx.x / groups) * tb;
  const int t_end = min(t_begin + tb, p.N);
  if (t_begin >= t_end) return;                              // uniform across the workgroup
  int r = request_of_block(p, t_begin);
  if (c >= p.C) return;
  const IO* __restrict__ x = static_cast<const IO*>(p.x);
  IO* __restrict__ out = static_cast<IO*>(p.output);

  float w[K][4], bias[4];
  load_channel_major<K>(p.weight + (size_t)c * K, w);
  {
    const rsrc_t rb = make_rsrc(p.bias, p.bias != nullptr ? p.C * 4 : 0);   // no bias: zeros
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) bias[ch] = buf_load_f32(rb, (c + ch) * 4);
  }

  // the K - 1 inputs before token t_begin: e[j .. j + K - 2], j = t_begin - start
  int start = seq_start(p, r), end = max(seq_start(p, r + 1), start);
  int ncap = p.state_update != nullptr ? capture_rows(p, r, end - start) : 0;
  float win[K - 1][4];
  window_at<IO, K>(x, p.C, c, start, max(t_begin - start, 0), state_ref(p.initial_state, state_slot(p.initial_slots, r, p.num_slots), p.C, c, K), win);

  int t = t_begin;
  while (t < t_end) {
    if (t >= end) {                                          // next non-empty request
      while (r + 1 < p.R && seq_start(p, r + 1) <= t) ++r;
      start = seq_start(p, r);
      end = max(seq_start(p, r + 1), start);
      ncap = p.state_update != nullptr ? capture_rows(p, r, end - start) : 0;
      window_at<IO, K>(x, p.C, c, start, 0, state_ref(p.initial_state, state_slot(p.initial_slots, r, p.num_slots), p.C, c, K), win);
    }
    const int stop = min(t_end, max(end, t + 1));           // this request's tokens here
    // U tokens' inputs are loaded before any of them is used, so a thread keeps
    // several loads in flight instead of waiting on each in turn
    for (; t < stop; t += U) {
      // loads past `stop` repeat the last token's row (in bounds, unused), so
      // none of them waits behind a branch
      float4_t xs[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        xs[u] = Io4<IO>::load(x + (size_t)min(t + u, stop - 1) * p.C + c);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t + u >= stop) break;
        const float xv[4] = {xs[u].x, xs[u].y, xs[u].z, xs[u].w};
        float y[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          float z = bias[ch];
#pragma unroll
          for (int m = 0; m < K - 1; ++m) z = fmaf(w[m][ch], win[m][ch], z);
          z = fmaf(w[K - 1][ch], xv[ch], z);
          y[ch] = p.silu ? silu(z) : z;
        }
        Io4<IO>::store_stream(out + (size_t)(t + u) * p.C + c, float4_t{y[0], y[1], y[2], y[3]});
        const int j = t + u - start;
        if (j >= 0 && j < ncap)
          *reinterpret_cast<float4_t*>(p.state_update + ((size_t)r * p.capacity + j) * p.C + c) = xs[u];
#pragma unroll
        for (int m = 0; m + 1 < K - 1; ++m)
#pragma unroll
          for (int ch = 0; ch < 4; ++ch) win[m][ch] = win[m + 1][ch];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) win[K - 2][ch] = xv[ch];
      }
    }
    t = stop;
    // the window now holds e[L .. L + K - 2], the request's final state
    if (t == end && p.final_state != nullptr && final_in_forward(start, end, tb, p.final_in_place)) {
      float* fin = state_of(p.final_state, state_slot(p.final_slots, r, p.num_slots), p.C, c, K);
      if (fin != nullptr) store_channel_major<K - 1>(fin, win);
    }
  }
}

// final[r] = e[L .. L + K - 2] for 4 channels per thread, for the requests the
// forward kernel leaves (empty ones, and in-place ones spanning workgroups). It
// runs after the forward kernel and reads every value before writing, so
// final_state may be initial_state.
template <typename IO, int K>
__global__ void __launch_bounds__(kConvThreads) gdn_conv_final_k(ConvArgs p) {
  const int groups = (p.C + kConvChannelsPerBlock - 1) / kConvChannelsPerBlock;
  const int c = 4 * ((int)(blockIdx.x % groups) * kConvThreads + threadIdx.x);
  const int r = (int)(blockIdx.x / groups);
  if (c >= p.C) return;
  const int start = seq_start(p, r), end = max(seq_start(p, r + 1), start);
  if (final_in_forward(start, end, p.tokens_per_block, p.final_in_place)) return;
  float e[K - 1][4];
  window_at<IO, K>(static_cast<const IO*>(p.x), p.C, c, start, end - start,
                   state_ref(p.initial_state, state_slot(p.initial_slots, r, p.num_slots), p.C, c, K), e);
  float* fin = state_of(p.final_state, state_slot(p.final_slots, r, p.num_slots), p.C, c, K);
  if (fin != nullptr) store_channel_major<K - 1>(fin, e);
}

// dst[r] = the last K - 1 of [src[r], capture[r, 0 .. m - 1]], 4 channels per thread.
template <int K>
__global__ void __launch_bounds__(kConvThreads) gdn_conv_replay_k(ConvReplayArgs p) {
  const int groups = (p.C + kConvChannelsPerBlock - 1) / kConvChannelsPerBlock;
  const int c = 4 * ((int)(blockIdx.x % groups) * kConvThreads + threadIdx.x);
  const int r = (int)(blockIdx.x / groups);
  if (c >= p.C) return;
  const int m = min(max(p.accepted[r], 0), p.capacity);
  float e[K - 1][4];
  // the capture rows of request r are its inputs from row 0 on
  float* dst = state_of(p.dst, state_slot(p.dst_slots, r, p.num_slots), p.C, c, K);
  if (dst == nullptr) return;                      // no slot to write
  window_at<float, K>(p.capture + (size_t)r * p.capacity * p.C, p.C, c, 0, m,
                      state_ref(p.src, state_slot(p.src_slots, r, p.num_slots), p.C, c, K), e);
  store_channel_major<K - 1>(dst, e);
}

template <typename IO, int K>
hipError_t launch_conv_k(const ConvArgs& p, hipStream_t stream) {
  const unsigned groups = (unsigned)conv_channel_groups(p.C);
  if (p.N > 0) {
    const unsigned blocks = (unsigned)((p.N + p.tokens_per_block - 1) / p.tokens_per_block);
    if (p.tokens_per_block > kConvUnrollShort)
      hipLaunchKernelGGL((gdn_conv_forward_k<IO, K, kConvUnrollLong>), dim3(blocks * groups), dim3(kConvThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((gdn_conv_forward_k<IO, K, kConvUnrollShort>), dim3(blocks * groups), dim3(kConvThreads), 0,
                         stream, p);
  }
  if (p.final_state != nullptr && p.final_pending)
    hipLaunchKernelGGL((gdn_conv_final_k<IO, K>), dim3((unsigned)p.R * groups), dim3(kConvThreads), 0,
                       stream, p);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_conv_io(const ConvArgs& p, hipStream_t stream) {
  switch (p.K) {
    case 2: return launch_conv_k<IO, 2>(p, stream);
    case 3: return launch_conv_k<IO, 3>(p, stream);
    case 4: return launch_conv_k<IO, 4>(p, stream);
    case 5: return launch_conv_k<IO, 5>(p, stream);
    case 6: return launch_conv_k<IO, 6>(p, stream);
    case 7: return launch_conv_k<IO, 7>(p, stream);
    case 8: return launch_conv_k<IO, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv(const ConvArgs& p, int io_dtype, hipStream_t stream) {
  if (p.R == 0) return hipSuccess;
  return io_dtype == 1 ? launch_conv_io<_Float16>(p, stream) : launch_conv_io<float>(p, stream);
}

hipError_t launch_conv_replay(const ConvReplayArgs& p, hipStream_t stream) {
  if (p.R == 0) return hipSuccess;
  const dim3 grid((unsigned)p.R * (unsigned)conv_channel_groups(p.C));
  switch (p.K) {
    case 2: hipLaunchKernelGGL(gdn_conv_replay_k<2>, grid, dim3(kConvThreads), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(gdn_conv_replay_k<3>, grid, dim3(kConvThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(gdn_conv_replay_k<4>, grid, dim3(kConvThreads), 0, stream, p); break;
    case 5: hipLaunchKernelGGL(gdn_conv_replay_k<5>, grid, dim3(kConvThreads), 0, stream, p); break;
    case 6: hipLaunchKernelGGL(gdn_conv_replay_k<6>, grid, dim3(kConvThreads), 0, stream, p); break;
    case 7: hipLaunchKernelGGL(gdn_conv_replay_k<7>, grid, dim3(kConvThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(gdn_conv_replay_k<8>, grid, dim3(kConvThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn

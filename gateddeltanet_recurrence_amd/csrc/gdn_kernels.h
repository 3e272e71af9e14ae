// Internal launch interface between the C ABI (gdn_api.cpp) and the HIP kernels.
// Not installed; the public interface is include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Arguments of the token-recurrent kernels (decode and capsule capture).
struct RecurrentArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu_seqlens;    // null: dense layout, dense_len tokens per request
  const float* initial_state;   // may be null (zero state)
  float* final_state;           // may be null; may equal initial_state
  void* output;
  float* state_update;          // may be null
  const int32_t* capture_count; // may be null
  int32_t N;                    // packed tokens; device cu_seqlens are clamped to [0, N]
  int32_t R, Hk, Hv, Dk, Dv;
  int32_t group;                // Hv / Hk
  int32_t capacity;
  int32_t capsule_width;        // Hv + Hk*Dk + Hv*Dv
  float scale;
  int32_t dense_len;            // tokens per request when cu_seqlens is null
  int32_t gate_none;            // a, b are the effective alpha, beta (no activation)
  const int32_t* initial_slots; // state pools: slot read / written per request
  const int32_t* final_slots;
  int32_t num_slots;            // 0: states indexed by request
  int32_t k_major;              // states stored [.., Dk, Dv] (else V-major [.., Dv, Dk])
  int32_t gated;                // update rule applies the decay alpha (else alpha = 1, a not read)
  int32_t delta;                // update rule writes beta (v - alpha S k^) (else v, b not read)
  // Fused replay (capsule capture only, V-major): before the tokens, the leading
  // accepted[r] rows of replay_capsule are applied to the initial state and the
  // result is written to replay_state, at the slot final_slots names with pools
  // (the final state is not written then).
  const float* replay_capsule;  // null: no replay
  const int32_t* accepted;
  float* replay_state;
  // Fused causal convolution (decode, V-major, no capture): q, k, v are the
  // convolution of `mixed` [N, conv_channels] (channels [q | k | v], conv_channels
  // = 2 Hk Dk + Hv Dv) with kernel size kConvFusedK, conv_weight [C, K],
  // conv_bias [C] or null, carried inputs conv_init [R, C, K - 1] (null: zeros),
  // the last K - 1 inputs written to conv_final (null: not written).
  const void* mixed;            // may be null when there are no tokens
  const float* conv_weight;
  const float* conv_bias;
  const float* conv_init;
  float* conv_final;
  int32_t conv_channels;        // 0: no fused convolution (q, k, v read as given)
  int32_t conv_silu;            // SiLU after the convolution (else the identity)
};

// Kernel size of the fused convolution.
constexpr int kConvFusedK = 4;

struct ReplayArgs {
  const float* src;
  const float* capsule;
  const int32_t* accepted;
  float* dst;
  int32_t R, Hk, Hv, Dk, Dv;
  int32_t group;
  int32_t capacity;
  int32_t capsule_width;
  const int32_t* src_slots;     // state pools: slot read / written per request
  const int32_t* dst_slots;
  int32_t num_slots;            // 0: states indexed by request
  int32_t k_major;              // states stored [.., Dk, Dv] (else V-major [.., Dv, Dk])
};

// Chunked prefill (Dk = Dv = 128, chunk 64).
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu_seqlens;    // null: dense layout, dense_len tokens per request
  const float* initial_state;
  float* final_state;
  void* output;
  void* workspace;
  int32_t N, R, Hk, Hv, group;
  int32_t max_chunks;           // chunk slots the workspace holds
  float scale;
  int32_t dense_len;            // tokens per request when cu_seqlens is null
  int32_t gate_none;            // a, b are the effective alpha, beta (no activation)
  const int32_t* initial_slots; // state pools: slot read / written per request
  const int32_t* final_slots;
  int32_t num_slots;            // 0: states indexed by request
  int32_t k_major;              // states stored [.., Dk, Dv] (else V-major [.., Dv, Dk])
  int32_t gated;                // update rule applies the decay alpha (else alpha = 1, a not read)
  int32_t delta;                // update rule writes beta (v - alpha S k^) (else v, b not read)
};

// Slot of request r's state. Without a pool (num_slots = 0) or without a slot
// array it is r; otherwise slots[r] when that lies in [0, num_slots), and -1
// (no state: read as zeros, not written) for any other value, so no index a
// device array holds can reach outside the pool.
__device__ inline int state_slot(const int32_t* slots, int r, int num_slots) {
  if (num_slots == 0 || slots == nullptr) return r;
  const int s = slots[r];
  return (s >= 0 && s < num_slots) ? s : -1;
}

// Start of (slot, head h) in a state array of per-head blocks of head_elems
// floats, or null when there is no array or no slot.
template <typename T>
__device__ inline T* state_head(T* base, int slot, int Hv, int h, size_t head_elems) {
  return (base != nullptr && slot >= 0) ? base + ((size_t)slot * Hv + h) * head_elems : nullptr;
}

// First token of request i (i = R: the end of the last request), clamped to
// [0, N]; from cu_seqlens, or i * dense_len for the dense layout.
template <typename Args>
__host__ __device__ inline int seq_start(const Args& p, int i) {
  const int64_t x = p.cu_seqlens != nullptr ? (int64_t)p.cu_seqlens[i] : (int64_t)i * p.dense_len;
  return (int)(x < 0 ? 0 : x > p.N ? p.N : x);
}

constexpr int kChunk = 64;

// Compact causal convolution (depthwise conv1d + activation with K - 1 carried inputs).
struct ConvArgs {
  const void* x;
  const float* weight;          // [C, K]
  const float* bias;            // [C] or null
  const int32_t* cu_seqlens;    // null: dense layout, dense_len tokens per request
  const float* initial_state;   // [R, C, K - 1] or null
  float* final_state;           // [R, C, K - 1] or null; may equal initial_state
  void* output;
  float* state_update;          // [R, capacity, C] or null
  const int32_t* capture_count; // [R] or null
  int32_t N, R, C, K;
  int32_t dense_len;
  int32_t silu;                 // 1: SiLU, 0: identity
  int32_t capacity;
  int32_t tokens_per_block;
  int32_t final_in_place;       // final_state == initial_state
  int32_t final_pending;        // 0: every request's final state is written by the forward kernel
  const int32_t* initial_slots; // state pools: slot read / written per request
  const int32_t* final_slots;
  int32_t num_slots;            // 0: states indexed by request
};

// Convolution workgroups: 256 threads of 4 adjacent channels each.
constexpr int kConvBlockThreads = 256;
__host__ __device__ inline int64_t conv_channel_groups(int64_t C) {
  return (C + 4 * kConvBlockThreads - 1) / (4 * kConvBlockThreads);
}

// Which kernel writes a request's final state. The workgroup that convolves the
// request's last token holds the last K - 1 inputs and writes it, unless the
// update is in place and other workgroups may still read the request's carried
// inputs: then only a request whose tokens all fall in that one workgroup
// (tokens_per_block tokens each) is written there. Empty requests, and the
// in-place requests spanning workgroups, are left to the final-state kernel,
// which runs after the forward kernel.
__host__ __device__ inline bool final_in_forward(int start, int end, int tokens_per_block, bool in_place) {
  return end > start && (!in_place || start / tokens_per_block == (end - 1) / tokens_per_block);
}

struct ConvReplayArgs {
  const float* src;
  const float* capture;
  const int32_t* accepted;
  float* dst;
  int32_t R, C, K, capacity;
  const int32_t* src_slots;     // state pools: slot read / written per request
  const int32_t* dst_slots;
  int32_t num_slots;            // 0: states indexed by request
};

// io_dtype: 0 = f32, 1 = f16 (gdn_dtype values).
hipError_t launch_recurrent(const RecurrentArgs& args, int io_dtype, hipStream_t stream);
hipError_t launch_recurrent_kmajor(const RecurrentArgs& args, int io_dtype, hipStream_t stream);
hipError_t launch_replay(const ReplayArgs& args, hipStream_t stream);
hipError_t launch_chunk(const ChunkArgs& args, int io_dtype, hipStream_t stream);
hipError_t launch_conv(const ConvArgs& args, int io_dtype, hipStream_t stream);
hipError_t launch_conv_replay(const ConvReplayArgs& args, hipStream_t stream);
hipError_t launch_publish(int32_t R, int32_t* committed, int32_t* inactive, hipStream_t stream);

// Workspace bytes of the chunk path for `chunk_slots` chunks and these heads.
size_t chunk_workspace_bytes(int64_t chunk_slots, int R, int Hk, int Hv);

}  // namespace gdn

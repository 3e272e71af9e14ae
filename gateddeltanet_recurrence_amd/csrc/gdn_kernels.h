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
};

struct ReplayArgs {
  const float* src;
  const float* capsule;
  const int32_t* accepted;
  float* dst;
  int32_t R, Hk, Hv, Dk, Dv;
  int32_t group;
  int32_t capacity;
  int32_t capsule_width;
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
};

// First token of request i (i = R: the end of the last request), clamped to
// [0, N]; from cu_seqlens, or i * dense_len for the dense layout.
template <typename Args>
__host__ __device__ inline int seq_start(const Args& p, int i) {
  const int64_t x = p.cu_seqlens != nullptr ? (int64_t)p.cu_seqlens[i] : (int64_t)i * p.dense_len;
  return (int)(x < 0 ? 0 : x > p.N ? p.N : x);
}

constexpr int kChunk = 64;

// io_dtype: 0 = f32, 1 = f16 (gdn_dtype values).
hipError_t launch_recurrent(const RecurrentArgs& args, int io_dtype, hipStream_t stream);
hipError_t launch_replay(const ReplayArgs& args, hipStream_t stream);
hipError_t launch_chunk(const ChunkArgs& args, int io_dtype, hipStream_t stream);

// Workspace bytes of the chunk path for `chunk_slots` chunks and these heads.
size_t chunk_workspace_bytes(int64_t chunk_slots, int R, int Hk, int Hv);

}  // namespace gdn

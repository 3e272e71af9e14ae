/*
 * gdn_conv.h - C ABI of the compact causal convolution in libgdn.so.
 *
 * The depthwise causal conv1d + SiLU with a carried state that runs directly
 * upstream of the GatedDeltaNet operator in every hybrid layer ("Add
 * GatedDeltaNet evaluation export for Qwen hybrid models", Copilot review of the
 * builder: CausalConvWithState / VarlenCausalConvWithState on dense or packed
 * token-major inputs), in its compact form ("[CUDA] Add compact GatedDeltaNet
 * operator", the embedded VarlenCausalConv commit, Description and Motivation):
 * three outputs [output, final_state, state_update], where state_update keeps
 * only the appended input values needed to replay an accepted speculative
 * prefix, [batch, capacity, channels], with an optional per-request
 * capture_count, and the full state is [channels, kernel_size - 1].
 *
 * Per request r (tokens cu[r] .. cu[r+1]-1, L of them) and channel c, with the
 * K - 1 carried inputs s[r, c, 0 .. K-2] (oldest first):
 *   e         = [s_0 .. s_{K-2}, x_0 .. x_{L-1}]
 *   out_j     = act(bias[c] + sum_{i<K} weight[c, i] * e[j + i])   (x_j is e[j + K - 1])
 *   final     = e[L .. L + K - 2]                                   the last K - 1 inputs
 *   capture_j = x_j  for j < n_r = min(L, capture_count[r] clamped to [0, capacity],
 *                                   or capacity when capture_count is NULL)
 * act is SiLU(z) = z / (1 + exp(-z)) or the identity. weight is in the
 * cross-correlation orientation of conv1d: weight[c, K-1] multiplies the newest
 * input. The state and the capture are FP32; x and the output are FP16 or FP32.
 *
 * x, weight, output and the state and capture buffers must be 16-byte aligned
 * (each thread moves 4 adjacent channels as one vector).
 *
 * Conventions as in gdn.h: the caller owns every buffer, nothing is allocated,
 * every check runs on the host before anything is enqueued (a status other than
 * GDN_ERR_HIP means no device write), all work is asynchronous on `stream`, and
 * the status codes are gdn_status.
 */
#ifndef GDN_CONV_H_
#define GDN_CONV_H_

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_conv_activation { GDN_CONV_SILU = 0, GDN_CONV_NONE = 1 } gdn_conv_activation;

typedef struct gdn_conv_params {
  int32_t num_tokens;            /* N >= 0: packed tokens over all requests         */
  int32_t num_reqs;              /* R >= 0                                          */
  int32_t channels;              /* C >= 4, a multiple of 4                         */
  int32_t kernel_size;           /* K in 2 .. 8                                     */
  int32_t io_dtype;              /* gdn_dtype of x and output: GDN_F16 or GDN_F32   */
  int32_t activation;            /* gdn_conv_activation                             */
  int32_t state_update_capacity; /* capture rows per request; 0: no capture         */
} gdn_conv_params;

typedef struct gdn_conv_tensors {
  const void* x;                 /* device, io  [N, C]                               */
  const float* weight;           /* device, f32 [C, K]                               */
  const float* bias;             /* device, f32 [C], or NULL for zero                */
  const int32_t* cu_seqlens;     /* device, i32 [R + 1] as in gdn.h, or NULL for the
                                    dense layout [R, N / R, C] (N a multiple of R)   */
  const int32_t* cu_seqlens_host;/* host mirror of cu_seqlens, or NULL; validated
                                    when given; must be NULL when cu_seqlens is      */
  const float* initial_state;    /* device, f32 [R, C, K - 1], or NULL for zeros     */
  float* final_state;            /* device, f32 [R, C, K - 1], or NULL (not written);
                                    may equal initial_state exactly (in place)      */
  void* output;                  /* device, io  [N, C]                               */
  float* state_update;           /* device, f32 [R, capacity, C], or NULL (no
                                    capture). Row j of request r holds the input of
                                    token cu[r] + j; rows j >= n_r are not written.  */
  const int32_t* capture_count;  /* device, i32 [R], or NULL                         */
} gdn_conv_tensors;

/* Runs one forward call: output, final_state (if non-NULL) and the capture (if
 * state_update is non-NULL; then state_update_capacity must be > 0). Errors:
 * GDN_ERR_NULL (x, weight or output missing with N > 0; params or tensors NULL),
 * GDN_ERR_SHAPE (sizes out of range, malformed host cu_seqlens, N not a multiple
 * of R in the dense layout, misaligned vectors), GDN_ERR_DTYPE, GDN_ERR_ALIAS
 * (outputs overlapping inputs or each other, other than final_state ==
 * initial_state), GDN_ERR_CAPACITY, GDN_ERR_RULE (unknown activation). */
int gdn_conv_forward(const gdn_conv_params* params, const gdn_conv_tensors* tensors, void* stream);

/* Advances the committed state by the leading accepted[r] captured inputs of
 * every request and writes the result to an inactive bank ("Replay compact
 * fixed state for hybrid decoding", Summary, for the convolution state):
 *   dst[r] = the last K - 1 entries of [src[r], capture[r, 0 .. m_r - 1]]
 *   src_state     device, f32 [R, C, K - 1], read only
 *   state_update  device, f32 [R, capacity, C] as written by gdn_conv_forward
 *   accepted      device, i32 [R]; m_r = accepted[r] clamped to [0, capacity]
 *   accepted_host host mirror or NULL; when given every value must lie in
 *                 [0, capacity] (else GDN_ERR_CAPACITY)
 *   dst_state     device, f32 [R, C, K - 1]; must not overlap src_state,
 *                 state_update or accepted. m_r = 0 copies the committed state. */
int gdn_conv_replay(int32_t num_reqs, int32_t channels, int32_t kernel_size,
                    int32_t state_update_capacity, const float* src_state,
                    const float* state_update, const int32_t* accepted,
                    const int32_t* accepted_host, float* dst_state, void* stream);

/* ---- The convolution fused into the GatedDeltaNet decode.
 *
 * In a hybrid layer the convolution's output is exactly the q, k and v the
 * GatedDeltaNet operator reads ("Add GatedDeltaNet evaluation export for Qwen
 * hybrid models", Summary: the layer keeps its Q/K/V layout and causal
 * convolution ahead of the recurrent operator). gdn_conv_decode_forward runs
 * both in one kernel: every workgroup convolves the channels it needs for each
 * token in registers and LDS, so q, k and v never go through HBM.
 *
 * The convolution runs over the concatenated channels
 *   mixed[t] = [q (Hk Dk) | k (Hk Dk) | v (Hv Dv)],  Cm = 2 Hk Dk + Hv Dv,
 * with the semantics of gdn_conv_forward above (kernel size K, weight [Cm, K],
 * optional bias, SiLU or the identity, K - 1 carried inputs per channel), and
 * its output, rounded to io_dtype exactly as gdn_conv_forward stores it, is
 * split into q, k, v for the token recurrence of gdn_forward. The results equal
 * gdn_conv_forward followed by gdn_forward on the split output, bit for bit. */
typedef struct gdn_conv_fused {
  const void* mixed;             /* device, io  [N, Cm] in the token order of the GDN
                                    call (its cu_seqlens or dense layout); 16-byte
                                    aligned; may be NULL when N = 0                  */
  const float* weight;           /* device, f32 [Cm, K]; 16-byte aligned             */
  const float* bias;             /* device, f32 [Cm], or NULL for zero               */
  const float* initial_state;    /* device, f32 [R, Cm, K - 1], or NULL for zeros;
                                    16-byte aligned                                  */
  float* final_state;            /* device, f32 [R, Cm, K - 1], or NULL (not written);
                                    16-byte aligned. It must not overlap
                                    initial_state: several workgroups read a
                                    channel's carried inputs while one writes them. */
  int32_t kernel_size;           /* K; only 4 is supported                           */
  int32_t activation;            /* gdn_conv_activation                              */
} gdn_conv_fused;

/* One decode (or short-segment) call of the fused pair. params and tensors are
 * as for gdn_forward, with these differences:
 *   tensors->q, k, v must be NULL (the convolution supplies them);
 *   the token-recurrent kernel runs whatever the segment lengths: plan AUTO or
 *   RECURRENT (CHUNK is GDN_ERR_PLAN);
 *   no capsule (state_update NULL) and the V-major state layout only
 *   (GDN_ERR_SHAPE otherwise).
 * Errors as for gdn_forward, plus: GDN_ERR_NULL (conv NULL, or mixed or weight
 * missing with N > 0), GDN_ERR_SHAPE (kernel_size other than 4, a misaligned
 * convolution buffer), GDN_ERR_RULE (unknown activation), GDN_ERR_ALIAS (the
 * convolution's final_state overlapping its initial_state or any other
 * argument, or an output overlapping a convolution input). */
int gdn_conv_decode_forward(const gdn_params* params, const gdn_tensors* tensors, const gdn_conv_fused* conv,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CONV_H_ */

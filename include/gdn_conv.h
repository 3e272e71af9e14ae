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

#ifdef __cplusplus
}
#endif

#endif /* GDN_CONV_H_ */

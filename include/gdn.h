/*
 * gdn.h - C ABI of the MI355X (gfx950) GatedDeltaNet operator library, libgdn.so.
 *
 * The operator runs the gated delta rule (or, on request, one of the related
 * update rules of gdn_rule) on packed ragged inputs and keeps an FP32 V-major
 * recurrent state per request and value head:
 *
 *   alpha_t = exp(-exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]))
 *   beta_t  = sigmoid(b[t,h])
 *   k^_t    = k[t,g] / sqrt(|k[t,g]|^2 + 1e-6)          g = h / (Hv / Hk)
 *   q^_t    = q[t,g] / sqrt(|q[t,g]|^2 + 1e-6) * scale
 *   u_t     = beta_t * (v[t,h] - alpha_t * S k^_t)
 *   S       = alpha_t * S + u_t k^_t^T                    S is [Dv, Dk]
 *   out[t,h] = S q^_t
 *
 * Sources, by page and section:
 *  - "Add GatedDeltaNet evaluation export for Qwen hybrid models", What changed:
 *    packed THD q/k/v with cumulative sequence lengths, FP32 V-major state,
 *    the gated_delta update rule, an FP32 gate ABI, FP16/FP32 I/O only (BF16
 *    rejected); Dependency: dt_bias is one scalar per head, a forced plan,
 *    update-rule validation and an initial/final state alias.
 *  - "[CUDA] Add compact GatedDeltaNet operator", Description: recurrent decode
 *    and chunked prefill paths, ragged inputs, gate arithmetic fused from raw
 *    A_log, and the three outputs [output, final_state, state_update] where the
 *    FP32 state_update capsule packs decay, shared key and delta per token.
 *  - The same page's embedded VarlenCausalConv commit, Description: a bounded
 *    state_update_capacity and an optional per-request capture_count, the
 *    capture shaped [batch, capacity, channels].
 *  - "Replay compact fixed state for hybrid decoding", Summary and Key Changes:
 *    replay of only an accepted prefix into an inactive state bank, and a
 *    replay ABI with a version number.
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; "_host" pointers point to host memory.
 *  - The caller owns every buffer. The library keeps no pointer after a call
 *    returns, allocates no device memory and holds no global mutable state:
 *    calls on different streams may run concurrently as long as their buffers
 *    do not overlap. (Host-side checks of slot mirrors, gdn_pool.h, use
 *    temporary host memory.) The one exception is gdn_forward_no_alloc, whose
 *    workspace is a static device array per GPU (see there).
 *  - All device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and runs asynchronously; no call blocks on the device.
 *  - Every argument check runs on the host before anything is enqueued. A
 *    nonzero status other than GDN_ERR_HIP means nothing was enqueued and no
 *    device memory was written. GDN_ERR_HIP means a kernel launch failed.
 *  - Sizes are element counts unless named _bytes.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of this ABI: structs, entry points and the capsule layout.
 * 2: gdn_params.gate_activation; cu_seqlens may be NULL (dense rank-4 layout).
 * 3: gdn_params.state_layout; the causal convolution (gdn_conv.h) and the state
 *    pools (gdn_pool.h).
 * 4: gdn_forward_no_alloc and GDN_ERR_SCRATCH.
 * 5: the update rules GDN_RULE_DELTA, GDN_RULE_GATED and GDN_RULE_LINEAR.
 * 6: gdn_replay_forward (replay and verify in one pass over the committed state)
 *    and its pooled form gdn_replay_forward_pooled (gdn_pool.h). */
#define GDN_ABI_VERSION 7

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,       /* a required pointer is NULL                          */
  GDN_ERR_SHAPE = 2,      /* a size is out of range or cu_seqlens is malformed   */
  GDN_ERR_DTYPE = 3,      /* io dtype other than FP16 / FP32 (BF16 is rejected)  */
  GDN_ERR_ALIAS = 4,      /* buffers overlap in a way the call does not allow    */
  GDN_ERR_CAPACITY = 5,   /* capacity < 0, or capture/accepted beyond capacity   */
  GDN_ERR_WORKSPACE = 6,  /* workspace missing or smaller than required          */
  GDN_ERR_PLAN = 7,       /* forced plan not possible for these arguments        */
  GDN_ERR_RULE = 8,       /* unknown update rule or gate activation              */
  GDN_ERR_HIP = 9,        /* the HIP runtime rejected a launch                   */
  GDN_ERR_SCRATCH = 10    /* gdn_forward_no_alloc: the call needs more scratch
                             than its static array holds                         */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_F16 = 1, GDN_BF16 = 2 } gdn_dtype;

/* Kernel path. CHUNK (fp16 MFMA, chunk 64) needs fp16 I/O and Dk = Dv = 128 and
 * writes no capsule. AUTO takes RECURRENT when a capsule is requested, when the
 * CHUNK conditions do not hold, or when the longest request (from
 * cu_seqlens_host, else the mean N / R) is at most 32 tokens; otherwise CHUNK.
 * A forced plan overrides this ("forced-plan behavior", first page, Dependency);
 * forcing CHUNK where it cannot run is GDN_ERR_PLAN. */
typedef enum gdn_plan { GDN_PLAN_AUTO = 0, GDN_PLAN_RECURRENT = 1, GDN_PLAN_CHUNK = 2 } gdn_plan;

/* Update rule ("update-rule selection" and "update-rule input validation", first
 * page, What changed and Dependency; the page names the gated_delta rule). The
 * others are read as the family that name composes: the decay gate and the delta
 * correction each on or off. With u the value written and S = alpha S + u k^^T:
 *   GDN_RULE_GATED_DELTA  u = beta (v - alpha S k^)   alpha from a   (Gated DeltaNet)
 *   GDN_RULE_DELTA        u = beta (v - S k^)         alpha = 1      (DeltaNet)
 *   GDN_RULE_GATED        u = v                       alpha from a   (gated linear attention)
 *   GDN_RULE_LINEAR       u = v                       alpha = 1      (linear attention)
 * and out = S q^ for all four. The ungated rules read neither a nor A_log nor
 * dt_bias (they may be NULL); the rules without the delta correction do not read
 * b (it may be NULL). The capsule holds (alpha, k^, u) as above for every rule,
 * so gdn_replay is the same for all. Any other value is GDN_ERR_RULE. */
typedef enum gdn_rule {
  GDN_RULE_GATED_DELTA = 0,
  GDN_RULE_DELTA = 1,
  GDN_RULE_GATED = 2,
  GDN_RULE_LINEAR = 3
} gdn_rule;

/* What a and b hold.
 *  GDN_GATE_RAW:  the raw gate inputs; the operator forms
 *                 alpha = exp(-exp(A_log) softplus(a + dt_bias)) and beta = sigmoid(b)
 *                 ("[CUDA] Add compact GatedDeltaNet operator", Description: gate
 *                 normalization fused from raw A_log).
 *  GDN_GATE_NONE: precomputed effective gates, activation none: alpha = a and
 *                 beta = b, in FP32 ("Add GatedDeltaNet evaluation export for Qwen
 *                 hybrid models", What changed). alpha is taken clamped to [0, 1],
 *                 the range of the raw form. A_log and dt_bias are not read and may
 *                 be NULL. */
typedef enum gdn_gate_activation { GDN_GATE_RAW = 0, GDN_GATE_NONE = 1 } gdn_gate_activation;

/* How the FP32 state of a (request, value head) is stored.
 *  GDN_STATE_V_MAJOR: [Dv, Dk], each dv row of Dk floats contiguous - the packed
 *                     GatedDeltaNet contract ("Add GatedDeltaNet evaluation export
 *                     for Qwen hybrid models", What changed: FP32 V-major state).
 *  GDN_STATE_K_MAJOR: [Dk, Dv], the transpose - the dense LinearAttention layout
 *                     [B, heads, key_dim, value_dim] (same page, Copilot review).
 * The capsule layout does not depend on it. */
typedef enum gdn_state_layout { GDN_STATE_V_MAJOR = 0, GDN_STATE_K_MAJOR = 1 } gdn_state_layout;

typedef struct gdn_params {
  int32_t num_tokens;            /* N: packed tokens over all requests, >= 0      */
  int32_t num_reqs;              /* R: requests (state batch), >= 0               */
  int32_t num_k_heads;           /* Hk >= 1, divides Hv                            */
  int32_t num_v_heads;           /* Hv >= 1                                        */
  int32_t head_k_dim;            /* Dk in {16, 32, 64, 128}                        */
  int32_t head_v_dim;            /* Dv in {16, 32, 64, 128}                        */
  int32_t io_dtype;              /* gdn_dtype of q, k, v and output                */
  float scale;                   /* query scale; <= 0 selects Dk^-1/2              */
  int32_t chunk;                 /* chunk length of the CHUNK plan; 0 selects 64;
                                    only 64 is supported                           */
  int32_t state_update_capacity; /* capsule rows per request; 0: no capsule        */
  int32_t plan;                  /* gdn_plan                                       */
  int32_t update_rule;           /* gdn_rule                                       */
  int32_t gate_activation;       /* gdn_gate_activation of a and b                 */
  int32_t state_layout;          /* gdn_state_layout of initial and final states   */
} gdn_params;

/* Tensors of one forward call. Layouts are dense row-major with the last
 * index fastest; "io" is the element type named by io_dtype. */
typedef struct gdn_tensors {
  const void* q;                 /* device, io  [N, Hk, Dk]                        */
  const void* k;                 /* device, io  [N, Hk, Dk]                        */
  const void* v;                 /* device, io  [N, Hv, Dv]                        */
  const float* a;                /* device, f32 [N, Hv]  decay input (see
                                    gdn_gate_activation); NULL allowed for the
                                    ungated rules                                  */
  const float* b;                /* device, f32 [N, Hv]  beta input; NULL allowed
                                    for the rules without the delta correction     */
  const float* A_log;            /* device, f32 [Hv]; may be NULL with GDN_GATE_NONE
                                    or an ungated rule                             */
  const float* dt_bias;          /* device, f32 [Hv]  one scalar per value head;
                                    may be NULL with GDN_GATE_NONE or an ungated
                                    rule                                           */
  const int32_t* cu_seqlens;     /* device, i32 [R + 1]: 0 = cu[0] <= ... <= cu[R] = N;
                                    request r owns tokens cu[r] .. cu[r+1]-1.
                                    NULL selects the dense rank-4 layout ("ragged
                                    and rank-4 inputs", third page, Description):
                                    every request holds S = N / R tokens (N must be
                                    a multiple of R), i.e. q is [R, S, Hk, Dk] and
                                    v, output [R, S, Hv, Dv] - the same bytes as
                                    the packed layout with equal lengths.          */
  const int32_t* cu_seqlens_host;/* host mirror of cu_seqlens, or NULL. When given
                                    it is validated and used for planning. Must be
                                    NULL when cu_seqlens is NULL.                  */
  const float* initial_state;    /* device, f32 [R, Hv, Dv, Dk] (K-major: [R, Hv, Dk,
                                    Dv]), or NULL for zeros. With the K-major
                                    layout, v and output must be 16-byte aligned. */
  float* final_state;            /* device, f32, as initial_state, or NULL (not
                                    written). May equal initial_state exactly
                                    (in-place update); any other overlap is an error */
  void* output;                  /* device, io  [N, Hv, Dv]                        */
  float* state_update;           /* device, f32 [R, capacity, W] with
                                    W = Hv + Hk*Dk + Hv*Dv, or NULL (no capsule).
                                    Row j of request r holds token cu[r]+j as
                                    [alpha for Hv heads | k^ for Hk heads (Dk each)
                                     | u for Hv heads (Dv each)]. Rows j >= n_r are
                                    not written.                                   */
  const int32_t* capture_count;  /* device, i32 [R] or NULL. Request r captures its
                                    leading n_r = min(len_r, c_r) tokens, c_r being
                                    capture_count[r] clamped to [0, capacity], or
                                    capacity when NULL.                            */
} gdn_tensors;

/* Runs one forward call: output, final_state (if non-NULL) and the capsule
 * (if state_update is non-NULL). The CHUNK plan needs a device workspace of
 * gdn_forward_workspace_bytes() bytes, disjoint from every tensor; RECURRENT
 * needs none (workspace may be NULL). */
int gdn_forward(const gdn_params* params, const gdn_tensors* tensors,
                void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static scratch array behind gdn_forward_no_alloc: 128 MiB per GPU. */
#define GDN_NO_ALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* gdn_forward for callers that cannot allocate device memory or provide a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, checks, kernels and results as gdn_forward;
 * the CHUNK plan's workspace (chunk offsets, T' and P fragments, per-token
 * factors) is a static device array of GDN_NO_ALLOC_SCRATCH_BYTES bytes instead,
 * one per GPU, held from the library's first call on that GPU until the process
 * ends. The call itself allocates nothing.
 *  - A call whose workspace (gdn_forward_workspace_bytes, the exact figure with a
 *    cu_seqlens_host mirror, else its upper bound) exceeds the array returns
 *    GDN_ERR_SCRATCH before anything is enqueued. At Hv = 32, 128 MiB holds about
 *    315 chunks of 64 tokens (about 20k tokens); the RECURRENT plan needs none.
 *  - Every call on one GPU uses that GPU's one array, and nothing in it needs to
 *    start at zero (each call writes what it reads). Calls that overlap on one
 *    GPU (concurrent streams, or threads) race on it: serialize them. */
int gdn_forward_no_alloc(const gdn_params* params, const gdn_tensors* tensors, void* stream);

/* Workspace bytes gdn_forward needs for these params, written to *bytes.
 * cu_seqlens_host may be NULL; the result then is an upper bound that is valid
 * for every cu_seqlens with the same N and R. Resolves the plan exactly as
 * gdn_forward does (state_update_capacity > 0 is taken to mean a capsule). */
int gdn_forward_workspace_bytes(const gdn_params* params, const int32_t* cu_seqlens_host,
                                size_t* bytes);

/* The plan gdn_forward would run for these params (GDN_PLAN_RECURRENT or
 * GDN_PLAN_CHUNK), written to *plan; capsule as for the workspace query. */
int gdn_resolve_plan(const gdn_params* params, const int32_t* cu_seqlens_host, int32_t* plan);

/* Replays the leading accepted[r] capsule rows of every request r onto the
 * committed V-major state and writes the result to an inactive bank ("Replay
 * compact fixed state for hybrid decoding", Summary); gdn_replay_pooled
 * (gdn_pool.h) takes the state layout and pools:
 *   dst[r,h] = src[r,h];  for j < m_r:  dst[r,h] = alpha_j * dst[r,h] + u_j k^_j^T
 * with alpha_j, k^_j (key head h / (Hv/Hk)) and u_j read from capsule row j.
 *   src_state     device, f32 [R, Hv, Dv, Dk]  committed bank, read only
 *   state_update  device, f32 [R, capacity, W] as written by gdn_forward
 *   accepted      device, i32 [R]; m_r = accepted[r] clamped to [0, capacity]
 *   accepted_host host mirror of accepted or NULL; when given every value must
 *                 lie in [0, capacity] (else GDN_ERR_CAPACITY)
 *   dst_state     device, f32 [R, Hv, Dv, Dk]; must not overlap src_state,
 *                 state_update or accepted. m_r = 0 copies the committed state.
 * The caller guarantees m_r <= n_r (rows beyond n_r hold no capture). */
int gdn_replay(int32_t num_reqs, int32_t num_k_heads, int32_t num_v_heads,
               int32_t head_k_dim, int32_t head_v_dim, int32_t state_update_capacity,
               const float* src_state, const float* state_update, const int32_t* accepted,
               const int32_t* accepted_host, float* dst_state, void* stream);

/* One speculative decoding step with a single read of the committed state:
 * replays the accepted prefix of the previous step's capsule onto the committed
 * bank, writes the result to the inactive bank, and verifies this step's draft
 * tokens from that state ("Replay compact fixed state for hybrid decoding",
 * Summary: accepted-prefix replay into an inactive bank; "[CUDA] Add compact
 * GatedDeltaNet operator", Description: the state_update capsule). It returns
 * the same statuses and writes the same bytes as
 *   gdn_replay(R, Hk, Hv, Dk, Dv, capacity, tensors->initial_state,
 *              prev_state_update, accepted, accepted_host, replay_state, stream);
 *   gdn_forward(params, tensors with initial_state = replay_state, NULL, 0, stream);
 * but reads the committed bank once instead of twice.
 *   params, tensors as gdn_forward, with a capsule (state_update non-NULL,
 *                 state_update_capacity > 0, so the RECURRENT plan) and V-major
 *                 states; tensors->initial_state is the committed bank [R, Hv,
 *                 Dv, Dk] (required, read only); tensors->final_state is NULL or
 *                 a further buffer that receives the state after this step's
 *                 tokens, disjoint from the committed bank.
 *   prev_state_update device, f32 [R, capacity, W]: the previous step's
 *                 capsule, W as for state_update (same capacity)
 *   accepted      device, i32 [R]; m_r = accepted[r] clamped to [0, capacity]
 *   accepted_host host mirror of accepted or NULL; when given every value must
 *                 lie in [0, capacity] (else GDN_ERR_CAPACITY)
 *   replay_state  device, f32 [R, Hv, Dv, Dk], 16-byte aligned: the inactive
 *                 bank; it overlaps no other buffer of the call.
 * Errors as gdn_forward; GDN_ERR_NULL for a missing capsule, committed bank,
 * previous capsule, accepted or replay_state; GDN_ERR_SHAPE for the K-major
 * layout; GDN_ERR_ALIAS for the overlaps above. The caller guarantees
 * m_r <= the rows the previous step captured. */
int gdn_replay_forward(const gdn_params* params, const gdn_tensors* tensors,
                       const float* prev_state_update, const int32_t* accepted,
                       const int32_t* accepted_host, float* replay_state, void* stream);

/* Static text for a status code. */
const char* gdn_strerror(int status);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

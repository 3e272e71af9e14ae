/*
 * gdn_pool.h - state pools for libgdn.so: per-request slot indices into
 * double-buffered fixed-state banks, and their publication.
 *
 * "Replay compact fixed state for hybrid decoding" (Key Changes and the
 * Copilot overview) keeps every request's fixed recurrent state - the
 * GatedDeltaNet state and the causal-convolution state - in a pool with
 * per-request ownership and double-buffered publication: a speculative step
 * verifies against the committed bank, replays the accepted prefix into the
 * inactive bank, and then publishes it. Here a pool is one device array of P
 * state slots, [P, Hv, Dv, Dk] for GatedDeltaNet or [P, C, K - 1] for the
 * convolution, and each call names, per request, the slot it reads and the
 * slot it writes. The entry points below are the ones of gdn.h and
 * gdn_conv.h with the state arrays read as pools; everything else about them
 * (layouts, checks, status codes, asynchrony) is as there.
 *
 * Slot rules, for every entry point here:
 *  - A read slot outside [0, P) (e.g. -1 for a new request) reads a zero state;
 *    a write slot outside [0, P) writes nothing. A NULL slot array means slot r
 *    for request r (then R <= P).
 *  - Two requests must not write the same slot, and no request may write a
 *    slot another request reads in the same call (pools that are one buffer).
 *    A request may write the slot it reads (an in-place update). When the host
 *    mirrors of the slot arrays are given these rules are checked (values must
 *    lie in [-1, P), else GDN_ERR_SHAPE; collisions are GDN_ERR_ALIAS);
 *    otherwise they are the caller's contract.
 *  - The read pool and the write pool may be the same buffer (the usual
 *    double-buffered pool of two slots per owner) or disjoint buffers.
 */
#ifndef GDN_POOL_H_
#define GDN_POOL_H_

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_conv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_slots {
  int32_t num_slots;                 /* P >= 1: slots in each pool                    */
  const int32_t* read_slots;         /* device, i32 [R]: slot request r reads, or NULL */
  const int32_t* write_slots;        /* device, i32 [R]: slot request r writes, or NULL */
  const int32_t* read_slots_host;    /* host mirrors of the two arrays, or NULL; must be
                                        NULL when the device array is NULL            */
  const int32_t* write_slots_host;
} gdn_slots;

/* gdn_forward with initial_state and final_state read as pools [P, Hv, Dv, Dk]
 * (or [P, Hv, Dk, Dv] K-major): request r starts from initial_state[read_slots[r]]
 * and, when final_state is non-NULL, leaves its state in
 * final_state[write_slots[r]]. */
int gdn_forward_pooled(const gdn_params* params, const gdn_tensors* tensors, const gdn_slots* slots,
                       void* workspace, size_t workspace_bytes, void* stream);

/* gdn_replay from and into pools: request r's committed state is
 * src_pool[read_slots[r]] and the replayed state goes to
 * dst_pool[write_slots[r]]; state_update and accepted as in gdn_replay. The
 * sizes and the state layout come from params (num_reqs, the head counts and
 * dims, state_update_capacity, state_layout; the other fields are not read).
 * slots may be NULL: the states are then indexed by request ([R, ...]) as in
 * gdn_replay, which makes this the replay of a K-major state too. */
int gdn_replay_pooled(const gdn_params* params, const float* src_pool, const float* state_update,
                      const int32_t* accepted, const int32_t* accepted_host, float* dst_pool,
                      const gdn_slots* slots, void* stream);

/* gdn_replay_forward over a pool: request r's committed state is
 * tensors->initial_state[read_slots[r]], its replayed state goes to
 * replay_pool[write_slots[r]] (a write slot outside [0, P) writes nothing), and
 * the verify runs from that state. tensors->final_state must be NULL (else
 * GDN_ERR_SHAPE). replay_pool may be the same pool as initial_state (distinct
 * read and write slots, as for gdn_replay_pooled) or a disjoint one. Otherwise
 * as gdn_replay_forward: the same bytes as gdn_replay_pooled followed by
 * gdn_forward_pooled from the write slots, with one read of the committed slots. */
int gdn_replay_forward_pooled(const gdn_params* params, const gdn_tensors* tensors, const gdn_slots* slots,
                              const float* prev_state_update, const int32_t* accepted,
                              const int32_t* accepted_host, float* replay_pool, void* stream);

/* gdn_conv_forward with initial_state and final_state read as pools [P, C, K - 1]. */
int gdn_conv_forward_pooled(const gdn_conv_params* params, const gdn_conv_tensors* tensors,
                            const gdn_slots* slots, void* stream);

/* gdn_conv_replay from and into pools [P, C, K - 1]. */
int gdn_conv_replay_pooled(int32_t num_reqs, int32_t channels, int32_t kernel_size,
                           int32_t state_update_capacity, const float* src_pool,
                           const float* state_update, const int32_t* accepted,
                           const int32_t* accepted_host, float* dst_pool, const gdn_slots* slots,
                           void* stream);

/* Double-buffered publication: for every request r, exchanges committed_slots[r]
 * and inactive_slots[r] (device, i32 [R], disjoint arrays) on the device, so
 * that the slot a replay has just written becomes the committed one without a
 * host round trip. Enqueue it after the replays of the step. Errors:
 * GDN_ERR_SHAPE (R < 0), GDN_ERR_NULL, GDN_ERR_ALIAS (the arrays overlap). */
int gdn_publish_slots(int32_t num_reqs, int32_t* committed_slots, int32_t* inactive_slots,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_POOL_H_ */

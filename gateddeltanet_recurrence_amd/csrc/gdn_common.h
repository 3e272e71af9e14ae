// Device helpers shared by the GatedDeltaNet HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kNormEps = 1e-6f;

// DPP lane permutations within a row of 16 lanes (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane i <- lane 7-i of its 8
constexpr int kDppRowMirror = 0x140;    // row_mirror: lane i <- lane 15-i of its 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of LANES (4 or 8) adjacent lanes; every lane of
// the group gets the total. All 64 lanes must be active.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group of 4, 8 or 16 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (LANES >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (LANES >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// io element access: 4 consecutive elements widened to float, one narrowed store.
template <typename IO> struct IoOps;

template <> struct IoOps<float> {
  static __device__ __forceinline__ float4_t load4(const float* p) {
    return *reinterpret_cast<const float4_t*>(p);
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
};

template <> struct IoOps<_Float16> {
  static __device__ __forceinline__ float4_t load4(const _Float16* p) {
    half4_t h = *reinterpret_cast<const half4_t*>(p);
    return float4_t{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
  }
  static __device__ __forceinline__ float load1(const _Float16* p) { return (float)*p; }
  // float -> half conversion rounds to nearest even
  static __device__ __forceinline__ void store1(_Float16* p, float x) { *p = (_Float16)x; }
};

// log(1 + e^x); above 20 the correction log1p(e^-x) < 2.1e-9 is below fp32 resolution of x.
__device__ __forceinline__ float softplus_f(float x) {
  return x > 20.0f ? x : log1pf(expf(x));
}

// Gate arithmetic from the raw inputs: alpha = exp(-exp(A_log) softplus(a + dt_bias)).
__device__ __forceinline__ float decay_from_raw(float a, float expA, float dt_bias) {
  return expf(-expA * softplus_f(a + dt_bias));
}

__device__ __forceinline__ float sigmoid_f(float b) { return 1.0f / (1.0f + expf(-b)); }

// SiLU(z) = z * sigmoid(z) after the causal convolution, with the hardware
// base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each) in
// place of a library exp and an IEEE division: the convolution does little else
// per element, so those would make it bound by vector ALU issue rather than by
// HBM. Limits: z -> -inf gives 2^(+inf) = inf, 1/inf = 0, result -0; z -> +inf
// gives 1/1, result z. The convolution kernels and the decode with the fused
// convolution share it, so both round alike.
__device__ __forceinline__ float silu(float z) {
  constexpr float kLog2e = 1.4426950408889634f;
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Precomputed effective decay (gate activation none), clamped to [0, 1], the
// range of the raw form.
__device__ __forceinline__ float effective_decay(float a) { return fminf(fmaxf(a, 0.f), 1.f); }

// alpha and beta of a token from its two gate inputs: raw (fused activations) or
// effective (activation none).
__device__ __forceinline__ float gate_alpha(float a, bool none, float expA, float dt_bias) {
  return none ? effective_decay(a) : decay_from_raw(a, expA, dt_bias);
}
__device__ __forceinline__ float gate_beta(float b, bool none) { return none ? b : sigmoid_f(b); }

// log alpha for the chunked form. An effective decay of 0 is taken as the
// smallest normal float (log -87.3): the state is then reset up to a factor
// 1.2e-38 instead of exactly.
__device__ __forceinline__ float gate_log_alpha(float a, bool none, float expA, float dt_bias) {
  return none ? logf(fmaxf(effective_decay(a), 1.17549435e-38f)) : -expA * softplus_f(a + dt_bias);
}

}  // namespace gdn

namespace gdn {

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (not its outstanding global loads) before s_barrier, so register prefetches
// of global data stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gdn

namespace gdn {

// Raw buffer access with a hardware range check: a load past `bytes` returns 0
// and a store past it is dropped, so ragged tails need no branches (which keeps
// the number of memory instructions per loop iteration fixed and lets the
// compiler wait for just the data it needs).
constexpr int kBufferWord3 = 0x00020000;   // gfx9-family raw buffer descriptor word 3
constexpr int kBufferNontemporal = 2;      // cache-policy operand of a buffer access: nt

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
}

__device__ __forceinline__ half8_t buf_load_h8(rsrc_t r, int byte_off) {
  return __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ half4_t buf_load_h4(rsrc_t r, int byte_off) {
  return __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

__device__ __forceinline__ float buf_load_f32(rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

__device__ __forceinline__ void buf_store_h1(_Float16 x, rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, byte_off, 0, 0);
}

}  // namespace gdn

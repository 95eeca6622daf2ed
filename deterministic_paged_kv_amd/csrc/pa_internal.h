// Internal declarations and device helpers shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pa.h"

namespace pa {

constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kHalfDim = kHeadDim / 2;
constexpr int kMaxGroup = 16;  // query heads per KV head: the 16 rows of one MFMA tile

// 1/sqrt(128) * log2(e), rounded once to FP32: scores are kept in the base-2 domain so the
// softmax uses the hardware exp2; the LSE is converted back with ln(2) at the end.
constexpr float kScoreScaleLog2 = (float)(1.4426950408889634074 / 11.313708498984760390);  // log2(e) / sqrt(128)
constexpr float kLn2 = (float)0.69314718055994530942;

}  // namespace pa

struct pa_plan_s {
  int32_t num_q_heads, num_kv_heads, group;
  int32_t max_batch, max_q_len, max_pages_per_row;
  int32_t table_rows;  // positions covered by the cos/sin table: max_pages_per_row * 16 + 1
  float rope_theta, rope_scale, rms_eps;
  int32_t split_policy;
  int device;
  float* d_rope;  // [table_rows][128]: cos of the 64 frequencies, then sin
};

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Operand layout shared by every kernel.
//
// A tile of 16 head vectors (16 keys, or up to 16 query heads of one GQA group) is spread
// over a 64-lane wavefront in the register layout of one operand of
// v_mfma_f32_16x16x32_bf16: lane l holds vector r = l % 16, and in register block
// kb = 0..3 the 8 dims 32*kb + 8*g + e (e = 0..7), g = l / 16.  The four lanes
// r, r+16, r+32, r+48 together hold the whole 128-dim vector.  In this layout the RoPE
// partner of dim d < 64 (d + 64) sits in the same lane (block kb + 2), so the rotation
// needs no data exchange, and one 16-byte load per block reads 8 contiguous dims.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& raw, float* x) {
  x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
  x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
  x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z);
  x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
}

// The Q/K prologue for one head vector held in the operand layout above:
//   y   = RMSNorm(x) * w     sum of squares exact (float64; every square of a BF16 value is
//                            exact and the 128-term float64 sum is exact for any realistic
//                            exponent spread, so lane order cannot change it); mean rounded
//                            to FP32; + eps in FP32; 1/sqrt correctly rounded via float64;
//                            then two FP32 multiplies, x * inv first, then * w.
//   out = bf16_rne(RoPE(y))  rotate-half pairs (i, i+64), FP32 multiplies and one add or
//                            subtract each, no fused multiply-add.
// Sources: "[WS2][PR7][Attention] Add FlashInfer RoPE-fused paged attention scaffold",
// section "Scope" (Q/K RMSNorm; same post-RoPE boundary on both sides); "WS2 Attention
// Cross-Configuration Integration", section "H100 Attention input and projection boundary"
// (RMSNorm, then RoPE); "WS2 PR7 Fused Attention Backend Alignment", section "FlashInfer
// RoPE Fusion" (Llama rotate-half RoPE, theta 1e6, rotary_dim = head_dim).
//
// raw: the lane's 4 blocks of 8 BF16 inputs.  w: the lane's 32 norm weights (block-major),
// ignored if !norm.  cs: the position's cos/sin row (cos[64] then sin[64]).  All four lanes
// of a vector must call this together (it exchanges partial sums across lanes l^16, l^32).
__device__ __forceinline__ void prologue_operand(const uint4 raw[4], const float w[32], bool norm, float eps,
                                                 const float* __restrict__ cs, int g, bf16x8 out[4]) {
#pragma clang fp contract(off)
  float x[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) unpack8(raw[kb], x[kb]);
  if (norm) {
    double ss = 0.0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (double)x[kb][e] * (double)x[kb][e];
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float ms = (float)(ss * (1.0 / kHeadDim));
    const float t = ms + eps;
    const float inv = (float)(1.0 / __builtin_sqrt((double)t));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kb][e] = (x[kb][e] * inv) * w[kb * 8 + e];
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float4* cp = reinterpret_cast<const float4*>(cs + 32 * kb + 8 * g);
    const float4* sp = reinterpret_cast<const float4*>(cs + kHalfDim + 32 * kb + 8 * g);
    const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y1 = x[kb][e], y2 = x[kb + 2][e];
      const float a = y1 * c[e];
      const float b = y2 * s[e];
      const float cc = y2 * c[e];
      const float d = y1 * s[e];
      out[kb][e] = (__bf16)(a - b);
      out[kb + 2][e] = (__bf16)(cc + d);
    }
  }
}

// Intra-wavefront LDS hand-off: make this lane's LDS writes visible to the other lanes of
// the same wavefront, and keep the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Fixed butterfly reductions over the 16 lanes of a row (lanes 16*g .. 16*g+15).  Every lane
// ends with the same value: at each level both partners add the same two operands.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + __shfl_xor(v, 1);
  v = v + __shfl_xor(v, 2);
  v = v + __shfl_xor(v, 4);
  v = v + __shfl_xor(v, 8);
  return v;
}

struct DecodeParams {
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t num_pages, num_indices, max_pages_per_row, table_rows;
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* last_page_len;
  const int32_t* qpos;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const float* q_norm;
  const float* k_norm;
  uint16_t* out;
  float* lse;
  const float* rope;
  float eps;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

struct ValidateParams {
  int32_t batch, q_len, num_pages, num_indices, max_pages_per_row;
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* last_page_len;
  const int32_t* cache_position;
  const int32_t* qpos;
  const int32_t* kpos;
  int32_t* page_count;            // scratch [num_pages]
  unsigned long long* report;     // scratch [1]: min over (rule rank << 40 | index)
};

hipError_t launch_validate(const ValidateParams& p, hipStream_t stream);

struct PrefillParams {
  int32_t batch, q_len, num_q_heads, num_kv_heads, group;
  int32_t num_pages, num_indices, max_pages_per_row, table_rows;
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* last_page_len;
  const int32_t* qpos;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const float* q_norm;
  const float* k_norm;
  uint16_t* out;
  float* lse;
  const float* rope;
  float eps;
  void* workspace;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Prefill workspace: q^ [B][Hq][Sq][128] bf16, then k^ [Hkv][nnz * 16][128] bf16.
inline size_t prefill_workspace_bytes(int hq, int hkv, int batch, int q_len, int num_indices) {
  return align256((size_t)batch * hq * q_len * kHeadDim * 2) +
         align256((size_t)hkv * num_indices * kPageSize * kHeadDim * 2);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace pa

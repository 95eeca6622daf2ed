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
constexpr int kMaxGroup = 16;
constexpr int kRopeBlockFloats = 8 * 64 * 4;  // one block of 16 positions of the RoPE table  // query heads per KV head: the 16 rows of one MFMA tile

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
  int32_t split_chunk_pages;  // PA_SPLIT_FIXED: pages per chunk (chunk tokens / 16); else 0
  int device;
  int32_t num_cus;  // compute units of that device (work placement only, never arithmetic)
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

// Exchanges between lanes l and l^16 / l^32 with v_permlane16_swap / v_permlane32_swap
// (plain VALU operations, no LDS round trip).  Swapping a register with itself leaves the
// lane's own value in one half of the result and its partner's in the other, so both lanes
// of a pair combine the same two operands and end with the same value.
__device__ __forceinline__ float pair16_sum(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float pair16_max(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ double pair16_sum(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  return __builtin_bit_cast(double, (uint64_t)lo[0] | ((uint64_t)hi[0] << 32)) +
         __builtin_bit_cast(double, (uint64_t)lo[1] | ((uint64_t)hi[1] << 32));
}
__device__ __forceinline__ double pair32_sum(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  return __builtin_bit_cast(double, (uint64_t)lo[0] | ((uint64_t)hi[0] << 32)) +
         __builtin_bit_cast(double, (uint64_t)lo[1] | ((uint64_t)hi[1] << 32));
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
// ignored if !norm.  cs: the lane's 32 cos/sin values for its vector's position, as loaded by
// load_cos_sin (cos of frequencies 8g..8g+7, 32+8g..32+8g+7, then sin of the same).  All four
// lanes of a vector must call this together (it exchanges partial sums across lanes l^16, l^32).
__device__ __forceinline__ void prologue_operand(const uint4 raw[4], const float w[32], bool norm, float eps,
                                                 const float4 cs[8], bf16x8 out[4]) {
#pragma clang fp contract(off)
  float x[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) unpack8(raw[kb], x[kb]);
  if (norm) {
    // x*x is exact in float64 and so is the sum (the terms have 16 significant bits), so the
    // four partial sums give the same result as any other order
    double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) s4[kb] = __builtin_fma((double)x[kb][e], (double)x[kb][e], s4[kb]);
    double ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    ss = pair16_sum(ss);
    ss = pair32_sum(ss);
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
    const float4 c0 = cs[2 * kb], c1 = cs[2 * kb + 1], s0 = cs[4 + 2 * kb], s1 = cs[4 + 2 * kb + 1];
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

// Same prologue with the norm weights read from LDS (w_lds: the 128 weights) instead of
// registers.  The arithmetic and its order are identical.
__device__ __forceinline__ void prologue_operand_lds_w(const uint4 raw[4], const float* w_lds, bool norm, float eps,
                                                       const float4 cs[8], int g, bf16x8 out[4]) {
#pragma clang fp contract(off)
  float x[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) unpack8(raw[kb], x[kb]);
  if (norm) {
    double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) s4[kb] = __builtin_fma((double)x[kb][e], (double)x[kb][e], s4[kb]);
    double ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    ss = pair16_sum(ss);
    ss = pair32_sum(ss);
    const float ms = (float)(ss * (1.0 / kHeadDim));
    const float t = ms + eps;
    const float inv = (float)(1.0 / __builtin_sqrt((double)t));
    // the eight weight reads go out together (the LDS latency is paid once)
    float4 wv[8];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      wv[2 * kb] = *reinterpret_cast<const float4*>(w_lds + 32 * kb + 8 * g);
      wv[2 * kb + 1] = *reinterpret_cast<const float4*>(w_lds + 32 * kb + 8 * g + 4);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 w0 = wv[2 * kb], w1 = wv[2 * kb + 1];
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kb][e] = (x[kb][e] * inv) * w[e];
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float4 c0 = cs[2 * kb], c1 = cs[2 * kb + 1], s0 = cs[4 + 2 * kb], s1 = cs[4 + 2 * kb + 1];
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

// The lane's 32 cos/sin values for position `pos` from the RoPE table (blocks of 16
// positions in lane order, built at plan time): cs[0..3] the cos of frequencies
// 8g..8g+7, 32+8g..32+8g+7, cs[4..7] their sin.  When the 16 lanes r of a group read the 16
// positions of one block (pos = 16 B + r), each load is 1 KB of contiguous memory.
__device__ __forceinline__ void load_cos_sin(const float* __restrict__ rope, int pos, int g, float4 cs[8]) {
  const float4* blk = reinterpret_cast<const float4*>(rope + (size_t)(pos >> 4) * kRopeBlockFloats);
  const int lane = (pos & 15) + 16 * g;
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = blk[e * 64 + lane];
}

// Wave-uniform read of a read-only int32 array through the constant address space, so the
// compiler issues a scalar load (counted separately from the vector loads in flight).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int i) {
  return ((const_i32_ptr)p)[i];
}
typedef const __attribute__((address_space(4))) float* const_f32_ptr;
__device__ __forceinline__ float load_uniform_f32(const float* p, int i) {
  return ((const_f32_ptr)p)[i];
}

// Intra-wavefront LDS hand-off: make this lane's LDS writes visible to the other lanes of
// the same wavefront, and keep the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS writes of every wavefront of the workgroup visible to all of them: waits for this
// wavefront's LDS operations, then the workgroup barrier.  Vector memory loads in flight are
// not waited for.
__device__ __forceinline__ void workgroup_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Most chunks one row may have under the fixed-chunk policy (the fold keeps their maxima and
// sums in LDS).
constexpr int kMaxFixedChunks = 4096;

struct DecodeParams {
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t num_pages, num_indices, max_pages_per_row, table_rows;
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* last_page_len;
  const int32_t* cache_position;  // [B, Sq]; must equal qpos
  const int32_t* qpos;            // [B, Sq]
  const int32_t* kpos;            // [nnz * 16]; key j of row b at indptr[b] * 16 + j, must be j
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const float* q_norm;
  const float* k_norm;
  uint16_t* out;
  float* lse;
  const float* rope;
  float eps;
  int32_t chunk_pages;  // 0: the fixed 16-stream tree; > 0: fixed chunks of this many pages
  int32_t num_cus;      // compute units of the device (work placement only, never arithmetic)
};

// Decode.  chunk_pages == 0 and workspace == NULL: one workgroup per (row, KV head).
// chunk_pages == 0 with a workspace (at least decode_workspace_bytes, any contents): one
// wavefront per (row, KV head, stream) on separate compute units, then a combining kernel;
// same bits either way.  chunk_pages > 0 (needs a workspace): one wavefront per (row, KV
// head, chunk), then a kernel folding the chunks in ascending order.
size_t decode_workspace_bytes(int batch, int num_kv_heads, int group, int chunk_pages, int max_pages_per_row);
hipError_t launch_decode(const DecodeParams& p, void* workspace, hipStream_t stream);

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
  const int32_t* cache_position;  // [B, Sq]; must equal qpos
  const int32_t* qpos;            // [B, Sq]
  const int32_t* kpos;            // [nnz * 16]; key j of row b at indptr[b] * 16 + j, must be j
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const float* q_norm;
  const float* k_norm;
  uint16_t* out;
  float* lse;
  const float* rope;
  float eps;
  int32_t num_cus;
  void* workspace;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Prefill workspace, three regions written by the prologue kernel and read by the attention
// kernel of the same call:
//   k^     [Hkv][nnz * 16][128] bf16, then 32 rows of padding (the attention kernel loads whole
//          32-key tiles; rows past a row's keys are masked, and the padding keeps the last
//          row's tile in bounds);
//   q^     [B][Hq][Sq][128] bf16;
//   units  one record of kUnitInts int32 per work unit (row, block of kPrefillQB queries),
//          stored in the order the attention kernel takes the units (longest first): the
//          unit's number and what the kernel needs of its row and queries (extent, length,
//          tiles, poison, the row's first page numbers), see pa_prefill.hip.
constexpr int kPrefillQB = 32;  // queries per work unit of the attention kernel
constexpr int kUnitInts = 32;
inline size_t prefill_kh_bytes(int hkv, int num_indices) {
  return align256(((size_t)hkv * num_indices * kPageSize + 32) * kHeadDim * 2);
}
inline size_t prefill_qh_bytes(int hq, int batch, int q_len) {
  return align256((size_t)batch * hq * q_len * kHeadDim * 2);
}
inline size_t prefill_unit_bytes(int batch, int q_len) {
  return align256((size_t)batch * ((q_len + kPrefillQB - 1) / kPrefillQB) * kUnitInts * 4);
}
inline size_t prefill_workspace_bytes(int hq, int hkv, int batch, int q_len, int num_indices) {
  return prefill_kh_bytes(hkv, num_indices) + prefill_qh_bytes(hq, batch, q_len) + prefill_unit_bytes(batch, q_len);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// Backward of full-prefill attention (dense training layout).
struct BackwardArgs {
  int32_t batch, seq, num_q_heads, num_kv_heads, table_rows;
  const int32_t* positions;
  const void *q, *k, *v, *out, *dout;
  const float* lse;
  const float *q_norm, *k_norm;
  const float* rope;
  float eps;
  float *dq, *dk, *dv, *dq_norm, *dk_norm;
  void* workspace;
};
size_t backward_workspace_bytes(int batch, int seq, int hq, int hkv);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

}  // namespace pa

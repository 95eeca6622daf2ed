// Chunked paged prefill: Sq trailing queries per row attend causally to the row's cached keys.
//
// Sources: "WS2 PR7 Fused Attention Backend Alignment", sections "Current Implementation"
// (paged prefill wrapper; out [B, Hq, Sq, D], lse [B, Hq, Sq]) and "FlashInfer RoPE Fusion"
// (pre-RoPE Q and K cache, Llama RoPE, trailing contiguous query positions); "[WS2][PR7]
// [Attention] Add FlashInfer RoPE-fused paged attention scaffold", section "Scope" (logical
// K/V order before arithmetic, Split-KV disabled, FP32 LSE, same post-RoPE boundary).
//
// Two kernels per call.
//  1. prologue_kernel: every query vector and every cached key (per KV head) goes once through
//     the shared Q/K prologue (RMSNorm, RoPE, BF16).  q^ is written in q's own layout
//     [B][Hq][Sq][128]; k^ is written in logical order, [Hkv][nnz * 16][128], key j of row b at
//     (kv_indptr[b] * 16 + j); slots past a row's length are written as zeros.
//  2. attend_kernel: one workgroup per (query block of 32, row, KV head, group of up to 4
//     query heads); wavefront w handles one query head of the KV head's GQA group, so those
//     heads share each staged V tile.  Key tiles
//     of 64 (4 pages) are visited in ascending order up to the block's last visible key; per
//     tile S^T = K^ Q^T (bf16 MFMA, FP32 accumulation), causal mask on logical positions
//     (key j visible to a query at position p iff j <= p), FP32 online softmax with a fixed
//     reduction order, O^T += V^T P^T (P rounded to bf16 for the MFMA, FP32 accumulation).
//  The tiling is a constant of the library, so each row's reduction order depends only on
//  the row itself, never on the batch or the plan width.
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kQBlock = 32;   // queries per wavefront (two 16-row MFMA tiles)
constexpr int kKTile = 64;    // keys per tile (4 pages)
constexpr int kVRow = kHeadDim + 8;

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(uint16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ uint4 as_u4(const bf16x8& v) { return __builtin_bit_cast(uint4, v); }

// ---------------------------------------------------------------------------------------
// 1. prologue
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prologue_kernel(const PrefillParams P, uint16_t* __restrict__ qh,
                                                       uint16_t* __restrict__ kh) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nq = P.batch * P.num_q_heads * P.q_len;
  const int q_tiles = (nq + 15) / 16;
  const int k_tiles = P.num_indices * P.num_kv_heads;
  const int waves = gridDim.x * (blockDim.x >> 6);
  const bool qnorm = P.q_norm != nullptr;
  const bool knorm = P.k_norm != nullptr;
  float qw[32], kw[32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qw[kb * 8 + e] = qnorm ? P.q_norm[32 * kb + 8 * g + e] : 1.0f;
      kw[kb * 8 + e] = knorm ? P.k_norm[32 * kb + 8 * g + e] : 1.0f;
    }
  const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  for (int task = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); task < q_tiles + k_tiles; task += waves) {
    uint4 raw[4];
    bf16x8 op[4];
    if (task < q_tiles) {
      const int v = task * 16 + r;  // flattened (b, h, i)
      const bool live = v < nq;
      int pos = 0;
      bool bad = false;
      if (live) {
        const int b = v / (P.num_q_heads * P.q_len);
        const int i = v % P.q_len;
        pos = P.qpos[(size_t)b * P.q_len + i];
        if (pos < 0 || pos >= P.table_rows) { bad = true; pos = 0; }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) raw[kb] = live ? ldg16(P.q + (size_t)v * kHeadDim + 32 * kb + 8 * g) : zero4;
      float4 cs[8];
      load_cos_sin(P.rope + (size_t)pos * kHeadDim, g, cs);
      prologue_operand(raw, qw, qnorm, P.eps, cs, op);
      if (live) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) stg16(qh + (size_t)v * kHeadDim + 32 * kb + 8 * g, bad ? nan4 : as_u4(op[kb]));
      }
    } else {
      const int kt = task - q_tiles;
      const int hk = kt / P.num_indices;
      const int gp = kt % P.num_indices;  // page slot in kv_indices
      // row owning this page slot: last b with indptr[b] <= gp
      int lo = 0, hi = P.batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (P.indptr[mid] <= gp) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int p0 = P.indptr[b], p1 = P.indptr[b + 1];
      const int n = p1 - p0, pr = gp - p0;
      const int lpl = P.last_page_len[b];
      const bool row_ok = p0 >= 0 && n > 0 && p1 <= P.num_indices && n <= P.max_pages_per_row && pr >= 0 &&
                          pr < n && lpl >= 1 && lpl <= kPageSize;
      const int L = row_ok ? (n - 1) * kPageSize + lpl : 0;
      const int j = pr * kPageSize + r;  // logical key index = key position
      const bool live = row_ok && j < L;
      int phys = P.indices[gp];
      const bool page_ok = phys >= 0 && phys < P.num_pages;
      if (!page_ok) phys = 0;
      const size_t src = (((size_t)phys * kPageSize + r) * P.num_kv_heads + hk) * kHeadDim + 8 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) raw[kb] = live ? ldg16(P.k_cache + src + 32 * kb) : zero4;
      float4 cs[8];
      load_cos_sin(P.rope + (size_t)(live ? j : 0) * kHeadDim, g, cs);
      prologue_operand(raw, kw, knorm, P.eps, cs, op);
      uint16_t* dst = kh + ((size_t)hk * P.num_indices * kPageSize + (size_t)gp * kPageSize + r) * kHeadDim + 8 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) stg16(dst + 32 * kb, !page_ok ? nan4 : (live ? as_u4(op[kb]) : zero4));
    }
  }
}

// ---------------------------------------------------------------------------------------
// 2. causal attention over the prepared q^ / k^ and the paged V
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attend_kernel(const PrefillParams P, const uint16_t* __restrict__ qh,
                                                      const uint16_t* __restrict__ kh) {
  __shared__ uint16_t sv[kKTile][kVRow];
  __shared__ int s_poison;
  const int G = P.group;
  const int Hkv = P.num_kv_heads;
  const int nqb = (P.q_len + kQBlock - 1) / kQBlock;
  // longest work first: the last query blocks of every row see the most keys
  const int nhg = (G + 3) / 4;
  const int per_qb = P.batch * Hkv * nhg;
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);
  int rest = blockIdx.x % per_qb;
  const int hg = rest % nhg;
  rest /= nhg;
  const int b = rest / Hkv;
  const int hk = rest % Hkv;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int gi = hg * 4 + wave;          // head within the GQA group
  const bool head_live = gi < G;         // trailing waves of a partial group only help stage V
  const int h = hk * G + (head_live ? gi : 0);
  const int Sq = P.q_len;

  const int p0 = P.indptr[b];
  const int p1 = P.indptr[b + 1];
  const int n = p1 - p0;
  const int lpl = P.last_page_len[b];
  const bool bad = p0 < 0 || n < 0 || p1 > P.num_indices || n > P.max_pages_per_row ||
                   (n > 0 && (lpl < 1 || lpl > kPageSize));
  const int L = (n > 0 && !bad) ? (n - 1) * kPageSize + lpl : 0;

  // positions of this lane's two queries (-1: past the chunk, sees nothing)
  int qp[2];
  int i_of[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = qb * kQBlock + 16 * t + r;
    i_of[t] = i;
    qp[t] = i < Sq ? P.qpos[(size_t)b * Sq + i] : -1;
  }
  // last key any query of the block can see
  int qmax = max(qp[0], qp[1]);
  qmax = max(qmax, __shfl_xor(qmax, 1));
  qmax = max(qmax, __shfl_xor(qmax, 2));
  qmax = max(qmax, __shfl_xor(qmax, 4));
  qmax = max(qmax, __shfl_xor(qmax, 8));
  const int kend = min(L, qmax + 1);
  const int ntiles = kend > 0 ? (kend + kKTile - 1) / kKTile : 0;

  if (tid == 0) s_poison = 0;

  bf16x8 qop[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const size_t off = (((size_t)b * P.num_q_heads + h) * Sq + i_of[t]) * kHeadDim + 32 * kb + 8 * g;
      qop[t][kb] = __builtin_bit_cast(bf16x8, (head_live && i_of[t] < Sq) ? ldg16(qh + off) : make_uint4(0, 0, 0, 0));
    }

  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_run[2] = {0.0f, 0.0f};
  f32x4 acc[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t kh_head = (size_t)hk * P.num_indices * kPageSize;
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    // stage the V tile [64 keys][128 dims] from the pages (zeros past the row's end)
    for (int s = tid; s < kKTile * 16; s += nthreads) {
      const int row = s >> 4, col = s & 15;
      const int j = kt * kKTile + row;
      const int pr = j / kPageSize;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < L) {
        int phys = P.indices[p0 + pr];
        if (phys < 0 || phys >= P.num_pages) { s_poison = 1; phys = 0; }
        v = ldg16(P.v_cache + (((size_t)phys * kPageSize + (j % kPageSize)) * Hkv + hk) * kHeadDim + col * 8);
      }
      *reinterpret_cast<uint4*>(&sv[row][col * 8]) = v;
    }
    __syncthreads();

    f32x4 sc[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int pr = kt * 4 + ks;
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[t][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (pr < n && head_live) {
        bf16x8 ka[4];
        const uint16_t* src = kh + (kh_head + (size_t)(p0 + pr) * kPageSize + r) * kHeadDim + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) ka[kb] = __builtin_bit_cast(bf16x8, ldg16(src + 32 * kb));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            sc[t][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qop[t][kb], sc[t][ks], 0, 0, 0);
      }
    }

    i16x4 pb[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float tv[4][4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kt * kKTile + 16 * ks + 4 * g + i;
          tv[ks][i] = (j < L && j <= qp[t]) ? sc[t][ks][i] * kScoreScaleLog2 : -__builtin_inff();
          mx = fmaxf(mx, tv[ks][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[t], mx);
      const bool any = m_new != -__builtin_inff();
      const float alpha = any ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.0f;
      float ps = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = any ? __builtin_amdgcn_exp2f(tv[ks][i] - m_new) : 0.0f;
          ps += p;
          pb[t][ks][i] = __builtin_bit_cast(short, (__bf16)p);
        }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run[t] = l_run[t] * alpha + ps;
      m_run[t] = m_new;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[t][nb] = acc[t][nb] * alpha;
    }

#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (kt * 4 + ks >= n || !head_live) continue;
        i16x4 va;  // V^T rows: dim 16*nb + r, keys 16*ks + 4g .. +3
#pragma unroll
        for (int e = 0; e < 4; ++e) va[e] = (short)sv[16 * ks + 4 * g + e][16 * nb + r];
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[t][ks], acc[t][nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const bool poison = bad || s_poison != 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = i_of[t];
    if (i >= Sq || !head_live) continue;
    const size_t row = ((size_t)b * P.num_q_heads + h) * Sq + i;
    const bool empty = l_run[t] == 0.0f;
    const float inv = empty ? 0.0f : 1.0f / l_run[t];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      uint2 w;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = poison ? __builtin_nanf("") : acc[t][nb][e] * inv;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16);
      *reinterpret_cast<uint2*>(P.out + row * kHeadDim + 16 * nb + 4 * g) = w;
    }
    if (g == 0) {
      float lse = empty ? -__builtin_inff() : (m_run[t] + __builtin_log2f(l_run[t])) * kLn2;
      if (poison) lse = __builtin_nanf("");
      P.lse[row] = lse;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  uint16_t* qh = (uint16_t*)p.workspace;
  uint16_t* kh = (uint16_t*)((char*)p.workspace + align256((size_t)p.batch * p.num_q_heads * p.q_len * kHeadDim * 2));
  const long long tasks = ((long long)p.batch * p.num_q_heads * p.q_len + 15) / 16 +
                          (long long)p.num_indices * p.num_kv_heads;
  const unsigned pro_blocks = (unsigned)std::min<long long>(std::max<long long>((tasks + 3) / 4, 1), 8192);
  hipLaunchKernelGGL(prologue_kernel, dim3(pro_blocks), dim3(256), 0, stream, p, qh, kh);
  const unsigned nqb = (unsigned)((p.q_len + kQBlock - 1) / kQBlock);
  const unsigned nhg = (unsigned)((p.group + 3) / 4);
  const unsigned grid = nqb * (unsigned)p.batch * (unsigned)p.num_kv_heads * nhg;
  const unsigned threads = 64u * (unsigned)std::min(p.group, 4);
  if (grid > 0) hipLaunchKernelGGL(attend_kernel, dim3(grid), dim3(threads), 0, stream, p, qh, kh);
  return hipGetLastError();
}

}  // namespace pa

// Paged decode: one workgroup per (row, KV head), no Split-KV.
//
// What it computes: for the G = Hq/Hkv query heads of one GQA group, softmax attention of
// the single query against every key of the row, with the Q/K prologue (RMSNorm, RoPE,
// BF16 rounding) fused into the page walk.  Sources: "[WS2][PR7][Attention] Add FlashInfer
// RoPE-fused paged attention scaffold", section "Scope" (logical K/V order before
// arithmetic; Split-KV disabled; FP32 LSE; GQA packing from the head layout);
// "flashinfer_fa2 backend for NVIDIA Ada (SM89)", sections "Summary" (page 16, head_dim 128,
// NHD) and "Design notes" (CSR metadata; with Split-KV disabled a row's result does not
// depend on the plan width or the batch).
//
// Reduction order.  The workgroup's W wavefronts take the row's pages round-robin (wave w
// takes logical pages w, w+W, w+2W, ...).  Each wave runs an FP32 online softmax over its
// pages in ascending order, one page (16 keys) per step: S^T = K^ Q^T by bf16 MFMA with FP32
// accumulation, a page max and sum per head taken in a fixed order (4 keys in registers, then
// a 2-step lane butterfly), and O^T += V^T P^T by bf16 MFMA into FP32 with P split into two
// bf16 parts (hi + lo), so the probabilities keep about 16 significant bits.  The W wave states are
// then combined in wave order 0..W-1 through LDS.  Every choice depends only on the row's own
// length, so the bits of a row are the same whatever batch it is in, whatever the plan width
// and wherever its pages sit.
//
// Memory layout.  k_cache/v_cache are NHD [page][slot][Hkv][128] bf16: one KV head of one
// page is 16 rows of 256 B at a stride of Hkv * 256 B.  A lane (r = lane % 16, g = lane / 16)
// loads key/value row r of the page as four 16-byte pieces (dims 32*kb + 8*g ..), so one
// load instruction covers 64 contiguous bytes of each of the 16 rows.  K goes straight from
// registers through the prologue into the MFMA A operand; V is staged in LDS and read back
// with keys along the MFMA reduction dimension.
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kDecodeWaves = 8;
constexpr int kDecodeThreads = kDecodeWaves * 64;
// V staging rows are padded by 16 bytes so that the transposed reads (one key row per lane
// group g) fall on different LDS banks.
constexpr int kVRow = kHeadDim + 8;

struct DecodeSmem {
  union {
    uint16_t v[kDecodeWaves][kPageSize][kVRow];   // per-wave V page, [key][dim]
    float acc[kDecodeWaves][4][kHeadDim];          // per-wave outputs of 4 heads (merge)
  } u;
  float m[kDecodeWaves][kMaxGroup];
  float l[kDecodeWaves][kMaxGroup];
  int poison[kDecodeWaves];
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const DecodeParams P) {
  __shared__ DecodeSmem sm;
  const int unit = blockIdx.x;
  const int b = unit / P.num_kv_heads;
  const int hk = unit % P.num_kv_heads;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int G = P.group;
  const int Hkv = P.num_kv_heads;

  // ---- row geometry (CSR block table) and bounds checks -------------------------------
  const int p0 = P.indptr[b];
  const int p1 = P.indptr[b + 1];
  const int n = p1 - p0;
  const int lpl = P.last_page_len[b];
  const int qp = P.qpos[b];
  const bool bad = p0 < 0 || n < 0 || p1 > P.num_indices || n > P.max_pages_per_row || qp < 0 ||
                   qp >= P.table_rows || (n > 0 && (lpl < 1 || lpl > kPageSize));
  const int L = (n > 0 && !bad) ? (n - 1) * kPageSize + lpl : 0;
  const size_t head0 = (size_t)b * P.num_q_heads + (size_t)hk * G;  // first head of the group
  if (bad || L == 0) {
    for (int i = tid; i < G * kHeadDim; i += kDecodeThreads) {
      const int h = i / kHeadDim, d = i % kHeadDim;
      P.out[(head0 + h) * kHeadDim + d] = bad ? (uint16_t)0x7FC0 : (uint16_t)0;
      if (d == 0) P.lse[head0 + h] = bad ? __builtin_nanf("") : -__builtin_inff();
    }
    return;
  }

  const bool qnorm = P.q_norm != nullptr;
  const bool knorm = P.k_norm != nullptr;

  // ---- q^ of the group's heads in the operand layout (vector r = head r < G) -----------
  bf16x8 qop[4];
  {
    float w[32];
    uint4 raw[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      raw[kb] = make_uint4(0, 0, 0, 0);
      if (r < G) raw[kb] = ldg16(P.q + (head0 + r) * kHeadDim + 32 * kb + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[kb * 8 + e] = qnorm ? P.q_norm[32 * kb + 8 * g + e] : 1.0f;
    }
    prologue_operand(raw, w, qnorm, P.eps, P.rope + (size_t)qp * kHeadDim, g, qop);
  }
  float kw[32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) kw[kb * 8 + e] = knorm ? P.k_norm[32 * kb + 8 * g + e] : 1.0f;

  // ---- per-wave online softmax over pages w, w+W, ... ---------------------------------
  // S^T tile (MFMA C of K^ . Q^T): lane (r, g) holds keys 4g+i (i = 0..3) of head r.  The
  // same registers, rounded to bf16, are the B operand (P^T) of O^T += V^T . P^T, whose C
  // layout gives lane (r, g) dims 16*nb + 4g + i of head r.  m, l of head r live in every
  // lane with that r.
  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  int poison = 0;

  for (int pg = wave; pg < n; pg += kDecodeWaves) {
    int phys = P.indices[p0 + pg];
    if (phys < 0 || phys >= P.num_pages) { poison = 1; phys = 0; }
    const size_t row_off = (((size_t)phys * kPageSize + r) * Hkv + hk) * kHeadDim + 8 * g;
    uint4 kraw[4], vraw[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      kraw[kb] = ldg16(P.k_cache + row_off + 32 * kb);
      vraw[kb] = ldg16(P.v_cache + row_off + 32 * kb);
    }
    // stage V for the transposed read; rows past the row's end are zero
    const bool vlive = pg * kPageSize + r < L;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      *reinterpret_cast<uint4*>(&sm.u.v[wave][r][32 * kb + 8 * g]) = vlive ? vraw[kb] : make_uint4(0, 0, 0, 0);

    bf16x8 kop[4];
    prologue_operand(kraw, kw, knorm, P.eps, P.rope + (size_t)(pg * kPageSize + r) * kHeadDim, g, kop);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb], qop[kb], s, 0, 0, 0);

    float t[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = pg * kPageSize + 4 * g + i;  // logical key index = key position
      t[i] = (j < L && j <= qp) ? s[i] * kScoreScaleLog2 : -__builtin_inff();
      mx = fmaxf(mx, t[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool any = m_new != -__builtin_inff();
    const float alpha = any ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    float pr[4];
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = any ? __builtin_amdgcn_exp2f(t[i] - m_new) : 0.0f;
      ps += pr[i];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // P^T as two bf16 parts, hi + lo, so the P.V product keeps ~16 bits of each probability
    i16x4 pb_hi, pb_lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 hi = (__bf16)pr[i];
      pb_hi[i] = __builtin_bit_cast(short, hi);
      pb_lo[i] = __builtin_bit_cast(short, (__bf16)(pr[i] - (float)hi));
    }

    wave_lds_sync();
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      i16x4 va;  // V^T rows: dim 16*nb + r, keys 4g .. 4g+3
#pragma unroll
      for (int e = 0; e < 4; ++e) va[e] = (short)sm.u.v[wave][4 * g + e][16 * nb + r];
      acc[nb] = acc[nb] * alpha;
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_hi, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_lo, acc[nb], 0, 0, 0);
    }
    wave_lds_sync();
  }

  // ---- combine the W wave states in wave order -----------------------------------------
  if (g == 0 && r < G) { sm.m[wave][r] = m_run; sm.l[wave][r] = l_run; }
  if (lane == 0) sm.poison[wave] = poison;
  __syncthreads();
  int any_poison = 0;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) any_poison |= sm.poison[w];

  // heads are merged four at a time through LDS
  for (int h0 = 0; h0 < G; h0 += 4) {
    if (r >= h0 && r < h0 + 4) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.u.acc[wave][r - h0][16 * nb + 4 * g + i] = acc[nb][i];
    }
    __syncthreads();
    const int nh = min(4, G - h0);
    for (int idx = tid; idx < nh * kHeadDim; idx += kDecodeThreads) {
      const int hi = idx / kHeadDim, d = idx % kHeadDim;
      const int h = h0 + hi;
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm.m[w][h]);
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float mw = sm.m[w][h];
        const float sc = mw == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        num += sm.u.acc[w][hi][d] * sc;
        den += sm.l[w][h] * sc;
      }
      float o = num / den;
      float lse = (M + __builtin_log2f(den)) * kLn2;
      if (any_poison) { o = __builtin_nanf(""); lse = __builtin_nanf(""); }
      P.out[(head0 + h) * kHeadDim + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
      if (d == 0) P.lse[head0 + h] = lse;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.batch * (unsigned)p.num_kv_heads;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa

// Deterministic backward of full-prefill attention (the training layout).
//
// Sources: "[WS2][PR7][Attention] Add FlashInfer RoPE-fused paged attention scaffold",
// section "Scope" (the strict path requires a deterministic backward, dropout 0); "WS2 PR7
// Fused Attention Backend Alignment", sections "Goal" (a training full-prefill lane) and
// "Original PR7 Requirements" (the training forward is full prefill; dq/dk/dv belong to the
// training backward).  The forward it differentiates is the library's: q^ = bf16(RoPE(
// RMSNorm(q) w_q)), k^ likewise, s = q^.k^ / sqrt(128) over keys at positions <= the query's,
// softmax, out = P V.  The BF16 roundings at the post-RoPE boundary and of out pass gradients
// through unchanged.
//
// Layout: q, dout, out [B, Hq, S, 128] bf16; k, v [B, Hkv, S, 128] bf16; positions [B, S]
// (token i of row b has its query and its key at positions[b][i]); lse [B, Hq, S] fp32 (the
// forward's, natural log).  Outputs dq [B, Hq, S, 128], dk and dv [B, Hkv, S, 128] fp32, and
// the gradients of the two RMSNorm weights, fp32 [128].
//
// Four kernels, every sum in a fixed order (no atomics):
//  1. bwd_prep_kernel: k^ (the forward's prologue, bit for bit) into the workspace, and the
//     least and greatest position of every 16 tokens.
//  2. bwd_dq_kernel: one workgroup per (32 queries, row, KV head, up to 4 query heads), as in
//     the forward.  It first computes its queries' q^ (the forward's prologue, bit for bit) and
//     Dv = sum_d dout * out (FP32: a lane's 32 terms in order, then the four lanes of the query
//     pairwise), and writes both to the workspace for kernel 3.  Then per 32-key tile, staged
//     in LDS for the 4 heads: S^T = K^ Q^T, P^T from the
//     forward's LSE, dP^T = V dO^T, dS^T = P^T (dP^T - Dv), dQ^T += K^T dS^T (key tiles in
//     ascending order; tiles whose keys all follow every query are not visited).  The
//     epilogue applies the transposed rotation and the RMSNorm backward, writes dq, and writes
//     this wavefront's share of the q weight gradient.
//  3. bwd_dkdv_kernel: one workgroup per (64 keys, row, KV head), 16 keys per wavefront; the
//     group's query heads in ascending order, each head's 32-query tiles in ascending order
//     (staged in LDS once for the four wavefronts; tiles whose queries all precede every key
//     are not visited): S = Q^ K^T, P, dV^T += dO^T P, dP = dO V^T, dS, dK^T += Q^T dS.  The
//     epilogue writes dv, and dk through the prologue backward, and the wavefront's share of
//     the k weight gradient.
//  4. bwd_sum_rows_kernel: the weight-gradient shares summed by a fixed tree (256 rows per
//     workgroup, levels until one row is left; one launch per level for both weights).
// MFMA operands are BF16 (q^, k^, v, dout, and P and dS rounded to BF16), accumulation FP32.
#include "pa_internal.h"
#include "pa_lds_dma.h"

namespace pa {

namespace {

constexpr int kQB = 32;                 // queries per wavefront (dq kernel) / per tile (dkdv kernel)
constexpr int kKTile = 32;              // keys per tile (dq kernel)
constexpr int kBwdThreads = 256;
constexpr float kLog2e = 1.4426950408889634074f;
constexpr float kSoftmaxScale = 0.08838834764831844055f;  // 1 / sqrt(128)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ i16x8 concat4(const i16x4& a, const i16x4& b) {
  return i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ i16x4 pack4_bf16(float a, float b, float c, float d) {
  return i16x4{__builtin_bit_cast(short, (__bf16)a), __builtin_bit_cast(short, (__bf16)b),
               __builtin_bit_cast(short, (__bf16)c), __builtin_bit_cast(short, (__bf16)d)};
}

// cos/sin of the frequencies of the accumulator layout: lane group g, block nb = 0..3 holds
// frequencies 16 nb + 4 g + i (i = 0..3), the rotation partners of dims 16 nb + 4 g + i and
// 64 + 16 nb + 4 g + i.  Read from the plan's table (blocks of 16 positions, [e][lane][4]; entry
// q of lane (pos % 16) + 16 g' holds the cos of frequencies f(q, g') .. + 3, entry 4 + q the
// sin, f(q, g') = 8 g' + 4 q for q < 2 and 32 + 8 g' + 4 (q - 2) otherwise).
__device__ __forceinline__ void load_cos_sin_acc(const float* rope, int pos, int g, float4 c[4], float4 s[4]) {
  const float4* blk = reinterpret_cast<const float4*>(rope + (size_t)(pos >> 4) * kRopeBlockFloats);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int f0 = 16 * nb + 4 * g;
    const int gp = f0 < 32 ? (f0 >> 3) : ((f0 - 32) >> 3);
    const int q = f0 < 32 ? ((f0 >> 2) & 1) : 2 + (((f0 - 32) >> 2) & 1);
    const int lane = (pos & 15) + 16 * gp;
    c[nb] = blk[q * 64 + lane];
    s[nb] = blk[(4 + q) * 64 + lane];
  }
}

struct BwdParams {
  int32_t batch, seq, num_q_heads, num_kv_heads, group, table_rows;
  const int32_t* pos;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;
  const float* q_norm;
  const float* k_norm;
  const float* rope;
  float eps;
  float* dq;
  float* dk;
  float* dv;
  float* dq_norm;
  float* dk_norm;
  // workspace
  uint16_t* qh;   // [B, Hq, S, 128]
  uint16_t* kh;   // [B, Hkv, S, 128]
  float* dvec;    // [B, Hq, S]
  int* tmin;       // [B, ceil(S / 16)]: least position of each 16 tokens (INT32_MAX past the row)
  int* tmax;       // [B, ceil(S / 16)]: greatest position of each 16 tokens (-1 past the row)
  float* dwq_part;  // [dq workgroups][4][128]
  float* dwk_part;  // [dkdv workgroups][4][128]
  int32_t dq_wgs, dkdv_wgs;
};

__device__ __forceinline__ int safe_pos(const BwdParams& P, int b, int i, bool& bad) {
  int p = P.pos[(size_t)b * P.seq + i];
  if (p < 0 || p >= P.table_rows) { bad = true; p = 0; }
  return p;
}

// ---------------------------------------------------------------------------------------
// 1. k^ and the 16-token position bounds.  One wavefront per 16 keys of one KV head.  (q^ and
// Dv are computed by the dq kernel, whose workgroups each own their queries.)
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(const BwdParams P) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int tiles = (P.seq + 15) / 16;
  const int k_tasks = P.batch * P.num_kv_heads * tiles;
  const int waves = gridDim.x * (blockDim.x >> 6);
  const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  for (int u = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); u < k_tasks; u += waves) {
    const int tile = u % tiles;
    const int bh = u / tiles;  // b * Hkv + hk
    const int b = bh / P.num_kv_heads;
    const int i = tile * 16 + r;
    const bool live = i < P.seq;
    bool bad = false;
    const int pos = live ? safe_pos(P, b, i, bad) : 0;
    const size_t row = ((size_t)bh * P.seq + (live ? i : 0)) * kHeadDim + 8 * g;
    uint4 raw[4];
    float w[32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      raw[kb] = live ? ldg16(P.k + row + 32 * kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[kb * 8 + e] = P.k_norm ? P.k_norm[32 * kb + 8 * g + e] : 1.0f;
    }
    if (bh % P.num_kv_heads == 0) {
      // the position bounds of these 16 tokens (the same for every head), for tile skipping
      int lo = live ? pos : INT32_MAX, hi = live ? pos : -1;
#pragma unroll
      for (int sh = 1; sh < 16; sh <<= 1) {
        lo = min(lo, __shfl_xor(lo, sh));
        hi = max(hi, __shfl_xor(hi, sh));
      }
      if (lane == 0) {
        P.tmin[(size_t)b * tiles + tile] = lo;
        P.tmax[(size_t)b * tiles + tile] = hi;
      }
    }
    float4 cs[8];
    load_cos_sin(P.rope, pos, g, cs);
    bf16x8 op[4];
    prologue_operand(raw, w, P.k_norm != nullptr, P.eps, cs, op);
    if (live) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        *reinterpret_cast<uint4*>(P.kh + row + 32 * kb) = bad ? nan4 : __builtin_bit_cast(uint4, op[kb]);
    }
  }
}

// The prologue backward of one token in the accumulator layout (lane (r, g): dims 16 nb + 4 g
// + i, nb = 0..7), on the four lanes r, r+16, r+32, r+48 together.  grad: d loss / d (rotated
// vector); x: the pre-norm input; w: the norm weights of the lane's dims (1 without a norm).
// Writes dx (the gradient of the input) and accumulates x r dy into dw (the weight gradient).
//   dy1 = g1 c + g2 s, dy2 = -g1 s + g2 c          (the inverse rotation)
//   dx  = r w dy - x r^3 (1/128) sum_k x_k w_k dy_k,  r = (mean(x^2) + eps)^-1/2
__device__ __forceinline__ void prologue_backward(const f32x4 grad[8], const float x[8][4], const float4 wv[8],
                                                  bool norm, float eps, const float4 c[4], const float4 s[4],
                                                  float dx[8][4], float dw[8][4]) {
  float dy[8][4];
  const float* cf = reinterpret_cast<const float*>(c);
  const float* sf = reinterpret_cast<const float*>(s);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g1 = grad[nb][i], g2 = grad[nb + 4][i];
      const float cc = cf[4 * nb + i], ss = sf[4 * nb + i];
      dy[nb][i] = g1 * cc + g2 * ss;
      dy[nb + 4][i] = g2 * cc - g1 * ss;
    }
  if (!norm) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dx[nb][i] = dy[nb][i];
    return;
  }
  // r from the exact sum of squares (as the forward)
  double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = __builtin_fma((double)x[nb][i], (double)x[nb][i], s4[i]);
  double ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  ss = pair16_sum(ss);
  ss = pair32_sum(ss);
  const float ms = (float)(ss * (1.0 / kHeadDim));
  const float rr = (float)(1.0 / __builtin_sqrt((double)(ms + eps)));
  const float* wf = reinterpret_cast<const float*>(wv);
  float sum = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sum = __builtin_fmaf(x[nb][i], wf[4 * nb + i] * dy[nb][i], sum);
  sum = pair32_sum(pair16_sum(sum));
  const float k3 = rr * rr * rr * sum * (1.0f / kHeadDim);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dx[nb][i] = rr * wf[4 * nb + i] * dy[nb][i] - x[nb][i] * k3;
      dw[nb][i] = __builtin_fmaf(x[nb][i] * rr, dy[nb][i], dw[nb][i]);
    }
}

// x (bf16 input) and the norm weights of the lane's accumulator-layout dims for one token
__device__ __forceinline__ void load_acc_layout(const uint16_t* rowp, const float* w, int g, float x[8][4],
                                                float4 wv[8], bool live) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const uint2 u = live ? *reinterpret_cast<const uint2*>(rowp + 16 * nb + 4 * g) : make_uint2(0, 0);
    x[nb][0] = bf16_lo(u.x); x[nb][1] = bf16_hi(u.x);
    x[nb][2] = bf16_lo(u.y); x[nb][3] = bf16_hi(u.y);
    wv[nb] = w ? *reinterpret_cast<const float4*>(w + 16 * nb + 4 * g) : make_float4(1.f, 1.f, 1.f, 1.f);
  }
}

// Sum over the 16 lanes of a lane group (a fixed butterfly; both lanes of a pair add the same
// two values, and IEEE addition is commutative, so they agree) of each of the 32 values.
__device__ __forceinline__ void sum16(float v[8][4]) {
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[nb][i] = v[nb][i] + __shfl_xor(v[nb][i], sh);
}

// ---------------------------------------------------------------------------------------
// 2. dq
// ---------------------------------------------------------------------------------------
// k^ and V tiles in LDS: rows of 256 bytes, the 16-byte chunk c of row j stored at chunk
// c ^ dq_swz(j), dq_swz(j) = 2 (j mod 8).  Both read patterns then use all 64 banks without
// conflict (measured with the LDS bank-conflict counter on these exact patterns):
//  - the S and dP operands: 16-byte reads, lane (r, g) = (lane % 16, lane / 16) at row r,
//    chunk 4 kb + g.  Such a read is served 16 lanes per LDS cycle, and the 16 lanes of a
//    cycle are those with equal lane bit 5 and equal parity of lane bits 2..4 (not 16
//    consecutive lanes: a swizzle giving each run of 16 consecutive lanes 16 distinct chunks
//    still took two cycles per group).  g ^ dq_swz(r) is then distinct within every group.
//  - the transposed K^T (dQ) or dO^T / Q^T (dK/dV) reads: 8-byte reads, 32 lanes per cycle,
//    32 bytes of each of 8 consecutive rows; the chunk pair {2 m, 2 m + 1} of row j lands on
//    pair m ^ (j mod 8), distinct over the 8 rows.
// (A padded 288-byte pitch was conflict-free for the second pattern only.)
// The tiles are arrays of 16-byte chunks, so that the compiler emits whole 16-byte LDS
// accesses (it splits them into 4-byte pairs where it cannot prove the alignment).  The dK/dV
// kernel's q^ and dout tiles have the same layout and the same two read patterns.
__device__ __forceinline__ int dq_swz(int row) { return 2 * (row & 7); }
// chunk index of the 16-byte chunk c (dims 8 c .. 8 c + 7) of row j in a swizzled tile
__device__ __forceinline__ int dq_chunk(int row, int c) { return row * (kHeadDim / 8) + (c ^ dq_swz(row)); }
struct alignas(16) DqSmem {
  uint4 k[2][kKTile * kHeadDim / 8];
  uint4 v[2][kKTile * kHeadDim / 8];
  int kpos[2][kKTile];
};

__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(const BwdParams P) {
  __shared__ DqSmem sm;
  const int G = P.group;
  const int Hkv = P.num_kv_heads;
  const int S = P.seq;
  const int nqb = (S + kQB - 1) / kQB;
  const int nhg = (G + 3) / 4;
  const int per_qb = P.batch * Hkv * nhg;
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);  // longest first
  int rest = blockIdx.x % per_qb;
  const int hg = rest % nhg;
  rest /= nhg;
  const int b = rest / Hkv;
  const int hk = rest % Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int gi = hg * 4 + wave;
  const bool head_live = gi < G;
  const int h = hk * G + (head_live ? gi : 0);
  const size_t qrow0 = ((size_t)b * P.num_q_heads + h) * S;   // token 0 of this head
  const size_t krow0 = ((size_t)b * Hkv + hk) * S;

  // this lane's queries (t = 0, 1: query 16 t + r of the block)
  int qpos[2], qi[2];
  float lse2[2], dv_[2];
  bf16x8 qop[2][4], dop[2][4];
  int qmax = -1;
  bool bad[2] = {false, false};  // the query's position is outside the RoPE table
  // q^ (the forward's prologue, same bits) and Dv = sum over dims of dout * out, for the
  // block's queries; the workgroup owns them, so it also writes both for the dK/dV kernel
  const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = qb * kQB + 16 * t + r;
    qi[t] = i;
    const bool live = i < S;
    qpos[t] = live ? safe_pos(P, b, i, bad[t]) : -1;
    qmax = max(qmax, qpos[t]);
    lse2[t] = live ? P.lse[qrow0 + i] * kLog2e : 0.0f;
    const size_t row = (qrow0 + (live ? i : 0)) * kHeadDim + 8 * g;
    uint4 raw[4];
    float w[32];
    float dsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      raw[kb] = live ? ldg16(P.q + row + 32 * kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[kb * 8 + e] = P.q_norm ? P.q_norm[32 * kb + 8 * g + e] : 1.0f;
      const uint4 d = live ? ldg16(P.dout + row + 32 * kb) : make_uint4(0, 0, 0, 0);
      dop[t][kb] = __builtin_bit_cast(bf16x8, d);
      float a[8], o[8];
      unpack8(d, a);
      unpack8(live ? ldg16(P.out + row + 32 * kb) : make_uint4(0, 0, 0, 0), o);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf(a[e], o[e], dsum);
    }
    dsum = pair32_sum(pair16_sum(dsum));
    dv_[t] = live ? dsum : 0.0f;
    float4 cs[8];
    load_cos_sin(P.rope, live ? qpos[t] : 0, g, cs);
    bf16x8 op[4];
    prologue_operand(raw, w, P.q_norm != nullptr, P.eps, cs, op);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 v = !live ? make_uint4(0, 0, 0, 0) : bad[t] ? nan4 : __builtin_bit_cast(uint4, op[kb]);
      qop[t][kb] = __builtin_bit_cast(bf16x8, v);
      if (head_live && live) *reinterpret_cast<uint4*>(P.qh + row + 32 * kb) = v;
    }
    if (head_live && live && g == 0) P.dvec[qrow0 + i] = dsum;
  }
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) qmax = max(qmax, __shfl_xor(qmax, sh));
  qmax = __builtin_amdgcn_readfirstlane(qmax);
  // every wavefront of the block has the same queries: the key tiles to visit are the ones
  // holding a key at or before the last query position (keys are visited in token order)
  const int ntiles = (S + kKTile - 1) / kKTile;

  f32x4 acc[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int jr = 4 * g + (r >> 2);
  const int jc = 4 * (r & 3);

  // A tile goes to LDS one tile ahead: its k^ and V rows by direct-to-LDS loads, wavefront w
  // rows 8 w .. 8 w + 7 of each (two loads of four rows: lane l, row 4 i + l / 16, physical
  // chunk l % 16, which holds logical chunk (l % 16) ^ swizzle(row)); and (threads < 32) one
  // key's position through a register, written after the current tile is used.  The direct
  // loads are waited for before the barrier that publishes the tile.
  uint32_t dma_off[2];
  int dma_row[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    dma_row[u] = 8 * wave + 4 * u + (lane >> 4);
    dma_off[u] = 16u * (uint32_t)((lane & 15) ^ dq_swz(dma_row[u]));
  }
  const uint16_t* kbase = P.kh + krow0 * kHeadDim;
  const uint16_t* vbase = P.v + krow0 * kHeadDim;
  int kp_next = INT32_MAX;
  bool klive_next = false;
  auto load_tile = [&](int kt, int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // a key past the row reads key 0: its position (INT32_MAX) makes its P and dS zero
      const int j = kt * kKTile + dma_row[u];
      const uint32_t voff = (uint32_t)(j < S ? j : 0) * (kHeadDim * 2) + dma_off[u];
      const int slot = 2 * wave + u;  // 1 KB slot of the tile: rows 4 slot .. 4 slot + 3
      lds_dma16(lds_address(&sm.k[buf][64 * slot]), kbase, voff);
      lds_dma16(lds_address(&sm.v[buf][64 * slot]), vbase, voff);
    }
    if (tid < kKTile) {
      // the raw position, checked in store_tile (so that no wait for it falls inside the
      // current tile's work)
      const int j = kt * kKTile + tid;
      klive_next = j < S;
      kp_next = P.pos[(size_t)b * S + (klive_next ? j : 0)];
    }
  };
  auto store_tile = [&](int buf) {
    // keys past the row get a position no query can see; a position outside the RoPE table
    // reads as 0 (the key's own rows are poisoned)
    if (tid < kKTile) sm.kpos[buf][tid] = !klive_next ? INT32_MAX : (kp_next < 0 || kp_next >= P.table_rows ? 0 : kp_next);
  };
  // the first key tile at or after kt holding a key at or before the block's last query
  // position (tiles whose keys all come after every query contribute nothing)
  const int n16 = (S + 15) / 16;
  // (the visibility of 64 consecutive tiles is one ballot; the window is kept, so the walk
  // loads the bounds once per 64 tiles instead of waiting for them at every tile)
  int wbase = -64;
  unsigned long long wmask = 0;
  auto next_tile = [&](int kt) -> int {
    while (kt < ntiles) {
      if (kt < wbase || kt >= wbase + 64) {
        wbase = kt;
        const int c = kt + lane;
        int m = INT32_MAX;
        if (c < ntiles) {
          m = P.tmin[(size_t)b * n16 + 2 * c];
          if (2 * c + 1 < n16) m = min(m, P.tmin[(size_t)b * n16 + 2 * c + 1]);
        }
        wmask = __builtin_amdgcn_ballot_w64(m <= qmax);
      }
      const unsigned long long hit = wmask >> (kt - wbase);
      if (hit != 0) return kt + (int)__builtin_ctzll(hit);
      kt = wbase + 64;
    }
    return ntiles;
  };
  const int first = __builtin_amdgcn_readfirstlane(next_tile(0));
  if (first < ntiles) {
    load_tile(first, 0);
    store_tile(0);
    wait_vmcnt<0>();
    __syncthreads();
    int buf = 0;
    for (int kt = first;;) {
      const int nk = __builtin_amdgcn_readfirstlane(next_tile(kt + 1));
      const bool more = nk < ntiles;
      if (more) load_tile(nk, buf ^ 1);
      if (head_live) {
        f32x4 s[2][2], dp[2][2];  // [ks][t]: keys 16 ks + 4 g + i, query 16 t + r
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 ka[4], va[4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            ka[kb] = __builtin_bit_cast(bf16x8, sm.k[buf][dq_chunk(16 * ks + r, 4 * kb + g)]);
            va[kb] = __builtin_bit_cast(bf16x8, sm.v[buf][dq_chunk(16 * ks + r, 4 * kb + g)]);
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            s[ks][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[ks][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              s[ks][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qop[t][kb], s[ks][t], 0, 0, 0);
              dp[ks][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[kb], dop[t][kb], dp[ks][t], 0, 0, 0);
            }
          }
        }
        // dS^T = P^T (dP^T - Dv), P^T = 2^(s c log2e - lse log2e) on visible keys, else 0
        i16x4 dsb[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            float d4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kp = sm.kpos[buf][16 * ks + 4 * g + i];
              const float p = kp <= qpos[t] ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks][t][i], kScoreScaleLog2, -lse2[t])) : 0.0f;
              d4[i] = p * (dp[ks][t][i] - dv_[t]);
            }
            dsb[t][ks] = pack4_bf16(d4[0], d4[1], d4[2], d4[3]);
          }
        // dQ^T += K^T dS^T over the tile's 32 keys: k-slot 8g+e holds key 4g+e (e < 4) and key
        // 16+4g+(e-4) (e >= 4) in both operands; K^T from two transposed reads per column block
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          // dims 16 nb + jc .. +3: chunk 2 nb + jc / 8, its half jc % 8 / 4
          const i16x4 k0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(reinterpret_cast<char*>(&sm.k[buf][dq_chunk(jr, 2 * nb + (jc >> 3))]) + 2 * (jc & 7)));
          const i16x4 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(reinterpret_cast<char*>(&sm.k[buf][dq_chunk(16 + jr, 2 * nb + (jc >> 3))]) + 2 * (jc & 7)));
          const bf16x8 kt8 = __builtin_bit_cast(bf16x8, concat4(k0, k1));
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                kt8, __builtin_bit_cast(bf16x8, concat4(dsb[t][0], dsb[t][1])), acc[t][nb], 0, 0, 0);
        }
      }
      if (more) store_tile(buf ^ 1);
      wait_vmcnt<0>();
      __syncthreads();
      if (!more) break;
      kt = nk;
      buf ^= 1;
    }
  }
  if (!head_live) {
    // a trailing slot of a partial group: its share of the weight gradient is zero
    if (P.q_norm != nullptr && r == 0) {
      float* part = P.dwq_part + ((size_t)blockIdx.x * 4 + wave) * kHeadDim;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) *reinterpret_cast<float4*>(part + 16 * nb + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }

  // epilogue: dq^ = c acc, then the prologue backward; lane (r, g) of tile t holds query 16t+r,
  // dims 16 nb + 4 g + i
  float dwq[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dwq[nb][i] = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = qi[t];
    const bool live = i < S;
    f32x4 grad[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) grad[nb] = acc[t][nb] * kSoftmaxScale;
    float x[8][4];
    float4 wv[8];
    load_acc_layout(P.q + (qrow0 + (live ? i : 0)) * kHeadDim, P.q_norm, g, x, wv, live);
    float4 c[4], sn[4];
    load_cos_sin_acc(P.rope, live ? qpos[t] : 0, g, c, sn);
    float dx[8][4];
    float dwt[8][4];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dwt[nb][e] = 0.0f;
    prologue_backward(grad, x, wv, P.q_norm != nullptr, P.eps, c, sn, dx, dwt);
    if (live) {
      float* dst = P.dq + (qrow0 + i) * kHeadDim;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        float4 o = make_float4(dx[nb][0], dx[nb][1], dx[nb][2], dx[nb][3]);
        if (bad[t]) o = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
        *reinterpret_cast<float4*>(dst + 16 * nb + 4 * g) = o;
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dwq[nb][e] += dwt[nb][e];
    }
  }
  if (P.q_norm != nullptr) {
    sum16(dwq);
    if (r == 0) {
      float* part = P.dwq_part + ((size_t)blockIdx.x * 4 + wave) * kHeadDim;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        *reinterpret_cast<float4*>(part + 16 * nb + 4 * g) = make_float4(dwq[nb][0], dwq[nb][1], dwq[nb][2], dwq[nb][3]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// 3. dk, dv
// ---------------------------------------------------------------------------------------
constexpr int kKBlock = 64;   // keys per workgroup, 16 per wavefront

// one 32-query tile of one query head, shared by the workgroup's four wavefronts
struct alignas(16) DkdvTile {
  uint4 q[kQB * kHeadDim / 8];  // q^ rows, 16-byte chunks swizzled as in the dq kernel (dq_chunk)
  uint4 d[kQB * kHeadDim / 8];  // dout rows, likewise
  float lse2[kQB];
  float dvec[kQB];
  int qpos[kQB];
};

__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(const BwdParams P) {
  __shared__ DkdvTile sm[2];
  const int G = P.group;
  const int Hkv = P.num_kv_heads;
  const int S = P.seq;
  const int units = P.batch * Hkv;
  const int kblk = (int)blockIdx.x / units;  // the first key blocks see the most queries: launched first
  const int unit = (int)blockIdx.x % units;
  const int b = unit / Hkv;
  const int hk = unit % Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const size_t krow0 = ((size_t)b * Hkv + hk) * S;
  const int n16 = (S + 15) / 16;
  const int nqt = (S + kQB - 1) / kQB;

  // this lane's key (column r of the wavefront's score tiles) and the wavefront's operands
  const int j = kblk * kKBlock + 16 * wave + r;
  const bool klive = j < S;
  bool bad = false;
  const int kpos = klive ? safe_pos(P, b, j, bad) : INT32_MAX;
  int kmin = kpos;
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) kmin = min(kmin, __shfl_xor(kmin, sh));
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  // the block's least key position, from the bounds of its four 16-token groups
  int bmin = INT32_MAX;
  {
    const int t16 = kblk * 4 + (lane & 3);
    if (t16 < n16) bmin = P.tmin[(size_t)b * n16 + t16];
    bmin = min(bmin, __shfl_xor(bmin, 1));
    bmin = min(bmin, __shfl_xor(bmin, 2));
    bmin = __builtin_amdgcn_readfirstlane(bmin);
  }
  bf16x8 kop[4], vop[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const size_t off = (krow0 + (klive ? j : 0)) * kHeadDim + 32 * kb + 8 * g;
    kop[kb] = __builtin_bit_cast(bf16x8, klive ? ldg16(P.kh + off) : make_uint4(0, 0, 0, 0));
    vop[kb] = __builtin_bit_cast(bf16x8, klive ? ldg16(P.v + off) : make_uint4(0, 0, 0, 0));
  }
  f32x4 dk[8], dvv[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) { dk[nb] = f32x4{0.f, 0.f, 0.f, 0.f}; dvv[nb] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  const int jr = 4 * g + (r >> 2);
  const int jc = 4 * (r & 3);

  // the first query tile at or after qt holding a query that some key of the block can see
  // (tiles where every query precedes every key contribute nothing and are not visited)
  // (the visibility of 64 consecutive tiles is one ballot; the window is kept, so the walk
  // loads the bounds once per 64 tiles instead of waiting for them at every tile, and every
  // query head of the group walks the same tiles)
  int wbase = -64;
  unsigned long long wmask = 0;
  int wmax = -1;  // lane c: the greatest query position of tile wbase + c
  auto next_tile = [&](int qt) -> int {
    while (qt < nqt) {
      if (qt < wbase || qt >= wbase + 64) {
        wbase = qt;
        const int c = qt + lane;
        int m = -1;
        if (c < nqt) {
          m = P.tmax[(size_t)b * n16 + 2 * c];
          if (2 * c + 1 < n16) m = max(m, P.tmax[(size_t)b * n16 + 2 * c + 1]);
        }
        wmax = m;
        wmask = __builtin_amdgcn_ballot_w64(m >= bmin);
      }
      const unsigned long long hit = wmask >> (qt - wbase);
      if (hit != 0) return qt + (int)__builtin_ctzll(hit);
      qt = wbase + 64;
    }
    return nqt;
  };
  // the greatest query position of tile qt, which the current window holds
  auto tile_qmax = [&](int qt) -> int { return __builtin_amdgcn_readlane(wmax, qt - wbase); };

  // A tile goes to LDS one tile ahead: its q^ and dout rows by direct-to-LDS loads, wavefront w
  // rows 8 w .. 8 w + 7 of each (two loads of four rows: lane l, row 4 i + l / 16, physical
  // chunk l % 16, which holds logical chunk (l % 16) ^ swizzle(row)); and (threads < 32) one
  // query's lse, Dv and position through registers, written after the current tile is used.
  // (Nothing reads a loaded value before store_tile, so no wait falls inside the current
  // tile's work; the direct loads are waited for before the barrier that publishes the tile.)
  uint32_t dma_off[2];
  int dma_row[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    dma_row[u] = 8 * wave + 4 * u + (lane >> 4);
    dma_off[u] = 16u * (uint32_t)((lane & 15) ^ dq_swz(dma_row[u]));
  }
  float lse_n = 0.0f, dv_n = 0.0f;
  int qp_n = -1;
  bool qlive_n = false;
  auto load_tile = [&](int gi, int qt, int buf) {
    const size_t qrow0 = ((size_t)b * P.num_q_heads + hk * G + gi) * S;
    const uint16_t* qb = P.qh + qrow0 * kHeadDim;
    const uint16_t* db = P.dout + qrow0 * kHeadDim;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // a query past the row reads query 0: its position (-1) makes its P and dS zero
      const int i = qt * kQB + dma_row[u];
      const uint32_t voff = (uint32_t)(i < S ? i : 0) * (kHeadDim * 2) + dma_off[u];
      const int slot = 2 * wave + u;  // 1 KB slot of the tile: rows 4 slot .. 4 slot + 3
      lds_dma16(lds_address(&sm[buf].q[64 * slot]), qb, voff);
      lds_dma16(lds_address(&sm[buf].d[64 * slot]), db, voff);
    }
    if (tid < kQB) {
      const int i = qt * kQB + tid;
      qlive_n = i < S;
      const int ic = qlive_n ? i : 0;
      lse_n = P.lse[qrow0 + ic];
      dv_n = P.dvec[qrow0 + ic];
      qp_n = P.pos[(size_t)b * S + ic];
    }
  };
  auto store_tile = [&](int buf) {
    if (tid < kQB) {
      // a position outside the RoPE table reads as 0 (the query's own rows are poisoned)
      sm[buf].lse2[tid] = qlive_n ? lse_n * kLog2e : 0.0f;
      sm[buf].dvec[tid] = qlive_n ? dv_n : 0.0f;
      sm[buf].qpos[tid] = qlive_n ? (qp_n < 0 || qp_n >= P.table_rows ? 0 : qp_n) : -1;
    }
  };

  // query heads of the group in ascending order, each head's visited tiles in ascending order
  // (each tile's greatest query position comes from the window, read when the tile is chosen)
  const int first = __builtin_amdgcn_readfirstlane(next_tile(0));
  if (first < nqt) {
    int gi = 0, qt = first, buf = 0;
    int qmax = __builtin_amdgcn_readfirstlane(tile_qmax(first));
    load_tile(gi, qt, 0);
    store_tile(0);
    wait_vmcnt<0>();
    __syncthreads();
    while (true) {
      int ngi = gi;
      int nq = __builtin_amdgcn_readfirstlane(next_tile(qt + 1));
      if (nq >= nqt) {
        ngi = gi + 1;
        nq = __builtin_amdgcn_readfirstlane(next_tile(first));  // = first, with the window holding it
      }
      const bool more = ngi < G;
      const int qmax_next = __builtin_amdgcn_readfirstlane(tile_qmax(nq < nqt ? nq : wbase));
      if (more) load_tile(ngi, nq, buf ^ 1);
      const DkdvTile& T = sm[buf];
      if (qmax >= kmin) {
        // S = Q^ K^T and dP = dO V^T: [t] queries 16 t + 4 g + i, key r.  The 16 operand
        // reads go out first, so their LDS latency is paid once per tile.
        bf16x8 qa[2][4], da[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            qa[t][kb] = __builtin_bit_cast(bf16x8, T.q[dq_chunk(16 * t + r, 4 * kb + g)]);
            da[t][kb] = __builtin_bit_cast(bf16x8, T.d[dq_chunk(16 * t + r, 4 * kb + g)]);
          }
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
        f32x4 sc[2], dp[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t][kb], kop[kb], sc[t], 0, 0, 0);
            dp[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[t][kb], vop[kb], dp[t], 0, 0, 0);
          }
        }
        // the dV and dK operands (transposed reads, 32 per tile) go out before the softmax
        // arithmetic, which covers their LDS latency; the per-query values come as 16-byte reads
        bf16x8 dto[8], qto[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          // dims 16 nb + jc .. +3: chunk 2 nb + jc / 8, its half jc % 8 / 4
          const int ch = 2 * nb + (jc >> 3);
          const int hb = 2 * (jc & 7);
          const i16x4 d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(reinterpret_cast<const char*>(&T.d[dq_chunk(jr, ch)]) + hb));
          const i16x4 d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(reinterpret_cast<const char*>(&T.d[dq_chunk(16 + jr, ch)]) + hb));
          const i16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(reinterpret_cast<const char*>(&T.q[dq_chunk(jr, ch)]) + hb));
          const i16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(reinterpret_cast<const char*>(&T.q[dq_chunk(16 + jr, ch)]) + hb));
          dto[nb] = __builtin_bit_cast(bf16x8, concat4(d0, d1));
          qto[nb] = __builtin_bit_cast(bf16x8, concat4(q0, q1));
        }
        float4 lse4[2], dv4[2];
        int4 qp4[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          lse4[t] = *reinterpret_cast<const float4*>(&T.lse2[16 * t + 4 * g]);
          dv4[t] = *reinterpret_cast<const float4*>(&T.dvec[16 * t + 4 * g]);
          qp4[t] = *reinterpret_cast<const int4*>(&T.qpos[16 * t + 4 * g]);
        }
        i16x4 pb[2], dsb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float lq[4] = {lse4[t].x, lse4[t].y, lse4[t].z, lse4[t].w};
          const float dq[4] = {dv4[t].x, dv4[t].y, dv4[t].z, dv4[t].w};
          const int pq[4] = {qp4[t].x, qp4[t].y, qp4[t].z, qp4[t].w};
          float p4[4], d4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = kpos <= pq[i] ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][i], kScoreScaleLog2, -lq[i])) : 0.0f;
            p4[i] = p;
            d4[i] = p * (dp[t][i] - dq[i]);
          }
          pb[t] = pack4_bf16(p4[0], p4[1], p4[2], p4[3]);
          dsb[t] = pack4_bf16(d4[0], d4[1], d4[2], d4[3]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the tile's 32 queries: k-slot 8g+e holds query
        // 4g+e (e < 4) and 16+4g+(e-4) (e >= 4) in both operands
        const bf16x8 pk = __builtin_bit_cast(bf16x8, concat4(pb[0], pb[1]));
        const bf16x8 dk8 = __builtin_bit_cast(bf16x8, concat4(dsb[0], dsb[1]));
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          dvv[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dto[nb], pk, dvv[nb], 0, 0, 0);
          dk[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qto[nb], dk8, dk[nb], 0, 0, 0);
        }
      }
      if (more) store_tile(buf ^ 1);
      wait_vmcnt<0>();
      __syncthreads();
      if (!more) break;
      gi = ngi;
      qt = nq;
      qmax = qmax_next;
      buf ^= 1;
    }
  }

  // epilogue: lane (r, g) holds key r of the wavefront, dims 16 nb + 4 g + i
  if (klive) {
    float* dst = P.dv + (krow0 + j) * kHeadDim;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      *reinterpret_cast<float4*>(dst + 16 * nb + 4 * g) = make_float4(dvv[nb][0], dvv[nb][1], dvv[nb][2], dvv[nb][3]);
  }
  // dk through the prologue backward
  f32x4 grad[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) grad[nb] = dk[nb] * kSoftmaxScale;
  float x[8][4];
  float4 wv[8];
  load_acc_layout(P.k + (krow0 + (klive ? j : 0)) * kHeadDim, P.k_norm, g, x, wv, klive);
  float4 c[4], sn[4];
  load_cos_sin_acc(P.rope, klive ? kpos : 0, g, c, sn);
  float dx[8][4], dwt[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) dwt[nb][e] = 0.0f;
  prologue_backward(grad, x, wv, P.k_norm != nullptr, P.eps, c, sn, dx, dwt);
  if (klive) {
    float* dst = P.dk + (krow0 + j) * kHeadDim;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      float4 o = make_float4(dx[nb][0], dx[nb][1], dx[nb][2], dx[nb][3]);
      if (bad) o = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
      *reinterpret_cast<float4*>(dst + 16 * nb + 4 * g) = o;
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dwt[nb][e] = 0.0f;
  }
  if (P.k_norm != nullptr) {
    sum16(dwt);
    if (r == 0) {
      float* part = P.dwk_part + ((size_t)blockIdx.x * 4 + wave) * kHeadDim;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        *reinterpret_cast<float4*>(part + 16 * nb + 4 * g) = make_float4(dwt[nb][0], dwt[nb][1], dwt[nb][2], dwt[nb][3]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// 4. weight gradients: a fixed tree over the shares.  Each workgroup sums 256 consecutive rows
// of in[rows][128]: four groups of 128 threads take 64 rows each in ascending order, and the
// group sums are added in group order; levels repeat until one row is left.
// ---------------------------------------------------------------------------------------
constexpr int kSumRows = 256;  // rows per workgroup and level of the tree
// One level of the two weight-gradient trees (q's, then k's): workgroup c < nq sums rows
// 256 c .. 256 c + 255 of tree q, the others those of tree k.  Column d of a workgroup: four
// groups of 64 consecutive rows, each summed in row order, then the four group sums in order.
struct SumLevel {
  const float* in[2];
  float* out[2];
  int rows[2];
  int chunks0;
};
__global__ __launch_bounds__(512) void bwd_sum_rows_kernel(const SumLevel L) {
  __shared__ float part[4][kHeadDim];
  const int tree = (int)blockIdx.x < L.chunks0 ? 0 : 1;
  const int c = (int)blockIdx.x - (tree == 0 ? 0 : L.chunks0);
  const float* in = L.in[tree];
  const int rows = L.rows[tree];
  const int d = threadIdx.x & (kHeadDim - 1);
  const int grp = threadIdx.x >> 7;
  const int r0 = c * kSumRows + grp * (kSumRows / 4);
  float s = 0.0f;
#pragma unroll
  for (int i0 = 0; i0 < kSumRows / 4; i0 += 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = r0 + i0 + i < rows ? in[(size_t)(r0 + i0 + i) * kHeadDim + d] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = i0 + i == 0 ? v[0] : s + v[i];
  }
  part[grp][d] = s;
  __syncthreads();
  if (grp == 0) L.out[tree][(size_t)c * kHeadDim + d] = ((part[0][d] + part[1][d]) + part[2][d]) + part[3][d];
}

// floats of the intermediate levels of the tree over `rows` rows
size_t sum_scratch_floats(long long rows) {
  size_t n = 0;
  while (rows > 1) {
    rows = (rows + kSumRows - 1) / kSumRows;
    if (rows > 1) n += (size_t)rows * kHeadDim;
  }
  return n;
}

// Both trees level by level, one launch per level (a tree with 0 rows, or already summed,
// takes no workgroups).
void launch_sum_rows(const float* in_q, long long rows_q, float* scratch_q, float* out_q, const float* in_k,
                     long long rows_k, float* scratch_k, float* out_k, hipStream_t stream) {
  const float* in[2] = {in_q, in_k};
  long long rows[2] = {rows_q, rows_k};
  float* scratch[2] = {scratch_q, scratch_k};
  float* out[2] = {out_q, out_k};
  while (rows[0] > 0 || rows[1] > 0) {
    SumLevel L;
    long long chunks[2];
    for (int t = 0; t < 2; ++t) {
      chunks[t] = (rows[t] + kSumRows - 1) / kSumRows;
      L.in[t] = in[t];
      L.rows[t] = (int)rows[t];
      L.out[t] = chunks[t] == 1 ? out[t] : scratch[t];
    }
    L.chunks0 = (int)chunks[0];
    hipLaunchKernelGGL(bwd_sum_rows_kernel, dim3((unsigned)(chunks[0] + chunks[1])), dim3(512), 0, stream, L);
    for (int t = 0; t < 2; ++t) {
      if (chunks[t] == 0) continue;
      if (chunks[t] == 1) {
        rows[t] = 0;  // summed
        continue;
      }
      in[t] = scratch[t];
      scratch[t] += (size_t)chunks[t] * kHeadDim;
      rows[t] = chunks[t];
    }
  }
}

int dq_workgroups(int batch, int seq, int hkv, int group) {
  return ((seq + kQB - 1) / kQB) * batch * hkv * ((group + 3) / 4);
}
int dkdv_workgroups(int batch, int seq, int hkv) { return ((seq + kKBlock - 1) / kKBlock) * batch * hkv; }

// The workspace, in order: q^, k^ (bf16), Dv, the 16-token position bounds, the weight-gradient
// shares of the dq and dkdv workgroups (4 rows of 128 each), and the levels of their sums.
struct BwdLayout {
  size_t qh, kh, dvec, tmin, tmax, dwq_part, dwk_part, dwq_sum, dwk_sum, total;
  long long dwq_rows, dwk_rows;
};

BwdLayout backward_layout(int batch, int seq, int hq, int hkv) {
  BwdLayout L;
  const size_t tok_q = (size_t)batch * hq * seq, tok_k = (size_t)batch * hkv * seq;
  const size_t n16 = (size_t)batch * ((seq + 15) / 16);
  L.dwq_rows = (long long)dq_workgroups(batch, seq, hkv, hq / hkv) * 4;
  L.dwk_rows = (long long)dkdv_workgroups(batch, seq, hkv) * 4;
  size_t o = 0;
  L.qh = o;       o += align256(tok_q * kHeadDim * 2);
  L.kh = o;       o += align256(tok_k * kHeadDim * 2);
  L.dvec = o;     o += align256(tok_q * 4);
  L.tmin = o;     o += align256(n16 * 4);
  L.tmax = o;     o += align256(n16 * 4);
  L.dwq_part = o; o += align256((size_t)L.dwq_rows * kHeadDim * 4);
  L.dwk_part = o; o += align256((size_t)L.dwk_rows * kHeadDim * 4);
  L.dwq_sum = o;  o += align256(sum_scratch_floats(L.dwq_rows) * 4);
  L.dwk_sum = o;  o += align256(sum_scratch_floats(L.dwk_rows) * 4);
  L.total = o;
  return L;
}

}  // namespace

size_t backward_workspace_bytes(int batch, int seq, int hq, int hkv) {
  return backward_layout(batch, seq, hq, hkv).total;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  BwdParams p;
  p.batch = a.batch;
  p.seq = a.seq;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.table_rows = a.table_rows;
  p.pos = a.positions;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.out = (const uint16_t*)a.out;
  p.dout = (const uint16_t*)a.dout;
  p.lse = a.lse;
  p.q_norm = a.q_norm;
  p.k_norm = a.k_norm;
  p.rope = a.rope;
  p.eps = a.eps;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dq_norm = a.q_norm ? a.dq_norm : nullptr;
  p.dk_norm = a.k_norm ? a.dk_norm : nullptr;
  p.dq_wgs = dq_workgroups(a.batch, a.seq, a.num_kv_heads, p.group);
  p.dkdv_wgs = dkdv_workgroups(a.batch, a.seq, a.num_kv_heads);
  const BwdLayout L = backward_layout(a.batch, a.seq, a.num_q_heads, a.num_kv_heads);
  char* ws = (char*)a.workspace;
  p.qh = (uint16_t*)(ws + L.qh);
  p.kh = (uint16_t*)(ws + L.kh);
  p.dvec = (float*)(ws + L.dvec);
  p.tmin = (int*)(ws + L.tmin);
  p.tmax = (int*)(ws + L.tmax);
  p.dwq_part = (float*)(ws + L.dwq_part);
  p.dwk_part = (float*)(ws + L.dwk_part);
  const long long tasks = (long long)a.batch * a.num_kv_heads * ((a.seq + 15) / 16);
  const unsigned prep_blocks = (unsigned)std::min<long long>((tasks + 3) / 4, 8192);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(prep_blocks), dim3(kBwdThreads), 0, stream, p);
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(p.dq_wgs), dim3(kBwdThreads), 0, stream, p);
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(p.dkdv_wgs), dim3(kBwdThreads), 0, stream, p);
  launch_sum_rows(p.dwq_part, p.dq_norm ? L.dwq_rows : 0, (float*)(ws + L.dwq_sum), p.dq_norm, p.dwk_part,
                  p.dk_norm ? L.dwk_rows : 0, (float*)(ws + L.dwk_sum), p.dk_norm, stream);
  return hipGetLastError();
}

}  // namespace pa

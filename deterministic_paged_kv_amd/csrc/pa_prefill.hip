// Chunked paged prefill: Sq trailing queries per row attend causally to the row's cached keys.
//
// Sources: "WS2 PR7 Fused Attention Backend Alignment", sections "Current Implementation"
// (paged prefill wrapper; out [B, Hq, Sq, D], lse [B, Hq, Sq]) and "FlashInfer RoPE Fusion"
// (pre-RoPE Q and K cache, Llama RoPE, trailing contiguous query positions); "[WS2][PR7]
// [Attention] Add FlashInfer RoPE-fused paged attention scaffold", section "Scope" (logical
// K/V order before arithmetic, Split-KV disabled, FP32 LSE, same post-RoPE boundary).
//
// Two kernels per call.
//  1. key_prologue_kernel: every cached key of every KV head of every valid row goes once
//     through the shared Q/K prologue (RMSNorm, RoPE, BF16); k^ is written in logical order
//     to the workspace, [Hkv][nnz * 16][128], key j of row b at (kv_indptr[b] * 16 + j);
//     slots past a row's length are written as zeros.
//  2. attend_kernel: one workgroup per (block of 32 queries, row, KV head, group of up to 4
//     query heads); wavefront w handles one query head of the KV head's GQA group and runs
//     the prologue of its own queries.  Key tiles of 32 (2 pages) are visited in ascending
//     order up to the block's last visible key; the workgroup stages each tile's k^ and V in
//     LDS once for all its heads, with two tiles' loads in flight, and the step is software-
//     pipelined (the scores of the next tile on the matrix cores during this tile's softmax).
//     Long and short items are paired on compute units.  Per tile: S^T = K^ Q^T (bf16 MFMA, FP32 accumulation), causal mask on logical
//     positions (key j visible to a query at position p iff j <= p) on tiles that cross the
//     diagonal, FP32 online softmax with a fixed reduction order, O^T += V^T P^T (P rounded
//     to bf16 for the MFMA, FP32 accumulation).  The softmax reference of a query follows its
//     running maximum lazily (moved only when exceeded by more than 2^8 in probability), which
//     leaves out = sum(p v) / sum(p) and the LSE unchanged up to rounding.
//  The tiling is a constant of the library, so each row's reduction order depends only on
//  the row itself, never on the batch or the plan width.
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kQBlock = 32;          // queries per work item (two 16-row MFMA tiles)
constexpr int kKT = 32;              // keys per tile (2 pages)
constexpr int kRow = kHeadDim + 16;  // LDS row, padded by 32 bytes (conflict-free transposed reads)
// Workgroup shape: H wavefronts per query head, each taking 32 / H of the item's 32 queries
// (H = 1: one wavefront per head with both 16-query tiles; H = 2: two wavefronts per head with
// one tile each).  Every query's arithmetic is the same either way (the bits are identical);
// H = 2 doubles the wavefronts that walk one item's keys, which shortens the longest items.
template <int H>
struct Shape {
  static constexpr int kQT = kQBlock / 16 / H;         // 16-query MFMA tiles per wavefront
  static constexpr int kThreads = 256 * H;             // 4 query heads x H wavefronts
  static constexpr int kTileRows = kThreads / 16;      // tile rows one pass of the threads covers
  static constexpr int kRowsPerThread = 32 / kTileRows;  // key rows of a 32-key tile per thread
};
// A query's softmax reference is moved only when a tile's scaled score exceeds it by more
// than this (log2 domain), so probabilities stay below 2^8 and rescaling is rare.
constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(uint16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ uint4 as_u4(const bf16x8& v) { return __builtin_bit_cast(uint4, v); }

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i16x8 concat4(const i16x4& a, const i16x4& b) {
  return i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four FP32 values rounded to BF16 (nearest-even) and packed in order (two v_cvt_pk_bf16_f32).
__device__ __forceinline__ i16x4 pack_bf16(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){c, d}, bf16x2));
  return __builtin_bit_cast(i16x4, make_uint2(lo, hi));
}

// max of three floats in one v_max3_f32.  The operands are MFMA results or -inf, never
// signalling NaNs, so the operand quieting that fmaxf would add is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// True iff kv_indptr[0..b+1] is non-decreasing.  Rows whose extents lie in such a prefix
// never share an index slot (and so never share k^ workspace rows); a row past a decrease
// could overlap another row's extent and is treated as bad by both kernels.  Every thread of
// the workgroup must call it (it ends with a workgroup-wide AND).
__device__ __forceinline__ bool indptr_prefix_monotone(const int32_t* indptr, int b, int tid, int nthreads) {
  int ok = 1;
  for (int i = tid; i <= b; i += nthreads) ok &= indptr[i] <= indptr[i + 1] ? 1 : 0;
  return __syncthreads_and(ok) != 0;
}

// ---------------------------------------------------------------------------------------
// 1. k^ for every cached key
// ---------------------------------------------------------------------------------------
// Row b = blockIdx.y; its tasks are spread over the x blocks, 4 wavefronts each.  A task is
// one page of the row and HG consecutive KV heads: the wavefront reads the page's RoPE rows once
// and issues the K loads of all HG heads before the first prologue, so the 16 positions' cos/sin
// (512 B each) are fetched once per HG heads.  Only the keys of valid rows are written; nothing
// reads the other slots.
template <int HG>
__global__ __launch_bounds__(256) void key_prologue_kernel(const PrefillParams P, uint16_t* __restrict__ kh) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.y;
  const int p0 = P.indptr[b], p1 = P.indptr[b + 1];
  const int n = p1 - p0;
  const int lpl = P.last_page_len[b];
  const bool mono = indptr_prefix_monotone(P.indptr, b, threadIdx.x, blockDim.x);
  const bool row_ok = mono && p0 >= 0 && n > 0 && p1 <= P.num_indices && n <= P.max_pages_per_row && lpl >= 1 &&
                      lpl <= kPageSize;
  if (!row_ok) return;  // the attention kernel treats such a row as empty or poisoned
  const int L = (n - 1) * kPageSize + lpl;
  const int Hkv = P.num_kv_heads;
  const int groups = Hkv / HG;
  const bool knorm = P.k_norm != nullptr;
  float kw[32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) kw[kb * 8 + e] = knorm ? P.k_norm[32 * kb + 8 * g + e] : 1.0f;
  const uint4 nan4 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  const int tasks = n * groups;
  const int stride = gridDim.x * (blockDim.x >> 6);
  for (int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); t < tasks; t += stride) {
    const int pr = t / groups;
    const int hk0 = (t % groups) * HG;
    const int j = pr * kPageSize + r;  // logical key index = key position
    const bool live = j < L;
    float4 cs[8];
    load_cos_sin(P.rope, live ? j : 0, g, cs);  // depends on the position only: goes out first
    int phys = P.indices[p0 + pr];
    // the key's key_position_ids entry must be its logical index (the rotation uses j); a
    // wrong one, like an out-of-range page, makes the key NaN for every query that sees it
    const int kp = live ? P.kpos[(size_t)(p0 + pr) * kPageSize + r] : j;
    const bool key_ok = phys >= 0 && phys < P.num_pages && kp == j;
    if (phys < 0 || phys >= P.num_pages) phys = 0;
    // the HG heads of slot r are contiguous: HG * 256 bytes
    const size_t src = (((size_t)phys * kPageSize + r) * Hkv + hk0) * kHeadDim + 8 * g;
    uint4 raw[HG][4];
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) raw[h][kb] = live ? ldg16(P.k_cache + src + h * kHeadDim + 32 * kb) : zero4;
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      bf16x8 op[4];
      prologue_operand(raw[h], kw, knorm, P.eps, cs, op);
      uint16_t* dst =
          kh + ((size_t)(hk0 + h) * P.num_indices * kPageSize + (size_t)(p0 + pr) * kPageSize + r) * kHeadDim + 8 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) stg16(dst + 32 * kb, !key_ok ? nan4 : (live ? as_u4(op[kb]) : zero4));
    }
  }
}

template <int HG>
void launch_key_prologue(const PrefillParams& p, uint16_t* kh, hipStream_t stream) {
  // per row: up to max_pages_per_row * Hkv / HG tasks, 4 per block, at most 512 blocks per row
  const long long row_tasks = (long long)std::min(p.max_pages_per_row, p.num_indices) * (p.num_kv_heads / HG);
  const unsigned bx = (unsigned)std::min<long long>((row_tasks + 3) / 4, 512);
  hipLaunchKernelGGL(key_prologue_kernel<HG>, dim3(bx, (unsigned)p.batch), dim3(256), 0, stream, p, kh);
}

// ---------------------------------------------------------------------------------------
// 2. causal attention: q^ made here, k^ from the workspace, V from the pages
// ---------------------------------------------------------------------------------------
struct AttendSmem {
  uint16_t k[3][kKT][kRow];
  uint16_t v[3][kKT][kRow];
};

// Work placement: tiles per unit, and the unit picked.
constexpr int kMaxRankUnits = 512;
struct RankSmem {
  int tiles[kMaxRankUnits];
  int sel;
};

// The tile's share of one thread: k^ and V rows rt + kTileRows u of the tile (rt = tid / 16),
// 16 bytes each at column chunk tid % 16.  Keys past the row's end read the row's last key, so
// every load is in bounds and finite (their scores are masked and their probabilities are 0).
template <int H>
struct TileRegs {
  uint4 k[Shape<H>::kRowsPerThread];
  uint4 v[Shape<H>::kRowsPerThread];
};

template <int H>
__device__ __forceinline__ void store_tile(const TileRegs<H>& tr, AttendSmem& sm, int buf, int tid) {
  constexpr int kTileRows = Shape<H>::kTileRows;
  constexpr int kRowsPerThread = Shape<H>::kRowsPerThread;
  const int rt = tid >> 4;
  const int col = tid & 15;
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    *reinterpret_cast<uint4*>(&sm.k[buf][kTileRows * u + rt][col * 8]) = tr.k[u];
    *reinterpret_cast<uint4*>(&sm.v[buf][kTileRows * u + rt][col * 8]) = tr.v[u];
  }
}

// Units (row b, query block qb) are numbered u = (nqb - 1 - qb) * batch + b.  The key tiles a
// unit visits: its row's keys up to the last query's position (the block's last query stands
// in for the largest position; only the placement of work depends on it).
__device__ int unit_tiles(const PrefillParams& P, int nqb, int u) {
  const int b = u % P.batch;
  const int qb = nqb - 1 - u / P.batch;
  const int p0 = P.indptr[b], p1 = P.indptr[b + 1];
  const int n = p1 - p0;
  const int lpl = P.last_page_len[b];
  const bool bad = p0 < 0 || n < 0 || p1 > P.num_indices || n > P.max_pages_per_row ||
                   (n > 0 && (lpl < 1 || lpl > kPageSize));
  const int L = (n > 0 && !bad) ? (n - 1) * kPageSize + lpl : 0;
  const int i_last = min(qb * kQBlock + kQBlock - 1, P.q_len - 1);
  int qlast = P.qpos[(size_t)b * P.q_len + i_last];
  if (qlast < 0 || qlast >= P.table_rows) qlast = -1;
  const int kend = min(L, qlast + 1);
  return kend > 0 ? (kend + kKT - 1) / kKT : 0;
}

// The unit of rank `target` in the order: more tiles first, then lower unit number.
// All threads of the workgroup call it; U <= kMaxRankUnits.
__device__ int unit_of_rank(const PrefillParams& P, int nqb, int U, int target, int tid, int nthreads,
                            RankSmem& rs) {
  for (int u = tid; u < U; u += nthreads) rs.tiles[u] = unit_tiles(P, nqb, u);
  __syncthreads();
  for (int u = tid; u < U; u += nthreads) {
    const int c = rs.tiles[u];
    int rank = 0;
    for (int v = 0; v < U; ++v) {
      const int cv = rs.tiles[v];
      rank += (cv > c || (cv == c && v < u)) ? 1 : 0;
    }
    if (rank == target) rs.sel = u;
  }
  __syncthreads();
  return rs.sel;
}

template <int H>
__global__ __launch_bounds__(256 * H) __attribute__((amdgpu_waves_per_eu(2 * H, 2 * H))) void attend_kernel(
    const PrefillParams P, const uint16_t* __restrict__ kh) {
  constexpr int kQT = Shape<H>::kQT;
  constexpr int kAttendThreads = Shape<H>::kThreads;
  constexpr int kTileRows = Shape<H>::kTileRows;
  constexpr int kRowsPerThread = Shape<H>::kRowsPerThread;
  __shared__ AttendSmem sm;
  __shared__ RankSmem sched;
  const int G = P.group;
  const int Hkv = P.num_kv_heads;
  const int Sq = P.q_len;
  const int nqb = (Sq + kQBlock - 1) / kQBlock;
  const int nhg = (G + 3) / 4;
  const int tid = threadIdx.x;
  // This workgroup's item: a unit (row b, query block qb) and a head slot (KV head hk, group
  // of query heads hg).  The order only places work; every item's arithmetic is the same
  // wherever it runs.
  const int HH = Hkv * nhg;
  const int U = P.batch * nqb;
  const int N = U * HH;
  int unit, head;
  if (N > P.num_cus && N <= 2 * P.num_cus && U <= kMaxRankUnits) {
    // One dispatch round that puts workgroups i and i + num_cus on the same compute unit:
    // give them the items of ranks k and N-1-k of the longest-first order (ranked by the
    // number of key tiles each unit visits), so every compute unit holds one long and one
    // short item.
    const int rank = (int)blockIdx.x < P.num_cus ? (int)blockIdx.x : N - 1 - ((int)blockIdx.x - P.num_cus);
    unit = unit_of_rank(P, nqb, U, rank / HH, tid, kAttendThreads, sched);
    head = rank % HH;
  } else {
    // Otherwise longest first in launch order: the last query blocks of every row see the
    // most keys.
    unit = (int)blockIdx.x / HH;
    head = (int)blockIdx.x % HH;
  }
  const int qb = nqb - 1 - unit / P.batch;
  const int b = unit % P.batch;
  const int hg = head % nhg;
  const int hk = head / nhg;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2;         // which 32 / H queries of the block (0 when H = 1)
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int gi = hg * 4 + (wave & 3);  // head within the GQA group
  const bool head_live = gi < G;      // trailing waves of a partial group only help stage tiles
  const int h = hk * G + (head_live ? gi : 0);

  const int p0 = P.indptr[b];
  const int p1 = P.indptr[b + 1];
  const int n = p1 - p0;
  const int lpl = P.last_page_len[b];
  const bool mono = indptr_prefix_monotone(P.indptr, b, tid, kAttendThreads);
  const bool bad = !mono || p0 < 0 || n < 0 || p1 > P.num_indices || n > P.max_pages_per_row ||
                   (n > 0 && (lpl < 1 || lpl > kPageSize));
  const int L = (n > 0 && !bad) ? (n - 1) * kPageSize + lpl : 0;

  // positions of the block's queries (-1: past the chunk, sees nothing): every wavefront takes
  // the first and last key positions over all 32 (the tile walk is the block's, the same in
  // every wavefront), then keeps those of its own 16
  int qp_blk[kQBlock / 16];
  int poison = bad;
#pragma unroll
  for (int t = 0; t < kQBlock / 16; ++t) {
    const int i = qb * kQBlock + 16 * t + r;
    qp_blk[t] = i < Sq ? P.qpos[(size_t)b * Sq + i] : -1;
    const int cp = i < Sq ? P.cache_position[(size_t)b * Sq + i] : -1;
    if (i < Sq && (qp_blk[t] < 0 || qp_blk[t] >= P.table_rows || cp != qp_blk[t])) { poison = 1; qp_blk[t] = -1; }
  }
  int qp[kQT];
  int i_of[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    i_of[t] = qb * kQBlock + 16 * (half * kQT + t) + r;
    qp[t] = half == 0 ? qp_blk[t] : qp_blk[kQT + t];
  }
  int qmax = qp_blk[0], qmin = qp_blk[0] < 0 ? INT32_MAX : qp_blk[0];
#pragma unroll
  for (int t = 1; t < kQBlock / 16; ++t) {
    qmax = max(qmax, qp_blk[t]);
    if (qp_blk[t] >= 0) qmin = min(qmin, qp_blk[t]);
  }
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) {
    qmax = max(qmax, __shfl_xor(qmax, sh));
    qmin = min(qmin, __shfl_xor(qmin, sh));
  }
  // identical in every lane after the exchange: make them wave-uniform (scalar)
  qmax = __builtin_amdgcn_readfirstlane(qmax);
  qmin = __builtin_amdgcn_readfirstlane(qmin);
  const int kend = min(L, qmax + 1);
  const int ntiles = kend > 0 ? (kend + kKT - 1) / kKT : 0;
  // tiles ending at or before this key need no mask: every key is < L and <= every query
  const int free_end = min(L, qmin == INT32_MAX ? 0 : qmin + 1);

  // q^ of this wavefront's queries, in the operand layout (vector r = query 16t + r)
  bf16x8 qop[kQT][4];
  {
    const bool qnorm = P.q_norm != nullptr;
    float w[32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[kb * 8 + e] = qnorm ? P.q_norm[32 * kb + 8 * g + e] : 1.0f;
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      uint4 raw[4];
      const bool live = head_live && i_of[t] < Sq;
      const size_t off = (((size_t)b * P.num_q_heads + h) * Sq + (live ? i_of[t] : 0)) * kHeadDim + 8 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) raw[kb] = live ? ldg16(P.q + off + 32 * kb) : make_uint4(0, 0, 0, 0);
      float4 cs[8];
      load_cos_sin(P.rope, max(qp[t], 0), g, cs);
      prologue_operand(raw, w, qnorm, P.eps, cs, qop[t]);
    }
  }

  // Per query: reference m (log2 domain, scaled), m_neg = -m (0 while m is -inf), and this
  // lane's partial sum of p over its own key slots (the four lanes of a query are summed once,
  // in a fixed order, at the end).
  float m_run[kQT], m_neg[kQT], l_part[kQT];
  f32x4 acc[kQT][8];
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
    m_run[t] = -__builtin_inff();
    m_neg[t] = 0.0f;
    l_part[t] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint16_t* kh_row0 = kh + ((size_t)hk * P.num_indices + p0) * kPageSize * kHeadDim;  // key 0 of the row
  const int jr = 4 * g + (r >> 2);  // transposed-read row within a 16-key subtile
  const int jc = 4 * (r & 3);

  // Software pipeline over 32-key tiles: three LDS buffers and a ring of three register sets.
  // At the start of step kt, tiles kt and kt+1 are in LDS (buffers kt % 3 and (kt+1) % 3),
  // S(kt) is in registers and tile kt+2 is in flight or in registers.  Step kt:
  //   A. S(kt+1) = K^(kt+1) Q^T on the matrix cores while the vector unit runs the softmax of
  //      S(kt) with the current references (straight-line code); a rare fix-up follows when
  //      some query's reference has to move.
  //   B. the loads of tile kt+3 are issued, O^T += V(kt)^T P(kt)^T, tile kt+2 goes to LDS
  //      buffer (kt+2) % 3 (free since the barrier that ended step kt-1), barrier.
  // Tiles past the block's last one are loaded, stored and multiplied all the same (keys and
  // pages clamped to the row's last key, so every access is in bounds and finite); their
  // results are never used.  Page numbers come through vector loads (one per tile, lane u
  // holding the page of the tile's half u), so no scalar load shares a counter with the LDS
  // reads.
  constexpr int kRing = 3;
  TileRegs<H> ring[kRing];
  const int32_t* row_idx = P.indices + p0;
  const size_t page_elems = (size_t)kPageSize * Hkv * kHeadDim;
  const int rt = tid >> 4;
  const int col = tid & 15;
  const uint32_t v_lane_off = (uint32_t)hk * kHeadDim + col * 8;
  static_assert(kTileRows % 16 == 0 || kRowsPerThread * kTileRows == 32, "tile rows must split into pages");
  // page numbers of tile t (lane u: page min(2t + u, n - 1)); only called with n >= 1
  auto page_vec = [&](int t) -> int { return row_idx[min(2 * t + (lane & 1), n - 1)]; };
  auto load = [&](TileRegs<H>& tr, int t, int pv) {
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int ro = kTileRows * u + rt;  // row of the tile; its page is the tile's half ro / 16
      int phys = __builtin_amdgcn_readlane(pv, __builtin_amdgcn_readfirstlane(ro >> 4));
      // only the block's own tiles count: the ring also loads up to three tiles past the
      // last one, whose results are thrown away
      if (phys < 0 || phys >= P.num_pages) { poison |= t < ntiles ? 1 : 0; phys = 0; }
      const int j = min(t * kKT + ro, L - 1);  // logical key (clamped)
      tr.k[u] = ldg16(kh_row0 + (uint32_t)j * kHeadDim + col * 8);
      tr.v[u] = ldg16(P.v_cache + (size_t)phys * page_elems + ((uint32_t)(j & (kPageSize - 1)) * Hkv * kHeadDim + v_lane_off));
    }
  };
  // S^T = K^ Q^T for the two 16-key subtiles of the tile in LDS buffer `buf`
  auto scores = [&](int buf, f32x4 (&out)[kQT][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 ka[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        ka[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sm.k[buf][16 * ks + r][32 * kb + 8 * g]));
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        out[t][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          out[t][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qop[t][kb], out[t][ks], 0, 0, 0);
      }
    }
  };
  // last key position + 1 each query may see (0: none)
  int lim[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) lim[t] = min(L, qp[t] + 1);

  int pv_next = 0;
  if (ntiles > 0) {
    const int pv0 = page_vec(0), pv1 = page_vec(1), pv2 = page_vec(2);
    load(ring[0], 0, pv0);
    load(ring[1], 1, pv1);
    load(ring[2], 2, pv2);
    pv_next = page_vec(3);
    store_tile<H>(ring[0], sm, 0, tid);
    store_tile<H>(ring[1], sm, 1, tid);
  }
  __syncthreads();
  f32x4 sc[kQT][2];
  if (ntiles > 0) scores(0, sc);

  // p = 2^(s c - m) of a query's 8 scores in this lane, their sum (in key order) and BF16 copy
  auto tile_p = [&](const f32x4 (&s_)[2], float mneg, float& sum, i16x4 (&pbt)[2]) {
    float p[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[ks][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_[ks][i], kScoreScaleLog2, mneg));
    sum = p[0][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) sum += p[e >> 2][e & 3];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pbt[ks] = pack_bf16(p[ks][0], p[ks][1], p[ks][2], p[ks][3]);
  };
  auto step = [&](const int kt, TileRegs<H>& to_load, TileRegs<H>& to_store) {
    // ---- A: causal mask (tiles that reach past the block's first query), then S(kt+1) and
    // the softmax of S(kt)
    if ((kt + 1) * kKT > free_end) {
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        const int d = lim[t] - kt * kKT - 4 * g;  // key 16 ks + 4 g + i is visible iff 16 ks + i < d
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[t][ks][i] = 16 * ks + i < d ? sc[t][ks][i] : -__builtin_inff();
      }
    }
    f32x4 sn[kQT][2];
    scores((kt + 1) % 3, sn);
    float mx[kQT], lp[kQT];
    i16x4 pb[kQT][2];
    bool need = false;
#pragma unroll
    for (int t = 0; t < kQT; ++t) {
      // raw-score maximum of this lane's keys (the scale c > 0 commutes with max)
      mx[t] = max3f(max3f(max3f(sc[t][0][0], sc[t][0][1], sc[t][0][2]), max3f(sc[t][0][3], sc[t][1][0], sc[t][1][1]),
                          sc[t][1][2]),
                    sc[t][1][3], sc[t][1][3]);
      need |= mx[t] * kScoreScaleLog2 > m_run[t] + kLazyMax;
      // p = 2^(s c - m) with the current reference (0 for masked keys, and while m is -inf)
      tile_p(sc[t], m_neg[t], lp[t], pb[t]);
    }
    // Fix-up, rare: a query whose tile maximum exceeds its reference by more than kLazyMax
    // (the test is exact per query: a lane's keys are a subset of the query's) moves its
    // reference to the tile's scaled maximum, rescales what it has summed so far, and
    // recomputes the tile's p.
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int t = 0; t < kQT; ++t) {
        const float rowmax = pair32_max(pair16_max(mx[t])) * kScoreScaleLog2;
        if (rowmax > m_run[t] + kLazyMax) {
          const float alpha = m_run[t] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run[t] - rowmax);
          m_run[t] = rowmax;
          m_neg[t] = -rowmax;
          l_part[t] *= alpha;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) acc[t][nb] = acc[t][nb] * alpha;
          tile_p(sc[t], m_neg[t], lp[t], pb[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kQT; ++t) l_part[t] += lp[t];
    // ---- B: loads of tile kt+3, P.V of tile kt, tile kt+2 to LDS
    const int pv = pv_next;
    pv_next = page_vec(kt + 4);
    load(to_load, kt + 3, pv);
    // O^T += V^T P^T over the tile's 32 keys in one K=32 MFMA per (query tile, column block):
    // k-slot 8g+e holds key 4g+e for e < 4 and key 16+4g+(e-4) for e >= 4, in both operands.
    // V^T comes from two transposed LDS reads (one per 16-key subtile).
    const int buf = kt % 3;
    bf16x8 pk[kQT];
#pragma unroll
    for (int t = 0; t < kQT; ++t) pk[t] = __builtin_bit_cast(bf16x8, concat4(pb[t][0], pb[t][1]));
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sm.v[buf][jr][16 * nb + jc]));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sm.v[buf][16 + jr][16 * nb + jc]));
      const bf16x8 va = __builtin_bit_cast(bf16x8, concat4(v0, v1));
#pragma unroll
      for (int t = 0; t < kQT; ++t)
        acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk[t], acc[t][nb], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kQT; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) sc[t][ks] = sn[t][ks];
    store_tile<H>(to_store, sm, (kt + 2) % 3, tid);
    __syncthreads();
  };
  // whole rounds of the ring, then the last one or two tiles (no exit from inside a round)
  int kt = 0;
  for (; kt + kRing <= ntiles; kt += kRing) {
    step(kt, ring[0], ring[2]);
    step(kt + 1, ring[1], ring[0]);
    step(kt + 2, ring[2], ring[1]);
  }
  if (kt < ntiles) step(kt, ring[0], ring[2]);
  if (kt + 1 < ntiles) step(kt + 1, ring[1], ring[0]);

  // any out-of-range page index seen by any thread poisons the whole block's output
  const bool out_poison = __syncthreads_or(poison) != 0;
  float l_run[kQT];
#pragma unroll
  for (int t = 0; t < kQT; ++t) l_run[t] = pair32_sum(pair16_sum(l_part[t]));
#pragma unroll
  for (int t = 0; t < kQT; ++t) {
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
      for (int e = 0; e < 4; ++e) o[e] = out_poison ? __builtin_nanf("") : acc[t][nb][e] * inv;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16);
      *reinterpret_cast<uint2*>(P.out + row * kHeadDim + 16 * nb + 4 * g) = w;
    }
    if (g == 0) {
      float lse = empty ? -__builtin_inff() : (m_run[t] + __builtin_log2f(l_run[t])) * kLn2;
      if (out_poison) lse = __builtin_nanf("");
      P.lse[row] = lse;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  uint16_t* kh = (uint16_t*)p.workspace;
  if (p.num_indices > 0) {
    // two KV heads per wavefront: half the cos/sin reads, still about two wavefronts per SIMD
    // (four heads per wavefront leave too few wavefronts to hide the load latency)
    if (p.num_kv_heads % 2 == 0) launch_key_prologue<2>(p, kh, stream);
    else launch_key_prologue<1>(p, kh, stream);
  }
  const unsigned nqb = (unsigned)((p.q_len + kQBlock - 1) / kQBlock);
  const unsigned nhg = (unsigned)((p.group + 3) / 4);
  const unsigned grid = nqb * (unsigned)p.batch * (unsigned)p.num_kv_heads * nhg;
  if (grid > 0) {
    // Two wavefronts per query head when the items fit one dispatch round (the longest-first
    // pairing on compute units is in use and the longest items decide the time); one otherwise.
    const unsigned U = nqb * (unsigned)p.batch;
    if (grid > (unsigned)p.num_cus && grid <= 2u * (unsigned)p.num_cus && U <= (unsigned)kMaxRankUnits)
      hipLaunchKernelGGL(attend_kernel<2>, dim3(grid), dim3(Shape<2>::kThreads), 0, stream, p, kh);
    else
      hipLaunchKernelGGL(attend_kernel<1>, dim3(grid), dim3(Shape<1>::kThreads), 0, stream, p, kh);
  }
  return hipGetLastError();
}

}  // namespace pa

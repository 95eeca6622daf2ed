// Chunked paged prefill: Sq trailing queries per row attend causally to the row's cached keys.
//
// Sources: "WS2 PR7 Fused Attention Backend Alignment", sections "Current Implementation"
// (paged prefill wrapper; out [B, Hq, Sq, D], lse [B, Hq, Sq]) and "FlashInfer RoPE Fusion"
// (pre-RoPE Q and K cache, Llama RoPE, trailing contiguous query positions); "[WS2][PR7]
// [Attention] Add FlashInfer RoPE-fused paged attention scaffold", section "Scope" (logical
// K/V order before arithmetic, Split-KV disabled, FP32 LSE, same post-RoPE boundary).
//
// Two kernels per call.
//  1. prologue_kernel: every cached key of every KV head of every valid row, and every query
//     vector, goes once through the shared Q/K prologue (RMSNorm, RoPE, BF16); k^ is written
//     to the workspace in logical order, key j of row b at index slot kv_indptr[b] + j / 16
//     (slots past a row's length are zeros), q^ as [B][Hq][Sq][128]; the work units' records
//     are written in the attention kernel's order, longest first.
//  2. attend_kernel: one workgroup per (block of 32 queries, row, KV head, group of up to 4
//     query heads); each wavefront holds 16 queries of two query heads of the KV head's GQA
//     group.  Key tiles of 32 (2 pages) are split
//     into two fixed streams (even and odd tiles) walked in ascending order up to the block's
//     last visible key and merged at the end in stream order; the workgroup stages each tile's
//     k^ and V in LDS once for all its heads, with loads two to three steps ahead, and each
//     step overlaps the scores of the next tile and P.V of the previous one with the softmax
//     of the current one.  Long items are placed first.  Per tile: S^T = K^ Q^T (bf16 MFMA,
//     FP32 accumulation), causal mask on logical positions (key j visible to a query at
//     position p iff j <= p) on tiles that cross the diagonal, FP32 online softmax with a
//     fixed reduction order, O^T += V^T P^T (P rounded to bf16 for the MFMA, FP32
//     accumulation).  The softmax reference of a query follows its running maximum lazily
//     (moved only when exceeded by more than 2^8 in probability), which leaves
//     out = sum(p v) / sum(p) and the LSE unchanged up to rounding.
//  The tiling is a constant of the library, so each row's reduction order depends only on
//  the row itself, never on the batch or the plan width.
#include <type_traits>

#include "pa_internal.h"
#include "pa_lds_dma.h"

namespace pa {

namespace {

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
// Work items and tiles of the attention kernel
// ---------------------------------------------------------------------------------------
// Work item: (row b, KV head hk, group hg of up to 4 query heads of hk's GQA group, block of
// 32 queries).  Eight wavefronts, two per SIMD.  Wavefront w holds 32 query rows: the 16
// queries 16 qg .. 16 qg + 15 of the block (qg = (w >> 1) & 1) of the two head slots
// 2 hp, 2 hp + 1 (hp = w >> 2), the GQA group packed into the matrix N dimension, and walks
// key stream st = w & 1 of the item: stream 0 takes the 32-key tiles 0, 2, 4, ..., stream 1
// the tiles 1, 3, 5, ...  Each stream is an FP32 online softmax over its tiles in ascending
// order; at the end the two streams of each query row are merged in the order stream 0,
// stream 1.  The split depends only on the row (its tile count), never on the batch or the
// plan.
//
// Per tile and wavefront (v_mfma_f32_32x32x16_bf16; lane l holds MFMA column n = l % 32 and
// half hh = l / 32):
//   S^T [32 keys x 32 query rows] = K^ Q^T     8 MFMAs (8 dim steps)
//   softmax on S^T                              lane (n, hh) holds 16 keys of query row n
//   O^T [128 dims x 32 rows] += V^T P^T          8 MFMAs (4 dim blocks x 2 key steps)
// Column n is query 16 qg + n % 16 of head slot 2 hp + n / 16.  S^T register i of lane
// (n, hh) is key 8 (i / 4) + 4 hh + i % 4 of the tile; rounded to BF16 those registers are
// directly the B operand of the P.V MFMA, with V^T's k-slots read from LDS in the same key
// order (two transposed 4-key reads per operand).
//
// The walk is software-pipelined in every wavefront: between two workgroup barriers (step t)
// a wavefront computes S of tile t + 1 and adds P.V of tile t - 1 on the matrix cores while
// its vector units run the softmax of tile t; the three do not depend on one another, so the
// matrix cores and the vector units overlap.  hp only picks which loads the wavefront issues
// (hp = 0: k^ tiles, three steps ahead; hp = 1: V pages, two steps ahead).
constexpr int kQB = kPrefillQB;      // queries per work item
constexpr int kKT = 32;              // keys per tile (2 pages)
constexpr int kStreams = 2;          // key streams per item
constexpr int kBufs = 4;             // LDS tile buffers per stream
constexpr int kAttendThreads = 512;
// A query row's softmax reference moves only when a tile's probabilities, taken against the
// current reference, sum past 2^kLazyMax in one lane (or the reference is still unset): the
// fix-up then moves it to the row maximum if that exceeds it by more than kLazyMax (log2
// domain), so every probability stays below 2^kLazyMax and rescaling is rare.
constexpr float kLazyMax = 8.0f;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One tile of one stream in LDS (64 banks of 4 bytes).
//   k^: 32 rows (keys) of 256 bytes; the 16-byte chunk j of row r holds dims 8 (j ^ (r % 16))
//       .. +7.  The S operands are 16-byte reads, 16 lanes per LDS cycle: 16 consecutive keys
//       at the same logical chunk, which the swizzle spreads over all 16 physical chunks.
//   V:  32 rows (keys) of 256 bytes; the 64-byte block j of row r holds dims 32 (j ^ (r % 4))
//       .. +31.  The P.V operands are transposed 8-byte reads, 32 lanes per LDS cycle: 64
//       bytes of four consecutive rows at the same logical block, which the swizzle spreads
//       over the four physical blocks.
// Both layouts were checked free of bank conflicts with the LDS bank-conflict counter.
struct alignas(16) TileBuf {
  uint16_t k[kKT][kHeadDim];
  uint16_t v[kKT][kHeadDim];
};

// The row's physical page numbers, for rows of up to kPageTable pages: the V loads look their
// pages up here instead of with scalar loads, which share a wait counter with the LDS reads
// and return out of order (a wait for one would drain every LDS read in flight).
constexpr int kPageTable = 2048;
// The output rows of one wavefront (32 rows of 128 BF16), padded to 264 bytes so that the
// staging writes (lane = row, 8 bytes) spread over all banks.
constexpr int kOutPitch = kHeadDim + 4;
struct alignas(16) AttendSmem {
  union {
    TileBuf tiles[kStreams][kBufs];            // the walk (128 KB)
    struct {
      float merge[4][2][2 + 32][64];           // per pair and stream: what it hands the other
      uint16_t out[4][32][kOutPitch];          // the pair's output rows, staged for row-wise stores
    } m;
  } u;
  int32_t pt[kPageTable];                      // 8 KB
};

// Work placement: the tiles every unit visits, for ranking the units.
constexpr int kMaxRankUnits = 512;
struct RankSmem {
  int tiles[kMaxRankUnits];
};

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
  const int i_last = min(qb * kQB + kQB - 1, P.q_len - 1);
  int qlast = P.qpos[(size_t)b * P.q_len + i_last];
  if (qlast < 0 || qlast >= P.table_rows) qlast = -1;
  const int kend = min(L, qlast + 1);
  return kend > 0 ? (kend + kKT - 1) / kKT : 0;
}

// ---------------------------------------------------------------------------------------
// 1. the prologue: k^ of every cached key, q^ of every query, the work units' records
// ---------------------------------------------------------------------------------------
// One launch of 256-thread workgroups of three kinds:
//   [0, B * kx)        k^: row b = id / kx; its tasks are spread over its kx workgroups, 4
//                      wavefronts each.  A task is one page of the row and HG consecutive KV
//                      heads: the wavefront reads the page's RoPE rows once and issues the K
//                      loads of all HG heads before the first prologue, so the 16 positions'
//                      cos/sin (512 B each) are fetched once per HG heads.  Only the keys of
//                      valid rows are written; nothing reads the other slots.
//   [B * kx, + nq)     q^: 16 query vectors per wavefront, (b, head, i) in [B][Hq][Sq] order,
//                      written in that order, [B][Hq][Sq][128] bf16.
//   the rest           the work units' records, 8 units per workgroup, each stored at its rank
//                      (the attention kernel's order, longest first).
//
// k^ layout: per KV head, key j of row b at row (kv_indptr[b] * 16 + j) of [nnz * 16][128]
// bf16 (the key's 128 dims contiguous), so a 32-key tile is 8 KB of contiguous workspace.
constexpr int kPrologueThreads = 256;
union PrologueSmem {
  RankSmem rank;
};

template <int HG>
__device__ void key_part(const PrefillParams& P, uint16_t* __restrict__ kh, int b, int xb, int kx) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
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
  const int stride = kx * (blockDim.x >> 6);
  for (int t = xb * (blockDim.x >> 6) + (threadIdx.x >> 6); t < tasks; t += stride) {
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
      uint16_t* row = kh + (((size_t)(hk0 + h) * P.num_indices + (size_t)(p0 + pr)) * kPageSize + r) * kHeadDim;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) stg16(row + 32 * kb + 8 * g, !key_ok ? nan4 : (live ? as_u4(op[kb]) : zero4));
    }
  }
}

// 16 consecutive queries of one row and kQH consecutive query heads per wavefront (lane r +
// 16 g: query i0 + r, dims 32 kb + 8 g .. +7): the queries' cos/sin are loaded once for the
// kQH heads, and all the wavefront's loads go out before the first prologue.  (Measured on
// the chunked-prefill workload: 2 heads per wavefront beat 1 and 4.)
constexpr int kQH = 2;
__device__ void query_part(const PrefillParams& P, uint16_t* __restrict__ qh, int qblk) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nqi = (P.q_len + 15) / 16;
  const int nhq = (P.num_q_heads + kQH - 1) / kQH;
  const int task = qblk * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (task >= P.batch * nhq * nqi) return;
  const int iq = task % nqi;
  const int h0 = (task / nqi % nhq) * kQH;
  const int b = task / (nqi * nhq);
  const int i = 16 * iq + r;
  const bool live_q = i < P.q_len;
  int qp = live_q ? P.qpos[(size_t)b * P.q_len + i] : 0;
  if (qp < 0 || qp >= P.table_rows) qp = 0;  // the attention kernel poisons such a query's rows
  float4 cs[8];
  load_cos_sin(P.rope, qp, g, cs);
  uint4 raw[kQH][4];
#pragma unroll
  for (int h = 0; h < kQH; ++h) {
    const bool live = live_q && h0 + h < P.num_q_heads;
    const size_t v = ((size_t)b * P.num_q_heads + (live ? h0 + h : 0)) * P.q_len + (live ? i : 0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) raw[h][kb] = ldg16(P.q + v * kHeadDim + 32 * kb + 8 * g);
  }
  const bool qnorm = P.q_norm != nullptr;
  float wq[32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) wq[kb * 8 + e] = qnorm ? P.q_norm[32 * kb + 8 * g + e] : 1.0f;
#pragma unroll
  for (int h = 0; h < kQH; ++h) {
    if (h0 + h >= P.num_q_heads) break;  // uniform over the wavefront
    bf16x8 op[4];
    prologue_operand(raw[h], wq, qnorm, P.eps, cs, op);
    if (live_q) {
      const size_t v = ((size_t)b * P.num_q_heads + h0 + h) * P.q_len + i;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) stg16(qh + v * kHeadDim + 32 * kb + 8 * g, as_u4(op[kb]));
    }
  }
}

// The record of work unit u (row b = u % B, query block qb = nqb - 1 - u / B): one half-
// wavefront per unit, lane i for query qb * kQB + i.  Fields (int32):
//   0 p0        kv_indptr[b]
//   1 nidx      pages of the row
//   2 lpl       kv_last_page_len[b]
//   3 L         keys of the row (0 if the row is empty or bad)
//   4 ntiles    32-key tiles up to the block's last visible key
//   5 free_end  tiles ending at or before this key need no causal mask
//   6 poison    1 if the row is bad (extent out of range, or past a decrease of kv_indptr) or a
//               query of the block has a position out of the RoPE table or a cache_position
//               that differs from it: every output of the unit is then NaN
// A bad row's or query's position counts as -1 (sees nothing) in ntiles and free_end.
//   7 unit      the unit's number u (records are stored by rank, see below)
enum { kUnitP0 = 0, kUnitNidx, kUnitLpl, kUnitL, kUnitTiles, kUnitFreeEnd, kUnitPoison, kUnitId, kUnitPage0 = 8 };
// the record also holds the physical numbers of the row's pages 0 .. kUnitPages - 1 (clamped to
// the last page; 0 for an empty or bad row): the V loads issued before the walk take them from
// there instead of from the page table, one memory latency earlier
constexpr int kUnitPages = 12;
static_assert(kUnitPage0 + kUnitPages <= kUnitInts, "unit record size");
// The records are stored in the attention kernel's order: by rank, more tiles first, then
// lower unit number (units past kMaxRankUnits go in number order).  Every workgroup of this
// kind ranks its own units against all of them, so no other workgroup has to finish first.
// All threads of the workgroup call it.
__device__ void unit_part(const PrefillParams& P, int32_t* __restrict__ units, int ublk, RankSmem& rs) {
  const int lane = threadIdx.x & 63;
  const int i32 = lane & 31;
  const int nqb = (P.q_len + kQB - 1) / kQB;
  const int U = P.batch * nqb;
  const int u = (ublk * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool live_unit = u < U;
  const bool ranked = U <= kMaxRankUnits;
  if (ranked) {
    for (int v = threadIdx.x; v < U; v += blockDim.x) rs.tiles[v] = unit_tiles(P, nqb, v);
  }
  __syncthreads();
  int slot = u;
  if (ranked) {
    const int c = rs.tiles[live_unit ? u : 0];
    int before = 0;
    for (int v = i32; v < U; v += 32) {
      const int cv = rs.tiles[v];
      before += (cv > c || (cv == c && v < u)) ? 1 : 0;
    }
#pragma unroll
    for (int sh = 1; sh < 32; sh <<= 1) before += __shfl_xor(before, sh);
    slot = before;
  }
  const int uu = live_unit ? u : 0;
  const int b = uu % P.batch;
  const int qb = nqb - 1 - uu / P.batch;
  const int p0 = P.indptr[b], p1 = P.indptr[b + 1];
  const int nidx = p1 - p0;
  const int lpl = P.last_page_len[b];
  // kv_indptr[0..b+1] non-decreasing (rows in such a prefix never share index slots)
  int ok = 1;
  for (int i = i32; i <= b; i += 32) ok &= P.indptr[i] <= P.indptr[i + 1] ? 1 : 0;
  const uint64_t okm = __builtin_amdgcn_ballot_w64(ok != 0);
  const uint32_t half = (uint32_t)(okm >> (lane & 32));
  const bool mono = half == 0xFFFFFFFFu;
  const bool bad = !mono || p0 < 0 || nidx < 0 || p1 > P.num_indices || nidx > P.max_pages_per_row ||
                   (nidx > 0 && (lpl < 1 || lpl > kPageSize));
  const int L = (nidx > 0 && !bad) ? (nidx - 1) * kPageSize + lpl : 0;
  const int i = qb * kQB + i32;
  int qp = i < P.q_len ? P.qpos[(size_t)b * P.q_len + i] : -1;
  const int cp = i < P.q_len ? P.cache_position[(size_t)b * P.q_len + i] : -1;
  const bool qbad = i < P.q_len && (qp < 0 || qp >= P.table_rows || cp != qp);
  if (qbad) qp = -1;
  int qmax = qp, qmin = qp < 0 ? INT32_MAX : qp;
#pragma unroll
  for (int sh = 1; sh < 32; sh <<= 1) {
    qmax = max(qmax, __shfl_xor(qmax, sh));
    qmin = min(qmin, __shfl_xor(qmin, sh));
  }
  const bool any_qbad = (uint32_t)(__builtin_amdgcn_ballot_w64(qbad) >> (lane & 32)) != 0u;
  const int kend = min(L, qmax + 1);
  const int rec[8] = {p0, nidx, lpl, L, kend > 0 ? (kend + kKT - 1) / kKT : 0,
                      min(L, qmin == INT32_MAX ? 0 : qmin + 1), (bad || any_qbad) ? 1 : 0, u};
  if (live_unit && i32 < 8) {
    int v = rec[0];
#pragma unroll
    for (int f = 1; f < 8; ++f) v = i32 == f ? rec[f] : v;
    units[(size_t)slot * kUnitInts + i32] = v;
  }
  if (live_unit && i32 >= kUnitPage0 && i32 < kUnitPage0 + kUnitPages) {
    const int k = i32 - kUnitPage0;
    units[(size_t)slot * kUnitInts + i32] = (!bad && nidx > 0) ? P.indices[p0 + min(k, nidx - 1)] : 0;
  }
}

template <int HG>
__global__ __launch_bounds__(kPrologueThreads) void prologue_kernel(const PrefillParams P, uint16_t* __restrict__ kh,
                                                                    uint16_t* __restrict__ qh,
                                                                    int32_t* __restrict__ units, int kx, int nq) {
  __shared__ PrologueSmem sm;
  const int blk = (int)blockIdx.x;
  const int nk = P.batch * kx;
  if (blk < nk) {
    key_part<HG>(P, kh, blk / kx, blk % kx, kx);
  } else if (blk < nk + nq) {
    query_part(P, qh, blk - nk);
  } else {
    unit_part(P, units, blk - nk - nq, sm.rank);
  }
}

// ---------------------------------------------------------------------------------------
// 2. causal attention: q^ and k^ from the workspace, V from the pages
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kAttendThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_kernel(
    const PrefillParams P, const uint16_t* __restrict__ kh, const uint16_t* __restrict__ qh,
    const int32_t* __restrict__ units) {
  __shared__ AttendSmem sm;
  const int G = P.group;
  const int Hkv = P.num_kv_heads;
  const int Sq = P.q_len;
  const int nqb = (Sq + kQB - 1) / kQB;
  const int nhg = (G + 3) / 4;
  const int tid = threadIdx.x;
  // This workgroup's item: a unit (row b, query block qb) and a head slot (KV head hk, group
  // hg of query heads).  Consecutive workgroups take consecutive head slots of the same rank,
  // so the dispatch's round robin over the XCDs keeps each head slot's k^ and V in few L2s;
  // ranks go longest first.  The order only places work; every item's arithmetic is the same
  // wherever it runs.
  const int HH = Hkv * nhg;
  const int rank = (int)blockIdx.x / HH;
  const int head = (int)blockIdx.x % HH;
  // the unit's record, stored at its rank by the prologue kernel
  const int32_t* rec = units + (size_t)rank * kUnitInts;
  const int unit = load_uniform(rec, kUnitId);
  const int qb = nqb - 1 - unit / P.batch;
  const int b = unit % P.batch;
  const int hg = head % nhg;
  const int hk = head / nhg;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int st = w & 1;         // key stream
  const int qg = (w >> 1) & 1;  // query group: queries 16 qg .. 16 qg + 15 of the block
  const int hp = w >> 2;        // head pair: slots 2 hp, 2 hp + 1; also the step phase
  const int role = 2 * hp + qg; // which part of the stream's tile loads this wavefront issues
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hh = lane >> 5;

  // the unit's record (written by the prologue kernel) and this lane's query (column n: query
  // 16 qg + n % 16) with the last key it may see + 1; a query whose position is out of range
  // sees nothing (the unit is then poisoned anyway)
  const int p0 = load_uniform(rec, kUnitP0);
  const int nidx = load_uniform(rec, kUnitNidx);
  const int lpl = load_uniform(rec, kUnitLpl);
  const int L = load_uniform(rec, kUnitL);
  const int ntiles = load_uniform(rec, kUnitTiles);
  const int free_end = load_uniform(rec, kUnitFreeEnd);
  int poison = load_uniform(rec, kUnitPoison);
  const int nsteps = (ntiles + kStreams - 1) / kStreams;
  // the row's page numbers, loaded now and written to the LDS page table before the walk
  const bool use_pt = nidx <= kPageTable;
  constexpr int kPtPerThread = kPageTable / kAttendThreads;
  int32_t ptv[kPtPerThread];
#pragma unroll
  for (int j = 0; j < kPtPerThread; ++j) {
    const int i = tid + kAttendThreads * j;
    ptv[j] = use_pt && i < nidx ? P.indices[p0 + i] : 0;
  }
  const int qi = qb * kQB + 16 * qg + (n & 15);
  int qp = qi < Sq ? P.qpos[(size_t)b * Sq + qi] : -1;
  if (qp < 0 || qp >= P.table_rows) qp = -1;
  const int lim = min(L, qp + 1);

  // ---- q^ of the wavefront's 32 query rows, in the B-operand layout of the S MFMAs: lane
  // (n, hh) holds row n (head slot 2 hp + n / 16, query 16 qg + n % 16), dims 16 s + 8 hh .. +7
  // for s = 0..7.  A row past the chunk or the group takes the q^ of query 0 of the group's
  // first head: its column computes on valid data and is never stored (columns are
  // independent).  The loads are unconditional and nothing selects on them, so they stay in
  // flight until the single wait before the walk.
  bf16x8 qop[8];
  {
    const int gi = hg * 4 + 2 * hp + (n >> 4);
    const bool live = gi < G && qi < Sq;
    const uint16_t* src =
        qh + (((size_t)b * P.num_q_heads + hk * G + (live ? gi : 0)) * Sq + (live ? qi : 0)) * kHeadDim + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qop[s] = __builtin_bit_cast(bf16x8, ldg16(src + 16 * s));
  }

  // ---- the walk
  float m_run = -__builtin_inff(), m_neg = 0.0f, l_part = 0.0f;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  TileBuf(&tb)[kBufs] = sm.u.tiles[st];
  // Direct-to-LDS loads of the stream's tiles, four instructions per wavefront and step.  One
  // instruction writes 1 KB of contiguous LDS, lane l the 16 bytes at 16 l, each lane from its
  // own global address.
  //   k^ (roles 0 and 1, keys 16 qg .. 16 qg + 15 of the tile): instruction i writes keys
  //      16 qg + 4 i .. +3, lane l physical chunk l % 16 of key 16 qg + 4 i + l / 16, which
  //      holds logical chunk (l % 16) ^ (key % 16) (the swizzle above).  A row's last tile may
  //      reach past the row: those keys are masked, and the workspace is padded so the copy
  //      stays in bounds.
  //   V (roles 2 and 3, page 2 kt + qg = rows 16 qg .. 16 qg + 15 of the tile): instruction i
  //      writes rows 4 i .. 4 i + 3 of the page, lane l physical chunk l % 16 of row 4 i + l / 16,
  //      which holds logical chunk 4 ((l % 16) / 4 ^ row % 4) + l % 4 of the row (the swizzle
  //      above).  Slots past the row's end read its last key, so every value read is finite
  //      (their probabilities are 0).
  const char* kh_plane = (const char*)(kh + ((size_t)hk * P.num_indices + p0) * kPageSize * kHeadDim);
  const uint32_t v_row_bytes = (uint32_t)Hkv * kHeadDim * 2u;
  const uint32_t v_page_bytes = v_row_bytes * kPageSize;
  const char* v_head = (const char*)(P.v_cache + (size_t)hk * kHeadDim);  // the KV head's slice of page 0
  // k^: doff = byte offset of the key's logical chunk in the tile; V: doff = byte offset of
  // the slot's row in the page, dch = of the logical chunk in the row
  uint32_t doff[4], dch[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);  // 0..15
    const int pch = lane & 15;
    const int key = 16 * qg + row;
    const int lch = 4 * ((pch >> 2) ^ (row & 3)) + (pch & 3);
    doff[i] = role < 2 ? (uint32_t)key * 256u + 16u * (pch ^ (key & 15)) : (uint32_t)row * v_row_bytes;
    dch[i] = 16u * lch;
  }
  // The walk is written once per phase (HP = hp: 0 loads k^ and computes S at the start of a
  // step, 1 loads V and computes S at its end), so neither path branches on its role.
  // Physical page of this wavefront's half of the stream's tile at step t (clamped to the
  // row); phase 0 needs none.
  // (PT: from the LDS page table, which the walk fills before its first step; otherwise and
  // before that, with a scalar load)
  auto page_of = [&](auto hpc, auto ptc, int t) -> int {
    constexpr int HP = decltype(hpc)::value;
    constexpr bool PT = decltype(ptc)::value;
    const int kt = kStreams * t + st;
    if constexpr (HP == 0) return 0;
    else if constexpr (PT) return nidx > 0 ? __builtin_amdgcn_readfirstlane(sm.pt[min(2 * kt + qg, nidx - 1)]) : 0;
    else return nidx > 0 ? load_uniform(P.indices, p0 + min(2 * kt + qg, nidx - 1)) : 0;
  };
  auto issue = [&](auto hpc, int t, int buf, int phys) {
    constexpr int HP = decltype(hpc)::value;
    const int kt = kStreams * t + st;
    if constexpr (HP == 0) {
      const char* kb = kh_plane + (size_t)min(kt, ntiles - 1) * kKT * kHeadDim * 2;
      const uint32_t dst = lds_address(&tb[buf].k[16 * qg][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16(dst + 1024u * i, kb, doff[i]);
    } else {
      // only the item's own tiles count: the walk also loads for steps past a stream's end
      // an out-of-range page reads page 0 (and poisons the item if the tile is the item's own)
      const bool phys_ok = (uint32_t)phys < (uint32_t)P.num_pages;
      poison |= (!phys_ok && kt < ntiles) ? 1 : 0;
      const char* vb = v_head + (uint64_t)(phys_ok ? (uint32_t)phys : 0u) * v_page_bytes;
      const uint32_t dst = lds_address(&tb[buf].v[16 * qg][0]);
      // the last slot of the page holding a key of the row (15 unless the page reaches the
      // row's end): the slots after it read that one (no branch: the step stays one block)
      const uint32_t smax_off = (uint32_t)(2 * kt + qg >= nidx - 1 ? lpl - 1 : 15) * v_row_bytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16(dst + 1024u * i, vb, min(doff[i], smax_off) + dch[i]);
    }
  };
  // End of step t: step t + 1 computes the scores of tile t + 2 and adds P.V of tile t, so
  // k^ of step t + 2 (issued at step t - 1) and V of step t (issued at step t - 2) must have
  // landed.  The loads issued after them may stay in flight: k^ of step t + 3, V of steps
  // t + 1 and t + 2 (4 instructions each).  Loads complete in issue order.
  auto wait_end = [&](auto hpc) {
    constexpr int HP = decltype(hpc)::value;
    if constexpr (HP == 0) wait_vmcnt<4>();
    else wait_vmcnt<8>();
  };
  // The k^ operand of dim step s, lane (n, hh): key n, dims 16 s + 8 hh .. +7 = logical chunk
  // 2 s + hh of row n, one 16-byte read at physical chunk (2 s + hh) ^ (n % 16).
  uint32_t k_addr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) k_addr[s] = lds_address(&tb[0].k[n][8 * ((2 * s + hh) ^ (n & 15))]);
  auto read_k = [&](int buf, bf16x8 (&ka)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      ka[s] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          (uintptr_t)(k_addr[s] + (uint32_t)(buf * sizeof(TileBuf))));
  };
  // S^T = k^ q^T of one tile
  auto mma_s = [&](const bf16x8 (&ka)[8], f32x16& s_out) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s_out[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) s_out = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qop[s], s_out, 0, 0, 0);
  };
  // transposed V reads, operand 2 db + ks: key rows 16 ks + vr (+ 8), dims 32 db + vc .. +3
  const int vr = 4 * hh + ((lane & 15) >> 2);
  const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto read_v = [&](int buf, bf16x8 (&va)[8]) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // rows 16 ks + vr and 16 ks + 8 + vr are both = vr (mod 4): physical block db ^ (vr % 4)
        const int col = 32 * (db ^ (vr & 3)) + vc;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&tb[buf].v[16 * ks + vr][col]));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&tb[buf].v[16 * ks + 8 + vr][col]));
        va[2 * db + ks] = __builtin_bit_cast(bf16x8, concat4(v0, v1));
      }
  };

  const int key_of = 4 * hh;  // S^T register i of this lane is key 8 (i / 4) + 4 hh + i % 4 of the tile
  // p = 2^(s C - m) of the lane's 16 keys, their sum (in register order) and the BF16 B
  // operands of the two P.V key steps
  auto tile_p = [&](const f32x16& sc, float mneg, float& sum, bf16x8 (&pb)[2]) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], kScoreScaleLog2, mneg));
    sum = p[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += p[i];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i16x4 lo = pack_bf16(p[8 * ks + 0], p[8 * ks + 1], p[8 * ks + 2], p[8 * ks + 3]);
      const i16x4 hi = pack_bf16(p[8 * ks + 4], p[8 * ks + 5], p[8 * ks + 6], p[8 * ks + 7]);
      pb[ks] = __builtin_bit_cast(bf16x8, concat4(lo, hi));
    }
  };

  // P.V of one tile: O^T += V^T P^T
  auto mma_pv = [&](const bf16x8 (&va)[8], const bf16x8 (&pb)[2]) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * db + ks], pb[ks], acc[db], 0, 0, 0);
  };

  // One step of a stream's walk, between two workgroup barriers.  Tile k's k^ is loaded three
  // steps ahead (at step k - 3) and its V two steps ahead; at the start of step t, k^ of steps t
  // + 1 and V of steps t - 1 and t are in LDS, s_cur holds the scores of step t and pb_prev the
  // probabilities of step t - 1.  The step computes the scores of step t + 1 and adds P.V of
  // step t - 1 on the matrix cores while the vector units run the softmax of step t: none of the
  // three depends on another, so the matrix cores and the vector units overlap.  A lazy
  // reference move at step t rescales the accumulator after P.V of step t - 1 (relative to the
  // old reference) has been added.  On a stream's last step the scores of the next buffer are
  // computed but never used (no load into that buffer is then in flight).
  auto step = [&](auto hpc, auto ptc, const int t, const int b_k, const int b_v, const int b_kload, const int b_vload,
                  int& phys_next, f32x16& s_cur, f32x16& s_nxt, bf16x8 (&pb_prev)[2]) {
    constexpr int HP = decltype(hpc)::value;
    const int kt = kStreams * t + st;
    // the page of the next step's V load, looked up before this step's LDS reads (so that
    // waiting for it does not wait for them)
    const int ld = HP == 0 ? t + 3 : t + 2;
    const int phys_after = page_of(hpc, ptc, ld + 1);
    // causal mask on tiles that reach past the block's first query, and on tiles past the
    // item's last one (a stream with one tile fewer than the other runs that step masked)
    if (kt >= ntiles || (kt + 1) * kKT > free_end) {
      const int d = (kt < ntiles ? lim : 0) - kt * kKT - key_of;  // key 8 (i/4) + key_of + i%4 visible iff < lim
#pragma unroll
      for (int i = 0; i < 16; ++i) s_cur[i] = 8 * (i >> 2) + (i & 3) < d ? s_cur[i] : -__builtin_inff();
    }
    bf16x8 ka[8], va[8];
    read_v(b_v, va);
    read_k(b_k, ka);
    mma_pv(va, pb_prev);
    // V reads first (P.V needs them first), then the P.V MFMAs each behind two k^ reads, so
    // the LDS queue is not filled by one wavefront's whole burst before its MFMAs issue
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // k^ of step t + 3 (phase 0) or V of step t + 2 (phase 1), into the buffer freed at the
    // previous barrier.  Issued on every step (past the stream's end the tile index is clamped
    // and the loads land in buffers nothing reads), so the step has no branch around them.
    issue(hpc, ld, HP == 0 ? b_kload : b_vload, phys_next);
    phys_next = phys_after;
    mma_s(ka, s_nxt);
    float lp;
    tile_p(s_cur, m_neg, lp, pb_prev);
    // the S MFMAs spread over the softmax's vector work
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
    }
    // the fix-up below runs when the probabilities against the current reference sum past
    // 2^kLazyMax (or overflow, or are NaN), or when the reference is unset and a key is visible
    // (lp is a sum of non-negative terms, so lp != 0 is !(lp <= 0): one compare either way)
    const float lp_max = m_run == -__builtin_inff() ? 0.0f : 256.0f;
    const bool need = !(lp <= lp_max);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      float mx = s_cur[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s_cur[i]);
      const float rowmax = pair32_max(mx) * kScoreScaleLog2;
      if (rowmax > m_run + kLazyMax || (m_run == -__builtin_inff() && rowmax > -__builtin_inff())) {
        const float alpha = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - rowmax);
        m_run = rowmax;
        m_neg = -rowmax;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = acc[db] * alpha;
        tile_p(s_cur, m_neg, lp, pb_prev);
      }
    }
    l_part += lp;
    wait_end(hpc);
    __syncthreads();
  };

  auto walk = [&](auto hpc, auto ptc) {
    constexpr int HP = decltype(hpc)::value;
    // k^ of steps 0-2 (phase 0) or V of steps 0-1 (phase 1) go out right behind the q^ loads,
    // and one wait covers both (a single memory latency before the walk).  The wait also tells
    // the compiler, which does not count the direct-to-LDS loads (inline assembly), that q^ has
    // landed on every path: otherwise it places a wait for q^ inside the walk, where it would
    // drain every tile load in flight.  V buffer 3 stands in for the tile of step -1: zeros,
    // so the first step's P.V adds nothing.
    int phys_next = 0;
    if (nsteps > 0) {
      if constexpr (HP == 0) {
        issue(hpc, 0, 0, 0);
        issue(hpc, 1, 1, 0);
        issue(hpc, 2, 2, 0);
      } else {
        // pages 2 kt + qg of tiles kt = st, 2 + st, 4 + st: from the unit record
        issue(hpc, 0, 0, load_uniform(rec, kUnitPage0 + 2 * st + qg));
        issue(hpc, 1, 1, load_uniform(rec, kUnitPage0 + 4 + 2 * st + qg));
        phys_next = load_uniform(rec, kUnitPage0 + 8 + 2 * st + qg);
      }
    }
    wait_vmcnt<0>();
    // every thread writes its share of the page table (whatever its own role), before the
    // barrier below
    if (use_pt) {
#pragma unroll
      for (int j = 0; j < kPtPerThread; ++j) {
        const int i = tid + kAttendThreads * j;
        if (i < nidx) sm.pt[i] = ptv[j];
      }
    }
    {
      uint32_t* z = reinterpret_cast<uint32_t*>(&tb[3].v[0][0]);
      constexpr int kWords = kKT * kHeadDim / 2;
      for (int i = (w >> 1) * 64 + lane; i < kWords; i += 256) z[i] = 0u;  // the stream's four wavefronts
    }
    __syncthreads();
    f32x16 s0, s1;
    bf16x8 pb[2];
    pb[0] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    pb[1] = pb[0];
    if (nsteps > 0) {
      bf16x8 ka[8];
      read_k(0, ka);
      mma_s(ka, s0);
    }
    // whole rounds of the four buffers, then the last steps (no exit inside a round); buffer
    // of step k is k % 4 for both k^ and V
    int t = 0;
    for (; t + kBufs <= nsteps; t += kBufs) {
      step(hpc, ptc, t, 1, 3, 3, 2, phys_next, s0, s1, pb);
      step(hpc, ptc, t + 1, 2, 0, 0, 3, phys_next, s1, s0, pb);
      step(hpc, ptc, t + 2, 3, 1, 1, 0, phys_next, s0, s1, pb);
      step(hpc, ptc, t + 3, 0, 2, 2, 1, phys_next, s1, s0, pb);
    }
    if (t < nsteps) step(hpc, ptc, t, 1, 3, 3, 2, phys_next, s0, s1, pb);
    if (t + 1 < nsteps) step(hpc, ptc, t + 1, 2, 0, 0, 3, phys_next, s1, s0, pb);
    if (t + 2 < nsteps) step(hpc, ptc, t + 2, 3, 1, 1, 0, phys_next, s0, s1, pb);
    // P.V of the last step (its V landed before the last barrier); the loads issued past the
    // end drain before the tile buffers become the merge area
    if (nsteps > 0) {
      bf16x8 va[8];
      read_v((nsteps - 1) & 3, va);
      mma_pv(va, pb);
    }
    wait_vmcnt<0>();
  };
  const std::integral_constant<int, 0> phase0;
  const std::integral_constant<int, 1> phase1;
  const std::integral_constant<bool, true> table;
  const std::integral_constant<bool, false> no_table;
  if (hp == 0) walk(phase0, no_table);  // phase 0 looks up no pages
  else if (use_pt) walk(phase1, table);
  else walk(phase1, no_table);

  // ---- merge the two streams of each query row (stream 0, then stream 1) and write out.  The
  // two wavefronts of a pair (the same rows, streams 0 and 1) each write half of every row:
  // stream 0 dims 0..63 (accumulator blocks 0, 1), stream 1 dims 64..127 (blocks 2, 3).  Each
  // hands the other its reference, partial sum and the two blocks the other writes, through
  // LDS.  Both evaluate the merge with stream 0's terms in stream 0's roles, and the sums add
  // two terms, which gives the same bits in either order.
  const bool out_poison = __syncthreads_or(poison) != 0;  // also: every wavefront is done with the tiles
  const int pair = w >> 1;  // wavefronts 2 pair and 2 pair + 1 hold the same rows, streams 0 and 1
  auto merge_out = [&](auto stc) {
#pragma clang fp contract(off)
    constexpr int ST = decltype(stc)::value;
    constexpr int kOwn = 2 * ST;       // first accumulator block this wavefront writes out
    constexpr int kGive = 2 - 2 * ST;  // first block the other wavefront writes out
    {
      float(&snd)[2 + 32][64] = sm.u.m.merge[pair][ST];
      snd[0][lane] = m_run;
      snd[1][lane] = l_part;
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) snd[2 + 16 * k + i][lane] = acc[kGive + k][i];
    }
    __syncthreads();
    const float(&rcv)[2 + 32][64] = sm.u.m.merge[pair][1 - ST];
    const float m_other = rcv[0][lane];
    const float l_other = rcv[1][lane];
    const float m0 = ST == 0 ? m_run : m_other;
    const float m1 = ST == 0 ? m_other : m_run;
    const float mx = fmaxf(m0, m1);
    const float a0 = m0 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m0 - mx);
    const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
    const float a_own = ST == 0 ? a0 : a1;
    const float a_other = ST == 0 ? a1 : a0;
    const float l = pair32_sum(l_part * a_own + l_other * a_other);
    const int gi = hg * 4 + 2 * hp + (n >> 4);  // head within the GQA group
    const bool live = gi < G && qi < Sq;
    const bool empty = l == 0.0f;
    const float inv = empty ? 0.0f : 1.0f / l;
    const size_t row = ((size_t)b * P.num_q_heads + hk * G + (gi < G ? gi : 0)) * Sq + (qi < Sq ? qi : 0);
    // the pair's rows go through LDS (lane (n, hh) holds dims 32 db + 8 q4 + 4 hh .. +3 of row
    // n) and out as half rows: 16 bytes per lane, eight rows per store
    uint16_t(&stage)[32][kOutPitch] = sm.u.m.out[pair];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int db = kOwn + k;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          const float v = acc[db][i] * a_own + rcv[2 + 16 * k + i][lane] * a_other;
          o[e] = out_poison ? __builtin_nanf("") : v * inv;
        }
        *reinterpret_cast<i16x4*>(&stage[n][32 * db + 8 * q4 + 4 * hh]) = pack_bf16(o[0], o[1], o[2], o[3]);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + (lane >> 3);     // row (column n of the MFMAs)
      const int ch = 8 * ST + (lane & 7);    // 16-byte chunk of the row
      const int gr = hg * 4 + 2 * hp + (r >> 4);
      const int qr = qb * kQB + 16 * qg + (r & 15);
      const uint2 lo = *reinterpret_cast<const uint2*>(&stage[r][8 * ch]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&stage[r][8 * ch + 4]);
      if (gr < G && qr < Sq) {
        const size_t orow = ((size_t)b * P.num_q_heads + hk * G + gr) * Sq + qr;
        stg16(P.out + orow * kHeadDim + 8 * ch, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
    if (ST == 0 && live && hh == 0) {
      float lse = empty ? -__builtin_inff() : (mx + __builtin_log2f(l)) * kLn2;
      if (out_poison) lse = __builtin_nanf("");
      P.lse[row] = lse;
    }
  };
  if (st == 0) merge_out(std::integral_constant<int, 0>{});
  else merge_out(std::integral_constant<int, 1>{});
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  char* ws = (char*)p.workspace;
  const size_t kh_bytes = prefill_kh_bytes(p.num_kv_heads, p.num_indices);
  const size_t qh_bytes = prefill_qh_bytes(p.num_q_heads, p.batch, p.q_len);
  uint16_t* kh = (uint16_t*)ws;
  uint16_t* qh = (uint16_t*)(ws + kh_bytes);
  int32_t* units = (int32_t*)(ws + kh_bytes + qh_bytes);
  // k^: per row up to max_pages_per_row * Hkv / HG tasks, 4 per workgroup, at most 512
  // workgroups per row; two KV heads per wavefront when Hkv is even, so each page's cos/sin is
  // read once per two heads (measured: faster than one or four).  q^: 4 wavefront tasks per
  // workgroup.  Unit records: 8 units per workgroup.
  const int hg = p.num_kv_heads % 2 == 0 ? 2 : 1;
  const long long row_tasks = (long long)std::min(p.max_pages_per_row, p.num_indices) * (p.num_kv_heads / hg);
  const int kx = (int)std::min<long long>((row_tasks + 3) / 4, 512);
  const long long qtasks =
      (long long)p.batch * ((p.num_q_heads + kQH - 1) / kQH) * ((p.q_len + 15) / 16);
  const int nq = (int)((qtasks + 3) / 4);
  const int nqb = (p.q_len + kQB - 1) / kQB;
  const int U = p.batch * nqb;
  const int nu = (U + 7) / 8;
  const unsigned pgrid = (unsigned)((long long)p.batch * kx + nq + nu);
  if (hg == 2)
    hipLaunchKernelGGL(prologue_kernel<2>, dim3(pgrid), dim3(kPrologueThreads), 0, stream, p, kh, qh, units, kx, nq);
  else
    hipLaunchKernelGGL(prologue_kernel<1>, dim3(pgrid), dim3(kPrologueThreads), 0, stream, p, kh, qh, units, kx, nq);
  const unsigned nhg = (unsigned)((p.group + 3) / 4);
  const unsigned grid = (unsigned)U * (unsigned)p.num_kv_heads * nhg;
  if (grid > 0)
    hipLaunchKernelGGL(attend_kernel, dim3(grid), dim3(kAttendThreads), 0, stream, p, kh, qh, units);
  return hipGetLastError();
}

}  // namespace pa

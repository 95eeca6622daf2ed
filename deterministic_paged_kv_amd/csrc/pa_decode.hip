// Paged decode, no Split-KV: a fixed reduction tree per (row, KV head), run by one
// workgroup, or by one wavefront per stream on separate compute units with identical bits.
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
// Reduction tree.  The row's pages are dealt to 16 streams: stream s takes logical pages
// s, s+16, s+32, ...  Each stream runs an FP32 online softmax over its pages in ascending
// order, one page (16 keys) per step: S^T = K^ Q^T by bf16 MFMA with FP32 accumulation, a
// page max and sum per head taken in a fixed order (4 keys in registers, then a 2-step lane
// exchange), and O^T += V^T P^T by bf16 MFMA into FP32 with P split into two bf16 parts
// (hi + lo), so the probabilities keep about 16 significant bits.  The 16 stream states are
// then combined in stream order 0..15.  The tree depends only on the row's own length, so the
// bits of a row are the same whatever batch it is in, whatever the plan width and wherever
// its pages sit.
//
// Two schedules run this same tree with the same device code (floating-point contraction is
// pinned off in it, so both compile to the same arithmetic):
//  * one workgroup of 8 wavefronts per (row, KV head), wavefront w walking pages w, w+8, ...
//    and so running streams w and w+8, states combined through LDS (no workspace);
//  * one wavefront per (row, KV head, stream), states written to a caller workspace, and a
//    second kernel that combines each unit's states in stream order.  This spreads a long row
//    over 16 compute units; the bits are identical.  Rows are launched longest first.  When
//    the batch fills the device, the wavefronts of up to four KV heads of one (row, stream)
//    form a workgroup: they walk the same pages, so each page's cos/sin rows are read once
//    and shared through LDS instead of once per KV head.
//
// Memory layout.  k_cache/v_cache are NHD [page][slot][Hkv][128] bf16: one KV head of one
// page is 16 rows of 256 B at a stride of Hkv * 256 B.  A lane (r = lane % 16, g = lane / 16)
// loads key/value row r of the page as four 16-byte pieces (dims 32*kb + 8*g ..), so one
// load instruction covers 64 contiguous bytes of each of the 16 rows.  K goes straight from
// registers through the prologue into the MFMA A operand; V is staged in LDS and read back
// with keys along the MFMA reduction dimension.
#include <type_traits>

#include "pa_internal.h"

namespace pa {

namespace {

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kStreams = 16;                 // streams of the reduction tree
constexpr int kUnitWaves = 8;                // wavefronts of the one-workgroup schedule
constexpr int kDecodeThreads = kUnitWaves * 64;
// pages in flight per wavefront: the unit schedule runs 2 wavefronts per SIMD, the
// multi-CU schedule one or two with the register file to itself
constexpr int kUnitRing = 2;
constexpr int kStreamRing = 2;
// V staging rows are padded by 16 bytes to spread the transposed reads over the LDS banks.
constexpr int kVRow = kHeadDim + 8;
typedef uint16_t VSlot[kPageSize][kVRow];

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Row geometry from the CSR block table, with the bounds checks every kernel applies.
struct RowInfo {
  int p0, n, L, qp;
  bool bad;
  size_t head0;  // index of the group's first query head in [B * Hq]
};

// From the row's five metadata values (indptr[b], indptr[b + 1], last_page_len[b], qpos[b],
// cache_position[b]).  A cache position that differs from the query position breaks the rule
// cache_position == query_position_ids and makes the row bad, like an out-of-range value.
__device__ __forceinline__ RowInfo row_info_of(const DecodeParams& P, int b, int hk, int p0, int p1, int lpl, int qp,
                                               int cp) {
  RowInfo ri;
  ri.p0 = p0;
  ri.n = p1 - ri.p0;
  ri.qp = qp;
  ri.bad = ri.p0 < 0 || ri.n < 0 || p1 > P.num_indices || ri.n > P.max_pages_per_row || ri.qp < 0 ||
           ri.qp >= P.table_rows || cp != qp || (ri.n > 0 && (lpl < 1 || lpl > kPageSize));
  ri.L = (ri.n > 0 && !ri.bad) ? (ri.n - 1) * kPageSize + lpl : 0;
  ri.head0 = (size_t)b * P.num_q_heads + (size_t)hk * P.group;
  return ri;
}

__device__ __forceinline__ RowInfo row_info(const DecodeParams& P, int b, int hk) {
  return row_info_of(P, b, hk, P.indptr[b], P.indptr[b + 1], P.last_page_len[b], P.qpos[b], P.cache_position[b]);
}

// Output of a row with no keys (0, -inf) or with out-of-range metadata (NaN, NaN).
__device__ __forceinline__ void write_degenerate(const DecodeParams& P, const RowInfo& ri, int tid, int nthreads) {
  for (int i = tid; i < P.group * kHeadDim; i += nthreads) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    P.out[(ri.head0 + h) * kHeadDim + d] = ri.bad ? (uint16_t)0x7FC0 : (uint16_t)0;
    if (d == 0) P.lse[ri.head0 + h] = ri.bad ? __builtin_nanf("") : -__builtin_inff();
  }
}

// One page of one KV head as this lane holds it: key row r (dims 32*kb + 8*g ..) of K and V.
struct PageIn {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ void issue_page(PageIn& in, const DecodeParams& P, int phys, int hk, int r, int g) {
  const size_t row_off = (((size_t)phys * kPageSize + r) * P.num_kv_heads + hk) * kHeadDim + 8 * g;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) in.k[kb] = ldg16(P.k_cache + row_off + 32 * kb);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) in.v[kb] = ldg16(P.v_cache + row_off + 32 * kb);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Softmax state of one stream: running max and sum of head r (in every lane with that r),
// and O^T (lane (r, g) holds dims 16*nb + 4g + i of head r).
struct StreamState {
  float m, l;
  f32x4 acc[8];
  int poison;
};
struct Scored {
  i16x4 p_hi, p_lo;  // P^T of the page as two bf16 parts (hi + lo)
  float alpha;       // rescale of the accumulator before this page's P.V
};

// Scores of page pg: stage V in LDS, run the K prologue, S^T = K^ Q^T, and advance the
// running max and sum.  Lane (r, g) holds keys 4g+i of head r.
// K norm weights: read from LDS by every page (the one-workgroup schedule, short of
// registers), or held in registers.
struct KwLds {
  const float* p;
  __device__ __forceinline__ void prologue(const uint4 raw[4], bool knorm, float eps, const float4 cs[8], int g,
                                           bf16x8 out[4]) const {
    prologue_operand_lds_w(raw, p, knorm, eps, cs, g, out);
  }
};
struct KwRegs {
  float w[32];
  __device__ __forceinline__ void load(const float* k_norm, int g) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) w[kb * 8 + e] = k_norm != nullptr ? k_norm[32 * kb + 8 * g + e] : 1.0f;
  }
  __device__ __forceinline__ void prologue(const uint4 raw[4], bool knorm, float eps, const float4 cs[8], int g,
                                           bf16x8 out[4]) const {
    (void)g;
    prologue_operand(raw, w, knorm, eps, cs, out);
  }
};

template <class Kw>
__device__ __forceinline__ Scored score_page(const PageIn& in, const float4 cs[8], int pg, StreamState& st,
                                             const bf16x8 qop[4], const Kw& kw, bool knorm, float eps, int L,
                                             int qp, int r, int g, VSlot& sv) {
#pragma clang fp contract(off)
  // keys at or past `live_end` are invisible (past the row, or after the query): only a row's
  // last pages have any, so the masking sits behind a wave-uniform test
  const int live_end = min(L, qp + 1);
  const bool tail = pg * kPageSize + kPageSize > live_end;
  if (!tail) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<uint4*>(&sv[r][32 * kb + 8 * g]) = in.v[kb];
  } else {
    const bool vlive = pg * kPageSize + r < L;  // value rows past the row's end are zero
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      *reinterpret_cast<uint4*>(&sv[r][32 * kb + 8 * g]) = vlive ? in.v[kb] : make_uint4(0, 0, 0, 0);
  }

  bf16x8 kop[4];
  kw.prologue(in.k, knorm, eps, cs, g, kop);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb], qop[kb], s, 0, 0, 0);

  float t[4];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[i] = s[i] * kScoreScaleLog2;
    if (tail) {
      const int j = pg * kPageSize + 4 * g + i;  // logical key index = key position
      t[i] = j < live_end ? t[i] : -__builtin_inff();
    }
    mx = fmaxf(mx, t[i]);
  }
  mx = pair32_max(pair16_max(mx));
  const float m_new = fmaxf(st.m, mx);
  const bool any = m_new != -__builtin_inff();
  Scored sc;
  sc.alpha = any ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.0f;
  float pr[4];
  float ps = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[i] = any ? __builtin_amdgcn_exp2f(t[i] - m_new) : 0.0f;
    ps = ps + pr[i];
  }
  ps = pair32_sum(pair16_sum(ps));
  st.l = __builtin_fmaf(st.l, sc.alpha, ps);
  st.m = m_new;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 hi = (__bf16)pr[i];
    sc.p_hi[i] = __builtin_bit_cast(short, hi);
    sc.p_lo[i] = __builtin_bit_cast(short, (__bf16)(pr[i] - (float)hi));
  }
  return sc;
}

// acc = acc * alpha + P.V for a scored page whose V sits in `sv`.
__device__ __forceinline__ void pv_page(const Scored& sc, StreamState& st, int r, int g, VSlot& sv) {
#pragma clang fp contract(off)
  // rescale only when some head's max moved: multiplying by exactly 1 changes nothing
  if (__builtin_amdgcn_ballot_w64(sc.alpha != 1.0f) != 0) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) st.acc[nb] = st.acc[nb] * sc.alpha;
  }
  // V^T operand by transposed LDS reads: in each 16-lane group g, lane j points at keys
  // 4g + j/4, dims 16*nb + 4*(j%4) .. +3; lane r then receives keys 4g .. 4g+3 of dim 16*nb + r.
  // One K=32 MFMA takes both parts of P: k-slots 8g..8g+3 pair V rows 4g..4g+3 with P_hi,
  // k-slots 8g+4..8g+7 pair the same rows with P_lo.
  const int jr = 4 * g + (r >> 2);
  const int jc = 4 * (r & 3);
  const bf16x8 pb = __builtin_bit_cast(
      bf16x8, i16x8{sc.p_hi[0], sc.p_hi[1], sc.p_hi[2], sc.p_hi[3], sc.p_lo[0], sc.p_lo[1], sc.p_lo[2], sc.p_lo[3]});
  // all eight reads in flight before the first MFMA consumes one
  i16x4 va[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) va[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sv[jr][16 * nb + jc]));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const bf16x8 vv =
        __builtin_bit_cast(bf16x8, i16x8{va[nb][0], va[nb][1], va[nb][2], va[nb][3], va[nb][0], va[nb][1], va[nb][2], va[nb][3]});
    st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb, st.acc[nb], 0, 0, 0);
  }
}

// Where a walk step's cos/sin rows come from (one row of 64 cos and 64 sin per key position,
// 512 bytes).  CsOwn: the wavefront loads its own, one step ahead.  CsShared<HW>: the HW
// wavefronts of a workgroup walk the same pages for HW KV heads, so they need the same rows;
// each loads 8/HW of the eight 16-byte pieces per lane two steps ahead, they are staged in
// an LDS ring of two slots, and a workgroup barrier per step publishes them.  The values are
// the same either way, only the traffic differs (the rows of a page are read from the cache
// hierarchy once per workgroup instead of once per KV head).
struct CsOwn {
  float4 cs[8];
  int g;
  __device__ __forceinline__ CsOwn(int g_) : g(g_) {}
  template <class KP>
  __device__ __forceinline__ void start(const DecodeParams& P, KP key_pos) { load_cos_sin(P.rope, key_pos(0), g, cs); }
  template <int K>
  __device__ __forceinline__ const float4* get() const { return cs; }
  template <int K, class KP>
  __device__ __forceinline__ void after_score(const DecodeParams& P, KP key_pos, int t) {
    load_cos_sin(P.rope, key_pos(t + 1), g, cs);
  }
  template <int K>
  __device__ __forceinline__ void end_step() {}
};

typedef f32x4 CsSlots[2][8][64];  // LDS ring: slot, piece, lane (native vectors: kept in registers)

template <int HW>
struct CsShared {
  static constexpr int kPieces = 8 / HW;  // pieces this wavefront loads
  f32x4 share0[kPieces], share1[kPieces];  // in flight for even / odd steps
  float4 cs[8];
  template <int K>
  __device__ __forceinline__ f32x4 (&share())[kPieces] {
    if constexpr ((K & 1) == 0) return share0;
    else return share1;
  }
  CsSlots& slots;
  int g, lane, w;
  __device__ __forceinline__ CsShared(CsSlots& s, int g_, int lane_, int w_) : slots(s), g(g_), lane(lane_), w(w_) {}
  __device__ __forceinline__ void load_share(const DecodeParams& P, int pos, f32x4 (&dst)[kPieces]) {
    const f32x4* blk = reinterpret_cast<const f32x4*>(P.rope + (size_t)(pos >> 4) * kRopeBlockFloats);
    const int l = (pos & 15) + 16 * g;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) dst[i] = blk[(w * kPieces + i) * 64 + l];
  }
  __device__ __forceinline__ void publish(int slot, const f32x4 (&src)[kPieces]) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) slots[slot][w * kPieces + i][lane] = src[i];
    workgroup_lds_sync();
  }
  template <class KP>
  __device__ __forceinline__ void start(const DecodeParams& P, KP key_pos) {
    load_share(P, key_pos(0), share0);
    load_share(P, key_pos(1), share1);
    publish(0, share0);
  }
  // K: the walk step's parity (steps go in pairs, so the slots are compile-time constants)
  template <int K>
  __device__ __forceinline__ const float4* get() {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 v = slots[K & 1][e][lane];
      cs[e] = make_float4(v[0], v[1], v[2], v[3]);
    }
    return cs;
  }
  template <int K, class KP>
  __device__ __forceinline__ void after_score(const DecodeParams& P, KP key_pos, int t) {
    load_share(P, key_pos(t + 2), share<K>());
  }
  template <int K>
  __device__ __forceinline__ void end_step() { publish((K + 1) & 1, share<K + 1>()); }
};

// One wavefront's walk over the pages first, first + stride, first + 2 stride, ... of one
// (row, KV head) unit, at most `count` of them.  Walk step t feeds state st[t % NS]: with stride = kStreams and NS = 1
// the wavefront is stream `first`; with stride = kStreams / 2 and NS = 2 it runs streams
// `first` (even steps) and `first` + kStreams / 2 (odd steps).  Either way each stream sees its
// own pages in ascending order.
// R pages of K and V are in flight: walk step t sits in ring slot t % R, and once it is scored
// the slot is refilled with step t + R.  The cos/sin rows of the keys (mostly cache hits, read
// by every KV head) run RC steps ahead in a ring of their own.  The physical page numbers come
// 64 at a time in one vector load (lane l: walk step 64 blk + l) and are taken out with
// readlane, so they never wait behind other loads.  Steps past the row's end load the row's
// last page (their data is never used), so every step issues the same loads.
template <int R, int NS, class Kw, class Cs>
__device__ __forceinline__ void run_walk(const DecodeParams& P, const RowInfo& ri, int hk, int first, int stride,
                                         int count, int lane, VSlot& sv, const Kw& kw, Cs& csrc,
                                         StreamState (&st)[NS]) {
  static_assert(R % NS == 0 && R % 2 == 0, "the state cycle must divide the K/V ring, which holds whole pairs of steps");
  const int r = lane & 15;
  const int g = lane >> 4;
  const int G = P.group;
  const int n = ri.n, L = ri.L, qp = ri.qp, p0 = ri.p0;
  const bool qnorm = P.q_norm != nullptr;
  const bool knorm = P.k_norm != nullptr;
  const int steps = min(count, n > first ? (n - first + stride - 1) / stride : 0);

  // the query's inputs go out first: they depend on nothing loaded here
  uint4 qraw[4];
  float qw[32];
  float4 qcs[8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    qraw[kb] = make_uint4(0, 0, 0, 0);
    if (r < G) qraw[kb] = ldg16(P.q + (ri.head0 + r) * kHeadDim + 32 * kb + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) qw[kb * 8 + e] = qnorm ? P.q_norm[32 * kb + 8 * g + e] : 1.0f;
  }
  load_cos_sin(P.rope, qp, g, qcs);

#pragma unroll
  for (int i = 0; i < NS; ++i) st[i].poison = 0;
  // lane l's page slot for block blk: walk step 64 blk + l, clamped to the row
  auto index_block = [&](int blk) {
    const int pg = min(first + (64 * blk + lane) * stride, n - 1);
    return P.indices[p0 + pg];
  };
  int vcur = index_block(0);
  int vnext = index_block(1);
  int cur_blk = 0;
  auto phys_at = [&](int t) {  // physical page of walk step t (t within blocks cur_blk, +1)
    const int a = __builtin_amdgcn_readlane(vcur, t & 63);
    const int c = __builtin_amdgcn_readlane(vnext, t & 63);
    int phys = (t >> 6) == cur_blk ? a : c;
    if (phys < 0 || phys >= P.num_pages) { st[0].poison |= t < steps; phys = 0; }
    return phys;
  };
  // position of key r of walk step t (steps past the end read the last page's)
  auto key_pos = [&](int t) { return min(first + t * stride, n - 1) * kPageSize + r; };
  // key_position_ids entry of key r of walk step t: the rotation above uses the logical index,
  // which is what the entry must hold; it is loaded with the page and checked when the page is
  // scored (live keys of the walk's own steps only)
  auto kpos_of = [&](int t) { return P.kpos[(size_t)p0 * kPageSize + key_pos(t)]; };
  auto check_kpos = [&](int t, int kp) {
    const int j = key_pos(t);
    const bool wrong = t < steps && j < L && kp != j;
    st[0].poison |= __builtin_amdgcn_ballot_w64(wrong) != 0 ? 1 : 0;
  };

  // q^ of the group's heads in the operand layout (vector r = head r < G), before any page
  // load is issued: when every wavefront of the grid starts at once, the query's few bytes
  // would otherwise queue behind the first pages of all of them
  bf16x8 qop[4];
  prologue_operand(qraw, qw, qnorm, P.eps, qcs, qop);
  __builtin_amdgcn_sched_barrier(0);

  PageIn in[R];
  int kp[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    issue_page(in[k], P, phys_at(k), hk, r, g);
    kp[k] = kpos_of(k);
  }
  csrc.start(P, key_pos);

#pragma unroll
  for (int i = 0; i < NS; ++i) {
    st[i].m = -__builtin_inff();
    st[i].l = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) st[i].acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // one walk step; K = t % R is a compile-time constant (ring slots stay in registers)
  auto step = [&](auto kc, int t0) {
    constexpr int k = decltype(kc)::value;
    const int t = t0 + k;
    StreamState& sk = st[k % NS];
    const Scored sc =
        score_page(in[k], csrc.template get<k>(), first + t * stride, sk, qop, kw, knorm, P.eps, L, qp, r, g, sv);
    check_kpos(t, kp[k]);
    csrc.template after_score<k>(P, key_pos, t);
    // refill the slot with step t + R; a new block of page numbers is due when t + R
    // enters the next one
    const int u = t + R;
    if ((u & 63) == 0 && (u >> 6) != cur_blk) {
      vcur = vnext;
      cur_blk = u >> 6;
      vnext = index_block(cur_blk + 1);
      // wait for the new block here, on this rare path, so that the common path after the
      // branch does not have to wait for every load in flight
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    issue_page(in[k], P, phys_at(u), hk, r, g);
    kp[k] = kpos_of(u);
    wave_lds_sync();
    pv_page(sc, sk, r, g, sv);
    wave_lds_sync();
    csrc.template end_step<k>();
  };
  // Whole pairs of steps, then the odd last one.  No path through the loop body skips a step,
  // so the wait counts at the loop head know both slots' loads are in flight and wait only
  // for the older one.
  static_assert(R == 2, "the walk below is written out for a ring of two");
  int t0 = 0;
  for (; t0 + 2 <= steps; t0 += 2) {
    step(std::integral_constant<int, 0>{}, t0);
    step(std::integral_constant<int, 1>{}, t0);
  }
  if (t0 < steps) step(std::integral_constant<int, 0>{}, t0);
}

// Combine the kStreams states of head h at dim d in stream order and write out (and lse at
// d == 0).  m(w), l(w), acc(w) read stream w's values.
template <class M, class Lf, class A>
__device__ __forceinline__ void combine_one(const DecodeParams& P, const RowInfo& ri, int h, int d, bool poison,
                                            M m, Lf l, A acc) {
#pragma clang fp contract(off)
  float mx = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kStreams; ++w) mx = fmaxf(mx, m(w));
  float num = 0.0f, den = 0.0f;
#pragma unroll
  for (int w = 0; w < kStreams; ++w) {
    const float mw = m(w);
    const float sc = mw == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw - mx);
    num = __builtin_fmaf(acc(w), sc, num);
    den = __builtin_fmaf(l(w), sc, den);
  }
  float o = num / den;
  float lse = (mx + __builtin_log2f(den)) * kLn2;
  if (poison) { o = __builtin_nanf(""); lse = __builtin_nanf(""); }
  P.out[(ri.head0 + h) * kHeadDim + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
  if (d == 0) P.lse[ri.head0 + h] = lse;
}

// ---------------------------------------------------------------------------------------
// Schedule 1: one workgroup per unit, stream s on wavefront s, combine through LDS.
// ---------------------------------------------------------------------------------------
struct UnitSmem {
  union {
    VSlot v[kUnitWaves];                   // per-wave V page
    float acc[kStreams][4][kHeadDim];      // per-stream outputs of 4 heads (combine)
  } u;
  float m[kStreams][kMaxGroup];
  float l[kStreams][kMaxGroup];
  float kw[kHeadDim];  // K RMSNorm weights
  int poison[kStreams];
};

__global__ __launch_bounds__(kDecodeThreads) void decode_unit_kernel(const DecodeParams P) {
  static_assert(kStreams == 2 * kUnitWaves, "each wavefront of the workgroup runs two streams");
  __shared__ UnitSmem sm;
  const int unit = blockIdx.x;
  const int b = unit / P.num_kv_heads;
  const int hk = unit % P.num_kv_heads;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int G = P.group;
  const RowInfo ri = row_info(P, b, hk);
  if (ri.bad || ri.L == 0) {
    write_degenerate(P, ri, tid, kDecodeThreads);
    return;
  }
  for (int i = tid; i < kHeadDim; i += kDecodeThreads) sm.kw[i] = P.k_norm != nullptr ? P.k_norm[i] : 1.0f;
  __syncthreads();

  // wavefront w walks pages w, w+8, ...: streams w (even steps) and w+8 (odd steps)
  StreamState st[2];
  CsOwn cso(g);
  run_walk<kUnitRing, 2>(P, ri, hk, wave, kUnitWaves, INT32_MAX, lane, sm.u.v[wave], KwLds{sm.kw}, cso, st);

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sid = wave + i * kUnitWaves;
    if (g == 0 && r < G) { sm.m[sid][r] = st[i].m; sm.l[sid][r] = st[i].l; }
    if (lane == 0) sm.poison[sid] = st[i].poison;
  }
  __syncthreads();
  int poison = 0;
#pragma unroll
  for (int w = 0; w < kStreams; ++w) poison |= sm.poison[w];
  // heads are combined four at a time through LDS
  for (int h0 = 0; h0 < G; h0 += 4) {
    if (r >= h0 && r < h0 + 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.u.acc[wave + i * kUnitWaves][r - h0][16 * nb + 4 * g + e] = st[i].acc[nb][e];
    }
    __syncthreads();
    const int nh = min(4, G - h0);
    for (int idx = tid; idx < nh * kHeadDim; idx += kDecodeThreads) {
      const int hi = idx / kHeadDim, d = idx % kHeadDim;
      const int h = h0 + hi;
      combine_one(P, ri, h, d, poison != 0, [&](int w) { return sm.m[w][h]; }, [&](int w) { return sm.l[w][h]; },
                  [&](int w) { return sm.u.acc[w][hi][d]; });
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Schedule 2: one single-wavefront workgroup per (unit, stream) writes its stream state to
// the workspace; a second kernel combines each unit's states in stream order.  The kernel
// boundary makes the states visible, so neither kernel needs a device-wide fence.
// Workspace: an int32 poison flag per (unit, stream), then per unit and stream G records of
// [m, l, 128 accumulators].
// ---------------------------------------------------------------------------------------

template <int HW>
__global__ __launch_bounds__(64 * HW) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_stream_kernel(
    const DecodeParams P, int32_t* __restrict__ poisons, float* __restrict__ states) {
  __shared__ VSlot svs[HW];
  __shared__ CsSlots cs_slots;  // used only when HW > 1
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  VSlot& sv = svs[w];
  // Placement.  When the grid is one dispatch round of two workgroups per compute unit,
  // workgroups i and i + #CU share a compute unit: the second round takes the order backwards,
  // so the longest rows' streams share compute units with the shortest rows'.
  const int nwg = (int)gridDim.x;
  int slot = (int)blockIdx.x;
  if (nwg > P.num_cus && nwg <= 2 * P.num_cus && slot >= P.num_cus) slot = nwg - 1 - (slot - P.num_cus);
  const int s = slot % kStreams;
  const int hgroups = P.num_kv_heads / HW;
  const int hk = ((slot / kStreams) % hgroups) * HW + w;
  const int rank = slot / (kStreams * hgroups);
  // Launch order: rows with more pages first, ties by row (up to 64 rows; beyond that, row
  // order).  The long rows' streams finish last; starting them first puts their first pages
  // at the head of the memory queue.  Only where a stream runs depends on it, not its bits.
  // Lane j holds row j's metadata (one round of loads for the whole batch); the row picked is
  // then read out of the lanes instead of being loaded again.
  int b = rank;
  RowInfo ri;
  if (P.batch <= 64) {
    const bool lv = lane < P.batch;
    const int ip0 = lv ? P.indptr[lane] : 0;
    const int ip1 = lv ? P.indptr[lane + 1] : 0;
    const int lpl = lv ? P.last_page_len[lane] : 0;
    const int qpl = lv ? P.qpos[lane] : 0;
    const int cpl = lv ? P.cache_position[lane] : 0;
    const int my = lv ? ip1 - ip0 : -1;
    int rk = 0;
    for (int j = 0; j < P.batch; ++j) {
      const int nj = __builtin_amdgcn_readlane(my, j);
      rk += (nj > my || (nj == my && j < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(lv && rk == rank);
    b = hit ? (int)__builtin_ctzll(hit) : rank;
    ri = row_info_of(P, b, hk, __builtin_amdgcn_readlane(ip0, b), __builtin_amdgcn_readlane(ip1, b),
                     __builtin_amdgcn_readlane(lpl, b), __builtin_amdgcn_readlane(qpl, b),
                     __builtin_amdgcn_readlane(cpl, b));
  } else {
    ri = row_info(P, b, hk);
  }
  const int unit = b * P.num_kv_heads + hk;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int G = P.group;
  if (ri.bad || ri.L == 0) return;  // the combine kernel writes these rows
  KwRegs kw;
  kw.load(P.k_norm, g);

  StreamState st[1];
  if constexpr (HW == 1) {
    CsOwn cso(g);
    run_walk<kStreamRing, 1>(P, ri, hk, s, kStreams, INT32_MAX, lane, sv, kw, cso, st);
  } else {
    CsShared<HW> css(cs_slots, g, lane, w);
    run_walk<kStreamRing, 1>(P, ri, hk, s, kStreams, INT32_MAX, lane, sv, kw, css, st);
  }

  const size_t rec = (size_t)G * (2 + kHeadDim);  // floats per stream state
  if (r < G) {
    float* hrec = states + ((size_t)unit * kStreams + s) * rec + (size_t)r * (2 + kHeadDim);
    if (g == 0) { hrec[0] = st[0].m; hrec[1] = st[0].l; }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) *reinterpret_cast<f32x4*>(hrec + 2 + 16 * nb + 4 * g) = st[0].acc[nb];
  }
  if (lane == 0) poisons[unit * kStreams + s] = st[0].poison;
}

// One workgroup per (unit, query head h), one thread per output dimension d.  The stream
// maxima, sums and poison flags are the same for every thread of the workgroup (wave-uniform
// loads); each thread reads its own dimension of the 16 accumulators.
__global__ __launch_bounds__(kHeadDim) void decode_combine_kernel(const DecodeParams P,
                                                                  const int32_t* __restrict__ poisons,
                                                                  const float* __restrict__ states) {
  const int G = P.group;
  const int unit = blockIdx.x / G;
  const int h = blockIdx.x % G;
  const int b = unit / P.num_kv_heads;
  const int hk = unit % P.num_kv_heads;
  const int d = threadIdx.x;
  // The states are read before the row's metadata is looked at (both go out together); the
  // workspace holds a record for every unit, so the reads are in bounds for any row.
  const size_t rec = (size_t)G * (2 + kHeadDim);
  const float* hs = states + (size_t)unit * kStreams * rec + (size_t)h * (2 + kHeadDim);
  float mw[kStreams], lw[kStreams], a[kStreams];
  int poison = 0;
#pragma unroll
  for (int w = 0; w < kStreams; ++w) {
    mw[w] = load_uniform_f32(hs + (size_t)w * rec, 0);
    lw[w] = load_uniform_f32(hs + (size_t)w * rec, 1);
    poison |= load_uniform(poisons, unit * kStreams + w);
    a[w] = hs[(size_t)w * rec + 2 + d];
  }
  const RowInfo ri = row_info(P, b, hk);
  // keep the state reads ahead of the branch (the compiler would otherwise issue them after it)
  asm volatile("" ::"v"(a[0]), "v"(a[kStreams - 1]));
#pragma unroll
  for (int w = 0; w < kStreams; ++w) asm volatile("" ::"s"(mw[w]), "s"(lw[w]));
  if (ri.bad || ri.L == 0) {
    P.out[(ri.head0 + h) * kHeadDim + d] = ri.bad ? (uint16_t)0x7FC0 : (uint16_t)0;
    if (d == 0) P.lse[ri.head0 + h] = ri.bad ? __builtin_nanf("") : -__builtin_inff();
    return;
  }
  combine_one(P, ri, h, d, poison != 0, [&](int w) { return mw[w]; }, [&](int w) { return lw[w]; },
              [&](int w) { return a[w]; });
}

// ---------------------------------------------------------------------------------------
// Fixed-chunk policy: the row's pages are cut into chunks of chunk_pages consecutive pages;
// chunk c (pages c * chunk_pages ..) is one online softmax over its pages in ascending order,
// on one wavefront, and the chunk states are folded in ascending chunk order.  The tree
// depends only on the row's length and the chunk size.  Workspace: an int32 poison flag per
// (unit, chunk slot), then per unit and chunk slot G records of [m, l, 128 accumulators].
// ---------------------------------------------------------------------------------------
// One wavefront per (row, KV head, chunk); as in the stream schedule, the wavefronts of up to
// HW KV heads of one (row, chunk) form a workgroup and share the chunk's cos/sin rows.
template <int HW>
__global__ __launch_bounds__(64 * HW) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_chunk_kernel(
    const DecodeParams P, int max_chunks, int32_t* __restrict__ poisons, float* __restrict__ states) {
  __shared__ VSlot svs[HW];
  __shared__ CsSlots cs_slots;  // used only when HW > 1
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  VSlot& sv = svs[w];
  const int hgroups = P.num_kv_heads / HW;
  const int grp = blockIdx.x / max_chunks;
  const int c = blockIdx.x % max_chunks;
  const int b = grp / hgroups;
  const int hk = (grp % hgroups) * HW + w;
  const int unit = b * P.num_kv_heads + hk;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int G = P.group;
  const RowInfo ri = row_info(P, b, hk);
  if (ri.bad || ri.L == 0) return;                       // the fold kernel writes these rows
  if (c * P.chunk_pages >= ri.n) return;                 // past the row's last chunk
  KwRegs kw;
  kw.load(P.k_norm, g);

  StreamState st[1];
  if constexpr (HW == 1) {
    CsOwn cso(g);
    run_walk<kStreamRing, 1>(P, ri, hk, c * P.chunk_pages, 1, P.chunk_pages, lane, sv, kw, cso, st);
  } else {
    CsShared<HW> css(cs_slots, g, lane, w);
    run_walk<kStreamRing, 1>(P, ri, hk, c * P.chunk_pages, 1, P.chunk_pages, lane, sv, kw, css, st);
  }

  const size_t rec = (size_t)G * (2 + kHeadDim);  // floats per chunk state
  if (r < G) {
    float* hrec = states + ((size_t)unit * max_chunks + c) * rec + (size_t)r * (2 + kHeadDim);
    if (g == 0) { hrec[0] = st[0].m; hrec[1] = st[0].l; }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) *reinterpret_cast<f32x4*>(hrec + 2 + 16 * nb + 4 * g) = st[0].acc[nb];
  }
  if (lane == 0) poisons[unit * max_chunks + c] = st[0].poison;
}

// Fold of (m, l, acc) in ascending chunk order: with m' = max(m, m_c),
//   l <- l 2^(m - m') + l_c 2^(m_c - m'),  acc <- acc 2^(m - m') + acc_c 2^(m_c - m'),  m <- m'
// (a state with m = -inf weighs 0), then out = acc / l and lse = (m + log2 l) ln 2.
// One workgroup per (unit, query head h), one thread per output dimension d: the chunk states
// are folded left to right, c = 0, 1, ..., in FP32.  The chunk maxima and sums go to LDS first
// (one load per thread); the accumulators then come in batches of kFoldBatch chunks whose
// loads all go out before the batch is folded.  Only the arithmetic is sequential.
constexpr int kFoldBatch = 32;
__global__ __launch_bounds__(kHeadDim) void decode_fold_kernel(const DecodeParams P, int max_chunks,
                                                               const int32_t* __restrict__ poisons,
                                                               const float* __restrict__ states) {
#pragma clang fp contract(off)
  __shared__ float ml[kMaxFixedChunks][2];
  const int G = P.group;
  const int unit = blockIdx.x / G;
  const int h = blockIdx.x % G;
  const int b = unit / P.num_kv_heads;
  const int hk = unit % P.num_kv_heads;
  const int d = threadIdx.x;
  const RowInfo ri = row_info(P, b, hk);
  if (ri.bad || ri.L == 0) {
    P.out[(ri.head0 + h) * kHeadDim + d] = ri.bad ? (uint16_t)0x7FC0 : (uint16_t)0;
    if (d == 0) P.lse[ri.head0 + h] = ri.bad ? __builtin_nanf("") : -__builtin_inff();
    return;
  }
  const int nch = (ri.n + P.chunk_pages - 1) / P.chunk_pages;  // <= kMaxFixedChunks (checked at plan time)
  const size_t rec = (size_t)G * (2 + kHeadDim);
  const float* hs = states + (size_t)unit * max_chunks * rec + (size_t)h * (2 + kHeadDim);
  int poison = 0;
  for (int c = d; c < nch; c += kHeadDim) {
    poison |= poisons[unit * max_chunks + c];
    ml[c][0] = hs[(size_t)c * rec];
    ml[c][1] = hs[(size_t)c * rec + 1];
  }
  const bool poisoned = __syncthreads_or(poison) != 0;
  float m = -__builtin_inff(), l = 0.0f, a = 0.0f;
  auto fold_one = [&](int c, float ac) {
    const float mc = ml[c][0], lc = ml[c][1];
    const float mn = fmaxf(m, mc);
    const float s0 = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    const float s1 = mc == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mc - mn);
    l = l * s0 + lc * s1;
    a = a * s0 + ac * s1;
    m = mn;
  };
  // whole batches with no exit inside (their loads all go out first), then the last one
  int c0 = 0;
  for (; c0 + kFoldBatch <= nch; c0 += kFoldBatch) {
    float ac[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) ac[i] = hs[(size_t)(c0 + i) * rec + 2 + d];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) fold_one(c0 + i, ac[i]);
  }
  if (c0 < nch) {
    float ac[kFoldBatch];
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) ac[i] = hs[(size_t)min(c0 + i, nch - 1) * rec + 2 + d];
    // the loads are used here, before any exit, so none of them waits for the previous step
    asm volatile("" ::"v"(ac[0]), "v"(ac[kFoldBatch / 2]), "v"(ac[kFoldBatch - 1]));
#pragma unroll
    for (int i = 0; i < kFoldBatch; ++i) {
      if (c0 + i >= nch) break;
      fold_one(c0 + i, ac[i]);
    }
  }
  float o = a / l;
  float lse = (m + __builtin_log2f(l)) * kLn2;
  if (poisoned) { o = __builtin_nanf(""); lse = __builtin_nanf(""); }
  P.out[(ri.head0 + h) * kHeadDim + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
  if (d == 0) P.lse[ri.head0 + h] = lse;
}

// KV heads per workgroup of the multi-CU and chunk schedules.  The KV heads of one (row, stream
// or chunk) share a workgroup when the grid is large enough (at least four wavefronts per compute
// unit): they walk the same pages and need the same cos/sin rows.  A smaller grid keeps one
// wavefront per workgroup and spreads over more compute units.  Where a wavefront runs never
// changes its bits.
int heads_per_workgroup(const DecodeParams& p, long long waves) {
  if (waves < 4LL * p.num_cus) return 1;
  if (p.num_kv_heads % 4 == 0) return 4;
  if (p.num_kv_heads % 2 == 0) return 2;
  return 1;
}

int max_chunks_of(int chunk_pages, int max_pages_per_row) {
  return (max_pages_per_row + chunk_pages - 1) / chunk_pages;
}

}  // namespace

size_t decode_workspace_bytes(int batch, int num_kv_heads, int group, int chunk_pages, int max_pages_per_row) {
  const size_t units = (size_t)batch * num_kv_heads;
  const size_t slots = chunk_pages > 0 ? (size_t)max_chunks_of(chunk_pages, max_pages_per_row) : (size_t)kStreams;
  return align256(units * slots * sizeof(int32_t)) + units * slots * group * (2 + kHeadDim) * sizeof(float);
}

hipError_t launch_decode(const DecodeParams& p, void* workspace, hipStream_t stream) {
  const unsigned units = (unsigned)p.batch * (unsigned)p.num_kv_heads;
  if (units == 0) return hipSuccess;
  if (p.chunk_pages > 0) {
    const int max_chunks = max_chunks_of(p.chunk_pages, p.max_pages_per_row);
    char* ws = (char*)workspace;
    int32_t* poisons = (int32_t*)ws;
    ws += align256((size_t)units * max_chunks * sizeof(int32_t));
    float* states = (float*)ws;
    const int hw = heads_per_workgroup(p, (long long)units * max_chunks);
    if (hw == 4)
      hipLaunchKernelGGL(decode_chunk_kernel<4>, dim3(units / 4 * (unsigned)max_chunks), dim3(256), 0, stream, p,
                         max_chunks, poisons, states);
    else if (hw == 2)
      hipLaunchKernelGGL(decode_chunk_kernel<2>, dim3(units / 2 * (unsigned)max_chunks), dim3(128), 0, stream, p,
                         max_chunks, poisons, states);
    else
      hipLaunchKernelGGL(decode_chunk_kernel<1>, dim3(units * (unsigned)max_chunks), dim3(64), 0, stream, p,
                         max_chunks, poisons, states);
    hipLaunchKernelGGL(decode_fold_kernel, dim3(units * (unsigned)p.group), dim3(kHeadDim), 0, stream, p, max_chunks,
                       (const int32_t*)poisons, (const float*)states);
  } else if (workspace == nullptr) {
    hipLaunchKernelGGL(decode_unit_kernel, dim3(units), dim3(kDecodeThreads), 0, stream, p);
  } else {
    char* ws = (char*)workspace;
    int32_t* poisons = (int32_t*)ws;
    ws += align256((size_t)units * kStreams * sizeof(int32_t));
    float* states = (float*)ws;
    const int hw = heads_per_workgroup(p, (long long)units * kStreams);
    if (hw == 4)
      hipLaunchKernelGGL(decode_stream_kernel<4>, dim3(units / 4 * kStreams), dim3(256), 0, stream, p, poisons, states);
    else if (hw == 2)
      hipLaunchKernelGGL(decode_stream_kernel<2>, dim3(units / 2 * kStreams), dim3(128), 0, stream, p, poisons, states);
    else
      hipLaunchKernelGGL(decode_stream_kernel<1>, dim3(units * kStreams), dim3(64), 0, stream, p, poisons, states);
    hipLaunchKernelGGL(decode_combine_kernel, dim3(units * (unsigned)p.group), dim3(kHeadDim), 0, stream, p,
                       (const int32_t*)poisons, (const float*)states);
  }
  return hipGetLastError();
}

}  // namespace pa

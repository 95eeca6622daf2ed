// Device-side validation of the paged-KV metadata, before execution.
//
// Rules (sources cited by page title and section):
//   "WS2 PR7 Fused Attention Backend Alignment", section "Original PR7 Requirements": the page
//   table, cache_position, query_position_ids, key_position_ids and logical token order are
//   validated before execution; section "Current Implementation": page bounds, logical
//   order, key positions, duplicate pages and non-canonical inactive rows are rejected,
//   cache_position must equal query_position_ids and query positions must be trailing and
//   contiguous ("FlashInfer RoPE Fusion").
//   "flashinfer_fa2 backend for NVIDIA Ada (SM89)", section "Code audit": indptr is the
//   cumulative page count starting at 0, empty rows carry last_page_len 1, and a row count
//   that does not match is rejected.
//
// Every violation is folded into one 64-bit minimum, (rule rank << 40) | element index, with
// atomicMin.  The minimum does not depend on thread order, so the report is deterministic:
// the first rule in rank order and, within it, the lowest offending element.
#include "pa_internal.h"

namespace pa {

namespace {

// rule ranks (report order)
enum : unsigned long long {
  kRankIndptr = 1,
  kRankCapacity = 2,
  kRankPageOob = 3,
  kRankDuplicate = 4,
  kRankLastPageLen = 5,
  kRankKeyPos = 6,
  kRankQueryPos = 7,
  kRankCachePos = 8,
};

__device__ __forceinline__ void flag(unsigned long long* report, unsigned long long rank, long long index) {
  atomicMin(report, (rank << 40) | (unsigned long long)index);
}

__global__ void clear_kernel(int32_t* count, int32_t n, unsigned long long* report) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) count[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) *report = ~0ull;
}

// Row-level rules: indptr shape, capacity, last_page_len, query and cache positions.
__global__ void rows_kernel(const ValidateParams P) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b <= P.batch; b += gridDim.x * blockDim.x) {
    if (b == 0 && P.indptr[0] != 0) flag(P.report, kRankIndptr, 0);
    if (b == P.batch) {
      if (P.indptr[b] != P.num_indices) flag(P.report, kRankIndptr, b);
      continue;
    }
    const int p0 = P.indptr[b], p1 = P.indptr[b + 1];
    if (p1 < p0 || p0 < 0 || p1 > P.num_indices) { flag(P.report, kRankIndptr, b + 1); continue; }
    const int n = p1 - p0;
    if (n > P.max_pages_per_row) flag(P.report, kRankCapacity, b);
    const int lpl = P.last_page_len[b];
    const bool lpl_ok = n > 0 ? (lpl >= 1 && lpl <= kPageSize) : lpl == 1;
    if (!lpl_ok) { flag(P.report, kRankLastPageLen, b); continue; }
    const long long L = n > 0 ? (long long)(n - 1) * kPageSize + lpl : 0;
    const long long base = (long long)b * P.q_len;
    const int q0 = P.qpos[base];
    for (int i = 0; i < P.q_len; ++i) {
      const int qi = P.qpos[base + i];
      if (qi != q0 + i || qi < 0) { flag(P.report, kRankQueryPos, base + i); break; }
    }
    const long long last = (long long)q0 + P.q_len - 1;
    if (last != L - 1 && last != L) flag(P.report, kRankQueryPos, base + P.q_len - 1);
    for (int i = 0; i < P.q_len; ++i)
      if (P.cache_position[base + i] != P.qpos[base + i]) { flag(P.report, kRankCachePos, base + i); break; }
  }
}

// Page bounds, and a count of every in-range page for the duplicate check.
__global__ void pages_kernel(const ValidateParams P) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < P.num_indices; i += gridDim.x * blockDim.x) {
    const int page = P.indices[i];
    if (page < 0 || page >= P.num_pages) flag(P.report, kRankPageOob, i);
    else atomicAdd(&P.page_count[page], 1);
  }
}

__global__ void duplicates_kernel(const ValidateParams P) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < P.num_indices; i += gridDim.x * blockDim.x) {
    const int page = P.indices[i];
    if (page >= 0 && page < P.num_pages && P.page_count[page] > 1) flag(P.report, kRankDuplicate, i);
  }
}

// key_position_ids of row b must read 0, 1, ..., L_b - 1 (logical order).  One block per row.
__global__ void keypos_kernel(const ValidateParams P) {
  const int b = blockIdx.x;
  const int p0 = P.indptr[b], p1 = P.indptr[b + 1];
  if (p1 < p0 || p0 < 0 || p1 > P.num_indices) return;  // reported by rows_kernel
  const int n = p1 - p0;
  const int lpl = P.last_page_len[b];
  if (n == 0 || lpl < 1 || lpl > kPageSize) return;
  const long long L = (long long)(n - 1) * kPageSize + lpl;
  const long long base = (long long)p0 * kPageSize;
  for (long long j = threadIdx.x; j < L; j += blockDim.x)
    if (P.kpos[base + j] != j) flag(P.report, kRankKeyPos, base + j);
}

}  // namespace

hipError_t launch_validate(const ValidateParams& p, hipStream_t stream) {
  const int threads = 256;
  auto blocks_for = [&](long long n) { return (unsigned)std::max(1LL, std::min(4096LL, (n + threads - 1) / threads)); };
  hipLaunchKernelGGL(clear_kernel, dim3(blocks_for(p.num_pages)), dim3(threads), 0, stream, p.page_count,
                     p.num_pages, p.report);
  hipLaunchKernelGGL(rows_kernel, dim3(blocks_for(p.batch + 1)), dim3(threads), 0, stream, p);
  if (p.num_indices > 0) {
    hipLaunchKernelGGL(pages_kernel, dim3(blocks_for(p.num_indices)), dim3(threads), 0, stream, p);
    hipLaunchKernelGGL(duplicates_kernel, dim3(blocks_for(p.num_indices)), dim3(threads), 0, stream, p);
  }
  if (p.batch > 0) hipLaunchKernelGGL(keypos_kernel, dim3(p.batch), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa

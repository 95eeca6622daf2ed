// Device-side construction of the CSR block table from a dense, -1-padded one.
//
// Source: "flashinfer_fa2 backend for NVIDIA Ada (SM89)", sections "Design notes" (the CSR
// metadata -- indptr, compact indices, last_page_len -- is built once per traversal with
// fixed shapes on the device; plans keyed by a width rounded up to a power of two) and
// "Code audit" / "Data flows checked" (indptr is the running sum of ceil(len / 16), the
// compact indices come from a fixed-shape scatter, rows without keys get last_page_len 1,
// and the construction must not synchronise the host).
//
// Two kernels, no host synchronisation, no memset (so the pair can be captured in a graph):
//  1. csr_rows_kernel (one workgroup): pages per row, their exclusive running sum (indptr)
//     and the keys in each row's last page.
//  2. csr_scatter_kernel: entry j < pages(b) of table row b goes to indices[indptr[b] + j];
//     the slots from indptr[B] to B * width - 1 get -1.  Every output slot is written by
//     exactly one thread.
// A row length outside [0, width * 16] cannot be represented: the row then takes its whole
// table row and last_page_len 0, which pa_validate_metadata reports and which the attention
// kernels turn into NaN for that row (the failure stays visible without a host read).
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kRowThreads = 1024;
constexpr int kScatterThreads = 256;

__device__ __forceinline__ bool len_ok(int L, int width) { return L >= 0 && L <= width * kPageSize; }

__device__ __forceinline__ int row_pages(int L, int width) {
  return len_ok(L, width) ? (L + kPageSize - 1) / kPageSize : width;
}

__device__ __forceinline__ int row_last(int L, int width) {
  if (!len_ok(L, width)) return 0;
  if (L == 0) return 1;
  return L - ((L + kPageSize - 1) / kPageSize - 1) * kPageSize;
}

__global__ __launch_bounds__(kRowThreads) void csr_rows_kernel(int batch, int width, const int32_t* __restrict__ lens,
                                                               int32_t* __restrict__ indptr,
                                                               int32_t* __restrict__ last) {
  __shared__ int32_t part[kRowThreads];
  const int t = threadIdx.x;
  // thread t owns rows [r0, r1): consecutive blocks, so the running sum stays in row order
  const int per = (batch + kRowThreads - 1) / kRowThreads;
  const int r0 = min(batch, t * per);
  const int r1 = min(batch, r0 + per);
  int own = 0;
  for (int b = r0; b < r1; ++b) own += row_pages(lens[b], width);
  part[t] = own;
  __syncthreads();
  // inclusive running sum over the threads (integer sums: exact)
  for (int off = 1; off < kRowThreads; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t > 0 ? part[t - 1] : 0;
  if (t == 0) indptr[0] = 0;
  for (int b = r0; b < r1; ++b) {
    const int L = lens[b];
    run += row_pages(L, width);
    indptr[b + 1] = run;
    last[b] = row_last(L, width);
  }
}

__global__ __launch_bounds__(kScatterThreads) void csr_scatter_kernel(int batch, int width,
                                                                      const int32_t* __restrict__ table,
                                                                      const int32_t* __restrict__ indptr,
                                                                      int32_t* __restrict__ indices) {
  const int total = batch * width;  // checked on the host to fit
  const int nnz = indptr[batch];
  for (int i = blockIdx.x * kScatterThreads + threadIdx.x; i < total; i += gridDim.x * kScatterThreads) {
    const int b = i / width;
    const int j = i - b * width;
    const int p0 = indptr[b];
    if (j < indptr[b + 1] - p0) indices[p0 + j] = table[i];
    if (i >= nnz) indices[i] = -1;
  }
}

}  // namespace

}  // namespace pa

extern "C" {

pa_status pa_build_csr(int32_t batch, int32_t width, const int32_t* block_table, const int32_t* kv_lens,
                       int32_t* kv_indptr, int32_t* kv_indices, int32_t* kv_last_page_len, void* stream) {
  using namespace pa;
  if (batch < 0 || width < 1 || width > INT32_MAX / kPageSize) return PA_ERR_INVALID_ARGUMENT;
  if ((int64_t)batch * width > INT32_MAX) return PA_ERR_INVALID_ARGUMENT;
  if (!kv_indptr) return PA_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (!block_table || !kv_lens || !kv_indices || !kv_last_page_len)) return PA_ERR_INVALID_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(csr_rows_kernel, dim3(1), dim3(kRowThreads), 0, s, batch, width, kv_lens, kv_indptr,
                     kv_last_page_len);
  const int total = batch * width;
  if (total > 0) {
    const int blocks = std::min((total + kScatterThreads - 1) / kScatterThreads, 4096);
    hipLaunchKernelGGL(csr_scatter_kernel, dim3(blocks), dim3(kScatterThreads), 0, s, batch, width, block_table,
                       (const int32_t*)kv_indptr, kv_indices);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_width_bucket(int32_t width, int32_t* bucket) {
  if (!bucket || width < 1 || width > (1 << 30)) return PA_ERR_INVALID_ARGUMENT;
  int32_t w = 1;
  while (w < width) w <<= 1;
  *bucket = w;
  return PA_OK;
}

}  // extern "C"

// Host side of the C ABI declared in include/pa.h: argument checks, the plan (with its RoPE
// table), validation and kernel launches.  pa_decode / pa_prefill only check host scalars
// and enqueue work: no allocation, no synchronisation, no device reads.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "pa_internal.h"

// Scratch of pa_decode_no_alloc: the multi-compute-unit decode workspace (per-stream or
// per-chunk softmax states and poison flags) in a file-scope device array, for callers that
// cannot allocate.  Each device holds its own copy until the process ends.  Host code never
// passes the array's name to a kernel (on the host it only stands for the symbol): its device
// address is looked up once per device and kept in g_scratch below.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

using namespace pa;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on `device`, which must be current; looked up on the first
// call for that device.  nullptr if the lookup fails.
void* scratch_on(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[device] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[device] = ptr;
  }
  return g_scratch[device];
}

bool plan_ok(pa_plan_t plan) { return plan != nullptr && plan->d_rope != nullptr; }

// The device a plan was made on must be current: its table lives there.
pa_status check_device(pa_plan_t plan) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  return dev == plan->device ? PA_OK : PA_ERR_INVALID_ARGUMENT;
}

// cos/sin of the RoPE angles: frequency i of position p has angle (p / scale) * theta^(-2i/D),
// formed and evaluated in float64 and rounded once to float32 ("WS2 PR7 Fused Attention
// Backend Alignment", section "FlashInfer RoPE Fusion": Llama RoPE, theta 1e6, scale 1.0,
// rotary_dim = head_dim).
//
// Layout (the order in which the kernels' lanes use the values): positions come in blocks of
// 16; block B holds [e = 0..7][lane = 0..63][4 floats], where lane = r + 16 g serves position
// 16 B + r for lane group g, and float c of entry e is
//   e = 0..3: cos of frequency f(e, g) + c,  e = 4..7: sin of frequency f(e - 4, g) + c,
//   f(q, g) = 8 g + 4 q (q = 0, 1),  32 + 8 g + 4 (q - 2) (q = 2, 3),
// i.e. a lane's 32 values are the cos and sin of its frequencies 8g..8g+7 and 32+8g..32+8g+7,
// the partners of its head dimensions 32 kb + 8 g + 0..7 in the rotate-half pairing.
std::vector<float> rope_table(int rows, double theta, double scale) {
  std::vector<double> inv_freq(kHalfDim);
  for (int i = 0; i < kHalfDim; ++i) inv_freq[i] = std::pow(theta, -(2.0 * i) / kHeadDim);
  const int blocks = (rows + kPageSize - 1) / kPageSize;
  std::vector<float> t((size_t)blocks * kRopeBlockFloats);
  for (int blk = 0; blk < blocks; ++blk)
    for (int e = 0; e < 8; ++e)
      for (int lane = 0; lane < 64; ++lane) {
        const int r = lane & 15, g = lane >> 4, q = e & 3;
        const double pos = (double)(blk * kPageSize + r) / scale;
        const int f0 = q < 2 ? 8 * g + 4 * q : 32 + 8 * g + 4 * (q - 2);
        float* dst = t.data() + (size_t)blk * kRopeBlockFloats + ((size_t)e * 64 + lane) * 4;
        for (int c = 0; c < 4; ++c) {
          const double a = pos * inv_freq[f0 + c];
          dst[c] = (float)(e < 4 ? std::cos(a) : std::sin(a));
        }
      }
  return t;
}

// Host-scalar checks shared by pa_decode and pa_prefill.
pa_status check_launch(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages, int32_t num_indices,
                       const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                       const int32_t* cache_position, const int32_t* query_position_ids,
                       const int32_t* key_position_ids, const void* q, const void* k_cache,
                       const void* v_cache, const void* out, const float* lse) {
  if (!plan_ok(plan)) return PA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || q_len < 1 || num_pages < 1 || num_indices < 0) return PA_ERR_INVALID_ARGUMENT;
  if (batch > plan->max_batch || q_len > plan->max_q_len) return PA_ERR_CAPACITY;
  if (batch == 0) return PA_OK;
  if (!kv_indptr || !kv_last_page_len || !cache_position || !query_position_ids || !q || !k_cache || !v_cache ||
      !out || !lse)
    return PA_ERR_INVALID_ARGUMENT;
  if (num_indices > 0 && (!kv_indices || !key_position_ids)) return PA_ERR_INVALID_ARGUMENT;
  return check_device(plan);
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY";
    case PA_ERR_HEAD_RATIO: return "PA_ERR_HEAD_RATIO";
    case PA_ERR_INDPTR: return "PA_ERR_INDPTR";
    case PA_ERR_PAGE_OOB: return "PA_ERR_PAGE_OOB";
    case PA_ERR_DUPLICATE_PAGE: return "PA_ERR_DUPLICATE_PAGE";
    case PA_ERR_LAST_PAGE_LEN: return "PA_ERR_LAST_PAGE_LEN";
    case PA_ERR_KEY_POSITION: return "PA_ERR_KEY_POSITION";
    case PA_ERR_QUERY_POSITION: return "PA_ERR_QUERY_POSITION";
    case PA_ERR_CACHE_POSITION: return "PA_ERR_CACHE_POSITION";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    default: return "PA_ERR_UNKNOWN";
  }
}

pa_status pa_plan(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                  int32_t max_batch, int32_t max_q_len, int32_t max_pages_per_row, float rope_theta,
                  float rope_scale, float rms_eps, int32_t split_policy, int32_t split_chunk_tokens,
                  pa_plan_t* plan_out) {
  if (!plan_out) return PA_ERR_INVALID_ARGUMENT;
  if (num_q_heads < 1 || num_kv_heads < 1 || max_batch < 1 || max_q_len < 1 || max_pages_per_row < 1)
    return PA_ERR_INVALID_ARGUMENT;
  if (!(rms_eps > 0.0f) || !std::isfinite(rms_eps)) return PA_ERR_INVALID_ARGUMENT;
  if (head_dim != kHeadDim || page_size != kPageSize) return PA_ERR_UNSUPPORTED;
  if (rope_theta != 1.0e6f || rope_scale != 1.0f) return PA_ERR_UNSUPPORTED;
  if (split_policy != PA_SPLIT_DISABLED && split_policy != PA_SPLIT_FIXED) return PA_ERR_UNSUPPORTED;
  if (split_policy == PA_SPLIT_FIXED && (split_chunk_tokens < kPageSize || split_chunk_tokens % kPageSize != 0))
    return PA_ERR_UNSUPPORTED;
  // the chunk states of a row are folded through an LDS table of kMaxFixedChunks entries
  if (split_policy == PA_SPLIT_FIXED &&
      ((long long)max_pages_per_row + split_chunk_tokens / kPageSize - 1) / (split_chunk_tokens / kPageSize) >
          kMaxFixedChunks)
    return PA_ERR_CAPACITY;
  if (num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > kMaxGroup) return PA_ERR_HEAD_RATIO;
  // positions stay int32 and the table below fits in memory
  if ((long long)max_pages_per_row * kPageSize + 1 > (1LL << 24)) return PA_ERR_CAPACITY;
  // (row, KV head) units and their streams index int32 arrays and grids
  if ((long long)max_batch * num_kv_heads > (1LL << 24)) return PA_ERR_CAPACITY;

  pa_plan_s* p = new (std::nothrow) pa_plan_s();
  if (!p) return PA_ERR_HIP;
  p->num_q_heads = num_q_heads;
  p->num_kv_heads = num_kv_heads;
  p->group = num_q_heads / num_kv_heads;
  p->max_batch = max_batch;
  p->max_q_len = max_q_len;
  p->max_pages_per_row = max_pages_per_row;
  p->table_rows = max_pages_per_row * kPageSize + 1;
  p->rope_theta = rope_theta;
  p->rope_scale = rope_scale;
  p->rms_eps = rms_eps;
  p->split_policy = split_policy;
  p->split_chunk_pages = split_policy == PA_SPLIT_FIXED ? split_chunk_tokens / kPageSize : 0;
  p->d_rope = nullptr;
  if (hipGetDevice(&p->device) != hipSuccess) { delete p; return PA_ERR_HIP; }
  if (hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device) != hipSuccess ||
      p->num_cus < 1) {
    delete p;
    return PA_ERR_HIP;
  }
  // set-up of pa_decode_no_alloc's scratch on this device (the device is current here)
  if (scratch_on(p->device) == nullptr) { delete p; return PA_ERR_HIP; }
  const std::vector<float> table = rope_table(p->table_rows, (double)rope_theta, (double)rope_scale);
  const size_t bytes = table.size() * sizeof(float);
  if (hipMalloc(&p->d_rope, bytes) != hipSuccess) { delete p; return PA_ERR_HIP; }
  if (hipMemcpy(p->d_rope, table.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p->d_rope);
    delete p;
    return PA_ERR_HIP;
  }
  *plan_out = p;
  return PA_OK;
}

pa_status pa_plan_destroy(pa_plan_t plan) {
  if (!plan) return PA_OK;
  pa_status st = PA_OK;
  if (plan->d_rope && hipFree(plan->d_rope) != hipSuccess) st = PA_ERR_HIP;
  delete plan;
  return st;
}

pa_status pa_validate_metadata(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages,
                               int32_t num_indices, const int32_t* kv_indptr, const int32_t* kv_indices,
                               const int32_t* kv_last_page_len, const int32_t* cache_position,
                               const int32_t* query_position_ids, const int32_t* key_position_ids,
                               void* stream, pa_validation_report* report) {
  pa_validation_report rep = {PA_OK, -1, -1, -1};
  auto finish = [&](pa_status st) {
    rep.code = st;
    if (report) *report = rep;
    return st;
  };
  if (!plan_ok(plan)) return finish(PA_ERR_INVALID_ARGUMENT);
  if (batch < 0 || q_len < 1 || num_pages < 1 || num_indices < 0) return finish(PA_ERR_INVALID_ARGUMENT);
  if (batch > plan->max_batch || q_len > plan->max_q_len) return finish(PA_ERR_CAPACITY);
  if (!kv_indptr || !kv_last_page_len || !cache_position || !query_position_ids || !key_position_ids ||
      (num_indices > 0 && !kv_indices))
    return finish(PA_ERR_INVALID_ARGUMENT);
  if (check_device(plan) != PA_OK) return finish(PA_ERR_INVALID_ARGUMENT);
  hipStream_t s = (hipStream_t)stream;

  void* scratch = nullptr;
  const size_t bytes = sizeof(unsigned long long) + (size_t)num_pages * sizeof(int32_t);
  if (hipMalloc(&scratch, bytes) != hipSuccess) return finish(PA_ERR_HIP);
  ValidateParams vp;
  vp.batch = batch;
  vp.q_len = q_len;
  vp.num_pages = num_pages;
  vp.num_indices = num_indices;
  vp.max_pages_per_row = plan->max_pages_per_row;
  vp.indptr = kv_indptr;
  vp.indices = kv_indices;
  vp.last_page_len = kv_last_page_len;
  vp.cache_position = cache_position;
  vp.qpos = query_position_ids;
  vp.kpos = key_position_ids;
  vp.report = (unsigned long long*)scratch;
  vp.page_count = (int32_t*)((char*)scratch + sizeof(unsigned long long));
  unsigned long long key = ~0ull;
  hipError_t e = launch_validate(vp, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&key, vp.report, sizeof(key), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  pa_status st = PA_OK;
  if (e != hipSuccess) {
    st = PA_ERR_HIP;
  } else if (key != ~0ull) {
    static const pa_status by_rank[] = {PA_OK, PA_ERR_INDPTR, PA_ERR_CAPACITY, PA_ERR_PAGE_OOB,
                                        PA_ERR_DUPLICATE_PAGE, PA_ERR_LAST_PAGE_LEN, PA_ERR_KEY_POSITION,
                                        PA_ERR_QUERY_POSITION, PA_ERR_CACHE_POSITION};
    const unsigned rank = (unsigned)(key >> 40);
    const long long index = (long long)(key & ((1ull << 40) - 1));
    st = rank < sizeof(by_rank) / sizeof(by_rank[0]) ? by_rank[rank] : PA_ERR_HIP;
    rep.index = index;
    // the row and the offending value, read back for the report
    const int32_t* src = nullptr;
    switch (st) {
      case PA_ERR_INDPTR: src = kv_indptr; rep.row = (int32_t)std::max(0LL, index - 1); break;
      case PA_ERR_CAPACITY: case PA_ERR_LAST_PAGE_LEN: src = kv_last_page_len; rep.row = (int32_t)index; break;
      case PA_ERR_PAGE_OOB: case PA_ERR_DUPLICATE_PAGE: src = kv_indices; break;
      case PA_ERR_KEY_POSITION: src = key_position_ids; break;
      case PA_ERR_QUERY_POSITION: src = query_position_ids; rep.row = (int32_t)(index / q_len); break;
      case PA_ERR_CACHE_POSITION: src = cache_position; rep.row = (int32_t)(index / q_len); break;
      default: break;
    }
    if (st == PA_ERR_CAPACITY) {
      int32_t pr[2];
      if (hipMemcpy(pr, kv_indptr + index, sizeof(pr), hipMemcpyDeviceToHost) == hipSuccess)
        rep.value = pr[1] - pr[0];
    } else if (src) {
      int32_t v = 0;
      if (hipMemcpy(&v, src + index, sizeof(v), hipMemcpyDeviceToHost) == hipSuccess) rep.value = v;
    }
    if (st == PA_ERR_PAGE_OOB || st == PA_ERR_DUPLICATE_PAGE || st == PA_ERR_KEY_POSITION) {
      // row owning the element: indptr is valid here (indptr violations rank first)
      std::vector<int32_t> indptr(batch + 1);
      if (hipMemcpy(indptr.data(), kv_indptr, sizeof(int32_t) * (batch + 1), hipMemcpyDeviceToHost) == hipSuccess) {
        const long long page_elem = st == PA_ERR_KEY_POSITION ? index / kPageSize : index;
        const auto it = std::upper_bound(indptr.begin(), indptr.end(), (int32_t)page_elem);
        rep.row = (int32_t)(it - indptr.begin()) - 1;
      }
    }
  }
  if (hipFree(scratch) != hipSuccess && st == PA_OK) st = PA_ERR_HIP;
  return finish(st);
}

}  // extern "C"

namespace {

// Shared body of pa_decode and pa_decode_no_alloc: `workspace` is the caller's buffer, the
// scratch array's device address, or NULL (one workgroup per unit).
pa_status decode_call(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages, int32_t num_indices,
                      const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                      const int32_t* cache_position, const int32_t* query_position_ids,
                      const int32_t* key_position_ids, const void* q, const void* k_cache, const void* v_cache,
                      const float* q_norm_weight, const float* k_norm_weight, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = check_launch(plan, batch, q_len, num_pages, num_indices, kv_indptr, kv_indices,
                              kv_last_page_len, cache_position, query_position_ids, key_position_ids, q,
                              k_cache, v_cache, out, lse);
  if (st != PA_OK || batch == 0) return st;
  if (q_len != 1) return PA_ERR_INVALID_ARGUMENT;
  const size_t need = decode_workspace_bytes(batch, plan->num_kv_heads, plan->group, plan->split_chunk_pages,
                                             plan->max_pages_per_row);
  if (plan->split_chunk_pages > 0 && !workspace) return PA_ERR_WORKSPACE;
  if (workspace && workspace_bytes < need) return PA_ERR_WORKSPACE;
  DecodeParams p;
  p.batch = batch;
  p.num_q_heads = plan->num_q_heads;
  p.num_kv_heads = plan->num_kv_heads;
  p.group = plan->group;
  p.num_pages = num_pages;
  p.num_indices = num_indices;
  p.max_pages_per_row = plan->max_pages_per_row;
  p.table_rows = plan->table_rows;
  p.indptr = kv_indptr;
  p.indices = kv_indices;
  p.last_page_len = kv_last_page_len;
  p.cache_position = cache_position;
  p.qpos = query_position_ids;
  p.kpos = key_position_ids;
  p.q = (const uint16_t*)q;
  p.k_cache = (const uint16_t*)k_cache;
  p.v_cache = (const uint16_t*)v_cache;
  p.q_norm = q_norm_weight;
  p.k_norm = k_norm_weight;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.rope = plan->d_rope;
  p.eps = plan->rms_eps;
  p.chunk_pages = plan->split_chunk_pages;
  p.num_cus = plan->num_cus;
  return launch_decode(p, workspace, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

pa_status pa_decode(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages, int32_t num_indices,
                    const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                    const int32_t* cache_position, const int32_t* query_position_ids,
                    const int32_t* key_position_ids, const void* q, const void* k_cache, const void* v_cache,
                    const float* q_norm_weight, const float* k_norm_weight, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(plan, batch, q_len, num_pages, num_indices, kv_indptr, kv_indices, kv_last_page_len,
                     cache_position, query_position_ids, key_position_ids, q, k_cache, v_cache, q_norm_weight,
                     k_norm_weight, out, lse, workspace, workspace_bytes, stream);
}

pa_status pa_decode_no_alloc(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages, int32_t num_indices,
                             const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                             const int32_t* cache_position, const int32_t* query_position_ids,
                             const int32_t* key_position_ids, const void* q, const void* k_cache,
                             const void* v_cache, const float* q_norm_weight, const float* k_norm_weight,
                             void* out, float* lse, void* stream) {
  if (!plan_ok(plan)) return PA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || batch > plan->max_batch) return batch < 0 ? PA_ERR_INVALID_ARGUMENT : PA_ERR_CAPACITY;
  if (decode_workspace_bytes(batch, plan->num_kv_heads, plan->group, plan->split_chunk_pages,
                             plan->max_pages_per_row) > kNoAllocScratchBytes)
    return PA_ERR_CAPACITY;
  void* ws = scratch_on(plan->device);
  if (ws == nullptr) return PA_ERR_HIP;
  return decode_call(plan, batch, q_len, num_pages, num_indices, kv_indptr, kv_indices, kv_last_page_len,
                     cache_position, query_position_ids, key_position_ids, q, k_cache, v_cache, q_norm_weight,
                     k_norm_weight, out, lse, ws, kNoAllocScratchBytes, stream);
}

pa_status pa_decode_workspace_size(pa_plan_t plan, int32_t batch, size_t* bytes) {
  if (!plan_ok(plan) || !bytes || batch < 0) return PA_ERR_INVALID_ARGUMENT;
  if (batch > plan->max_batch) return PA_ERR_CAPACITY;
  *bytes = decode_workspace_bytes(batch, plan->num_kv_heads, plan->group, plan->split_chunk_pages,
                                  plan->max_pages_per_row);
  return PA_OK;
}

pa_status pa_prefill_workspace_size(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_indices,
                                    size_t* bytes) {
  if (!plan_ok(plan) || !bytes || batch < 0 || q_len < 1 || num_indices < 0) return PA_ERR_INVALID_ARGUMENT;
  if (batch > plan->max_batch || q_len > plan->max_q_len) return PA_ERR_CAPACITY;
  *bytes = prefill_workspace_bytes(plan->num_q_heads, plan->num_kv_heads, batch, q_len, num_indices);
  return PA_OK;
}

pa_status pa_prefill(pa_plan_t plan, int32_t batch, int32_t q_len, int32_t num_pages, int32_t num_indices,
                     const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                     const int32_t* cache_position, const int32_t* query_position_ids,
                     const int32_t* key_position_ids, const void* q, const void* k_cache, const void* v_cache,
                     const float* q_norm_weight, const float* k_norm_weight, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = check_launch(plan, batch, q_len, num_pages, num_indices, kv_indptr, kv_indices,
                              kv_last_page_len, cache_position, query_position_ids, key_position_ids, q,
                              k_cache, v_cache, out, lse);
  if (st != PA_OK || batch == 0) return st;
  if (plan->split_policy != PA_SPLIT_DISABLED) return PA_ERR_UNSUPPORTED;  // prefill: one pass per row only
  const size_t need = prefill_workspace_bytes(plan->num_q_heads, plan->num_kv_heads, batch, q_len, num_indices);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  PrefillParams p;
  p.batch = batch;
  p.q_len = q_len;
  p.num_q_heads = plan->num_q_heads;
  p.num_kv_heads = plan->num_kv_heads;
  p.group = plan->group;
  p.num_pages = num_pages;
  p.num_indices = num_indices;
  p.max_pages_per_row = plan->max_pages_per_row;
  p.table_rows = plan->table_rows;
  p.indptr = kv_indptr;
  p.indices = kv_indices;
  p.last_page_len = kv_last_page_len;
  p.cache_position = cache_position;
  p.qpos = query_position_ids;
  p.kpos = key_position_ids;
  p.q = (const uint16_t*)q;
  p.k_cache = (const uint16_t*)k_cache;
  p.v_cache = (const uint16_t*)v_cache;
  p.q_norm = q_norm_weight;
  p.k_norm = k_norm_weight;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.rope = plan->d_rope;
  p.eps = plan->rms_eps;
  p.num_cus = plan->num_cus;
  p.workspace = workspace;
  return launch_prefill(p, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_prefill_backward_workspace_size(pa_plan_t plan, int32_t batch, int32_t seq_len, size_t* bytes) {
  if (!plan_ok(plan) || !bytes || batch < 0 || seq_len < 1) return PA_ERR_INVALID_ARGUMENT;
  if (batch > plan->max_batch || seq_len > plan->max_q_len) return PA_ERR_CAPACITY;
  *bytes = backward_workspace_bytes(batch, seq_len, plan->num_q_heads, plan->num_kv_heads);
  return PA_OK;
}

pa_status pa_prefill_backward(pa_plan_t plan, int32_t batch, int32_t seq_len, const int32_t* positions,
                              const void* q, const void* k, const void* v, const float* q_norm_weight,
                              const float* k_norm_weight, const void* out, const float* lse, const void* dout,
                              float* dq, float* dk, float* dv, float* dq_norm_weight, float* dk_norm_weight,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan_ok(plan)) return PA_ERR_INVALID_ARGUMENT;
  if (batch < 0 || seq_len < 1) return PA_ERR_INVALID_ARGUMENT;
  if (batch > plan->max_batch || seq_len > plan->max_q_len) return PA_ERR_CAPACITY;
  if (plan->split_policy != PA_SPLIT_DISABLED) return PA_ERR_UNSUPPORTED;
  if (batch == 0) return PA_OK;
  if (!positions || !q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return PA_ERR_INVALID_ARGUMENT;
  if ((q_norm_weight && !dq_norm_weight) || (k_norm_weight && !dk_norm_weight)) return PA_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < backward_workspace_bytes(batch, seq_len, plan->num_q_heads, plan->num_kv_heads))
    return PA_ERR_WORKSPACE;
  pa_status st = check_device(plan);
  if (st != PA_OK) return st;
  BackwardArgs a;
  a.batch = batch;
  a.seq = seq_len;
  a.num_q_heads = plan->num_q_heads;
  a.num_kv_heads = plan->num_kv_heads;
  a.table_rows = plan->table_rows;
  a.positions = positions;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.q_norm = q_norm_weight;
  a.k_norm = k_norm_weight;
  a.rope = plan->d_rope;
  a.eps = plan->rms_eps;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq_norm = dq_norm_weight;
  a.dk_norm = dk_norm_weight;
  a.workspace = workspace;
  return launch_backward(a, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"

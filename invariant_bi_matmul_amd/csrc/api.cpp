// extern "C" entry points of libbi.so (declared and documented in bi.h).
//
// Every entry point checks its host arguments completely before it enqueues
// anything, then launches on the caller's stream.  Nothing here allocates or
// synchronises; the one piece of state is bi_attn_decode_noalloc's scratch
// array and its per-device address table.
//
// Built with BI_DEBUG_CHECKS (libbi_debug.so), the attention entry points
// also validate the device index arrays before they launch anything: a
// check kernel reads kv_len, cu_q and the block table, the stream is
// synchronised, and a bad entry returns BI_ERR_INVALID_SHAPE with nothing
// else enqueued.  That build allocates one int per device for the result
// (once) and cannot run under stream capture.
#include "bi.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "kernels.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bi_status hip_status(hipError_t e) { return e == hipSuccess ? BI_OK : BI_ERR_HIP; }

constexpr int64_t kMaxGridX = 0x7fffffff;
constexpr int64_t kMaxGridYZ = 65535;

// Checks shared by the attention entry points.
int check_attn_shape(const bi_attn_shape* s) {
  if (s == nullptr) return BI_ERR_NULL_POINTER;
  if (s->num_seqs < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->head_dim <= 0 ||
      s->max_pages_per_seq <= 0 || s->num_pages <= 0)
    return BI_ERR_INVALID_SHAPE;
  if (s->num_q_heads % s->num_kv_heads != 0) return BI_ERR_INVALID_SHAPE;
  const int group = s->num_q_heads / s->num_kv_heads;
  if (group > 16 || (16 % group) != 0) return BI_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return BI_ERR_UNSUPPORTED;
  if (s->page_size != bi::kPage) return BI_ERR_UNSUPPORTED;
  if (!(s->softmax_scale > 0.0f) || !isfinite(s->softmax_scale)) return BI_ERR_INVALID_SHAPE;
  if (s->num_seqs > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

bi::AttnDims dims_of(const bi_attn_shape* s) {
  return bi::AttnDims{s->num_seqs, s->num_q_heads, s->num_kv_heads, s->head_dim,
                      s->max_pages_per_seq, s->softmax_scale};
}

#ifdef BI_DEBUG_CHECKS
// Validate the index arrays of an attention call (see checks.hip); BI_OK,
// BI_ERR_INVALID_SHAPE, or BI_ERR_HIP.
int debug_check_tables(const bi_attn_shape* s, const int32_t* kv_len, const int32_t* cu_q,
                       const int32_t* bt, int max_len, int max_q, int64_t total_q,
                       hipStream_t st) {
  static int* flags[64] = {};  // one device int per device, allocated once
  static std::mutex alloc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BI_ERR_HIP;
  {
    std::lock_guard<std::mutex> lock(alloc);
    if (flags[dev] == nullptr && hipMalloc((void**)&flags[dev], sizeof(int)) != hipSuccess)
      return BI_ERR_HIP;
  }
  if (bi::launch_check_attn_tables(kv_len, cu_q, bt, s->num_seqs, s->max_pages_per_seq,
                                   s->num_pages, max_len, max_q, total_q, flags[dev], st) !=
      hipSuccess)
    return BI_ERR_HIP;
  int bad = 0;
  if (hipMemcpyAsync(&bad, flags[dev], sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return BI_ERR_HIP;
  return bad == 0 ? BI_OK : BI_ERR_INVALID_SHAPE;
}
#define BI_CHECK_TABLES(...)                          \
  do {                                                \
    const int chk = debug_check_tables(__VA_ARGS__); \
    if (chk != BI_OK) return (bi_status)chk;         \
  } while (0)
#else
#define BI_CHECK_TABLES(...) \
  do {                       \
  } while (0)
#endif

size_t decode_ws_bytes(const bi_attn_shape* s, int64_t tokens, int64_t nsplit) {
  return (size_t)tokens * (size_t)s->num_q_heads * (size_t)nsplit *
         (size_t)bi::attn_rec_floats(s->head_dim) * sizeof(float);
}

}  // namespace

extern "C" {

int bi_abi_version(void) { return BI_ABI_VERSION; }

const char* bi_status_string(int status) {
  switch (status) {
    case BI_OK: return "ok";
    case BI_ERR_NULL_POINTER: return "a required pointer is NULL";
    case BI_ERR_INVALID_SHAPE: return "invalid or inconsistent sizes, or a misaligned pointer";
    case BI_ERR_UNSUPPORTED: return "outside the one compiled configuration";
    case BI_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than required";
    case BI_ERR_HIP: return "the HIP runtime refused a launch";
    case BI_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

// ---------------------------------------------------------------------------
static int check_rmsnorm(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
                         int64_t hidden) {
  if (rows < 0 || hidden < 0) return BI_ERR_INVALID_SHAPE;
  if (hidden % 8 != 0 || hidden < 8 || hidden > 16384) return BI_ERR_UNSUPPORTED;
  if (rows > kMaxGridX) return BI_ERR_UNSUPPORTED;
  if (rows == 0) return -1;  // no-op
  if (x == nullptr || gamma == nullptr || y == nullptr) return BI_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(y) || !aligned4(rstd))
    return BI_ERR_INVALID_SHAPE;
  return BI_OK;
}

bi_status bi_rmsnorm(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
               int64_t hidden, float eps, void* stream) {
  try {
    const int c = check_rmsnorm(x, gamma, y, rstd, rows, hidden);
    if (c < 0) return BI_OK;
    if (c != BI_OK) return (bi_status)c;
    if (!(eps >= 0.0f) || !isfinite(eps)) return BI_ERR_INVALID_SHAPE;
    return hip_status(
        bi::launch_rmsnorm(x, gamma, y, rstd, rows, (int)hidden, eps, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bix_rmsnorm_splitrow(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
                         int64_t hidden, float eps, int32_t chunks, void* workspace,
                         size_t workspace_bytes, void* stream) {
  try {
    const int c = check_rmsnorm(x, gamma, y, rstd, rows, hidden);
    if (c < 0) return BI_OK;
    if (c != BI_OK) return (bi_status)c;
    if (!(eps >= 0.0f) || !isfinite(eps)) return BI_ERR_INVALID_SHAPE;
    if (chunks <= 0) chunks = bi::rmsnorm_splitrow_auto_chunks(rows);
    if (chunks > 64 || chunks > hidden / 8) return BI_ERR_UNSUPPORTED;
    if (workspace == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned4(workspace)) return BI_ERR_INVALID_SHAPE;
    if (workspace_bytes < (size_t)rows * 64 * sizeof(float)) return BI_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(bi::launch_rmsnorm_splitrow(x, gamma, y, rstd, rows, (int)hidden, eps,
                                                  chunks, (float*)workspace,
                                                  (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

// ---------------------------------------------------------------------------
static int check_matmul(const void* a, const void* w, void* c, int c_dtype, int64_t m, int64_t n,
                        int64_t k) {
  if (m < 0 || n < 0 || k < 0) return BI_ERR_INVALID_SHAPE;
  if (c_dtype != BI_DTYPE_BF16 && c_dtype != BI_DTYPE_F32) return BI_ERR_INVALID_SHAPE;
  if (k % bi::kMatmulBK != 0 || n % 8 != 0) return BI_ERR_UNSUPPORTED;
  if (m > 0x7fffffff || n > 0x7fffffff || k > 0x7fffffff) return BI_ERR_UNSUPPORTED;
  // per-thread load offsets inside a 256-row / 64-k-row tile are 32-bit
  if (k > (int64_t)1 << 22 || n > (int64_t)1 << 24) return BI_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return -1;
  if (((m + 255) / 256) * ((n + 255) / 256) > kMaxGridX) return BI_ERR_UNSUPPORTED;
  if (c == nullptr || (k > 0 && (a == nullptr || w == nullptr))) return BI_ERR_NULL_POINTER;
  if (!aligned16(a) || !aligned16(w) || !aligned16(c)) return BI_ERR_INVALID_SHAPE;
  return BI_OK;
}

bi_status bi_matmul(const void* a, const void* w, void* c, int c_dtype, int64_t m, int64_t n, int64_t k,
              void* stream) {
  try {
    const int s = check_matmul(a, w, c, c_dtype, m, n, k);
    if (s < 0) return BI_OK;
    if (s != BI_OK) return (bi_status)s;
    return hip_status(
        bi::launch_matmul(a, w, c, c_dtype == BI_DTYPE_F32, m, n, k, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_matmul_pack_w(const void* w, void* wp, int64_t k, int64_t n, void* stream) {
  try {
    if (k < 0 || n < 0) return BI_ERR_INVALID_SHAPE;
    if (n % 32 != 0 || k > (int64_t)1 << 22 || n > (int64_t)1 << 24) return BI_ERR_UNSUPPORTED;
    if (k == 0 || n == 0) return BI_OK;
    if (w == nullptr || wp == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(w) || !aligned16(wp)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_matmul_pack_w(w, wp, k, n, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_matmul_packed(const void* a, const void* wp, void* c, int c_dtype, int64_t m,
                           int64_t n, int64_t k, void* stream) {
  try {
    const int s = check_matmul(a, wp, c, c_dtype, m, n, k);
    if (s < 0) return BI_OK;
    if (s != BI_OK) return (bi_status)s;
    if (n % 32 != 0) return BI_ERR_UNSUPPORTED;
    return hip_status(bi::launch_matmul(a, wp, c, c_dtype == BI_DTYPE_F32, m, n, k,
                                        (hipStream_t)stream, true));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bix_matmul_tile(int64_t m, int64_t n, int32_t* tile_m, int32_t* tile_n, int64_t* workgroups) {
  if (m < 1 || n < 1) return BI_ERR_INVALID_SHAPE;
  int bm, bn;
  int64_t grid;
  bi::matmul_tile(m, n, &bm, &bn, &grid);
  if (tile_m != nullptr) *tile_m = bm;
  if (tile_n != nullptr) *tile_n = bn;
  if (workgroups != nullptr) *workgroups = grid;
  return BI_OK;
}

size_t bix_matmul_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t split_k) {
  if (m < 0 || n < 0 || k < 0 || k % bi::kMatmulBK != 0) return 0;
  if (split_k <= 0) split_k = bi::matmul_splitk_auto(m, n, k);
  if (split_k < 1) split_k = 1;
  return (size_t)split_k * (size_t)m * (size_t)n * sizeof(float);
}

static bi_status matmul_splitk(const void* a, const void* w, void* c, int c_dtype, int64_t m,
                               int64_t n, int64_t k, int32_t split_k, void* workspace,
                               size_t workspace_bytes, void* stream, bool packed) {
  try {
    const int s = check_matmul(a, w, c, c_dtype, m, n, k);
    if (s < 0) return BI_OK;
    if (s != BI_OK) return (bi_status)s;
    if (packed && n % 32 != 0) return BI_ERR_UNSUPPORTED;
    if (k == 0) return BI_ERR_UNSUPPORTED;
    if (split_k <= 0) split_k = bi::matmul_splitk_auto(m, n, k);
    if (split_k > k / bi::kMatmulBK || split_k > 65535) return BI_ERR_UNSUPPORTED;
    if (workspace == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(workspace)) return BI_ERR_INVALID_SHAPE;
    if (workspace_bytes < (size_t)split_k * (size_t)m * (size_t)n * sizeof(float))
      return BI_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(bi::launch_matmul_splitk(a, w, c, c_dtype == BI_DTYPE_F32, m, n, k, split_k,
                                               (float*)workspace, (hipStream_t)stream, packed));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bix_matmul_splitk(const void* a, const void* w, void* c, int c_dtype, int64_t m,
                            int64_t n, int64_t k, int32_t split_k, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return matmul_splitk(a, w, c, c_dtype, m, n, k, split_k, workspace, workspace_bytes, stream,
                       false);
}

bi_status bix_matmul_splitk_packed(const void* a, const void* wp, void* c, int c_dtype, int64_t m,
                                   int64_t n, int64_t k, int32_t split_k, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return matmul_splitk(a, wp, c, c_dtype, m, n, k, split_k, workspace, workspace_bytes, stream,
                       true);
}

// ---------------------------------------------------------------------------
size_t bi_attn_workspace_bytes(const bi_attn_shape* s, int64_t num_tokens, int32_t max_kv_len) {
  if (check_attn_shape(s) != BI_OK || num_tokens < 0 || max_kv_len < 0) return 0;
  const int64_t ns = ((int64_t)max_kv_len + bi::kSplit - 1) / bi::kSplit;
  return decode_ws_bytes(s, num_tokens, ns > 0 ? ns : 1);
}

bi_status bi_attn_prefill(const bi_attn_shape* s, const void* q, const void* k_new, const void* v_new,
                    const int32_t* cu_q, const int32_t* kv_len, const int32_t* block_table,
                    void* k_cache, void* v_cache, void* out, float* lse, int64_t total_q,
                    int32_t max_q_per_seq, void* stream) {
  try {
    const int c = check_attn_shape(s);
    if (c != BI_OK) return (bi_status)c;
    if (total_q < 0 || max_q_per_seq < 0) return BI_ERR_INVALID_SHAPE;
    if (s->num_seqs == 0 || total_q == 0 || max_q_per_seq == 0) return BI_OK;
    if (max_q_per_seq > total_q) return BI_ERR_INVALID_SHAPE;
    if (max_q_per_seq > (int64_t)s->max_pages_per_seq * s->page_size) return BI_ERR_INVALID_SHAPE;
    if (total_q > kMaxGridX) return BI_ERR_UNSUPPORTED;
    if (!q || !k_new || !v_new || !cu_q || !kv_len || !block_table || !k_cache || !v_cache || !out)
      return BI_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out) || !aligned4(lse) || !aligned4(cu_q) ||
        !aligned4(kv_len) || !aligned4(block_table))
      return BI_ERR_INVALID_SHAPE;
    const bi::AttnDims d = dims_of(s);
    const hipStream_t st = (hipStream_t)stream;
    BI_CHECK_TABLES(s, kv_len, cu_q, block_table, s->max_pages_per_seq * s->page_size,
                    max_q_per_seq, total_q, st);
    hipError_t e = bi::launch_kv_append(d, k_new, v_new, cu_q, kv_len, block_table, k_cache,
                                        v_cache, max_q_per_seq, st);
    if (e != hipSuccess) return BI_ERR_HIP;
    return hip_status(bi::launch_attn_prefill(d, q, cu_q, kv_len, block_table, k_cache, v_cache,
                                              out, lse, max_q_per_seq, st));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

static int check_decode(const bi_attn_shape* s, const void* q, const void* k_new,
                        const void* v_new, const int32_t* kv_len, const int32_t* block_table,
                        void* k_cache, void* v_cache, void* out, float* lse, int32_t max_kv_len,
                        void* workspace) {
  const int c = check_attn_shape(s);
  if (c != BI_OK) return (bi_status)c;
  if (max_kv_len < 0) return BI_ERR_INVALID_SHAPE;
  if (s->num_seqs == 0) return -1;
  if (max_kv_len < 1 || max_kv_len > (int64_t)s->max_pages_per_seq * s->page_size)
    return BI_ERR_INVALID_SHAPE;
  if (!q || !k_new || !v_new || !kv_len || !block_table || !k_cache || !v_cache || !out ||
      !workspace)
    return BI_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned4(lse) || !aligned4(kv_len) ||
      !aligned4(block_table) || !aligned16(workspace))
    return BI_ERR_INVALID_SHAPE;
  return BI_OK;
}

bi_status bi_attn_decode(const bi_attn_shape* s, const void* q, const void* k_new, const void* v_new,
                   const int32_t* kv_len, const int32_t* block_table, void* k_cache,
                   void* v_cache, void* out, float* lse, int32_t max_kv_len, void* workspace,
                   size_t workspace_bytes, void* stream) {
  try {
    const int c = check_decode(s, q, k_new, v_new, kv_len, block_table, k_cache, v_cache, out, lse,
                               max_kv_len, workspace);
    if (c < 0) return BI_OK;
    if (c != BI_OK) return (bi_status)c;
    const int ns = (max_kv_len + bi::kSplit - 1) / bi::kSplit;
    if (workspace_bytes < decode_ws_bytes(s, s->num_seqs, ns)) return BI_ERR_WORKSPACE_TOO_SMALL;
    if ((int64_t)s->num_seqs * s->num_kv_heads * ns / 4 + 1 > kMaxGridX) return BI_ERR_UNSUPPORTED;
    const bi::AttnDims d = dims_of(s);
    const hipStream_t st = (hipStream_t)stream;
    BI_CHECK_TABLES(s, kv_len, nullptr, block_table, max_kv_len, 1, 0, st);
    // the decode kernel appends k_new / v_new itself
    return hip_status(bi::launch_attn_decode(d, q, k_new, v_new, kv_len, block_table, k_cache,
                                             v_cache, out, lse, ns, (float*)workspace, st));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

// ---- decode with no allocation --------------------------------------------
// The split-partial records of bi_attn_decode_noalloc live in this array: one
// copy per GPU, held until the process ends.  Host code never passes its name
// to a kernel (on the host it is only a stand-in for the symbol); it takes the
// device address that hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) float scratch[BI_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_dev[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call on that
// device; nullptr if the runtime cannot say.
float* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    scratch_dev[dev] = (float*)p;
  }
  return scratch_dev[dev];
}
}  // namespace

bi_status bi_attn_decode_noalloc(const bi_attn_shape* s, const void* q, const void* k_new,
                           const void* v_new, const int32_t* kv_len, const int32_t* block_table,
                           void* k_cache, void* v_cache, void* out, float* lse,
                           int32_t max_kv_len, void* stream) {
  try {
    // the array stands in for the workspace pointer in the shared checks
    const int c = check_decode(s, q, k_new, v_new, kv_len, block_table, k_cache, v_cache, out, lse,
                               max_kv_len, (void*)k_cache);
    if (c < 0) return BI_OK;
    if (c != BI_OK) return (bi_status)c;
    const int ns = (max_kv_len + bi::kSplit - 1) / bi::kSplit;
    if (decode_ws_bytes(s, s->num_seqs, ns) > (size_t)BI_DECODE_SCRATCH_BYTES)
      return BI_ERR_WORKSPACE_TOO_SMALL;
    if ((int64_t)s->num_seqs * s->num_kv_heads * ns / 4 + 1 > kMaxGridX) return BI_ERR_UNSUPPORTED;
    float* ws = scratch_for_current_device();
    if (ws == nullptr) return BI_ERR_HIP;
    const bi::AttnDims d = dims_of(s);
    const hipStream_t st = (hipStream_t)stream;
    return hip_status(bi::launch_attn_decode(d, q, k_new, v_new, kv_len, block_table, k_cache,
                                             v_cache, out, lse, ns, ws, st));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

size_t bix_attn_decode_workspace_bytes(const bi_attn_shape* s, int32_t max_kv_len,
                                       int32_t num_splits) {
  if (check_attn_shape(s) != BI_OK || max_kv_len < 1) return 0;
  if (num_splits <= 0) num_splits = bi::attn_splitkv_auto(s->num_seqs, s->num_kv_heads, max_kv_len);
  int64_t len = ((int64_t)max_kv_len + num_splits - 1) / num_splits;
  len = (len + 31) / 32 * 32;
  const int64_t ns = ((int64_t)max_kv_len + len - 1) / len;
  return decode_ws_bytes(s, s->num_seqs, ns);
}

bi_status bix_attn_decode_splitkv(const bi_attn_shape* s, const void* q, const void* k_new,
                            const void* v_new, const int32_t* kv_len, const int32_t* block_table,
                            void* k_cache, void* v_cache, void* out, float* lse,
                            int32_t max_kv_len, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  try {
    const int c = check_decode(s, q, k_new, v_new, kv_len, block_table, k_cache, v_cache, out, lse,
                               max_kv_len, workspace);
    if (c < 0) return BI_OK;
    if (c != BI_OK) return (bi_status)c;
    if (num_splits <= 0)
      num_splits = bi::attn_splitkv_auto(s->num_seqs, s->num_kv_heads, max_kv_len);
    if (num_splits > max_kv_len) return BI_ERR_UNSUPPORTED;
    if (workspace_bytes < bix_attn_decode_workspace_bytes(s, max_kv_len, num_splits))
      return BI_ERR_WORKSPACE_TOO_SMALL;
    const bi::AttnDims d = dims_of(s);
    const hipStream_t st = (hipStream_t)stream;
    BI_CHECK_TABLES(s, kv_len, nullptr, block_table, max_kv_len, 1, 0, st);
    hipError_t e = bi::launch_kv_append(d, k_new, v_new, nullptr, kv_len, block_table, k_cache,
                                        v_cache, 1, st);
    if (e != hipSuccess) return BI_ERR_HIP;
    return hip_status(bi::launch_attn_decode_splitkv(d, q, kv_len, block_table, k_cache, v_cache,
                                                     out, lse, max_kv_len, num_splits,
                                                     (float*)workspace, st));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

// ---- decoder-stack element-wise operations -----------------------------------

bi_status bi_embed(const int32_t* ids, const void* table, void* out, int64_t tokens, int64_t hidden,
             int64_t vocab, void* stream) {
  try {
    if (tokens < 0 || hidden < 0 || vocab < 0) return BI_ERR_INVALID_SHAPE;
    if (tokens == 0 || hidden == 0) return BI_OK;
    if (vocab == 0 || hidden % 8 != 0) return BI_ERR_INVALID_SHAPE;
    if (tokens > kMaxGridX) return BI_ERR_UNSUPPORTED;
    if (ids == nullptr || table == nullptr || out == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned4(ids) || !aligned16(table) || !aligned16(out)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_embed(ids, table, out, tokens, hidden, vocab, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_rope(void* q, void* k, const int32_t* pos, int64_t tokens, int32_t n_q, int32_t n_kv,
            int32_t head_dim, float theta, void* stream) {
  try {
    if (tokens < 0 || n_q < 0 || n_kv < 0) return BI_ERR_INVALID_SHAPE;
    if (tokens == 0 || n_q + n_kv == 0) return BI_OK;
    if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > 256) return BI_ERR_INVALID_SHAPE;
    if (!(theta > 1.0f) || !isfinite(theta)) return BI_ERR_INVALID_SHAPE;
    if (tokens > kMaxGridX || (int64_t)n_q + n_kv > kMaxGridYZ) return BI_ERR_UNSUPPORTED;
    if (pos == nullptr || (n_q > 0 && q == nullptr) || (n_kv > 0 && k == nullptr))
      return BI_ERR_NULL_POINTER;
    if (!aligned4(pos)) return BI_ERR_INVALID_SHAPE;
    return hip_status(
        bi::launch_rope(q, k, pos, tokens, n_q, n_kv, head_dim, theta, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_qkv_rope(const void* qkv, const int32_t* pos, void* q, void* k, void* v, int64_t tokens,
                int32_t n_q, int32_t n_kv, int32_t head_dim, float theta, void* stream) {
  try {
    if (tokens < 0 || n_q <= 0 || n_kv <= 0) return BI_ERR_INVALID_SHAPE;
    if (tokens == 0) return BI_OK;
    if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > 256) return BI_ERR_INVALID_SHAPE;
    if (!(theta > 1.0f) || !isfinite(theta)) return BI_ERR_INVALID_SHAPE;
    if (tokens > kMaxGridX || (int64_t)n_q + 2 * (int64_t)n_kv > kMaxGridYZ)
      return BI_ERR_UNSUPPORTED;
    if (!qkv || !pos || !q || !k || !v) return BI_ERR_NULL_POINTER;
    if (!aligned4(pos)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_qkv_rope(qkv, pos, q, k, v, tokens, n_q, n_kv, head_dim, theta,
                                          (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_swiglu_pair(const void* gu, void* out, int64_t rows, int64_t f, void* stream) {
  try {
    if (rows < 0 || f < 0 || f % 8 != 0) return BI_ERR_INVALID_SHAPE;
    if (rows == 0 || f == 0) return BI_OK;
    if (gu == nullptr || out == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(gu) || !aligned16(out)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_swiglu_pair(gu, out, rows, f, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_swiglu(const void* gate, const void* up, void* out, int64_t n, void* stream) {
  try {
    if (n < 0 || n % 8 != 0) return BI_ERR_INVALID_SHAPE;
    if (n == 0) return BI_OK;
    if (gate == nullptr || up == nullptr || out == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(out)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_swiglu(gate, up, out, n, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_add(const void* a, const void* b, void* out, int64_t n, void* stream) {
  try {
    if (n < 0 || n % 8 != 0) return BI_ERR_INVALID_SHAPE;
    if (n == 0) return BI_OK;
    if (a == nullptr || b == nullptr || out == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_add(a, b, out, n, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

// ---- measurement ---------------------------------------------------------------

bi_status bix_mfma_loop(int64_t iters, int32_t workgroups, int32_t varied, float* sink, void* stream) {
  try {
    if (iters < 0 || workgroups < 0) return BI_ERR_INVALID_SHAPE;
    if (iters == 0 || workgroups == 0) return BI_OK;
    if (sink == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned4(sink)) return BI_ERR_INVALID_SHAPE;
    return hip_status(
        bi::launch_mfma_loop(iters, workgroups, varied != 0, sink, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bix_read_stream(const void* p, int64_t bytes, int32_t workgroups, uint32_t* sink,
                    void* stream) {
  try {
    if (bytes < 0 || workgroups < 0 || bytes % 8192 != 0) return BI_ERR_INVALID_SHAPE;
    if (bytes == 0 || workgroups == 0) return BI_OK;
    if (p == nullptr || sink == nullptr) return BI_ERR_NULL_POINTER;
    if (((uintptr_t)p & 15) != 0 || !aligned4(sink)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_read_stream(p, bytes, workgroups, sink, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

// ---- int16 KV cache -----------------------------------------------------------

bi_status bi_attn_prefill_i16(const bi_attn_shape* s, const void* q, const void* k_new,
                        const void* v_new, const int32_t* cu_q, const int32_t* kv_len,
                        const int32_t* block_table, void* k_cache, void* v_cache, float* k_scale,
                        float* v_scale, void* out, float* lse, int64_t total_q,
                        int32_t max_q_per_seq, void* stream) {
  try {
    const int c = check_attn_shape(s);
    if (c != BI_OK) return (bi_status)c;
    if (total_q < 0 || max_q_per_seq < 0) return BI_ERR_INVALID_SHAPE;
    if (s->num_seqs == 0 || total_q == 0 || max_q_per_seq == 0) return BI_OK;
    if (max_q_per_seq > total_q) return BI_ERR_INVALID_SHAPE;
    if (max_q_per_seq > (int64_t)s->max_pages_per_seq * s->page_size) return BI_ERR_INVALID_SHAPE;
    if (total_q > kMaxGridX || (int64_t)max_q_per_seq * s->num_kv_heads > kMaxGridX)
      return BI_ERR_UNSUPPORTED;
    if (!q || !k_new || !v_new || !cu_q || !kv_len || !block_table || !k_cache || !v_cache ||
        !k_scale || !v_scale || !out)
      return BI_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(k_scale) || !aligned16(v_scale) || !aligned16(out) ||
        !aligned4(lse) || !aligned4(cu_q) || !aligned4(kv_len) || !aligned4(block_table))
      return BI_ERR_INVALID_SHAPE;
    const bi::AttnDims d = dims_of(s);
    const hipStream_t st = (hipStream_t)stream;
    BI_CHECK_TABLES(s, kv_len, cu_q, block_table, s->max_pages_per_seq * s->page_size,
                    max_q_per_seq, total_q, st);
    hipError_t e = bi::launch_kv_append_i16(d, k_new, v_new, cu_q, kv_len, block_table, k_cache,
                                            v_cache, k_scale, v_scale, max_q_per_seq, st);
    if (e != hipSuccess) return BI_ERR_HIP;
    return hip_status(bi::launch_attn_prefill(d, q, cu_q, kv_len, block_table, k_cache, v_cache,
                                              out, lse, max_q_per_seq, st, k_scale, v_scale));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_attn_decode_i16(const bi_attn_shape* s, const void* q, const void* k_new, const void* v_new,
                       const int32_t* kv_len, const int32_t* block_table, void* k_cache,
                       void* v_cache, float* k_scale, float* v_scale, void* out, float* lse,
                       int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                       void* stream) {
  try {
    const int c = check_decode(s, q, k_new, v_new, kv_len, block_table, k_cache, v_cache, out, lse,
                               max_kv_len, workspace);
    if (c < 0) return BI_OK;
    if (c != BI_OK) return (bi_status)c;
    if (!k_scale || !v_scale) return BI_ERR_NULL_POINTER;
    if (!aligned16(k_scale) || !aligned16(v_scale)) return BI_ERR_INVALID_SHAPE;
    const int ns = (max_kv_len + bi::kSplit - 1) / bi::kSplit;
    if (workspace_bytes < decode_ws_bytes(s, s->num_seqs, ns)) return BI_ERR_WORKSPACE_TOO_SMALL;
    if ((int64_t)s->num_seqs * s->num_kv_heads > kMaxGridX) return BI_ERR_UNSUPPORTED;
    const bi::AttnDims d = dims_of(s);
    const hipStream_t st = (hipStream_t)stream;
    BI_CHECK_TABLES(s, kv_len, nullptr, block_table, max_kv_len, 1, 0, st);
    hipError_t e = bi::launch_kv_append_i16(d, k_new, v_new, nullptr, kv_len, block_table,
                                            k_cache, v_cache, k_scale, v_scale, 1, st);
    if (e != hipSuccess) return BI_ERR_HIP;
    return hip_status(bi::launch_attn_decode(d, q, nullptr, nullptr, kv_len, block_table, k_cache,
                                             v_cache, out, lse, ns, (float*)workspace, st,
                                             k_scale, v_scale));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

// ---- error-compensated matmul ------------------------------------------------

bi_status bi_matmul_ec_pack_w(const float* w, void* w3, int64_t k, int64_t n, void* stream) {
  try {
    if (k < 0 || n < 0) return BI_ERR_INVALID_SHAPE;
    if (k == 0 || n == 0) return BI_OK;
    if (w == nullptr || w3 == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(w) || !aligned16(w3)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_ec_pack_w(w, w3, k, n, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

size_t bi_matmul_ec_workspace_bytes(int64_t m, int64_t k) {
  if (m < 0 || k < 0) return 0;
  return (size_t)m * (size_t)(3 * k) * 2;
}

bi_status bi_matmul_ec(const void* a, int a_dtype, const void* w3, void* c, int c_dtype, int64_t m,
                 int64_t n, int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (m < 0 || n < 0 || k < 0) return BI_ERR_INVALID_SHAPE;
    if (a_dtype != BI_DTYPE_BF16 && a_dtype != BI_DTYPE_F32) return BI_ERR_INVALID_SHAPE;
    if (k > ((int64_t)1 << 22) / 3 || k % bi::kMatmulBK != 0) return BI_ERR_UNSUPPORTED;
    // the product itself is bi_matmul over K' = 3k (fp32 a: [hi | hi | lo]
    // against all of w3) or K' = 2k (bf16 a, whose lo is 0: [a | a] against
    // w3's first 2k rows, [hi; lo])
    const int64_t kk = (a_dtype == BI_DTYPE_F32 ? 3 : 2) * k;
    const int st = check_matmul(workspace, w3, c, c_dtype, m, n, kk);
    if (st < 0) return BI_OK;
    if (st != BI_OK) return (bi_status)st;
    if (k > 0 && a == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned16(a)) return BI_ERR_INVALID_SHAPE;
    if (workspace_bytes < (size_t)m * (size_t)kk * 2) return BI_ERR_WORKSPACE_TOO_SMALL;
    const hipStream_t s = (hipStream_t)stream;
    if (k > 0) {
      const hipError_t e = a_dtype == BI_DTYPE_F32
                               ? bi::launch_ec_pack_a((const float*)a, workspace, m, k, s)
                               : bi::launch_ec_pack_a_bf16(a, workspace, m, k, s);
      if (e != hipSuccess) return BI_ERR_HIP;
    }
    return hip_status(
        bi::launch_matmul(workspace, w3, c, c_dtype == BI_DTYPE_F32, m, n, kk, s));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

bi_status bi_argmax(const float* x, int32_t* out, int64_t rows, int64_t n, void* stream) {
  try {
    if (rows < 0 || n < 0) return BI_ERR_INVALID_SHAPE;
    if (rows == 0) return BI_OK;
    if (n == 0 || n > 0x7ffffffe) return BI_ERR_INVALID_SHAPE;
    if (rows > kMaxGridX) return BI_ERR_UNSUPPORTED;
    if (x == nullptr || out == nullptr) return BI_ERR_NULL_POINTER;
    if (!aligned4(x) || !aligned4(out)) return BI_ERR_INVALID_SHAPE;
    return hip_status(bi::launch_argmax(x, out, rows, n, (hipStream_t)stream));
  } catch (...) {
    return BI_ERR_INTERNAL;
  }
}

}  // extern "C"

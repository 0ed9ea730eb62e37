// Validation of the attention calls' device index arrays, used only by the
// debug build of the library (api.cpp compiled with BI_DEBUG_CHECKS).
//
// One thread per sequence checks what the kernels otherwise trust: the
// sequence length lies in [1, max_len]; for a prefill call, the query ranges
// cu_q[b] .. cu_q[b+1] start at 0, never go back, hold at most max_q and at
// most kv_len[b] tokens, and end at total_q; and every block-table entry the
// length reaches names a page of the pool.  Every read stays inside the
// arrays the caller described (the block-table reads stop at max_pages per
// row), so a bad entry is reported, never followed.  Each problem class sets
// one bit of *flag.
#include "common.h"
#include "kernels.h"

namespace bi {
namespace {

__global__ void clear_flag_kernel(int* flag) { flag[0] = 0; }

__global__ __launch_bounds__(256) void check_attn_tables_kernel(
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ bt, int B, int max_pages, int64_t num_pages, int max_len,
    int max_q, int64_t total_q, int* flag) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int bad = 0;
  const int L = kv_len[b];
  if (L < 1 || L > max_len) bad |= kCheckLength;
  if (cu_q != nullptr) {
    const int64_t s = cu_q[b], e = cu_q[b + 1];
    if (e < s || e - s > max_q || e - s > (int64_t)L) bad |= kCheckQueries;
    if (b == 0 && s != 0) bad |= kCheckQueries;
    if (b == B - 1 && e != total_q) bad |= kCheckQueries;
  }
  const int pages = L < 1 ? 0 : min((L + kPage - 1) / kPage, max_pages);
  const int32_t* row = bt + (int64_t)b * max_pages;
  for (int i = 0; i < pages; ++i) {
    const int32_t p = row[i];
    if (p < 0 || (int64_t)p >= num_pages) {
      bad |= kCheckPage;
      break;
    }
  }
  if (bad) atomicOr(flag, bad);
}

}  // namespace

hipError_t launch_check_attn_tables(const int32_t* kv_len, const int32_t* cu_q, const int32_t* bt,
                                    int B, int max_pages, int64_t num_pages, int max_len,
                                    int max_q, int64_t total_q, int* flag, hipStream_t st) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, st, flag);
  hipLaunchKernelGGL(check_attn_tables_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st,
                     kv_len, cu_q, bt, B, max_pages, num_pages, max_len, max_q, total_q, flag);
  return hipGetLastError();
}

}  // namespace bi

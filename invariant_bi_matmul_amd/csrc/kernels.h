// Internal launchers behind the C ABI.  Each returns hipGetLastError() of its
// launches; argument checking happens in api.cpp before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bi {

// ---- RMSNorm -------------------------------------------------------------
hipError_t launch_rmsnorm(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
                          int hidden, float eps, hipStream_t st);
hipError_t launch_rmsnorm_splitrow(const void* x, const void* gamma, void* y, float* rstd,
                                   int64_t rows, int hidden, float eps, int chunks, float* ws,
                                   hipStream_t st);
int rmsnorm_splitrow_auto_chunks(int64_t rows);

// Compute units of the current device (cached per device).
int device_cus();

// ---- matmul ----------------------------------------------------------------
constexpr int kMatmulBK = 64;
// The tile launch_matmul uses for an m x n product (bm x bn) and its grid.
void matmul_tile(int64_t m, int64_t n, int* bm, int* bn, int64_t* grid);
// packed: w is in the strip layout of launch_matmul_pack_w
hipError_t launch_matmul(const void* a, const void* w, void* c, bool c_f32, int64_t m, int64_t n,
                         int64_t k, hipStream_t st, bool packed = false);
// W [k, n] row-major -> [n/32][k][32] (n % 32 == 0)
hipError_t launch_matmul_pack_w(const void* w, void* wp, int64_t k, int64_t n, hipStream_t st);
int matmul_splitk_auto(int64_t m, int64_t n, int64_t k);
hipError_t launch_mfma_loop(int64_t iters, int workgroups, bool varied, float* sink,
                            hipStream_t st);

// Debug-build validation of the attention index arrays: bits of *flag.
constexpr int kCheckLength = 1, kCheckQueries = 2, kCheckPage = 4;
hipError_t launch_check_attn_tables(const int32_t* kv_len, const int32_t* cu_q, const int32_t* bt,
                                    int B, int max_pages, int64_t num_pages, int max_len,
                                    int max_q, int64_t total_q, int* flag, hipStream_t st);
hipError_t launch_read_stream(const void* p, int64_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t st);
hipError_t launch_matmul_splitk(const void* a, const void* w, void* c, bool c_f32, int64_t m,
                                int64_t n, int64_t k, int split_k, float* ws, hipStream_t st,
                                bool packed = false);

// ---- attention -------------------------------------------------------------
constexpr int kSplit = 256;   // fixed key split
constexpr int kPage = 16;     // tokens per page
// Decode workspace record of one (sequence, q head, split): o[d], m, l and
// two pad floats, so that every record starts on a 16-byte boundary.
constexpr int attn_rec_floats(int d) { return d + 4; }

struct AttnDims {
  int B, nq, nkv, d, max_pages;
  float scale;
};

hipError_t launch_kv_append(const AttnDims& s, const void* k_new, const void* v_new,
                            const int32_t* cu_q, const int32_t* kv_len, const int32_t* bt,
                            void* kc, void* vc, int max_q_per_seq, hipStream_t st);
// kf/vf non-null: the caches hold int16 rows with per-(page, kv head, slot)
// fp32 dequantisation factors; cu_q == nullptr: one token per sequence.
hipError_t launch_attn_prefill(const AttnDims& s, const void* q, const int32_t* cu_q,
                               const int32_t* kv_len, const int32_t* bt, const void* kc,
                               const void* vc, void* out, float* lse, int max_q_per_seq,
                               hipStream_t st, const float* kf = nullptr,
                               const float* vf = nullptr);
hipError_t launch_kv_append_i16(const AttnDims& s, const void* k_new, const void* v_new,
                                const int32_t* cu_q, const int32_t* kv_len, const int32_t* bt,
                                void* kc, void* vc, float* kf, float* vf, int max_q_per_seq,
                                hipStream_t st);
// bf16 cache (kf == nullptr): the partial kernel also writes k_new / v_new
// ([B, nkv, d], one token per sequence) at position kv_len - 1, so no append
// launch precedes it.  int16 cache: the rows are appended beforehand
// (launch_kv_append_i16) and k_new / v_new are unused.
hipError_t launch_attn_decode(const AttnDims& s, const void* q, const void* k_new,
                              const void* v_new, const int32_t* kv_len, const int32_t* bt,
                              void* kc, void* vc, void* out, float* lse, int max_splits, float* ws,
                              hipStream_t st, const float* kf = nullptr,
                              const float* vf = nullptr);
hipError_t launch_attn_decode_splitkv(const AttnDims& s, const void* q, const int32_t* kv_len,
                                      const int32_t* bt, const void* kc, const void* vc, void* out,
                                      float* lse, int max_kv_len, int num_splits, float* ws,
                                      hipStream_t st);
int attn_splitkv_auto(int B, int nkv, int max_kv_len);

// ---- decoder-stack element-wise operations (model.hip) ----------------------
hipError_t launch_embed(const int32_t* ids, const void* table, void* out, int64_t tokens,
                        int64_t hidden, int64_t vocab, hipStream_t st);
hipError_t launch_rope(void* q, void* k, const int32_t* pos, int64_t tokens, int nq, int nkv,
                       int d, float theta, hipStream_t st);
hipError_t launch_qkv_rope(const void* qkv, const int32_t* pos, void* q, void* k, void* v,
                           int64_t tokens, int nq, int nkv, int d, float theta, hipStream_t st);
hipError_t launch_swiglu_pair(const void* gu, void* out, int64_t rows, int64_t f, hipStream_t st);
hipError_t launch_swiglu(const void* gate, const void* up, void* out, int64_t n, hipStream_t st);
hipError_t launch_add(const void* a, const void* b, void* out, int64_t n, hipStream_t st);
hipError_t launch_argmax(const float* x, int32_t* out, int64_t rows, int64_t n, hipStream_t st);
hipError_t launch_ec_pack_a(const float* a, void* a3, int64_t m, int64_t k, hipStream_t st);
hipError_t launch_ec_pack_a_bf16(const void* a, void* a2, int64_t m, int64_t k, hipStream_t st);
hipError_t launch_ec_pack_w(const float* w, void* w3, int64_t k, int64_t n, hipStream_t st);

}  // namespace bi

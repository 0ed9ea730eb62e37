/*
 * bi.h -- C ABI of libbi.so: batch-invariant RMSNorm, matmul and split-KV
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The operations and the property they keep come from "Defeating
 * Nondeterminism in LLM Inference" as summarised on mobiles-han.blogspot.com:
 * the section defining batch invariance (one input always goes through the
 * same computation strategy, whatever the batch size or concurrent work, and
 * so gives the same bits) and the approach table, whose three rows are
 * implemented here:
 *   - RMSNorm: always data-parallel, one order for every batch size;
 *   - MatMul: one kernel configuration, compiled ahead, for every shape;
 *   - Attention: cache and current tokens in one layout before the cache is
 *     read, and fixed-size splits independent of how the batch is made up.
 *
 * GUARANTEE.  For fixed logical inputs the output bits of every bi_* call do
 * not depend on: the number of rows / M / sequences in the call, a row's or
 * sequence's position in it, the other rows or sequences, how a prompt is
 * chunked into prefill calls, prefill versus decode, which physical pages hold
 * the keys, the stream, or how often the call is repeated.  Bits may differ
 * between builds of this library.
 *
 * CONVENTIONS (all entry points).
 *   - Every tensor argument is a DEVICE pointer to memory owned by the caller.
 *     The library allocates nothing, frees nothing and never synchronises.
 *     Its only mutable global state is bi_attn_decode_noalloc's scratch array
 *     (and the per-device table of its addresses, filled under a lock); every
 *     other entry point is reentrant.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *     Inputs must stay alive and unmodified until that work completes.
 *   - Every call but bi_abi_version and the *_bytes queries returns a
 *     bi_status (an int-sized enum).
 *   - Host arguments are checked before anything is enqueued.  On any non-OK
 *     status nothing has been enqueued.  Kernel faults surface, as usual in
 *     HIP, at the caller's next synchronisation.
 *   - bf16 tensors hold IEEE bfloat16 bit patterns; results are rounded to
 *     nearest even.  Sizes of 0 are no-ops returning BI_OK; negative sizes are
 *     BI_ERR_INVALID_SHAPE.
 *   - Contents of device index arrays (kv_len, cu_q, block_table) are trusted:
 *     entries outside the documented ranges are undefined behaviour.  The
 *     debug build of the library (libbi_debug.so, compiled with
 *     BI_DEBUG_CHECKS) checks them on the device before each attention call
 *     launches anything: 1 <= kv_len[b] <= the call's length bound (max_kv_len
 *     for decode, max_pages_per_seq * page_size otherwise); cu_q starts at 0,
 *     never decreases, gives each sequence at most max_q_per_seq and at most
 *     kv_len[b] tokens and ends at total_q; every block-table entry a
 *     sequence's length reaches is in [0, num_pages).  A violation returns
 *     BI_ERR_INVALID_SHAPE with nothing else enqueued.  That build
 *     synchronises the stream on every attention call, allocates one int per
 *     device (once) for the result, and cannot be captured into a graph.
 *   - No C++ exception crosses this interface.
 *   - Tensor pointers must be 16-byte aligned (BI_ERR_INVALID_SHAPE otherwise).
 */
#ifndef BI_H_
#define BI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BI_ABI_VERSION 5

typedef enum {
  BI_OK = 0,
  BI_ERR_NULL_POINTER = 1,        /* a required pointer is NULL                   */
  BI_ERR_INVALID_SHAPE = 2,       /* negative / inconsistent sizes, misalignment  */
  BI_ERR_UNSUPPORTED = 3,         /* valid, but outside the one compiled config   */
  BI_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes below the documented size    */
  BI_ERR_HIP = 5,                 /* the HIP runtime refused a launch             */
  BI_ERR_INTERNAL = 6
} bi_status;

typedef enum { BI_DTYPE_BF16 = 0, BI_DTYPE_F32 = 1 } bi_dtype;

/* Version of this interface (BI_ABI_VERSION of the build). */
int bi_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* bi_status_string(int status);

/* ------------------------------------------------------------------------- */
/* RMSNorm (approach table, RMSNorm row: data-parallel, one order per row).
 *
 *   rstd[r] = 1 / sqrt( (sum_c x[r,c]^2) / hidden + eps )
 *   y[r,c]  = bf16( (x[r,c] * rstd[r]) * gamma[c] )
 *
 * x     bf16 [rows, hidden] row-major.
 * gamma bf16 [hidden].
 * y     bf16 [rows, hidden]; may equal x (in place); no other overlap.
 * rstd  fp32 [rows], or NULL to skip.
 * Each row is reduced by one workgroup in an order that depends on `hidden`
 * only: per-lane sequential fp32 sums, a fixed wave64 butterfly, then the
 * waves' partials added in wave order.
 * Requires hidden % 8 == 0 and 8 <= hidden <= 16384 (else BI_ERR_UNSUPPORTED).
 */
bi_status bi_rmsnorm(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
               int64_t hidden, float eps, void* stream);

/* ------------------------------------------------------------------------- */
/* Matmul (approach table, MatMul row: one configuration for every shape).
 *
 *   c[i,j] = sum_k a[i,k] * w[k,j]     (fp32 accumulation; c bf16 or fp32)
 *
 * a  bf16 [m, k] row-major.
 * w  bf16 [k, n] row-major (n contiguous).
 * c  [m, n] row-major, bf16 (rounded from the fp32 sum) or fp32 per c_dtype.
 * One bf16 MFMA instruction for every m, n, k; each element's k-loop runs in
 * one fixed order (16-wide MFMA steps, ascending); no split-K.  The output
 * tile (256 x 256 or 256 x 128 for launches with a round of them; 128 x 128,
 * 128 x 64, 64 x 64 or 64 x 32 for launches too small to give those every CU;
 * bix_matmul_tile reports it) only decides which wave computes an element,
 * never its bits.  The bf16 result
 * is exactly the round-to-nearest-even of the fp32 result.
 * Requires k % 64 == 0, n % 8 == 0, k <= 2^22 and n <= 2^24 (else
 * BI_ERR_UNSUPPORTED).
 */
bi_status bi_matmul(const void* a, const void* w, void* c, int c_dtype, int64_t m, int64_t n, int64_t k,
              void* stream);

/* The same product with W in the strip layout written by bi_matmul_pack_w:
 * wp = bf16 [n/32][k][32], strip j holding columns 32j .. 32j+31 of w, each
 * strip contiguous along k.  A launch whose workgroups each stream one or two
 * strips (small m) then reads whole bursts of HBM rather than 64-byte pieces
 * of w's rows.  c is bitwise what bi_matmul(a, w, ...) gives: the same tiles,
 * MFMA and k order, only the global addresses of w differ.  Requires
 * n % 32 == 0 as well as bi_matmul's conditions (else BI_ERR_UNSUPPORTED).
 * A layout choice of the approach table's MatMul row, not a new reduction. */
bi_status bi_matmul_packed(const void* a, const void* wp, void* c, int c_dtype, int64_t m,
                           int64_t n, int64_t k, void* stream);

/* wp[j][r][i] = w[r][32j + i]: w bf16 [k, n] row-major into the strip layout
 * (k * n bf16 values, caller-owned, no overlap with w).  n % 32 == 0,
 * k <= 2^22, n <= 2^24 (else BI_ERR_UNSUPPORTED); k or n = 0 is a no-op. */
bi_status bi_matmul_pack_w(const void* w, void* wp, int64_t k, int64_t n, void* stream);

/* The output tile bi_matmul uses for an m x n product on the current device
 * (tile_m x tile_n) and the workgroups it launches.  Host-only; any pointer
 * may be NULL.  BI_ERR_INVALID_SHAPE for m or n < 1. */
bi_status bix_matmul_tile(int64_t m, int64_t n, int32_t* tile_m, int32_t* tile_n, int64_t* workgroups);

/* ------------------------------------------------------------------------- */
/* Paged attention (approach table, Attention row: one unified cache layout,
 * fixed-size splits).
 *
 * Key/value pool: k_cache, v_cache bf16 [num_pages, num_kv_heads, page_size,
 * head_dim].  Position p of sequence b lives in page block_table[b *
 * max_pages_per_seq + p / page_size], slot p % page_size.
 *
 * Each call first appends the new tokens' keys and values to the pool, then
 * computes attention reading keys and values from the pool only.  The query at
 * absolute position p of a sequence attends to its positions 0..p.  Query
 * head h reads kv head h / (num_q_heads / num_kv_heads).
 *
 * Keys are cut into fixed 256-position splits at absolute multiples of 256.
 * For each split the partial (m_s, l_s, o_s) -- max logit, sum of exponentials,
 * exponential-weighted sum of values -- is computed in one fixed order, and
 * the partials are folded left in ascending split order:
 *   m' = max(m, m_s);  l <- l e^(m-m') + l_s e^(m_s-m');  o <- o e^(m-m') + o_s e^(m_s-m')
 *   out = bf16(o / l),  lse = m + ln(l)   (natural log, fp32)
 * Prefill folds in registers; decode spreads splits over workgroups and folds
 * them in a second kernel with the same function, so a token's row is bitwise
 * the same through either entry point and any chunking.
 */
typedef struct {
  int32_t num_seqs;          /* B >= 0                                         */
  int32_t num_q_heads;       /* n_q, a multiple of num_kv_heads                */
  int32_t num_kv_heads;      /* n_kv >= 1                                      */
  int32_t head_dim;          /* d: 64 or 128                                   */
  int32_t page_size;         /* must be 16                                     */
  int32_t max_pages_per_seq; /* row stride of block_table                      */
  int64_t num_pages;         /* pages in the pool                              */
  float softmax_scale;       /* multiplies q.k, usually 1/sqrt(d)              */
} bi_attn_shape;

/* Split size in positions (fixed). */
#define BI_ATTN_SPLIT 256

/* Bytes of workspace bi_attn_decode needs for num_tokens (= num_seqs) queries
 * whose sequences hold at most max_kv_len positions after the append.
 * Returns 0 for invalid arguments. */
size_t bi_attn_workspace_bytes(const bi_attn_shape* s, int64_t num_tokens, int32_t max_kv_len);

/* Prefill (or any chunk): sequence b brings n_b = cu_q[b+1] - cu_q[b] new
 * tokens, at positions kv_len[b] - n_b .. kv_len[b] - 1.
 *   q      bf16 [total_q, n_q, d]     rows cu_q[b] .. cu_q[b+1]-1 are sequence b
 *   k_new, v_new bf16 [total_q, n_kv, d]
 *   cu_q   int32 [B + 1] device, cu_q[0] = 0, non-decreasing, cu_q[B] = total_q
 *   kv_len int32 [B] device, length of each sequence AFTER this call's append
 *   block_table int32 [B, max_pages_per_seq] device
 *   out    bf16 [total_q, n_q, d];  lse fp32 [total_q, n_q] or NULL
 *   max_q_per_seq (host) >= every n_b, used to size the grid.
 * Requires n_b <= kv_len[b] <= max_pages_per_seq * page_size (trusted).
 * No workspace. */
bi_status bi_attn_prefill(const bi_attn_shape* s, const void* q, const void* k_new, const void* v_new,
                    const int32_t* cu_q, const int32_t* kv_len, const int32_t* block_table,
                    void* k_cache, void* v_cache, void* out, float* lse, int64_t total_q,
                    int32_t max_q_per_seq, void* stream);

/* Decode: one new token per sequence, at position kv_len[b] - 1.
 *   q bf16 [B, n_q, d]; k_new, v_new bf16 [B, n_kv, d]; out bf16 [B, n_q, d];
 *   lse fp32 [B, n_q] or NULL.
 *   max_kv_len (host) >= every kv_len[b] (after the append), sizes the grid.
 * Requires 1 <= kv_len[b] <= max_kv_len (trusted).  The append runs inside
 * the split pass, in the one wave that reads the split holding that position
 * for that kv head: it writes the rows and then reads them from the pool like
 * every other row, so outputs and pool contents are those of an append
 * followed by attention.  A length beyond max_kv_len leaves its row
 * unwritten and its outputs undefined.
 *   workspace: device, >= bi_attn_workspace_bytes(s, B, max_kv_len) bytes,
 *   contents on entry ignored, scratch for the per-split partials. */
bi_status bi_attn_decode(const bi_attn_shape* s, const void* q, const void* k_new, const void* v_new,
                   const int32_t* kv_len, const int32_t* block_table, void* k_cache,
                   void* v_cache, void* out, float* lse, int32_t max_kv_len, void* workspace,
                   size_t workspace_bytes, void* stream);

/* bi_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split-partial records go to a scratch
 * array of BI_DECODE_SCRATCH_BYTES that the library holds in device memory,
 * one per GPU it runs on, until the process ends; its address is looked up
 * (hipGetSymbolAddress) on the first call on each device.  The call allocates
 * nothing and runs the same kernels as bi_attn_decode, so its outputs are
 * bitwise those of bi_attn_decode.
 *   Arguments as bi_attn_decode.  BI_ERR_WORKSPACE_TOO_SMALL (nothing
 *   enqueued) when bi_attn_workspace_bytes(s, B, max_kv_len) exceeds
 *   BI_DECODE_SCRATCH_BYTES; BI_ERR_HIP if the scratch address cannot be had.
 *   Every call on one GPU shares that GPU's array and leaves its records in
 *   it (each call writes every record it reads first, so nothing needs
 *   clearing): calls that can overlap on one GPU -- on different streams, or
 *   from different threads -- race and must be ordered by the caller.
 *   The debug library does not check the index arrays for this call. */
#define BI_DECODE_SCRATCH_BYTES (64u << 20)
bi_status bi_attn_decode_noalloc(const bi_attn_shape* s, const void* q, const void* k_new,
                           const void* v_new, const int32_t* kv_len, const int32_t* block_table,
                           void* k_cache, void* v_cache, void* out, float* lse,
                           int32_t max_kv_len, void* stream);

/* ------------------------------------------------------------------------- */
/* Non-invariant comparators (the strategies the approach table warns about).
 * Same inputs and outputs as their bi_* counterparts; they exist to measure
 * the cost of invariance and as negative controls: their results change with
 * the batch.  Not for production use.
 *
 * bix_rmsnorm_splitrow: each row's sum of squares is split over `chunks`
 * workgroups (chunks <= 0: chosen from `rows`, more chunks for fewer rows),
 * partials added by a second kernel.  workspace >= rows * 64 * 4 bytes. */
bi_status bix_rmsnorm_splitrow(const void* x, const void* gamma, void* y, float* rstd, int64_t rows,
                         int64_t hidden, float eps, int32_t chunks, void* workspace,
                         size_t workspace_bytes, void* stream);

/* bix_matmul_splitk: bi_matmul's tile for the shape, with the k range split
 * into `split_k` slices (split_k <= 0: enough slices for one workgroup per CU
 * over that tile's grid, at most 16 -- so more slices for smaller m); fp32
 * partials are summed in slice order by a second kernel.  With one slice it
 * is bi_matmul (no workspace is touched).  workspace >=
 * bix_matmul_workspace_bytes. */
size_t bix_matmul_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t split_k);
bi_status bix_matmul_splitk(const void* a, const void* w, void* c, int c_dtype, int64_t m, int64_t n,
                      int64_t k, int32_t split_k, void* workspace, size_t workspace_bytes,
                      void* stream);
/* The same comparator with W in bi_matmul_pack_w's strip layout (n % 32 == 0). */
bi_status bix_matmul_splitk_packed(const void* a, const void* wp, void* c, int c_dtype,
                                   int64_t m, int64_t n, int64_t k, int32_t split_k,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* bix_attn_decode_splitkv: decode whose key range is cut into `num_splits`
 * equal parts per sequence (num_splits <= 0: chosen from B and max_kv_len to
 * fill the GPU), so split boundaries move with the batch.  workspace >=
 * bix_attn_decode_workspace_bytes. */
size_t bix_attn_decode_workspace_bytes(const bi_attn_shape* s, int32_t max_kv_len,
                                       int32_t num_splits);
bi_status bix_attn_decode_splitkv(const bi_attn_shape* s, const void* q, const void* k_new,
                            const void* v_new, const int32_t* kv_len, const int32_t* block_table,
                            void* k_cache, void* v_cache, void* out, float* lse,
                            int32_t max_kv_len, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* stream);

/* bix_mfma_loop: measurement only, the MFMA ceiling.  `workgroups` workgroups
 * of four waves each run `iters` rounds of four independent bf16
 * v_mfma_f32_32x32x16 chains on register operands: 4 * 32768 * iters flops
 * per wave, no memory traffic.  varied != 0: the chains cycle through four
 * operand pairs of random-looking bits, so consecutive MFMAs see different
 * inputs as in a matmul (the pipe's power, and so the clock the chip holds,
 * depends on the bits); 0: one fixed, smooth pair.  sink: device float,
 * written never (it only keeps the work from being optimised away). */
bi_status bix_mfma_loop(int64_t iters, int32_t workgroups, int32_t varied, float* sink, void* stream);

/* bix_read_stream: measurement only, the HBM read ceiling.  Reads `bytes`
 * (a multiple of 8192) from device pointer p (16-byte aligned) once, as 8 KiB
 * chunks streamed through LDS by direct loads (the decode kernel's way of
 * reading), from `workgroups` workgroups of two waves.  sink: device uint32,
 * written never.  INVALID_SHAPE for a misaligned pointer or size. */
bi_status bix_read_stream(const void* p, int64_t bytes, int32_t workgroups, uint32_t* sink,
                    void* stream);

/* ---- Decoder-stack element-wise operations ---------------------------------
 * The rest of a dense Llama-style decoder layer around the three kernels
 * above, so that a whole stack can be run and its greedy output checked.  The
 * news.hada.io page on GPT-4's output varying at temperature 0 (its problem
 * statement) notes that greedy decoding of a dense decoder should be exactly
 * reproducible, the next-token logits being a function of the input sequence
 * and the weights alone; the operations below keep that per sequence.  The
 * pages define none of them: they are the standard Llama forms.  Each output
 * element depends only on its own row (and position), through one fixed fp32
 * sequence, so each is batch-invariant by construction. */

/* out[t, :] = table[ids[t], :].  ids int32 [tokens] (device; entries outside
 * [0, vocab) are clamped into it); table bf16 [vocab, hidden]; out bf16
 * [tokens, hidden].  hidden % 8 == 0.  Also a plain row gather. */
bi_status bi_embed(const int32_t* ids, const void* table, void* out, int64_t tokens, int64_t hidden,
             int64_t vocab, void* stream);

/* Rotary position embedding in place, "rotate half" pairing: for token t at
 * position p = pos[t], every head of q (bf16 [tokens, n_q, head_dim]) and of
 * k (bf16 [tokens, n_kv, head_dim]), and i < head_dim/2, with a = x[i],
 * b = x[i + head_dim/2] and angle = p * theta^(-2i/head_dim) (fp32):
 *   x[i] = bf16(a cos - b sin),  x[i + head_dim/2] = bf16(a sin + b cos).
 * head_dim even and <= 256; theta > 1.  q or k may be NULL when n_q or n_kv
 * is 0.  pos int32 [tokens] (device). */
bi_status bi_rope(void* q, void* k, const int32_t* pos, int64_t tokens, int32_t n_q, int32_t n_kv,
            int32_t head_dim, float theta, void* stream);

/* out = bf16(silu(gate) * up) element-wise, silu(g) = g / (1 + e^-g) in fp32.
 * gate, up, out bf16 [n], n % 8 == 0; out may alias gate or up. */
bi_status bi_swiglu(const void* gate, const void* up, void* out, int64_t n, void* stream);

/* The output of one fused q|k|v projection split into the q, k and v tensors
 * the attention calls take, with bi_rope's rotation (the same arithmetic)
 * applied to the q and k heads.  qkv bf16 [tokens, n_q + 2 n_kv, head_dim]
 * (row t: t's q heads, then k heads, then v heads); q bf16 [tokens, n_q,
 * head_dim], k and v bf16 [tokens, n_kv, head_dim], none overlapping qkv;
 * pos int32 [tokens].  head_dim even and <= 256; theta > 1.  A fused
 * projection (one bi_matmul against [W_q | W_k | W_v]) gives every column the
 * bits of the separate ones: a column's dot product does not depend on its
 * neighbours. */
bi_status bi_qkv_rope(const void* qkv, const int32_t* pos, void* q, void* k, void* v, int64_t tokens,
                int32_t n_q, int32_t n_kv, int32_t head_dim, float theta, void* stream);

/* bi_swiglu over the output of one fused gate|up projection: gu bf16
 * [rows, 2f] (row r: gate, then up), out bf16 [rows, f] not overlapping gu;
 * f % 8 == 0. */
bi_status bi_swiglu_pair(const void* gu, void* out, int64_t rows, int64_t f, void* stream);

/* out = bf16(a + b) element-wise (the residual add).  bf16 [n], n % 8 == 0;
 * out may alias a or b. */
bi_status bi_add(const void* a, const void* b, void* out, int64_t n, void* stream);

/* Greedy sampling: out[r] = the index of the largest of x[r, 0..n-1] (fp32
 * [rows, n], 4-byte aligned), the lowest such index on ties.  NaN is never
 * chosen; a row holding no number gives 0.  out int32 [rows]. */
bi_status bi_argmax(const float* x, int32_t* out, int64_t rows, int64_t n, void* stream);

/* ---- Int16 KV cache ----------------------------------------------------------
 * The HEAL page on gist.science (its new-solution section, item 1) packs the
 * attention keys and values as INT16 and unpacks them into two 16-bit values
 * for the matrix units, at no extra memory.  Reading followed here:
 *   - each (token, kv head) row x (d values) of K or V is stored as
 *     q = rint(x * (32767 / s)) in int16 (ties to even; fp32 arithmetic),
 *     s = max |x| over the row, with the dequantisation factor f = s / 32767
 *     (fp32; 0 for an all-zero row) in a separate array;
 *   - the caches are int16 [num_pages, n_kv, 16, d] (the bf16 layout, same
 *     bytes), the factors fp32 [num_pages, n_kv, 16] (16-byte aligned);
 *   - attention reads q as hi = bf16(q), lo = bf16(q - hi) (both exact, so
 *     hi + lo = q) and takes two MFMA products for Q K^T and for P V: the
 *     logit of a key is (q . k_int) * f_k * scale, and the value factor goes
 *     into the weight before it is rounded to bf16 (the softmax sum keeps
 *     the unscaled exponentials).
 * A per-token factor keeps a row's codes independent of what else is in the
 * cache, so chunking and batching leave them unchanged; splits, their fixed
 * 256-position boundaries and the fold order are those of bi_attn_prefill.
 * Inputs must be finite. */

/* As bi_attn_prefill, with the int16 caches and their factor arrays. */
bi_status bi_attn_prefill_i16(const bi_attn_shape* s, const void* q, const void* k_new,
                        const void* v_new, const int32_t* cu_q, const int32_t* kv_len,
                        const int32_t* block_table, void* k_cache, void* v_cache, float* k_scale,
                        float* v_scale, void* out, float* lse, int64_t total_q,
                        int32_t max_q_per_seq, void* stream);

/* Decode over the int16 cache, as bi_attn_decode: one new token per sequence
 * (q, k_new, v_new [B, ...]), quantised and appended, then the split
 * partials (the decode kernel, each unit's 256 key and value factors staged
 * with its q) and the fixed-order fold.  max_kv_len, workspace and
 * workspace_bytes as in bi_attn_decode (bi_attn_workspace_bytes sizes it). */
bi_status bi_attn_decode_i16(const bi_attn_shape* s, const void* q, const void* k_new, const void* v_new,
                       const int32_t* kv_len, const int32_t* block_table, void* k_cache,
                       void* v_cache, float* k_scale, float* v_scale, void* out, float* lse,
                       int32_t max_kv_len, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---- Error-compensated matmul ---------------------------------------------
 * The HEAL page on gist.science ("Demystifying Numerical Instability in LLM
 * Inference ... with HEAL", its new-solution section, item 2 on error
 * compensation) computes a GEMM as a main product in the fast 16-bit format
 * plus a quick clean-up product that recovers what the main one lost.  The
 * page gives no formula; the reading here: split each fp32 operand x into
 * hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in fp32; a non-finite hi
 * gets lo = 0), and accumulate
 *     C = hi(A) hi(W) + hi(A) lo(W) + lo(A) hi(W)        (lo lo dropped)
 * in fp32, in this order, as ONE bi_matmul over K' = 3K of the packed operands
 *     A3 = [hi(A) | hi(A) | lo(A)]  (bf16 [m, 3k], row by row)
 *     W3 = [hi(W) ; lo(W) ; hi(W)]  (bf16 [3k, n], stacked along k).
 * It inherits bi_matmul's invariance (one MFMA, one k order, no split-K) at
 * three times its MFMA work; the error is about 2^-16 of sum |a||w| instead
 * of bf16's 2^-8. */

/* W3 = [hi(w); lo(w); hi(w)]: w fp32 [k, n] -> w3 bf16 [3k, n] (a weight is
 * packed once). */
bi_status bi_matmul_ec_pack_w(const float* w, void* w3, int64_t k, int64_t n, void* stream);

/* Bytes of workspace bi_matmul_ec needs for any operand type: m * 3k * 2
 * (the packed A3; a bf16 a needs only m * 2k * 2). */
size_t bi_matmul_ec_workspace_bytes(int64_t m, int64_t k);

/* c [m, n] = the error-compensated product of a [m, k] and the packed
 * w3 bf16 [3k, n].
 *   a_dtype BI_DTYPE_F32: a fp32 [m, k]; the workspace receives
 *     A3 = [hi(a) | hi(a) | lo(a)] and c = one bi_matmul of A3 and w3 over
 *     K' = 3k: the three products above in that order.
 *   a_dtype BI_DTYPE_BF16: a bf16 [m, k], exactly representable, so lo(a) = 0
 *     and the third product vanishes; the workspace receives A2 = [a | a] and
 *     c = one bi_matmul of A2 and the first 2k rows of w3 ([hi(w); lo(w)])
 *     over K' = 2k.  The sum is the first two products in the same order
 *     (adding the vanished third product's zeros changes at most the sign
 *     of a zero sum).
 *   c_dtype BI_DTYPE_F32 (the fp32 sum) or BI_DTYPE_BF16 (its round to
 *   nearest even, as bi_matmul's bf16 output).
 * k % 64 == 0, n % 8 == 0, 3k <= 2^22 (else BI_ERR_UNSUPPORTED).  workspace:
 * device, >= m * K' * 2 bytes.  Rows are invariant as bi_matmul's are. */
bi_status bi_matmul_ec(const void* a, int a_dtype, const void* w3, void* c, int c_dtype, int64_t m,
                 int64_t n, int64_t k, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_H_ */

/*
 * kvq_oracle.h -- plain CPU oracle for append and decode attention over a
 * quantized KV cache (K as q8_0, V as q5_1).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Sources (docs.rs pages; cited by page title and item):
 *   [KvLayer]  memra-engine "Struct KvLayer" page and the memra-engine
 *              "Module cache" page, item KvLayer: K is q8_0 at 34 bytes per
 *              32 elements, V is q5_1 at 24 bytes per 32 elements, each token
 *              row keeps [kv_head, dim] order, element index
 *              kv_head*head_dim + d, block = index/32, lane = index%32, and
 *              head_dim must be a multiple of 32.
 *   [attend]   cortiq-engine "Struct LayerKvCache" page, methods attend_group
 *              and attend_group_upto, field sinks: grouped GQA (Q head h uses
 *              KV group h/hpk), score scale, first visible row, the causal
 *              `upto` bound, and the sink as a value-less softmax column.
 *   [len_d/base_d] "Struct KvLayer" page, fields len_d and base_d: the live
 *              view is rows [max(0, len - window), len), physical row =
 *              row - base.
 *
 * Parity status of each function is stated at its definition.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE 754 binary32 -> binary16 bits, round to nearest even. */
uint16_t kvqo_f32_to_f16(float x);
/* IEEE 754 binary16 bits -> binary32 (exact). */
float kvqo_f16_to_f32(uint16_t h);
/* Convert n floats (for exhaustive checks from Python). */
void kvqo_f32_to_f16_array(const float* x, uint16_t* out, int64_t n);

/* One 32-element block.  q8_0: 34 bytes.  q5_1: 24 bytes. */
void kvqo_q8_0_encode(const float* x, uint8_t* blk);
void kvqo_q8_0_decode(const uint8_t* blk, double* x);
void kvqo_q5_1_encode(const float* x, uint8_t* blk);
void kvqo_q5_1_decode(const uint8_t* blk, double* x);

/* e4m3 (OCP FP8 E4M3): one code's value (NaN for S.1111.111); the nearest
 * code to x, ties to even, saturating at +-448, keeping x's sign. */
double kvqo_e4m3_value(uint8_t c);
uint8_t kvqo_e4m3_from_f32(float x);
/* FP8 block, 34 bytes: fp16 scale + 32 e4m3 codes. */
void kvqo_f8_encode(const float* x, uint8_t* blk);
void kvqo_f8_decode(const uint8_t* blk, double* x);

/* Cache formats of the attention and importance routines. */
#define KVQO_FMT_Q8_Q5 0   /* K q8_0 blocks, V q5_1 blocks, consecutive in a row */
#define KVQO_FMT_E4M3 1    /* K and V FP8 rows (kvqo_quantize_f8_rows) */

/* Encode n_elems (a multiple of 32) consecutive floats as consecutive
 * blocks.  Because head_dim % 32 == 0 and a token row is laid out as
 * [kv_head, dim], this is exactly the byte image of n_elems/(Hkv*hd) rows. */
void kvqo_quantize_k(const float* x, int64_t n_elems, uint8_t* out);
void kvqo_quantize_v(const float* x, int64_t n_elems, uint8_t* out);
/* n_rows FP8 token rows of row_elems floats each: per row, the codes of its
 * 32-element blocks (kvqo_f8_encode) in element order, then the blocks'
 * fp16 scales in block order; row_elems / 32 * 34 bytes per row. */
void kvqo_quantize_f8_rows(const float* x, int64_t n_rows, int32_t row_elems, uint8_t* out);

/*
 * Exact-softmax decode attention in double precision.
 *   fmt      KVQO_FMT_Q8_Q5 or KVQO_FMT_E4M3 (the planes' format)
 *   q        [B, T, H, hd] floats (bf16 inputs widened exactly beforehand)
 *   k_plane  per session: pointer to the physical row 0 of its K plane
 *   v_plane  per session: pointer to the physical row 0 of its V plane
 *   base     per session: logical row held in physical row 0
 *   len      per session: rows committed, the last T are the query rows
 *   window   0 = full attention, else rows [max(0, upto-window), upto)
 *   sinks    [H] or NULL
 *   sel      flat (b*T + t)*H + h indices to compute, or NULL for all
 *   out      [B, T, H, hd] (only selected entries written)
 *   lse      [B, T, H] or NULL
 * Returns 0, or -1 on an argument the method does not define (a visible
 * set that would be empty, or a visible row outside the resident range).
 */
int kvqo_attention(int32_t fmt, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                   const float* q,
                   const uint8_t* const* k_plane, const uint8_t* const* v_plane,
                   const int64_t* base, const int64_t* len, int32_t window,
                   const float* sinks, float scale,
                   const int64_t* sel, int64_t n_sel,
                   float* out, float* lse);

/* Attention importance: adds to imp[b * cap + (row - base[b])], for every
 * row a query row sees, that row's softmax probability (sink in the
 * denominator), summed over the T query rows and H heads.  Returns 0 or -1
 * as kvqo_attention. */
int kvqo_importance(int32_t fmt, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                    const float* q, const uint8_t* const* k_plane,
                    const int64_t* base, const int64_t* len, int32_t window,
                    const float* sinks, float scale, double* imp, int64_t cap);

/* Threads the attention loops may use (OpenMP), for reporting. */
int kvqo_max_threads(void);
/* Threads the attention loops use from now on (n >= 1). */
void kvqo_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif

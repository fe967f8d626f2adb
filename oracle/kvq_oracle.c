/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline leg of the benchmark; never by the product path.  It shares no
 * code with the HIP library.  Build: gcc -O2 -fPIC -shared -fopenmp
 * -ffp-contract=off (no fast-math, so float division and rintf are IEEE).
 *
 * What is pinned, and by what (the tests under tests/ hold the pins):
 *   kvqo_f32_to_f16        IEEE 754 definition; checked against numpy's
 *                          float16 conversion on every float in the
 *                          half-precision-relevant exponent range.
 *   q8_0 / q5_1 codecs     byte sizes 34/24 from the KvLayer item; byte
 *                          images of hand-derived blocks (tests/golden);
 *                          exact reproduction of representable blocks;
 *                          half-even ties; the round-trip error bound.
 *                          Parity with another implementation's bytes is
 *                          unpinned: the pages print no encoded block.
 *   e4m3 / f8 codec        every code's value against the format's
 *                          printed landmarks (448, 2^-6, 2^-9, NaN) and
 *                          monotone order; the rounding of a float to a
 *                          code against torch's float8_e4m3fn conversion
 *                          on every quotient within +-448 (ties included);
 *                          a hand-derived block; the round-trip bound.
 *                          Parity with another implementation's bytes is
 *                          unpinned: the pages print no encoded block.
 *   FP8 rows               the row layout of the FP8 variant (codes of the
 *                          row's blocks in element order, then their fp16
 *                          scales) against a row image assembled by hand
 *                          from the hand-derived golden blocks; attention
 *                          over FP8 rows against textbook attention on
 *                          values the e4m3 codec stores exactly.
 *   kvqo_importance        per-row probability mass summed over query
 *                          rows and heads: it sums to T*H less the sinks'
 *                          shares (closed form); equals a numpy softmax of
 *                          each (row, head) with the sink as an extra
 *                          column (brute force on small inputs); rows
 *                          outside every window get 0.
 *   kvqo_attention         textbook attention (torch's fp64
 *                          scaled_dot_product_attention with repeated KV
 *                          heads and explicit masks) on K/V rows the codec
 *                          stores exactly, with a sink written as one extra
 *                          key whose value row is zero; closed forms at
 *                          len 1 and q = 0; window == masked full row;
 *                          T causal rows == T sequential single-row calls;
 *                          GQA == repeated KV heads; ring == flat cache;
 *                          truncate == fresh cache of the kept prefix.
 */
#include "kvq_oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* binary16 conversion, written from IEEE 754: a binary32 value is      */
/* m * 2^(e-23) with a 24-bit integer significand m; binary16 keeps an  */
/* 11-bit significand for exponents -14..15 and a fixed quantum 2^-24   */
/* below that.  Round the significand to the kept width, ties to even.  */
/* ------------------------------------------------------------------ */
uint16_t kvqo_f32_to_f16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t efield = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;

    if (efield == 0xFFu) /* infinity or NaN */
        return (uint16_t)(sign | 0x7C00u | (frac ? 0x0200u : 0u));
    if (efield == 0u)    /* zero or binary32 subnormal: below 2^-126, rounds to 0 */
        return sign;

    int e = (int)efield - 127;            /* value = m * 2^(e-23) */
    uint32_t m = frac | 0x800000u;        /* 24-bit significand */
    if (e > 15)
        return (uint16_t)(sign | 0x7C00u); /* overflow -> infinity */

    /* bits to drop: 13 for a normal result; more for a subnormal one */
    int shift = (e >= -14) ? 13 : 13 + (-14 - e);
    if (shift > 25)
        return sign;                       /* below half the smallest subnormal */
    uint32_t q = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;

    uint32_t bits;
    if (e >= -14)
        bits = ((uint32_t)(e + 14) << 10) + q; /* q in [1024, 2048]; a carry bumps the exponent */
    else
        bits = q;                              /* subnormal, or 0x400 if it rounded up */
    /* bits == 0x7C00 here means the rounding overflowed to infinity */
    return (uint16_t)(sign | bits);
}

float kvqo_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int efield = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (efield == 0)
        v = ldexp((double)frac, -24);
    else if (efield == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), efield - 25);
    return (float)(sign ? -v : v);
}

void kvqo_f32_to_f16_array(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = kvqo_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------ */
/* q8_0: 34 bytes = fp16 scale d (little-endian) + 32 signed 8-bit     */
/* codes.  Reading of the pages (sizes only are printed): symmetric     */
/* absolute-max scaling d = amax/127, codes from the STORED scale,      */
/* rounded half-to-even and clamped to [-127, 127].                     */
/* ------------------------------------------------------------------ */
void kvqo_q8_0_encode(const float* x, uint8_t* blk) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        assert(isfinite(x[i]));
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    uint16_t d16 = kvqo_f32_to_f16(d);
    float ds = kvqo_f16_to_f32(d16);
    blk[0] = (uint8_t)(d16 & 0xFF);
    blk[1] = (uint8_t)(d16 >> 8);
    for (int i = 0; i < 32; ++i) {
        int c = 0;
        if (ds != 0.0f) {
            float r = rintf(x[i] / ds);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            c = (int)r;
        }
        blk[2 + i] = (uint8_t)(int8_t)c;
    }
}

void kvqo_q8_0_decode(const uint8_t* blk, double* x) {
    uint16_t d16 = (uint16_t)(blk[0] | (blk[1] << 8));
    double ds = (double)kvqo_f16_to_f32(d16);
    for (int i = 0; i < 32; ++i)
        x[i] = ds * (double)(int8_t)blk[2 + i];
}

/* ------------------------------------------------------------------ */
/* e4m3: the 8-bit float of the FP8 K/V variant ("Module cache" index  */
/* page, item kv_fp8_on).  OCP FP8 E4M3: bit 7 sign, bits 6..3 biased  */
/* exponent (bias 7), bits 2..0 fraction.  Exponent field 0 holds zero  */
/* and the subnormals f * 2^-9; S.1111.111 is NaN; there is no          */
/* infinity, so the largest magnitude is 1.75 * 2^8 = 448.              */
/* ------------------------------------------------------------------ */
double kvqo_e4m3_value(uint8_t c) {
    const int neg = c >> 7, ex = (c >> 3) & 15, fr = c & 7;
    if (ex == 15 && fr == 7) return NAN;
    const double mag = (ex == 0) ? ldexp((double)fr, -9)           /* f/8 * 2^(1-7) */
                                 : ldexp(1.0 + fr / 8.0, ex - 7);
    return neg ? -mag : mag;
}

/* The code nearest to x: ties go to the code with an even fraction (of two
 * neighbours, whose codes differ by one, the even code), magnitudes past 448
 * give 0x7E = 448, the nearest finite code (saturation; the NaN code is
 * never chosen), and the sign bit is x's, also when the magnitude rounds to
 * zero.  The positive finite codes 0 .. 126 have rising values, so the two
 * candidates are the largest code whose value is at most |x| and the next
 * one; bisection finds them. */
static double e4m3_pos[127];              /* value of each positive finite code */

__attribute__((constructor)) static void e4m3_table(void) {
    for (int c = 0; c < 127; ++c) e4m3_pos[c] = kvqo_e4m3_value((uint8_t)c);
}

uint8_t kvqo_e4m3_from_f32(float x) {
    assert(!isnan(x));
    const double a = fabs((double)x);
    int best;
    if (a >= e4m3_pos[126]) {
        best = 126;
    } else {
        int lo = 0, hi = 126;             /* value(lo) <= a < value(hi) */
        while (hi - lo > 1) {
            const int mid = (lo + hi) / 2;
            if (e4m3_pos[mid] <= a) lo = mid; else hi = mid;
        }
        const double err_lo = a - e4m3_pos[lo];
        const double err_hi = e4m3_pos[hi] - a;
        if (err_lo < err_hi) best = lo;
        else if (err_hi < err_lo) best = hi;
        else best = (lo & 1) == 0 ? lo : hi;   /* a tie: the even code */
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

/* One block: 34 bytes = fp16 scale d (little-endian) + 32 e4m3 codes.   */
/* d = fp16(amax / 448); codes are e4m3(x / d) from the STORED d (an fp32 */
/* IEEE quotient rounded once to e4m3); all codes 0 when d is 0.          */
/* Value = d * e4m3 value.                                              */
void kvqo_f8_encode(const float* x, uint8_t* blk) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        assert(isfinite(x[i]));
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    }
    const uint16_t d16 = kvqo_f32_to_f16(amax / 448.0f);
    const float ds = kvqo_f16_to_f32(d16);
    blk[0] = (uint8_t)(d16 & 0xFF);
    blk[1] = (uint8_t)(d16 >> 8);
    for (int i = 0; i < 32; ++i)
        blk[2 + i] = (ds != 0.0f) ? kvqo_e4m3_from_f32(x[i] / ds) : 0;
}

void kvqo_f8_decode(const uint8_t* blk, double* x) {
    const double ds = (double)kvqo_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int i = 0; i < 32; ++i) x[i] = ds * kvqo_e4m3_value(blk[2 + i]);
}

/* ------------------------------------------------------------------ */
/* q5_1: 24 bytes = fp16 step d, fp16 offset m (the block minimum),     */
/* 4 bytes of fifth bits (bit i = bit 4 of code i, little-endian), 16   */
/* bytes of nibbles (byte j = code j low nibble | code j+16 << 4).      */
/* Codes from the STORED d and m, half-to-even, clamped to [0, 31].     */
/* Value = d*code + m.                                                  */
/* ------------------------------------------------------------------ */
void kvqo_q5_1_encode(const float* x, uint8_t* blk) {
    float mn = x[0], mx = x[0];
    for (int i = 0; i < 32; ++i) {
        assert(isfinite(x[i]));
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    /* signed zeros: a zero extreme is taken as +0, so that neither the stored
     * offset nor the step of a block is ever -0 */
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;
    float d = (mx - mn) / 31.0f;
    uint16_t d16 = kvqo_f32_to_f16(d);
    uint16_t m16 = kvqo_f32_to_f16(mn);
    float ds = kvqo_f16_to_f32(d16);
    float ms = kvqo_f16_to_f32(m16);
    int code[32];
    for (int i = 0; i < 32; ++i) {
        int c = 0;
        if (ds != 0.0f) {
            float r = rintf((x[i] - ms) / ds);
            if (r > 31.0f) r = 31.0f;
            if (r < 0.0f) r = 0.0f;
            c = (int)r;
        }
        code[i] = c;
    }
    uint32_t qh = 0;
    for (int i = 0; i < 32; ++i)
        qh |= (uint32_t)((code[i] >> 4) & 1) << i;
    blk[0] = (uint8_t)(d16 & 0xFF);
    blk[1] = (uint8_t)(d16 >> 8);
    blk[2] = (uint8_t)(m16 & 0xFF);
    blk[3] = (uint8_t)(m16 >> 8);
    for (int b = 0; b < 4; ++b)
        blk[4 + b] = (uint8_t)((qh >> (8 * b)) & 0xFF);
    for (int j = 0; j < 16; ++j)
        blk[8 + j] = (uint8_t)((code[j] & 15) | ((code[j + 16] & 15) << 4));
}

void kvqo_q5_1_decode(const uint8_t* blk, double* x) {
    uint16_t d16 = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t m16 = (uint16_t)(blk[2] | (blk[3] << 8));
    double ds = (double)kvqo_f16_to_f32(d16);
    double ms = (double)kvqo_f16_to_f32(m16);
    uint32_t qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) |
                  ((uint32_t)blk[6] << 16) | ((uint32_t)blk[7] << 24);
    for (int i = 0; i < 32; ++i) {
        int nib = (i < 16) ? (blk[8 + i] & 15) : (blk[8 + i - 16] >> 4);
        int c = nib | (int)(((qh >> i) & 1u) << 4);
        x[i] = ds * (double)c + ms;
    }
}

void kvqo_quantize_k(const float* x, int64_t n_elems, uint8_t* out) {
    assert(n_elems % 32 == 0);
    for (int64_t blk = 0; blk < n_elems / 32; ++blk)
        kvqo_q8_0_encode(x + 32 * blk, out + 34 * blk);
}

void kvqo_quantize_v(const float* x, int64_t n_elems, uint8_t* out) {
    assert(n_elems % 32 == 0);
    for (int64_t blk = 0; blk < n_elems / 32; ++blk)
        kvqo_q5_1_encode(x + 32 * blk, out + 24 * blk);
}

/* ------------------------------------------------------------------ */
/* FP8 token rows.  The pages name e4m3 K and V ("Module cache" index   */
/* page, kv_fp8_on) and give no layout.  Reading: a row of row_elems    */
/* (= n_kv_heads * head_dim) elements is encoded block by block as      */
/* kvqo_f8_encode does; the row holds the 32 codes of every block in    */
/* element order first (the code of element e is byte e), then the     */
/* fp16 scales of its blocks in block order (block k's at bytes         */
/* row_elems + 2k, little-endian): row_elems / 32 * 34 bytes, 34 per    */
/* 32 elements as for one block.                                        */
/* ------------------------------------------------------------------ */
void kvqo_quantize_f8_rows(const float* x, int64_t n_rows, int32_t row_elems, uint8_t* out) {
    assert(row_elems % 32 == 0);
    const int64_t row_bytes = (int64_t)row_elems / 32 * 34;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        uint8_t blk[34];
        uint8_t* row = out + r * row_bytes;
        for (int32_t k = 0; k < row_elems / 32; ++k) {
            kvqo_f8_encode(x + r * row_elems + 32 * k, blk);
            memcpy(row + 32 * k, blk + 2, 32);
            row[row_elems + 2 * k] = blk[0];
            row[row_elems + 2 * k + 1] = blk[1];
        }
    }
}

/* Bytes of one K or V token row, and the 32 dequantized values of block
 * kb of KV head g in such a row, for cache format fmt (KVQO_FMT_*). */
static int64_t row_bytes(int32_t fmt, int v_side, int32_t Hkv, int32_t nb) {
    if (fmt == KVQO_FMT_E4M3) return (int64_t)Hkv * nb * 34;
    return (int64_t)Hkv * nb * (v_side ? 24 : 34);
}

static void row_block(int32_t fmt, int v_side, const uint8_t* row, int32_t Hkv, int32_t nb,
                      int32_t g, int32_t kb, double* out) {
    const int64_t k = (int64_t)g * nb + kb;           /* block index in the row */
    if (fmt == KVQO_FMT_E4M3) {
        const int64_t row_elems = (int64_t)Hkv * nb * 32;
        const uint8_t* scale = row + row_elems + 2 * k;
        uint8_t blk[34];
        blk[0] = scale[0];
        blk[1] = scale[1];
        memcpy(blk + 2, row + 32 * k, 32);
        kvqo_f8_decode(blk, out);
    } else if (v_side) {
        kvqo_q5_1_decode(row + 24 * k, out);
    } else {
        kvqo_q8_0_decode(row + 34 * k, out);
    }
}

/* ------------------------------------------------------------------ */
/* Attention.  For session b, query row t and Q head h:                 */
/*   g     = h / hpk                       (GQA grouping)               */
/*   upto  = len_b - T + t + 1             (causal bound of row t)      */
/*   first = window ? max(0, upto - window) : 0                         */
/*   s_j   = scale * sum_d q[d] * K'[j, g, d]   for j in [first, upto)  */
/*   M     = max(max_j s_j, sink_h)        (sink only if given)         */
/*   Z     = sum_j exp(s_j - M) + exp(sink_h - M)                       */
/*   out   = sum_j exp(s_j - M) * V'[j, g, :] / Z,   lse = M + log Z    */
/* K', V' are the dequantized cache values, exact in double.            */
/* ------------------------------------------------------------------ */
static void one_query(int32_t fmt, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                      const float* q, const uint8_t* const* k_plane,
                      const uint8_t* const* v_plane, const int64_t* base,
                      const int64_t* len, int32_t window, const float* sinks,
                      float scale, int64_t b, int32_t t, int32_t h,
                      double* s, float* out, float* lse, int* bad) {
    const int32_t hpk = H / Hkv;
    const int32_t g = h / hpk;
    const int32_t nb = hd / 32;                    /* blocks per head */
    const int64_t k_row = row_bytes(fmt, 0, Hkv, nb);   /* bytes per K token row */
    const int64_t v_row = row_bytes(fmt, 1, Hkv, nb);   /* bytes per V token row */
    const int64_t upto = len[b] - T + t + 1;
    int64_t first = 0;
    if (window > 0) {
        first = upto - window;
        if (first < 0) first = 0;
    }
    if (upto <= first || first < base[b]) {
        *bad = 1;
        return;
    }
    const float* qv = q + (((int64_t)b * T + t) * H + h) * hd;
    double blk[32];

    double M = -INFINITY;
    for (int64_t j = first; j < upto; ++j) {
        const uint8_t* row = k_plane[b] + (j - base[b]) * k_row;
        double acc = 0.0;
        for (int32_t kb = 0; kb < nb; ++kb) {
            row_block(fmt, 0, row, Hkv, nb, g, kb, blk);
            for (int i = 0; i < 32; ++i)
                acc += (double)qv[32 * kb + i] * blk[i];
        }
        s[j - first] = (double)scale * acc;
        if (s[j - first] > M) M = s[j - first];
    }
    if (sinks && (double)sinks[h] > M) M = (double)sinks[h];

    double Z = 0.0;
    for (int64_t j = first; j < upto; ++j) {
        s[j - first] = exp(s[j - first] - M);   /* now the unnormalised weight */
        Z += s[j - first];
    }
    if (sinks) Z += exp((double)sinks[h] - M);

    float* o = out + (((int64_t)b * T + t) * H + h) * hd;
    double* acc = (double*)calloc((size_t)hd, sizeof(double));
    for (int64_t j = first; j < upto; ++j) {
        const uint8_t* row = v_plane[b] + (j - base[b]) * v_row;
        for (int32_t vb = 0; vb < nb; ++vb) {
            row_block(fmt, 1, row, Hkv, nb, g, vb, blk);
            for (int i = 0; i < 32; ++i)
                acc[32 * vb + i] += s[j - first] * blk[i];
        }
    }
    for (int32_t d = 0; d < hd; ++d)
        o[d] = (float)(acc[d] / Z);
    free(acc);
    if (lse) lse[((int64_t)b * T + t) * H + h] = (float)(M + log(Z));
}

int kvqo_attention(int32_t fmt, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                   const float* q,
                   const uint8_t* const* k_plane, const uint8_t* const* v_plane,
                   const int64_t* base, const int64_t* len, int32_t window,
                   const float* sinks, float scale,
                   const int64_t* sel, int64_t n_sel,
                   float* out, float* lse) {
    if (B <= 0 || T <= 0 || H <= 0 || Hkv <= 0 || hd <= 0 || hd % 32 != 0 ||
        H % Hkv != 0 || window < 0 || (fmt != KVQO_FMT_Q8_Q5 && fmt != KVQO_FMT_E4M3))
        return -1;
    int64_t max_rows = 0;
    for (int32_t b = 0; b < B; ++b)
        if (len[b] - base[b] > max_rows) max_rows = len[b] - base[b];
    const int64_t total = (int64_t)B * T * H;
    const int64_t n = sel ? n_sel : total;
    int bad = 0;

#pragma omp parallel reduction(| : bad)
    {
        double* s = (double*)malloc((size_t)(max_rows + 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            int64_t f = sel ? sel[i] : i;
            if (f < 0 || f >= total) { bad = 1; continue; }
            int32_t h = (int32_t)(f % H);
            int32_t t = (int32_t)((f / H) % T);
            int64_t b = f / ((int64_t)H * T);
            int lb = 0;
            one_query(fmt, T, H, Hkv, hd, q, k_plane, v_plane, base, len, window,
                      sinks, scale, b, t, h, s, out, lse, &lb);
            bad |= lb;
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Attention importance (cortiq-engine "Struct LayerKvCache",           */
/* attend_group's imp_acc and accumulate_imp): the probability mass     */
/* each stored row receives, summed over every query row t and Q head   */
/* h of the call.  With s_j, M and Z as for the attention above,        */
/*   p_j = exp(s_j - M) / Z     for j in [first, upto), else 0,         */
/* and imp[b][j - base_b] += p_j.  The sink takes its share of Z but    */
/* is no row, so nothing is added for it.  imp: double [B][cap],        */
/* indexed by physical row.                                             */
/* ------------------------------------------------------------------ */
int kvqo_importance(int32_t fmt, int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t hd,
                    const float* q, const uint8_t* const* k_plane,
                    const int64_t* base, const int64_t* len, int32_t window,
                    const float* sinks, float scale, double* imp, int64_t cap) {
    if (B <= 0 || T <= 0 || H <= 0 || Hkv <= 0 || hd <= 0 || hd % 32 != 0 ||
        H % Hkv != 0 || window < 0 || cap <= 0 || (fmt != KVQO_FMT_Q8_Q5 && fmt != KVQO_FMT_E4M3))
        return -1;
    const int32_t heads_per_group = H / Hkv;
    const int32_t blocks = hd / 32;
    const int64_t k_bytes = row_bytes(fmt, 0, Hkv, blocks);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t b = 0; b < B; ++b) {
        if (len[b] - base[b] > cap) { bad = 1; continue; }
        double* score = (double*)malloc((size_t)(len[b] + 1) * sizeof(double));
        double kdeq[32];
        for (int32_t t = 0; t < T && !bad; ++t) {
            const int64_t row_end = len[b] - T + t + 1;          /* rows below it are seen */
            const int64_t row_start = window > 0 && row_end > window ? row_end - window : 0;
            if (row_end <= row_start || row_start < base[b]) { bad = 1; break; }
            for (int32_t h = 0; h < H; ++h) {
                const int32_t kv_group = h / heads_per_group;
                const float* qrow = q + (((int64_t)b * T + t) * H + h) * hd;
                double top = -INFINITY;
                for (int64_t j = row_start; j < row_end; ++j) {
                    const uint8_t* krow = k_plane[b] + (j - base[b]) * k_bytes;
                    double dot = 0.0;
                    for (int32_t kb = 0; kb < blocks; ++kb) {
                        row_block(fmt, 0, krow, Hkv, blocks, kv_group, kb, kdeq);
                        for (int i = 0; i < 32; ++i) dot += kdeq[i] * (double)qrow[32 * kb + i];
                    }
                    score[j - row_start] = dot * (double)scale;
                    if (score[j - row_start] > top) top = score[j - row_start];
                }
                const double sink = sinks ? (double)sinks[h] : -INFINITY;
                if (sink > top) top = sink;
                double denom = sinks ? exp(sink - top) : 0.0;      /* the sink's share */
                for (int64_t j = row_start; j < row_end; ++j) denom += exp(score[j - row_start] - top);
                for (int64_t j = row_start; j < row_end; ++j)
                    imp[(int64_t)b * cap + (j - base[b])] += exp(score[j - row_start] - top) / denom;
            }
        }
        free(score);
    }
    return bad ? -1 : 0;
}

int kvqo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the attention loops use from now on (n >= 1); for timing the
 * oracle on one thread and on all of them. */
void kvqo_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

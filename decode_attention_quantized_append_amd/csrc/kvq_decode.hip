// kvq_decode.hip -- split-K flash decode over the quantized cache (gfx950).
// Included by kvq_kernels.hip (inside namespace kvq).
//
// What it computes (cortiq-engine "Struct LayerKvCache", attend_group and
// attend_group_upto; memra-engine "Struct KvLayer", len_d / base_d): for one
// session b, one KV head g and one chunk of logical rows, the unnormalised
// online-softmax partial (m, l, o) of each of the group's R = T*H/Hkv query
// rows.  Row r = t*hpk + hh is Q head g*hpk + hh at verify row t and sees the
// rows [max(0, upto_t - window), upto_t), upto_t = len - T + t + 1; the score is
// scale * <q, k> with k the dequantized q8_0 row.
//
// Organisation.  A workgroup is (session, chunk, KV head): 4 waves, each
// streaming its own 32-row tiles of the chunk (tiles w, w+4, ...) through a
// private LDS area, with no workgroup barrier inside the loop.  Per tile:
//   1. stage: K blocks are re-aligned (34-byte blocks sit at 2-byte alignment)
//      into [row][dim] code bytes plus fp32 scales; V blocks are unpacked from
//      q5_1 into [row][dim] code bytes (0..31) plus fp32 steps and fp16 offsets.
//   2. scores: S = Q K^T with v_mfma_f32_16x16x32_f16, one MFMA per 32-element
//      block: the codes are exact in fp16 and Q is split into fp16 hi (+ lo for
//      fp32 input); each lane owns one key of the output tile and scales the
//      block's partial dot products by that key's q8_0 scale in fp32.
//   3. online softmax in base 2 (v_exp_f32), row maxima by DPP row rotations.
//   4. P V with the same MFMA: P is written to LDS as [row][query] fp16 and
//      read back with ds_read_b64_tr_b16 as the A operand; V codes come back
//      as the B operand with ds_read_b64_tr_b8 (8 keys of one dim per lane),
//      so the token-major plane needs no explicit transpose.  The q5_1 step is
//      folded into P (P' = P * step per block) and the q5_1 offset term
//      sum_j P_j * m_j is one more MFMA against the [row][block] offsets.
// The four waves' partials are merged in a fixed order (deterministic), and
// one partial per (session, chunk, query row) goes to the workspace.
namespace dec {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i2 lds_i2;
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr int kWaves = 4;
constexpr int kTile = 32;                        // keys per wave tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int NB, int RT>
struct Layout {
    static constexpr int HD = NB * 32;
    static constexpr int KROW = NB * 32 + 16;    // padded row strides (bytes)
    static constexpr int VROW = NB * 32 + 16;
    static constexpr int PROW = 32;              // P rows: [rt][key][16] fp16
    static constexpr int KC = 0;                                  // K codes [32][KROW]
    static constexpr int VC = KC + kTile * KROW;                  // V codes [32][VROW]
    static constexpr int KS = VC + kTile * VROW;                  // K scales f32 [NB][32]
    static constexpr int VD = KS + ((kTile * NB * 4 + 15) & ~15); // V steps  f32 [NB][32]
    static constexpr int VM = VD + ((kTile * NB * 4 + 15) & ~15); // V offsets f16 [32][16]
    static constexpr int PU = VM + kTile * 32;                    // P  f16 [RT][32][16]
    static constexpr int PP = PU + RT * kTile * PROW;             // P' f16 [RT][32][16]
    static constexpr int WAVE = PP + RT * kTile * PROW;
    static constexpr int QFRAG = RT * NB * 64 * 16;               // Q fragments, fp16
    static constexpr int Q = kWaves * WAVE;
    static constexpr int ML = Q + 2 * QFRAG;                      // [wave][RT*16][2] f32
    static constexpr int QE = ML + kWaves * RT * 16 * 2 * 4;      // u32 exponent of the largest |q|
    static constexpr int BYTES = QE + 16;
    static_assert(BYTES <= kLdsBytes, "the per-head layout must fit a CU's LDS");
    static_assert(RT * 16 * HD * 4 <= kWaves * WAVE, "merge buffer must fit in the wave areas");
};

// 2^k as a binary32, for -126 <= k <= 127.
__device__ __forceinline__ float pow2(int k) { return __uint_as_float((uint32_t)(127 + k) << 23); }

// Query rows enter the matrix cores as fp16.  A row is first divided by a
// power of two chosen from the biased binary32 exponent e of its largest
// |q| (taken as at least 15): 2^(e - 141) maps that element into
// [2^14, 2^15), so every bf16 query is exact in fp16 whatever its magnitude,
// and the scores computed from the scaled row are multiplied back by
// q_up(e).  Both factors are normal binary32 numbers.
__device__ __forceinline__ float q_down(uint32_t e) { return pow2(141 - (int)max(e, 15u)); }
__device__ __forceinline__ float q_up(uint32_t e) { return pow2((int)max(e, 15u) - 141); }
// The biased exponent of a magnitude held as binary32 bits (sign cleared).
__device__ __forceinline__ uint32_t exp_of(uint32_t mag_bits) { return mag_bits >> 23; }

// P V takes P' = P * d (softmax weight times a V block's step) as fp16, with
// P <= 2^8.  While every step of a tile is below 2^7, P' < 2^15 (fp16 holds
// up to 65504).  A tile whose largest step dmax is larger has its steps
// stored times 2^-E, E = v_shift(dmax): then d * 2^-E < 2^7 again, and the
// wave's P V accumulator holds its sum in units of 2^-E (rescaled exactly,
// by a power of two, whenever E changes).
__device__ __forceinline__ int v_shift(float dmax) { return max(0, (int)(__float_as_uint(dmax) >> 23) - 133); }

__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false)));
    return v;
}

// Largest v over the wave, in every lane: DPP maxima within each row of 16
// lanes, then the four rows' results read as scalars (no lane-address
// registers, unlike shuffles).
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = row_max16(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Largest unsigned v over the wave, in every lane (as wave_max_dpp).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ float row_sum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
    return v;
}

// 4 unsigned bytes u -> two fp16 pairs (1024 + u): v_perm_b32 with 0x64 as the high byte.
__device__ __forceinline__ h2 bytes_lo(uint32_t x) {
    return __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u));
}
__device__ __forceinline__ h2 bytes_hi(uint32_t x) {
    return __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u));
}

// 8 signed q8_0 codes -> fp16 (exact): (c ^ 0x80) = c + 128, then 1024 + c + 128 - 1152.
__device__ __forceinline__ h8 k_codes_f16(uint32_t lo, uint32_t hi) {
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo ^= 0x80808080u;
    hi ^= 0x80808080u;
    h2 a = bytes_lo(lo) - off, b = bytes_hi(lo) - off, c = bytes_lo(hi) - off, d = bytes_hi(hi) - off;
    return (h8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 q5_1 codes (bytes 0..31) -> fp16 (exact).
__device__ __forceinline__ h8 v_codes_f16(uint32_t lo, uint32_t hi) {
    const h2 off = {(_Float16)1024.0f, (_Float16)1024.0f};
    h2 a = bytes_lo(lo) - off, b = bytes_hi(lo) - off, c = bytes_lo(hi) - off, d = bytes_hi(hi) - off;
    return (h8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// bit k of the low 4 bits of x -> bit 4 of byte k
__device__ __forceinline__ uint32_t fifth_bits(uint32_t x4) {
    uint32_t m;
    asm("v_mul_u32_u24 %0, %1, %2" : "=v"(m) : "v"(x4), "s"(0x204081u));
    return (m & 0x01010101u) << 4;
}

// LDS swizzles (32 banks of 4 bytes): a 16-lane group touches 32 distinct banks.
// K code rows: 8-byte chunk c of row `key` lives at chunk c ^ ((key >> 3) & 1).
__device__ __forceinline__ int kc_chunk(int key, int c) { return c ^ ((key >> 3) & 1); }
// P rows (16 halves = four 8-byte chunks): chunk c of row `key` at c ^ ((key >> 2) & 3).
__device__ __forceinline__ int p_chunk(int key, int c) { return c ^ ((key >> 2) & 3); }

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 tr16_pair(const uint8_t* p0, const uint8_t* p1) {
    s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
    s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1));
    h4 ha = __builtin_bit_cast(h4, a), hb = __builtin_bit_cast(h4, b);
    return (h8){ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
}

__device__ __forceinline__ void lds_order() {
    // DS instructions of one wave execute in order; this only stops the
    // compiler from moving LDS accesses across the point.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Raw blocks of one 32-row tile held in registers between the global loads
// and the LDS stores (software prefetch of the next tile).  Unit u = (row,
// block) with the block index fastest; lane handles units lane, lane+64, ...
template <int NB>
struct Raw {
    static constexpr int U = (kTile * NB + 63) / 64;
    uint32_t kw[U][8];     // aligned dwords from the code address rounded down
    uint32_t kt[U];        // code bytes 30, 31 (needed when the codes start 2 bytes in)
    uint32_t kh[U];        // scale bits | shift << 16
    uint2 va[U], vn0[U], vn1[U];
};

template <int NB>
__device__ __forceinline__ void stage_load(Raw<NB>& r, const uint8_t* kplane, const uint8_t* vplane,
                                           int k_row, int v_row, int t0, int lo, int c1, int base, int lane) {
#pragma unroll
    for (int x = 0; x < Raw<NB>::U; ++x) {
        const int u = x * 64 + lane;
        if (kTile * NB % 64 == 0 || u < kTile * NB) {
            const int key = u / NB, blk = u - key * NB;
            const int64_t row = (int64_t)(min(max(t0 + key, lo), c1 - 1) - base);
            const uint8_t* kb = kplane + row * k_row + blk * 34;
            const uint8_t* vb = vplane + row * v_row + blk * 24;
            // K: scale at kb, codes at kb + 2 (2-byte aligned)
            const uint32_t sh = (uint32_t)((reinterpret_cast<uintptr_t>(kb) + 2) & 3);
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(kb + 2 - sh);
#pragma unroll
            for (int i = 0; i < 8; ++i) r.kw[x][i] = kw[i];
            r.kt[x] = *reinterpret_cast<const uint16_t*>(kb + 32);
            r.kh[x] = (uint32_t)*reinterpret_cast<const uint16_t*>(kb) | (sh << 16);
            // V: [d16 | m16 << 16][fifth bits][16 nibble bytes], 8-byte aligned
            r.va[x] = reinterpret_cast<const uint2*>(vb)[0];
            r.vn0[x] = reinterpret_cast<const uint2*>(vb)[1];
            r.vn1[x] = reinterpret_cast<const uint2*>(vb)[2];
        }
    }
}

// Returns the largest V step this lane converted (for dec::v_shift).
template <int NB>
__device__ __forceinline__ float stage_store(const Raw<NB>& r, uint8_t* Wb, int lane, float sc2) {
    using LY = Layout<NB, 1>;
    float dmax = 0.0f;
    float* ks = reinterpret_cast<float*>(Wb + LY::KS);
    float* vd = reinterpret_cast<float*>(Wb + LY::VD);
    uint16_t* vm = reinterpret_cast<uint16_t*>(Wb + LY::VM);
#pragma unroll
    for (int x = 0; x < Raw<NB>::U; ++x) {
        const int u = x * 64 + lane;
        if (kTile * NB % 64 == 0 || u < kTile * NB) {
            const int key = u / NB, blk = u - key * NB;
            const uint32_t sh = r.kh[x] >> 16;
            uint32_t cd[8];
#pragma unroll
            for (int i = 0; i < 7; ++i) cd[i] = __builtin_amdgcn_alignbyte(r.kw[x][i + 1], r.kw[x][i], sh);
            cd[7] = __builtin_amdgcn_alignbyte(r.kt[x], r.kw[x][7], sh);
            uint4* kd = reinterpret_cast<uint4*>(Wb + LY::KC + key * LY::KROW + blk * 32);
            if (key & 8) {   // chunks 0<->1, 2<->3 (kc_chunk)
                kd[0] = (uint4){cd[2], cd[3], cd[0], cd[1]};
                kd[1] = (uint4){cd[6], cd[7], cd[4], cd[5]};
            } else {
                kd[0] = (uint4){cd[0], cd[1], cd[2], cd[3]};
                kd[1] = (uint4){cd[4], cd[5], cd[6], cd[7]};
            }
            ks[blk * kTile + key] = f16_value((uint16_t)(r.kh[x] & 0xFFFF)) * sc2;   // scale * log2(e) folded in
            const uint32_t qh = r.va[x].y;
            const uint32_t nib[4] = {r.vn0[x].x, r.vn0[x].y, r.vn1[x].x, r.vn1[x].y};
            uint32_t vc[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                vc[t] = (nib[t] & 0x0F0F0F0Fu) | fifth_bits((qh >> (4 * t)) & 15u);
                vc[4 + t] = ((nib[t] >> 4) & 0x0F0F0F0Fu) | fifth_bits((qh >> (16 + 4 * t)) & 15u);
            }
            uint4* vdst = reinterpret_cast<uint4*>(Wb + LY::VC + key * LY::VROW + blk * 32);
            vdst[0] = (uint4){vc[0], vc[1], vc[2], vc[3]};
            vdst[1] = (uint4){vc[4], vc[5], vc[6], vc[7]};
            const float dv = f16_value((uint16_t)(r.va[x].x & 0xFFFF));
            vd[blk * kTile + key] = dv;
            dmax = fmaxf(dmax, dv);
            vm[key * 16 + blk] = (uint16_t)(r.va[x].x >> 16);
        }
    }
    return dmax;
}

// Multiplies the V steps this lane stored (stage_store's units) by f.
template <int NB>
__device__ __forceinline__ void rescale_steps(uint8_t* Wb, int lane, float f) {
    float* vd = reinterpret_cast<float*>(Wb + Layout<NB, 1>::VD);
#pragma unroll
    for (int x = 0; x < Raw<NB>::U; ++x) {
        const int u = x * 64 + lane;
        if (kTile * NB % 64 == 0 || u < kTile * NB) vd[(u - (u / NB) * NB) * kTile + u / NB] *= f;
    }
}

// Per-wave state of the online softmax and the output accumulators.
template <int NB, int RT>
struct WaveState {
    f4 oacc[RT][2 * NB];     // O[r][d]: r = rt*16 + 4*q4 + i, d = 16*dt + j16
    f4 macc[RT];             // sum_key P[r][key] * m[key][blk], blk = j16
    float mrow[RT][4];       // reference max (base 2) of rows r
    float lsum[RT][4];       // this lane's share of the row sums
    int vis_lo[RT][4], vis_hi[RT][4];
    int full_lo, full_hi;    // every row sees all of [full_lo, full_hi)
    float qup;               // the query rows were divided by 1 / qup (q_down)
    int vsh;                 // oacc holds its sums in units of 2^-vsh (v_shift)
};

// One 32-row tile from the wave's LDS area: scores, online softmax, P V.
template <int NB, int RT, bool QLO>
__device__ __forceinline__ void tile_compute(WaveState<NB, RT>& ws, const uint8_t* smem, uint8_t* Wb,
                                             int t0, float sc2, int lane) {
    using LY = Layout<NB, RT>;
    const int q4 = lane >> 4, j16 = lane & 15;
    const float* ks = reinterpret_cast<const float*>(Wb + LY::KS);
    const float* vd = reinterpret_cast<const float*>(Wb + LY::VD);

    // ---- scores: sacc[rt][h][i] = S[r = rt*16 + 4*q4 + i][key = 16h + j16]
    f4 sacc[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sacc[rt][0] = sacc[rt][1] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        h8 qa[RT], ql[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            qa[rt] = *reinterpret_cast<const h8*>(smem + LY::Q + ((rt * NB + blk) * 64 + lane) * 16);
            if (QLO) ql[rt] = *reinterpret_cast<const h8*>(smem + LY::Q + LY::QFRAG + ((rt * NB + blk) * 64 + lane) * 16);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 16 * h + j16;
            const uint2 kraw = *reinterpret_cast<const uint2*>(Wb + LY::KC + key * LY::KROW + blk * 32 +
                                                               8 * kc_chunk(key, q4));
            const h8 kf = k_codes_f16(kraw.x, kraw.y);
            const float kscale = ks[blk * kTile + key];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f4 d = mfma(qa[rt], kf, (f4){0.f, 0.f, 0.f, 0.f});
                if (QLO) d = mfma(ql[rt], kf, d);
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[rt][h][i] = fmaf(kscale, d[i], sacc[rt][h][i]);
            }
        }
    }

    // ---- online softmax in base 2 against a reference max mrow that only
    // moves when a score exceeds it by more than 8 (so p = 2^(s - mrow) <= 256,
    // well inside fp16).  The common case needs no row maximum: one compare
    // per score and a wave vote; only when some score passes its row's
    // threshold are the row maxima taken and the accumulators rescaled.
    float sv[RT][2][4];
    const bool interior = t0 >= ws.full_lo && t0 + kTile <= ws.full_hi;   // no score masked
    bool over = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s0 = sacc[rt][0][i] * ws.qup, s1 = sacc[rt][1][i] * ws.qup;
            if (!interior) {
                const int j0 = t0 + j16, j1 = t0 + 16 + j16;
                s0 = (j0 >= ws.vis_lo[rt][i] && j0 < ws.vis_hi[rt][i]) ? s0 : -INFINITY;
                s1 = (j1 >= ws.vis_lo[rt][i] && j1 < ws.vis_hi[rt][i]) ? s1 : -INFINITY;
            }
            sv[rt][0][i] = s0;
            sv[rt][1][i] = s1;
            over |= fmaxf(s0, s1) > ws.mrow[rt][i] + 8.0f;      // -inf never passes
        }
    if (__any(over)) {
        float alpha[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mt = row_max16(fmaxf(sv[rt][0][i], sv[rt][1][i]));
                const float mold = ws.mrow[rt][i];
                const bool move = mt > mold + 8.0f;
                alpha[rt][i] = move ? __builtin_amdgcn_exp2f(mold - mt) : 1.0f;   // 0 when mold is -inf
                ws.mrow[rt][i] = move ? mt : mold;
                ws.lsum[rt][i] *= alpha[rt][i];
            }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt) ws.oacc[rt][dt][i] *= alpha[rt][i];
                ws.macc[rt][i] *= alpha[rt][i];
            }
    }
    float pv[RT][2][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m = ws.mrow[rt][i];
            // rows that have seen nothing yet (m = -inf) give p = 0
            const float p0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[rt][0][i] - m);
            const float p1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[rt][1][i] - m);
            ws.lsum[rt][i] += p0 + p1;
            pv[rt][0][i] = p0;
            pv[rt][1][i] = p1;
        }
    // P to LDS as [rt][key][16] fp16
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const h4 ph = {(_Float16)pv[rt][h][0], (_Float16)pv[rt][h][1], (_Float16)pv[rt][h][2],
                           (_Float16)pv[rt][h][3]};
            const int key = 16 * h + j16;
            *reinterpret_cast<h4*>(Wb + LY::PU + (rt * kTile + key) * LY::PROW + 8 * p_chunk(key, q4)) = ph;
        }

    // ---- P V.  tr16 rows: keys 8*q4 + (j16>>2) (+4), columns r; lane j16 supplies chunk j16&3.
    const int trow = 8 * q4 + (j16 >> 2);
    const int tcol = 8 * (j16 & 3);                           // unswizzled (offset rows)
    const int pcol0 = 8 * p_chunk(trow, j16 & 3);             // P rows trow
    const int pcol1 = 8 * p_chunk(trow + 4, j16 & 3);         // P rows trow + 4
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 16 * h + j16;
            const float st = vd[blk * kTile + key];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const h4 ph = {(_Float16)(pv[rt][h][0] * st), (_Float16)(pv[rt][h][1] * st),
                               (_Float16)(pv[rt][h][2] * st), (_Float16)(pv[rt][h][3] * st)};
                *reinterpret_cast<h4*>(Wb + LY::PP + (rt * kTile + key) * LY::PROW + 8 * p_chunk(key, q4)) = ph;
            }
        }
        lds_order();
        h8 pa[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            pa[rt] = tr16_pair(Wb + LY::PP + (rt * kTile + trow) * LY::PROW + pcol0,
                               Wb + LY::PP + (rt * kTile + trow + 4) * LY::PROW + pcol1);
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
            const int d0 = blk * 32 + 16 * dd;
            const i2 vb = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i2*)(Wb + LY::VC + (8 * q4 + (j16 >> 1)) * LY::VROW + d0 + 8 * (j16 & 1)));
            const h8 vf = v_codes_f16((uint32_t)vb[0], (uint32_t)vb[1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) ws.oacc[rt][2 * blk + dd] = mfma(pa[rt], vf, ws.oacc[rt][2 * blk + dd]);
        }
        lds_order();   // the next block overwrites P'
    }
    // q5_1 offset term: macc[r][blk] += sum_key P[r][key] * m[key][blk]
    {
        const h8 mb = tr16_pair(Wb + LY::VM + trow * 32 + tcol, Wb + LY::VM + (trow + 4) * 32 + tcol);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const h8 pu = tr16_pair(Wb + LY::PU + (rt * kTile + trow) * LY::PROW + pcol0,
                                    Wb + LY::PU + (rt * kTile + trow + 4) * LY::PROW + pcol1);
            ws.macc[rt] = mfma(pu, mb, ws.macc[rt]);
        }
    }
    lds_order();   // the next tile's staging overwrites this tile
}

// Tiles prefetched ahead of the one being computed: two, unless the register
// file cannot hold them next to the accumulators (head_dim 256 with 32 rows).
template <int NB, int RT>
constexpr int prefetch_depth() { return NB * RT >= 12 ? 1 : 2; }

// Workgroups per CU the register allocation targets: two (two waves per SIMD)
// where the accumulators and the prefetch buffers fit in 256 registers.
template <int NB, int RT>
constexpr int min_blocks() { return NB * RT <= 4 ? 2 : 1; }

// Unit u of the decode grid -> (session b, chunk s).  The units are the
// (session, chunk) pairs that hold rows, sessions in order, so that the grid
// has no empty workgroups and an XCD's contiguous share of it is a fair share
// of the rows whatever the length mix.  Chunk counts come from the device
// lengths, 64 sessions per step (a wave-wide prefix sum).  b = -1 past the
// last unit; len and base are session b's counters, read in the same step.
// Every lane of the wave calls it with the same u.
__device__ __forceinline__ void locate_unit(const DecodeParams& p, int u, int& b, int& s, int& len_b, int& base_b) {
    const int lane = threadIdx.x & 63;
    int fb = -1, fs = 0, fl = 0, fbase = 0;
    for (int b0 = 0; b0 < p.B && fb < 0; b0 += 64) {
        const int bb = b0 + lane;
        int n = 0, len = 0, base = 0;
        if (bb < p.B) {
            len = p.len_d[bb];
            base = p.base_d[bb];
            const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
            const int span = len - (lo & ~31);
            n = span > 0 ? (span + p.chunk - 1) / p.chunk : 0;
        }
        int incl = n;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (u < total) {
            const int lb = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(incl > u)));
            fb = b0 + lb;
            fs = u - __builtin_amdgcn_readlane(incl - n, lb);
            fl = __builtin_amdgcn_readlane(len, lb);
            fbase = __builtin_amdgcn_readlane(base, lb);
        } else {
            u -= total;
        }
    }
    b = __builtin_amdgcn_readfirstlane(fb);
    s = __builtin_amdgcn_readfirstlane(fs);
    len_b = __builtin_amdgcn_readfirstlane(fl);
    base_b = __builtin_amdgcn_readfirstlane(fbase);
}

template <int NB, int RT, bool QLO>
__global__ __launch_bounds__(256, (min_blocks<NB, RT>())) void decode_mfma(DecodeParams p) {
    using LY = Layout<NB, RT>;
    constexpr int HD = LY::HD;
    constexpr int KSEG = NB * 34;
    constexpr int VSEG = NB * 24;
    constexpr int NFRAG = RT * NB * 64;
    constexpr int FPT = (NFRAG + 255) / 256;              // Q fragments per thread
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q4 = lane >> 4, j16 = lane & 15;

    // XCD-aware order: consecutive logical items (the KV heads of one chunk)
    // land on one XCD, which receives every 8th workgroup id.
    const int W = gridDim.x;
    const int wid = blockIdx.x;
    const int L = (wid & 7) * (W >> 3) + (wid >> 3);
    const int g = L % p.Hkv;
    int b, s, len, base;
    locate_unit(p, L / p.Hkv, b, s, len, base);
    if (b < 0) return;
    // query rows tq0 .. tq0 + Tq - 1 of the T: the grid's y index is the
    // group of Tg rows
    const int tq0 = blockIdx.y * p.Tg, Tq = min(p.Tg, p.T - tq0);
    const int R = Tq * p.hpk;

    // Q fragment (rt, blk) lane l: q[r = rt*16 + l%16][blk*32 + 8*(l/16) .. +7].
    // Loaded first: they do not depend on the session length.
    float qv[FPT][8];
#pragma unroll
    for (int x = 0; x < FPT; ++x) {
        const int f = x * 256 + tid;
        const int l = f & 63, fb = f >> 6;
        const int blk = fb % NB, rt = fb / NB;
        const int r = rt * 16 + (l & 15);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[x][e] = 0.0f;
        if (f < NFRAG && r < R) {
            const int t = tq0 + r / p.hpk, hh = r % p.hpk;
            const size_t i0 = (((size_t)b * p.T + t) * p.H + g * p.hpk + hh) * HD + blk * 32 + 8 * (l >> 4);
            if (p.dtype == 1) {
                const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + i0);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    qv[x][2 * e] = __uint_as_float(w4[e] << 16);
                    qv[x][2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
                }
            } else {
                const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + i0);
                const float4 c = *reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + i0 + 4);
                qv[x][0] = a.x; qv[x][1] = a.y; qv[x][2] = a.z; qv[x][3] = a.w;
                qv[x][4] = c.x; qv[x][5] = c.y; qv[x][6] = c.z; qv[x][7] = c.w;
            }
        }
    }

    const int lo_all = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int c0 = (lo_all & ~31) + s * p.chunk;   // chunks start on a 32-row boundary
    const int c1 = min(c0 + p.chunk, len);
    if (c0 >= c1) return;

    const uint8_t* kplane = p.k_planes + (int64_t)b * p.k_stride + (int64_t)g * KSEG;
    const uint8_t* vplane = p.v_planes + (int64_t)b * p.v_stride + (int64_t)g * VSEG;
    constexpr int kStride = kWaves * kTile;
    constexpr int kDepth = prefetch_depth<NB, RT>();
    // prefetch the wave's first kDepth tiles before anything waits on memory
    // (row indices are clamped to [lo_all, c1 - 1], so every load reads a
    // resident row)
    const int first = c0 + wave * kTile;
    Raw<NB> raw[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
        stage_load<NB>(raw[i], kplane, vplane, p.k_row, p.v_row, first + i * kStride, lo_all, c1, base, lane);

    // the exponent of the largest |q| of the workgroup's query rows (whose
    // fragments every wave holds a part of) meets in LDS; the rows are
    // divided by q_down of it, and the scores multiplied back by q_up
    uint32_t* const qexp = reinterpret_cast<uint32_t*>(smem + LY::QE);
    if (tid == 0) *qexp = 0;
    __syncthreads();
    {
        uint32_t mag = 0;
#pragma unroll
        for (int x = 0; x < FPT; ++x)
#pragma unroll
            for (int e = 0; e < 8; ++e) mag = max(mag, __float_as_uint(qv[x][e]) & 0x7FFFFFFFu);
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, m));
        if (lane == 0) atomicMax(qexp, exp_of(mag));
    }
    __syncthreads();
    const uint32_t qe = __builtin_amdgcn_readfirstlane(*qexp);
#pragma unroll
    for (int x = 0; x < FPT; ++x) {
        const int f = x * 256 + tid;
        if (f < NFRAG) {
            const float down = q_down(qe);
            h8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xs = qv[x][e] * down;
                const _Float16 xh = (_Float16)xs;
                hi[e] = xh;
                lo[e] = (_Float16)(xs - (float)xh);
            }
            *reinterpret_cast<h8*>(smem + LY::Q + f * 16) = hi;
            if (QLO) *reinterpret_cast<h8*>(smem + LY::Q + LY::QFRAG + f * 16) = lo;
        }
    }

    WaveState<NB, RT> ws;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        ws.macc[rt] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt) ws.oacc[rt][dt] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ws.mrow[rt][i] = -INFINITY;
            ws.lsum[rt][i] = 0.0f;
            const int r = rt * 16 + 4 * q4 + i;
            int hi = 0, lo = 0;
            if (r < R) {
                hi = len - p.T + tq0 + r / p.hpk + 1;
                lo = p.window > 0 ? max(0, hi - p.window) : 0;
            }
            ws.vis_lo[rt][i] = max(lo, c0);
            ws.vis_hi[rt][i] = min(hi, c1);
        }
    }
    ws.qup = q_up(qe);
    ws.vsh = 0;
    // rows' visible ranges are nested by t; the intersection over real rows
    ws.full_hi = min(len - p.T + tq0 + 1, c1);
    ws.full_lo = max(p.window > 0 ? max(0, len - p.window) : 0, c0);
    const float sc2 = p.scale * kLog2e;
    __syncthreads();   // Q fragments are in LDS

    uint8_t* Wb = smem + wave * LY::WAVE;
    // kDepth-deep pipeline, unrolled so that the register buffers keep static
    // indices, and branch-free inside so that the compiler's wait counts see
    // the loads of every buffer in issue order: a tile past c1 (only in a
    // session's last chunk) is computed fully masked and adds nothing.
    for (int t0 = first; t0 < c1; t0 += kDepth * kStride) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {
            const int tt = t0 + i * kStride;
            const float dmax = stage_store<NB>(raw[i], Wb, lane, sc2);
            // steps of 2^7 or more: the tile's steps are stored times
            // 2^-vsh (v_shift) and the accumulators switch units
            const bool big = __any(dmax >= 128.0f);   // wave-uniform
            if (big || ws.vsh != 0) {
                const int want = big ? __builtin_amdgcn_readfirstlane(v_shift(wave_max_dpp(dmax))) : 0;
                if (want != ws.vsh) {
                    const float f = pow2(ws.vsh - want);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                            for (int e = 0; e < 4; ++e) ws.oacc[rt][dt][e] *= f;
                    ws.vsh = want;
                }
                rescale_steps<NB>(Wb, lane, pow2(-ws.vsh));
            }
            lds_order();
            stage_load<NB>(raw[i], kplane, vplane, p.k_row, p.v_row, tt + kDepth * kStride, lo_all, c1, base, lane);
            tile_compute<NB, RT, QLO>(ws, smem, Wb, tt, sc2, lane);
        }
    }

    // ---- finish the wave: full row sums, fold the offset term into O
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ws.lsum[rt][i] = row_sum16(ws.lsum[rt][i]);
    const float ounit = pow2(ws.vsh);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ws.oacc[rt][dt][i] = fmaf(ws.oacc[rt][dt][i], ounit, __shfl(ws.macc[rt][i], 16 * q4 + dt / 2));

    // ---- merge the four waves in a fixed order
    float* ml = reinterpret_cast<float*>(smem + LY::ML);
    if (j16 == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rt * 16 + 4 * q4 + i;
                ml[(wave * RT * 16 + r) * 2] = ws.mrow[rt][i];
                ml[(wave * RT * 16 + r) * 2 + 1] = ws.lsum[rt][i];
            }
    }
    __syncthreads();   // all waves are past their tiles; the wave areas become the merge buffer
    float fac[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = rt * 16 + 4 * q4 + i;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[(w * RT * 16 + r) * 2]);
            fac[rt][i] = (ws.mrow[rt][i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ws.mrow[rt][i] - M);
        }
    float* obuf = reinterpret_cast<float*>(smem);
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = rt * 16 + 4 * q4 + i;
                        float* o = obuf + r * HD + 16 * dt + j16;
                        const float v = ws.oacc[rt][dt][i] * fac[rt][i];
                        *o = (w == 0) ? v : *o + v;
                    }
        }
        __syncthreads();
    }
    const size_t row0 = ((size_t)b * p.splits + s) * p.T;
    for (int r = tid; r < R; r += 256) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[(w * RT * 16 + r) * 2]);
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = ml[(w * RT * 16 + r) * 2];
            if (mw != -INFINITY) l += ml[(w * RT * 16 + r) * 2 + 1] * __builtin_amdgcn_exp2f(mw - M);
        }
        const int t = tq0 + r / p.hpk, h = g * p.hpk + r % p.hpk;
        const size_t idx = (row0 + t) * p.H + h;
        p.part_ml[2 * idx] = (M == -INFINITY) ? -INFINITY : M * kLn2;
        p.part_ml[2 * idx + 1] = l;
    }
    for (int e = tid; e < R * HD; e += 256) {
        const int r = e / HD, d = e - r * HD;
        const int t = tq0 + r / p.hpk, h = g * p.hpk + r % p.hpk;
        p.part_o[((row0 + t) * p.H + h) * HD + d] = obuf[r * HD + d];
    }
}

}  // namespace dec

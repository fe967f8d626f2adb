// kvq_decode_prime.hip -- split-K decode for many query rows per KV head (a
// prompt chunk), each KV tile unpacked once for eight query-row groups
// (gfx950).  Included by kvq_kernels.hip (inside namespace kvq), after
// kvq_decode_stream.hip.
//
// The same partials as the other decode kernels (cortiq-engine "Struct
// LayerKvCache", attend_group_upto: every query row of the chunk attends
// causally, within its window; memra-engine "Module cache", prime of a
// prompt chunk into the ring):
//   * a workgroup is (session, chunk of rows, KV head) on the grid's x index
//     and a block of eight query-row groups on its y index; wave w computes
//     group 8 y + w (32 query rows: Tg positions x hpk heads, two 16-row
//     tiles) over all the head's dims.
//   * per 32-row tile, the eight waves copy the tile's q8_0 / q5_1 blocks of
//     the head into LDS together (global_load_lds_dwordx4, one instruction or
//     two per wave) and then convert them together, once, into fp16 operands
//     in LDS.  K: each element d * c (step times code) as an exact pair of
//     fp16 values hi + lo (c has 8 significant bits and d 11, so hi holds the
//     product rounded to 11 bits and lo the rest exactly), which lets the
//     matrix cores sum the four blocks of a head in one accumulator with no
//     per-block scaling.  V: the codes as fp16 subnormals c * 2^-24 (exact),
//     the steps and the offsets; as in the stream kernel each wave multiplies
//     its fp16 P by the steps (P' = P * d, the A operand of P V) and takes
//     the offset term sum_key P * m, with the row sums from a column of ones,
//     as one more product.  FP8 (e4m3) rows (memra-engine "Module cache",
//     kv_fp8_on): K the same pairs (a code has 4 significant bits), V the
//     codes' fp16 values (exact) with no offsets; rows past the loaded ones
//     are written as zeros (e4m3 has NaN codes).  Each wave reads its
//     matrix-core operands from
//     there: ds_read_b128 for the K blocks (A of S^T = K Q^T), pairs of
//     ds_read_b64_tr_b16 for the V codes (B of P V, 8 keys of one dim per
//     lane).
//   * three raw tile buffers and three converted ones, one workgroup barrier
//     per tile: in the iteration of tile t a wave takes the scores of tile
//     t + 1 on the matrix cores before the softmax and P V of tile t, the
//     waves convert tile t + 2 (whose rows have landed), and tiles t + 3 and
//     t + 4 are in flight.  The two waves that share a SIMD take the
//     conversion and the products in opposite orders, so that one works the
//     vector ALU while the other works the matrix cores.
//   * ranges: a tile with a K step of 2^8 (FP8: 2^7) or more stores its K products
//     times 2^-E (and its scores are multiplied back by 2^E), a tile with a
//     V step of 2^7 or more its steps times 2^-E (and the P V accumulators
//     switch units), so that no fp16 product overflows; the query rows are
//     scaled by a power of two as in the stream kernel, and P (at most 2^8,
//     the lazily moved reference max) enters as fp16.
namespace prime {

using dec::f4;
using dec::h8;
using dec::kLn2;
using dec::kLog2e;

constexpr int kTile = kRowTile;
constexpr int kWaves = kPrimeGroups;
constexpr int kRawBufs = kPrimeRawBufs;
constexpr int kConvBufs = kPrimeConvBufs;

// vmcnt(n) for a count known only at run time (n < 0: wait for all).
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 1: stream::wait_loads_upto<1>(); break;
        case 2: stream::wait_loads_upto<2>(); break;
        case 3: stream::wait_loads_upto<3>(); break;
        case 4: stream::wait_loads_upto<4>(); break;
        case 5: stream::wait_loads_upto<5>(); break;
        case 6: stream::wait_loads_upto<6>(); break;
        case 7: stream::wait_loads_upto<7>(); break;
        default:
            if (n >= 8) stream::wait_loads_upto<8>();
            else stream::wait_loads_upto<0>();
    }
}

template <int NB, bool QLO, bool F8>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_prime(DecodeParams p) {
    using LY = PrimeLayout<NB, F8>;
    static_assert(LY::BYTES <= kLdsBytes, "the prime layout must fit a CU's LDS");
    using WN = typename LY::WN;
    constexpr int HD = LY::HD;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q4 = lane >> 4, j16 = lane & 15;

    // ---- the unit: (session, chunk, KV head) from the grid's x index, XCD by XCD
    const int W = gridDim.x, wid = blockIdx.x;
    const int L = (wid & 7) * (W >> 3) + (wid >> 3);
    const int g = L % p.Hkv;
    int b, s, len, base;
    dec::locate_unit(p, L / p.Hkv, b, s, len, base);
    if (b < 0) return;
    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int c0 = (lo & ~(kTile - 1)) + s * p.chunk;
    const int c1 = min(c0 + p.chunk, len);
    if (c0 >= c1) return;
    // this workgroup's query positions, and the rows any of them sees
    const int ngroups = (p.T + p.Tg - 1) / p.Tg;
    const int gfirst = blockIdx.y * kWaves;
    const int wlo = gfirst * p.Tg, whi = min(p.T, (gfirst + kWaves) * p.Tg);
    const int seen_lo = p.window > 0 ? max(0, len - p.T + wlo + 1 - p.window) : 0;
    const int seen_hi = len - p.T + whi;          // one past the last row the last position sees
    const int t_begin = max(c0, seen_lo & ~(kTile - 1));
    const int t_end = min(c1, seen_hi);
    const int ntiles = t_begin < t_end ? (t_end - t_begin + kTile - 1) / kTile : 0;

    // this wave's query rows
    const int grp = gfirst + wave;
    const bool active = grp < ngroups;
    const int tq0 = active ? grp * p.Tg : 0;
    const int Tq = active ? min(p.Tg, p.T - tq0) : 0;
    const int R = Tq * p.hpk;

    // ---- tile loads: instruction i of a tile's NIT (K pieces, then V pieces)
    // is issued by wave i mod 8.  q8_0 / q5_1: the K blocks from the 16-byte
    // boundary at or below them (kofs bytes before), the V blocks exactly.
    // FP8 rows: the head's codes (16-byte aligned), then the 16-byte piece of
    // the row's scale area that holds its NB scales (at sofs within it); the
    // same for K and V.
    const int kstart = F8 ? g * NB * 32 : g * NB * 34;
    const int kofs = F8 ? 0 : (kstart & 15);
    const int sofs = F8 ? (g * 2 * NB) & 15 : 0;
    const int spiece = F8 ? p.Hkv * p.hd + ((g * 2 * NB) & ~15) : 0;
    const uint8_t* const kwin = p.k_planes + (int64_t)b * p.k_stride + (F8 ? 0 : kstart - kofs);
    const uint8_t* const vwin = p.v_planes + (int64_t)b * p.v_stride + (F8 ? 0 : g * NB * 24);
    // this wave's load instructions for the tile at t0: 0 past the last
    // tile, -1 for a partial tile (its wave-wide empty loads may be skipped,
    // so that only a wait for all loads is safe behind it)
    auto my_loads = [&](int t0) -> int {
        if (t0 >= t_begin + ntiles * kTile) return 0;
        if (t0 + kTile > c1) return -1;
        return (LY::NIT - wave + kWaves - 1) / kWaves;
    };
    auto issue = [&](int t0, int buf) {
        asm volatile("" ::: "memory");
        const int nrows = min(kTile, c1 - t0);
        uint8_t* const rb = smem + buf * LY::RAW;
        for (int i = wave; i < LY::NIT; i += kWaves) {
            if (i < WN::NKI) {
                const int pc = i * 64 + lane, row = pc / WN::KWP, col = pc - row * WN::KWP;
                const uint32_t off = F8 ? (uint32_t)(row * p.k_row + (col < 2 * NB ? kstart + col * 16 : spiece))
                                        : (uint32_t)(row * p.k_row + min(col, WN::KW - 1) * 16);
                if (pc < nrows * WN::KWP)
                    stream::dma16(kwin + (int64_t)(t0 - base) * p.k_row, off, rb + LY::RK + i * 1024);
            } else {
                const int x = i - WN::NKI;
                const int pc = x * 64 + lane, row = pc / WN::VWP, col = pc - row * WN::VWP;
                const uint32_t off = F8 ? (uint32_t)(row * p.v_row + (col < 2 * NB ? kstart + col * 16 : spiece))
                                        : (uint32_t)(row * p.v_row + min(col, WN::VW - 1) * 16);
                if (pc < nrows * WN::VWP)
                    stream::dma16(vwin + (int64_t)(t0 - base) * p.v_row, off, rb + LY::RV + x * 1024);
            }
        }
    };

    // ---- conversion of one tile's raw rows into fp16 operands (all waves).
    // First every wave finds the tile's range shifts itself (the same values
    // in every wave): E_k for K steps of 2^8 or more (FP8: 2^7, codes up to
    // 448), E_v for V steps of 2^7 or more (fp16 bits 0x5C00, 0x5800).  Rows
    // past c1 were not loaded: their steps and offsets are taken as 0, so
    // that their products are 0 whatever stale bytes their q8_0 / q5_1 codes
    // hold, and their FP8 codes (which may be NaN) as 0.
    uint32_t ksh_next = 0, vsh_next = 0;     // the shifts of the tile last converted
    auto convert = [&](int t0, int rbuf, int cbuf) {
        const uint8_t* const rk = smem + rbuf * LY::RAW + LY::RK;
        const uint8_t* const rv = smem + rbuf * LY::RAW + LY::RV;
        uint8_t* const cv = smem + kRawBufs * LY::RAW + cbuf * LY::CONV;
        const int tid = threadIdx.x;
        // a K row's step (its fp16 bits, sign cleared); a V row's step in the
        // low half and (q5_1) its offset in the high half
        auto kstep = [&](int key, int blk) -> uint32_t {
            const int o = F8 ? key * WN::KSTR + 32 * NB + sofs + 2 * blk : key * WN::KSTR + kofs + blk * 34;
            return t0 + key < c1 ? *reinterpret_cast<const uint16_t*>(rk + o) & 0x7FFFu : 0u;
        };
        auto vstepm = [&](int key, int blk) -> uint32_t {
            if constexpr (F8)
                return t0 + key < c1 ? *reinterpret_cast<const uint16_t*>(rv + key * WN::VSTR + 32 * NB + sofs + 2 * blk) : 0u;
            return t0 + key < c1 ? *reinterpret_cast<const uint32_t*>(rv + key * WN::VSTR + blk * 24) : 0u;
        };
        {
            uint32_t km = 0, vm = 0;
#pragma unroll
            for (int x = 0; x < (kTile * NB + 63) / 64; ++x) {
                const int u = x * 64 + lane;
                if (kTile * NB % 64 == 0 || u < kTile * NB) {
                    km = max(km, kstep(u / NB, u % NB));
                    vm = max(vm, vstepm(u / NB, u % NB) & 0x7FFFu);
                }
            }
            constexpr uint32_t kbig = F8 ? 0x5800u : 0x5C00u, kexp = F8 ? 21u : 22u;
            ksh_next = __any(km >= kbig) ? (dec::wave_max_u32(km) >> 10) - kexp : 0u;
            vsh_next = __any(vm >= 0x5800u) ? (dec::wave_max_u32(vm) >> 10) - 21u : 0u;
        }
        const _Float16 kdown = (_Float16)dec::pow2(-(int)ksh_next);
        // K: task (key, blk, quarter) -> 8 products d * c as hi + lo
        for (int u = tid; u < kTile * NB * 4; u += 64 * kWaves) {
            const int key = u / (NB * 4), rem = u - key * (NB * 4), blk = rem >> 2, qq = rem & 3;
            h8 c;
            if constexpr (F8) {
                const uint2 c8 = t0 + key < c1 ? *reinterpret_cast<const uint2*>(rk + key * WN::KSTR + blk * 32 + 8 * qq)
                                               : make_uint2(0u, 0u);
                c = stream::e4m3_codes(c8.x, c8.y);
            } else {
                const int ca = key * WN::KSTR + kofs + blk * 34 + 2 + 8 * qq;
                const uint32_t* const w = reinterpret_cast<const uint32_t*>(rk + (ca & ~3));
                const uint32_t sh = (uint32_t)(ca & 3) * 8;
                c = dec::k_codes_f16(__builtin_amdgcn_alignbit(w[1], w[0], sh), __builtin_amdgcn_alignbit(w[2], w[1], sh));
            }
            const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)kstep(key, blk)) * kdown;
            const h8 dv = {d, d, d, d, d, d, d, d};
            const h8 hi = c * dv;
            const h8 lo = __builtin_elementwise_fma(c, dv, -hi);   // c * d - hi fits in fp16 (exactly, unless tiny)
            const int o = key * LY::ROWH + (blk * 32 + 8 * qq) * 2;
            *reinterpret_cast<h8*>(cv + LY::KH + o) = hi;
            *reinterpret_cast<h8*>(cv + LY::KL + o) = lo;
        }
        // V: task (key, blk, part) -> dims 8 part .. 8 part + 7 of the block
        for (int u = tid; u < kTile * NB * 4; u += 64 * kWaves) {
            const int key = u / (NB * 4), rem = u - key * (NB * 4), blk = rem >> 2, part = rem & 3;
            if constexpr (F8) {
                const uint2 c8 = t0 + key < c1 ? *reinterpret_cast<const uint2*>(rv + key * WN::VSTR + blk * 32 + 8 * part)
                                               : make_uint2(0u, 0u);
                *reinterpret_cast<h8*>(cv + LY::VH + key * LY::ROWV + (blk * 32 + 8 * part) * 2) = stream::e4m3_codes(c8.x, c8.y);
                continue;
            }
            const uint8_t* const vb = rv + key * WN::VSTR + blk * 24;
            const uint2 nibw = *reinterpret_cast<const uint2*>(vb + 8 + 8 * (part & 1));
            const uint32_t qh = *reinterpret_cast<const uint32_t*>(vb + 4);
            const uint32_t hb = (qh >> (8 * part)) & 0xFFu;    // the fifth bits of dims 8 part .. + 7
            const uint32_t shn = (part >> 1) * 4;              // high nibbles for dims 16 ..
            // bit i of a 4-bit x goes to bit 0 of byte i: x * (1 + 2^7 + 2^14 + 2^21)
            const uint32_t s0 = ((hb & 0xFu) * 0x00204081u) & 0x01010101u;
            const uint32_t s1 = ((hb >> 4) * 0x00204081u) & 0x01010101u;
            const uint32_t c0w = ((nibw.x >> shn) & 0x0F0F0F0Fu) | (s0 << 4);
            const uint32_t c1w = ((nibw.y >> shn) & 0x0F0F0F0Fu) | (s1 << 4);
            *reinterpret_cast<h8*>(cv + LY::VH + key * LY::ROWV + (blk * 32 + 8 * part) * 2) = stream::v_codes_sub(c0w, c1w);
        }
        // V steps (times 2^-E_v) and offsets: task (key, blk)
        const float vdown = dec::pow2(-(int)vsh_next);
        for (int u = tid; u < kTile * NB; u += 64 * kWaves) {
            const int key = u / NB, blk = u - key * NB;
            const uint32_t dm = vstepm(key, blk);
            reinterpret_cast<_Float16*>(cv + LY::VD)[blk * kTile + key] = (_Float16)(f16_value((uint16_t)(dm & 0xFFFFu)) * vdown);
            reinterpret_cast<uint16_t*>(cv + LY::VM)[key * LY::VMS + blk] = (uint16_t)(dm >> 16);
        }
    };
    // the columns of ones after each offset row, in both converted buffers (never rewritten)
    for (int cb = 0; cb < kConvBufs; ++cb) {
        uint16_t* const vm = reinterpret_cast<uint16_t*>(smem + kRawBufs * LY::RAW + cb * LY::CONV + LY::VM);
        constexpr int NO = LY::VMS - NB;
        for (int u = threadIdx.x; u < kTile * NO; u += 64 * kWaves) vm[(u / NO) * LY::VMS + NB + u % NO] = 0x3C00;
    }

    // ---- this wave's query rows as fp16 B operands, divided per wave by the
    // power of two that puts their largest |q| in [2^14, 2^15)
    constexpr int RTW = 2;
    h8 qh[RTW][NB], ql[RTW][NB];
    constexpr int QW = QLO ? 8 : 4;
    uint32_t qw[RTW][NB][QW];
    uint32_t mag = 0;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int r = rt * 16 + j16;
        const bool real = r < R;
        const int t = real ? tq0 + r / p.hpk : 0, hh = real ? r % p.hpk : 0;
        const size_t row0q = (((size_t)b * p.T + t) * p.H + g * p.hpk + hh) * HD + 8 * q4;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            uint32_t w[QW];
#pragma unroll
            for (int e = 0; e < QW; ++e) w[e] = 0u;
            if (real) {
                if constexpr (QLO) {
                    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(p.q) + row0q + blk * 32);
                    const uint4 a = src[0], c = src[1];
                    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
                    if constexpr (QW == 8) { w[4] = c.x; w[5] = c.y; w[6] = c.z; w[7] = c.w; }
                } else {
                    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + row0q + blk * 32);
                    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
                }
            }
#pragma unroll
            for (int e = 0; e < QW; ++e) {
                if (QLO) mag = max(mag, w[e] & 0x7FFFFFFFu);
                else mag = max(mag, max((w[e] << 16) & 0x7FFFFFFFu, w[e] & 0x7FFF0000u));
                qw[rt][blk][e] = w[e];
            }
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, m));
    const uint32_t qexp = __builtin_amdgcn_readfirstlane(dec::exp_of(mag));
    const float qdown = dec::q_down(qexp), qup = dec::q_up(qexp);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = QLO ? __uint_as_float(qw[rt][blk][e % QW])
                                    : __uint_as_float((e & 1) ? (qw[rt][blk][e / 2] & 0xFFFF0000u) : (qw[rt][blk][e / 2] << 16));
                const float x = v * qdown;
                const _Float16 xh = (_Float16)x;
                qh[rt][blk][e] = xh;
                if (QLO) ql[rt][blk][e] = (_Float16)(x - (float)xh);
            }

    f4 oacc[RTW][2 * NB], macc[RTW];
    float mrow[RTW], lsum[RTW];
    int vis_lo[RTW], vis_hi[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        macc[rt] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt) oacc[rt][dt] = (f4){0.f, 0.f, 0.f, 0.f};
        mrow[rt] = stream::kNoMax;
        lsum[rt] = 0.0f;
        vis_lo[rt] = vis_hi[rt] = 0;
        const int r = rt * 16 + j16;
        if (r < R) {
            vis_hi[rt] = len - p.T + tq0 + r / p.hpk + 1;
            vis_lo[rt] = p.window > 0 ? max(0, vis_hi[rt] - p.window) : 0;
        }
    }
    // rows every query row of this wave sees (no masks needed inside)
    const int full_hi = min(len - p.T + tq0 + 1, c1);
    const int full_lo = max(p.window > 0 ? max(0, len - p.T + tq0 + Tq - p.window) : 0, c0);
    const int mk0 = stream::pkey(q4, j16 >> 2), mk1 = stream::pkey(q4, 4 + (j16 >> 2));
    const int mc = (4 * (j16 & 3) < LY::VMS) ? (j16 & 3) : 0;
    int vsh = 0;

    const float sc2 = p.scale * kLog2e;
    // ---- the raw scores of one converted tile (converted buffer cb) for
    // this wave's query rows: acc[rt][h][i] = sum over the head's dims of
    // (d * c)(key 16h + 4*q4 + i) * q'(row rt*16 + j16), hi and lo parts
    auto scores = [&](int cb, f4 (&acc)[RTW][2]) {
        const uint8_t* const cv = smem + kRawBufs * LY::RAW + cb * LY::CONV;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int h = 0; h < 2; ++h) acc[rt][h] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = (16 * h + j16) * LY::ROWH + (blk * 32 + 8 * q4) * 2;
                const h8 kh = *reinterpret_cast<const h8*>(cv + LY::KH + o);
                const h8 kl = *reinterpret_cast<const h8*>(cv + LY::KL + o);
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) {
                    acc[rt][h] = dec::mfma(kh, qh[rt][blk], acc[rt][h]);
                    acc[rt][h] = dec::mfma(kl, qh[rt][blk], acc[rt][h]);
                    if (QLO) {
                        acc[rt][h] = dec::mfma(kh, ql[rt][blk], acc[rt][h]);
                        acc[rt][h] = dec::mfma(kl, ql[rt][blk], acc[rt][h]);
                    }
                }
            }
    };
    // ---- softmax and P V of one tile (at t0, converted buffer cb) from its
    // raw scores; ksh, vsh_t: the tile's range shifts
    auto finish = [&](int cb, int t0, f4 (&acc)[RTW][2], uint32_t ksh, uint32_t vsh_t) {
        const uint8_t* const cv = smem + kRawBufs * LY::RAW + cb * LY::CONV;
        // base-2 scores: the raw ones times scale * log2 e, times 2^ksh, times
        // the query rows' power of two
        const float fs = sc2 * qup * dec::pow2((int)ksh);
        // ---- online softmax against a reference max that moves only when a
        // score passes it by more than 8 (so p <= 256, inside fp16)
        const bool interior = t0 >= full_lo && t0 + kTile <= full_hi;
        if (!interior) {   // edge tiles: one unsigned compare per key against the row's visible range
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                const int jb = t0 + 4 * q4 - vis_lo[rt];
                const uint32_t span = (uint32_t)(vis_hi[rt] - vis_lo[rt]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rt][h][i] = (uint32_t)(jb + 16 * h + i) < span ? acc[rt][h][i] : -INFINITY;
            }
        }
        h8 pu[RTW];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const float smax = fmaxf(fmaxf(fmaxf(acc[rt][0][0], acc[rt][0][1]), fmaxf(acc[rt][0][2], acc[rt][0][3])),
                                     fmaxf(fmaxf(acc[rt][1][0], acc[rt][1][1]), fmaxf(acc[rt][1][2], acc[rt][1][3]))) * fs;
            if (__any(smax > mrow[rt] + 8.0f)) {
                float mt = fmaxf(smax, __shfl_xor(smax, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                const bool move = mt > mrow[rt] + 8.0f;
                const float alpha = move ? __builtin_amdgcn_exp2f(mrow[rt] - mt) : 1.0f;
                mrow[rt] = move ? mt : mrow[rt];
                float ar[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i);
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) oacc[rt][dt][i] *= ar[i];
#pragma unroll
                for (int i = 0; i < 4; ++i) macc[rt][i] *= ar[i];
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pu[rt][4 * h + i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(acc[rt][h][i], fs, -mrow[rt]));
        }
        // ---- the accumulators take the tile's V units (2^-vsh_t)
        if (vsh_t != (uint32_t)vsh) {
            const float f = dec::pow2(vsh - (int)vsh_t);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) oacc[rt][dt][i] *= f;
            vsh = (int)vsh_t;
        }
        // ---- P V: P' = fp16(P) * step (steps times 2^-vsh), 16 dims per product
        const uint16_t* const VDa = reinterpret_cast<const uint16_t*>(cv + LY::VD);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const h8 dh = stream::steps_of(VDa + blk * kTile, q4);
            h8 pa[RTW];
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) pa[rt] = pu[rt] * dh;
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const int col = blk * 32 + 16 * dd + 4 * (j16 & 3);
                const h8 vf = dec::tr16_pair(cv + LY::VH + mk0 * LY::ROWV + col * 2, cv + LY::VH + mk1 * LY::ROWV + col * 2);
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) oacc[rt][2 * blk + dd] = dec::mfma(pa[rt], vf, oacc[rt][2 * blk + dd]);
            }
        }
        // q5_1 offset term and the row sums (the ones column)
        const h8 mb = dec::tr16_pair(cv + LY::VM + (mk0 * LY::VMS + 4 * mc) * 2, cv + LY::VM + (mk1 * LY::VMS + 4 * mc) * 2);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) macc[rt] = dec::mfma(pu[rt], mb, macc[rt]);
    };

    // ---- the pipeline.  Tile t's rows go to raw buffer t mod 3 and its
    // operands to converted buffer t mod 3.  Iteration it (after one barrier)
    // requests tile it + 4, computes the scores of tile it + 1, the softmax
    // and P V of tile it (whose scores the previous iteration computed) and
    // converts tile it + 2; so the matrix cores take tile it + 1's scores
    // while the vector ALU works tile it's softmax.
    auto ring3 = [](int x) { return x == 2 ? 0 : x + 1; };
    for (int x = 0; x < kRawBufs; ++x)
        if (x < ntiles) issue(t_begin + x * kTile, x);
    uint32_t ksh0 = 0, vsh0 = 0, ksh1 = 0, vsh1 = 0;   // the shifts of tiles it and it + 1
    if (ntiles > 0) {
        const int a = my_loads(t_begin + kTile), c = my_loads(t_begin + 2 * kTile);
        wait_vmcnt(a < 0 || c < 0 ? 0 : a + c);
        stream::lds_barrier();                       // every wave's pieces of tile 0 have landed
        convert(t_begin, 0, 0);
        ksh0 = ksh_next;
        vsh0 = vsh_next;
    }
    if (ntiles > 1) {
        wait_vmcnt(my_loads(t_begin + 2 * kTile));
        stream::lds_barrier();                       // tile 1 has landed; tile 0's raw buffer is free
        if (ntiles > 3) issue(t_begin + 3 * kTile, 0);
        convert(t_begin + kTile, 1, 1);
        ksh1 = ksh_next;
        vsh1 = vsh_next;
    }

    f4 acc_c[RTW][2], acc_n[RTW][2];
    int b0 = 0;                                      // raw and converted buffer of tile it
    for (int it = 0; it < ntiles; ++it) {
        const int t0 = t_begin + it * kTile;
        const int b1 = ring3(b0), b2 = ring3(b1);
        // tile it + 2 has landed (tile it + 3 may still be in flight); after
        // the barrier tiles it and it + 1 are converted by all waves, tile
        // it - 1's operands are no longer read, and tile it + 1's raw buffer
        // is free
        if (it + 2 < ntiles) wait_vmcnt(my_loads(t0 + 3 * kTile));
        stream::lds_barrier();
        if (it + 4 < ntiles) issue(t0 + 4 * kTile, b1);
        // the conversion of tile it + 2 and the products, in opposite orders
        // on the two waves that share a SIMD (waves w and w + 4)
        const bool convert_first = wave < kWaves / 2;
        if (convert_first && it + 2 < ntiles) convert(t0 + 2 * kTile, b2, b2);
        if (active) {
            if (it == 0) scores(b0, acc_c);
            if (it + 1 < ntiles) scores(b1, acc_n);
            finish(b0, t0, acc_c, ksh0, vsh0);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                for (int h = 0; h < 2; ++h) acc_c[rt][h] = acc_n[rt][h];
        }
        if (!convert_first && it + 2 < ntiles) convert(t0 + 2 * kTile, b2, b2);
        ksh0 = ksh1;
        vsh0 = vsh1;
        ksh1 = ksh_next;
        vsh1 = vsh_next;
        b0 = b1;
    }

    if (!active) return;
    // ---- finish: row sums from the ones column; offsets into O (the q5_1
    // code products carry 2^-24, FP8 ones none; P * step carries 2^-vsh)
    const float ounit = dec::pow2((F8 ? 0 : 24) + vsh);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int src = 16 * (j16 >> 2) + NB;
        const float l0 = __shfl(macc[rt][0], src), l1 = __shfl(macc[rt][1], src);
        const float l2 = __shfl(macc[rt][2], src), l3 = __shfl(macc[rt][3], src);
        lsum[rt] = (j16 & 2) ? ((j16 & 1) ? l3 : l2) : ((j16 & 1) ? l1 : l0);
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[rt][dt][i] = fmaf(oacc[rt][dt][i], ounit, __shfl(macc[rt][i], 16 * q4 + dt / 2));
    }
    const size_t row0 = ((size_t)b * p.splits + s) * p.T;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int r = rt * 16 + j16;
        if (q4 == 0 && r < R) {
            const int t = tq0 + r / p.hpk, hq = g * p.hpk + r % p.hpk;
            const size_t idx = (row0 + t) * p.H + hq;
            p.part_ml[2 * idx] = (mrow[rt] == stream::kNoMax) ? -INFINITY : mrow[rt] * kLn2;
            p.part_ml[2 * idx + 1] = lsum[rt];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ro = rt * 16 + 4 * q4 + i;
            if (ro < R) {
                const int t = tq0 + ro / p.hpk, hq = g * p.hpk + ro % p.hpk;
                float* o = p.part_o + ((row0 + t) * p.H + hq) * HD + j16;
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt) o[16 * dt] = oacc[rt][dt][i];
            }
        }
    }
}

}  // namespace prime

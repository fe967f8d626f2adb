// kvq_decode_stream.hip -- split-K flash decode, each wave streaming one KV
// head's row windows through LDS (gfx950).  Included by kvq_kernels.hip
// (inside namespace kvq), after kvq_decode.hip.
//
// The same partials as the other decode kernels (cortiq-engine "Struct
// LayerKvCache", attend_group and attend_group_upto; memra-engine "Struct
// KvLayer", len_d and base_d):
//   * a workgroup is (session, chunk of rows, group of gh KV heads, group of
//     query rows on the grid's y index); by default wave w is KV head
//     g = hg*gh + w and computes all R query rows of its group (one or two
//     16-row tiles).  Other layouts give a head two waves: row streams (RS,
//     alternate tiles of a longer chunk, merged in LDS at the end), row
//     groups (RG, 16 query rows each, sharing two tile buffers) or dim halves
//     (DS, half of the head's dims each, partial scores added through LDS).
//   * per 32-row tile, a wave copies its head's K window (the q8_0 blocks,
//     from the 16-byte boundary at or below them) and V window (the q5_1
//     blocks) of every row into LDS with global_load_lds_dwordx4.  With one
//     buffer per wave, the next tile's K rows are requested as soon as the
//     scores have read this tile's and its V rows as soon as P V has read
//     these; with two buffers per head the tile after next is requested.  A
//     workgroup barrier before each K refill keeps the heads of a row in
//     step, so that cache lines shared by adjacent head slices are fetched
//     once.  Row strides in LDS are odd numbers of 16-byte pieces, which
//     keeps 8 consecutive rows on distinct banks.
//   * scores are computed transposed, S^T = K Q^T, one v_mfma_f32_16x16x32_f16
//     per 32-element block, 16 keys and row tile; the K codes, exact in fp16,
//     are converted once per tile and feed every row tile.  Each lane ends up
//     with 8 keys of one query row, which after the softmax are the A operand
//     of the P V product, in key order 4*q4 + i, 16 + 4*q4 + i.
//   * the V operand comes straight from the q5_1 bytes: ds_read_b64_tr_b8 of
//     the 16 nibble bytes of 8 keys gives a lane the codes of its dimension
//     (low nibble) and of dimension + 16 (high nibble); a second transposed
//     read of the block headers gives the high-bit bytes, which DPP row
//     broadcasts hand to the lanes that need them.
//   * the q5_1 step multiplies P per block (P' = P * step, fp16); the offset
//     term sum_key P * m is one more MFMA per tile against the offsets.
namespace stream {

using dec::f4;
using dec::h8;
using dec::i2;
using dec::kLn2;
using dec::kLog2e;
using dec::lds_i2;

constexpr int kTile = kRowTile;

// Barrier for LDS hand-offs between the waves of a workgroup.  It waits for
// this wave's LDS operations only: the tile loads in flight into the other
// buffer are global->LDS transfers counted by vmcnt, which a fenced
// __syncthreads() would drain.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 16-byte piece per lane, from base + off to LDS address lds + 16 * lane
// (global_load_lds_dwordx4, scalar base form).  Written as asm because the
// compiler's wait-count pass, unable to tell these LDS writes from the LDS
// reads of the other buffer, would otherwise wait for them before every such
// read; the kernel waits for them itself with explicit vmcnt counts.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint8_t* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)(lds_u8*)lds;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(l) : "memory");
}

// Lane L's value of x in every lane of its 16-lane row (DPP row_newbcast).
template <int L>
__device__ __forceinline__ uint32_t row_bcast(int x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x150 + L, 0xF, 0xF, true);
}

// Key of slot k (0..7) of lane group q4 in the P V operands.
__device__ __forceinline__ int pkey(int q4, int k) { return (k < 4) ? 4 * q4 + k : 16 + 4 * q4 + (k - 4); }

// The window geometry of one format: q8_0 / q5_1 blocks, or FP8 rows.
template <int NB, bool F8>
struct WinOf {
    using type = StreamWin<NB>;
};
template <int NB>
struct WinOf<NB, true> {
    using type = StreamWinF8<NB>;
};

// 8 e4m3 codes (bytes of lo, then hi) -> fp16, exactly (every e4m3 value is an
// fp16 value); the hardware conversion with a scale of 1.
__device__ __forceinline__ h8 e4m3_codes(uint32_t lo, uint32_t hi) {
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    const h2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const h2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const h2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const h2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return (h8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The reference max of a row that has seen no visible key yet: finite, so
// that exp2(score - max) needs no test (a masked score is -inf and gives 0),
// and below every finite score, so that the first one always moves it.
constexpr float kNoMax = -3.402823466e38f;

// The fp16 steps of keys 4*q4 + i and 16 + 4*q4 + i (i = 0..3) of one block,
// in the key order of the P V operands.
__device__ __forceinline__ h8 steps_of(const uint16_t* vd, int q4) {
    const uint2 a = *reinterpret_cast<const uint2*>(vd + 4 * q4);
    const uint2 b = *reinterpret_cast<const uint2*>(vd + 16 + 4 * q4);
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(h8, (u4v){a.x, a.y, b.x, b.y});
}

template <int NL>
__device__ __forceinline__ void wait_loads_upto() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((NL & 15) | 0x0F70 | (((NL >> 4) & 3) << 14));   // vmcnt(NL)
    asm volatile("" ::: "memory");
}

// Two bytes of x (selector: 0x0401_0400 bytes 0,1; 0x0403_0402 bytes 2,3) as
// the fp16 values 1024 + byte.
__device__ __forceinline__ uint32_t spread_1024(uint32_t x, uint32_t sel) {
    return __builtin_amdgcn_perm(0x64646464u, x, sel);
}
// Two bytes of x as fp16 subnormals, byte * 2^-24 (exact; the matrix cores
// keep fp16 subnormal inputs).
__device__ __forceinline__ uint32_t spread_sub(uint32_t x, uint32_t sel) {
    return __builtin_amdgcn_perm(0u, x, sel);
}
constexpr uint32_t kSel01 = 0x04010400u, kSel23 = 0x04030402u;

// 8 signed q8_0 codes, the pairs given by (word, selector), -> fp16 exactly:
// (c ^ 0x80) = c + 128 in the low byte of 1024 + (c + 128), less 1152.
__device__ __forceinline__ h8 k_codes(uint32_t w0, uint32_t s0, uint32_t w1, uint32_t s1, uint32_t w2, uint32_t s2,
                                      uint32_t w3, uint32_t s3) {
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    const h2v off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const h2v a = __builtin_bit_cast(h2v, spread_1024(w0, s0)) - off;
    const h2v b = __builtin_bit_cast(h2v, spread_1024(w1, s1)) - off;
    const h2v c = __builtin_bit_cast(h2v, spread_1024(w2, s2)) - off;
    const h2v d = __builtin_bit_cast(h2v, spread_1024(w3, s3)) - off;
    return (h8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 q5_1 codes (bytes 0..31 of lo, hi) -> fp16 subnormals code * 2^-24.
__device__ __forceinline__ h8 v_codes_sub(uint32_t lo, uint32_t hi) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const u4v w = {spread_sub(lo, kSel01), spread_sub(lo, kSel23), spread_sub(hi, kSel01), spread_sub(hi, kSel23)};
    return __builtin_bit_cast(h8, w);
}

// NB blocks of 32 dims per head; RTW row tiles of 16 per wave; QLO: fp32
// queries (a low fp16 part kept beside the high one); RS row streams (waves
// of one head taking alternate tiles); RG row groups (waves of one head
// taking 16 query rows each of the same tiles, which they load in step so
// that the second copy comes from L2); DS dim halves; F8: K and V as FP8
// rows (a head's codes, then the piece of the row's scale area holding its
// scales) instead of q8_0 / q5_1 blocks.
template <int NB, int RTW, bool QLO, int RS, int RG, int DS, bool F8>
__global__ __launch_bounds__(64 * (DS == 2 ? 8 : RS == 2 ? 16 : RG == 2 ? 8 : RTW == 1 ? 8 : 4),
                             DS == 2 ? stream_ds_waves_per_simd(NB) : stream_waves_per_simd(NB, RTW, QLO)) void decode_stream(
    DecodeParams p) {
    static_assert(RS == 1 || RTW == 1 || DS == 2, "row streams need one row tile per wave, or dim halves");
    static_assert(RG == 1 || (RTW == 1 && RS == 1 && RG == 2), "row groups are two, one row tile per wave");
    static_assert(DS == 1 || (DS == 2 && RTW == 2 && RG == 1), "dim halves hold both row tiles");
    using WN = typename WinOf<NB, F8>::type;
    constexpr int HD = NB * 32;     // dims of this wave's slice of a head
    // DS = 2: the two waves of a head take half of its dims each (NB blocks
    // of the 2 NB), for all R query rows: each loads and unpacks only its
    // half of the K and V windows, and the two partial score sums meet in
    // LDS (XCH bytes per wave, two slots by tile parity).
    constexpr int HDR = HD * DS;    // dims of a head
    constexpr int XCH = DS == 2 ? 2 * RTW * 2 * 64 * 16 : 0;
    constexpr int WSTR = WN::BYTES + XCH;
    // SH: the two row-group waves of a head share two tile buffers (each
    // wave copies 16 of the 32 rows), so that a second tile is in flight
    // while one is computed; per-wave scale arrays follow the shared buffers.
    constexpr bool SH = RG == 2;
    constexpr int RAW = SH ? WN::KS : WN::BYTES;          // bytes of one buffer's K and V rows
    constexpr int NKH = SH ? (16 * WN::KWP + 63) / 64 : WN::NKI;   // load instructions per copy
    constexpr int NVH = SH ? (16 * WN::VWP + 63) / 64 : WN::NVI;

    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q4 = lane >> 4, j16 = lane & 15;
    const int gh = p.gh, ngrp = p.Hkv / gh;
    constexpr int rs = RS;
    const int wv = DS == 2 ? wave >> 1 : wave;         // wave index without the dim half
    const int gi = wv % gh;                            // head in the group
    const int half = DS == 2 ? wave & 1 : 0;          // DS = 2: this wave's half of the dims
    const int str = RS > 1 ? wv / gh : 0;        // row stream
    const int rb = RG > 1 ? (wv / gh) * 16 : 0;     // first query row of this wave
    // row tile rt holds query rows rb + 16 (rt ^ rsw) ..: with dim halves
    // each wave's row tile 0 is the one whose softmax it takes
    const int rsw = DS == 2 ? half : 0;

    const int W = gridDim.x, wid = blockIdx.x;
    const int L = (wid & 7) * (W >> 3) + (wid >> 3);
    const int hg = L % ngrp;
    int b, s, len, base;
    dec::locate_unit(p, L / ngrp, b, s, len, base);
    if (b < 0) return;
    const int g = hg * gh + gi;
    // query rows tq0 .. tq0 + Tq - 1 of the T: the grid's y index is the
    // group of Tg rows
    const int tq0 = blockIdx.y * p.Tg, Tq = min(p.Tg, p.T - tq0);
    const int R = Tq * p.hpk;

    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int c0 = (lo & ~(kTile - 1)) + s * p.chunk;
    const int c1 = min(c0 + p.chunk, len);
    if (c0 >= c1) return;

    uint8_t* const wb = smem + wave * WSTR;
    // tile buffers: this wave's own, or its head's two shared ones
    uint8_t* const tb0 = SH ? smem + gi * 2 * RAW : wb;
    // scale arrays: at the end of the wave's buffer, or one set per head after
    // all shared buffers (each of the head's two waves fills in its own rows)
    uint8_t* const scb = SH ? smem + gh * 2 * RAW + gi * (WN::BYTES - WN::KS) - WN::KS : wb;
    const uint8_t* rk = tb0 + WN::KB;   // K rows of the current tile, stride KSTR
    const uint8_t* rv = tb0 + WN::VB;   // V rows of the current tile, stride VSTR
    const int hrow = SH ? rb : 0;       // first tile row this wave copies
    // This head's windows.  q8_0 / q5_1: K from the 16-byte boundary at or
    // below its first block (kofs bytes before it), V exactly its blocks.
    // FP8: the codes of its blocks (16-byte aligned in the row), then the
    // 16-byte piece of the row's scale area that holds its NB scales (at
    // sofs within it); the same for K and V.
    const int hs = g * DS + half;                       // this wave's NB-block slice of a row
    const int kstart = F8 ? hs * NB * 32 : hs * NB * 34;
    const int kofs = F8 ? 0 : (kstart & 15);
    const int sofs = F8 ? (hs * 2 * NB) & 15 : 0;
    const int spiece = F8 ? p.Hkv * p.hd + ((hs * 2 * NB) & ~15) : 0;
    const uint8_t* const kwin = p.k_planes + (int64_t)b * p.k_stride + (F8 ? 0 : kstart - kofs);
    const uint8_t* const vwin = p.v_planes + (int64_t)b * p.v_stride + (F8 ? 0 : hs * NB * 24);
    // per lane, the byte offset of its piece (instruction x) from the tile's
    // first row (FP8 K and V rows have one size and layout: one set serves both)
    uint32_t koff[NKH], voff[F8 ? 1 : NVH];
#pragma unroll
    for (int x = 0; x < NKH; ++x) {
        const int pc = x * 64 + lane, row = pc / WN::KWP, col = pc - row * WN::KWP;
        koff[x] = F8 ? (uint32_t)((hrow + row) * p.k_row + (col < 2 * NB ? kstart + col * 16 : spiece))
                     : (uint32_t)((hrow + row) * p.k_row + min(col, WN::KW - 1) * 16);
    }
#pragma unroll
    for (int x = 0; x < (F8 ? 0 : NVH); ++x) {
        const int pc = x * 64 + lane, row = pc / WN::VWP, col = pc - row * WN::VWP;
        voff[x] = (uint32_t)((hrow + row) * p.v_row + min(col, WN::VW - 1) * 16);   // the pad piece re-reads a real one
    }
    // kept in registers as they are (not recomputed at each use)
#pragma unroll
    for (int x = 0; x < NKH; ++x) asm volatile("" : "+v"(koff[x]));
#pragma unroll
    for (int x = 0; x < (F8 ? 0 : NVH); ++x) asm volatile("" : "+v"(voff[x]));
    constexpr int CROWS = SH ? 16 : kTile;   // rows of one copy
    // Copy the K (or V) rows of the tile [t0, t0 + 32) into the buffer.  Rows
    // from c1 on (a session's last tile) are not loaded; rows below lo (first
    // tile) are resident and masked.  Every LDS read of the half being
    // refilled has returned first.
    auto issue_k = [&](int t0, uint8_t* tb) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        const int nrows = SH ? min(16, max(0, c1 - t0 - hrow)) : min(kTile, c1 - t0);
        const uint8_t* const kt = kwin + (int64_t)(t0 - base) * p.k_row;
        uint8_t* const d = tb + WN::KB + hrow * WN::KSTR;
        if (nrows == CROWS) {
            // a whole copy: every instruction but a partial last one takes all lanes
#pragma unroll
            for (int x = 0; x < NKH; ++x)
                if ((x + 1) * 64 <= CROWS * WN::KWP || lane < CROWS * WN::KWP - x * 64) dma16(kt, koff[x], d + x * 1024);
        } else {
#pragma unroll
            for (int x = 0; x < NKH; ++x)
                if (lane < nrows * WN::KWP - x * 64) dma16(kt, koff[x], d + x * 1024);
        }
    };
    auto issue_v = [&](int t0, uint8_t* tb) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        const int nrows = SH ? min(16, max(0, c1 - t0 - hrow)) : min(kTile, c1 - t0);
        const uint8_t* const vt = vwin + (int64_t)(t0 - base) * p.v_row;
        uint8_t* const d = tb + WN::VB + hrow * WN::VSTR;
        if (nrows == CROWS) {
#pragma unroll
            for (int x = 0; x < NVH; ++x)
                if ((x + 1) * 64 <= CROWS * WN::VWP || lane < CROWS * WN::VWP - x * 64)
                    dma16(vt, F8 ? koff[x] : voff[x], d + x * 1024);
        } else {
#pragma unroll
            for (int x = 0; x < NVH; ++x)
                if (lane < nrows * WN::VWP - x * 64) dma16(vt, F8 ? koff[x] : voff[x], d + x * 1024);
        }
    };

    // macc: the q5_1 offset product, whose column NB is the row sums of P
    // (FP8: a product with ones, every column the row sums)
    f4 oacc[RTW][2 * NB], macc[RTW];
    float mrow[RTW], lsum[RTW];
    int vis_lo[RTW], vis_hi[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        macc[rt] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt) oacc[rt][dt] = (f4){0.f, 0.f, 0.f, 0.f};
        mrow[rt] = kNoMax;
        lsum[rt] = 0.0f;
        vis_lo[rt] = vis_hi[rt] = 0;
        const int r = rb + (rt ^ rsw) * 16 + j16;
        if (r < R) {
            vis_hi[rt] = len - p.T + tq0 + r / p.hpk + 1;
            vis_lo[rt] = p.window > 0 ? max(0, vis_hi[rt] - p.window) : 0;
        }
    }
    const int full_hi = min(len - p.T + tq0 + 1, c1);
    const int full_lo = max(p.window > 0 ? max(0, len - p.window) : 0, c0);
    const float sc2 = p.scale * kLog2e;
    float* const KSa = reinterpret_cast<float*>(scb + WN::KS);
    uint16_t* const VDa = reinterpret_cast<uint16_t*>(scb + WN::VD);   // fp16 V steps
    uint16_t* const VMa = reinterpret_cast<uint16_t*>(scb + WN::VM);   // q5_1 offsets (not FP8)
    const int vkey = pkey(q4, j16 >> 1);                 // V row of this lane's tr8 reads
    const int mk0 = pkey(q4, j16 >> 2), mk1 = pkey(q4, 4 + (j16 >> 2));
    // columns of the offset product: NB offsets, then ones (column NB gives the
    // row sums); the columns past the stored ones are unused
    const int mc = (4 * (j16 & 3) < WN::VMS) ? (j16 & 3) : 0;
    const int sh_rot = ((j16 & 7) - 4) & 31;             // moves bit (j16 & 7) of each byte to bit 4
    const bool hi8 = j16 >= 8;                            // this lane's dims take high-bit bytes 1 and 3

    // Loads in issue order: K(0) V(0) | K(1) .. V(1) | ...  K(t+1) is issued
    // once the scores of tile t have read the K rows, V(t+1) once its P V has
    // read the V rows.
    // Row stream str takes the chunk's tiles str, str + rs, ...; a stream
    // with fewer tiles than stream 0 meets stream 0's remaining barriers
    // after its loop.
    if constexpr (!F8) {
        // the columns of ones after each row's NB offsets (never rewritten;
        // with shared buffers both waves of a head write the same values)
        constexpr int NO = WN::VMS - NB;
        for (int u = lane; u < kTile * NO; u += 64) VMa[(u / NO) * WN::VMS + NB + u % NO] = 0x3C00;   // fp16 1.0
    }
    if constexpr (F8) {
        // A tile's rows past c1 are not loaded, and P V still multiplies their
        // V codes (by a weight of 0).  Any byte is a valid q5_1 code, but
        // e4m3 has NaN codes: zero this wave's V rows once, so that such rows
        // hold zeros or an earlier tile's codes, never stale LDS bytes.
        constexpr int VROWS = SH ? 16 : kTile;
#pragma unroll
        for (int bi = 0; bi < (SH ? 2 : 1); ++bi) {
            uint8_t* const z = tb0 + bi * RAW + WN::VB + hrow * WN::VSTR;
            for (int o = lane * 16; o < VROWS * WN::VSTR; o += 64 * 16)
                *reinterpret_cast<uint4*>(z + o) = make_uint4(0u, 0u, 0u, 0u);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zeros are written before any load lands
    }
    const int ntiles = (c1 - c0 + kTile - 1) / kTile;
    const int nit = (ntiles + rs - 1) / rs;                   // stream 0's tiles
    const int mine = ntiles > str ? (ntiles - str + rs - 1) / rs : 0;
    const int first = c0 + str * kTile;
    if (first < c1) {
        issue_k(first, tb0);
        issue_v(first, tb0);
        if (SH && first + kTile < c1) {
            issue_k(first + kTile, tb0 + RAW);
            issue_v(first + kTile, tb0 + RAW);
        }
    }

    // Q rows (tile rt, j16) as the B operand of S^T = K Q^T, read while the
    // first tile's rows are in flight.  The wave's rows are divided by the
    // power of two that puts their largest |q| in [2^14, 2^15) (dec::q_down;
    // with dim halves the exponent covers both halves, so that their partial
    // scores add up), which makes bf16 queries exact in fp16 at any
    // magnitude; qup multiplies the scores back.
    h8 qh[RTW][NB], ql[RTW][NB];
    constexpr int QW = QLO ? 8 : 4;          // words per lane and block: 8 fp32 or 8 bf16 values
    uint32_t qw[RTW][NB][QW];
    uint32_t mag = 0;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int r = rb + (rt ^ rsw) * 16 + j16;
        const bool real = r < R;
        const int t = real ? tq0 + r / p.hpk : 0, hh = real ? r % p.hpk : 0;
        const size_t row0q = (((size_t)b * p.T + t) * p.H + g * p.hpk + hh) * HDR + 8 * q4;
#pragma unroll
        for (int hf = 0; hf < DS; ++hf) {
            // hf 0: this wave's dims; hf 1 (dim halves): the other half's,
            // for the exponent only
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                uint32_t w[QW];
#pragma unroll
                for (int e = 0; e < QW; ++e) w[e] = 0u;
                if (real) {
                    const size_t i0 = row0q + (half ^ hf) * HD + blk * 32;
                    if constexpr (QLO) {
                        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(p.q) + i0);
                        const uint4 a = src[0], c = src[1];
                        const uint32_t w8[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
                        for (int e = 0; e < QW; ++e) w[e] = w8[e];
                    } else {
                        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + i0);
                        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
                    }
                }
#pragma unroll
                for (int e = 0; e < QW; ++e) {
                    if (QLO) mag = max(mag, w[e] & 0x7FFFFFFFu);
                    else mag = max(mag, max((w[e] << 16) & 0x7FFFFFFFu, w[e] & 0x7FFF0000u));
                    if (hf == 0) qw[rt][blk][e] = w[e];
                }
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
    // E of dec::v_shift: the P V accumulators hold their sums in units of
    // 2^-vsh (0 unless a tile held a V step of 2^7 or more)
    int vsh = 0;

    for (int it = 0; it < mine; ++it) {
        const int t0 = first + it * rs * kTile;
        const int tn = t0 + rs * kTile;                  // its next tile
        const bool whole = t0 + kTile <= c1;             // this tile issued all its loads
        const bool next = tn < c1;
        const bool next_whole = tn + kTile <= c1;
        float sv[RTW][2][4];
        uint8_t* const tb = SH ? tb0 + (it & 1) * RAW : tb0;   // this tile's buffer
        rk = tb + WN::KB;
        rv = tb + WN::VB;
        const bool has2 = tn + kTile < c1;                // SH: the tile after next
        if constexpr (SH) {
            // K(t) has landed (both copies); after it come V(t), K(t+1), V(t+1)
            if (!whole) wait_loads_upto<0>();
            else if (!next) wait_loads_upto<NVH>();
            else if (next_whole) wait_loads_upto<NVH + NKH + NVH>();
            else wait_loads_upto<0>();
        } else {
            // K(t) has landed; V(t), issued after it, may still be in flight
            if (whole) wait_loads_upto<WN::NVI>(); else wait_loads_upto<0>();
        }

        // ---- K scales (rows past c1 hold stale bytes); with shared buffers
        // each wave converts the rows it copied, and the barrier that follows
        // makes both halves of the rows and of the scales visible
        constexpr int SROWS = SH ? 16 : kTile;
#pragma unroll
        for (int x = 0; x < (SROWS * NB + 63) / 64; ++x) {
            const int u = x * 64 + lane;
            if (SROWS * NB % 64 == 0 || u < SROWS * NB) {
                const int key = hrow + u / NB, blk = u - (u / NB) * NB;
                const uint16_t kd = F8 ? *reinterpret_cast<const uint16_t*>(rk + key * WN::KSTR + 32 * NB + sofs + 2 * blk)
                                       : *reinterpret_cast<const uint16_t*>(rk + key * WN::KSTR + kofs + blk * 34);
                KSa[blk * kTile + key] = (t0 + key < c1) ? f16_value(kd) * sc2 : 0.0f;
            }
        }
        if constexpr (SH) lds_barrier(); else dec::lds_order();

        // ---- scores S^T: sv[rt][h][i] = S[row of tile rt, j16][key 16h + 4*q4 + i] (base 2)
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[rt][h][i] = 0.0f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const float4 ks0 = *reinterpret_cast<const float4*>(KSa + blk * kTile + 4 * q4);
            const float4 ks1 = *reinterpret_cast<const float4*>(KSa + blk * kTile + 16 + 4 * q4);
            const float ksv[2][4] = {{ks0.x, ks0.y, ks0.z, ks0.w}, {ks1.x, ks1.y, ks1.z, ks1.w}};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = 16 * h + j16;
                // kofs is a multiple of 4, so the codes start 2 bytes into a
                // word for even blocks and on a word for odd ones
                const int cb = blk * 34 + 2;
                const uint32_t* w = reinterpret_cast<const uint32_t*>(
                    rk + (uint32_t)(key * WN::KSTR + kofs + 8 * q4) + (cb & ~3));
                h8 kf;
                if constexpr (F8) {
                    const uint2 c8 = *reinterpret_cast<const uint2*>(rk + key * WN::KSTR + blk * 32 + 8 * q4);
                    kf = e4m3_codes(c8.x, c8.y);
                } else if ((cb & 3) == 2) {
                    const uint32_t x0 = w[0] ^ 0x80808080u, x1 = w[1] ^ 0x80808080u, x2 = w[2] ^ 0x80808080u;
                    kf = k_codes(x0, kSel23, x1, kSel01, x1, kSel23, x2, kSel01);
                } else {
                    const uint32_t x0 = w[0] ^ 0x80808080u, x1 = w[1] ^ 0x80808080u;
                    kf = k_codes(x0, kSel01, x0, kSel23, x1, kSel01, x1, kSel23);
                }
                // tie this block's products to the previous block's sums, so
                // that the products of all blocks are not held at once
                if (NB >= 4) {
#pragma unroll
                    for (int rt = 0; rt < RTW; ++rt)
                        asm volatile("" : "+v"(kf) : "v"(sv[rt][h][0]), "v"(sv[rt][h][1]), "v"(sv[rt][h][2]), "v"(sv[rt][h][3]));
                }
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) {
                    f4 d = dec::mfma(kf, qh[rt][blk], (f4){0.f, 0.f, 0.f, 0.f});
                    if (QLO) d = dec::mfma(kf, ql[rt][blk], d);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sv[rt][h][i] = fmaf(ksv[h][i], d[i], sv[rt][h][i]);
                }
            }
        }
        // The waves of a workgroup read adjacent head slices of the same rows,
        // which share cache lines at the slice edges; requesting the next
        // tile together lets those lines be fetched from HBM once (and keeps
        // the row streams of a CU in step).
        if constexpr (SH) {
            lds_barrier();                          // both copies of K(t) are read
            if (has2) issue_k(tn + kTile, tb);
        } else if constexpr (DS == 1) {
            if (gh * rs > 1) __builtin_amdgcn_s_barrier();
            if (next) issue_k(tn, tb);
        }

        // ---- online softmax against a reference max that moves only when a
        // score passes it by more than 8 (so p <= 256, well inside fp16)
        // Edge tiles: scores of keys outside a row's visible range become
        // -inf (one unsigned compare per key, in one branch for the tile).
        const bool interior = t0 >= full_lo && t0 + kTile <= full_hi;
        h8 pu[RTW];   // P in fp16, the A operand of the products with V
        // the O and row-sum accumulators of row tile rt times alpha (each
        // lane holds the factor of its row j16)
        auto rescale_rows = [&](auto rt_c, float alpha) {
            constexpr int rt = decltype(rt_c)::value;
            float ar[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i);   // O rows 4*q4 + i
#pragma unroll
            for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[rt][dt][i] *= ar[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) macc[rt][i] *= ar[i];
        };
        auto softmax_rows = [&](auto rt_c) {
            constexpr int rt = decltype(rt_c)::value;
            if (!interior) {
                const int jb = t0 + 4 * q4 - vis_lo[rt];
                const uint32_t span = (uint32_t)(vis_hi[rt] - vis_lo[rt]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sv[rt][h][i] = (uint32_t)(jb + 16 * h + i) < span ? sv[rt][h][i] : -INFINITY;
            }
            float smax = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) smax = fmaxf(smax, sv[rt][h][i]);
            smax *= qup;                           // the scores of the scaled query rows, times qup
            if (__any(smax > mrow[rt] + 8.0f)) {   // -inf never passes, nor does a row's first finite max fail to
                float mt = fmaxf(smax, __shfl_xor(smax, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                const bool move = mt > mrow[rt] + 8.0f;
                const float alpha = move ? __builtin_amdgcn_exp2f(mrow[rt] - mt) : 1.0f;
                mrow[rt] = move ? mt : mrow[rt];
                rescale_rows(rt_c, alpha);
            }
            // a masked score gives exp2(-inf) = 0, also while mrow is still kNoMax
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pu[rt][4 * h + i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sv[rt][h][i], qup, -mrow[rt]));
        };
        if constexpr (DS == 2) {
            // Dim halves: each wave owns its row tile 0 (query rows 16 * half
            // on).  It hands its partial scores of row tile 1 to its partner
            // (whose row tile 0 they are) and adds the partner's partial of
            // its own, so that each score is summed once, takes the softmax
            // of row tile 0 only, and hands over that tile's fp16 P and row
            // maxima; the partner rescales its accumulators of those rows by
            // the same factor exp2(old max - new max), computed from the same
            // two maxima.  Two slots by tile parity: the scores a wave sends
            // in the first half of its slot, its P and maxima in the second.
            f4* const xo = reinterpret_cast<f4*>(wb + WN::BYTES) + (it & 1) * (RTW * 2 * 64);
            const f4* const xp =
                reinterpret_cast<const f4*>(smem + (wave ^ 1) * WSTR + WN::BYTES) + (it & 1) * (RTW * 2 * 64);
#pragma unroll
            for (int h = 0; h < 2; ++h) xo[h * 64 + lane] = (f4){sv[1][h][0], sv[1][h][1], sv[1][h][2], sv[1][h][3]};
            lds_barrier();
            if (next) issue_k(tn, tb);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f4 y = xp[h * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[0][h][i] += y[i];
            }
            softmax_rows(std::integral_constant<int, 0>{});
            *reinterpret_cast<h8*>(xo + 2 * 64 + lane) = pu[0];
            reinterpret_cast<float*>(xo + 3 * 64)[lane] = mrow[0];
            lds_barrier();
            pu[1] = *reinterpret_cast<const h8*>(xp + 2 * 64 + lane);
            const float mn = reinterpret_cast<const float*>(xp + 3 * 64)[lane];
            if (__any(mn != mrow[1])) {
                const float alpha = mn != mrow[1] ? __builtin_amdgcn_exp2f(mrow[1] - mn) : 1.0f;
                mrow[1] = mn;
                rescale_rows(std::integral_constant<int, 1>{}, alpha);
            }
        } else {
            softmax_rows(std::integral_constant<int, 0>{});
            if constexpr (RTW > 1) softmax_rows(std::integral_constant<int, RTW - 1>{});
        }

        if constexpr (SH) {
            // V(t) has landed (both copies); after it come K(t+1), V(t+1), K(t+2)
            if (!next || !next_whole) wait_loads_upto<0>();
            else if (!has2) wait_loads_upto<NKH + NVH>();
            else if (tn + 2 * kTile <= c1) wait_loads_upto<NKH + NVH + NKH>();
            else wait_loads_upto<0>();
        } else {
            // V(t) has landed; K(t+1), issued after it, may still be in flight
            if (!next) wait_loads_upto<0>();
            else if (next_whole) wait_loads_upto<WN::NKI>();
            else wait_loads_upto<0>();
        }
        // ---- V steps and offsets of the tile (rows past c1 hold stale bytes)
        uint32_t dmx = 0;   // the largest step this lane copies (fp16 bits; steps are >= 0)
#pragma unroll
        for (int x = 0; x < (SROWS * NB + 63) / 64; ++x) {
            const int u = x * 64 + lane;
            if (SROWS * NB % 64 == 0 || u < SROWS * NB) {
                const int key = hrow + u / NB, blk = u - (u / NB) * NB;
                const bool live = t0 + key < c1;
                if constexpr (F8) {
                    const uint16_t dq = *reinterpret_cast<const uint16_t*>(rv + key * WN::VSTR + 32 * NB + sofs + 2 * blk);
                    const uint32_t dv = live ? dq : 0u;
                    VDa[blk * kTile + key] = (uint16_t)dv;
                    dmx = max(dmx, dv);
                } else {
                    const uint32_t dm = live ? *reinterpret_cast<const uint32_t*>(rv + key * WN::VSTR + blk * 24) : 0u;
                    VDa[blk * kTile + key] = (uint16_t)(dm & 0xFFFF);
                    dmx = max(dmx, dm & 0xFFFF);
                    VMa[key * WN::VMS + blk] = (uint16_t)(dm >> 16);
                }
            }
        }
        if constexpr (SH) {
            lds_barrier();
            // the other wave of the head converted the other 16 rows; both
            // waves see every step and so take the same decisions below
#pragma unroll
            for (int x = 0; x < (16 * NB + 63) / 64; ++x) {
                const int u = x * 64 + lane;
                if (16 * NB % 64 == 0 || u < 16 * NB) dmx = max(dmx, (uint32_t)VDa[(u - (u / NB) * NB) * kTile + (hrow ^ 16) + u / NB]);
            }
        } else {
            dec::lds_order();
        }
        // A tile with a step of 2^7 or more: its steps are stored times
        // 2^-vsh (dec::v_shift; each lane rescales the ones it converted) and
        // the accumulators switch units.
        const bool big = __any(dmx >= 0x5800u);   // fp16 128.0; wave-uniform
        if (big || vsh != 0) {
            const int want = big ? __builtin_amdgcn_readfirstlane(dec::v_shift(dec::wave_max_dpp(f16_value((uint16_t)dmx)))) : 0;
            if (want != vsh) {
                const float f = dec::pow2(vsh - want);
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                    for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) oacc[rt][dt][i] *= f;
                vsh = want;
            }
            if (vsh != 0) {
                const float f = dec::pow2(-vsh);
#pragma unroll
                for (int x = 0; x < (SROWS * NB + 63) / 64; ++x) {
                    const int u = x * 64 + lane;
                    if (SROWS * NB % 64 == 0 || u < SROWS * NB) {
                        uint16_t& e = VDa[(u - (u / NB) * NB) * kTile + hrow + u / NB];
                        e = __builtin_bit_cast(uint16_t, (_Float16)(f16_value(e) * f));
                    }
                }
                if constexpr (SH) lds_barrier(); else dec::lds_order();
            }
        }

        // ---- P V, FP8: ds_read_b64_tr_b8 of the code bytes of 8 keys gives a
        // lane dim j16 (and, 16 bytes on, dim 16 + j16) of the block
        if constexpr (F8) {
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const uint8_t* vb = rv + vkey * WN::VSTR + blk * 32 + 8 * (j16 & 1);
                const i2 ca = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(vb));
                const i2 cb = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(vb + 16));
                const h8 vf0 = e4m3_codes((uint32_t)ca[0], (uint32_t)ca[1]);
                const h8 vf1 = e4m3_codes((uint32_t)cb[0], (uint32_t)cb[1]);
                const h8 dh = steps_of(VDa + blk * kTile, q4);
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) {
                    const h8 pa = pu[rt] * dh;
                    oacc[rt][2 * blk] = dec::mfma(pa, vf0, oacc[rt][2 * blk]);
                    oacc[rt][2 * blk + 1] = dec::mfma(pa, vf1, oacc[rt][2 * blk + 1]);
                }
                if (NB > 4) asm volatile("" ::: "memory");
            }
            const h8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                             (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) macc[rt] = dec::mfma(pu[rt], ones, macc[rt]);
        } else {
        // ---- P V with the V codes built from the q5_1 bytes of 8 keys per lane group
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const uint8_t* vb = rv + vkey * WN::VSTR + blk * 24 + 8 * (j16 & 1);
            const i2 nib = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(vb + 8));   // nibble bytes
            const i2 hdr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(vb));       // d, m, high bits
            // lanes 4..7 of each 16-lane group now hold high-bit bytes 0..3 of
            // the 8 keys.  Dims j16 (first half) take byte j16 >> 3, dims
            // 16 + j16 byte 2 + (j16 >> 3): DPP row broadcasts of lanes 4 and
            // 5 (6 and 7), one of the two kept per lane (vector ALU only; a
            // ds_bpermute would wait on the LDS pipe).  The broadcasts run
            // with every lane active (a lane outside the mask would read as
            // 0), so they are pinned before the per-lane choice.
            uint32_t b4[2] = {row_bcast<4>(hdr[0]), row_bcast<4>(hdr[1])};
            uint32_t b5[2] = {row_bcast<5>(hdr[0]), row_bcast<5>(hdr[1])};
            uint32_t b6[2] = {row_bcast<6>(hdr[0]), row_bcast<6>(hdr[1])};
            uint32_t b7[2] = {row_bcast<7>(hdr[0]), row_bcast<7>(hdr[1])};
            asm volatile("" : "+v"(b4[0]), "+v"(b4[1]), "+v"(b5[0]), "+v"(b5[1]), "+v"(b6[0]), "+v"(b6[1]),
                              "+v"(b7[0]), "+v"(b7[1]));
            const uint32_t qa0 = hi8 ? b5[0] : b4[0], qa1 = hi8 ? b5[1] : b4[1];
            const uint32_t qb0 = hi8 ? b7[0] : b6[0], qb1 = hi8 ? b7[1] : b6[1];
            // code = nibble | high bit << 4: rotating the high-bit bytes right by
            // (j16 & 7) - 4 puts bit (j16 & 7) of each byte at bit 4
            const uint32_t m4 = 0x10101010u, m0 = 0x0F0F0F0Fu;
            const uint32_t c00 = (__builtin_amdgcn_alignbit(qa0, qa0, sh_rot) & m4) | ((uint32_t)nib[0] & m0);
            const uint32_t c01 = (__builtin_amdgcn_alignbit(qa1, qa1, sh_rot) & m4) | ((uint32_t)nib[1] & m0);
            const uint32_t c10 = (__builtin_amdgcn_alignbit(qb0, qb0, sh_rot) & m4) | (((uint32_t)nib[0] >> 4) & m0);
            const uint32_t c11 = (__builtin_amdgcn_alignbit(qb1, qb1, sh_rot) & m4) | (((uint32_t)nib[1] >> 4) & m0);
            const h8 vf0 = v_codes_sub(c00, c01);
            const h8 vf1 = v_codes_sub(c10, c11);
            const h8 dh = steps_of(VDa + blk * kTile, q4);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                const h8 pa = pu[rt] * dh;
                oacc[rt][2 * blk] = dec::mfma(pa, vf0, oacc[rt][2 * blk]);
                oacc[rt][2 * blk + 1] = dec::mfma(pa, vf1, oacc[rt][2 * blk + 1]);
            }
            if (NB > 4) asm volatile("" ::: "memory");
        }
        // q5_1 offset term: macc[rt][row][blk] += sum_key P[row][key] * m[key][blk]
        {
            const h8 mb = dec::tr16_pair(scb + WN::VM + (mk0 * WN::VMS + 4 * mc) * 2,
                                         scb + WN::VM + (mk1 * WN::VMS + 4 * mc) * 2);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) macc[rt] = dec::mfma(pu[rt], mb, macc[rt]);
        }
        }   // q5_1
        if constexpr (SH) {
            lds_barrier();                          // both copies of V(t) are read
            if (has2) issue_v(tn + kTile, tb);
        } else {
            if (next) issue_v(tn, tb);
        }
    }
    if (RS > 1)
        for (int it = mine; it < nit; ++it) {
            __builtin_amdgcn_s_barrier();
            if (DS == 2) __builtin_amdgcn_s_barrier();   // dim halves meet twice per tile
        }

    // ---- finish: row sums over the four lane groups; offsets into O
    // q5_1 code products carry 2^-24 (codes as fp16 subnormals), FP8 ones
    // none; P carries 2^-vsh
    const float ounit = dec::pow2((F8 ? 0 : 24) + vsh);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        // row j16's sum: element j16 & 3 of lane 16 * (j16 >> 2) + column
        const int src = 16 * (j16 >> 2) + (F8 ? 0 : NB);
        const float l0 = __shfl(macc[rt][0], src), l1 = __shfl(macc[rt][1], src);
        const float l2 = __shfl(macc[rt][2], src), l3 = __shfl(macc[rt][3], src);
        lsum[rt] = (j16 & 2) ? ((j16 & 1) ? l3 : l2) : ((j16 & 1) ? l1 : l0);
#pragma unroll
        for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oacc[rt][dt][i] = F8 ? oacc[rt][dt][i] * ounit
                                     : fmaf(oacc[rt][dt][i], ounit, __shfl(macc[rt][i], 16 * q4 + dt / 2));
    }
    // ---- row streams: the other streams hand (m, l, O) to stream 0 through
    // their own LDS buffers (lane-major, so that the 64 lanes hit 64 banks);
    // one-row-tile shapes, and dim halves (whose hand-off also covers their
    // score slots: every wave's last read of its partner's slot is done
    // first)
    if constexpr (RS > 1) {
        constexpr int MOFS = RTW * 2 * NB * 4 * 64;      // floats before m, l
        static_assert((MOFS + 64 * RTW) * 4 <= WSTR, "row-stream hand-off does not fit the wave buffer");
        if constexpr (DS == 2) lds_barrier();
        __builtin_amdgcn_s_waitcnt(0xC07F);              // this wave's reads of its buffer are done
        float* const xb = reinterpret_cast<float*>(wb);
        if (str > 0) {
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xb[((rt * 2 * NB + dt) * 4 + i) * 64 + lane] = oacc[rt][dt][i];
                if (q4 == 0) {
                    xb[MOFS + rt * 32 + j16] = mrow[rt];
                    xb[MOFS + rt * 32 + 16 + j16] = lsum[rt];
                }
            }
        }
        lds_barrier();
        if (str == 0) {
            for (int o = 1; o < rs; ++o) {
                const float* const yb = reinterpret_cast<const float*>(smem + (wave + o * gh * DS) * WSTR);
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt) {
                    const float m1 = yb[MOFS + rt * 32 + j16], l1 = yb[MOFS + rt * 32 + 16 + j16];
                    const float M = fmaxf(mrow[rt], m1);
                    const float a0 = (mrow[rt] == kNoMax) ? 0.0f : __builtin_amdgcn_exp2f(mrow[rt] - M);
                    const float a1 = (m1 == kNoMax) ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
                    lsum[rt] = a0 * lsum[rt] + a1 * l1;
                    mrow[rt] = M;
                    float A0[4], A1[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {   // O rows 4*q4 + i
                        A0[i] = __shfl(a0, 4 * q4 + i);
                        A1[i] = __shfl(a1, 4 * q4 + i);
                    }
#pragma unroll
                    for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            oacc[rt][dt][i] = A0[i] * oacc[rt][dt][i] +
                                              A1[i] * yb[((rt * 2 * NB + dt) * 4 + i) * 64 + lane];
                }
            }
        }
        if (str > 0) return;
    }
    // ---- partials of this (session, chunk)
    const size_t row0 = ((size_t)b * p.splits + s) * p.T;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int r = rb + (rt ^ rsw) * 16 + j16;
        if (q4 == 0 && r < R && half == 0) {
            const int t = tq0 + r / p.hpk, hq = g * p.hpk + r % p.hpk;
            const size_t idx = (row0 + t) * p.H + hq;
            p.part_ml[2 * idx] = (mrow[rt] == kNoMax) ? -INFINITY : mrow[rt] * kLn2;
            p.part_ml[2 * idx + 1] = lsum[rt];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ro = rb + (rt ^ rsw) * 16 + 4 * q4 + i;
            if (ro < R) {
                const int t = tq0 + ro / p.hpk, hq = g * p.hpk + ro % p.hpk;
                float* o = p.part_o + ((row0 + t) * p.H + hq) * HDR + half * HD + j16;
#pragma unroll
                for (int dt = 0; dt < 2 * NB; ++dt) o[16 * dt] = oacc[rt][dt][i];
            }
        }
    }
}

}  // namespace stream

// kvq_decode_rows.hip -- split-K flash decode over whole-row tiles (gfx950).
// Included by kvq_kernels.hip (inside namespace kvq), after kvq_decode.hip.
//
// The same partials as dec::decode_mfma (cortiq-engine "Struct LayerKvCache",
// attend_group and attend_group_upto; memra-engine "Struct KvLayer", len_d and
// base_d), organised around the HBM stream rather than around one KV head:
//   * a workgroup is (session, chunk of rows, group of gh KV heads).  In the
//     token-major planes the group's blocks of one row are gh*hd/32 adjacent
//     q8_0 blocks and gh*hd/32 adjacent q5_1 blocks, so a 32-row tile is 64
//     contiguous byte ranges.  Consecutive lanes fetch consecutive 16-byte
//     pieces of them with global_load_lds_dwordx4, straight into LDS, into
//     one of two buffers of 32*sub rows: the next buffer is in flight while
//     this one is computed, 32 rows at a time.  K rows are padded by 16 bytes when that makes the row stride
//     an odd number of 16-byte pieces, which spreads 8 consecutive rows over
//     all 32 banks.
//   * a wave is (KV head of the group, 16 query rows).  The waves that share
//     a head unpack its q5_1 blocks once, into a per-head area of byte codes
//     (0..31) plus fp32 steps, fp16 offsets and the fp32 K scales.
//   * scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_f16,
//     one per 32-element block and 16 keys), so that each lane ends up with 8
//     keys of one query row: after the softmax these are already the A
//     operand of the P V product and never pass through LDS.  The keys of
//     that operand come in the order 4*q4 + i, 16 + 4*q4 + i; the V operand
//     is read in the same order with ds_read_b64_tr_b8, whose rows are
//     addressed per lane pair.
//   * the q5_1 step multiplies P per block (P' = P * step, fp16); the offset
//     term sum_key P * m is one more MFMA per tile against the [key][block]
//     offsets.
// Each wave writes the partial (m, l, o) of its own query rows: no merge.
namespace rows {

using dec::f4;
using dec::h4;
using dec::h8;
using dec::i2;
using dec::kLn2;
using dec::kLog2e;
using dec::lds_i2;
using dec::lds_s4;
using dec::s4;

constexpr int kTile = kRowTile;   // rows per tile

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
// read; the kernel waits for them itself (wait_tile_loads) before the barrier
// that hands the buffer over.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint8_t* lds) {
    const uint32_t l = (uint32_t)(uintptr_t)(lds_u8*)lds;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(l) : "memory");
}

__device__ __forceinline__ void wait_tile_loads() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
}

// Head area: VC [32 keys][NB*32 codes] (16-byte pieces swizzled by key),
// VD [NB][32] f32 steps, KS [NB][32] f32 K scales (times scale * log2 e),
// VM [32][VMS] fp16 offsets (VMS = max(NB, 4), so that rows are 8-byte aligned).
template <int NB>
struct HeadArea {
    static constexpr int VC = 0;
    static constexpr int VD = NB * 1024;
    static constexpr int KS = VD + NB * 128;
    static constexpr int VM = KS + NB * 128;
    static constexpr int VMS = NB < 4 ? 4 : NB;
    static constexpr int SWZ = (2 * NB - 1) & 7;   // piece index XOR mask
};

// Position of key `key`'s 16-byte piece `c` inside VC.
template <int NB>
__device__ __forceinline__ int vc_off(int key, int c) {
    return key * (NB * 32) + ((c ^ (key & HeadArea<NB>::SWZ)) << 4);
}

// Key of slot k (0..7) of lane group q4 in the P V operands.
__device__ __forceinline__ int pkey(int q4, int k) { return (k < 4) ? 4 * q4 + k : 16 + 4 * q4 + (k - 4); }

template <int NB, int RT, bool QLO>
__global__ __launch_bounds__(512) void decode_rows(DecodeParams p) {
    using HA = HeadArea<NB>;
    constexpr int HD = NB * 32;
    constexpr int MAXS = kRowMaxSlots;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps load slots scalar
    const int q4 = lane >> 4, j16 = lane & 15;
    const int gh = p.gh, nw = gh * RT, ngrp = p.Hkv / gh;

    // workgroup -> (session, chunk, head group), head group fastest; an XCD
    // receives every 8th workgroup id, so logical neighbours share its L2 and
    // each XCD gets an equal share of the chunks
    const int W = gridDim.x, wid = blockIdx.x;
    const int L = (wid & 7) * (W >> 3) + (wid >> 3);
    const int hg = L % ngrp;
    int b, s, len, base;
    dec::locate_unit(p, L / ngrp, b, s, len, base);
    if (b < 0) return;
    const int gi = wave % gh, rt = wave / gh, g = hg * gh + gi;
    // query rows tq0 .. tq0 + Tq - 1 of the T: the grid's y index is the
    // group of Tg rows
    const int tq0 = blockIdx.y * p.Tg, Tq = min(p.Tg, p.T - tq0);
    const int R = Tq * p.hpk;

    // Q rows of this wave as the B operand of S^T = K Q^T:
    // lane (q4, j16) holds Q[row rt*16 + j16][blk*32 + 8*q4 .. +7]
    h8 qh[NB], ql[NB];
    {
        const int r = rt * 16 + j16;
        const bool real = r < R;
        const int t = real ? tq0 + r / p.hpk : 0, hh = real ? r % p.hpk : 0;
        const size_t i0 = (((size_t)b * p.T + t) * p.H + g * p.hpk + hh) * HD + 8 * q4;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = 0.0f;
            if (real) {
                if (p.dtype == 1) {
                    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + i0 + blk * 32);
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qv[2 * e] = __uint_as_float(w4[e] << 16);
                        qv[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
                    }
                } else {
                    const float* src = static_cast<const float*>(p.q) + i0 + blk * 32;
                    const float4 a = *reinterpret_cast<const float4*>(src);
                    const float4 c = *reinterpret_cast<const float4*>(src + 4);
                    qv[0] = a.x; qv[1] = a.y; qv[2] = a.z; qv[3] = a.w;
                    qv[4] = c.x; qv[5] = c.y; qv[6] = c.z; qv[7] = c.w;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const _Float16 xh = (_Float16)qv[e];
                qh[blk][e] = xh;
                if (QLO) ql[blk][e] = (_Float16)(qv[e] - (float)xh);
            }
        }
    }

    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int c0 = (lo & ~(kTile - 1)) + s * p.chunk;
    const int c1 = min(c0 + p.chunk, len);
    if (c0 >= c1) return;

    const RowGeo& G = p.geo;
    const int NI = G.NKI + G.NVI;
    uint8_t* const head = smem + 2 * G.RAWB + gi * G.HB;

    // Load slots of this wave: slot x is the wave-wide instruction j = wave + x*nw
    // of a buffer (K pieces for j < NKI, else V pieces); per lane, the byte
    // offset of its piece from the buffer's first row.
    const uint8_t* const kseg = p.k_planes + (int64_t)b * p.k_stride + (int64_t)hg * G.SK;
    const uint8_t* const vseg = p.v_planes + (int64_t)b * p.v_stride + (int64_t)hg * G.SV;
    auto slot_off = [&](int j) -> uint32_t {
        if (j < G.NKI) {
            const uint32_t pc = (uint32_t)(j * 64 + lane);
            const uint32_t row = __umulhi(pc, G.kmagic);
            return row * (uint32_t)p.k_row + min(pc - row * (uint32_t)G.KCP, (uint32_t)G.KC - 1) * 16u;   // the pad piece re-reads a real one
        }
        const uint32_t pc = (uint32_t)((j - G.NKI) * 64 + lane);
        const uint32_t row = __umulhi(pc, G.vmagic);
        return row * (uint32_t)p.v_row + min(pc - row * (uint32_t)G.VCP, (uint32_t)G.VC - 1) * 16u;
    };
    uint32_t soff[MAXS];
#pragma unroll
    for (int x = 0; x < MAXS; ++x) {
        const int j = wave + x * nw;
        soff[x] = j < NI ? slot_off(j) : 0u;
    }
    // Issue the loads of the buffer starting at row t0 into buffer `buf`.  Rows
    // from c1 on (only in a session's last buffer) are not loaded: they keep
    // stale LDS bytes, their scores are masked and their V steps and offsets
    // are zeroed when unpacked.  Rows below lo in the first buffer are resident
    // (the host checks that the 32-row-aligned start is at or above base) and
    // are masked.
    auto issue = [&](int t0, int buf) {
        uint8_t* const dst = smem + buf * G.RAWB;
        const int nrows = min(G.TRB, c1 - t0);
        const int limk = nrows * G.KCP, limv = nrows * G.VCP;
        const uint8_t* const kt = kseg + (int64_t)(t0 - base) * p.k_row;
        const uint8_t* const vt = vseg + (int64_t)(t0 - base) * p.v_row;
#pragma unroll
        for (int x = 0; x < MAXS; ++x) {
            const int j = wave + x * nw;
            // opaque to the optimiser, so that base + offset is formed here and
            // not hoisted out of the tile loop as one 64-bit register pair per slot
            uint32_t o = soff[x];
            asm volatile("" : "+v"(o));
            if (j < G.NKI) {
                if (lane < limk - j * 64) dma16(kt, o, dst + j * 1024);
            } else if (j < NI) {
                if (lane < limv - (j - G.NKI) * 64) dma16(vt, o, dst + G.TRB * G.KSTR + (j - G.NKI) * 1024);
            }
        }
    };

    // online-softmax state of this lane's query row (row16 = j16), and the
    // output accumulators O[row 4*q4 + i][dim 16*dt + j16]
    f4 oacc[2 * NB], macc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 2 * NB; ++dt) oacc[dt] = (f4){0.f, 0.f, 0.f, 0.f};
    float mrow = -INFINITY, lsum = 0.0f;
    int vis_lo = 0, vis_hi = 0;
    {
        const int r = rt * 16 + j16;
        if (r < R) {
            vis_hi = len - p.T + tq0 + r / p.hpk + 1;
            vis_lo = p.window > 0 ? max(0, vis_hi - p.window) : 0;
        }
    }
    // every real row of the call sees all of [full_lo, full_hi)
    const int full_hi = min(len - p.T + tq0 + 1, c1);
    const int full_lo = max(p.window > 0 ? max(0, len - p.window) : 0, c0);
    const float sc2 = p.scale * kLog2e;
    const int kcol = gi * NB * 34;   // this head's first K block inside the row segment
    const int vcol = gi * NB * 24;

    issue(c0, 0);
    int buf = 0;
    for (int tb = c0; tb < c1; tb += G.TRB, buf ^= 1) {
        wait_tile_loads();
        lds_barrier();   // the buffer is in LDS; every wave is done with the previous one
        if (tb + G.TRB < c1) issue(tb + G.TRB, buf ^ 1);
      for (int sb = 0; sb < p.sub && tb + sb * kTile < c1; ++sb) {
        const int t0 = tb + sb * kTile;
        const uint8_t* const rk = smem + buf * G.RAWB + sb * kTile * G.KSTR;     // K rows, stride KSTR
        const uint8_t* const rv = smem + buf * G.RAWB + G.TRB * G.KSTR + sb * kTile * G.VSTR;   // V rows, stride VSTR
        if (sb > 0) {   // the head area is about to be overwritten
            if (RT > 1) lds_barrier(); else dec::lds_order();
        }

        // ---- unpack this head's q5_1 blocks (shared by its RT waves) and K scales
#pragma unroll 1
        for (int u = rt * 64 + lane; u < kTile * NB; u += 64 * RT) {
            const int key = u / NB, blk = u - (u / NB) * NB;
            const uint8_t* vb = rv + key * G.VSTR + vcol + blk * 24;
            const uint2 va = reinterpret_cast<const uint2*>(vb)[0];
            const uint2 n0 = reinterpret_cast<const uint2*>(vb)[1];
            const uint2 n1 = reinterpret_cast<const uint2*>(vb)[2];
            const uint32_t qhb = va.y;
            const uint32_t nib[4] = {n0.x, n0.y, n1.x, n1.y};
            uint32_t vc[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                vc[t] = (nib[t] & 0x0F0F0F0Fu) | dec::fifth_bits((qhb >> (4 * t)) & 15u);
                vc[4 + t] = ((nib[t] >> 4) & 0x0F0F0F0Fu) | dec::fifth_bits((qhb >> (16 + 4 * t)) & 15u);
            }
            *reinterpret_cast<uint4*>(head + HA::VC + vc_off<NB>(key, 2 * blk)) = (uint4){vc[0], vc[1], vc[2], vc[3]};
            *reinterpret_cast<uint4*>(head + HA::VC + vc_off<NB>(key, 2 * blk + 1)) = (uint4){vc[4], vc[5], vc[6], vc[7]};
            const bool live = t0 + key < c1;   // rows past c1 hold stale bytes
            const uint16_t kd = *reinterpret_cast<const uint16_t*>(rk + key * G.KSTR + kcol + blk * 34);
            reinterpret_cast<float*>(head + HA::VD)[blk * kTile + key] = live ? f16_value((uint16_t)(va.x & 0xFFFF)) : 0.0f;
            reinterpret_cast<uint16_t*>(head + HA::VM)[key * HA::VMS + blk] = live ? (uint16_t)(va.x >> 16) : (uint16_t)0;
            reinterpret_cast<float*>(head + HA::KS)[blk * kTile + key] = live ? f16_value(kd) * sc2 : 0.0f;
        }
        if (RT > 1) lds_barrier(); else dec::lds_order();

        // ---- scores S^T: s[h][i] = S[row j16][key 16h + 4*q4 + i] (base 2)
        float sv[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[h][i] = 0.0f;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const float4 ks0 = *reinterpret_cast<const float4*>(head + HA::KS + (blk * kTile + 4 * q4) * 4);
            const float4 ks1 = *reinterpret_cast<const float4*>(head + HA::KS + (blk * kTile + 16 + 4 * q4) * 4);
            const float ksv[2][4] = {{ks0.x, ks0.y, ks0.z, ks0.w}, {ks1.x, ks1.y, ks1.z, ks1.w}};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = 16 * h + j16;
                // 8 code bytes of `key`, block blk, dims 8*q4..: 2-byte aligned in LDS
                const uint32_t a = (uint32_t)(key * G.KSTR + kcol + blk * 34 + 2 + 8 * q4);
                const uint32_t* w = reinterpret_cast<const uint32_t*>(rk + (a & ~3u));
                const uint32_t sh = a & 3u;
                const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
                h8 kf = dec::k_codes_f16(__builtin_amdgcn_alignbyte(w1, w0, sh),
                                         __builtin_amdgcn_alignbyte(w2, w1, sh));
                // tie this block's product to the previous block's sums, so the
                // products of all blocks are not issued at once (each holds 4
                // registers until it is scaled)
                asm volatile("" : "+v"(kf) : "v"(sv[h][0]), "v"(sv[h][1]), "v"(sv[h][2]), "v"(sv[h][3]));
                f4 d = dec::mfma(kf, qh[blk], (f4){0.f, 0.f, 0.f, 0.f});
                if (QLO) d = dec::mfma(kf, ql[blk], d);
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[h][i] = fmaf(ksv[h][i], d[i], sv[h][i]);
            }
            asm volatile("" ::: "memory");   // keep each block's LDS reads with its block
        }

        // ---- online softmax against a reference max that moves only when a
        // score passes it by more than 8 (so p <= 256, well inside fp16)
        const bool interior = t0 >= full_lo && t0 + kTile <= full_hi;
        bool over = false;
        float smax = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = sv[h][i];
                if (!interior) {
                    const int j = t0 + 16 * h + 4 * q4 + i;
                    x = (j >= vis_lo && j < vis_hi) ? x : -INFINITY;
                }
                sv[h][i] = x;
                smax = fmaxf(smax, x);
            }
        over = smax > mrow + 8.0f;   // -inf never passes
        if (__any(over)) {
            float mt = fmaxf(smax, __shfl_xor(smax, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const bool move = mt > mrow + 8.0f;
            const float alpha = move ? __builtin_amdgcn_exp2f(mrow - mt) : 1.0f;   // 0 when mrow is -inf
            mrow = move ? mt : mrow;
            lsum *= alpha;
            // O rows 4*q4 + i live in lanes j16 = 4*q4 + i
            float ar[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * q4 + i);
#pragma unroll
            for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[dt][i] *= ar[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) macc[i] *= ar[i];
        }
        float pv[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pe = (mrow == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sv[h][i] - mrow);
                pv[h][i] = pe;
                lsum += pe;
            }

        // ---- P V.  A operand: P[row j16][key pkey(q4, k)], k = 0..7.
        // V rows for the tr8 reads: lane pair (2i, 2i+1) of group q4 addresses
        // key pkey(q4, i), 8 bytes each.
        const int vkey = pkey(q4, j16 >> 1);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const float4 d0 = *reinterpret_cast<const float4*>(head + HA::VD + (blk * kTile + 4 * q4) * 4);
            const float4 d1 = *reinterpret_cast<const float4*>(head + HA::VD + (blk * kTile + 16 + 4 * q4) * 4);
            const h8 pa = {(_Float16)(pv[0][0] * d0.x), (_Float16)(pv[0][1] * d0.y),
                           (_Float16)(pv[0][2] * d0.z), (_Float16)(pv[0][3] * d0.w),
                           (_Float16)(pv[1][0] * d1.x), (_Float16)(pv[1][1] * d1.y),
                           (_Float16)(pv[1][2] * d1.z), (_Float16)(pv[1][3] * d1.w)};
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const i2 vb = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_i2*)(head + HA::VC + vc_off<NB>(vkey, 2 * blk + dd) + 8 * (j16 & 1)));
                const h8 vf = dec::v_codes_f16((uint32_t)vb[0], (uint32_t)vb[1]);
                oacc[2 * blk + dd] = dec::mfma(pa, vf, oacc[2 * blk + dd]);
            }
            asm volatile("" ::: "memory");
        }
        // q5_1 offset term: macc[row][blk] += sum_key P[row][key] * m[key][blk].
        // tr16 rows from lanes 4i..4i+3: key pkey(q4, i) (then i + 4), halves
        // 4*(j16&3)..+3 of its offsets.  Columns past NB of the product are
        // never used, so those lanes re-read the first halves.
        {
            const int c = (4 * (j16 & 3) < NB) ? (j16 & 3) : 0;
            const int k0 = pkey(q4, j16 >> 2), k1 = pkey(q4, 4 + (j16 >> 2));
            const uint8_t* a0 = head + HA::VM + (k0 * HA::VMS + 4 * c) * 2;
            const uint8_t* a1 = head + HA::VM + (k1 * HA::VMS + 4 * c) * 2;
            const h8 mb = dec::tr16_pair(a0, a1);
            const h8 pu = {(_Float16)pv[0][0], (_Float16)pv[0][1], (_Float16)pv[0][2], (_Float16)pv[0][3],
                           (_Float16)pv[1][0], (_Float16)pv[1][1], (_Float16)pv[1][2], (_Float16)pv[1][3]};
            macc = dec::mfma(pu, mb, macc);
        }
      }
    }

    // ---- finish: row sums over the four lane groups; offsets into O
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
#pragma unroll
    for (int dt = 0; dt < 2 * NB; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] += __shfl(macc[i], 16 * q4 + dt / 2);

    const size_t row0 = ((size_t)b * p.splits + s) * p.T;
    {
        const int r = rt * 16 + j16;
        if (q4 == 0 && r < R) {
            const int t = tq0 + r / p.hpk, hq = g * p.hpk + r % p.hpk;
            const size_t idx = (row0 + t) * p.H + hq;
            p.part_ml[2 * idx] = (mrow == -INFINITY) ? -INFINITY : mrow * kLn2;
            p.part_ml[2 * idx + 1] = lsum;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + 4 * q4 + i;
        if (r < R) {
            const int t = tq0 + r / p.hpk, hq = g * p.hpk + r % p.hpk;
            float* o = p.part_o + ((row0 + t) * p.H + hq) * HD + j16;
#pragma unroll
            for (int dt = 0; dt < 2 * NB; ++dt) o[16 * dt] = oacc[dt][i];
        }
    }
}

}  // namespace rows

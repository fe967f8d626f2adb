// kvq_kernels.hip -- HIP kernels for gfx950 (MI355X) and their launchers.
//
// Formats (memra-engine "Struct KvLayer" page, struct description): K rows
// are q8_0 blocks of 34 bytes (fp16 scale, 32 int8 codes), V rows are q5_1
// blocks of 24 bytes (fp16 step, fp16 offset, 4 bytes of fifth bits, 16 bytes
// of nibbles with codes j and j+16 in the low / high nibble of byte j); a
// token row keeps [kv_head, dim] order.
//
// Kernels:
//   set_kernel      writes a few int32 counters (len_d / base_d) from
//                   launch arguments: create, truncate and rebase.
//   move_kernel     one non-overlapping slab of a ring rebase.
//   append_kernel   fused quantize-and-append at slot len_d - base_d, with
//                   the len_d advance (stopped at the plane) done by the last
//                   workgroup to finish.
//   decode kernels  split-K flash decode (kvq_decode.hip, kvq_decode_stream.hip):
//                   online softmax of a group of query rows over a chunk of
//                   rows, unnormalised partial (m, l, o).
//   combine_kernel  log-sum-exp fold of the splits plus the sink column.
//   importance_kernel  per-row attention mass from the decode's lse.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "kvq_internal.h"

// Device scratch of kvq_decode_noalloc (the split-K partials of one call),
// one copy per device, held until the process ends.  Host code never uses
// this name as an address: kvq::scratch_region looks the device address up
// with hipGetSymbolAddress once per device and every launch takes that.
static __device__ __align__(256) uint8_t scratch[kvq::kScratchBytes];

namespace kvq {
namespace {

__device__ __forceinline__ float load_in(const void* base, int dtype, size_t i) {
    if (dtype == 1) {  // bf16: the upper half of a binary32
        uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16;
        return __uint_as_float(u);
    }
    return static_cast<const float*>(base)[i];
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
    _Float16 h = static_cast<_Float16>(x);  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// The OCP FP8 E4M3 code nearest to y (finite): bit 7 the sign (kept also
// when the magnitude rounds to zero), magnitudes from 2^-6 up rounded to a
// 3-bit fraction half to even, below 2^-6 to a multiple of 2^-9 half to
// even, and everything past 448 (the largest finite value) saturated to 448.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a > 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);   // 0 .. 8; 8 is 2^-6 = code 0x08
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);          // round the 23-bit fraction to 3 bits, half to even
    const uint32_t e = (u >> 23) - 120u;       // biased exponent 127 -> 7
    const uint32_t code = (e << 3) | ((u >> 20) & 7u);
    return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// ---------------------------------------------------------------------------
__global__ void set_kernel(SetParams p) {
    int i = threadIdx.x;
    if (i >= p.n) return;
    if (p.add) {
        const int b = p.idx[i];
        const int base = p.dst[p.B + b];
        const int floor = base > 0 ? base + p.window : 0;
        p.dst[b] = max(p.dst[b] + p.val[i], floor);
    } else {
        p.dst[p.idx[i]] = p.val[i];
    }
}

// ---------------------------------------------------------------------------
template <typename U>
__device__ void copy_units(uint8_t* dst, const uint8_t* src, int64_t bytes) {
    const int64_t n = bytes / (int64_t)sizeof(U);
    U* d = reinterpret_cast<U*>(dst);
    const U* s = reinterpret_cast<const U*>(src);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        d[i] = s[i];
}

__device__ void copy_bytes(uint8_t* dst, const uint8_t* src, int64_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | (uintptr_t)bytes;
    if ((a & 15) == 0) copy_units<uint4>(dst, src, bytes);
    else if ((a & 7) == 0) copy_units<uint2>(dst, src, bytes);
    else if ((a & 3) == 0) copy_units<uint32_t>(dst, src, bytes);
    else copy_units<uint16_t>(dst, src, bytes);   // rows are an even number of bytes
}

// grid.y = slab entry; grid.x strides over the bytes.  Source and destination
// ranges of one entry do not overlap (the host cuts slabs no longer than the
// shift); entries of one launch belong to distinct sessions.
__global__ void move_kernel(MoveParams p) {
    const int i = blockIdx.y;
    const int b = p.sess[i];
    if (p.zero) {
        float* const e = p.imp + (int64_t)b * p.capacity + p.dst_row[i];
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < p.rows[i];
             j += (int64_t)gridDim.x * blockDim.x)
            e[j] = 0.0f;
        return;
    }
    if (p.imp) {
        float* const e = p.imp + (int64_t)b * p.capacity;
        copy_bytes(reinterpret_cast<uint8_t*>(e + p.dst_row[i]), reinterpret_cast<const uint8_t*>(e + p.src_row[i]),
                   (int64_t)p.rows[i] * 4);
    }
    uint8_t* kp = p.k_planes + (int64_t)b * p.k_stride;
    uint8_t* vp = p.v_planes + (int64_t)b * p.v_stride;
    copy_bytes(kp + (int64_t)p.dst_row[i] * p.k_row, kp + (int64_t)p.src_row[i] * p.k_row,
               (int64_t)p.rows[i] * p.k_row);
    copy_bytes(vp + (int64_t)p.dst_row[i] * p.v_row, vp + (int64_t)p.src_row[i] * p.v_row,
               (int64_t)p.rows[i] * p.v_row);
}

// ---------------------------------------------------------------------------
// Append.  One 32-lane half-wave encodes one 32-element block index `blk` of
// one (session, row): lane i holds element i of the K block and of the V block
// (the same element range: both planes use the same blocking).  Every lane of
// the wave runs the arithmetic (inactive lanes on zeros) so that the
// cross-lane reductions and the ballot see converged waves.
// The codes are computed exactly as the format reading fixes them: scale from
// the block's absolute maximum (K) or its range (V) with IEEE division,
// rounded to fp16 to nearest even, and codes from the STORED fp16 values,
// rounded half to even (v_rndne_f32) and clamped.
#pragma clang fp contract(off)
__device__ __forceinline__ void append_unit(const AppendParams& p, int64_t unit, int64_t units, int nblk) {
    const int lane = threadIdx.x & 31;
    bool active = unit < units;
    int bi = 0, t = 0, blk = 0;
    if (active) {
        blk = (int)(unit % nblk);
        const int64_t rt = unit / nblk;
        t = (int)(rt % p.T);
        bi = (int)(rt / p.T);
        active = t < p.n_new[bi];
    }
    const int b = p.b0 + bi;
    float xk = 0.0f, xv = 0.0f;
    int64_t prow = 0;
    if (active) {
        prow = (int64_t)p.len_d[b] + t - p.base_d[b];
        if (prow < 0 || prow >= p.capacity) active = false;   // never write outside the plane
        const size_t src = ((size_t)b * p.T + t) * (size_t)(p.Hkv * p.hd) + (size_t)blk * 32 + lane;
        xk = load_in(p.k_new, p.dtype, src);
        xv = load_in(p.v_new, p.dtype, src);
    }
    if (p.f8) {
        // FP8 rows: each block's fp16 scale d = amax / 448, code = e4m3(x /
        // stored d); a row holds its blocks' codes, then their scales
        const int n_elem = nblk * 32;
        const int64_t row_bytes = (int64_t)nblk * 34;
        float ak = fabsf(xk), av = fabsf(xv);
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) {
            ak = fmaxf(ak, __shfl_xor(ak, m));
            av = fmaxf(av, __shfl_xor(av, m));
        }
        const uint16_t dk = f16_bits(ak / 448.0f), dv = f16_bits(av / 448.0f);
        const float dks = f16_value(dk), dvs = f16_value(dv);
        const uint32_t ck = dks != 0.0f ? e4m3_code(xk / dks) : 0u;
        const uint32_t cv = dvs != 0.0f ? e4m3_code(xv / dvs) : 0u;
        // four lanes' codes per word (lanes 4i .. 4i+3 of the half wave)
        uint32_t wk = ck, wv = cv;
#pragma unroll
        for (int s = 1; s < 4; ++s) {
            wk |= (uint32_t)__shfl_down((int)ck, s) << (8 * s);
            wv |= (uint32_t)__shfl_down((int)cv, s) << (8 * s);
        }
        if (active) {
            uint8_t* kr = p.k_planes + (int64_t)b * p.k_stride + prow * row_bytes;
            uint8_t* vr = p.v_planes + (int64_t)b * p.v_stride + prow * row_bytes;
            if ((lane & 3) == 0) {
                *reinterpret_cast<uint32_t*>(kr + blk * 32 + lane) = wk;
                *reinterpret_cast<uint32_t*>(vr + blk * 32 + lane) = wv;
            }
            if (lane == 0) {
                *reinterpret_cast<uint16_t*>(kr + n_elem + 2 * blk) = dk;
                *reinterpret_cast<uint16_t*>(vr + n_elem + 2 * blk) = dv;
            }
        }
        return;
    }
    // q8_0
    float amax = fabsf(xk);
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const uint16_t dk16 = f16_bits(amax / 127.0f);
    const float dks = f16_value(dk16);
    int ck = 0;
    if (dks != 0.0f) ck = (int)fminf(fmaxf(rintf(xk / dks), -127.0f), 127.0f);
    // q5_1
    float mn = xv, mx = xv;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    // signed zeros: a zero extreme is taken as +0, so that neither the stored
    // offset nor the step of a block is ever -0
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;
    const uint16_t dv16 = f16_bits((mx - mn) / 31.0f);
    const uint16_t mv16 = f16_bits(mn);
    const float dvs = f16_value(dv16);
    const float mvs = f16_value(mv16);
    int cv = 0;
    if (dvs != 0.0f) cv = (int)fminf(fmaxf(rintf((xv - mvs) / dvs), 0.0f), 31.0f);
    const uint64_t fifth = __ballot((cv >> 4) & 1);
    const uint32_t qh = (uint32_t)(fifth >> (threadIdx.x & 32));
    const int cv_hi = __shfl_xor(cv, 16);          // lane j < 16 gets code j + 16
    // stores of whole 16- and 32-bit words: K code pairs (a K block starts at
    // an even byte, its codes 2 bytes on), and V nibble bytes by fours (a V
    // block starts on 8 bytes)
    const uint32_t kb = (uint32_t)ck & 0xFFu;
    const uint32_t kpair = kb | (((uint32_t)__shfl_down((int)kb, 1) & 0xFFu) << 8);
    const uint32_t nib = (uint32_t)((cv & 15) | ((cv_hi & 15) << 4));
    uint32_t nw = nib;
#pragma unroll
    for (int s = 1; s < 4; ++s) nw |= ((uint32_t)__shfl_down((int)nib, s) & 0xFFu) << (8 * s);
    if (active) {
        uint8_t* kd = p.k_planes + (int64_t)b * p.k_stride + prow * (int64_t)(nblk * 34) + blk * 34;
        if (lane == 0) *reinterpret_cast<uint16_t*>(kd) = dk16;
        if ((lane & 1) == 0) *reinterpret_cast<uint16_t*>(kd + 2 + lane) = (uint16_t)kpair;
        uint8_t* vd = p.v_planes + (int64_t)b * p.v_stride + prow * (int64_t)(nblk * 24) + blk * 24;
        if (lane == 0) {
            *reinterpret_cast<uint32_t*>(vd) = (uint32_t)dv16 | ((uint32_t)mv16 << 16);
            *reinterpret_cast<uint32_t*>(vd + 4) = qh;
        }
        if (lane < 16 && (lane & 3) == 0) *reinterpret_cast<uint32_t*>(vd + 8 + lane) = nw;
    }
}

// Advances len_d of the launch's sessions by their rows, as far as the plane
// holds them: rows past physical row capacity - 1 were not written, len_d
// stops at base_d + capacity and the overflow flag is set.  The host checks
// room before every append it enqueues; this guard is for launches replayed
// from a captured graph, which the host does not see.
__device__ void advance_lengths(const AppendParams& p) {
    for (int i = 0; i < p.nsess; ++i) {
        const int b = p.b0 + i;
        const int room = max(0, p.capacity - (p.len_d[b] - p.base_d[b]));
        const int n = min(p.n_new[i], room);
        if (n < p.n_new[i]) *p.overflow = 1;
        p.len_d[b] += n;
    }
}

// Grid-stride over units of 8 blocks per workgroup step; the last workgroup
// to finish advances len_d.  Every workgroup has consumed its len_d reads
// (they fix its store addresses) before thread 0 counts it done, so a relaxed
// device-scope counter orders the reads before the final write.
__global__ __launch_bounds__(1024) void append_kernel(AppendParams p) {
    const int nblk = p.Hkv * p.hd / 32;
    const int64_t units = (int64_t)p.nsess * p.T * nblk;
    const int per = blockDim.x >> 5;   // blocks per workgroup pass
    for (int64_t u0 = (int64_t)blockIdx.x * per; u0 < units; u0 += (int64_t)gridDim.x * per)
        append_unit(p, u0 + (threadIdx.x >> 5), units, nblk);
    __syncthreads();
    if (gridDim.x == 1) {   // a single workgroup (a few rows): no counter needed
        if (threadIdx.x == 0) advance_lengths(p);
        return;
    }
    if (threadIdx.x == 0) {
        const int prev = atomicAdd(p.done, 1);
        if (prev == (int)gridDim.x - 1) {
            advance_lengths(p);
            atomicExch(p.done, 0);
        }
    }
}
#pragma clang fp contract(on)

// ---------------------------------------------------------------------------
#include "kvq_decode.hip"
#include "kvq_decode_stream.hip"
#include "kvq_decode_prime.hip"

// One workgroup per (session, row t, Q head h): fold the session's split
// partials (m in natural-log units, l, o), adding the sink once as a
// value-less column.  Each thread first requests its slices of o: a 4-float
// slice of every G-th split (G = NT / (hd / 4) groups of splits), up to 8 at
// once, which do not depend on the weights.  Meanwhile thread s reads split
// s's (m, l); the block maximum M (the sink included) gives the weights
// e^(m_s - M) and Z = sum_s w_s l_s (+ e^(sink - M)).  The weighted slices are
// then summed, the G group sums added in a fixed order.  NT = 1024 threads
// when there are many splits (few workgroups, each with much to read), else
// 256.
template <int kCombineThreads>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeParams p) {
    constexpr int NT = kCombineThreads, NW = NT / 64;
    __shared__ float wts[kMaxSplits];
    __shared__ float red[2][NW];
    __shared__ __align__(16) float part[NT * 4];
    const int idx = blockIdx.x;
    const int h = idx % p.H;
    const int t = (idx / p.H) % p.T;
    const int b = idx / (p.H * p.T);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int len = p.len_d[b];
    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int org = lo & ~31;   // chunks start on a 32-row boundary
    const int ns = min(p.splits, (len - org + p.chunk - 1) / p.chunk);
    const size_t stride = (size_t)p.T * p.H;
    const size_t e0 = ((size_t)b * p.splits * p.T + t) * p.H + h;   // split 0 entry

    // this thread's slices of o: splits sg, sg + G, ... (the first 8 requested now)
    const int nq = p.hd >> 2;                 // float4 slices per row (16, 32 .. 64)
    const int G = NT / nq;                    // split groups
    const int dq = tid % nq, sg = tid / nq;
    const float* o = p.part_o + e0 * p.hd + 4 * dq;
    const size_t so = stride * p.hd;
    const int s0 = (sg < G) ? sg : ns;        // threads past G groups idle (hd not dividing NT)
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = (s0 + k * G < ns) ? *reinterpret_cast<const float4*>(o + (size_t)(s0 + k * G) * so)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);

    // thread s < ns holds split s's (m, l) (at most kMaxSplits = 1024 splits,
    // and fewer than 64 for the 256-thread variant); M = max over splits (and
    // the sink); weights; Z
    static_assert(kMaxSplits <= 1024, "a thread per split");
    const bool mine = tid < ns;
    const float2 mlv = mine ? *reinterpret_cast<const float2*>(p.part_ml + 2 * (e0 + tid * stride))
                            : make_float2(-INFINITY, 0.0f);
    float mw = wave_max(mlv.x);
    if (lane == 0) red[0][wave] = mw;
    __syncthreads();
    float M = red[0][0];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[0][w]);
    const bool has_sink = p.sinks != nullptr;
    const float sink = has_sink ? p.sinks[h] : 0.0f;
    if (has_sink) M = fmaxf(M, sink);
    const float w = (mlv.x == -INFINITY) ? 0.0f : expf(mlv.x - M);
    if (mine) wts[tid] = w;
    float z = wave_sum(w * mlv.y);
    if (lane == 0) red[1][wave] = z;
    __syncthreads();   // wts and red are complete
    float Z = 0.0f;
    for (int w = 0; w < NW; ++w) Z += red[1][w];
    if (has_sink) Z += expf(sink - M);

    // weighted sum of o over the splits
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int s = s0 + k * G;
        const float w = (s < ns) ? wts[s] : 0.0f;
        acc.x = fmaf(w, v[k].x, acc.x);
        acc.y = fmaf(w, v[k].y, acc.y);
        acc.z = fmaf(w, v[k].z, acc.z);
        acc.w = fmaf(w, v[k].w, acc.w);
    }
    for (int s = s0 + 8 * G; s < ns; s += G) {   // more than 8 splits per group
        const float4 x = *reinterpret_cast<const float4*>(o + (size_t)s * so);
        const float w = wts[s];
        acc.x = fmaf(w, x.x, acc.x);
        acc.y = fmaf(w, x.y, acc.y);
        acc.z = fmaf(w, x.z, acc.z);
        acc.w = fmaf(w, x.w, acc.w);
    }
    reinterpret_cast<float4*>(part)[sg * nq + dq] = acc;
    __syncthreads();
    if (tid < nq) {
        float4 r = reinterpret_cast<const float4*>(part)[tid];
        for (int g = 1; g < G; ++g) {
            const float4 x = reinterpret_cast<const float4*>(part)[g * nq + tid];
            r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
        }
        const float invZ = 1.0f / Z;
        r.x *= invZ; r.y *= invZ; r.z *= invZ; r.w *= invZ;
        reinterpret_cast<float4*>(p.out + (((size_t)b * p.T + t) * p.H + h) * p.hd)[tid] = r;
    }
    if (p.lse && tid == 0) p.lse[((size_t)b * p.T + t) * p.H + h] = M + logf(Z);
}

// ---------------------------------------------------------------------------
// Attention importance (cortiq-engine "Struct LayerKvCache": attend_group's
// imp_acc, accumulate_imp).  Workgroup (group, session) takes group_rows
// consecutive rows (keys) of the session's visible union.  Its waves first
// copy the group's whole K rows into LDS with global_load_lds_dwordx4 (all
// requests in flight at once; row r at r * rp 16-byte pieces, from the piece
// at or below its first byte), then share the (KV head, 16-row tile of query
// rows) pairs, one pair at a time each.  A wave converts its pair's query
// rows once (each row divided by the power of two that puts its largest |q|
// in [2^14, 2^15), dec::q_down, so that bf16 queries are exact in fp16 at
// any magnitude; fp32 queries as an fp16 high and low part) and walks the
// group's 16-key tiles: the scores of the 16 keys against the 16 query rows
// are S^T = K Q^T on v_mfma_f32_16x16x32_f16, one per 32-dim block (the K
// codes exact in fp16), each block's product scaled by its keys' q8_0 (or
// FP8) scales, which each lane reads from the rows in LDS for the keys of its
// output rows.  Lane (q4, j16) then holds keys 4 q4 + i against query row
// j16: the probability 2^(log2 e (scale s - lse)) where the key is visible
// to the row, else 0, summed over the 16 rows by DPP row rotations into the
// wave's own LDS slot of the key.  At the end the waves' slots are added in a fixed
// order and one thread per key adds the total to imp: with one workgroup per
// key group (pair_blocks = 1) in a fixed order, no atomics; with many query
// rows the pairs are shared by pair_blocks workgroups (the grid's z index),
// each adding its totals with a float atomic add.  Workgroups whose keys all
// lie past the session's length return at once (the grid covers the longest
// session, or in graph mode the plane).
constexpr int kImpMaxRows = 64;   // rows (keys) per workgroup, at most
// NB = head_dim / 32 (1 .. 8), the query dtype and the K format (F8: FP8 rows,
// the codes then the scales; else q8_0 blocks) are template arguments.
template <int NB, bool F32, bool F8>
__global__ __launch_bounds__(64 * kImpWaves) void importance_kernel(ImportanceParams p) {
    using dec::f4;
    using dec::h8;
    extern __shared__ __align__(16) uint8_t krows[];   // group_rows x rp pieces of 16 bytes
    __shared__ float slot[kImpWaves][kImpMaxRows];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int q4 = lane >> 4, j16 = lane & 15;
    const int len = p.len_d[b], base = p.base_d[b];
    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int GR = p.group_rows, RP = p.rp;
    const int kg0 = lo + blockIdx.x * GR;          // first key (logical row) of the group
    if (kg0 >= len) return;                        // past this session's rows (whole workgroup)
    const int nrows = min(GR, len - kg0);
    const int ntile = (nrows + 15) / 16;
    // this workgroup's share of the (KV head, row tile) pairs
    const int R = p.T * p.hpk;
    const int nrt = (R + 15) / 16;
    const int pairs = p.Hkv * nrt;
    const int per_block = (pairs + p.pair_blocks - 1) / p.pair_blocks;
    const int pair0 = blockIdx.z * per_block, pair1 = min(pairs, pair0 + per_block);
    if (pair0 >= pair1) return;

    // ---- the group's K rows into LDS; pad pieces re-read a row's last one
    const uint8_t* const plane = p.k_planes + (int64_t)b * p.k_stride;
    const int64_t row0 = (int64_t)(kg0 - base) * p.k_row;
    const uint8_t* const gbase = plane + (row0 & ~int64_t(15));
    const int delta0 = (int)(row0 & 15);           // the group's first byte, from gbase
    const int need = nrows * RP;
    for (int x = wave; x * 64 < need; x += nw) {
        const int s = x * 64 + lane;
        const int r = s / RP, c = s - r * RP;
        const int rb = delta0 + r * p.k_row;       // row r's first byte, from gbase
        const int pc = min(rb / 16 + c, (rb + p.k_row - 1) / 16);
        if (s < need) stream::dma16(gbase, (uint32_t)(pc * 16), krows + x * 1024);
    }
    for (int i = lane; i < kImpMaxRows; i += 64) slot[wave][i] = 0.0f;
    stream::wait_loads_upto<0>();
    __syncthreads();

    for (int pi = pair0 + wave; pi < pair1; pi += nw) {
        const int g = pi / nrt, rt = pi - g * nrt;
        // ---- the pair's query rows: this lane's row j16, dims 8 q4 .. of each block
        const int r = rt * 16 + j16;
        const bool real = r < R;
        const int t = real ? r / p.hpk : 0, h = g * p.hpk + (real ? r % p.hpk : 0);
        const size_t qi = (((size_t)b * p.T + t) * p.H + h) * p.hd + 8 * q4;
        // raw words (8 bf16 or 8 fp32 values per block), the row's largest
        // magnitude from their bits, then the fp16 parts
        constexpr int QW = F32 ? 8 : 4;
        uint32_t qw[NB][QW];
        uint32_t mag = 0;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            if constexpr (!F32) {
                const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qi + blk * 32);
                qw[blk][0] = u.x; qw[blk][1] = u.y; qw[blk][2] = u.z; qw[blk][3] = u.w;
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(p.q) + qi + blk * 32);
                const uint4 a = src[0], c = src[1];
                qw[blk][0] = a.x; qw[blk][1] = a.y; qw[blk][2] = a.z; qw[blk][3] = a.w;
                qw[blk][4] = c.x; qw[blk][5] = c.y; qw[blk][6] = c.z; qw[blk][7] = c.w;
            }
#pragma unroll
            for (int e = 0; e < QW; ++e) {
                qw[blk][e] = real ? qw[blk][e] : 0u;
                if (F32) mag = max(mag, qw[blk][e] & 0x7FFFFFFFu);
                else mag = max(mag, max((qw[blk][e] << 16) & 0x7FFFFFFFu, qw[blk][e] & 0x7FFF0000u));
            }
        }
        mag = max(mag, (uint32_t)__shfl_xor((int)mag, 16));
        mag = max(mag, (uint32_t)__shfl_xor((int)mag, 32));
        const float down = dec::q_down(dec::exp_of(mag)), up = dec::q_up(dec::exp_of(mag));
        h8 qh[NB], ql[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t wv = F32 ? qw[blk][e % QW] : ((e & 1) ? (qw[blk][e / 2] & 0xFFFF0000u) : (qw[blk][e / 2] << 16));
                const float x = __uint_as_float(wv) * down;
                qh[blk][e] = (_Float16)x;
                if (F32) ql[blk][e] = (_Float16)(x - (float)qh[blk][e]);
            }
        const float l2 = real ? p.lse[((size_t)b * p.T + t) * p.H + h] * dec::kLog2e : 0.0f;
        const int upto = len - p.T + t + 1;
        const int first = p.window > 0 ? max(0, upto - p.window) : 0;
        const float su2 = p.scale * up * dec::kLog2e;

        // ---- the group's 16-key tiles.  Rows past the group's length hold
        // stale bytes; their keys lie at or past the session's length, where
        // the visibility test below selects 0 whatever their scores are.
        for (int ti = 0; ti < ntile; ++ti) {
            const int kr = ti * 16 + j16;          // this lane's key row (A operand)
            const int krow = kr * RP * 16 + ((delta0 + kr * p.k_row) & 15);   // the row's first byte in LDS
            // the first bytes of the rows whose keys this lane's D rows hold (4 q4 + i)
            int srow[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ti * 16 + 4 * q4 + i;
                srow[i] = r * RP * 16 + ((delta0 + r * p.k_row) & 15);
            }
            f4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                // fp32 queries: one block's reads at a time (tied to the
                // previous block's sums), so that the reads of all blocks
                // are not held at once
                if (F32 && NB >= 5) asm volatile("" : "+v"(sv));
                // the lane's 8 codes from the 3 aligned words holding them
                const int ca = krow + (F8 ? (g * NB + blk) * 32 : (g * NB + blk) * 34 + 2) + 8 * q4;
                const uint32_t* const cw = reinterpret_cast<const uint32_t*>(krows + (ca & ~3));
                const uint32_t sh = (uint32_t)(ca & 3) * 8;
                const uint32_t c0 = __builtin_amdgcn_alignbit(cw[1], cw[0], sh);
                const uint32_t c1 = __builtin_amdgcn_alignbit(cw[2], cw[1], sh);
                const h8 kf = F8 ? stream::e4m3_codes(c0, c1) : dec::k_codes_f16(c0, c1);
                f4 d = dec::mfma(kf, qh[blk], (f4){0.f, 0.f, 0.f, 0.f});
                if constexpr (F32) d = dec::mfma(kf, ql[blk], d);   // fp32 queries: the low part too
                // the scales of the keys of this lane's D rows, read directly
                const int so = F8 ? p.Hkv * p.hd + 2 * (g * NB + blk) : (g * NB + blk) * 34;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sv[i] = fmaf(f16_value(*reinterpret_cast<const uint16_t*>(krows + srow[i] + so)), d[i], sv[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kg0 + ti * 16 + 4 * q4 + i;
                const float pr = (real && key >= first && key < upto) ? __builtin_amdgcn_exp2f(fmaf(su2, sv[i], -l2)) : 0.0f;
                const float tot = dec::row_sum16(pr);   // over the 16 query rows of the tile
                if (j16 == 0) slot[wave][ti * 16 + 4 * q4 + i] += tot;
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nrows; i += blockDim.x) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += slot[w][i];
        float* const dst = p.imp + (size_t)b * p.capacity + (kg0 + i - base);
        if (p.pair_blocks == 1) *dst += s;
        else atomicAdd(dst, s);
    }
}

// Few splits (at most 16) and head_dim 64, 128 or 256: hd / 4 lanes per
// (session, row t, Q head h) item, 64 / (hd / 4) items per wave, four waves
// per workgroup.  Every lane reads all of its item's (m, l) pairs (the same
// addresses across the item's lanes) and its 4-float slice of every split's
// o in one round of loads, then forms M (the sink included), the weights
// e^(m_s - M), Z and the weighted sum itself: no cross-lane traffic.  The
// sink enters once, in M and Z.
constexpr int kCombineWaveSplits = 16;
__global__ __launch_bounds__(256) void combine_wave_kernel(DecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int nq = p.hd >> 2;                      // lanes per item
    const int idx = (blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / nq) + lane / nq;
    if (idx >= p.B * p.T * p.H) return;
    const int dq = lane % nq;
    const int h = idx % p.H;
    const int t = (idx / p.H) % p.T;
    const int b = idx / (p.H * p.T);
    const int len = p.len_d[b];
    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int org = lo & ~31;
    const int ns = min(p.splits, (len - org + p.chunk - 1) / p.chunk);
    const size_t stride = (size_t)p.T * p.H;
    const size_t e0 = ((size_t)b * p.splits * p.T + t) * p.H + h;
    float2 ml[kCombineWaveSplits];
    float4 v[kCombineWaveSplits];
#pragma unroll
    for (int k = 0; k < kCombineWaveSplits; ++k) {
        const bool live = k < ns;
        ml[k] = live ? *reinterpret_cast<const float2*>(p.part_ml + 2 * (e0 + k * stride)) : make_float2(-INFINITY, 0.f);
        v[k] = live ? *reinterpret_cast<const float4*>(p.part_o + (e0 + k * stride) * p.hd + 4 * dq)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const bool has_sink = p.sinks != nullptr;
    const float sink = has_sink ? p.sinks[h] : 0.0f;
    float M = has_sink ? sink : -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombineWaveSplits; ++k) M = fmaxf(M, ml[k].x);
    float Z = has_sink ? expf(sink - M) : 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kCombineWaveSplits; ++k) {
        const float w = (ml[k].x == -INFINITY) ? 0.0f : expf(ml[k].x - M);
        Z = fmaf(w, ml[k].y, Z);
        acc.x = fmaf(w, v[k].x, acc.x);
        acc.y = fmaf(w, v[k].y, acc.y);
        acc.z = fmaf(w, v[k].z, acc.z);
        acc.w = fmaf(w, v[k].w, acc.w);
    }
    const float invZ = 1.0f / Z;
    acc.x *= invZ; acc.y *= invZ; acc.z *= invZ; acc.w *= invZ;
    reinterpret_cast<float4*>(p.out + (((size_t)b * p.T + t) * p.H + h) * p.hd)[dq] = acc;
    if (p.lse && dq == 0) p.lse[((size_t)b * p.T + t) * p.H + h] = M + logf(Z);
}

// ---------------------------------------------------------------------------
int check(const char** err) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return 1;
    }
    return 0;
}

int launch_combine(const DecodeParams& p, hipStream_t st, const char** err) {
    const int items = p.B * p.T * p.H;
    // hd / 4 lanes per item where the splits are few and an item's 4-float
    // slices fill a wave in whole items (head_dim 64, 128 or 256)
    if (p.splits <= kCombineWaveSplits && (p.hd == 64 || p.hd == 128 || p.hd == 256)) {
        const int per_wg = 4 * (64 / (p.hd / 4));   // items per workgroup
        hipLaunchKernelGGL(combine_wave_kernel, dim3((items + per_wg - 1) / per_wg), dim3(256), 0, st, p);
    } else if (p.splits >= 64)
        hipLaunchKernelGGL(combine_kernel<1024>, dim3(p.B * p.T * p.H), dim3(1024), 0, st, p);
    else
        hipLaunchKernelGGL(combine_kernel<256>, dim3(p.B * p.T * p.H), dim3(256), 0, st, p);
    return check(err);
}

template <int NB, int RT, bool QLO>
int launch_decode_t(const DecodeParams& p, hipStream_t st, const char** err) {
    constexpr int lds = dec::Layout<NB, RT>::BYTES;
    static bool configured = false;
    if (!configured) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&dec::decode_mfma<NB, RT, QLO>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) {
            *err = "cannot raise the LDS limit of the decode kernel";
            return 1;
        }
        configured = true;
    }
    const int items = std::max(1, p.units) * p.Hkv;
    const int grid = (items + 7) & ~7;
    hipLaunchKernelGGL((dec::decode_mfma<NB, RT, QLO>), dim3(grid, (p.T + p.Tg - 1) / p.Tg), dim3(256), lds, st, p);
    return check(err);
}

template <int NB, int RTW, bool QLO, int RS, int RG, int DS, bool F8>
int launch_stream_t(const DecodeParams& p, hipStream_t st, const char** err) {
    static bool configured = false;
    if (!configured) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&stream::decode_stream<NB, RTW, QLO, RS, RG, DS, F8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess) {
            *err = "cannot raise the LDS limit of the decode kernel";
            return 1;
        }
        configured = true;
    }
    const int items = std::max(1, p.units) * (p.Hkv / p.gh);
    const int grid = (items + 7) & ~7;
    hipLaunchKernelGGL((stream::decode_stream<NB, RTW, QLO, RS, RG, DS, F8>), dim3(grid, (p.T + p.Tg - 1) / p.Tg),
                       dim3(64 * p.gh * RS * RG * DS), p.lds, st, p);
    return check(err);
}

template <int NB, bool QLO, bool F8>
int launch_prime_t(const DecodeParams& p, hipStream_t st, const char** err) {
    constexpr int lds = PrimeLayout<NB, F8>::BYTES;
    static bool configured = false;
    if (!configured) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&prime::decode_prime<NB, QLO, F8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) {
            *err = "cannot raise the LDS limit of the decode kernel";
            return 1;
        }
        configured = true;
    }
    const int items = std::max(1, p.units) * p.Hkv;
    const int grid = (items + 7) & ~7;
    const int groups = (p.T + p.Tg - 1) / p.Tg;
    hipLaunchKernelGGL((prime::decode_prime<NB, QLO, F8>), dim3(grid, (groups + kPrimeGroups - 1) / kPrimeGroups),
                       dim3(64 * kPrimeGroups), lds, st, p);
    return check(err);
}

template <int NB, bool F8>
int launch_stream_fmt(const DecodeParams& p, hipStream_t st, const char** err) {
    const int R = p.Tg * p.hpk;   // query rows per KV head of one group
    const bool qlo = p.dtype == 0;
    if (R > 16) {
        if (p.ds == 2) {   // two waves per head, each half of its dims (head_dim 128 or 256)
            constexpr int NH = NB / 2;
            if constexpr (NB == 8 || NB == 4) {
                if (p.rs == 2)   // and two row streams
                    return qlo ? launch_stream_t<NH, 2, true, 2, 1, 2, F8>(p, st, err)
                               : launch_stream_t<NH, 2, false, 2, 1, 2, F8>(p, st, err);
                return qlo ? launch_stream_t<NH, 2, true, 1, 1, 2, F8>(p, st, err)
                           : launch_stream_t<NH, 2, false, 1, 1, 2, F8>(p, st, err);
            }
            *err = "dim halves are built for head_dim 128 and 256";
            return 1;
        }
        if (p.rg == 2)   // two 16-row groups, one wave each
            return qlo ? launch_stream_t<NB, 1, true, 1, 2, 1, F8>(p, st, err)
                       : launch_stream_t<NB, 1, false, 1, 2, 1, F8>(p, st, err);
        return qlo ? launch_stream_t<NB, 2, true, 1, 1, 1, F8>(p, st, err)
                   : launch_stream_t<NB, 2, false, 1, 1, 1, F8>(p, st, err);
    }
    if (p.rs == 2) {
        // two row streams: bf16 queries and head_dim 64 or 128 only (the planner's rule)
        if constexpr (NB <= 4) {
            if (!qlo) return launch_stream_t<NB, 1, false, 2, 1, 1, F8>(p, st, err);
        }
        *err = "two row streams are not built for this shape";
        return 1;
    }
    return qlo ? launch_stream_t<NB, 1, true, 1, 1, 1, F8>(p, st, err)
               : launch_stream_t<NB, 1, false, 1, 1, 1, F8>(p, st, err);
}

template <int NB>
int launch_stream_nb(const DecodeParams& p, hipStream_t st, const char** err) {
    return p.f8 ? launch_stream_fmt<NB, true>(p, st, err) : launch_stream_fmt<NB, false>(p, st, err);
}

template <int NB>
int launch_decode_nb(const DecodeParams& p, hipStream_t st, const char** err) {
    const int R = p.Tg * p.hpk;   // query rows per KV head of one group
    const bool qlo = p.dtype == 0;   // fp32 queries keep a low fp16 part
    if (R <= 16) return qlo ? launch_decode_t<NB, 1, true>(p, st, err) : launch_decode_t<NB, 1, false>(p, st, err);
    return qlo ? launch_decode_t<NB, 2, true>(p, st, err) : launch_decode_t<NB, 2, false>(p, st, err);
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int scratch_region(void** ptr, const char** err) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = "cannot tell the current device";
        return 1;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? hipGetErrorString(e) : "the scratch symbol has no device address";
            return 1;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return 0;
}

int device_compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

int launch_set(const SetParams& p, void* stream, const char** err) {
    hipLaunchKernelGGL(set_kernel, dim3(1), dim3(kMaxSetPerLaunch), 0, (hipStream_t)stream, p);
    return check(err);
}

int launch_move(const MoveParams& p, void* stream, const char** err) {
    int64_t maxbytes = 0;
    for (int i = 0; i < p.n; ++i) maxbytes = std::max<int64_t>(maxbytes, (int64_t)p.rows[i] * (p.zero ? 4 : p.k_row));
    int gx = (int)std::min<int64_t>(1024, (maxbytes / 16 + 255) / 256 + 1);
    hipLaunchKernelGGL(move_kernel, dim3(gx, p.n), dim3(256), 0, (hipStream_t)stream, p);
    return check(err);
}

int launch_append(const AppendParams& p, void* stream, const char** err) {
    const int64_t units = (int64_t)p.nsess * p.T * (p.Hkv * p.hd / 32);
    // up to 32 blocks in one workgroup of 1024 threads, which then needs no
    // completion counter
    if (units <= 32) {
        hipLaunchKernelGGL(append_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, p);
        return check(err);
    }
    // At most 256 workgroups: every workgroup adds to the completion counter,
    // and those device-scope atomics on one word are served one at a time,
    // so past that count more workgroups cost more than the extra passes of
    // fewer ones.  256 threads (8 blocks a pass) while one pass of them
    // covers the launch, else 1024 (32 blocks a pass).
    if ((units + 7) / 8 <= 256) {
        hipLaunchKernelGGL(append_kernel, dim3((unsigned)((units + 7) / 8)), dim3(256), 0, (hipStream_t)stream, p);
        return check(err);
    }
    const int64_t grid = std::min<int64_t>((units + 31) / 32, 256);
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)grid), dim3(1024), 0, (hipStream_t)stream, p);
    return check(err);
}

namespace {
int launch_partials(const DecodeParams& p, hipStream_t st, const char** err) {
    if (p.kernel == kPrime) {
        const bool qlo = p.dtype == 0;
#define KVQ_PRIME(NB, F8) return qlo ? launch_prime_t<NB, true, F8>(p, st, err) : launch_prime_t<NB, false, F8>(p, st, err)
        switch ((p.hd / 32) * 2 + (p.f8 ? 1 : 0)) {
            case 4: KVQ_PRIME(2, false);
            case 5: KVQ_PRIME(2, true);
            case 8: KVQ_PRIME(4, false);
            case 9: KVQ_PRIME(4, true);
            default: *err = "the prime decode supports head_dim 64 and 128"; return 1;
        }
#undef KVQ_PRIME
    }
    if (p.kernel == kStream) {
        switch (p.hd / 32) {
            case 2: return launch_stream_nb<2>(p, st, err);
            case 4: return launch_stream_nb<4>(p, st, err);
            case 8: return launch_stream_nb<8>(p, st, err);
            default: *err = "the stream decode supports head_dim 64, 128 and 256"; return 1;
        }
    }
    if (p.f8) {
        *err = "the per-head decode reads q8_0 / q5_1 blocks only";
        return 1;
    }
    switch (p.hd / 32) {
        case 1: return launch_decode_nb<1>(p, st, err);
        case 2: return launch_decode_nb<2>(p, st, err);
        case 3: return launch_decode_nb<3>(p, st, err);
        case 4: return launch_decode_nb<4>(p, st, err);
        case 5: return launch_decode_nb<5>(p, st, err);
        case 6: return launch_decode_nb<6>(p, st, err);
        case 7: return launch_decode_nb<7>(p, st, err);
        case 8: return launch_decode_nb<8>(p, st, err);
        default: *err = "unsupported head_dim"; return 1;
    }
}
}  // namespace

template <bool F32>
bool launch_importance_dtype(const ImportanceParams& p, hipStream_t st) {
    // a workgroup's share of the (KV head, row tile) pairs over at most
    // kImpWaves waves
    const int pairs = p.Hkv * ((p.T * p.hpk + 15) / 16);
    const int per_block = (pairs + p.pair_blocks - 1) / p.pair_blocks;
    const dim3 grid((p.tiles * 16 + p.group_rows - 1) / p.group_rows, p.B, p.pair_blocks),
        block(64 * std::min(per_block, kImpWaves));
    const size_t lds = (size_t)p.group_rows * p.rp * 16;
#define KVQ_IMP(NB, F8) hipLaunchKernelGGL((importance_kernel<NB, F32, F8>), grid, block, lds, st, p); return true
    if (p.f8) {   // FP8 rows: head_dim 64, 128 or 256
        switch (p.hd / 32) {
            case 2: KVQ_IMP(2, true);
            case 4: KVQ_IMP(4, true);
            case 8: KVQ_IMP(8, true);
            default: return false;
        }
    }
    switch (p.hd / 32) {
        case 1: KVQ_IMP(1, false);
        case 2: KVQ_IMP(2, false);
        case 3: KVQ_IMP(3, false);
        case 4: KVQ_IMP(4, false);
        case 5: KVQ_IMP(5, false);
        case 6: KVQ_IMP(6, false);
        case 7: KVQ_IMP(7, false);
        case 8: KVQ_IMP(8, false);
        default: return false;
    }
#undef KVQ_IMP
}

int launch_importance(const ImportanceParams& p, void* stream, const char** err) {
    if (p.hd % 32 != 0 || !(p.dtype == 0 ? launch_importance_dtype<true>(p, (hipStream_t)stream)
                                         : launch_importance_dtype<false>(p, (hipStream_t)stream))) {
        *err = "importance: head_dim must be 32 .. 256 in steps of 32";
        return 1;
    }
    return check(err);
}

int launch_decode(const DecodeParams& p, void* stream, void* const ev[3], const char** err) {
    hipStream_t st = (hipStream_t)stream;
    auto mark = [&](int i) {
        if (!ev[i]) return 0;
        const hipError_t e = hipEventRecord((hipEvent_t)ev[i], st);
        if (e != hipSuccess) {
            *err = hipGetErrorString(e);
            return 1;
        }
        return 0;
    };
    if (mark(0) || launch_partials(p, st, err) || mark(1) || launch_combine(p, st, err)) return 1;
    return mark(2);
}

}  // namespace kvq

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
//                   the len_d advance done by the last workgroup to finish.
//   decode_kernel   split-K flash decode over one (session, row chunk,
//                   KV head): online softmax of the group's T*H/Hkv query
//                   rows, unnormalised partial (m, l, o).
//   combine_kernel  log-sum-exp fold of the splits plus the sink column.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvq_internal.h"

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
    if (i < p.n) p.dst[p.idx[i]] = p.val[i];
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
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int nblk = p.Hkv * p.hd / 32;
    const int lane = threadIdx.x & 31;
    const int64_t unit = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
    const int64_t units = (int64_t)p.nsess * p.T * nblk;
    bool active = unit < units;
    int bi = 0, t = 0, blk = 0;
    if (active) {
        blk = (int)(unit % nblk);
        int64_t rt = unit / nblk;
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
    if (active) {
        uint8_t* kd = p.k_planes + (int64_t)b * p.k_stride + prow * (int64_t)(nblk * 34) + blk * 34;
        if (lane == 0) *reinterpret_cast<uint16_t*>(kd) = dk16;
        kd[2 + lane] = (uint8_t)(int8_t)ck;
        uint8_t* vd = p.v_planes + (int64_t)b * p.v_stride + prow * (int64_t)(nblk * 24) + blk * 24;
        if (lane == 0) {
            *reinterpret_cast<uint32_t*>(vd) = (uint32_t)dv16 | ((uint32_t)mv16 << 16);
            *reinterpret_cast<uint32_t*>(vd + 4) = qh;
        }
        if (lane < 16) vd[8 + lane] = (uint8_t)((cv & 15) | ((cv_hi & 15) << 4));
    }
    // The last workgroup to finish advances len_d: every workgroup has read
    // its slot from len_d before it counts itself done.
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const int prev = atomicAdd(p.done, 1);
        if (prev == (int)gridDim.x - 1) {
            for (int i = 0; i < p.nsess; ++i) p.len_d[p.b0 + i] += p.n_new[i];
            atomicExch(p.done, 0);
            __threadfence();
        }
    }
}
#pragma clang fp contract(on)

// ---------------------------------------------------------------------------
// Decode, first version: plain fp32 VALU arithmetic on codes staged in LDS.
// Workgroup = (session b, split s, KV head g), 256 threads; the split covers
// rows [lo + s*chunk, min(lo + (s+1)*chunk, len)) of the union of the visible
// ranges of the T query rows.  Query row r = t*hpk + hh is Q head g*hpk + hh
// at verify row t.
constexpr int kTK = 64;   // keys per tile

__device__ __forceinline__ int round16(int x) { return (x + 15) & ~15; }

template <int NB>
__host__ __device__ constexpr int decode_lds_bytes(int R) {
    return R * NB * 32 * 4 + ((kTK * NB * 34 + 15) & ~15) + ((kTK * NB * 24 + 15) & ~15) +
           R * kTK * 4 + 3 * kMaxRows * 4;
}

template <int NB>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    constexpr int HD = NB * 32;
    constexpr int KSEG = NB * 34;
    constexpr int VSEG = NB * 24;
    constexpr int RG = (256 / HD) > 0 ? 256 / HD : 1;       // row groups in the PV phase
    constexpr int MAXO = kMaxQFloats / 256;                  // accumulators per thread
    extern __shared__ __align__(16) uint8_t smem[];
    const int R = p.T * p.hpk;
    float* q_s = reinterpret_cast<float*>(smem);
    uint8_t* kt = smem + R * HD * 4;
    uint8_t* vt = kt + round16(kTK * KSEG);
    float* sp = reinterpret_cast<float*>(vt + round16(kTK * VSEG));
    float* m_s = sp + R * kTK;
    float* l_s = m_s + kMaxRows;
    float* a_s = l_s + kMaxRows;

    // XCD-aware order: consecutive logical items (the KV heads of one chunk)
    // land on the same XCD, which dispatches workgroup ids round-robin.
    const int W = gridDim.x;
    const int w = blockIdx.x;
    const int L = (w & 7) * (W >> 3) + (w >> 3);
    const int g = L % p.Hkv;
    const int s = (L / p.Hkv) % p.splits;
    const int b = L / (p.Hkv * p.splits);
    if (b >= p.B) return;
    const int len = p.len_d[b];
    const int base = p.base_d[b];
    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int c0 = lo + s * p.chunk;
    const int c1 = min(c0 + p.chunk, len);
    if (c0 >= c1) return;
    const int tid = threadIdx.x;

    for (int i = tid; i < R * HD; i += 256) {
        const int r = i / HD, d = i % HD;
        const int t = r / p.hpk, hh = r % p.hpk;
        q_s[i] = load_in(p.q, p.dtype, (((size_t)b * p.T + t) * p.H + g * p.hpk + hh) * HD + d);
    }
    for (int r = tid; r < R; r += 256) {
        m_s[r] = -INFINITY;
        l_s[r] = 0.0f;
    }
    const int d = tid % HD;
    const int rg = tid / HD;
    float o[MAXO];
#pragma unroll
    for (int i = 0; i < MAXO; ++i) o[i] = 0.0f;
    __syncthreads();

    const uint8_t* kp = p.k_planes + (int64_t)b * p.k_stride + (int64_t)g * KSEG;
    const uint8_t* vp = p.v_planes + (int64_t)b * p.v_stride + (int64_t)g * VSEG;
    for (int j0 = c0; j0 < c1; j0 += kTK) {
        const int nk = min(kTK, c1 - j0);
        // stage the group's K and V segments of rows j0 .. j0+nk-1
        for (int u = tid; u < nk * (KSEG / 2); u += 256) {
            const int key = u / (KSEG / 2), off = u % (KSEG / 2);
            reinterpret_cast<uint16_t*>(kt + key * KSEG)[off] =
                reinterpret_cast<const uint16_t*>(kp + (int64_t)(j0 + key - base) * p.k_row)[off];
        }
        for (int u = tid; u < nk * (VSEG / 2); u += 256) {
            const int key = u / (VSEG / 2), off = u % (VSEG / 2);
            reinterpret_cast<uint16_t*>(vt + key * VSEG)[off] =
                reinterpret_cast<const uint16_t*>(vp + (int64_t)(j0 + key - base) * p.v_row)[off];
        }
        __syncthreads();
        // scores: thread -> key tid%64, rows r = tid/64 + 4*i
        {
            const int key = tid & 63;
            const int r0 = tid >> 6;
            float acc[kMaxRows / 4];
#pragma unroll
            for (int i = 0; i < kMaxRows / 4; ++i) acc[i] = 0.0f;
            if (key < nk) {
                const uint16_t* kr = reinterpret_cast<const uint16_t*>(kt + key * KSEG);
                for (int kb = 0; kb < NB; ++kb) {
                    const float ds = f16_value(kr[kb * 17]);
                    float c[32];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const uint16_t wd = kr[kb * 17 + 1 + i];
                        c[2 * i] = (float)(int8_t)(wd & 0xFF);
                        c[2 * i + 1] = (float)(int8_t)(wd >> 8);
                    }
#pragma unroll
                    for (int i = 0; i < kMaxRows / 4; ++i) {
                        const int r = r0 + 4 * i;
                        if (r < R) {
                            const float* qr = q_s + r * HD + kb * 32;
                            float dot = 0.0f;
#pragma unroll
                            for (int e = 0; e < 32; ++e) dot = fmaf(qr[e], c[e], dot);
                            acc[i] = fmaf(ds, dot, acc[i]);
                        }
                    }
                }
            }
            const int j = j0 + key;
#pragma unroll
            for (int i = 0; i < kMaxRows / 4; ++i) {
                const int r = r0 + 4 * i;
                if (r < R) {
                    const int t = r / p.hpk;
                    const int hi = len - p.T + t + 1;
                    const int lo_t = p.window > 0 ? max(0, hi - p.window) : 0;
                    const bool vis = key < nk && j >= lo_t && j < hi;
                    sp[r * kTK + key] = vis ? acc[i] * p.scale : -INFINITY;
                }
            }
        }
        __syncthreads();
        // online softmax: wave -> rows r = wave + 4*i, lane -> key
        {
            const int wv = tid >> 6, lane = tid & 63;
            for (int r = wv; r < R; r += 4) {
                const float sv = sp[r * kTK + lane];
                const float m_old = m_s[r];
                const float m_new = fmaxf(m_old, wave_max(sv));
                float pv = 0.0f, alpha = 1.0f;
                if (m_new != -INFINITY) {
                    pv = (sv == -INFINITY) ? 0.0f : expf(sv - m_new);
                    alpha = (m_old == -INFINITY) ? 0.0f : expf(m_old - m_new);
                }
                const float sum = wave_sum(pv);
                sp[r * kTK + lane] = pv;
                if (lane == 0) {
                    l_s[r] = l_s[r] * alpha + sum;
                    m_s[r] = m_new;
                    a_s[r] = alpha;
                }
            }
        }
        __syncthreads();
        // P.V: thread -> dim d, rows r = rg + RG*i
        {
            const int blk = d >> 5, e = d & 31;
#pragma unroll
            for (int i = 0; i < MAXO; ++i) {
                const int r = rg + RG * i;
                if (r < R) o[i] *= a_s[r];
            }
            for (int key = 0; key < nk; ++key) {
                const uint8_t* vb = vt + key * VSEG + blk * 24;
                const float dsv = f16_value(*reinterpret_cast<const uint16_t*>(vb));
                const float msv = f16_value(*reinterpret_cast<const uint16_t*>(vb + 2));
                const uint32_t qh = *reinterpret_cast<const uint32_t*>(vb + 4);
                const int nib = (vb[8 + (e & 15)] >> ((e >> 4) * 4)) & 15;
                const int code = nib | (int)(((qh >> e) & 1u) << 4);
                const float v = fmaf(dsv, (float)code, msv);
#pragma unroll
                for (int i = 0; i < MAXO; ++i) {
                    const int r = rg + RG * i;
                    if (r < R) o[i] = fmaf(sp[r * kTK + key], v, o[i]);
                }
            }
        }
        __syncthreads();
    }
    // partials
    const size_t row0 = ((size_t)b * p.splits + s) * p.T;
    for (int r = tid; r < R; r += 256) {
        const int t = r / p.hpk, h = g * p.hpk + r % p.hpk;
        const size_t idx = (row0 + t) * p.H + h;
        p.part_ml[2 * idx] = m_s[r];
        p.part_ml[2 * idx + 1] = l_s[r];
    }
#pragma unroll
    for (int i = 0; i < MAXO; ++i) {
        const int r = rg + RG * i;
        if (r < R) {
            const int t = r / p.hpk, h = g * p.hpk + r % p.hpk;
            p.part_o[((row0 + t) * p.H + h) * HD + d] = o[i];
        }
    }
}

// One 64-lane workgroup per (session, row t, Q head h): fold the session's
// splits, adding the sink once as a value-less column.
__global__ __launch_bounds__(64) void combine_kernel(DecodeParams p) {
    const int idx = blockIdx.x;
    const int h = idx % p.H;
    const int t = (idx / p.H) % p.T;
    const int b = idx / (p.H * p.T);
    const int len = p.len_d[b];
    const int lo = p.window > 0 ? max(0, len - p.T + 1 - p.window) : 0;
    const int ns = min(p.splits, (len - lo + p.chunk - 1) / p.chunk);
    const size_t stride = (size_t)p.T * p.H;
    const size_t e0 = ((size_t)b * p.splits * p.T + t) * p.H + h;   // split 0 entry
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p.part_ml[2 * (e0 + s * stride)]);
    const bool has_sink = p.sinks != nullptr;
    const float sink = has_sink ? p.sinks[h] : 0.0f;
    if (has_sink) M = fmaxf(M, sink);
    float Z = has_sink ? expf(sink - M) : 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float m = p.part_ml[2 * (e0 + s * stride)];
        if (m != -INFINITY) Z += p.part_ml[2 * (e0 + s * stride) + 1] * expf(m - M);
    }
    const float invZ = 1.0f / Z;
    for (int d = threadIdx.x; d < p.hd; d += 64) {
        float acc = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const float m = p.part_ml[2 * (e0 + s * stride)];
            if (m != -INFINITY) acc += expf(m - M) * p.part_o[(e0 + s * stride) * p.hd + d];
        }
        p.out[(((size_t)b * p.T + t) * p.H + h) * p.hd + d] = acc * invZ;
    }
    if (p.lse && threadIdx.x == 0) p.lse[((size_t)b * p.T + t) * p.H + h] = M + logf(Z);
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

template <int NB>
int launch_decode_nb(const DecodeParams& p, hipStream_t st, const char** err) {
    const int R = p.T * p.hpk;
    const int lds = decode_lds_bytes<NB>(R);
    static int configured = 0;
    if (!configured) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<NB>),
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                decode_lds_bytes<NB>(kMaxRows)) != hipSuccess) {
            *err = "cannot raise the LDS limit of the decode kernel";
            return 1;
        }
        configured = 1;
    }
    const int items = p.B * p.splits * p.Hkv;
    const int grid = (items + 7) & ~7;
    hipLaunchKernelGGL(decode_kernel<NB>, dim3(grid), dim3(256), lds, st, p);
    if (check(err)) return 1;
    hipLaunchKernelGGL(combine_kernel, dim3(p.B * p.T * p.H), dim3(64), 0, st, p);
    return check(err);
}

}  // namespace

int launch_set(const SetParams& p, void* stream, const char** err) {
    hipLaunchKernelGGL(set_kernel, dim3(1), dim3(kMaxSetPerLaunch), 0, (hipStream_t)stream, p);
    return check(err);
}

int launch_move(const MoveParams& p, void* stream, const char** err) {
    int64_t maxbytes = 0;
    for (int i = 0; i < p.n; ++i) maxbytes = std::max<int64_t>(maxbytes, (int64_t)p.rows[i] * p.k_row);
    int gx = (int)std::min<int64_t>(1024, (maxbytes / 16 + 255) / 256 + 1);
    hipLaunchKernelGGL(move_kernel, dim3(gx, p.n), dim3(256), 0, (hipStream_t)stream, p);
    return check(err);
}

int launch_append(const AppendParams& p, void* stream, const char** err) {
    const int64_t units = (int64_t)p.nsess * p.T * (p.Hkv * p.hd / 32);
    const int64_t grid = (units * 32 + 255) / 256;
    if (grid > INT32_MAX) {
        *err = "append too large for one launch";
        return 1;
    }
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, p);
    return check(err);
}

int launch_decode(const DecodeParams& p, void* stream, const char** err) {
    hipStream_t st = (hipStream_t)stream;
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

}  // namespace kvq

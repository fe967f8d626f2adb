// kvq_internal.h -- parameter blocks passed by value from the host library
// (kvq_host.cpp) to the kernel launchers (kvq_kernels.hip), and the launcher
// interface.  Free of HIP types so that the host logic also builds, with a
// recording launcher (kvq_nodev.cpp), as a plain C++ library for CPU tests.
#pragma once

#include <cstddef>
#include <cstdint>

namespace kvq {

constexpr int kMaxSessionsPerLaunch = 64;   // by-value per-session arrays
constexpr int kMaxSetPerLaunch = 128;
constexpr int kMaxRows = 32;                // query rows per KV head in one decode workgroup (Tg * H / Hkv)
constexpr int kMaxSplits = 1024;            // split-K chunks per session
constexpr int kMaxHeadDim = 256;
constexpr int kSplitQuantum = 64;           // split-K chunk rows are a multiple of this

// Quantize rows of k_new / v_new and write them at slot len_d[b] - base_d[b] + t,
// then advance len_d[b] by the session's row count (last workgroup to finish).
struct AppendParams {
    const void* k_new;          // [B, T, Hkv, hd]
    const void* v_new;
    uint8_t* k_planes;
    uint8_t* v_planes;
    int64_t k_stride;           // bytes between sessions' K planes
    int64_t v_stride;
    int32_t* len_d;
    int32_t* base_d;
    int32_t* done;              // completion counter, 0 between launches
    int32_t* overflow;          // set to 1 when rows did not fit the plane (sticky)
    int32_t f8;                 // 1: K and V as FP8 rows (codes, then scales); 0: q8_0 / q5_1
    int32_t dtype;              // kvq_dtype
    int32_t B;                  // sessions in the input tensors
    int32_t T;                  // rows per session in the input tensors
    int32_t Hkv;
    int32_t hd;
    int32_t capacity;
    int32_t b0;                 // this launch covers sessions [b0, b0 + nsess)
    int32_t nsess;
    int32_t n_new[kMaxSessionsPerLaunch];   // rows appended per covered session
};

// dst[idx[i]] = val[i] for i < n.
struct SetParams {
    int32_t* dst;
    int32_t n;
    int32_t add;                // 0: dst[idx] = val.  1: dst[idx] += val for len_d entries
                                // (idx < B), stopping at the shortest length whose
                                // window is still resident: base_d + window when
                                // base_d > 0, else 0
    int32_t B, window;
    int32_t idx[kMaxSetPerLaunch];
    int32_t val[kMaxSetPerLaunch];
};

// One non-overlapping slab per listed session: physical rows
// [src_row, src_row + rows) -> [dst_row, dst_row + rows) of the K and V planes
// (and of imp, when set).  zero = 1: instead, imp's entries [dst_row, dst_row
// + rows) of each listed session are set to 0 (the planes are not touched).
struct MoveParams {
    float* imp;                 // [B, capacity] importance by physical row, or null
    int32_t capacity;
    int32_t zero;
    uint8_t* k_planes;
    uint8_t* v_planes;
    int64_t k_stride;
    int64_t v_stride;
    int32_t k_row;              // bytes per K row
    int32_t v_row;
    int32_t n;
    int32_t sess[kMaxSessionsPerLaunch];
    int32_t src_row[kMaxSessionsPerLaunch];
    int32_t dst_row[kMaxSessionsPerLaunch];
    int32_t rows[kMaxSessionsPerLaunch];
};

// Attention importance: per session b and row j of the T query rows' union,
// imp[b][j - base] += sum over (t, h) of exp(scale q.K'_j - lse[b, t, h]).
struct ImportanceParams {
    const void* q;              // [B, T, H, hd]
    int32_t f8;                 // K as FP8 rows (1) or q8_0 blocks (0)
    int32_t dtype;
    int32_t B, T, H, Hkv, hd, hpk, window, capacity;
    const uint8_t* k_planes;
    int64_t k_stride;
    int32_t k_row;
    const int32_t* len_d;
    const int32_t* base_d;
    float scale;
    const float* lse;           // [B, T, H], natural log, the sink included
    float* imp;                 // [B, capacity] by physical row
    int32_t tiles;              // 16-row tiles per session in the grid
    int32_t group_rows;         // rows (keys) per workgroup: a multiple of 16, at most 64
    int32_t rp;                 // 16-byte pieces per K row in LDS (odd, >= (k_row + 30) / 16)
    int32_t pair_blocks;        // workgroups per key group, each a share of its (KV head, row tile) pairs
};


constexpr int kRowTile = 32;          // rows per tile of the stream kernel
constexpr int kImpWaves = 8;          // waves per importance workgroup, at most
constexpr int kImpPairsPerWave = 4;   // (KV head, row tile) pairs per importance wave before the pairs are split
constexpr int kLdsBytes = 160 * 1024;

// The importance workgroup's rows and its LDS row stride in pieces for K
// rows of k_row bytes: as many rows (16 .. 64, a multiple of 16) as half the
// LDS holds next to the 2 KiB of per-wave key sums, so that two workgroups
// share a CU, or all of it for long rows.  Returns false when not even 16
// rows fit.
inline bool importance_group(int k_row, int* rows, int* rp) {
    *rp = ((k_row + 30) / 16) | 1;
    const int bytes_per_row = *rp * 16;
    int r = (kLdsBytes / 2 - 2048) / bytes_per_row;
    if (r < 16) r = (kLdsBytes - 2048) / bytes_per_row;
    r = r / 16 * 16;
    if (r < 16) return false;
    *rows = r > 64 ? 64 : r;
    return true;
}

// Geometry of the per-wave stream decode kernel for head_dim = 32 * NB (NB
// even): each wave copies its KV head's row windows of a 32-row tile, in
// 16-byte pieces, into one private LDS buffer (K rows, then V rows), and
// builds per-tile scale arrays.
template <int NB>
struct StreamWin {
    static constexpr int MAXKOFS = (NB % 8 == 0) ? 0 : (NB % 4 == 0) ? 8 : 12;   // (g*NB*34) mod 16, at most
    static constexpr int KW = (MAXKOFS + 34 * NB + 15) / 16;   // K pieces per row window
    static constexpr int KWP = KW | 1;                          // LDS row stride in pieces (odd)
    static constexpr int VW = 24 * NB / 16;                     // V pieces per row
    static constexpr int VWP = VW | 1;
    static constexpr int TR = kRowTile;                         // rows per tile
    static constexpr int KSTR = KWP * 16, VSTR = VWP * 16;
    static constexpr int NKI = (TR * KWP + 63) / 64;            // load instructions per tile, K
    static constexpr int NVI = (TR * VWP + 63) / 64;            // and V
    static constexpr int KB = 0;                                // K rows
    static constexpr int VB = TR * KSTR;                        // V rows
    // V offset rows: the NB offsets, then at least one column of ones (the
    // offset product's column NB is then the row sums of P)
    static constexpr int VMS = (NB + 4) & ~3;
    static constexpr int KS = VB + TR * VSTR;                   // f32 [NB][32] K scales * scale * log2 e
    static constexpr int VD = KS + NB * kRowTile * 4;           // fp16 [NB][32] V steps
    static constexpr int VM = VD + NB * kRowTile * 2;           // fp16 [32][VMS] V offsets, then ones
    static constexpr int BYTES = VM + kRowTile * VMS * 2;       // per wave
    static_assert(NKI <= 32 && NVI <= 32, "load counts must fit vmcnt");
};

// The same for FP8 rows, where a head's codes are 32 * NB contiguous,
// 16-byte aligned bytes of the row and its NB fp16 scales lie in one 16-byte
// piece of the row's scale area: a row window is the 2 NB code pieces plus
// that piece (an odd count), for K and for V alike.  No V offsets.
template <int NB>
struct StreamWinF8 {
    static constexpr int KW = 2 * NB + 1;                       // K pieces per row window
    static constexpr int KWP = KW;
    static constexpr int VW = KW;
    static constexpr int VWP = VW;
    static constexpr int TR = kRowTile;
    static constexpr int KSTR = KWP * 16, VSTR = VWP * 16;
    static constexpr int NKI = (TR * KWP + 63) / 64;
    static constexpr int NVI = (TR * VWP + 63) / 64;
    static constexpr int KB = 0;
    static constexpr int VB = TR * KSTR;
    static constexpr int SC = 32 * NB;                          // scale piece within a row window
    static constexpr int VMS = 0;
    static constexpr int KS = VB + TR * VSTR;                   // f32 [NB][32] K scales * scale * log2 e
    static constexpr int VD = KS + NB * kRowTile * 4;           // fp16 [NB][32] V scales
    static constexpr int VM = VD + NB * kRowTile * 2;           // (no offsets)
    static constexpr int BYTES = VM;
    static_assert(NKI <= 32 && NVI <= 32, "load counts must fit vmcnt");
};

// The prime decode kernel (many query rows per KV head): a workgroup of
// kPrimeGroups waves, one 32-row query group each, shares each KV tile.  Its
// LDS for head_dim = 32 * NB: kPrimeRawBufs raw tile buffers (the stream
// kernel's row windows, K rows then V rows) and kPrimeConvBufs converted ones (K step x
// code as fp16 hi and lo parts, V codes as fp16 (q5_1: subnormals code x
// 2^-24; FP8: their values), V steps, V offset rows with ones).
constexpr int kPrimeGroups = 8;
constexpr int kPrimeRawBufs = 3;    // raw tile buffers: two tiles in flight while one is converted
constexpr int kPrimeConvBufs = 3;   // converted tiles: one in softmax and P V, one in scores, one being written
template <int NB, bool F8>
struct PrimeWin {
    using type = StreamWin<NB>;
};
template <int NB>
struct PrimeWin<NB, true> {
    using type = StreamWinF8<NB>;
};
template <int NB, bool F8 = false>
struct PrimeLayout {
    using WN = typename PrimeWin<NB, F8>::type;
    static constexpr int HD = NB * 32;
    static constexpr int RAW = kRowTile * (WN::KSTR + WN::VSTR);
    static constexpr int RK = 0, RV = kRowTile * WN::KSTR;
    // fp16 rows of a head, padded by 8 banks a row: K rows (read 16 bytes a
    // lane, 16 rows at once; with a pad of 4 banks the kernel counted 4 times
    // the bank-conflict cycles) and V rows (transposed 8-byte reads of 4 rows)
    static constexpr int ROWH = HD * 2 + 32;
    static constexpr int ROWV = HD * 2 + 32;
    static constexpr int VMS = (NB + 4) & ~3;                   // offsets (0 for FP8 rows), then ones
    static constexpr int KH = 0;                                // fp16 [32][HD] K products, high parts
    static constexpr int KL = KH + kRowTile * ROWH;             // fp16 [32][HD] K products, low parts
    static constexpr int VH = KL + kRowTile * ROWH;             // fp16 [32][HD] V codes * 2^-24
    static constexpr int VD = VH + kRowTile * ROWV;             // fp16 [NB][32] V steps
    static constexpr int VM = VD + NB * kRowTile * 2;           // fp16 [32][VMS] V offsets, then ones
    static constexpr int CONV = VM + kRowTile * VMS * 2;        // one converted buffer
    static constexpr int BYTES = kPrimeRawBufs * RAW + kPrimeConvBufs * CONV;
    static constexpr int NIT = WN::NKI + WN::NVI;               // load instructions per tile
    static_assert(RAW % 16 == 0 && CONV % 16 == 0 && ROWH % 16 == 0 && ROWV % 16 == 0, "16-byte alignment");
};
inline int prime_lds_bytes(int NB, bool f8 = false) {
    if (f8) return NB == 2 ? PrimeLayout<2, true>::BYTES : NB == 4 ? PrimeLayout<4, true>::BYTES : 0;
    return NB == 2 ? PrimeLayout<2>::BYTES : NB == 4 ? PrimeLayout<4>::BYTES : 0;
}

inline int stream_wave_bytes(int NB, bool f8 = false) {
    switch (NB) {
        case 2: return f8 ? StreamWinF8<2>::BYTES : StreamWin<2>::BYTES;
        case 4: return f8 ? StreamWinF8<4>::BYTES : StreamWin<4>::BYTES;
        case 8: return f8 ? StreamWinF8<8>::BYTES : StreamWin<8>::BYTES;
        default: return 0;
    }
}
// LDS bytes per wave of the dim-split stream kernel (two waves per head of
// head_dim / 2 dims each, both row tiles): the half-head window buffer and
// two slots of partial scores.
inline int stream_ds_wave_bytes(int head_dim, bool f8 = false) {
    return stream_wave_bytes(head_dim == 256 ? 4 : 2, f8) + 2 * 2 * 2 * 64 * 16;
}
inline int stream_rows_per_buffer(int) { return kRowTile; }
// Waves per SIMD the stream kernel is compiled for (its register budget is
// 512 / this): as many as its registers allow without spilling.  NB blocks of
// 32 dims per head, RTW row tiles of 16 per wave, QLO = fp32 queries (a low
// fp16 part is kept beside the high one).
constexpr int stream_waves_per_simd(int NB, int RTW, bool QLO) {
    return RTW > 1 ? 1 : NB >= 8 ? 2 : NB >= 4 ? (QLO ? 3 : 4) : 4;
}

// Waves per SIMD of the dim-split stream kernel, by the blocks of its half
// head: 3 for 128-dim heads (64-dim halves), 2 for 256-dim heads.
constexpr int stream_ds_waves_per_simd(int NB_half) { return NB_half <= 2 ? 3 : 2; }

enum DecodeKernel : int32_t { kPerHead = 0, kStream = 2, kPrime = 3 };

// Split-K decode plus the log-sum-exp combine.
struct DecodeParams {
    const void* q;              // [B, T, H, hd]
    int32_t f8;                 // 1: K and V as FP8 rows (codes, then scales); 0: q8_0 / q5_1
    int32_t dtype;
    int32_t B, T, H, Hkv, hd, hpk, window;
    int32_t Tg;                 // query rows per decode workgroup: the grid's y index
                                // runs over the groups of Tg rows (Tg * hpk <= 32)
    const uint8_t* k_planes;
    const uint8_t* v_planes;
    int64_t k_stride;
    int64_t v_stride;
    int32_t k_row;              // bytes per K token row
    int32_t v_row;
    const int32_t* len_d;
    const int32_t* base_d;
    int32_t chunk;              // rows per split (multiple of kSplitQuantum); chunks
                                // start at the first visible row rounded down to 32
    int32_t splits;             // split slots per session
    int32_t units;              // (session, chunk) pairs with rows, over all sessions
    int32_t kernel;             // DecodeKernel
    int32_t gh;                 // KV heads per workgroup (stream kernel)
    int32_t rs;                 // stream kernel: waves per KV head in a workgroup, each
                                // taking every rs-th tile of the chunk (1 or 2)
    int32_t rg;                 // stream kernel: waves per KV head in a workgroup, each
                                // taking 16 of the query rows (1 or 2)
    int32_t ds;                 // stream kernel: 2 = two waves per KV head, each taking half
                                // of its dims for all query rows (head_dim 256); else 1
    int32_t lds;                // dynamic LDS bytes of the decode workgroup
    float scale;
    float* part_ml;             // [B, splits, T, H, 2]  running max, running sum
    float* part_o;              // [B, splits, T, H, hd] unnormalised output
    const float* sinks;         // [H] or null
    float* out;                 // [B, T, H, hd]
    float* lse;                 // [B, T, H] or null
};

// Compute units of the current device (0 if it cannot be read).
int device_compute_units();

// The library's device scratch for kvq_decode_noalloc: a file-scope device
// array of kScratchBytes per device.  Fills *ptr with its address on the
// current device (looked up once per device, then cached).
constexpr size_t kScratchBytes = size_t(64) << 20;
int scratch_region(void** ptr, const char** err);

// Launchers: return 0 on success, nonzero with a message in *err otherwise.
int launch_append(const AppendParams& p, void* stream, const char** err);
int launch_set(const SetParams& p, void* stream, const char** err);
int launch_move(const MoveParams& p, void* stream, const char** err);
// ev[0..2] (hipEvent_t or null): recorded on the stream before the partials
// kernel, between it and the combine, and after the combine.
int launch_decode(const DecodeParams& p, void* stream, void* const ev[3], const char** err);
int launch_importance(const ImportanceParams& p, void* stream, const char** err);

}  // namespace kvq

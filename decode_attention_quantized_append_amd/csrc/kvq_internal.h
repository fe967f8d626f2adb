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
constexpr int kMaxRows = 32;                // R = T * H / Hkv query rows per KV head
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
    int32_t idx[kMaxSetPerLaunch];
    int32_t val[kMaxSetPerLaunch];
};

// One non-overlapping slab per listed session: physical rows
// [src_row, src_row + rows) -> [dst_row, dst_row + rows) of the K and V planes.
struct MoveParams {
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

// Split-K decode plus the log-sum-exp combine.
struct DecodeParams {
    const void* q;              // [B, T, H, hd]
    int32_t dtype;
    int32_t B, T, H, Hkv, hd, hpk, window;
    const uint8_t* k_planes;
    const uint8_t* v_planes;
    int64_t k_stride;
    int64_t v_stride;
    int32_t k_row;              // bytes per K token row
    int32_t v_row;
    const int32_t* len_d;
    const int32_t* base_d;
    int32_t chunk;              // rows per split (multiple of kSplitQuantum)
    int32_t splits;             // split slots per session
    float scale;
    float* part_ml;             // [B, splits, T, H, 2]  running max, running sum
    float* part_o;              // [B, splits, T, H, hd] unnormalised output
    const float* sinks;         // [H] or null
    float* out;                 // [B, T, H, hd]
    float* lse;                 // [B, T, H] or null
};

// Launchers: return 0 on success, nonzero with a message in *err otherwise.
int launch_append(const AppendParams& p, void* stream, const char** err);
int launch_set(const SetParams& p, void* stream, const char** err);
int launch_move(const MoveParams& p, void* stream, const char** err);
int launch_decode(const DecodeParams& p, void* stream, const char** err);

}  // namespace kvq

// kvq_host.cpp -- the C ABI of libkvq (include/kvq.h): argument validation,
// the host mirror of len/base, the ring planner, the split-K plan, and the
// enqueueing of kernels through the launcher interface (kvq_internal.h).
//
// Pages followed (docs.rs):
//  * memra-engine "Struct KvLayer": len is kept in lock-step with the device
//    counter len_d; base_d mirrors ring.base(); physical = row - base; the
//    live window is [max(0, len - window), len); the rebase arm is the only
//    writer of base_d and runs on the host; rewinds move len only.
//  * memra-engine "Struct Cache", rollback: full-attention KV is rolled back
//    by setting len, with no copy.
//  * memra-engine "Struct KvLayer", physical_rows: a logical range that is not
//    resident is an error (here KVQ_ERANGE), not a silent clamp.
//  * cortiq-engine "Struct LayerKvCache", export_wire / import_wire: geometry
//    is checked, not assumed, and a call refuses rather than half-applying.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

struct kvq_cache {
    kvq_config cfg;
    kvq_sizes sz;
    uint8_t* k;
    uint8_t* v;
    int32_t* counters;
    std::vector<int64_t> len;    // host mirror of len_d
    std::vector<int64_t> base;   // host mirror of base_d
    int32_t split_rows;
    int32_t decode_kernel;       // kvq_decode_kernel (KVQ_DECODE_AUTO: chosen per call)
    int32_t head_group;          // KV heads per workgroup (0: chosen per call)
    int32_t sub_tiles;           // stream kernel: waves per KV head (0: chosen per call)
    int32_t graph_mode;          // plan decodes for every session's largest span
    int32_t cus;                 // compute units of the device the handle was created on
    void* trace[3];              // events kvq_decode records around its kernels (or null)
    void* scratch;               // the library's device scratch on the handle's device
    float* imp;                  // importance moved along by rebases (kvq_set_importance), or null
};

namespace {

thread_local std::string g_err;

kvq_status fail(kvq_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kvq_status check_config(const kvq_config* c) {
    if (!c) return fail(KVQ_EINVAL, "config is NULL");
    const bool q8q5 = c->k_fmt == KVQ_FMT_Q8_0 && c->v_fmt == KVQ_FMT_Q5_1;
    const bool f8 = c->k_fmt == KVQ_FMT_E4M3 && c->v_fmt == KVQ_FMT_E4M3;
    if (!q8q5 && !f8)
        return fail(KVQ_EUNSUPPORTED, "the formats must be K = q8_0 with V = q5_1, or K = V = e4m3");
    if (c->n_seqs < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1)
        return fail(KVQ_EINVAL, "n_seqs, n_q_heads and n_kv_heads must be >= 1");
    if (c->n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
    if (c->head_dim < 32 || c->head_dim % 32 != 0)
        return fail(KVQ_EINVAL, "head_dim must be a positive multiple of 32");
    if (c->head_dim > kvq::kMaxHeadDim)
        return fail(KVQ_EUNSUPPORTED, "head_dim above 256 is not implemented");
    if (c->capacity < 1) return fail(KVQ_EINVAL, "capacity must be >= 1");
    if (c->window < 0 || c->ring_step < 0) return fail(KVQ_EINVAL, "window and ring_step must be >= 0");
    if (c->ring_step > 0 && (c->window <= 0 || (int64_t)c->window + c->ring_step > c->capacity))
        return fail(KVQ_EINVAL, "a ring needs window > 0 and window + ring_step <= capacity");
    // FP8 rows are decoded by the stream kernel only: 64-, 128- or 256-dim
    // heads, and a ring base that stays on a 32-row boundary
    if (f8 && c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
        return fail(KVQ_EUNSUPPORTED, "e4m3 K/V need head_dim 64, 128 or 256");
    if (f8 && c->ring_step % 32 != 0)
        return fail(KVQ_EUNSUPPORTED, "e4m3 K/V need a ring_step that is a multiple of 32");
    int64_t row = (int64_t)c->n_kv_heads * c->head_dim / 32 * 34;
    if (row * (int64_t)c->capacity > (int64_t)INT32_MAX * 4)
        return fail(KVQ_EUNSUPPORTED, "a session plane above 8 GiB is not supported");
    if ((int64_t)c->n_kv_heads * c->head_dim > (1 << 20))
        return fail(KVQ_EUNSUPPORTED, "row too wide");
    return KVQ_OK;
}

void sizes_of(const kvq_config* c, kvq_sizes* s) {
    int64_t blocks = (int64_t)c->n_kv_heads * c->head_dim / 32;
    s->k_row_bytes = (size_t)(blocks * 34);
    s->v_row_bytes = (size_t)(blocks * (c->v_fmt == KVQ_FMT_E4M3 ? 34 : 24));
    s->k_session_stride = (size_t)round_up((int64_t)s->k_row_bytes * c->capacity, 256);
    s->v_session_stride = (size_t)round_up((int64_t)s->v_row_bytes * c->capacity, 256);
    // + a 256-byte tail on each: the decode reads each KV head's q8_0 blocks
    // from the 16-byte boundary at or below them, up to 12 bytes past the last
    // head's blocks of a row, and an FP8 row's scales as the 16-byte piece that
    // holds them, up to 12 bytes past the row
    s->k_planes_bytes = s->k_session_stride * (size_t)c->n_seqs + 256;
    s->v_planes_bytes = s->v_session_stride * (size_t)c->n_seqs + 256;
    s->counters_bytes = (size_t)round_up(((int64_t)2 * c->n_seqs + 4) * 4, 256);
}

bool is_f8(const kvq_config& c) { return c.k_fmt == KVQ_FMT_E4M3; }

int32_t* len_d(const kvq_cache* h) { return h->counters; }
int32_t* base_d(const kvq_cache* h) { return h->counters + h->cfg.n_seqs; }
int32_t* scratch_d(const kvq_cache* h) { return h->counters + 2 * h->cfg.n_seqs; }

// Write dst[idx[i]] = val[i], in launches of up to kMaxSetPerLaunch entries.
kvq_status enqueue_sets(int32_t* dst, const std::vector<int32_t>& idx,
                        const std::vector<int32_t>& val, void* stream, int add = 0, int B = 0, int window = 0) {
    for (size_t i0 = 0; i0 < idx.size(); i0 += kvq::kMaxSetPerLaunch) {
        kvq::SetParams p{};
        p.dst = dst;
        p.add = add;
        p.B = B;
        p.window = window;
        p.n = (int32_t)std::min<size_t>(kvq::kMaxSetPerLaunch, idx.size() - i0);
        for (int i = 0; i < p.n; ++i) {
            p.idx[i] = idx[i0 + i];
            p.val[i] = val[i0 + i];
        }
        const char* err = nullptr;
        if (kvq::launch_set(p, stream, &err)) return fail(KVQ_EDEVICE, err ? err : "set kernel launch failed");
    }
    return KVQ_OK;
}

// Rows of the union of the T query rows' visible ranges: [lo, len).
int64_t visible_lo(const kvq_cache* h, int64_t len, int32_t T) {
    if (h->cfg.window <= 0) return 0;
    return std::max<int64_t>(0, len - T + 1 - h->cfg.window);
}

struct Plan {
    int32_t kernel;    // kvq::DecodeKernel
    int32_t chunk;
    int32_t splits;
    int32_t units;     // (session, chunk) pairs with rows
    int32_t gh;        // KV heads per workgroup (stream kernel)
    int32_t rs;        // stream kernel: row streams (waves per KV head)
    int32_t rg;        // stream kernel: row groups of 16 query rows (waves per KV head)
    int32_t ds;        // stream kernel: 2 = two waves per KV head, each half of its dims
    int32_t lds;       // dynamic LDS bytes
    int32_t rows;      // rows per buffer (chunks are a multiple)
    size_t ml_bytes;
    size_t o_bytes;
};

// Is the per-wave stream kernel built for gh heads (one wave each) at this shape?
bool stream_ok(const kvq_config& c, int R, int gh) {
    const int NB = c.head_dim / 32;
    if (NB != 2 && NB != 4 && NB != 8) return false;
    if (gh < 1 || c.n_kv_heads % gh != 0) return false;
    const int RT = (R + 15) / 16;
    if (gh > (RT == 1 ? 8 : 4)) return false;
    return gh * kvq::stream_wave_bytes(NB, is_f8(c)) <= kvq::kLdsBytes;
}

// Can the stream kernel run two waves per KV head (two row streams) in one
// workgroup: one row tile per wave, and twice the waves and LDS still fit a CU?
bool stream_rs2_ok(const kvq_config& c, int R, int gh) {
    const int NB = c.head_dim / 32;
    if (R > 16) return false;
    const int waves = 4 * kvq::stream_waves_per_simd(NB, 1, false);
    return 2 * gh * kvq::stream_wave_bytes(NB, is_f8(c)) <= kvq::kLdsBytes && 2 * gh <= waves;
}

// Can the stream kernel give each of the two 16-row groups of R > 16 query
// rows its own wave (one row tile each, both loading the same tiles in step),
// with twice the waves and LDS still fitting a CU?
bool stream_rg2_ok(const kvq_config& c, int R, int gh, bool f32_queries) {
    const int NB = c.head_dim / 32;
    if (R <= 16) return false;
    const int waves = 4 * kvq::stream_waves_per_simd(NB, 1, f32_queries);
    return 2 * gh * kvq::stream_wave_bytes(NB, is_f8(c)) <= kvq::kLdsBytes && 2 * gh <= waves;
}

// Can the stream kernel give each 128- or 256-dim KV head two waves of half
// its dims (both row tiles of 17..32 query rows each), with 2 * gh waves and
// their LDS fitting a CU?
bool stream_ds_ok(const kvq_config& c, int R, int gh) {
    if ((c.head_dim != 128 && c.head_dim != 256) || R <= 16 || R > 32) return false;
    if (gh < 1 || c.n_kv_heads % gh != 0) return false;
    if (2 * gh > 8 || 2 * gh > 4 * kvq::stream_ds_waves_per_simd(c.head_dim / 64)) return false;
    return gh * 2 * kvq::stream_ds_wave_bytes(c.head_dim, is_f8(c)) <= kvq::kLdsBytes;
}

// Can dim halves also run two row streams per head (four waves per head,
// alternate tiles of a twice-as-long chunk, half as many partials)?  At
// head_dim 256 only: with 128-dim heads (three waves per SIMD) the prime
// chunk ran 12 % slower with them.
bool stream_ds_rs2_ok(const kvq_config& c, int R, int gh) {
    if (c.head_dim != 256 || !stream_ds_ok(c, R, gh)) return false;
    const int waves = 4 * gh;
    return waves <= 8 && waves <= 4 * kvq::stream_ds_waves_per_simd(c.head_dim / 64) &&
           gh * 4 * kvq::stream_ds_wave_bytes(c.head_dim, is_f8(c)) <= kvq::kLdsBytes;
}

// Is every session's first visible row, rounded down to 32, still resident?
bool aligned_start_resident(const kvq_cache* h, int32_t T) {
    for (int b = 0; b < h->cfg.n_seqs; ++b)
        if ((visible_lo(h, h->len[b], T) & ~int64_t(31)) < h->base[b]) return false;
    return true;
}

// Rows each session's chunks cover: from the first visible row rounded down
// to 32 up to len.  In graph mode, the most they can cover while the session
// stays within its plane: the window plus T - 1 rows plus 31 of alignment,
// or the whole plane; a decode captured in a graph then stays valid while the
// lengths grow.
int64_t span_of(const kvq_cache* h, int b, int32_t T) {
    if (h->graph_mode) {
        const int64_t cap = h->cfg.capacity;
        return h->cfg.window > 0 ? std::min<int64_t>(cap + 31, h->cfg.window + T - 1 + 31) : cap;
    }
    return std::max<int64_t>(0, h->len[b] - (visible_lo(h, h->len[b], T) & ~int64_t(31)));
}

// Groups of query rows from which the planner takes the prime kernel.
constexpr int64_t kPrimeMinGroups = 4;

// Is the prime kernel built for this shape: head_dim 64 or 128 and more than
// one group of query rows.
bool prime_ok(const kvq_config& c, int R, int32_t T) {
    const int NB = c.head_dim / 32;
    const int hpk = c.n_q_heads / c.n_kv_heads;
    return (NB == 2 || NB == 4) && T > R / hpk;
}

// Chooses the decode kernel and its tiling.  Returns false when a kernel or
// tiling set with kvq_set_decode_tiling does not fit the shape.
bool choose_kernel(const kvq_cache* h, int R, int32_t T, bool f32_queries, Plan* p) {
    const kvq_config& c = h->cfg;
    const int NB = c.head_dim / 32;
    p->kernel = kvq::kPerHead;
    p->gh = 0;
    p->lds = 0;
    p->rows = 256;
    int want = h->decode_kernel;
    if (want == KVQ_DECODE_AUTO) want = (NB == 2 || NB == 4 || NB == 8) ? KVQ_DECODE_STREAM : KVQ_DECODE_PER_HEAD;
    if (want == KVQ_DECODE_PER_HEAD) return !is_f8(c);   // the per-head kernel reads q8_0 / q5_1 only
    // Many query rows per KV head (a prompt chunk): the prime kernel, whose
    // eight waves share each converted KV tile, from kPrimeMinGroups groups
    // of query rows on (fewer leave most of its waves idle)
    const int hpk = c.n_q_heads / c.n_kv_heads;
    const bool prime = want == KVQ_DECODE_PRIME ||
                       (h->decode_kernel == KVQ_DECODE_AUTO && prime_ok(c, R, T) &&
                        ceil_div(T, R / hpk) >= kPrimeMinGroups);
    if (prime) {
        if (!prime_ok(c, R, T)) return false;
        if (!aligned_start_resident(h, T)) return !is_f8(c);   // the per-head kernel, as for the stream kernel
        p->kernel = kvq::kPrime;
        p->gh = 1;
        p->rs = p->rg = p->ds = 1;
        p->lds = kvq::prime_lds_bytes(NB, is_f8(c));
        p->rows = kvq::kRowTile;
        return true;
    }
    // The stream kernel starts a session's first tile at the first visible
    // row rounded down to 32 and reads it whole, so that row must still be
    // resident (at or above base); else one KV head per workgroup, whose
    // loads clamp rows to the visible range.
    if (!aligned_start_resident(h, T)) return !is_f8(c);   // FP8 rings rebase in 32-row steps: never
    // 128- and 256-dim heads with 17..32 query rows: two waves per head,
    // each half of the dims (no unpacking done twice), in independent
    // workgroups of one head unless a head group is set.  FP8 rows: two
    // heads per workgroup, whose waves then read the 16-byte pieces of a
    // row's scale area together (with one head per workgroup those pieces
    // were fetched from HBM about twice over: the FP8 verify kernel read
    // 1.125 times its K and V bytes, 1.002 with two heads, and ran 7 %
    // faster); q8_0 / q5_1 rows hold their scales in their blocks, and two
    // heads per workgroup made the verify kernel 5 % slower.
    const bool ds = h->sub_tiles == 3 || (h->sub_tiles == 0 && stream_ds_ok(c, R, 1));
    int gh = h->head_group;
    if (gh == 0 && ds) gh = (is_f8(c) && c.n_kv_heads % 2 == 0 && stream_ds_ok(c, R, 2)) ? 2 : 1;
    if (gh == 0)
        // the largest head group: the waves of one workgroup share the
        // cache lines at the edges of adjacent head slices
        for (int k = std::min(c.n_kv_heads, 8); k >= 1 && gh == 0; --k)
            if (stream_ok(c, R, k)) gh = k;
    if (!stream_ok(c, R, gh)) return h->decode_kernel == KVQ_DECODE_AUTO;
    p->kernel = kvq::kStream;
    p->gh = gh;
    p->ds = 1;
    p->rs = 1;
    p->rg = 1;
    p->lds = gh * kvq::stream_wave_bytes(NB, is_f8(c));
    p->rows = kvq::stream_rows_per_buffer(NB);
    if (ds) {
        // two waves per KV head, each half of a 128- or 256-dim head's
        // dims for all 17..32 query rows; row streams chosen with the chunk
        if (!stream_ds_ok(c, R, gh)) return false;
        p->ds = 2;
        p->rs = 0;
        p->lds = gh * 2 * kvq::stream_ds_wave_bytes(c.head_dim, is_f8(c));
        return true;
    }
    // sub_tiles = waves per KV head: row streams for R <= 16 query rows,
    // row groups above
    p->rs = R <= 16 ? h->sub_tiles : 1;         // 0: chosen with the chunk
    p->rg = R > 16 ? (h->sub_tiles == 1 ? 1 : stream_rg2_ok(c, R, gh, f32_queries) ? 2 : 0) : 1;
    if (p->rg == 0) {
        if (h->sub_tiles == 2) return false;
        p->rg = 1;
    }
    if (p->rs == 2 && !stream_rs2_ok(c, R, gh)) return false;
    p->lds = gh * std::max(1, p->rs) * p->rg * kvq::stream_wave_bytes(NB, is_f8(c));
    p->rows = kvq::stream_rows_per_buffer(NB);
    return true;
}

Plan make_plan(const kvq_cache* h, int32_t T, bool f32_queries, bool* fits = nullptr) {
    const kvq_config& c = h->cfg;
    // the decode kernels take the T query rows in groups of at most 32 / hpk
    // rows; R is the query rows per KV head of one group
    const int hpk = c.n_q_heads / c.n_kv_heads;
    const int R = std::min<int>(T, kvq::kMaxRows / hpk) * hpk;
    const int64_t groups = ceil_div(T, R / hpk);   // workgroups per (session, chunk, head group)
    int64_t total = 0, maxvis = 1;
    for (int b = 0; b < c.n_seqs; ++b) {
        const int64_t vis = span_of(h, b, T);
        total += vis;
        maxvis = std::max(maxvis, vis);
    }
    Plan p{};
    const bool ok = choose_kernel(h, R, T, f32_queries, &p);
    if (fits) *fits = ok;
    int64_t chunk = h->split_rows;
    if (p.kernel == kvq::kPrime) {
        // one workgroup per CU (eight waves of up to 256 registers): about
        // as many workgroups as CUs, each a whole number of tiles
        const int64_t yblocks = ceil_div(groups, kvq::kPrimeGroups);
        const int64_t slots = std::max<int64_t>(1, h->cus);
        if (chunk <= 0) {
            chunk = round_up(std::max<int64_t>(1, ceil_div(total * c.n_kv_heads * yblocks, slots)), p.rows);
            for (;;) {
                int64_t wgs = 0;
                for (int b = 0; b < c.n_seqs; ++b) wgs += ceil_div(span_of(h, b, T), chunk) * c.n_kv_heads * yblocks;
                if (wgs <= slots) break;
                chunk += p.rows;
            }
        }
        chunk = round_up(chunk, p.rows);
    } else if (p.kernel != kvq::kPerHead) {
        const int64_t ngrp = c.n_kv_heads / p.gh;
        const int RT = (R + 15) / 16;
        // one round of workgroups: as many as fit on the device's CUs at once
        // (bound by LDS and by the waves the register file holds), each a
        // whole number of buffers
        auto one_round = [&](int rs) {
            const bool ds = p.ds == 2;
            const int64_t waves_per_wg = p.gh * rs * p.rg * p.ds;
            const int rtw = p.rg == 2 ? 1 : RT;   // row tiles per wave
            const int64_t waves_per_cu = ds ? 4 * kvq::stream_ds_waves_per_simd(c.head_dim / 64)
                                            : 4 * kvq::stream_waves_per_simd(c.head_dim / 32, rtw, f32_queries);
            const int64_t lds = ds ? p.gh * rs * 2 * kvq::stream_ds_wave_bytes(c.head_dim, is_f8(c))
                                   : p.gh * rs * p.rg * kvq::stream_wave_bytes(c.head_dim / 32, is_f8(c));
            const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kvq::kLdsBytes / lds,
                                                                           waves_per_cu / waves_per_wg));
            const int64_t slots = (int64_t)h->cus * per_cu;
            int64_t ch = round_up(std::max<int64_t>(1, ceil_div(total * ngrp * groups, slots)), p.rows);
            for (;;) {
                int64_t wgs = 0;
                for (int b = 0; b < c.n_seqs; ++b) wgs += ceil_div(span_of(h, b, T), ch) * ngrp * groups;
                if (wgs <= slots) break;
                ch += p.rows;
            }
            return ch;
        };
        {
            // two row streams per head when each still gets a few tiles of
            // its chunk: the waves of a CU then advance together, and there
            // are half as many partials to combine
            const bool rs2 = p.ds == 2 ? stream_ds_rs2_ok(c, R, p.gh) : stream_rs2_ok(c, R, p.gh) && !f32_queries;
            if (p.rs == 0) p.rs = (rs2 && (chunk > 0 ? chunk : one_round(2)) >= 4 * 32) ? 2 : 1;
            if (p.rs == 2 && !rs2 && fits) *fits = false;
            p.lds = p.ds == 2 ? p.gh * p.rs * 2 * kvq::stream_ds_wave_bytes(c.head_dim, is_f8(c))
                              : p.gh * p.rs * p.rg * kvq::stream_wave_bytes(c.head_dim / 32, is_f8(c));
        }
        if (chunk <= 0) {
            chunk = one_round(p.rs);
            // a chunk of one tile leaves each wave a single load-then-compute
            // pass: with half the heads per workgroup, as many workgroups take
            // two tiles each (the second in flight while the first is
            // computed) and write half as many partials
            if (h->head_group == 0 && p.rs == 1 && p.rg == 1 && p.ds == 1 &&
                p.gh % 2 == 0 && chunk <= p.rows) {
                p.gh /= 2;
                p.lds = p.gh * kvq::stream_wave_bytes(c.head_dim / 32, is_f8(c));
                chunk = 2 * p.rows;
            }
        }
        chunk = round_up(chunk, p.rows);
    } else if (chunk <= 0) {
        // About 2048 workgroups of (session, chunk, KV head), i.e. several per
        // CU so that the last round is a small fraction of the work, but at
        // least 64 rows per query row so that the partials (R x (hd + 2)
        // floats written and read back per chunk) stay within a few percent
        // of the chunk's K/V bytes (R x (hd + 2) x 8 / (64 R x 1.8125 hd)).
        chunk = round_up(ceil_div(std::max<int64_t>(total, 1) * c.n_kv_heads * groups, 2048), kvq::kSplitQuantum);
        chunk = std::min<int64_t>(std::max<int64_t>(chunk, std::max<int64_t>(256, 64 * (int64_t)R)), 1 << 16);
        chunk = round_up(chunk, 256);   // whole rounds of 4 waves x 32 rows x 2 prefetched tiles
    }
    // at most kMaxSplits chunks per session
    chunk = std::max<int64_t>(chunk, round_up(ceil_div(maxvis, kvq::kMaxSplits), p.rows));
    p.chunk = (int32_t)chunk;
    p.splits = (int32_t)std::max<int64_t>(1, ceil_div(maxvis, chunk));
    p.units = 0;
    for (int b = 0; b < c.n_seqs; ++b) p.units += (int32_t)ceil_div(span_of(h, b, T), chunk);
    int64_t entries = (int64_t)c.n_seqs * p.splits * T * c.n_q_heads;
    p.ml_bytes = (size_t)round_up(entries * 2 * 4, 256);
    p.o_bytes = (size_t)round_up(entries * c.head_dim * 4, 256);
    return p;
}

// kvq_decode and kvq_decode_noalloc: the partials go to the caller's
// workspace ws, or (ws == nullptr with use_scratch) to the library's scratch.
kvq_status decode_impl(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T, const float* sinks, float scale,
                       float* out, float* lse, void* ws, size_t ws_bytes, kvq_stream stream, bool use_scratch) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (!q || !out) return fail(KVQ_EINVAL, "q or out is NULL");
    if (dtype != KVQ_F32 && dtype != KVQ_BF16) return fail(KVQ_EINVAL, "dtype must be F32 or BF16");
    if (!std::isfinite(scale)) return fail(KVQ_EINVAL, "scale must be finite");
    const kvq_config& c = h->cfg;
    const int hpk = c.n_q_heads / c.n_kv_heads;
    if (T < 1) return fail(KVQ_EINVAL, "T must be >= 1");
    if (hpk > kvq::kMaxRows) return fail(KVQ_EINVAL, "need n_q_heads / n_kv_heads <= 32");
    for (int b = 0; b < c.n_seqs; ++b) {
        if (h->len[b] < T)
            return fail(KVQ_EINVAL, "session " + std::to_string(b) + " holds fewer than T rows");
        if (visible_lo(h, h->len[b], T) < h->base[b])
            return fail(KVQ_ERANGE, "session " + std::to_string(b) + ": visible rows were rebased away");
    }
    bool fits = true;
    Plan p = make_plan(h, T, dtype == KVQ_F32, &fits);
    if (!fits) return fail(KVQ_EINVAL, "the decode tiling set with kvq_set_decode_tiling does not fit this shape");
    if (use_scratch) {
        if (p.ml_bytes + p.o_bytes > kvq::kScratchBytes)
            return fail(KVQ_ECAPACITY, "the decode partials of this call need " +
                                           std::to_string(p.ml_bytes + p.o_bytes) +
                                           " bytes; the library's scratch holds " +
                                           std::to_string(kvq::kScratchBytes) + " (use kvq_decode with a workspace)");
        ws = h->scratch;
        ws_bytes = kvq::kScratchBytes;
    }
    if (!ws || ws_bytes < p.ml_bytes + p.o_bytes) return fail(KVQ_EINVAL, "workspace missing or too small");
    if (!aligned(ws, 256)) return fail(KVQ_EINVAL, "workspace must be 256-byte aligned");
    kvq::DecodeParams dp{};
    dp.q = q;
    dp.f8 = is_f8(c);
    dp.dtype = dtype;
    dp.B = c.n_seqs;
    dp.T = T;
    dp.H = c.n_q_heads;
    dp.Hkv = c.n_kv_heads;
    dp.hd = c.head_dim;
    dp.hpk = hpk;
    dp.window = c.window;
    dp.k_planes = h->k;
    dp.v_planes = h->v;
    dp.k_stride = (int64_t)h->sz.k_session_stride;
    dp.v_stride = (int64_t)h->sz.v_session_stride;
    dp.k_row = (int32_t)h->sz.k_row_bytes;
    dp.v_row = (int32_t)h->sz.v_row_bytes;
    dp.len_d = len_d(h);
    dp.base_d = base_d(h);
    dp.chunk = p.chunk;
    dp.splits = p.splits;
    dp.units = p.units;
    dp.kernel = p.kernel;
    dp.gh = p.gh;
    dp.rs = p.rs;
    dp.rg = p.rg;
    dp.ds = p.kernel == kvq::kStream ? p.ds : 1;
    dp.lds = p.lds;
    dp.scale = scale;
    dp.part_ml = static_cast<float*>(ws);
    dp.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.ml_bytes);
    dp.sinks = sinks;
    dp.out = out;
    dp.lse = lse;
    // workgroups take groups of at most 32 / hpk query rows; the combine
    // folds all T rows
    dp.Tg = std::min(T, kvq::kMaxRows / hpk);
    const char* err = nullptr;
    if (kvq::launch_decode(dp, stream, h->trace, &err)) return fail(KVQ_EDEVICE, err ? err : "decode launch failed");
    return KVQ_OK;
}

}  // namespace

extern "C" {

const char* kvq_last_error(void) { return g_err.c_str(); }

kvq_status kvq_ring_rows(int32_t window, int32_t max_chunk, int32_t ring_step, int32_t* rows) {
    if (!rows) return fail(KVQ_EINVAL, "rows is NULL");
    if (window < 1 || max_chunk < 1 || ring_step < 1)
        return fail(KVQ_EINVAL, "window, max_chunk and ring_step must be >= 1");
    // An append of n rows at length L rebases to the smallest base b' (a
    // multiple of ring_step) with L + n - b' <= capacity, so b' < L + n -
    // capacity + ring_step; its decode starts at (L + 1 - window) & ~31,
    // which is >= b' for every L and n <= max_chunk when capacity >= window +
    // max_chunk + ring_step - 2 (b' and the start both multiples of 32), or 31
    // rows more when ring_step is not a multiple of 32.
    int64_t r = (int64_t)window + max_chunk + ring_step - 2 + (ring_step % 32 == 0 ? 0 : 31);
    r = std::max<int64_t>(r, (int64_t)window + ring_step);
    if (r > INT32_MAX) return fail(KVQ_EINVAL, "ring rows overflow int32");
    *rows = (int32_t)r;
    return KVQ_OK;
}

kvq_status kvq_required_bytes(const kvq_config* cfg, kvq_sizes* out) {
    kvq_status s = check_config(cfg);
    if (s != KVQ_OK) return s;
    if (!out) return fail(KVQ_EINVAL, "out is NULL");
    sizes_of(cfg, out);
    return KVQ_OK;
}

kvq_status kvq_create(const kvq_config* cfg, void* k_planes, void* v_planes,
                      int32_t* counters, kvq_stream stream, kvq_cache** out) {
    kvq_status s = check_config(cfg);
    if (s != KVQ_OK) return s;
    if (!out) return fail(KVQ_EINVAL, "out is NULL");
    if (!k_planes || !v_planes || !counters) return fail(KVQ_EINVAL, "a device buffer is NULL");
    if (!aligned(k_planes, 256) || !aligned(v_planes, 256) || !aligned(counters, 256))
        return fail(KVQ_EINVAL, "planes and counters must be 256-byte aligned");
    kvq_cache* h = new kvq_cache();
    h->cfg = *cfg;
    sizes_of(cfg, &h->sz);
    h->k = static_cast<uint8_t*>(k_planes);
    h->v = static_cast<uint8_t*>(v_planes);
    h->counters = counters;
    h->len.assign(cfg->n_seqs, 0);
    h->base.assign(cfg->n_seqs, 0);
    h->split_rows = 0;
    h->decode_kernel = KVQ_DECODE_AUTO;
    h->head_group = 0;
    h->sub_tiles = 0;
    h->graph_mode = 0;
    h->trace[0] = h->trace[1] = h->trace[2] = nullptr;
    // the split plan sizes one round of workgroups to the device's CUs
    h->cus = kvq::device_compute_units();
    if (h->cus <= 0) {
        delete h;
        return fail(KVQ_EDEVICE, "cannot read the compute-unit count of the current device");
    }
    // the device address of the library's scratch (kvq_decode_noalloc),
    // looked up once per device
    {
        const char* err = nullptr;
        if (kvq::scratch_region(&h->scratch, &err)) {
            delete h;
            return fail(KVQ_EDEVICE, std::string("cannot locate the library's device scratch: ") +
                                         (err ? err : "unknown error"));
        }
    }
    int n = 2 * cfg->n_seqs + 4;
    std::vector<int32_t> idx(n), val(n, 0);
    for (int i = 0; i < n; ++i) idx[i] = i;
    s = enqueue_sets(counters, idx, val, stream);
    if (s != KVQ_OK) {
        delete h;
        return s;
    }
    *out = h;
    return KVQ_OK;
}

kvq_status kvq_append(kvq_cache* h, const void* k_new, const void* v_new, kvq_dtype dtype,
                      int32_t T, const int32_t* n_new, kvq_stream stream) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (!k_new || !v_new) return fail(KVQ_EINVAL, "k_new or v_new is NULL");
    if (dtype != KVQ_F32 && dtype != KVQ_BF16) return fail(KVQ_EINVAL, "dtype must be F32 or BF16");
    if (T < 1) return fail(KVQ_EINVAL, "T must be >= 1");
    const kvq_config& c = h->cfg;
    const int B = c.n_seqs;
    std::vector<int64_t> cnt(B, T), nbase(h->base);
    if (n_new)
        for (int b = 0; b < B; ++b) {
            if (n_new[b] < 0 || n_new[b] > T) return fail(KVQ_EINVAL, "n_new[b] must lie in [0, T]");
            cnt[b] = n_new[b];
        }
    // Plan every session before touching anything.
    for (int b = 0; b < B; ++b) {
        if (cnt[b] == 0) continue;
        int64_t L = h->len[b];
        if (L + cnt[b] > INT32_MAX) return fail(KVQ_EINVAL, "length would overflow int32");
        if (c.ring_step == 0) {
            if (L + cnt[b] > c.capacity)
                return fail(KVQ_ECAPACITY, "session " + std::to_string(b) + ": append past capacity");
            continue;
        }
        int64_t nb = h->base[b];
        while (L + cnt[b] - nb > c.capacity) nb += c.ring_step;
        if (nb != h->base[b] && std::max<int64_t>(0, L + 1 - c.window) < nb)
            return fail(KVQ_ERANGE, "session " + std::to_string(b) +
                                        ": rebase would drop rows the first new row still sees");
        nbase[b] = nb;
    }
    // Rebase: move the surviving rows down in non-overlapping slabs, then base_d.
    std::vector<int32_t> set_idx, set_val;
    int64_t max_slabs = 0;
    for (int b = 0; b < B; ++b)
        if (nbase[b] != h->base[b]) {
            int64_t shift = nbase[b] - h->base[b];
            int64_t keep = h->len[b] - nbase[b];
            max_slabs = std::max(max_slabs, ceil_div(std::max<int64_t>(keep, 0), shift));
            set_idx.push_back(B + b);
            set_val.push_back((int32_t)nbase[b]);
        }
    for (int64_t slab = 0; slab < max_slabs; ++slab) {
        kvq::MoveParams mp{};
        mp.imp = h->imp;
        mp.capacity = c.capacity;
        mp.k_planes = h->k;
        mp.v_planes = h->v;
        mp.k_stride = (int64_t)h->sz.k_session_stride;
        mp.v_stride = (int64_t)h->sz.v_session_stride;
        mp.k_row = (int32_t)h->sz.k_row_bytes;
        mp.v_row = (int32_t)h->sz.v_row_bytes;
        mp.n = 0;
        auto flush = [&]() -> kvq_status {
            if (mp.n == 0) return KVQ_OK;
            const char* err = nullptr;
            if (kvq::launch_move(mp, stream, &err)) return fail(KVQ_EDEVICE, err ? err : "move kernel launch failed");
            mp.n = 0;
            return KVQ_OK;
        };
        for (int b = 0; b < B; ++b) {
            if (nbase[b] == h->base[b]) continue;
            int64_t shift = nbase[b] - h->base[b];
            int64_t keep = h->len[b] - nbase[b];
            int64_t k0 = slab * shift;
            if (k0 >= keep) continue;
            mp.sess[mp.n] = b;
            mp.src_row[mp.n] = (int32_t)(shift + k0);
            mp.dst_row[mp.n] = (int32_t)k0;
            mp.rows[mp.n] = (int32_t)std::min(shift, keep - k0);
            if (++mp.n == kvq::kMaxSessionsPerLaunch) {
                kvq_status s = flush();
                if (s != KVQ_OK) return s;
            }
        }
        kvq_status s = flush();
        if (s != KVQ_OK) return s;
    }
    if (h->imp) {
        // the registered importance: the positions the survivors left are cleared
        kvq::MoveParams zp{};
        zp.imp = h->imp;
        zp.capacity = c.capacity;
        zp.zero = 1;
        for (int b = 0; b < B; ++b) {
            if (nbase[b] == h->base[b]) continue;
            const int64_t keep = std::max<int64_t>(0, h->len[b] - nbase[b]);
            zp.sess[zp.n] = b;
            zp.dst_row[zp.n] = (int32_t)keep;
            zp.rows[zp.n] = (int32_t)(c.capacity - keep);
            if (++zp.n == kvq::kMaxSessionsPerLaunch || b == B - 1) {
                const char* err = nullptr;
                if (kvq::launch_move(zp, stream, &err)) return fail(KVQ_EDEVICE, err ? err : "move kernel launch failed");
                zp.n = 0;
            }
        }
        if (zp.n > 0) {
            const char* err = nullptr;
            if (kvq::launch_move(zp, stream, &err)) return fail(KVQ_EDEVICE, err ? err : "move kernel launch failed");
        }
    }
    if (!set_idx.empty()) {
        kvq_status s = enqueue_sets(h->counters, set_idx, set_val, stream);
        if (s != KVQ_OK) return s;
    }
    // Quantize-and-append, sessions in launches of up to kMaxSessionsPerLaunch.
    for (int b0 = 0; b0 < B; b0 += kvq::kMaxSessionsPerLaunch) {
        kvq::AppendParams ap{};
        ap.k_new = k_new;
        ap.v_new = v_new;
        ap.k_planes = h->k;
        ap.v_planes = h->v;
        ap.k_stride = (int64_t)h->sz.k_session_stride;
        ap.v_stride = (int64_t)h->sz.v_session_stride;
        ap.len_d = len_d(h);
        ap.base_d = base_d(h);
        ap.done = scratch_d(h);
        ap.overflow = scratch_d(h) + 1;
        ap.f8 = is_f8(c);
        ap.dtype = dtype;
        ap.B = B;
        ap.T = T;
        ap.Hkv = c.n_kv_heads;
        ap.hd = c.head_dim;
        ap.capacity = c.capacity;
        ap.b0 = b0;
        ap.nsess = std::min(kvq::kMaxSessionsPerLaunch, B - b0);
        int64_t any = 0;
        for (int i = 0; i < ap.nsess; ++i) {
            ap.n_new[i] = (int32_t)cnt[b0 + i];
            any += cnt[b0 + i];
        }
        if (!any) continue;
        const char* err = nullptr;
        if (kvq::launch_append(ap, stream, &err)) return fail(KVQ_EDEVICE, err ? err : "append kernel launch failed");
    }
    for (int b = 0; b < B; ++b) {
        h->base[b] = nbase[b];
        h->len[b] += cnt[b];
    }
    return KVQ_OK;
}

kvq_status kvq_decode_workspace_bytes(const kvq_cache* h, int32_t T, size_t* bytes) {
    if (!h || !bytes) return fail(KVQ_EINVAL, "NULL argument");
    if (T < 1) return fail(KVQ_EINVAL, "T must be >= 1");
    if (h->cfg.n_q_heads / h->cfg.n_kv_heads > kvq::kMaxRows)
        return fail(KVQ_EINVAL, "need n_q_heads / n_kv_heads <= 32");
    // the larger of the plans for fp32 and bf16 queries
    const Plan p32 = make_plan(h, T, true), p16 = make_plan(h, T, false);
    *bytes = std::max(p32.ml_bytes + p32.o_bytes, p16.ml_bytes + p16.o_bytes);
    return KVQ_OK;
}

kvq_status kvq_decode(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T, const float* sinks,
                      float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                      kvq_stream stream) {
    return decode_impl(h, q, dtype, T, sinks, scale, out, lse, ws, ws_bytes, stream, false);
}

kvq_status kvq_decode_noalloc(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T, const float* sinks,
                              float scale, float* out, float* lse, kvq_stream stream) {
    return decode_impl(h, q, dtype, T, sinks, scale, out, lse, nullptr, 0, stream, true);
}

kvq_status kvq_importance(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T, float scale,
                          const float* lse, float* imp, kvq_stream stream) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (!q || !lse || !imp) return fail(KVQ_EINVAL, "q, lse or imp is NULL");
    if (dtype != KVQ_F32 && dtype != KVQ_BF16) return fail(KVQ_EINVAL, "dtype must be F32 or BF16");
    if (!std::isfinite(scale)) return fail(KVQ_EINVAL, "scale must be finite");
    if (T < 1) return fail(KVQ_EINVAL, "T must be >= 1");
    const kvq_config& c = h->cfg;
    int64_t maxspan = 0;
    for (int b = 0; b < c.n_seqs; ++b) {
        if (h->len[b] < T)
            return fail(KVQ_EINVAL, "session " + std::to_string(b) + " holds fewer than T rows");
        const int64_t lo = visible_lo(h, h->len[b], T);
        if (lo < h->base[b])
            return fail(KVQ_ERANGE, "session " + std::to_string(b) + ": visible rows were rebased away");
        // rows of the union (in graph mode, of the largest one the plane allows)
        maxspan = std::max(maxspan, span_of(h, b, T));
    }
    kvq::ImportanceParams ip{};
    ip.q = q;
    ip.f8 = is_f8(c);
    ip.dtype = dtype;
    ip.B = c.n_seqs;
    ip.T = T;
    ip.H = c.n_q_heads;
    ip.Hkv = c.n_kv_heads;
    ip.hd = c.head_dim;
    ip.hpk = c.n_q_heads / c.n_kv_heads;
    ip.window = c.window;
    ip.capacity = c.capacity;
    ip.k_planes = h->k;
    ip.k_stride = (int64_t)h->sz.k_session_stride;
    ip.k_row = (int32_t)h->sz.k_row_bytes;
    ip.len_d = len_d(h);
    ip.base_d = base_d(h);
    ip.scale = scale;
    ip.lse = lse;
    ip.imp = imp;
    ip.tiles = (int32_t)ceil_div(std::max<int64_t>(maxspan, 1), 16);
    if (!kvq::importance_group(ip.k_row, &ip.group_rows, &ip.rp))
        return fail(KVQ_EUNSUPPORTED, "importance: 16 K rows do not fit the LDS");
    // Many query rows (a prompt chunk): the (KV head, 16-row tile) pairs of a
    // key group are shared by several workgroups, each adding its sums with
    // atomics, so that the grid fills the device; up to kImpPairsPerWave
    // pairs per wave, one workgroup per key group, whose sums are added in a
    // fixed order.
    const int64_t pairs = (int64_t)c.n_kv_heads * ceil_div((int64_t)T * ip.hpk, 16);
    ip.pair_blocks = (int32_t)std::max<int64_t>(1, ceil_div(pairs, (int64_t)kvq::kImpWaves * kvq::kImpPairsPerWave));
    const char* err = nullptr;
    if (kvq::launch_importance(ip, stream, &err)) return fail(KVQ_EDEVICE, err ? err : "importance launch failed");
    return KVQ_OK;
}

kvq_status kvq_truncate(kvq_cache* h, const int32_t* new_len, kvq_stream stream) {
    if (!h || !new_len) return fail(KVQ_EINVAL, "NULL argument");
    const kvq_config& c = h->cfg;
    for (int b = 0; b < c.n_seqs; ++b) {
        if (new_len[b] < 0 || new_len[b] > h->len[b])
            return fail(KVQ_EINVAL, "session " + std::to_string(b) + ": truncate only shrinks");
        if (c.ring_step > 0 && std::max<int64_t>(0, (int64_t)new_len[b] - c.window) < h->base[b])
            return fail(KVQ_ERANGE, "session " + std::to_string(b) +
                                        ": the ring no longer holds rows the new length would expose");
    }
    std::vector<int32_t> idx, val;
    for (int b = 0; b < c.n_seqs; ++b)
        if (new_len[b] != h->len[b]) {
            idx.push_back(b);
            val.push_back(new_len[b]);
        }
    kvq_status s = enqueue_sets(h->counters, idx, val, stream);
    if (s != KVQ_OK) return s;
    for (int b = 0; b < c.n_seqs; ++b) h->len[b] = new_len[b];
    return KVQ_OK;
}

kvq_status kvq_rollback(kvq_cache* h, const int32_t* drop, kvq_stream stream) {
    if (!h || !drop) return fail(KVQ_EINVAL, "NULL argument");
    const kvq_config& c = h->cfg;
    for (int b = 0; b < c.n_seqs; ++b) {
        if (drop[b] < 0 || drop[b] > h->len[b])
            return fail(KVQ_EINVAL, "session " + std::to_string(b) + ": drop must lie in [0, len]");
        const int64_t nl = h->len[b] - drop[b];
        if (c.ring_step > 0 && std::max<int64_t>(0, nl - c.window) < h->base[b])
            return fail(KVQ_ERANGE, "session " + std::to_string(b) +
                                        ": the ring no longer holds rows the new length would expose");
    }
    std::vector<int32_t> idx, val;
    for (int b = 0; b < c.n_seqs; ++b)
        if (drop[b] != 0) {
            idx.push_back(b);
            val.push_back(-drop[b]);
        }
    kvq_status s = enqueue_sets(h->counters, idx, val, stream, 1, c.n_seqs, c.window);
    if (s != KVQ_OK) return s;
    for (int b = 0; b < c.n_seqs; ++b) h->len[b] -= drop[b];
    return KVQ_OK;
}

kvq_status kvq_set_split_rows(kvq_cache* h, int32_t rows) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (rows < 0 || rows % kvq::kSplitQuantum != 0)
        return fail(KVQ_EINVAL, "split rows must be 0 or a positive multiple of 64");
    h->split_rows = rows;
    return KVQ_OK;
}

kvq_status kvq_set_decode_tiling(kvq_cache* h, int32_t kernel, int32_t head_group, int32_t sub_tiles) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (kernel != KVQ_DECODE_AUTO && kernel != KVQ_DECODE_PER_HEAD && kernel != KVQ_DECODE_STREAM &&
        kernel != KVQ_DECODE_PRIME)
        return fail(KVQ_EINVAL, "unknown decode kernel");
    if (head_group < 0 || (head_group > 0 && h->cfg.n_kv_heads % head_group != 0))
        return fail(KVQ_EINVAL, "head_group must be 0 or a divisor of n_kv_heads");
    if (head_group > 0 && kernel != KVQ_DECODE_STREAM)
        return fail(KVQ_EINVAL, "head_group applies to the stream kernel");
    if (sub_tiles != 0 && !(kernel == KVQ_DECODE_STREAM && sub_tiles >= 1 && sub_tiles <= 3))
        return fail(KVQ_EINVAL, "sub_tiles must be 0, or 1, 2 or 3 for the stream kernel");
    h->decode_kernel = kernel;
    h->head_group = head_group;
    h->sub_tiles = sub_tiles;
    return KVQ_OK;
}

kvq_status kvq_info(const kvq_cache* h, kvq_info_t* out) {
    if (!h || !out) return fail(KVQ_EINVAL, "NULL argument");
    out->config = h->cfg;
    out->sizes = h->sz;
    out->k_planes = h->k;
    out->v_planes = h->v;
    out->counters = h->counters;
    out->split_rows = h->split_rows;
    return KVQ_OK;
}

kvq_status kvq_host_lengths(const kvq_cache* h, int64_t* len, int64_t* base) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    for (int b = 0; b < h->cfg.n_seqs; ++b) {
        if (len) len[b] = h->len[b];
        if (base) base[b] = h->base[b];
    }
    return KVQ_OK;
}

kvq_status kvq_set_importance(kvq_cache* h, float* imp) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (!aligned(imp, 4)) return fail(KVQ_EINVAL, "imp must be 4-byte aligned");
    h->imp = imp;
    return KVQ_OK;
}

kvq_status kvq_set_trace_events(kvq_cache* h, void* before_partials, void* before_combine,
                                void* after_combine) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    h->trace[0] = before_partials;
    h->trace[1] = before_combine;
    h->trace[2] = after_combine;
    return KVQ_OK;
}

kvq_status kvq_set_graph_mode(kvq_cache* h, int32_t on) {
    if (!h) return fail(KVQ_EINVAL, "handle is NULL");
    if (on != 0 && on != 1) return fail(KVQ_EINVAL, "on must be 0 or 1");
    h->graph_mode = on;
    return KVQ_OK;
}

kvq_status kvq_set_host_lengths(kvq_cache* h, const int64_t* len, const int64_t* base) {
    if (!h || !len || !base) return fail(KVQ_EINVAL, "NULL argument");
    const kvq_config& c = h->cfg;
    for (int b = 0; b < c.n_seqs; ++b) {
        if (base[b] < 0 || len[b] < base[b] || len[b] > INT32_MAX || len[b] - base[b] > c.capacity)
            return fail(KVQ_EINVAL, "session " + std::to_string(b) + ": need 0 <= base <= len <= base + capacity");
        if (c.ring_step == 0 && base[b] != 0)
            return fail(KVQ_EINVAL, "session " + std::to_string(b) + ": a flat cache has base 0");
    }
    for (int b = 0; b < c.n_seqs; ++b) {
        h->len[b] = len[b];
        h->base[b] = base[b];
    }
    return KVQ_OK;
}

void kvq_destroy(kvq_cache* h) { delete h; }

}  // extern "C"

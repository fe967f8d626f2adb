/*
 * kvq.h -- C ABI of libkvq: append to, and decode attention over, a per-layer
 * quantized KV cache on an AMD Instinct MI355X (gfx950).
 *
 * The cache (memra-engine, "Struct KvLayer" page, struct description and
 * fields k, v, k_tok_bytes, v_tok_bytes, len, ring, len_d, base_d):
 *   - K is stored q8_0: 34 bytes per 32 elements (fp16 scale d, then 32
 *     signed 8-bit codes; value = d * code).
 *   - V is stored q5_1: 24 bytes per 32 elements (fp16 step d, fp16 offset m,
 *     4 bytes holding bit 4 of each code, 16 bytes of nibbles where byte j
 *     holds code j in its low and code j+16 in its high nibble;
 *     value = d * code + m).
 *   - A token row keeps [kv_head, dim] order: element index kv_head*head_dim+d,
 *     block index/32, lane index%32; head_dim % 32 == 0, so no block
 *     straddles a head.  K row bytes = n_kv_heads*head_dim/32*34, V row bytes
 *     = n_kv_heads*head_dim/32*24.
 *   - FP8 variant (memra-engine "Module cache" page, kv_fp8_on: full-attention
 *     layers may hold K and V as e4m3; the pages give no layout): with
 *     k_fmt = v_fmt = KVQ_FMT_E4M3 every 32-element block has an fp16 scale
 *     d = amax/448 (round to nearest even) and 32 OCP FP8 E4M3 codes, each the
 *     code nearest to x / stored d (ties to the even code, magnitudes past 448
 *     saturating to +-448, the sign kept on zero; all 0 when d is 0); value =
 *     d * code.  A token row of n = n_kv_heads*head_dim elements holds the
 *     codes of all its blocks in element order (bytes 0 .. n-1), then the
 *     blocks' scales in block order (block k's at bytes n + 2k): 34 bytes per
 *     32 elements for K and for V.  Needs head_dim 64, 128 or 256 and a
 *     ring_step that is a multiple of 32 (else EUNSUPPORTED).
 *   - Every session has a device-resident committed length len_d (int32) and
 *     ring base base_d (int32).  An append writes its rows at the slot held
 *     in len_d and then advances len_d; a decode takes its length from len_d;
 *     so a step needs no device-to-host read.  A logical row lives at
 *     physical row (row - base); the live view of a windowed session is
 *     [max(0, len - window), len).  Only a ring rebase moves base; a truncate
 *     moves len only.
 *
 * Attention (cortiq-engine, "Struct LayerKvCache" page, methods attend_group
 * and attend_group_upto, field sinks): Q head h reads KV head h / (H/Hkv);
 * query row t of a T-row call sees logical rows [first_t, upto_t) with
 * upto_t = len - T + t + 1 and first_t = max(0, upto_t - window) (0 without a
 * window); score = scale * <q, k>; an optional per-Q-head sink logit joins the
 * softmax max and denominator and carries no value.  Output per (b, t, h) is
 *   out = sum_j e^(s_j - M) v_j / (sum_j e^(s_j - M) + e^(sink_h - M)),
 *   lse = M + log(denominator),   M = max(max_j s_j, sink_h).
 *
 * Ownership: the caller owns every device buffer (planes, counters, inputs,
 * outputs, workspace) and every stream.  The library owns only the host
 * handle.  It never allocates device memory, never synchronizes and never
 * reads device memory back to the host.
 *
 * Ordering: every call enqueues its work on the given stream (NULL = the
 * default stream).  All calls on one handle must be stream-ordered (the same
 * stream, or ordered by the caller), because the host keeps a mirror of
 * len/base in lock-step with the device counters.  A handle is not
 * thread-safe; distinct handles are independent.
 *
 * Errors: a call that returns anything but KVQ_OK enqueued nothing and
 * changed nothing (host mirror and device state are as before), except
 * KVQ_EDEVICE, which reports a failed kernel launch.  kvq_last_error() gives
 * a thread-local message for the last failure.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_EINVAL = 1,       /* bad argument, size, alignment or state */
    KVQ_ECAPACITY = 2,    /* a flat cache has no physical row left */
    KVQ_ERANGE = 3,       /* a row the call needs is no longer resident in the ring */
    KVQ_EUNSUPPORTED = 4, /* a format or shape this build does not implement */
    KVQ_EDEVICE = 5       /* a kernel launch failed */
} kvq_status;

typedef enum kvq_dtype {
    KVQ_F32 = 0,   /* IEEE binary32 */
    KVQ_BF16 = 1   /* bfloat16, widened exactly to binary32 on load */
} kvq_dtype;

typedef enum kvq_format {
    KVQ_FMT_Q8_0 = 1,
    KVQ_FMT_Q5_1 = 2,
    KVQ_FMT_E4M3 = 3   /* FP8 rows, for K and V together (see below) */
} kvq_format;

/* Geometry of one attention layer's cache for n_seqs sessions. */
typedef struct kvq_config {
    int32_t n_seqs;      /* B >= 1 */
    int32_t n_q_heads;   /* H >= 1, a multiple of n_kv_heads */
    int32_t n_kv_heads;  /* Hkv >= 1 */
    int32_t head_dim;    /* hd: a multiple of 32, at most 256 */
    int32_t capacity;    /* physical rows per session (max context, or ring rows) */
    int32_t window;      /* 0 = full attention; else the sliding-window length */
    int32_t ring_step;   /* 0 = flat [0, capacity); else rebase granularity in rows
                            (needs window > 0 and window + ring_step <= capacity) */
    int32_t k_fmt;       /* KVQ_FMT_Q8_0 with v_fmt KVQ_FMT_Q5_1, or KVQ_FMT_E4M3 for both */
    int32_t v_fmt;
} kvq_config;

/* Device bytes the caller must provide for a configuration. */
typedef struct kvq_sizes {
    size_t k_planes_bytes;    /* n_seqs * k_session_stride + 256 (read-only tail the
                                 decode may read past the last row; never written) */
    size_t v_planes_bytes;    /* n_seqs * v_session_stride + 256 (read-only tail as for K) */
    size_t counters_bytes;    /* int32 len_d[B], base_d[B], then library scratch:
                                 [2B] the append's completion counter, [2B + 1]
                                 the overflow word (see kvq_set_graph_mode) */
    size_t k_row_bytes;       /* Hkv*hd/32*34 */
    size_t v_row_bytes;       /* Hkv*hd/32*24 (q5_1) or Hkv*hd/32*34 (e4m3) */
    size_t k_session_stride;  /* capacity*k_row_bytes rounded up to 256 */
    size_t v_session_stride;  /* capacity*v_row_bytes rounded up to 256 */
} kvq_sizes;

typedef struct kvq_cache kvq_cache;   /* opaque host handle */
typedef void* kvq_stream;             /* a hipStream_t; NULL = default stream */

/* State of a handle, for callers and tests. */
typedef struct kvq_info_t {
    kvq_config config;
    kvq_sizes sizes;
    void* k_planes;       /* session b's K plane at k_planes + b*k_session_stride */
    void* v_planes;
    int32_t* counters;    /* len_d at counters[0..B), base_d at counters[B..2B) */
    int32_t split_rows;   /* rows per split-K chunk; 0 = chosen per call */
} kvq_info_t;

/* Fills *out for cfg: the device bytes of the K and V planes, sized up front
 * for capacity rows per session, and of the counters.  Pure host computation.
 * Defined by: memra-engine "Module cache" page, functions
 * cache_bytes_per_token (context-linear bytes per cached token) and
 * kv_blk_bytes (bytes per 32-element block of the selected K and V formats);
 * "Struct KvLayer" page, fields k_tok_bytes / v_tok_bytes (bytes per token
 * row) and struct description (34 and 24 bytes per 32 elements); "Struct
 * Cache" page, new (caches sized by the model geometry and the maximum
 * context).
 * Errors: EINVAL (NULL pointer, bad geometry), EUNSUPPORTED (format, head_dim). */
kvq_status kvq_required_bytes(const kvq_config* cfg, kvq_sizes* out);

/* Physical rows per session (kvq_config.capacity) of a ring that serves a
 * window-row sliding window to prompt chunks of up to max_chunk rows, with
 * base advancing ring_step rows at a time.  A decode starts each session at
 * its first visible row rounded down to 32: for a chunk appended at length
 * base_len that is (base_len - (window - 1)) & ~31, so at most 31 masked rows
 * precede the window.  With at least *rows rows, every append of 1 to
 * max_chunk rows, in any sequence from an empty session, neither drops a row
 * it still sees (no ERANGE) nor moves base above that 32-aligned start (so
 * the decode of its rows reads from the ring as it stands).  *rows =
 * window + max_chunk + ring_step - 2, plus 31 when ring_step is not a
 * multiple of 32, and at least window + ring_step; when ring_step is a
 * multiple of 32 no smaller ring has both properties.
 * Defined by: memra-engine "Module cache" page, constant
 * PRIME_CHUNK_MAX_TOKENS (the ring carries one whole maximum-size prime
 * chunk beyond the reader's window) and trait swa_ring_rows (the rows the
 * reader contract requires; prime starts at the window's first row rounded
 * down to 32).  The ring_step term is this library's: its ring rebases in
 * whole steps instead of wrapping.  Pure host computation.
 * Errors: EINVAL (rows NULL, an argument < 1, or a result above INT32_MAX). */
kvq_status kvq_ring_rows(int32_t window, int32_t max_chunk, int32_t ring_step, int32_t* rows);

/* Creates a handle over caller-owned device memory: k_planes / v_planes
 * (256-byte aligned, at least the sizes from kvq_required_bytes) and counters
 * (256-byte aligned, counters_bytes).  Enqueues the zeroing of len_d, base_d
 * and the library scratch on `stream`; plane contents are not touched.  The
 * host mirror starts at len = base = 0 (an empty cache).  The current device
 * is the one the handle's launches run on; its compute-unit count, read
 * here, sizes the split-K plans.
 * Defined by: memra-engine "Struct Cache" page, new (GPU-resident caches
 * sized by architecture and maximum context); "Struct KvLayer" page, fields
 * k, v (the planes), len, len_d and base_d (the counters); cortiq-engine
 * "Struct LayerKvCache" page, new (a layer cache for num_kv_heads heads of
 * head_dim).
 * Errors: EINVAL, EUNSUPPORTED, EDEVICE (also when the device's compute-unit
 * count cannot be read; then no handle is made and nothing is enqueued). */
kvq_status kvq_create(const kvq_config* cfg, void* k_planes, void* v_planes,
                      int32_t* counters, kvq_stream stream, kvq_cache** out);

/* Appends rows (memra KvLayer append-dc / append_kv_quantized_dcw, cortiq
 * LayerKvCache::append).  k_new and v_new are device arrays
 * [n_seqs, T, n_kv_heads, head_dim] of dtype.  Session b appends its first
 * n_new[b] rows (n_new is a HOST array of n_seqs entries in [0, T], or NULL
 * for all T).  The rows are quantized (K to q8_0, V to q5_1, each 32-element
 * block from its own absmax / min-max with fp16 scales rounded to nearest
 * even and codes computed from the stored scales, rounded half to even) and
 * written at physical rows len_d[b] - base_d[b] + t; len_d[b] then grows by
 * n_new[b] inside the same launch (rows that would pass the plane are never
 * written: see kvq_set_graph_mode).  In ring mode, if a session's rows would
 * pass the last physical row, the library first rebases it: base grows by
 * whole ring_step units until the rows fit, the surviving rows
 * [new_base, len) are moved to physical row 0, and base_d is updated.
 * Errors: EINVAL (NULL, dtype, T < 1, n_new out of range), ECAPACITY (flat
 * cache full), ERANGE (a rebase would drop rows the first new row still
 * sees), EDEVICE. */
kvq_status kvq_append(kvq_cache* h, const void* k_new, const void* v_new,
                      kvq_dtype dtype, int32_t T, const int32_t* n_new,
                      kvq_stream stream);

/* Device workspace bytes kvq_decode needs for T query rows at the handle's
 * current lengths (in graph mode, at every length the plane allows): the
 * split-K partials (m, l, o) of every (session, chunk, query row, Q head).
 * No passage defines it: the pages' decode has no caller workspace.  It
 * exists because this library never allocates device memory, so the
 * partials of the split-K decode live in a caller buffer.
 * Errors: EINVAL (NULL, T < 1, H/Hkv above 32). */
kvq_status kvq_decode_workspace_bytes(const kvq_cache* h, int32_t T, size_t* bytes);

/* Decode attention (memra fa_decode_dc / fa_decode_dcw; cortiq attend_group
 * and attend_group_upto).  q: device [n_seqs, T, n_q_heads, head_dim] of
 * dtype; its T rows are the last T committed rows of every session (causal
 * among themselves).  sinks: device float[n_q_heads] or NULL.  scale: the
 * score scale (normally 1/sqrt(head_dim)).  out: device float
 * [n_seqs, T, n_q_heads, head_dim].  lse: device float [n_seqs, T, n_q_heads]
 * or NULL.  ws: device workspace of at least kvq_decode_workspace_bytes
 * bytes, 256-byte aligned.  The committed length is read from len_d on the
 * device.  Requires len >= T for every session and H/Hkv <= 32.  Any T is
 * accepted (a prompt chunk attending causally, cortiq attend_group_upto with
 * many rows): the rows go in groups of 32/(H/Hkv) (the launch's y index;
 * from four groups on, with q8_0 / q5_1 rows at head_dim 64 or 128, eight
 * groups share each workgroup and its converted KV tiles), and one combine
 * folds all T rows; the workspace holds the partials of all T rows.
 * Input range: any finite queries and any q8_0 / q5_1 blocks (fp16 steps,
 * offsets and K scales up to 65504), as long as the scores scale * <q, k>
 * and the weighted V sums stay within binary32 range.  Query rows are
 * divided by a power of two before their fp16 cast (exact, so bf16 queries
 * keep every bit; fp32 queries keep about 22 bits as an fp16 high and low
 * part), V steps of 2^7 or more switch the P V accumulator to units of a
 * power of two, and (prompt chunks) K steps of 2^8 or more scale a tile's K
 * products by a power of two, so nothing overflows fp16.  The softmax weights enter
 * P V as fp16 (relative error 2^-11 each), so an output is within about
 * 2^-11 sum_j p_j |v_j| / sum_j p_j of the exact one.
 * Errors: EINVAL, ERANGE (a visible row was rebased away), EDEVICE. */
kvq_status kvq_decode(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T,
                      const float* sinks, float scale, float* out, float* lse,
                      void* ws, size_t ws_bytes, kvq_stream stream);

/* kvq_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the split-K partials go to the library's own
 * device scratch, a file-scope device array of 64 MiB (67108864 bytes) per
 * device, held from the library's load until the process ends.  Its device
 * address is looked up once per device by kvq_create; this call allocates
 * nothing and frees nothing.  Same arguments, semantics and errors as
 * kvq_decode otherwise, plus ECAPACITY when the call's partials (the bytes
 * kvq_decode_workspace_bytes reports for T) exceed 64 MiB; then nothing is
 * enqueued.  Every call on one device shares that device's scratch and
 * leaves its partials there: two calls whose executions overlap on one
 * device (on different streams, or from different threads without
 * ordering) race and give wrong results; calls ordered on one stream are
 * safe.  Nothing in the scratch needs to start at zero (each call writes
 * every partial its combine reads).
 * Errors: EINVAL, ERANGE, ECAPACITY, EDEVICE. */
kvq_status kvq_decode_noalloc(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T,
                              const float* sinks, float scale, float* out, float* lse,
                              kvq_stream stream);

/* Attention importance (cortiq LayerKvCache attend_group's imp_acc and
 * accumulate_imp: the attention mass each stored row receives, summed over
 * heads).  For the q, dtype, T and scale of a kvq_decode call, and the lse it
 * wrote (natural log, the sink included), adds to imp[b][row - base_b], for
 * every row a query row t sees, the sum over t and the n_q_heads heads of
 * exp(scale * q.K'_row - lse[b, t, h]): the row's softmax probability.  Rows
 * no query row sees get nothing; the sink's share is in lse but lands on no
 * row.  imp: device float [n_seqs, capacity], indexed by physical row (a ring
 * rebase moves K and V rows, and moves imp with them only when imp is
 * registered with kvq_set_importance).  Call it before the cache
 * changes again.  One launch; the rows are cut into groups of up to 64
 * consecutive rows of a session, each group taken by one workgroup, which
 * alone adds to its rows in a fixed order; with more than 32 (KV head,
 * 16-row tile of T * hpk query rows) pairs (a prompt chunk) a group's pairs
 * are shared by several workgroups, each adding its sums with a float atomic
 * add (the order of those additions, and so the last bits, may vary between
 * calls); in graph mode the groups cover every length the plane allows, like
 * kvq_decode's plan.  Queries of any
 * finite magnitude are taken as kvq_decode takes them; each probability is
 * exp of a binary32 score less the lse, so its relative error grows with
 * the score's magnitude (about 1e-2 at |score| near 1e5, 1e-4 near 1e3).
 * Errors: EINVAL, ERANGE (a visible row was rebased away), EUNSUPPORTED (K
 * rows of more than 296 blocks of 32 elements, e.g. more than 37 KV heads of
 * 256 dims: a workgroup stages 16 whole rows in its LDS), EDEVICE. */
kvq_status kvq_importance(kvq_cache* h, const void* q, kvq_dtype dtype, int32_t T, float scale,
                          const float* lse, float* imp, kvq_stream stream);

/* Rollback (memra Cache::rollback, full-attention part: len = snapshot_len +
 * accept_len, no copy; cortiq LayerKvCache::truncate_last).  new_len is a
 * HOST array of n_seqs lengths, each <= the current length.  Enqueues the
 * write of len_d; rows at or past new_len become dead and are not cleared;
 * base is never moved.
 * Errors: EINVAL (NULL, growth, negative), ERANGE (a windowed ring would
 * expose rows it no longer holds), EDEVICE. */
kvq_status kvq_truncate(kvq_cache* h, const int32_t* new_len, kvq_stream stream);

/* Rollback relative to the device length (memra Cache::rollback: drafted
 * rows not accepted; cortiq LayerKvCache::truncate_last): len_d[b] -= drop[b]
 * on the device, so that a captured append -> decode -> rollback round
 * replays from a graph while the lengths grow (see kvq_set_graph_mode).
 * drop is a HOST array of n_seqs entries in [0, len]; the host mirror moves
 * by the same amount.  On the device the length never goes below the
 * shortest one whose window is still resident (base_d + window in a rebased
 * ring, else 0).  Rows past the new length become dead; base never moves.
 * Errors: EINVAL, ERANGE (a windowed ring would expose rows it no longer
 * holds), EDEVICE. */
kvq_status kvq_rollback(kvq_cache* h, const int32_t* drop, kvq_stream stream);

/* Tuning: rows per split-K chunk of kvq_decode (a positive multiple of 64),
 * or 0 to let each call choose; a call raises it when a session would need
 * more than 1024 chunks.  The result does not depend on it beyond float
 * rounding: the chunks' partials are merged by the log-sum-exp identity, so
 * the attention of cortiq-engine "Struct LayerKvCache" attend_group is the
 * same for any split.  Errors: EINVAL. */
kvq_status kvq_set_split_rows(kvq_cache* h, int32_t rows);

/* Decode kernels (kvq_set_decode_tiling).  The value 2 is not used. */
typedef enum kvq_decode_kernel {
    KVQ_DECODE_AUTO = 0,        /* chosen per call */
    KVQ_DECODE_PER_HEAD = 1,    /* one KV head per workgroup, any head_dim, q8_0 / q5_1 rows only */
    KVQ_DECODE_STREAM = 3,      /* one or two waves per KV head, each streaming its rows through LDS */
    KVQ_DECODE_PRIME = 4        /* many query rows per KV head (a prompt chunk): eight groups of query
                                 * rows share each KV tile, converted once; q8_0 / q5_1 or FP8 rows,
                                 * head_dim 64 or 128, more than one group of query rows */
} kvq_decode_kernel;

/* Tuning: which kernel kvq_decode runs and how it tiles the cache (the
 * work split of cortiq-engine "Struct LayerKvCache" attend_group over the
 * GPU; the pages fix no tiling).
 * head_group: KV heads per workgroup for the stream kernel (a divisor of
 * n_kv_heads), 0 = chosen per call.  sub_tiles: waves per KV head for the
 * stream kernel: 1 or 2 row streams (up to 16 query rows per head), 1 wave
 * holding both 16-row tiles or 2 row-group waves (17 to 32 rows), or 3 = two
 * waves each taking half of a 128- or 256-dim head for all rows (17 to 32
 * rows); 0 = chosen per call.  The stream kernel needs head_dim 64, 128 or
 * 256; the prime kernel (no head_group, no sub_tiles) head_dim 64 or 128
 * and more than one group of 32 / hpk query rows.  A
 * kernel or tiling that does not fit a call's shape makes that kvq_decode
 * fail with EINVAL, except that a session whose first visible row, rounded
 * down to 32, was rebased away is served by the per-head kernel (FP8
 * rings rebase in steps of 32 rows, so it never happens to them).  The
 * automatic choice takes the prime kernel from four groups of query rows
 * on; for FP8 rows with dim halves it puts two KV heads in a workgroup.
 * The result does not depend on the choice beyond float rounding.
 * Errors: EINVAL (unknown kernel, head_group not dividing n_kv_heads,
 * head_group or sub_tiles given for a kernel other than the stream one). */
kvq_status kvq_set_decode_tiling(kvq_cache* h, int32_t kernel, int32_t head_group, int32_t sub_tiles);

/* Copies the handle's configuration, sizes and buffer pointers.
 * Defined by: cortiq-engine "Struct LayerKvCache" page, head_keys and
 * head_len (a head's stored rows and how many there are: here the plane
 * pointers, row bytes and capacity from which they are addressed);
 * memra-engine "Struct KvLayer" page, fields k, v, k_tok_bytes, v_tok_bytes.
 * Errors: EINVAL (NULL). */
kvq_status kvq_info(const kvq_cache* h, kvq_info_t* out);

/* Copies the host mirror: len[b] and base[b] for every session (HOST arrays
 * of n_seqs entries; either may be NULL).
 * Defined by: memra-engine "Struct KvLayer" page, fields len (the host
 * length, kept in step with len_d) and ring / base_d (the ring base);
 * cortiq-engine "Struct LayerKvCache" page, head_len.
 * Errors: EINVAL (NULL handle). */
kvq_status kvq_host_lengths(const kvq_cache* h, int64_t* len, int64_t* base);

/* Graph mode (memra KvLayer len_d: steps with no host round-trip; a captured
 * append -> decode chain replayed while the lengths grow).  When on (1),
 * kvq_decode and kvq_decode_workspace_bytes plan for every session's largest
 * span instead of its current one: the window plus T - 1 rows (plus 31 rows
 * of alignment) for a windowed cache, the whole plane otherwise.  The decode
 * kernels find each session's rows from len_d and base_d on the device, so a
 * decode captured in a graph stays valid at any later length as long as no
 * rebase is due.  Appends replayed from a graph are not seen by the host:
 * the append kernel itself writes only rows that fit the plane, stops len_d
 * at base_d + capacity, and then sets the overflow word counters[2 * n_seqs
 * + 1] to 1 (it stays 1).  After replays, kvq_set_host_lengths brings the
 * host mirror back in step.  Off (0) by default.  Errors: EINVAL. */
kvq_status kvq_set_graph_mode(kvq_cache* h, int32_t on);

/* Registers a device float array imp [n_seqs, capacity] (as kvq_importance
 * fills, indexed by physical row; NULL unregisters) that every later ring
 * rebase of this handle moves together with the K and V rows: the entries
 * of the surviving rows go where their rows go, and the entries of the
 * physical rows the rebase leaves unused (from the survivors' count up to
 * capacity) are set to 0, so that imp stays the mass of the row stored at
 * each position.  Flat caches never move rows.  The array must stay valid
 * until it is unregistered or the handle destroyed.
 * Defined by: cortiq-engine "Struct LayerKvCache" page, accumulate_imp (the
 * importance accumulated per stored row); memra-engine "Struct KvLayer"
 * page, base_d (the ring view that a rebase moves).
 * Errors: EINVAL (NULL handle, imp not 4-byte aligned). */
kvq_status kvq_set_importance(kvq_cache* h, float* imp);

/* Instrumentation: events (hipEvent_t, created by the caller; NULL = none)
 * that every later kvq_decode on this handle records on its stream: before
 * the split-K partials kernel, between it and the log-sum-exp combine, and
 * after the combine, so that a caller can time each kernel of the call
 * with hipEventElapsedTime.  All three NULL (the default) records nothing.
 * The events are recorded into a graph that captures the call.  No passage
 * defines it; it exists so that the kernels' durations can be measured
 * without a profiler.
 * Errors: EINVAL (NULL handle). */
kvq_status kvq_set_trace_events(kvq_cache* h, void* before_partials, void* before_combine,
                                void* after_combine);

/* Sets the host mirror of len and base (HOST arrays of n_seqs entries), for
 * example to the device counters read back after graph replays (memra-engine
 * "Struct KvLayer" page, len_d: the host len and the device counter are kept
 * in step; here the caller restores that after replays the host did not
 * see).  Requires 0 <= base <= len <= base + capacity, and base 0 for a flat
 * cache.  Nothing is enqueued.  Errors: EINVAL (nothing changed). */
kvq_status kvq_set_host_lengths(kvq_cache* h, const int64_t* len, const int64_t* base);

/* Frees the host handle only; device memory stays with the caller, as it
 * was allocated by the caller.  Defined by: cortiq-engine "Struct
 * LayerKvCache" page, clear (the cache of a conversation is dropped; a new
 * handle over the same planes starts empty, like a cleared cache).  NULL is
 * accepted and ignored. */
void kvq_destroy(kvq_cache* h);

/* Thread-local message describing the last failed call on this thread.
 * Defined by: memra-engine "Struct KvLayer" page, physical_rows (a failure
 * is returned with its message, Err(String), rather than clamped), and
 * "Struct Cache" page, new / rollback (Result with a boxed error).  The
 * string stays valid until the next failing call on the same thread. */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */

/*
 * kvdec -- single-query (one new token per slot) grouped-query decode
 * attention over a long KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method is split-KV flash decoding.  A slot's cells are cut into
 * 128-cell tiles; each workgroup streams a contiguous range of tiles of one
 * (slot, KV head) and produces an online-softmax partial (running maximum m,
 * sum l, unnormalised output o); a log-sum-exp merge combines the partials.
 * The same merge joins a resident window with a tail streamed from pinned
 * host memory ("Rolling-KV -- overflow throughput evaluations
 * (consolidated)", sections 1 and 3: the window is attended on the device,
 * the host tail is re-read every step, and the log-sum-exp channel is what
 * lets the two results combine).  Caches may be f16 or block-scaled int8 /
 * 4-bit, and cells may be given either as a contiguous range or as an
 * indirect list that the planner turns into a record-grouped plan with -1
 * holes ("KVARN KV Performance optimizations", beellama.cpp issue 140,
 * "What was implemented", items 3, 4 and 9).
 *
 * What is computed, for slot s and query head h (G = n_q_heads / n_kv_heads,
 * KV head g = floor(h / G), C_s the slot's attended cells):
 *     s_c = scale * sum_d q[s,h,d] * K[c,g,d]             for c in C_s
 *     m = max_c s_c,  l = sum_c e^(s_c - m),  o = sum_c e^(s_c - m) V[c,g,:]
 *     out[s,h,:] = o / l,   lse[s,h] = m + ln l
 * An empty C_s gives out = 0 and lse = -inf.  K and V are the dequantised
 * cache values: f16 as stored; int8 code q -> d * q; 4-bit code u -> d * (u - 8),
 * with one f16 scale d per 32 consecutive elements of a (cell, KV head) row
 * and element 2i of a 4-bit row in the low nibble of byte i.
 *
 * Arithmetic: fp32 accumulation.  q and the softmax weights may be rounded
 * to f16 inside packed dot products; results match a float64 evaluation of
 * the formula above to 2e-3 absolute for inputs of the magnitudes a decode
 * step sees (|q| far below the f16 limit of 65504).
 *
 * Ownership and threading.  The caller owns every buffer: q, the caches,
 * outputs and the workspace (device memory) and the pinned host tail.  The
 * library never allocates device memory and keeps no pointer after a call
 * returns, apart from work it has enqueued on the caller's streams.  A plan
 * is an immutable host object, safe to share between threads; it must be
 * rebuilt whenever the cache metadata it was built from changes.  A
 * workspace must not be used by two calls that may run at the same time.
 *
 * Errors.  Every entry point returns KVDEC_OK (0) or a negative code.
 * Arguments are validated before anything is enqueued, so a failed call has
 * no side effects; kvdec_last_error() gives a message for the calling
 * thread's most recent failure.  Faults inside enqueued device work surface
 * at the next synchronisation of the stream, as for any HIP kernel.
 */
#ifndef KVDEC_H
#define KVDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVDEC_VERSION 10801 /* 1.8.1: k, v, their scales and plan_cells may be NULL where no cell or entry exists */

/* Status codes. */
#define KVDEC_OK 0
#define KVDEC_E_INVALID (-1)     /* bad shape, null or misaligned pointer, bad enum */
#define KVDEC_E_RANGE (-2)       /* a cell >= capacity, or negative and not -1 */
#define KVDEC_E_UNSUPPORTED (-3) /* valid request with no compiled kernel for it */
#define KVDEC_E_WORKSPACE (-4)   /* workspace null or smaller than the plan needs */
#define KVDEC_E_NOMEM (-5)       /* host allocation failed */
#define KVDEC_E_DEVICE (-6)      /* a HIP runtime call failed */

/* Cache storage kinds (k_type, v_type). */
#define KVDEC_F16 0    /* binary16, 2 bytes per element */
#define KVDEC_Q8_B32 1 /* int8 codes + one f16 scale per 32 elements */
#define KVDEC_Q4_B32 2 /* 4-bit codes, two per byte, + one f16 scale per 32 elements */

/* Cells per tile and per physical record of an indirect plan. */
#define KVDEC_TILE_CELLS 128

/* Largest slot count a single plan accepts. */
#define KVDEC_MAX_SLOTS 64

/* kvdec_problem.kernel */
#define KVDEC_KERNEL_AUTO 0
#define KVDEC_KERNEL_STREAMED 1
#define KVDEC_KERNEL_ONESHOT 2

/* kvdec_attend_static: the library's own per-device scratch array holds a
 * merge-ticket area of KVDEC_STATIC_TICKET_BYTES followed by a workspace of
 * KVDEC_STATIC_WORKSPACE_BYTES (16 MiB + 1 MiB of device memory per GPU the
 * library runs on, held until the process ends). */
#define KVDEC_STATIC_TICKET_BYTES (1024 * 1024)

/* The merge-ticket area at the start of every plan's workspace: this size
 * for plans with up to KVDEC_TICKET_AREA_BYTES / 128 merge tickets, a
 * multiple of it beyond (kvdec_plan_info.ticket_bytes). */
#define KVDEC_TICKET_AREA_BYTES (1024 * 1024)
#define KVDEC_STATIC_WORKSPACE_BYTES (16 * 1024 * 1024)

/*
 * Problem description, read by kvdec_plan (host memory only; nothing is
 * retained after the call returns).
 *
 * n_q_heads, n_kv_heads: n_q_heads must be a multiple of n_kv_heads and the
 *   group size G = n_q_heads / n_kv_heads must lie in 1..16; kernels are
 *   built for G <= 8, larger groups give KVDEC_E_UNSUPPORTED.
 * head_dim: 64, 128 or 256.
 * n_slots: 1..KVDEC_MAX_SLOTS.
 * k_type, v_type: KVDEC_F16 / KVDEC_Q8_B32 / KVDEC_Q4_B32.  Kernels exist for
 *   K stored at least as finely as V: equal kinds, or (K, V) = (f16, int8),
 *   (f16, 4-bit), (int8, 4-bit) -- int8 K with 4-bit V is the pair of the
 *   resident-compression anchors ("Rolling-KV -- overflow throughput
 *   evaluations (consolidated)", section 5); other pairs give
 *   KVDEC_E_UNSUPPORTED.
 * scale: multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 * capacity_cells: number of device cells addressable through the K/V
 *   pointers of kvdec_attend; every attended cell must lie below it.  At
 *   most 2^48 (so is tail_capacity_cells), else KVDEC_E_INVALID.
 *
 * Cell selection, one of:
 *   contiguous (cells == NULL): slot s attends device cells
 *     [cell_begin[s], cell_begin[s] + n_occupied[s]); cell_begin may be NULL
 *     (all zero).  n_occupied[s] may be 0.
 *   indirect (cells != NULL): slot s's raw list is
 *     cells[cells_off[s] .. cells_off[s+1]-1]; -1 entries are holes, any other
 *     negative entry or an entry >= capacity_cells is KVDEC_E_RANGE, and
 *     duplicates are dropped (first occurrence kept).  The planner groups the
 *     kept cells by physical 128-cell record (cell / 128), takes the records
 *     in ascending order and emits one 128-entry segment per record whose
 *     entry k is record*128 + k when that cell was kept and -1 otherwise
 *     ("KVARN KV Performance optimizations", items 3 and 4).
 *
 *   device-built (cells == NULL, max_records != NULL): an indirect plan whose
 *     entries are built on the device by kvdec_build_cells, for cell lists
 *     that change every step.  Slot s gets max_records[s] 128-entry segments
 *     (0 .. ceil(capacity_cells / 128)); records the lists do not fill are
 *     all holes.
 *
 * Host tail (optional, contiguous mode only): when n_tail != NULL, slot s
 *   also attends cells [tail_begin[s], tail_begin[s] + n_tail[s]) of the
 *   pinned host tail arrays passed to kvdec_attend (dense
 *   [tail cell][kv head][row], scales likewise); tail_begin may be NULL (all
 *   zero) and tail_capacity_cells bounds the tail arrays.  The tail is copied
 *   to the device in chunks of tail_chunk_cells (a multiple of 128; 0 picks
 *   32768: larger copies run closer to the link rate) through a ring of
 *   tail_ring_depth staging slots (2..16; 0 picks 4; never more than the
 *   call's chunks) inside the workspace.  With tail_zero_copy = 1 nothing is staged: the
 *   chunk kernels read the pinned host arrays in place over the link.  (The
 *   "KVARN KV Performance optimizations" notes on pinned-host projector
 *   weights found such in-place reads slower than one staging copy because
 *   a GEMM re-reads its tiles; attention reads every tail byte once.)  The
 *   arrays must then be device-mapped pinned memory (hipHostMalloc), and
 *   the ring takes no workspace.
 *
 * tiles_per_split: 128-cell tiles per workgroup; 0 lets the planner choose
 *   so that the launch fills the device.  Only the floating-point summation
 *   order depends on it.
 *
 * split_cells: cells (plan positions) per workgroup, a multiple of 32; it
 *   overrides tiles_per_split when nonzero.  Splits of the vector-ALU kernel
 *   may end inside a 128-cell tile; the matrix-core kernel works on whole
 *   tiles and rounds split_cells up to a multiple of 128.  The planner picks
 *   32-cell split boundaries itself for the vector-ALU kernel, so that a
 *   short context can still give every compute unit one equal split.
 *
 * kernel: which split kernel serves a one-query-row problem on the vector
 *   ALU (G <= 5).  KVDEC_KERNEL_AUTO lets the planner choose;
 *   KVDEC_KERNEL_STREAMED forces the kernel that streams a split in steps;
 *   KVDEC_KERNEL_ONESHOT asks for the one-shot kernel, which issues every
 *   load of a split at workgroup entry and needs head_dim 128, f16 K and V,
 *   contiguous cells and splits of at most 448 cells (KVDEC_E_UNSUPPORTED
 *   otherwise).  The planner picks the one-shot kernel when those hold and
 *   one split per compute unit covers the cache; results differ between
 *   the kernels only in floating-point summation order.
 *
 * n_queries: query rows per slot, 1..8 (0 means 1).  Several rows per slot
 *   are the verification step of speculative decoding: split decoding serves
 *   up to 8 query rows, and such a call carries an attention mask ("KVARN KV
 *   Performance optimizations", "What was implemented" item 7).  Here the
 *   mask is positional: query row t of slot s sees the slot's cells whose
 *   position is at most q_pos[s][t] (kvdec_io).  All G * n_queries rows of a
 *   KV head share every K / V row read; kernels exist for head_dim 128 / 256
 *   with G * n_queries <= 16 (and, with one query row, any G <= 8 and
 *   G <= 16 for head_dim 128 / 256).
 */
typedef struct kvdec_problem {
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t n_slots;
    int32_t k_type;
    int32_t v_type;
    float scale;
    int32_t tiles_per_split;
    int64_t capacity_cells;
    const int64_t* cell_begin; /* [n_slots] or NULL */
    const int64_t* n_occupied; /* [n_slots], contiguous mode */
    const int32_t* cells;      /* indirect mode raw lists, or NULL */
    const int64_t* cells_off;  /* [n_slots + 1], indirect mode */
    const int64_t* tail_begin; /* [n_slots] or NULL */
    const int64_t* n_tail;     /* [n_slots] or NULL (no tail) */
    int64_t tail_capacity_cells;
    int64_t tail_chunk_cells;
    int32_t tail_ring_depth;
    int32_t n_queries;      /* query rows per slot, 1..8; 0 means 1 */
    int32_t tail_zero_copy; /* 1: kernels read the host tail in place */
    int32_t split_cells;    /* cells per split, multiple of 32; 0: tiles_per_split */
    const int32_t* max_records; /* [n_slots]: device-built indirect plan, see kvdec_build_cells */
    int32_t kernel;         /* KVDEC_KERNEL_AUTO (0), _STREAMED (1) or _ONESHOT (2) */
    int32_t pad0;
} kvdec_problem;

/* Opaque, immutable plan. */
typedef struct kvdec_plan kvdec_plan_t;

/*
 * Device buffers and outputs of one kvdec_attend call.
 *
 * q: device fp32 [n_slots][n_queries][n_q_heads][head_dim] (n_queries = 1:
 *   [n_slots][n_q_heads][head_dim]); out, lse and the partial triple below
 *   carry the same [n_queries] axis after the slot.
 * k, v: device code arrays, non-null whenever capacity_cells > 0, even when
 *   no cell is attended (the matrix-core kernel reads row 0 in place of hole
 *   entries); with capacity_cells 0 nothing reads them and they may be
 *   NULL.  Row (cell c,
 *   KV head g) starts at byte
 *   c * cell_stride + g * head_stride; a row holds head_dim f16 values,
 *   head_dim int8 codes, or head_dim / 2 bytes of 4-bit codes.  A stride of 0
 *   means the dense layout [cell][kv head][row].  Base pointers and strides
 *   must be multiples of 16 bytes (of 8 bytes for 4-bit rows).
 * k_scales, v_scales: device f16 scales, dense [cell][kv head][head_dim/32],
 *   required for the block-scaled kinds when capacity_cells > 0 and ignored
 *   for f16; aligned to one row of scales, min(16, head_dim / 16) bytes.
 * plan_cells: device int32 copy of the plan's entries (kvdec_plan_cells) in
 *   indirect mode, else NULL (also NULL allowed for an indirect plan of no
 *   entries).  Entries outside [0, capacity_cells) are read as holes.
 * k_tail, v_tail (+ k_tail_scales, v_tail_scales): pinned host tail arrays
 *   when the plan has a tail, else NULL.  They must stay valid and unchanged
 *   until the work enqueued by the call has finished.
 * out: device fp32 [n_slots][n_queries][n_q_heads][head_dim] or NULL.
 * lse: device fp32 [n_slots][n_queries][n_q_heads] or NULL.
 * part_m, part_l, part_o: device fp32 [n_slots][n_queries][n_q_heads] (m, l)
 *   and [n_slots][n_queries][n_q_heads][head_dim] (o): the call's whole result as one
 *   partial (m in score units, l and o relative to e^m, o unnormalised), for
 *   merging with other partials through kvdec_merge; all three or none.
 * At least one of out and the partial triple must be given.
 * q_pos: device int32 [n_slots][n_queries], required when n_queries > 1 and
 *   ignored otherwise: the position of each query row.
 * cell_pos: device int32 [capacity_cells] positions of the device cells, or
 *   NULL: a device cell's position is its cell index.  A host-tail cell's
 *   position is its index in the tail arrays.  Used with n_queries > 1 only.
 * copy_after: a hipEvent_t or NULL.  The tail copies of a call may not
 *   overwrite staging slots that earlier calls on the same workspace still
 *   read; by default they wait for all work enqueued on `stream` before the
 *   call.  With copy_after they wait for that event instead, so a caller
 *   that alternates two workspaces between consecutive layers can record an
 *   event after call l and pass it to call l + 2: the copies of layer l + 1
 *   then overlap layer l's kernels (cross-layer tail prefetch).
 * live_records: device int32 [n_slots] or NULL, indirect plans only: slot s
 *   uses only its first live_records[s] 128-entry segments of entries (values
 *   below 0 read as 0, above the slot's segments as all of them); the rest
 *   are never read.  The first n_slots values of kvdec_build_cells'
 *   n_records output fit: the -1 segments that pad a device-built plan up
 *   to max_records are then skipped instead of scanned (the result is the
 *   same either way: a hole contributes nothing).
 */
typedef struct kvdec_io {
    const float* q;
    const void* k;
    const void* v;
    const void* k_scales;
    const void* v_scales;
    int64_t k_cell_stride;
    int64_t k_head_stride;
    int64_t v_cell_stride;
    int64_t v_head_stride;
    const int32_t* plan_cells;
    const void* k_tail;
    const void* v_tail;
    const void* k_tail_scales;
    const void* v_tail_scales;
    float* out;
    float* lse;
    float* part_m;
    float* part_l;
    float* part_o;
    const int32_t* q_pos;
    const int32_t* cell_pos;
    void* copy_after;
    const int32_t* live_records;
} kvdec_io;

/* One partial result set for kvdec_merge: rows are (slot, query head) pairs,
 * m and l are [n_rows], o is [n_rows][head_dim], all device fp32. */
typedef struct kvdec_partial {
    const float* m;
    const float* l;
    const float* o;
} kvdec_partial;

/*
 * Build a plan (host only, deterministic).  n_cu is the number of compute
 * units to fill; 0 queries the current HIP device.  On success *out receives
 * the plan and *workspace_bytes the size of the device workspace that
 * kvdec_attend needs with it (the tile/split partials, merge tickets and the
 * tail staging ring).  A workspace's merge-ticket area (its first
 * kvdec_plan_info.ticket_bytes) must be zero-filled once before its first
 * use; every completed call leaves it at zero again, and nothing else in a
 * workspace is read before the call writes it.  So plans with the same
 * ticket_bytes (all plans with up to KVDEC_TICKET_AREA_BYTES / 128 merge
 * tickets) can take turns on one workspace of the largest workspace_bytes.
 * Errors: KVDEC_E_INVALID, KVDEC_E_RANGE, KVDEC_E_UNSUPPORTED, KVDEC_E_NOMEM,
 * KVDEC_E_DEVICE (only when n_cu == 0 and the device query fails).
 */
int kvdec_plan(const kvdec_problem* problem, int32_t n_cu, kvdec_plan_t** out, size_t* workspace_bytes);

/* Copy out the plan's indirect entries (int32, -1 holes) and per-slot entry
 * offsets (int64 [n_slots + 1]) for upload to the device.  With
 * cells_out == NULL only *n_entries is written.  A contiguous plan has zero
 * entries; a device-built plan has no host entries (cells_out must be NULL,
 * offsets_out may be given).  Errors: KVDEC_E_INVALID. */
int kvdec_plan_cells(const kvdec_plan_t* plan, int32_t* cells_out, int64_t* offsets_out, int64_t* n_entries);

/*
 * Build the entries of a device-built indirect plan on the device (the
 * descriptor setup of "KVARN KV Performance optimizations", "What was
 * implemented" item 5, with the plan layout of items 3 and 4): per slot,
 * the raw list is deduplicated through a capacity-sized bitmap, the kept
 * cells are grouped by physical 128-cell record, a 1024-thread scan takes the
 * records in ascending order, and one 128-entry segment is emitted per
 * record (entry k = record*128 + k when kept, else -1), followed by
 * segments of -1 only up to max_records[s].  The result equals kvdec_plan_cells of a
 * host plan over the same lists, padded with -1 segments.
 *
 * raw_cells: device int32, slot s's list at raw_cells[raw_off[s] ..
 *   raw_off[s+1]-1]; -1 entries are holes, duplicates are allowed; entries
 *   below -1 or at / above capacity_cells are dropped and counted.
 * raw_off: device int64 [n_slots + 1].
 * plan_cells: device int32 [n_entries of the plan] (kvdec_plan_get_info),
 *   the plan_cells argument of kvdec_attend.
 * n_records: device int32 [n_slots + 1] or NULL: records each slot's list
 *   touches -- more than max_records[s] means records were left out -- and,
 *   last, the number of dropped entries.
 * workspace: the plan's workspace (its build area is separate from what an
 *   in-flight kvdec_attend on the same workspace uses only if enqueued on the
 *   same stream before it).
 * Asynchronous on `stream`.  Errors: KVDEC_E_INVALID (not a device-built
 *   plan, null or misaligned pointers), KVDEC_E_WORKSPACE, KVDEC_E_DEVICE.
 */
int kvdec_build_cells(const kvdec_plan_t* plan, const int32_t* raw_cells, const int64_t* raw_off, int32_t* plan_cells,
                      int32_t* n_records, void* workspace, size_t workspace_bytes, void* stream);

/* Summary of a plan, for logs and tests. */
typedef struct kvdec_plan_info {
    int32_t n_slots;
    int32_t group;            /* G */
    int32_t n_workgroups;     /* workgroups of the resident launch */
    int32_t tiles_per_split;  /* largest tile count of any split */
    int64_t n_tiles;          /* tiles over all slots and KV heads */
    int64_t n_entries;        /* indirect entries (0 when contiguous) */
    int64_t n_tail_chunks;    /* tail chunks over all slots */
    int64_t workspace_bytes;
    int32_t n_queries;        /* query rows per slot */
    int32_t matrix_cores;     /* 1: served by the matrix-core kernel */
    int32_t split_cells;      /* largest position count of any split */
    int32_t split_unit;       /* split boundaries fall on multiples of this many positions */
    int32_t waves;            /* waves per workgroup of the resident launch (4 or 8) */
    int32_t kernel;           /* KVDEC_KERNEL_STREAMED or _ONESHOT for the vector-ALU kernels, 0 on matrix cores */
    int32_t split_interleave; /* U > 0: split s of a (slot, KV head) holds the U-cell units s, s + n_splits,
                                 s + 2 n_splits, ... of its positions; 0: each split is a contiguous run */
    int64_t ticket_bytes;     /* the merge-ticket area at the start of the workspace (one 128-byte line per
                                 ticket); the rest of the workspace need not be zero */
} kvdec_plan_info;

int kvdec_plan_get_info(const kvdec_plan_t* plan, kvdec_plan_info* info);

/* Split table: for each workgroup of the resident launch, in launch order, 4 int64 values
 * (slot, kv head, first position, position count), positions clipped to the
 * slot's cells (contiguous) or plan entries (indirect).  For an interleaved
 * plan (kvdec_plan_info.split_interleave = U) the positions of a split are
 * its U-cell units first, first + U * n_splits, ... (n_splits = the slot's
 * splits per KV head) and the count is their total.  With splits_out ==
 * NULL only *n_splits is written. */
int kvdec_plan_splits(const kvdec_plan_t* plan, int64_t* splits_out, int64_t* n_splits);

void kvdec_plan_free(kvdec_plan_t* plan);

/*
 * Enqueue one decode-attention evaluation on `stream` (a hipStream_t; NULL is
 * the default stream).  `copy_stream` carries the host-to-device copies of
 * the tail (needed only when the plan has a tail; NULL then means `stream`).
 * workspace: device memory of at least the plan's workspace_bytes, 256-byte
 * aligned, zero-filled before its first use.  Asynchronous: returns once the
 * work is enqueued.
 * Errors: KVDEC_E_INVALID, KVDEC_E_WORKSPACE, KVDEC_E_UNSUPPORTED,
 * KVDEC_E_DEVICE.
 */
int kvdec_attend(const kvdec_plan_t* plan, const kvdec_io* io, void* workspace, size_t workspace_bytes,
                 void* stream, void* copy_stream);

/*
 * kvdec_attend without a caller workspace, for callers that cannot allocate
 * device memory: code recorded under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It enqueues exactly what kvdec_attend
 * enqueues for the same plan and io, with the workspace taken from a
 * file-scope device array of the library (KVDEC_STATIC_TICKET_BYTES of merge
 * tickets, then KVDEC_STATIC_WORKSPACE_BYTES of workspace, one copy per GPU);
 * it calls no allocating routine.  The first call on a device looks up that
 * device's copy and enqueues a clear of its ticket area on `stream` (a call
 * made under stream capture records the clear into the graph, and the next
 * call outside capture clears again); every completed call leaves the
 * tickets at zero.  All calls on one GPU share its array, so calls that may
 * overlap on one GPU (different streams, or a graph replay beside an eager
 * call) race and must be ordered by the caller.  The outputs never alias the
 * array; partial records from the previous call stay in it and are
 * overwritten before they are read.
 * Errors: as kvdec_attend, and KVDEC_E_WORKSPACE when the plan's
 * workspace_bytes exceed KVDEC_STATIC_WORKSPACE_BYTES or its merge tickets
 * (n_slots * n_kv_heads plus its cluster tickets) exceed the ticket area,
 * KVDEC_E_UNSUPPORTED for a plan with a copied host tail (its ring ordering
 * needs per-call events; a tail_zero_copy plan is accepted), KVDEC_E_DEVICE
 * when the device's array cannot be looked up.
 */
int kvdec_attend_static(const kvdec_plan_t* plan, const kvdec_io* io, void* stream);

/*
 * Log-sum-exp merge of n_parts partial sets over the same n_rows rows
 * (section 9 of "KVARN KV Performance optimizations": partial windows keep
 * their maximum, numerator and denominator and are merged afterwards):
 *     M = max_p m_p,  L = sum_p l_p e^(m_p - M),  O = sum_p o_p e^(m_p - M)
 *     out = O / L,    lse = M + ln L
 * Partials with m = -inf contribute nothing; rows where all are empty give
 * out = 0, lse = -inf and the merged partial (-inf, 0, 0).  out, lse and the
 * merged triple (merged_m, merged_l, merged_o) are each optional (NULL), but
 * at least one output must be given.  `parts` is host memory holding device
 * pointers; 1 <= n_parts <= 64; head_dim in 1..1024.  Asynchronous on stream.
 * Errors: KVDEC_E_INVALID, KVDEC_E_DEVICE.
 */
int kvdec_merge(int32_t n_parts, const kvdec_partial* parts, int64_t n_rows, int32_t head_dim, float* out,
                float* lse, float* merged_m, float* merged_l, float* merged_o, void* stream);

/* Static description of a status code. */
const char* kvdec_strerror(int status);

/* Message for the calling thread's most recent failure ("" if none). */
const char* kvdec_last_error(void);

/* KVDEC_VERSION of the built library. */
int kvdec_version(void);

/* Hash (16 hex digits) of the source files and compiler flags the library
 * was built from, fixed at build time; the build script writes the same
 * value of the current sources, so a caller can detect a stale binary.
 * Static storage, never NULL. */
const char* kvdec_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* KVDEC_H */

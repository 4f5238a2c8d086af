// Internal declarations shared by the planner, the host runtime and the HIP
// kernels of libkvdec.  Not part of the public C ABI (include/kvdec.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kvdec.h"

#ifdef __cplusplus
#include <string>
#include <vector>
#endif

namespace kvdec {

constexpr int kTile = KVDEC_TILE_CELLS;  // cells per tile / per physical record
constexpr int64_t kMaxCells = int64_t(1) << 48;  // bound of capacity_cells and tail_capacity_cells
constexpr int kBlock = 32;               // elements sharing one f16 scale
constexpr int kThreads = 256;            // threads per split workgroup (4 waves)
constexpr int kSplitUnit = 32;           // split boundary granularity of the vector-ALU kernel
// Merge tickets sit one per 128-byte line: device-scope atomics on one line
// are performed one after another, and the splits of every KV head arrive
// at about the same time.
constexpr int kTicketStride = 32;        // uint32 words from one ticket to the next
constexpr int kMergeMaxParts = 64;       // kvdec_merge fan-in

// Bytes of one stored (cell, KV head) row of codes.
inline constexpr int64_t row_bytes(int type, int head_dim) {
    return type == KVDEC_F16 ? 2 * (int64_t)head_dim : type == KVDEC_Q8_B32 ? (int64_t)head_dim : (int64_t)head_dim / 2;
}
inline constexpr bool is_scaled(int type) { return type != KVDEC_F16; }

// Which kernel serves a problem, and the rows of its split records (the
// query rows one (slot, KV head) workgroup serves).  One query row per slot
// with G <= 5 (or head_dim 64) runs on the VALU kernel, whose records hold
// the G rows; wider groups and several query rows per slot (head_dim 128 /
// 256, G * n_q <= 16) run on the matrix-core kernel, whose records hold the
// G * n_q rows padded to 8 or 16.
constexpr bool uses_matrix_cores(int group, int n_q, int head_dim) {
    return (n_q > 1 || group >= 6) && head_dim >= 128;
}
// Rows of a split record on the matrix-core kernel (mfma) or the VALU kernel.
constexpr int record_rows_of(bool mfma, int group, int n_q) {
    return mfma ? (group * n_q <= 8 ? 8 : 16) : group;
}
constexpr int record_rows(int group, int n_q, int head_dim) {
    return record_rows_of(uses_matrix_cores(group, n_q, head_dim), group, n_q);
}

// Split records one merge round reads: a merging workgroup issues the loads
// of this many records before it waits (UB records per thread and float4
// column, TS threads per column).
constexpr int merge_chunk(int head_dim, int group) {
    const int nv = group * head_dim / 4;  // float4 columns of a record's o
    const int ts = nv >= kThreads ? 1 : kThreads / nv;
    const int cols = (nv + kThreads - 1) / kThreads;
    const int ub = cols == 1 ? 32 : 32 / cols;
    return ub * ts < 64 ? ub * ts : 64;
}
// Records of 16 rows at head_dim 128 (512 float4 columns) take two columns
// per thread and, by merge_chunk, 16 records per round; the kernel holds up
// to 28 without spilling, so a group of at most 28 splits merges in one round
// instead of two (4-query Qwen3-8B-shaped layer 26.7 -> 25.4 us).  At
// head_dim 256 the larger round measured slower on the GQA-6 caches.
constexpr int merge_chunk_max(int head_dim, int group) {
    return head_dim == 128 && group == 16 ? 28 : merge_chunk(head_dim, group);
}
// Round size for the records of a (slot, KV head) with n_splits splits.
constexpr int merge_chunk_for(int head_dim, int group, int n_splits) {
    return n_splits <= merge_chunk_max(head_dim, group) ? merge_chunk_max(head_dim, group) : merge_chunk(head_dim, group);
}
// Clusters per (slot, KV head): one level of merging while it takes at most
// two rounds, else clusters of merge_chunk splits merged first, each into a
// cluster record, and the cluster records merged last.
constexpr int merge_clusters(int n_splits, int chunk) {
    return n_splits <= 2 * chunk ? 1 : (n_splits + chunk - 1) / chunk;
}

// Running partial of the window + tail chain: m2 [rows], l [rows], then o
// [rows][D] at this float offset -- 2 * rows rounded up to a multiple of 4,
// so the o rows stay 16-byte aligned (they are read and written as float4)
// whatever the row count.
inline constexpr int64_t acc_o_offset(int64_t rows) { return (2 * rows + 3) / 4 * 4; }
inline constexpr int64_t acc_floats(int64_t rows, int64_t head_dim) { return acc_o_offset(rows) + rows * head_dim; }

// Per-slot launch description, passed to the split kernel by value.
struct SlotArg {
    int64_t first;       // contiguous: first cell; indirect: first plan entry
    int64_t n;           // contiguous: occupied cells; indirect: plan entries
    int32_t n_units;     // ceil(n / split_unit): split boundaries fall on multiples of split_unit
    int32_t n_splits;    // splits per KV head (>= 1)
    int32_t wg_begin;    // first workgroup of this slot (n_kv_heads * n_splits of them)
    int32_t part_begin;  // first partial record of this slot
    int32_t to_acc;      // 1: the slot's result goes to acc_out (more partials follow)
    int32_t n_clusters;  // merge_clusters(n_splits, chunk)
    int32_t cl_begin;    // first cluster (ticket and record) of this slot
    int32_t chunk;       // records per merge round: merge_chunk_for(D, G, n_splits)
};

// Kernel arguments of one split launch (fits the 4 KiB kernarg segment).
struct SplitArgs {
    const float* q;          // [slots][Hq][D] fp32 (row of slot s: q + (slot_base + s) * Hq * D)
    const uint8_t* k;        // codes
    const uint8_t* v;
    const uint16_t* ks;      // f16 scales, dense [cell][Hkv][D/32]
    const uint16_t* vs;
    int64_t k_cs, k_hs;      // byte strides (cell, head) of K rows
    int64_t v_cs, v_hs;
    const int32_t* plan;     // indirect entries, or null for contiguous cells
    const int32_t* live_records;  // [slots] 128-entry records in use at the front of each slot's entries, or null
    int64_t capacity;        // cells addressable through k / v (indirect bound check)
    float* part_o;           // split partial records: o [record][G][D]
    float* part_m;           //   running max in log2 units [record][G]
    float* part_l;           //   sum [record][G]
    int64_t part_o_bytes;    // bytes of the o region (bound of its buffer resource)
    uint32_t* tickets;       // one per (slot, KV head), kTicketStride words apart
    uint32_t* ctickets;      // one per cluster of splits, kTicketStride words apart
    int32_t crec_base;       // record index of cluster 0's record
    int32_t waves;           // waves per workgroup of either kernel: 4 or 8
    float* out;              // [slots][Hq][D] or null
    float* lse;              // [slots][Hq] or null
    float* pm;               // whole-call partial (m natural units, l, o) or null
    float* pl;
    float* po;
    const float* acc_in;     // running partial merged in by the last workgroup, or null
    float* acc_out;          // running partial written for slots with to_acc
    int32_t acc_rows;        // rows of a running partial: m2 [rows], l [rows], o [rows][D] at acc_o_offset(rows)
    int32_t oneshot;         // > 0: the one-shot kernel with this many 8-cell loads per lane (planner's choice)
    int32_t interleave;      // one-shot kernel: split s holds split units s, s + n_splits, ... (else a contiguous run)
    int32_t n_q;             // query rows per slot (q, out, lse rows: [slot][n_q][Hq])
    const int32_t* q_pos;    // [slots][n_q] positions of the query rows (n_q > 1)
    const int32_t* cell_pos; // [capacity] positions of device cells, or null: cell index + pos_offset
    int64_t pos_offset;      // added to a cell index to give its position (no cell_pos)
    int32_t group;           // query heads per KV head (G)
    int32_t split_unit;      // positions per split unit (SlotArg::n_units)
    float scale_log2;        // scale * log2(e)
    int32_t n_slots;         // slots in this launch
    int32_t slot_base;       // index of slot 0 of this launch in q / out / lse / p*
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t n_workgroups;
    SlotArg slot[KVDEC_MAX_SLOTS];
#ifdef KVDEC_PHASE_TRACE
    unsigned long long* trace;  // diagnostic build: 32 clock stamps per workgroup (see split_kernels.h), or null
#endif
};

struct MergeArgs {
    const float* m[kMergeMaxParts];
    const float* l[kMergeMaxParts];
    const float* o[kMergeMaxParts];
    int32_t n_parts;
    int32_t head_dim;
    int64_t n_rows;
    float* out;
    float* lse;
    float* mm;
    float* ml;
    float* mo;
};

// Arguments of the device plan build (plan_device.hip).
struct BuildArgs {
    const int32_t* raw;      // raw lists
    const int64_t* raw_off;  // [n_slots + 1] (device)
    uint32_t* bitmap;        // [n_slots][words_per_slot]
    int32_t* list;           // present records, slot s at list_off[s]
    int32_t* count;          // [n_slots + 1]: records each slot touches, then dropped entries
    int32_t* n_records;      // caller copy of count, or null
    int32_t* out;            // plan entries
    int64_t capacity;
    int64_t words_per_slot;
    int64_t n_entries;
    int32_t n_slots;
    int32_t pad;
    int32_t max_records[KVDEC_MAX_SLOTS];
    int64_t list_off[KVDEC_MAX_SLOTS + 1];
    int64_t entry_off[KVDEC_MAX_SLOTS + 1];
};
int launch_build_cells(const BuildArgs& a, void* stream);

// Kernel launchers (kernels.hip, split_*.hip).  Return a hipError_t value.
// Per pair of storage kinds, the launcher of the split-kernel instance for
// (head_dim, group), or null.
using SplitLaunchFn = int (*)(const SplitArgs&, void*);
SplitLaunchFn pick_split_f16(int head_dim, int group, int n_q, bool mfma);
SplitLaunchFn pick_split_q8(int head_dim, int group, int n_q, bool mfma);
SplitLaunchFn pick_split_q4(int head_dim, int group, int n_q, bool mfma);
SplitLaunchFn pick_split_f16_q8(int head_dim, int group, int n_q, bool mfma);
SplitLaunchFn pick_split_f16_q4(int head_dim, int group, int n_q, bool mfma);
SplitLaunchFn pick_split_q8_q4(int head_dim, int group, int n_q, bool mfma);
int launch_split(int head_dim, int group, int n_q, int k_type, int v_type, bool mfma, const SplitArgs& a,
                 void* stream);
int launch_merge(const MergeArgs& a, void* stream);
// The calling thread's current device's copy of the static scratch array of
// kvdec_attend_static (set up on first use per device; the first use also
// enqueues a clear of the ticket area on `stream`).
int static_scratch(void* stream, void** base);  // a hipError_t
bool split_instance_exists(int head_dim, int group, int n_q, int k_type, int v_type, bool mfma);

}  // namespace kvdec

#ifdef __cplusplus
// The plan object behind the opaque kvdec_plan_t.
struct kvdec_plan {
    int32_t n_q_heads = 0, n_kv_heads = 0, head_dim = 0, n_slots = 0, group = 0;
    int32_t n_q = 1;       // query rows per slot
    int32_t rec_rows = 0;  // rows of a split record (record_rows)
    int32_t k_type = 0, v_type = 0;
    float scale = 0.f;
    int64_t capacity = 0;
    bool indirect = false;
    std::vector<kvdec::SlotArg> slots;
    int32_t n_workgroups = 0;
    int32_t n_part_records = 0;
    int32_t max_tiles_per_split = 0;
    int32_t split_unit = 0;        // positions per split unit: 32 (vector-ALU kernel) or 128
    int32_t max_split_cells = 0;   // largest split, in positions
    int32_t waves = 4;             // waves per split workgroup (4 or 8)
    int32_t oneshot = 0;           // resident launch on the one-shot kernel: 8-cell loads per lane (2, 4 or 7)
    bool interleave = false;       // one-shot splits hold every n_splits-th unit of 32 cells
    bool mfma = false;             // served by the matrix-core kernel
    int64_t n_tiles = 0;
    std::vector<int32_t> cells;      // indirect entries (host-built plans)
    std::vector<int64_t> cells_off;  // [n_slots + 1]
    // device-built indirect plans (kvdec_build_cells)
    bool device_cells = false;
    std::vector<int32_t> max_records;  // segments per slot
    int64_t n_device_entries = 0;
    int64_t bm_words_per_slot = 0;
    size_t off_build_bitmap = 0, off_build_list = 0, off_build_count = 0;

    // Tail: per slot, host cell range and chunking.
    bool has_tail = false;
    bool tail_zero_copy = false;     // chunk kernels read the host tail in place
    std::vector<int64_t> tail_begin, tail_n;
    int64_t tail_capacity = 0;
    int64_t chunk_cells = 0;
    int32_t ring_depth = 0;
    int32_t chunk_tiles_per_split = 1;
    int32_t chunk_splits = 0;        // splits per KV head of a full chunk
    int64_t n_tail_chunks = 0;

    // Workspace layout (byte offsets, 256-aligned).
    // acc0 / acc1: running partials (ping-pong) of the window + tail chain.
    size_t off_tickets = 0, off_parts = 0, off_acc0 = 0, off_acc1 = 0, off_ring = 0;
    size_t ticket_bytes = 0;  // the merge-ticket area at the start of the workspace
    int32_t n_part_capacity = 0;     // partial records the parts region holds
    int32_t crec_base = 0;           // record index of the first cluster record
    int32_t n_cluster_capacity = 0;  // cluster tickets / records reserved
    size_t off_parts_m = 0, off_parts_l = 0, parts_o_bytes = 0;
    size_t ring_slot_bytes = 0, ring_k = 0, ring_v = 0, ring_ks = 0, ring_vs = 0;
    size_t workspace_bytes = 0;
};

namespace kvdec {
// Host-only planning (plan.cpp).  Returns a status code; on failure `err`
// holds a message.
int build_plan(const kvdec_problem& p, int32_t n_cu, kvdec_plan_t& plan, std::string& err);
}  // namespace kvdec
#endif

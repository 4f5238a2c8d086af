// Host-only planner of libkvdec: validation, the record-grouped compact plan
// of indirect cell lists, the split decomposition over the compute units and
// the workspace layout.  No HIP dependency.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "internal.h"

namespace kvdec {
namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compact read plan of one slot's raw cell list ("KVARN KV Performance
// optimizations", "What was implemented" items 3 and 4): holes (-1) dropped,
// other negatives and cells >= capacity rejected, duplicates filtered with a
// capacity-sized bitmap (first occurrence kept), kept cells grouped by their
// physical 128-cell record, records in ascending order, one 128-entry segment
// per record with -1 in the positions that were not kept.  `bitmap` is
// capacity bits, all zero on entry and on return.
int compact_slot(const int32_t* raw, int64_t n, int64_t capacity, std::vector<uint64_t>& bitmap,
                 std::vector<int64_t>& records, std::vector<int32_t>& out, std::string& err) {
    records.clear();
    for (int64_t i = 0; i < n; ++i) {
        const int64_t c = raw[i];
        if (c == -1) continue;
        if (c < -1 || c >= capacity) {
            err = "cell " + std::to_string(c) + " at raw index " + std::to_string(i) + " outside [0, capacity)";
            std::fill(bitmap.begin(), bitmap.end(), 0);
            return KVDEC_E_RANGE;
        }
        uint64_t& word = bitmap[(size_t)c >> 6];
        const uint64_t bit = 1ull << (c & 63);
        if (word & bit) continue;  // duplicate: first occurrence already kept
        // A record is listed when its first cell is kept.
        const int64_t rec = c / kTile;
        bool rec_seen = false;
        for (int k = 0; k < kTile / 64; ++k)
            if (bitmap[(size_t)rec * (kTile / 64) + k]) rec_seen = true;
        if (!rec_seen) records.push_back(rec);
        word |= bit;
    }
    std::sort(records.begin(), records.end());
    for (int64_t rec : records) {
        for (int k = 0; k < kTile; ++k) {
            const int64_t c = rec * kTile + k;
            const bool kept = (bitmap[(size_t)c >> 6] >> (c & 63)) & 1;
            out.push_back(kept ? (int32_t)c : -1);
        }
        for (int k = 0; k < kTile / 64; ++k) bitmap[(size_t)rec * (kTile / 64) + k] = 0;
    }
    return KVDEC_OK;
}

}  // namespace

int build_plan(const kvdec_problem& p, int32_t n_cu, kvdec_plan_t& plan, std::string& err) {
    // ---- shape
    if (p.n_q_heads < 1 || p.n_kv_heads < 1 || p.n_q_heads % p.n_kv_heads != 0) {
        err = "n_q_heads must be a positive multiple of n_kv_heads";
        return KVDEC_E_INVALID;
    }
    const int group = p.n_q_heads / p.n_kv_heads;
    if (group > 16) {
        err = "group size n_q_heads / n_kv_heads must be at most 16";
        return KVDEC_E_INVALID;
    }
    if (p.head_dim != 64 && p.head_dim != 128 && p.head_dim != 256) {
        err = "head_dim must be 64, 128 or 256";
        return KVDEC_E_INVALID;
    }
    if (p.n_slots < 1) {
        err = "n_slots must be >= 1";
        return KVDEC_E_INVALID;
    }
    if (p.n_slots > KVDEC_MAX_SLOTS) {
        err = "n_slots above KVDEC_MAX_SLOTS";
        return KVDEC_E_UNSUPPORTED;
    }
    for (int t : {p.k_type, p.v_type})
        if (t != KVDEC_F16 && t != KVDEC_Q8_B32 && t != KVDEC_Q4_B32) {
            err = "k_type / v_type must be KVDEC_F16, KVDEC_Q8_B32 or KVDEC_Q4_B32";
            return KVDEC_E_INVALID;
        }
    if (!std::isfinite(p.scale)) {
        err = "scale must be finite";
        return KVDEC_E_INVALID;
    }
    if (p.capacity_cells < 0 || p.tiles_per_split < 0 || n_cu < 1) {
        err = "capacity_cells, tiles_per_split must be >= 0 and n_cu >= 1";
        return KVDEC_E_INVALID;
    }
    // far beyond any device's memory, and small enough that no cell index or
    // byte offset computed from it can overflow
    if (p.capacity_cells > kMaxCells || p.tail_capacity_cells > kMaxCells) {
        err = "capacity_cells and tail_capacity_cells must be at most 2^48";
        return KVDEC_E_INVALID;
    }
    const bool device_cells = p.cells == nullptr && p.max_records != nullptr;
    const bool indirect = p.cells != nullptr || device_cells;
    if (p.cells != nullptr && !p.cells_off) {
        err = "indirect mode needs cells_off";
        return KVDEC_E_INVALID;
    }
    if (!indirect && !p.n_occupied) {
        err = "contiguous mode needs n_occupied";
        return KVDEC_E_INVALID;
    }
    const bool has_tail = p.n_tail != nullptr;
    if (has_tail && indirect) {
        err = "a host tail is supported with contiguous cells only";
        return KVDEC_E_UNSUPPORTED;
    }
    if (p.n_queries < 0 || p.n_queries > 8) {
        err = "n_queries must be 0 (one) or 1..8";
        return KVDEC_E_INVALID;
    }
    const int n_q = p.n_queries ? p.n_queries : 1;
    if (!split_instance_exists(p.head_dim, group, n_q, p.k_type, p.v_type,
                               uses_matrix_cores(group, n_q, p.head_dim))) {
        err = "no kernel for this (head_dim, group, n_queries, k_type, v_type): groups above 8 and several "
              "query rows need head_dim 128 or 256 and G * n_queries <= 16, and K is stored at least as "
              "finely as V";
        return KVDEC_E_UNSUPPORTED;
    }

    plan.n_q_heads = p.n_q_heads;
    plan.n_kv_heads = p.n_kv_heads;
    plan.head_dim = p.head_dim;
    plan.n_slots = p.n_slots;
    plan.group = group;
    plan.n_q = n_q;
    plan.k_type = p.k_type;
    plan.v_type = p.v_type;
    plan.scale = p.scale;
    plan.capacity = p.capacity_cells;
    plan.indirect = indirect;
    plan.device_cells = device_cells;
    plan.slots.assign(p.n_slots, SlotArg{});

    // ---- cells of each slot
    if (device_cells) {
        // entries come from kvdec_build_cells: max_records[s] segments per slot
        // (none without cells: the matrix-core kernel reads row 0 of the
        // cache in place of a hole, so a segment needs a cache of >= 1 cell)
        const int64_t rec_cap = ceil_div(p.capacity_cells, kTile);
        plan.cells_off.assign(p.n_slots + 1, 0);
        plan.max_records.assign(p.n_slots, 0);
        for (int s = 0; s < p.n_slots; ++s) {
            const int64_t m = p.max_records[s];
            if (m < 0 || m > rec_cap) {
                err = "slot " + std::to_string(s) + ": max_records outside 0 .. ceil(capacity_cells / 128)";
                return KVDEC_E_INVALID;
            }
            plan.max_records[s] = (int32_t)m;
            plan.slots[s].first = plan.cells_off[s];
            plan.slots[s].n = m * kTile;
            plan.cells_off[s + 1] = plan.cells_off[s] + m * kTile;
        }
        plan.n_device_entries = plan.cells_off[p.n_slots];
    } else if (indirect) {
        plan.cells_off.assign(p.n_slots + 1, 0);
        for (int s = 0; s < p.n_slots; ++s) {
            if (p.cells_off[s] < 0 || p.cells_off[s + 1] < p.cells_off[s]) {
                err = "cells_off must be non-negative and non-decreasing";
                return KVDEC_E_INVALID;
            }
        }
        // the dedup bitmap covers the records up to the largest valid cell
        // listed (entries are int32, so at most 2^31 cells), not the whole
        // capacity; compact_slot reports the entries out of range
        int64_t top = 0;
        for (int64_t i = p.cells_off[0]; i < p.cells_off[p.n_slots]; ++i) {
            const int64_t c = p.cells[i];
            if (c >= 0 && c < p.capacity_cells && c + 1 > top) top = c + 1;
        }
        std::vector<uint64_t> bitmap((size_t)ceil_div(std::max<int64_t>(top, 1), kTile) * (kTile / 64), 0);
        std::vector<int64_t> records;
        for (int s = 0; s < p.n_slots; ++s) {
            const int64_t b = p.cells_off[s], e = p.cells_off[s + 1];
            const size_t before = plan.cells.size();
            const int st = compact_slot(p.cells + b, e - b, p.capacity_cells, bitmap, records, plan.cells, err);
            if (st != KVDEC_OK) {
                err = "slot " + std::to_string(s) + ": " + err;
                return st;
            }
            plan.slots[s].first = (int64_t)before;
            plan.slots[s].n = (int64_t)(plan.cells.size() - before);
            plan.cells_off[s + 1] = (int64_t)plan.cells.size();
        }
    } else {
        for (int s = 0; s < p.n_slots; ++s) {
            const int64_t b = p.cell_begin ? p.cell_begin[s] : 0;
            const int64_t n = p.n_occupied[s];
            if (b < 0 || n < 0 || b > p.capacity_cells || n > p.capacity_cells - b) {
                err = "slot " + std::to_string(s) + ": cells from " + std::to_string(b) + ", " + std::to_string(n) +
                      " of them, outside [0, capacity)";
                return KVDEC_E_RANGE;
            }
            plan.slots[s].first = b;
            plan.slots[s].n = n;
        }
    }

    // ---- split decomposition: tiles of every (slot, KV head) spread over
    // about two workgroups per compute unit.  Split boundaries fall on
    // multiples of 32 positions for the vector-ALU kernel (a split may end
    // inside a tile), on whole tiles for the matrix-core kernel.
    bool mfma = uses_matrix_cores(group, n_q, p.head_dim);
    int64_t total_tiles = 0;
    for (auto& sa : plan.slots) {
        const int64_t t = ceil_div(sa.n, kTile);
        if (t > (1 << 24)) {
            err = "slot too long";
            return KVDEC_E_UNSUPPORTED;
        }
        total_tiles += t * p.n_kv_heads;
    }
    // Workgroups when every (slot, KV head) is cut into splits of at most
    // `cells` positions, and whether that is 3/4 to one workgroup per CU.
    auto wgs_for = [&](int64_t cells) {
        int64_t w = 0;
        for (auto& sa : plan.slots) w += std::max<int64_t>(1, ceil_div(sa.n, cells)) * p.n_kv_heads;
        return w;
    };
    auto one_round = [&](int64_t w) { return 4 * w >= 3 * (int64_t)n_cu && w <= n_cu; };
    const bool auto_split = p.split_cells == 0 && p.tiles_per_split == 0;
    if (p.kernel != KVDEC_KERNEL_AUTO && p.kernel != KVDEC_KERNEL_STREAMED && p.kernel != KVDEC_KERNEL_ONESHOT) {
        err = "kernel must be KVDEC_KERNEL_AUTO, _STREAMED or _ONESHOT";
        return KVDEC_E_INVALID;
    }
    // One-shot kernel: head_dim 128, f16 K and V, G <= 5, one query row,
    // contiguous cells, splits of at most kOneShotCells.  Chosen when one
    // split per compute unit covers the cache: the split length that spreads
    // every (slot, KV head) over the compute units, on 32-cell boundaries,
    // at least 64 cells.
    constexpr int64_t kOneShotCells = 448;
    const bool oneshot_ok = !mfma && !indirect && n_q == 1 && group <= 5 && p.head_dim == 128 &&
                            p.k_type == KVDEC_F16 && p.v_type == KVDEC_F16;
    int64_t oneshot_cells = 0;
    if (oneshot_ok && p.kernel != KVDEC_KERNEL_STREAMED) {
        if (p.split_cells > 0 || p.tiles_per_split > 0) {
            oneshot_cells = p.split_cells > 0 ? p.split_cells : (int64_t)p.tiles_per_split * kTile;
        } else {
            // the shortest split (from the even share upward, on 32-cell
            // boundaries) for which every (slot, KV head) fits in one round
            int64_t cells = 0;
            for (auto& sa : plan.slots) cells += sa.n;
            int64_t c = std::max<int64_t>(64, ceil_div(ceil_div(cells * p.n_kv_heads, n_cu), kSplitUnit) * kSplitUnit);
            while (c < kOneShotCells && wgs_for(c) > std::max<int64_t>(n_cu, p.n_kv_heads)) c += kSplitUnit;
            oneshot_cells = c;
        }
        const bool fits = oneshot_cells <= kOneShotCells && wgs_for(oneshot_cells) <= std::max<int64_t>(n_cu, p.n_kv_heads);
        if (p.kernel == KVDEC_KERNEL_AUTO && !(auto_split && fits)) oneshot_cells = 0;
        if (p.kernel == KVDEC_KERNEL_ONESHOT && oneshot_cells > kOneShotCells) {
            err = "the one-shot kernel needs splits of at most 448 cells";
            return KVDEC_E_UNSUPPORTED;
        }
    }
    if (p.kernel == KVDEC_KERNEL_ONESHOT && !oneshot_ok) {
        err = "the one-shot kernel needs head_dim 128, f16 K and V, G <= 5, one query row and contiguous cells";
        return KVDEC_E_UNSUPPORTED;
    }
    // Five f16 query rows at head_dim 128 over short contexts (splits of at
    // most two tiles at two workgroups per CU) run faster on the matrix-core
    // kernel with four-tile splits (16384-cell layer 22.6 -> 20.8 us); long
    // splits stay on the vector-ALU kernel, whose LDS staging wins there.
    if (!mfma && oneshot_cells == 0 && p.kernel == KVDEC_KERNEL_AUTO && group == 5 && n_q == 1 &&
        p.head_dim == 128 && p.k_type == KVDEC_F16 && p.v_type == KVDEC_F16 && auto_split &&
        ceil_div(total_tiles, 2 * (int64_t)n_cu) <= 2 && one_round(wgs_for(4 * kTile)))
        mfma = true;
    plan.mfma = mfma;
    const int rec_rows = record_rows_of(mfma, group, n_q);
    plan.rec_rows = rec_rows;
    const bool staged = p.k_type == KVDEC_F16 && p.v_type == KVDEC_F16 && !mfma;
    const int64_t unit = mfma ? kTile : kSplitUnit;
    const int64_t upt = kTile / unit;  // units per tile
    plan.split_unit = (int32_t)unit;
    if (p.split_cells < 0 || p.split_cells % kSplitUnit != 0) {
        err = "split_cells must be a non-negative multiple of 32";
        return KVDEC_E_INVALID;
    }
    for (auto& sa : plan.slots) sa.n_units = (int32_t)ceil_div(sa.n, unit);
    plan.n_tiles = total_tiles;
    int64_t ups = 0;  // units per split
    if (oneshot_cells > 0) {
        ups = ceil_div(oneshot_cells, unit);
        plan.waves = 8;
    } else if (p.split_cells > 0) {
        ups = ceil_div((int64_t)p.split_cells, unit);
    } else if (p.tiles_per_split > 0) {
        ups = (int64_t)p.tiles_per_split * upt;
    } else {
        int64_t tps = std::max<int64_t>(1, ceil_div(total_tiles, 2 * (int64_t)n_cu));
        // Once splits are eight tiles or longer: one split per compute unit
        // when that covers every (slot, KV head) -- f16 caches on the
        // vector-ALU kernel stage the next step of a long split through LDS,
        // and the matrix-core kernel prefetches a step ahead, so one
        // workgroup keeps enough bytes in flight for its compute unit (on
        // the matrix-core kernel only for rows of 384 bytes or more per cell:
        // 4-bit K and V measured 5% faster at two workgroups per unit) --
        // else about eight splits per compute unit, which the dispatcher
        // balances (a second partial round of long splits would leave most
        // of the chip idle at the end).
        const bool heavy_rows = row_bytes(p.k_type, p.head_dim) + row_bytes(p.v_type, p.head_dim) >= 384;
        if ((staged || (mfma && heavy_rows)) && tps >= 8) {
            const int64_t one = ceil_div(total_tiles, (int64_t)n_cu);
            tps = wgs_for(one * kTile) <= n_cu ? one : std::max<int64_t>(8, ceil_div(total_tiles, 8 * (int64_t)n_cu));
        }
        ups = tps * upt;
        // Short contexts (splits of at most two steps at two workgroups per
        // compute unit): one eight-wave workgroup per compute unit instead,
        // each split exactly two of its steps.  The same waves are in flight,
        // and a (slot, KV head) leaves half as many records to merge.
        const int64_t step4 = 4 * (64 / (p.head_dim / 16)) * 4;  // cells per 4-wave step (G <= 5)
        const int64_t cells8 = 2 * 2 * step4;  // two 8-wave steps
        if (staged && p.head_dim <= 128 && group <= 5 && tps * kTile <= 2 * step4 && one_round(wgs_for(cells8))) {
            plan.waves = 8;
            ups = cells8 / unit;
        }
        // The matrix-core kernel likewise: short splits of at most two tiles
        // double to four when that still gives 3/4 to one workgroup per
        // compute unit (fewer, wider records to merge; 4-query Qwen3-8B-shaped
        // layer 28.5 -> 26.6 us).  With 16-row records at head_dim 128 the
        // four tiles are two steps of an eight-wave workgroup, whose 512
        // threads also publish and merge the wider records in fewer passes
        // (4-query layer 25.4 -> 24.8 us, 16-head groups 24.7 -> 23.7 us;
        // 8-row records measured 3% slower, so they keep four waves).
        if (mfma && tps <= 2 && one_round(wgs_for(4 * kTile))) {
            ups = 4 * upt;
            if (rec_rows == 16 && p.head_dim == 128) plan.waves = 8;
        }
    }
    int64_t wgs = 0;
    plan.max_tiles_per_split = 0;
    plan.max_split_cells = 0;
    for (auto& sa : plan.slots) {
        const int64_t ns = std::max<int64_t>(1, ceil_div(sa.n_units, ups));
        sa.n_splits = (int32_t)ns;
        // A device-built plan's entries are a record budget: its splits are
        // fixed runs of ups units (the last one ragged; positions past the
        // slot's entries are clipped), so the records in use split the same
        // way -- and give the same result, bit for bit -- whatever the budget.
        if (device_cells) sa.n_units = ns * ups;
        sa.wg_begin = (int32_t)wgs;
        sa.part_begin = (int32_t)wgs;
        sa.to_acc = 0;
        wgs += ns * p.n_kv_heads;
        if (wgs > (1ll << 30)) {
            err = "too many workgroups";
            return KVDEC_E_UNSUPPORTED;
        }
        const int64_t longest = std::min<int64_t>(sa.n, ceil_div(sa.n_units, ns) * unit);
        plan.max_split_cells = std::max<int32_t>(plan.max_split_cells, (int32_t)longest);
    }
    plan.max_tiles_per_split = (int32_t)ceil_div((int64_t)plan.max_split_cells, kTile);
    if (oneshot_cells > 0) {
        // 8-cell loads per lane: a wave takes an even number of cells, at
        // most 8 of them per load
        const int64_t cw = (ceil_div(plan.max_split_cells, 8) + 1) & ~1ll;
        const int64_t jm = ceil_div(cw, 8);
        plan.oneshot = jm <= 2 ? 2 : (jm <= 4 ? 4 : 7);
        // Splits take every n_splits-th 32-cell unit rather than a
        // contiguous run, so at any moment the workgroups read neighbouring
        // rows of the cache (a plain read of the Qwen3-8B-shaped layer's
        // bytes in this pattern: 11.30 -> 10.75 us).  A split of a slot then
        // holds at most one more unit than another, as with contiguous runs.
        plan.interleave = true;
    }
    plan.n_workgroups = (int32_t)wgs;
    plan.n_part_records = (int32_t)wgs;
    int64_t clusters = 0;
    for (auto& sa : plan.slots) {
        sa.chunk = merge_chunk_for(p.head_dim, rec_rows, sa.n_splits);
        sa.n_clusters = merge_clusters(sa.n_splits, sa.chunk);
        sa.cl_begin = (int32_t)clusters;
        if (sa.n_clusters > 1) clusters += (int64_t)sa.n_clusters * p.n_kv_heads;
    }

    // ---- host tail
    plan.has_tail = has_tail;
    if (p.tail_zero_copy != 0 && p.tail_zero_copy != 1) {
        err = "tail_zero_copy must be 0 or 1";
        return KVDEC_E_INVALID;
    }
    plan.tail_zero_copy = has_tail && p.tail_zero_copy == 1;
    int64_t part_capacity = wgs;
    if (has_tail) {
        plan.tail_capacity = p.tail_capacity_cells;
        // 32768-cell chunks: small copies leave the copy engines below the
        // link rate (a 26960-cell f16 tail, 8 KV heads x 128, measured 65% of
        // it at 2048-cell chunks, 86% at 8192, 92% at 16384, 96% whole)
        plan.chunk_cells = p.tail_chunk_cells ? p.tail_chunk_cells : 32768;
        plan.ring_depth = p.tail_ring_depth ? p.tail_ring_depth : 4;
        if (plan.chunk_cells < kTile || plan.chunk_cells % kTile != 0 || plan.ring_depth < 2 || plan.ring_depth > 16 ||
            plan.tail_capacity < 0) {
            err = "tail_chunk_cells must be a positive multiple of 128 and tail_ring_depth in 2..16";
            return KVDEC_E_INVALID;
        }
        plan.tail_begin.assign(p.n_slots, 0);
        plan.tail_n.assign(p.n_slots, 0);
        plan.n_tail_chunks = 0;
        for (int s = 0; s < p.n_slots; ++s) {
            const int64_t b = p.tail_begin ? p.tail_begin[s] : 0;
            const int64_t n = p.n_tail[s];
            if (b < 0 || n < 0 || b > plan.tail_capacity || n > plan.tail_capacity - b) {
                err = "slot " + std::to_string(s) + ": tail cells outside [0, tail_capacity_cells)";
                return KVDEC_E_RANGE;
            }
            plan.tail_begin[s] = b;
            plan.tail_n[s] = n;
            const int64_t chunks = ceil_div(n, plan.chunk_cells);
            plan.n_tail_chunks += chunks;
            plan.slots[s].to_acc = chunks > 0 ? 1 : 0;
        }
        // a call never holds more chunks in flight than it has
        plan.ring_depth = (int32_t)std::max<int64_t>(1, std::min<int64_t>(plan.ring_depth, plan.n_tail_chunks));
        const int64_t chunk_tiles = plan.chunk_cells / kTile;
        const int64_t ctps = std::max<int64_t>(1, ceil_div(chunk_tiles * p.n_kv_heads, 2 * (int64_t)n_cu));
        plan.chunk_tiles_per_split = (int32_t)ctps;
        plan.chunk_splits = (int32_t)std::max<int64_t>(1, ceil_div(chunk_tiles, ctps));
        part_capacity = std::max<int64_t>(part_capacity, (int64_t)plan.chunk_splits * p.n_kv_heads);
        const int cc = merge_clusters(plan.chunk_splits, merge_chunk_for(p.head_dim, rec_rows, plan.chunk_splits));
        if (cc > 1) clusters = std::max<int64_t>(clusters, (int64_t)cc * p.n_kv_heads);
    }
    // cluster records follow the split records
    plan.crec_base = (int32_t)part_capacity;
    plan.n_cluster_capacity = (int32_t)clusters;
    part_capacity += clusters;
    plan.n_part_capacity = (int32_t)part_capacity;

    // ---- workspace layout
    const size_t D = (size_t)p.head_dim;
    size_t off = 0;
    plan.off_tickets = off;
    // a fixed-size ticket area (a multiple of it for very many tickets), so
    // that plans can take turns on one workspace: every call leaves the area
    // zero, and no plan writes records where another keeps its tickets
    const size_t ticket_need = sizeof(uint32_t) * kTicketStride * ((size_t)p.n_slots * p.n_kv_heads + (size_t)clusters);
    plan.ticket_bytes = align_up(std::max<size_t>(ticket_need, 1), KVDEC_TICKET_AREA_BYTES);
    off += plan.ticket_bytes;
    plan.off_parts = off;
    plan.parts_o_bytes = sizeof(float) * (size_t)part_capacity * rec_rows * D;
    if (plan.parts_o_bytes >= (1ull << 31)) {
        err = "too many split records";
        return KVDEC_E_UNSUPPORTED;
    }
    off = align_up(off + plan.parts_o_bytes, 256);
    plan.off_parts_m = off;
    off = align_up(off + sizeof(float) * (size_t)part_capacity * rec_rows, 256);
    plan.off_parts_l = off;
    off = align_up(off + sizeof(float) * (size_t)part_capacity * rec_rows, 256);
    if (has_tail) {
        const size_t rows = (size_t)p.n_slots * n_q * p.n_q_heads;
        plan.off_acc0 = off;
        off = align_up(off + sizeof(float) * (size_t)acc_floats((int64_t)rows, (int64_t)D), 256);
        plan.off_acc1 = off;
        off = align_up(off + sizeof(float) * (size_t)acc_floats((int64_t)rows, (int64_t)D), 256);
        const size_t cc = (size_t)plan.chunk_cells * p.n_kv_heads;
        plan.ring_k = 0;
        size_t r = align_up(cc * (size_t)row_bytes(p.k_type, p.head_dim), 256);
        plan.ring_v = r;
        r = align_up(r + cc * (size_t)row_bytes(p.v_type, p.head_dim), 256);
        plan.ring_ks = r;
        if (is_scaled(p.k_type)) r = align_up(r + cc * (D / kBlock) * 2, 256);
        plan.ring_vs = r;
        if (is_scaled(p.v_type)) r = align_up(r + cc * (D / kBlock) * 2, 256);
        plan.ring_slot_bytes = r;
        plan.off_ring = off;
        if (!plan.tail_zero_copy) off += r * (size_t)plan.ring_depth;  // in-place reads need no ring
    }
    if (device_cells) {
        // build area of kvdec_build_cells: per-slot bitmaps (4 words per
        // record), the present records of each slot, counters
        plan.bm_words_per_slot = 4 * ceil_div(std::max<int64_t>(p.capacity_cells, 1), kTile);
        plan.off_build_bitmap = off;
        off = align_up(off + sizeof(uint32_t) * (size_t)p.n_slots * plan.bm_words_per_slot, 256);
        plan.off_build_list = off;
        off = align_up(off + sizeof(int32_t) * (size_t)std::max<int64_t>(1, plan.n_device_entries / kTile), 256);
        plan.off_build_count = off;
        off = align_up(off + sizeof(int32_t) * ((size_t)p.n_slots + 1), 256);
    }
    plan.workspace_bytes = align_up(std::max<size_t>(off, 256), 256);
    return KVDEC_OK;
}

}  // namespace kvdec

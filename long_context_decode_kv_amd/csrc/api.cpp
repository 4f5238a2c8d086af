// C-ABI entry points of libkvdec: plan construction, argument validation,
// kernel dispatch and the pinned-host tail streamer.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

#ifdef KVDEC_PHASE_TRACE
// Diagnostic build: where the next launches write their phase stamps.
unsigned long long* g_trace = nullptr;
#endif

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

int device_fail(hipError_t e, const char* what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return KVDEC_E_DEVICE;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Fill the per-launch fields shared by the resident and the tail launches.
void common_args(const kvdec_plan_t& p, const kvdec_io& io, kvdec::SplitArgs& a) {
    std::memset(&a, 0, sizeof(a));
    a.q = io.q;
    a.scale_log2 = p.scale * 1.4426950408889634f;
    a.n_q_heads = p.n_q_heads;
    a.n_kv_heads = p.n_kv_heads;
    a.out = io.out;
    a.lse = io.lse;
    a.pm = io.part_m;
    a.pl = io.part_l;
    a.po = io.part_o;
    a.acc_rows = p.n_slots * p.n_q * p.n_q_heads;
    a.n_q = p.n_q;
    a.group = p.group;
    a.split_unit = p.split_unit;
    a.waves = p.waves;
    a.oneshot = p.oneshot;
    a.interleave = p.interleave ? 1 : 0;
    // positions are used with several query rows per slot only
    a.q_pos = p.n_q > 1 ? io.q_pos : nullptr;
    a.cell_pos = p.n_q > 1 ? io.cell_pos : nullptr;
    a.pos_offset = 0;
#ifdef KVDEC_PHASE_TRACE
    a.trace = g_trace;
#endif
}

}  // namespace

#ifdef KVDEC_FAULT_INJECTION
namespace kvdec {
bool fi_fail_copy();
bool fi_fail_launch();
int fi_delay(void* stream);
}  // namespace kvdec
#endif

namespace {

// Host-to-device copy of tail rows (a test build can make one fail without
// enqueueing it).
hipError_t tail_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
#ifdef KVDEC_FAULT_INJECTION
    if (kvdec::fi_fail_copy()) return hipErrorUnknown;
#endif
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s);
}

// n events for the tail stream, kept per host thread and device and reused
// from call to call rather than created and destroyed each time.  Reuse is
// safe: a stream wait waits for the event's record that preceded it, and
// every wait a call enqueues follows a record the same call made.  The
// events live until the process ends.
hipError_t tail_events(int n, hipEvent_t* out) {
    struct Pool {
        int device;
        std::vector<hipEvent_t> ev;
    };
    thread_local std::vector<Pool> pools;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Pool* pool = nullptr;
    for (auto& pl : pools)
        if (pl.device == dev) pool = &pl;
    if (!pool) {
        pools.push_back(Pool{dev, {}});
        pool = &pools.back();
    }
    while ((int)pool->ev.size() < n) {
        hipEvent_t ev = nullptr;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return e;
        pool->ev.push_back(ev);
    }
    for (int i = 0; i < n; ++i) out[i] = pool->ev[i];
    return hipSuccess;
}

// Split-kernel launch for the plan (a test build can make one fail without
// enqueueing it).
int launch(const kvdec_plan_t& p, const kvdec::SplitArgs& a, void* stream) {
#ifdef KVDEC_FAULT_INJECTION
    if (kvdec::fi_fail_launch()) return (int)hipErrorLaunchFailure;
#endif
    return kvdec::launch_split(p.head_dim, p.group, p.n_q, p.k_type, p.v_type, p.mfma, a, stream);
}

// The checks of kvdec_io against a plan shared by kvdec_attend and
// kvdec_attend_static (everything but the workspace); no device calls.
int check_io(const kvdec_plan_t& p, const kvdec_io* io) {
    const int D = p.head_dim;
    if (!io->q || !aligned(io->q, 8)) return fail(KVDEC_E_INVALID, "q must be non-null and 8-byte aligned");
    // With no device cells (capacity_cells 0) no split holds a cell or a plan
    // entry, so no kernel reads k, v or their scales: they may be null.
    const bool cells = p.capacity > 0;
    if (cells && (!io->k || !io->v))
        return fail(KVDEC_E_INVALID, "k and v must be non-null when capacity_cells > 0");
    const int64_t krow = kvdec::row_bytes(p.k_type, D), vrow = kvdec::row_bytes(p.v_type, D);
    const int64_t k_cs = io->k_cell_stride ? io->k_cell_stride : krow * p.n_kv_heads;
    const int64_t k_hs = io->k_head_stride ? io->k_head_stride : krow;
    const int64_t v_cs = io->v_cell_stride ? io->v_cell_stride : vrow * p.n_kv_heads;
    const int64_t v_hs = io->v_head_stride ? io->v_head_stride : vrow;
    const size_t kal = p.k_type == KVDEC_Q4_B32 ? 8 : 16, val = p.v_type == KVDEC_Q4_B32 ? 8 : 16;
    if (!aligned(io->k, kal) || k_cs % (int64_t)kal || k_hs % (int64_t)kal || k_cs < 0 || k_hs < 0)
        return fail(KVDEC_E_INVALID, "k pointer and strides must be non-negative multiples of the row load size");
    if (!aligned(io->v, val) || v_cs % (int64_t)val || v_hs % (int64_t)val || v_cs < 0 || v_hs < 0)
        return fail(KVDEC_E_INVALID, "v pointer and strides must be non-negative multiples of the row load size");
    // one row of scales (head_dim/32 f16 values) is read with one load
    const size_t sal = std::min<size_t>(16, (size_t)p.head_dim / 16);
    if (kvdec::is_scaled(p.k_type) && ((cells && !io->k_scales) || !aligned(io->k_scales, sal)))
        return fail(KVDEC_E_INVALID, "k_scales required for block-scaled K, aligned to min(16, head_dim/16) bytes");
    if (kvdec::is_scaled(p.v_type) && ((cells && !io->v_scales) || !aligned(io->v_scales, sal)))
        return fail(KVDEC_E_INVALID, "v_scales required for block-scaled V, aligned to min(16, head_dim/16) bytes");
    // (a plan without entries leaves every slot empty: nothing reads plan_cells)
    const int64_t n_entries = p.device_cells ? p.n_device_entries : (int64_t)p.cells.size();
    if (p.indirect && n_entries > 0 && !io->plan_cells)
        return fail(KVDEC_E_INVALID, "indirect plan needs plan_cells on the device");
    const bool any_part = io->part_m || io->part_l || io->part_o;
    const bool all_part = io->part_m && io->part_l && io->part_o;
    if (any_part && !all_part) return fail(KVDEC_E_INVALID, "part_m, part_l and part_o go together");
    if (!io->out && !all_part) return fail(KVDEC_E_INVALID, "give out or the partial triple");
    if (!aligned(io->out, 16) || !aligned(io->part_o, 16) || !aligned(io->lse, 4) || !aligned(io->part_m, 4) ||
        !aligned(io->part_l, 4))
        return fail(KVDEC_E_INVALID, "out and part_o must be 16-byte aligned, lse / part_m / part_l 4-byte aligned");
    if (p.has_tail) {
        if (!io->k_tail || !io->v_tail) return fail(KVDEC_E_INVALID, "the plan has a tail: k_tail and v_tail needed");
        if ((kvdec::is_scaled(p.k_type) && !io->k_tail_scales) || (kvdec::is_scaled(p.v_type) && !io->v_tail_scales))
            return fail(KVDEC_E_INVALID, "tail scales needed for block-scaled kinds");
    }
    if (p.n_q > 1 && (!io->q_pos || !aligned(io->q_pos, 4)))
        return fail(KVDEC_E_INVALID, "several query rows per slot need q_pos (device int32 [n_slots][n_queries])");
    if (!aligned(io->cell_pos, 4)) return fail(KVDEC_E_INVALID, "cell_pos must be 4-byte aligned");
    if (io->live_records && (!p.indirect || !aligned(io->live_records, 4)))
        return fail(KVDEC_E_INVALID, "live_records needs an indirect plan and 4-byte alignment");
    if (!kvdec::split_instance_exists(D, p.group, p.n_q, p.k_type, p.v_type, p.mfma))
        return fail(KVDEC_E_UNSUPPORTED, "no kernel for this configuration");
    return KVDEC_OK;
}

// Enqueue the evaluation on a checked plan and io.  ws: the plan's workspace
// layout starts here; tickets: the merge ticket words (slot tickets, then
// cluster tickets), or NULL for the plan's own ticket region inside ws.
int attend_checked(const kvdec_plan_t& p, const kvdec_io* io, uint8_t* ws, uint32_t* tickets, void* stream,
                   void* copy_stream) {
    const int D = p.head_dim;
    const int64_t krow = kvdec::row_bytes(p.k_type, D), vrow = kvdec::row_bytes(p.v_type, D);
    const int64_t k_cs = io->k_cell_stride ? io->k_cell_stride : krow * p.n_kv_heads;
    const int64_t k_hs = io->k_head_stride ? io->k_head_stride : krow;
    const int64_t v_cs = io->v_cell_stride ? io->v_cell_stride : vrow * p.n_kv_heads;
    const int64_t v_hs = io->v_head_stride ? io->v_head_stride : vrow;
    const size_t kal = p.k_type == KVDEC_Q4_B32 ? 8 : 16, val = p.v_type == KVDEC_Q4_B32 ? 8 : 16;
    const size_t sal = std::min<size_t>(16, (size_t)p.head_dim / 16);
    kvdec::SplitArgs a;
    common_args(p, *io, a);
    a.k = static_cast<const uint8_t*>(io->k);
    a.v = static_cast<const uint8_t*>(io->v);
    a.ks = static_cast<const uint16_t*>(io->k_scales);
    a.vs = static_cast<const uint16_t*>(io->v_scales);
    a.k_cs = k_cs;
    a.k_hs = k_hs;
    a.v_cs = v_cs;
    a.v_hs = v_hs;
    a.plan = p.indirect ? io->plan_cells : nullptr;
    a.live_records = p.indirect ? io->live_records : nullptr;
    a.capacity = p.capacity;
    a.part_o = reinterpret_cast<float*>(ws + p.off_parts);
    a.part_m = reinterpret_cast<float*>(ws + p.off_parts_m);
    a.part_l = reinterpret_cast<float*>(ws + p.off_parts_l);
    a.part_o_bytes = (int64_t)p.parts_o_bytes;
    a.tickets = tickets ? tickets : reinterpret_cast<uint32_t*>(ws + p.off_tickets);
    a.ctickets = a.tickets + (size_t)kvdec::kTicketStride * p.n_slots * p.n_kv_heads;
    a.crec_base = p.crec_base;
    a.n_slots = p.n_slots;
    a.slot_base = 0;
    a.n_workgroups = p.n_workgroups;
    for (int s = 0; s < p.n_slots; ++s) a.slot[s] = p.slots[s];
    float* acc[2] = {nullptr, nullptr};
    if (p.has_tail) {
        acc[0] = reinterpret_cast<float*>(ws + p.off_acc0);
        acc[1] = reinterpret_cast<float*>(ws + p.off_acc1);
        a.acc_out = acc[0];
    }

    if (!p.has_tail) {
        const int e = launch(p, a, stream);
        if (e != hipSuccess) return device_fail((hipError_t)e, "split kernel launch");
        return KVDEC_OK;
    }

    // ---- resident window + pinned-host tail.
    // The window launch writes each tailed slot's partial to acc0; then every
    // tail chunk is copied host -> device into a ring slot on copy_stream and
    // attended on `stream`, its last workgroup merging the running partial
    // (acc0 <-> acc1 ping-pong) and, on the slot's last chunk, writing the
    // outputs.  Ring reuse is ordered by events: the copy into a ring slot
    // waits until the kernel that read the slot's previous chunk has finished.
    // With tail_zero_copy the chunk kernels read the host arrays in place and
    // nothing is copied.
    hipStream_t cs = static_cast<hipStream_t>(copy_stream ? copy_stream : stream);
    hipStream_t ks = static_cast<hipStream_t>(stream);
    const bool zc = p.tail_zero_copy;
    const int depth = zc ? 0 : p.ring_depth;
    hipEvent_t ev_start = nullptr, ev_landed[16] = {}, ev_free[16] = {};
    const uint8_t* hk = static_cast<const uint8_t*>(io->k_tail);
    const uint8_t* hv = static_cast<const uint8_t*>(io->v_tail);
    const uint8_t* hks = static_cast<const uint8_t*>(io->k_tail_scales);
    const uint8_t* hvs = static_cast<const uint8_t*>(io->v_tail_scales);
    hipError_t e = hipSuccess;
    if (zc) {
        if (!aligned(hk, kal) || !aligned(hv, val) || !aligned(hks, sal) || !aligned(hvs, sal))
            return fail(KVDEC_E_INVALID, "tail arrays read in place must be aligned like device K / V / scales");
        // device addresses of the pinned host arrays
        auto mapped = [](const uint8_t*& ptr) -> bool {
            if (!ptr) return true;
            hipPointerAttribute_t at;
            if (hipPointerGetAttributes(&at, ptr) != hipSuccess || !at.devicePointer) {
                (void)hipGetLastError();
                return false;
            }
            ptr = static_cast<const uint8_t*>(at.devicePointer);
            return true;
        };
        if (!mapped(hk) || !mapped(hv) || !mapped(hks) || !mapped(hvs))
            return fail(KVDEC_E_INVALID, "tail_zero_copy needs device-mapped pinned host tail arrays");
    } else {
        hipEvent_t ev[1 + 2 * 16];
        e = tail_events(1 + 2 * depth, ev);
        if (e != hipSuccess) return device_fail(e, "hipEventCreate");
        ev_start = ev[0];
        for (int i = 0; i < depth; ++i) {
            ev_landed[i] = ev[1 + i];
            ev_free[i] = ev[1 + depth + i];
        }
        // Copies start only after the work that may still read the ring:
        // everything already on `stream` (an earlier call on this workspace),
        // or the caller's copy_after event.
        if (io->copy_after) {
            if (cs != ks) e = hipStreamWaitEvent(cs, static_cast<hipEvent_t>(io->copy_after), 0);
        } else {
            e = hipEventRecord(ev_start, ks);
            if (e == hipSuccess && cs != ks) e = hipStreamWaitEvent(cs, ev_start, 0);
        }
        if (e != hipSuccess) return device_fail(e, "stream ordering");
    }
    int le = launch(p, a, stream);
    if (le != hipSuccess) return device_fail((hipError_t)le, "window kernel launch");

    const int64_t krow_b = kvdec::row_bytes(p.k_type, D) * p.n_kv_heads;
    const int64_t vrow_b = kvdec::row_bytes(p.v_type, D) * p.n_kv_heads;
    const int64_t srow_b = (int64_t)(D / kvdec::kBlock) * 2 * p.n_kv_heads;
    int64_t chunk_no = 0;
    for (int s = 0; s < p.n_slots && e == hipSuccess; ++s) {
        const int64_t n = p.tail_n[s];
        const int64_t n_chunks = (n + p.chunk_cells - 1) / p.chunk_cells;
        for (int64_t c = 0; c < n_chunks; ++c, ++chunk_no) {
            const int64_t c0 = p.tail_begin[s] + c * p.chunk_cells;
            const int64_t nc = std::min<int64_t>(p.chunk_cells, n - c * p.chunk_cells);
            const int r = zc ? 0 : (int)(chunk_no % depth);
            const uint8_t *ck, *cv, *cks, *cvs;  // the chunk's rows on the device
            if (zc) {
                ck = hk + c0 * krow_b;
                cv = hv + c0 * vrow_b;
                cks = hks ? hks + c0 * srow_b : nullptr;
                cvs = hvs ? hvs + c0 * srow_b : nullptr;
            } else {
                uint8_t* slot = ws + p.off_ring + (size_t)r * p.ring_slot_bytes;
                if (chunk_no >= depth) e = hipStreamWaitEvent(cs, ev_free[r], 0);
                if (e == hipSuccess)
                    e = tail_copy(slot + p.ring_k, hk + c0 * krow_b, nc * krow_b, cs);
                if (e == hipSuccess)
                    e = tail_copy(slot + p.ring_v, hv + c0 * vrow_b, nc * vrow_b, cs);
                if (e == hipSuccess && kvdec::is_scaled(p.k_type))
                    e = tail_copy(slot + p.ring_ks, hks + c0 * srow_b, nc * srow_b, cs);
                if (e == hipSuccess && kvdec::is_scaled(p.v_type))
                    e = tail_copy(slot + p.ring_vs, hvs + c0 * srow_b, nc * srow_b, cs);
                if (e == hipSuccess) e = hipEventRecord(ev_landed[r], cs);
                if (e == hipSuccess && cs != ks) e = hipStreamWaitEvent(ks, ev_landed[r], 0);
                if (e != hipSuccess) break;
                ck = slot + p.ring_k;
                cv = slot + p.ring_v;
                cks = slot + p.ring_ks;
                cvs = slot + p.ring_vs;
            }

            kvdec::SplitArgs t;
            common_args(p, *io, t);
            t.k = ck;
            t.v = cv;
            t.ks = reinterpret_cast<const uint16_t*>(cks);
            t.vs = reinterpret_cast<const uint16_t*>(cvs);
            t.k_hs = kvdec::row_bytes(p.k_type, D);
            t.k_cs = krow_b;
            t.v_hs = kvdec::row_bytes(p.v_type, D);
            t.v_cs = vrow_b;
            t.plan = nullptr;
            t.capacity = nc;
            t.part_o = a.part_o;
            t.part_m = a.part_m;
            t.part_l = a.part_l;
            t.part_o_bytes = a.part_o_bytes;
            t.tickets = a.tickets;
            t.ctickets = a.ctickets;
            t.crec_base = a.crec_base;
            t.n_slots = 1;
            t.slot_base = s;
            const int32_t tiles = (int32_t)((nc + kvdec::kTile - 1) / kvdec::kTile);
            const int32_t splits = std::max<int32_t>(1, (tiles + p.chunk_tiles_per_split - 1) / p.chunk_tiles_per_split);
            t.slot[0].first = 0;
            t.slot[0].n = nc;
            t.slot[0].n_units = tiles;  // whole-tile splits
            t.split_unit = kvdec::kTile;
            t.waves = 4;
            t.oneshot = 0;
            t.interleave = 0;
            t.slot[0].n_splits = splits;
            t.slot[0].wg_begin = 0;
            t.slot[0].part_begin = 0;
            t.slot[0].to_acc = (c + 1 < n_chunks) ? 1 : 0;
            t.slot[0].chunk = kvdec::merge_chunk_for(D, p.rec_rows, splits);
            t.slot[0].n_clusters = kvdec::merge_clusters(splits, t.slot[0].chunk);
            t.slot[0].cl_begin = 0;
            // a tail cell's position is its index in the host tail
            t.cell_pos = nullptr;
            t.pos_offset = c0;
            t.n_workgroups = splits * p.n_kv_heads;
            t.acc_in = acc[c % 2];
            t.acc_out = acc[(c + 1) % 2];
#ifdef KVDEC_FAULT_INJECTION
            le = kvdec::fi_delay(stream);  // a slow reader of the ring slot
            if (le != hipSuccess) {
                e = (hipError_t)le;
                break;
            }
#endif
            le = launch(p, t, stream);
            if (le != hipSuccess) {
                e = (hipError_t)le;
                break;
            }
            if (!zc) e = hipEventRecord(ev_free[r], ks);
        }
    }
    if (e != hipSuccess) return device_fail(e, "tail streaming");
    return KVDEC_OK;
}

}  // namespace

extern "C" {

int kvdec_version(void) { return KVDEC_VERSION; }

#ifndef KVDEC_SOURCE_HASH
#error "KVDEC_SOURCE_HASH is set by the build script"
#endif
const char* kvdec_source_hash(void) { return KVDEC_SOURCE_HASH; }

const char* kvdec_strerror(int status) {
    switch (status) {
        case KVDEC_OK: return "ok";
        case KVDEC_E_INVALID: return "invalid argument";
        case KVDEC_E_RANGE: return "cell index out of range";
        case KVDEC_E_UNSUPPORTED: return "unsupported configuration";
        case KVDEC_E_WORKSPACE: return "workspace missing or too small";
        case KVDEC_E_NOMEM: return "host out of memory";
        case KVDEC_E_DEVICE: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* kvdec_last_error(void) { return g_last_error.c_str(); }

int kvdec_plan(const kvdec_problem* problem, int32_t n_cu, kvdec_plan_t** out, size_t* workspace_bytes) {
    g_last_error.clear();
    if (!problem || !out) return fail(KVDEC_E_INVALID, "problem and out must be non-null");
    *out = nullptr;
    if (n_cu < 0) return fail(KVDEC_E_INVALID, "n_cu must be >= 0");
    if (n_cu == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return device_fail(e, "hipGetDevice");
        e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
    }
    kvdec_plan_t* plan = nullptr;
    try {
        plan = new kvdec_plan_t();
        std::string err;
        const int st = kvdec::build_plan(*problem, n_cu, *plan, err);
        if (st != KVDEC_OK) {
            delete plan;
            return fail(st, err);
        }
    } catch (const std::bad_alloc&) {
        delete plan;
        return fail(KVDEC_E_NOMEM, "host allocation failed while planning");
    } catch (const std::length_error&) {
        delete plan;
        return fail(KVDEC_E_NOMEM, "host allocation too large while planning");
    }
    *out = plan;
    if (workspace_bytes) *workspace_bytes = plan->workspace_bytes;
    return KVDEC_OK;
}

int kvdec_plan_cells(const kvdec_plan_t* plan, int32_t* cells_out, int64_t* offsets_out, int64_t* n_entries) {
    if (!plan || !n_entries) return fail(KVDEC_E_INVALID, "plan and n_entries must be non-null");
    if (plan->device_cells) {
        if (cells_out) return fail(KVDEC_E_INVALID, "a device-built plan's entries come from kvdec_build_cells");
        *n_entries = plan->n_device_entries;
    } else {
        *n_entries = (int64_t)plan->cells.size();
        if (cells_out && !plan->cells.empty()) std::memcpy(cells_out, plan->cells.data(), plan->cells.size() * 4);
    }
    if (offsets_out) {
        for (int s = 0; s <= plan->n_slots; ++s)
            offsets_out[s] = plan->indirect ? plan->cells_off[s] : 0;
    }
    return KVDEC_OK;
}

int kvdec_plan_get_info(const kvdec_plan_t* plan, kvdec_plan_info* info) {
    if (!plan || !info) return fail(KVDEC_E_INVALID, "plan and info must be non-null");
    info->n_slots = plan->n_slots;
    info->group = plan->group;
    info->n_workgroups = plan->n_workgroups;
    info->tiles_per_split = plan->max_tiles_per_split;
    info->n_tiles = plan->n_tiles;
    info->n_entries = plan->device_cells ? plan->n_device_entries : (int64_t)plan->cells.size();
    info->n_tail_chunks = plan->n_tail_chunks;
    info->workspace_bytes = (int64_t)plan->workspace_bytes;
    info->n_queries = plan->n_q;
    info->matrix_cores = plan->mfma ? 1 : 0;
    info->split_cells = plan->max_split_cells;
    info->split_unit = plan->split_unit;
    info->waves = plan->waves;
    info->kernel = plan->mfma ? 0 : (plan->oneshot > 0 ? KVDEC_KERNEL_ONESHOT : KVDEC_KERNEL_STREAMED);
    info->split_interleave = plan->interleave ? plan->split_unit : 0;
    info->ticket_bytes = (int64_t)plan->ticket_bytes;
    return KVDEC_OK;
}

int kvdec_plan_splits(const kvdec_plan_t* plan, int64_t* splits_out, int64_t* n_splits) {
    if (!plan || !n_splits) return fail(KVDEC_E_INVALID, "plan and n_splits must be non-null");
    *n_splits = plan->n_workgroups;
    if (!splits_out) return KVDEC_OK;
    int64_t i = 0;
    for (int s = 0; s < plan->n_slots; ++s) {
        const kvdec::SlotArg& sa = plan->slots[s];
        for (int sp = 0; sp < sa.n_splits; ++sp)  // workgroup order: split-major
            for (int g = 0; g < plan->n_kv_heads; ++g) {
                int64_t p0, count;
                if (plan->interleave) {
                    // units sp, sp + n_splits, ...: first position and cell count
                    const int64_t nu = sp < sa.n_units ? (sa.n_units - sp + sa.n_splits - 1) / sa.n_splits : 0;
                    p0 = std::min<int64_t>((int64_t)sp * plan->split_unit, sa.n);
                    const int64_t last = nu > 0 ? ((int64_t)sp + (nu - 1) * sa.n_splits) * plan->split_unit : 0;
                    count = nu > 0 ? (nu - 1) * plan->split_unit + std::min<int64_t>(plan->split_unit, sa.n - last) : 0;
                } else {
                    const int64_t u0 = (int64_t)sp * sa.n_units / sa.n_splits;
                    const int64_t u1 = (int64_t)(sp + 1) * sa.n_units / sa.n_splits;
                    p0 = std::min<int64_t>(u0 * plan->split_unit, sa.n);
                    count = std::min<int64_t>(u1 * plan->split_unit, sa.n) - p0;
                }
                splits_out[4 * i + 0] = s;
                splits_out[4 * i + 1] = g;
                splits_out[4 * i + 2] = p0;
                splits_out[4 * i + 3] = count;
                ++i;
            }
    }
    return KVDEC_OK;
}

void kvdec_plan_free(kvdec_plan_t* plan) { delete plan; }

int kvdec_attend(const kvdec_plan_t* plan, const kvdec_io* io, void* workspace, size_t workspace_bytes, void* stream,
                 void* copy_stream) {
    g_last_error.clear();
    if (!plan || !io) return fail(KVDEC_E_INVALID, "plan and io must be non-null");
    const kvdec_plan_t& p = *plan;
    if (!workspace || workspace_bytes < p.workspace_bytes)
        return fail(KVDEC_E_WORKSPACE, "workspace needs " + std::to_string(p.workspace_bytes) + " bytes");
    if (!aligned(workspace, 256)) return fail(KVDEC_E_INVALID, "workspace must be 256-byte aligned");
    const int rc = check_io(p, io);
    if (rc != KVDEC_OK) return rc;
    return attend_checked(p, io, static_cast<uint8_t*>(workspace), nullptr, stream, copy_stream);
}

int kvdec_attend_static(const kvdec_plan_t* plan, const kvdec_io* io, void* stream) {
    g_last_error.clear();
    if (!plan || !io) return fail(KVDEC_E_INVALID, "plan and io must be non-null");
    const kvdec_plan_t& p = *plan;
    if (p.workspace_bytes > (size_t)KVDEC_STATIC_WORKSPACE_BYTES)
        return fail(KVDEC_E_WORKSPACE, "the plan's workspace needs " + std::to_string(p.workspace_bytes) +
                                           " bytes, the static scratch holds " +
                                           std::to_string((size_t)KVDEC_STATIC_WORKSPACE_BYTES));
    const int64_t n_tickets = (int64_t)p.n_slots * p.n_kv_heads + p.n_cluster_capacity;
    if ((int64_t)p.ticket_bytes > (int64_t)KVDEC_STATIC_TICKET_BYTES)
        return fail(KVDEC_E_WORKSPACE, "the plan needs " + std::to_string(n_tickets) +
                                           " merge tickets, the static scratch holds " +
                                           std::to_string(KVDEC_STATIC_TICKET_BYTES / (4 * kvdec::kTicketStride)));
    if (p.has_tail && !p.tail_zero_copy)
        return fail(KVDEC_E_UNSUPPORTED, "a copied tail needs per-call events; use tail_zero_copy or kvdec_attend");
    const int rc = check_io(p, io);
    if (rc != KVDEC_OK) return rc;
    uint8_t* base = nullptr;
    const hipError_t e = (hipError_t)kvdec::static_scratch(stream, reinterpret_cast<void**>(&base));
    if (e != hipSuccess) return device_fail(e, "static scratch set-up");
    return attend_checked(p, io, base + KVDEC_STATIC_TICKET_BYTES, reinterpret_cast<uint32_t*>(base), stream, nullptr);
}

int kvdec_build_cells(const kvdec_plan_t* plan, const int32_t* raw_cells, const int64_t* raw_off, int32_t* plan_cells,
                      int32_t* n_records, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!plan) return fail(KVDEC_E_INVALID, "plan must be non-null");
    const kvdec_plan_t& p = *plan;
    if (!p.device_cells) return fail(KVDEC_E_INVALID, "not a device-built plan (kvdec_problem.max_records)");
    if (!raw_cells || !raw_off || !aligned(raw_cells, 4) || !aligned(raw_off, 8))
        return fail(KVDEC_E_INVALID, "raw_cells (4-byte) and raw_off (8-byte) must be aligned device pointers");
    if (p.n_device_entries > 0 && (!plan_cells || !aligned(plan_cells, 4)))
        return fail(KVDEC_E_INVALID, "plan_cells must be a 4-byte aligned device pointer");
    if (!aligned(n_records, 4)) return fail(KVDEC_E_INVALID, "n_records must be 4-byte aligned");
    if (!workspace || workspace_bytes < p.workspace_bytes)
        return fail(KVDEC_E_WORKSPACE, "workspace needs " + std::to_string(p.workspace_bytes) + " bytes");
    if (!aligned(workspace, 256)) return fail(KVDEC_E_INVALID, "workspace must be 256-byte aligned");
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    kvdec::BuildArgs a;
    std::memset(&a, 0, sizeof(a));
    a.raw = raw_cells;
    a.raw_off = raw_off;
    a.bitmap = reinterpret_cast<uint32_t*>(ws + p.off_build_bitmap);
    a.list = reinterpret_cast<int32_t*>(ws + p.off_build_list);
    a.count = reinterpret_cast<int32_t*>(ws + p.off_build_count);
    a.n_records = n_records;
    a.out = plan_cells;
    a.capacity = p.capacity;
    a.words_per_slot = p.bm_words_per_slot;
    a.n_entries = p.n_device_entries;
    a.n_slots = p.n_slots;
    for (int s = 0; s < p.n_slots; ++s) {
        a.max_records[s] = p.max_records[s];
        a.list_off[s + 1] = a.list_off[s] + p.max_records[s];
        a.entry_off[s + 1] = p.cells_off[s + 1];
    }
    const int e = kvdec::launch_build_cells(a, stream);
    if (e != hipSuccess) return device_fail((hipError_t)e, "plan build kernels");
    return KVDEC_OK;
}

int kvdec_merge(int32_t n_parts, const kvdec_partial* parts, int64_t n_rows, int32_t head_dim, float* out, float* lse,
                float* merged_m, float* merged_l, float* merged_o, void* stream) {
    g_last_error.clear();
    if (n_parts < 1 || n_parts > kvdec::kMergeMaxParts || !parts)
        return fail(KVDEC_E_INVALID, "n_parts must be in 1..64 with a parts array");
    if (n_rows < 0 || n_rows > 0x7fffffff || head_dim < 1 || head_dim > 1024)
        return fail(KVDEC_E_INVALID, "n_rows must be in 0..2^31-1 and head_dim in 1..1024");
    const bool any_m = merged_m || merged_l || merged_o;
    const bool all_m = merged_m && merged_l && merged_o;
    if (any_m && !all_m) return fail(KVDEC_E_INVALID, "merged_m, merged_l and merged_o go together");
    if (!out && !lse && !all_m) return fail(KVDEC_E_INVALID, "no output given");
    kvdec::MergeArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int i = 0; i < n_parts; ++i) {
        if (!parts[i].m || !parts[i].l || !parts[i].o) return fail(KVDEC_E_INVALID, "partial with a null pointer");
        a.m[i] = parts[i].m;
        a.l[i] = parts[i].l;
        a.o[i] = parts[i].o;
    }
    a.n_parts = n_parts;
    a.head_dim = head_dim;
    a.n_rows = n_rows;
    a.out = out;
    a.lse = lse;
    a.mm = merged_m;
    a.ml = merged_l;
    a.mo = merged_o;
    if (n_rows == 0) return KVDEC_OK;
    const int e = kvdec::launch_merge(a, stream);
    if (e != hipSuccess) return device_fail((hipError_t)e, "merge kernel launch");
    return KVDEC_OK;
}

#ifdef KVDEC_PHASE_TRACE
// Diagnostic build only (libkvdec_trace.so): launches enqueued from now on
// write phase stamps to `buffer` (device memory, 32 uint64 per workgroup of
// the launch, workgroup b at 32 b), or stop when it is null.  Process-wide;
// a captured graph keeps the pointer it was captured with.
void kvdec_trace_configure(void* buffer) { g_trace = static_cast<unsigned long long*>(buffer); }
#endif

}  // extern "C"

// Split-KV decode kernels of libkvdec for gfx950 (MI355X), as templates over
// head_dim, GQA group and K / V storage kinds.  Included by the split_*.hip
// translation units, each of which instantiates one pair of storage kinds
// (so the instances compile in parallel), and by kernels.hip for the shared
// helpers.
//
// Split kernel.  One workgroup (4 or 8 waves) streams a contiguous range of
// positions of one (slot, KV head), cut on 32-cell boundaries, in steps where
// each lane holds 4 cells and each wave's cells spread over the step.  R
// consecutive lanes share one cell and split its head_dim
// elements into R slices of D/R; every 16-byte (8-byte for 4-bit rows) load
// of a wave covers whole 128-byte lines of consecutive cells, so the KV
// stream is read with coalesced 128-bit loads.  The G query rows of the KV
// head's group are held in every lane (f16-packed, its D/R slice only), so
// each K row fetched once serves all G query heads ("KVARN KV Performance
// optimizations", "What was implemented" item 6: decoded K/V reused across
// query rows).  Scores are reduced over the R lanes of a cell with DPP
// moves; each group of lanes that shares a cell stream keeps its own online
// softmax state (m, l, o), and the states are merged at the end of the split
// with the log-sum-exp rule, first across the wave, then across the waves
// through LDS.
//
// Partials are written as (m2 = running max in log2 units, l, o).  When a
// (slot, KV head) has several splits, the last workgroup to finish (atomic
// ticket in the workspace) merges all of them and writes the output, so one
// launch does the whole evaluation -- the partials carry their max and sum
// in the same pass and nothing is recomputed ("Rolling-KV -- overflow
// throughput evaluations (consolidated)", section 3: the log-sum-exp channel
// replaced a per-tile recompute).

#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"


namespace kvdec {
namespace {

// Phase trace of the one-shot kernel and its merge (diagnostic build only,
// KVDEC_PHASE_TRACE; compiled out otherwise).  Each workgroup owns 32 slots
// of the buffer and writes the constant 100 MHz clock (s_memrealtime) into
// them: 0 entry, 1 loads issued, 2 query converted, 3 scores and maximum,
// 4 weights, 5 + w wave w's P.V done, 13 streams merged, 14 record stores
// issued, 15 record stores acknowledged, 16 ticket returned, 17 merge done
// (merging workgroup only, after its output stores), 18 (m, l) loads
// issued, 19 (m, l) reduced, 20 records accumulated, 21 columns combined,
// 22 + w wave w's last V data landed, 30 merge entered, 31 record loads
// issued.  Slots 0-4 and 13-21, 30, 31 are written by thread 0.
#ifdef KVDEC_PHASE_TRACE
#define KVDEC_TRACE(k)                                                                                        \
    do {                                                                                                      \
        if (a.trace && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 32 + (k)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#define KVDEC_TRACE_WAVE(k)                                                                                   \
    do {                                                                                                      \
        if (a.trace && (threadIdx.x & 63) == 0)                                                              \
            a.trace[(size_t)blockIdx.x * 32 + (k)] = __builtin_amdgcn_s_memrealtime();                       \
    } while (0)
#else
#define KVDEC_TRACE(k) \
    do {               \
    } while (0)
#define KVDEC_TRACE_WAVE(k) \
    do {                    \
    } while (0)
#endif

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
// Softmax weights are formed as 2^(s - m + kPOff) so that, when they are
// rounded to f16 for packed dot products, weights down to 2^-29 of the
// maximum stay normal f16 numbers; l and o carry the same factor, which is
// removed when a partial leaves the workgroup.
constexpr float kPOff = 15.0f;
constexpr float kPOffInv = 1.0f / 32768.0f;

__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }

// Two floats -> an f16 pair, each rounded to nearest (one v_cvt_pk_f16_f32).
// Softmax weights go through this: unbiased, so l summed from the rounded
// weights carries no systematic error into lse.
__device__ __forceinline__ h2 to_h2(float a, float b) { return __builtin_convertvector(f2v{a, b}, h2); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Values of x in the two 16-lane rows (S = 16) or 32-lane halves (S = 32)
// that lane and lane ^ S sit in, lower one first, for every lane: one VALU
// row swap instead of a trip through the LDS crossbar.  Combining (lo, hi)
// in that order gives every lane the same bits.
template <int S>
__device__ __forceinline__ void row_pair(float x, float& lo, float& hi) {
    // (elements of the returned pair are read with __uint_as_float: a
    // __builtin_bit_cast of element 1 was compiled as element 0)
    const uint32_t u = __float_as_uint(x);
    if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
    } else {
        static_assert(S == 32, "row pair stride");
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
    }
}
template <int S>
__device__ __forceinline__ float pair_sum(float x) {
    float lo, hi;
    row_pair<S>(x, lo, hi);
    return lo + hi;
}
template <int S>
__device__ __forceinline__ float pair_max(float x) {
    float lo, hi;
    row_pair<S>(x, lo, hi);
    return fmaxf(lo, hi);
}

// Sum over each group of R consecutive lanes; every lane receives its group's sum.
template <int R>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (R >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (R >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (R >= 8) x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (R >= 16) x += dpp<0x140>(x); // row_mirror
    if constexpr (R >= 32) x = pair_sum<16>(x);
    if constexpr (R >= 64) x = pair_sum<32>(x);
    return x;
}

// Rows of a G-row group padded to a power of two for scatter_sum8.
template <int G>
constexpr int scatter_rows() {
    return G <= 1 ? 1 : (G <= 2 ? 2 : (G <= 4 ? 4 : 8));
}

// The row whose full sum lane `sub` (0..7) of an 8-lane group receives from
// scatter_sum8<GS>.
template <int GS>
__device__ __forceinline__ int scatter_row(int sub) {
    return (GS >= 2 ? ((sub >> 2) & 1) * (GS / 2) : 0) + (GS >= 4 ? ((sub >> 1) & 1) * (GS / 4) : 0) +
           (GS >= 8 ? (sub & 1) : 0);
}

// One step of scatter_sum8 over N rows with the partner lane CTRL selects:
// with N > 1 the lane keeps the upper half of its rows when `up` is set (its
// partner's `up` is the opposite), the lower half otherwise, and adds the
// partner's copy of that half; with N = 1 it adds the partner's value.
template <int N, int CTRL>
__device__ __forceinline__ void scatter_step(float* x, bool up) {
    if constexpr (N == 1) {
        x[0] += dpp<CTRL>(x[0]);
    } else {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float keep = up ? x[i + N / 2] : x[i];
            const float send = up ? x[i] : x[i + N / 2];
            x[i] = keep + dpp<CTRL>(send);
        }
    }
}

// Reduce-scatter over each group of 8 consecutive lanes: every lane brings
// GS partial sums, one per row, and receives the group's full sum of row
// scatter_row<GS>(sub).  Partners: 7 - sub (row_half_mirror), then sub ^ 2
// and sub ^ 1 (quad_perm); 3 (GS - 1) + 3 - log2(GS) instructions where GS
// all-reduces take 3 GS, and whatever follows handles one value per lane.
template <int GS>
__device__ __forceinline__ float scatter_sum8(const float (&v)[GS], int sub) {
    float x[GS];
#pragma unroll
    for (int i = 0; i < GS; ++i) x[i] = v[i];
    scatter_step<GS, 0x141>(x, (sub & 4) != 0);
    scatter_step<(GS > 1 ? GS / 2 : 1), 0x4E>(x, (sub & 2) != 0);
    scatter_step<(GS > 2 ? GS / 4 : 1), 0xB1>(x, (sub & 1) != 0);
    return x[0];
}

// x of lane `l` (a constant over the wave), in a scalar register.
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Max / sum over the whole wave; every lane receives the result.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    x = pair_max<16>(x);
    return pair_max<32>(x);
}
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-workgroup records.  A split's partial record is read by the last
// workgroup of its (slot, KV head), which may run on another XCD.  The record
// is written and read with device-scope relaxed atomic accesses, which the
// hardware keeps coherent across the XCDs' L2 caches without the whole-L2
// write-back / invalidate that a device-scope fence costs; the writer waits
// for its stores to complete before the ticket increment that publishes them.
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Storage formats: a lane reads its d-slice of a row in chunks of at most 16
// bytes; EPC elements per chunk (a divisor of the 32-element scale block).
template <int T, int DL>
struct Fmt;
template <int DL>
struct Fmt<KVDEC_F16, DL> {
    static constexpr int EPC = DL < 8 ? DL : 8;
    static constexpr int CB = 2 * EPC;
    static constexpr bool scaled = false;
};
template <int DL>
struct Fmt<KVDEC_Q8_B32, DL> {
    static constexpr int EPC = DL < 16 ? DL : 16;
    static constexpr int CB = EPC;
    static constexpr bool scaled = true;
};
template <int DL>
struct Fmt<KVDEC_Q4_B32, DL> {
    static constexpr int EPC = DL < 16 ? DL : 16;
    static constexpr int CB = EPC / 2;
    static constexpr bool scaled = true;
};

template <int CB>
struct Chunk {
    uint32_t w[CB / 4];
};

template <int CB>
__device__ __forceinline__ Chunk<CB> load_chunk(const uint8_t* p) {
    Chunk<CB> c;
    if constexpr (CB == 16) {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        c.w[0] = x.x;
        c.w[1] = x.y;
        c.w[2] = x.z;
        c.w[3] = x.w;
    } else if constexpr (CB == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        c.w[0] = x.x;
        c.w[1] = x.y;
    } else {
        static_assert(CB == 4, "chunk size");
        c.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    return c;
}

template <int CB>
__device__ __forceinline__ Chunk<CB> zero_chunk() {
    Chunk<CB> c;
#pragma unroll
    for (int i = 0; i < CB / 4; ++i) c.w[i] = 0;
    return c;
}

// Stored codes of one chunk -> pairs (element 2i, element 2i+1) as f16, exactly.
// int8 code x: the byte x ^ 0x80 = x + 128 becomes the low byte of the f16
// 0x64__ = 1024 + (x + 128); subtracting 1152 leaves x.  4-bit code u: the
// nibble becomes the low byte of 0x64__ = 1024 + u; subtracting 1032 leaves
// u - 8.  Element 2i of a 4-bit row is the low nibble of byte i.
template <int T, int CB, int NP>
__device__ __forceinline__ void to_pairs(const Chunk<CB>& c, h2 (&p)[NP]) {
    constexpr int NW = CB / 4;
    if constexpr (T == KVDEC_F16) {
        static_assert(NP == NW, "pairs");
#pragma unroll
        for (int i = 0; i < NW; ++i) p[i] = as_h2(c.w[i]);
    } else if constexpr (T == KVDEC_Q8_B32) {
        static_assert(NP == 2 * NW, "pairs");
        const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const uint32_t x = c.w[i] ^ 0x80808080u;
            p[2 * i] = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
            p[2 * i + 1] = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
        }
    } else {
        static_assert(NP == 4 * NW, "pairs");
        const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const uint32_t lo = c.w[i] & 0x0F0F0F0Fu;
            const uint32_t hi = (c.w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b;
                p[4 * i + b] = as_h2(__builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u) - bias;
            }
        }
    }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// End of the positions of slot s worth reading: all of them, or for an
// indirect plan given the records in use per slot, the first
// live_records[s] 128-entry segments -- a device-built plan fills the rest
// of its record budget with segments of holes, which are then never visited.
__device__ __forceinline__ int64_t live_end(const SplitArgs& a, const SlotArg& sa, int s) {
    if (!a.plan || !a.live_records) return sa.n;
    const int64_t r = a.live_records[a.slot_base + s];
    const int64_t e = (r > 0 ? r : 0) * (int64_t)kTile;
    return e < sa.n ? e : sa.n;
}

// Splits of slot s whose positions start below live_end (split sp starts
// at floor(sp n_units / n_splits) units): with live_records the others hold
// only entries out of use, and their workgroups leave at once -- they
// publish nothing and the slot's merge neither waits for nor reads them.
// At least one, so a slot with nothing in use still writes its outputs.
__device__ __forceinline__ int live_splits(const SplitArgs& a, const SlotArg& sa, int s) {
    if (!a.plan || !a.live_records || sa.n_units <= 0) return sa.n_splits;
    const int64_t e = (live_end(a, sa, s) + a.split_unit - 1) / a.split_unit;  // units in use
    const int64_t n = (e * sa.n_splits + sa.n_units - 1) / sa.n_units;
    return n < 1 ? 1 : (n > sa.n_splits ? sa.n_splits : (int)n);
}

// Lane geometry.  Per-lane d-slice DL: 16 elements for groups up to 5, 8
// above (register budget).  R lanes per cell, CPW cells per wave per load,
// NB cells per lane per step, so a step of W waves covers W * CPW * NB cells.
template <int D, int G>
struct Geo {
    static constexpr int DL = (G <= 5) ? 16 : 8;
    static constexpr int R = D / DL;
    static constexpr int CPW = 64 / R;
    static constexpr int NB = 4;
    static_assert(R >= 4 && R <= 32, "lane geometry");
};

// Merge of two log2-domain partials (M, L, O) <- (mb, lb, ob), 4 columns.
__device__ __forceinline__ void merge4(float& M, float& L, float4& O, float mb, float lb, float4 ob) {
    const float mn = fmaxf(M, mb);
    const float fa = (M == kNegInf) ? 0.f : exp2_fast(M - mn);
    const float fb = (mb == kNegInf) ? 0.f : exp2_fast(mb - mn);
    L = L * fa + lb * fb;
    O.x = O.x * fa + ob.x * fb;
    O.y = O.y * fa + ob.y * fb;
    O.z = O.z * fa + ob.z * fb;
    O.w = O.w * fa + ob.w * fb;
    M = mn;
}

// Output of one row's columns d0 .. d0+3 after the merge: the final out /
// lse / partial triple, or the running partial when more partials follow.
__device__ __forceinline__ void emit4(const SplitArgs& a, int to_acc, int64_t row, int d0, int D, float M2, float L,
                                      float4 O) {
    if (to_acc) {
        float* acc = a.acc_out;
        if (d0 == 0) {
            acc[row] = M2;
            acc[a.acc_rows + row] = L;
        }
        *reinterpret_cast<float4*>(acc + acc_o_offset(a.acc_rows) + row * D + d0) = O;
        return;
    }
    const bool empty = !(L > 0.f);
    if (a.out) {
        const float4 r = empty ? make_float4(0.f, 0.f, 0.f, 0.f) : make_float4(O.x / L, O.y / L, O.z / L, O.w / L);
        *reinterpret_cast<float4*>(a.out + row * D + d0) = r;
    }
    if (d0 == 0) {
        if (a.lse) a.lse[row] = empty ? kNegInf : (M2 + log2f(L)) * kLn2;
        if (a.pm) {
            a.pm[row] = empty ? kNegInf : M2 * kLn2;
            a.pl[row] = L;
        }
    }
    if (a.po) *reinterpret_cast<float4*>(a.po + row * D + d0) = O;
}

// Running partial handed in from an earlier launch (window + tail chain).
__device__ __forceinline__ void merge_acc_in(const SplitArgs& a, int64_t row, int d0, int D, float& M, float& L,
                                             float4& O) {
    if (!a.acc_in) return;
    const float4 ob = *reinterpret_cast<const float4*>(a.acc_in + acc_o_offset(a.acc_rows) + row * D + d0);
    merge4(M, L, O, a.acc_in[row], a.acc_in[a.acc_rows + row], ob);
}

typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const SplitArgs& a) {
    return __builtin_amdgcn_make_buffer_rsrc(a.part_o, (short)0, (int)a.part_o_bytes, 0x00020000);
}
// Device-coherent (sc1) 16-byte store / load of a split record's o columns.
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, int64_t off_bytes, float4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(f4v{v.x, v.y, v.z, v.w}, r, (int)off_bytes, 0, 0x10);
}
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, int64_t off_bytes) {
    const f4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off_bytes, 0, 0x10);
    return make_float4(v.x, v.y, v.z, v.w);
}

// Output row of a record row.  A (slot, KV head) record holds the G query
// heads of each of the slot's n_q query rows, query-major; rows of q, out,
// lse and the partial outputs are [slot][n_q][Hq].  Record rows at or past
// `rows` are padding and have no output row.
struct RowMap {
    int64_t base;     // row of (slot, query 0, first head of the group)
    int32_t group;    // G
    int32_t n_q_heads;
    int32_t rows;     // G * n_q real rows
    __device__ __forceinline__ bool real(int h) const { return h < rows; }
    __device__ __forceinline__ int64_t row(int h) const {
        return base + (int64_t)(h / group) * n_q_heads + h % group;
    }
};

// Merge of `count` consecutive partial records of one (slot, KV head),
// starting at record rec0, by the last workgroup to finish among those that
// wrote them.  The records were written by workgroups that may sit on other
// XCDs, so every load here goes out to memory; the merge is organised so
// that each chunk of merge_chunk(D, G) records costs one round trip: a
// thread first issues the loads of all its o columns for the chunk, then
// the (m, l) loads, and only then waits.  Thread -> (float4 column, record
// residue class); the running maximum and sums per head are kept in LDS
// across chunks.  The result goes to the outputs (dest < 0) or, merged but
// not normalised, to record `dest` (a cluster record).
template <int D, int G, int NT = kThreads>
__device__ void merge_records(const SplitArgs& a, const SlotArg& sa, const RowMap& rm, int64_t rec0, int count,
                              int64_t dest, int chunk) {
    constexpr int NV = G * D / 4;                           // float4 columns of o
    constexpr int TS = NV >= NT ? 1 : NT / NV;              // threads per column
    constexpr int COLS = (NV + NT - 1) / NT;                // columns per thread
    constexpr int SPC_MAX = merge_chunk_max(D, G);          // largest round (one record per lane)
    constexpr int UB = (SPC_MAX + TS - 1) / TS;             // records per thread per round
    static_assert(SPC_MAX <= 64 && UB * COLS <= 56, "merge chunk");
    // this slot's round (a constant where the kernel has no choice)
    const int SPC = SPC_MAX == merge_chunk(D, G) ? SPC_MAX : chunk;
    constexpr int NW = NT / 64;                             // waves
    __shared__ float f_m[64 * G];
    __shared__ float run_m[G], run_l[G], scale_old[G];
    __shared__ float4 red[TS > 1 ? NT : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = tid % (NV < NT ? NV : NT);
    const int cls = tid / (NV < NT ? NV : NT);  // threads with cls >= TS idle
    const __amdgpu_buffer_rsrc_t rs = part_rsrc(a);
    const int n_splits = count;
    if constexpr (G <= 5 && NT == 512) if (dest < 0) KVDEC_TRACE(30);

    float4 acc[COLS];
#pragma unroll
    for (int c = 0; c < COLS; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < G) {
        run_m[tid] = kNegInf;
        run_l[tid] = 0.f;
    }
    for (int sp0 = 0; sp0 < n_splits; sp0 += SPC) {
        const int nsp = (n_splits - sp0) < SPC ? (n_splits - sp0) : SPC;
        // (m, l) of the chunk first -- a kilobyte the maxima and weights wait
        // for, which would otherwise queue behind the chunk's o loads in the
        // compute unit's address path: wave w takes record rows w, w + NW,
        // w + 2 NW, ..., one split per lane.
        constexpr int HW = (G + NW - 1) / NW;  // record rows per wave
        float mv[HW], lv[HW];
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            const int h = wave + NW * hh;
            mv[hh] = kNegInf;
            lv[hh] = 0.f;
            if (h < G && lane < nsp) {
                mv[hh] = ld_dev(a.part_m + (rec0 + sp0 + lane) * G + h);
                lv[hh] = ld_dev(a.part_l + (rec0 + sp0 + lane) * G + h);
            }
        }
        if constexpr (G <= 5 && NT == 512) if (dest < 0 && sp0 == 0) KVDEC_TRACE(18);
        __builtin_amdgcn_sched_barrier(0);  // issue them before the o loads
        // Round u of loads runs when some thread has a record in it (a
        // test uniform over the workgroup); a thread past the chunk's last
        // record reads that record again, which then gets weight 0.
        // (every thread has a column when NT is a multiple of NV or NV of NT)
        constexpr bool kAllCols = NV <= NT ? NT % NV == 0 : NV % NT == 0;
        float4 x[COLS][UB];
#pragma unroll
        for (int c = 0; c < COLS; ++c) {
            const int v = col + c * NT;
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                x[c][u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (u * TS < nsp && (kAllCols || (cls < TS && v < NV))) {
                    const int sp = cls + u * TS < nsp ? cls + u * TS : nsp - 1;
                    x[c][u] = ld_dev4(rs, ((rec0 + sp0 + sp) * (G * D) + 4 * v) * 4);
                }
            }
        }
        if constexpr (G <= 5 && NT == 512) if (dest < 0 && sp0 == 0) KVDEC_TRACE(31);
        __syncthreads();  // the previous chunk is done with f_m / scale_old
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            const int h = wave + NW * hh;
            if (h >= G) continue;  // uniform over the wave
            const float mo = run_m[h];
            const float mn = fmaxf(mo, wave_max(mv[hh]));
            const float f = (mv[hh] == kNegInf) ? 0.f : exp2_fast(mv[hh] - mn);
            const float so = (mo == kNegInf) ? 0.f : exp2_fast(mo - mn);
            const float ls = wave_sum(lv[hh] * f);
            if (lane < nsp) f_m[lane * G + h] = f;
            if (lane == 0) {
                scale_old[h] = so;
                run_l[h] = run_l[h] * so + ls;
                run_m[h] = mn;
            }
        }
        __syncthreads();
        if constexpr (G <= 5 && NT == 512) if (dest < 0 && sp0 == 0) KVDEC_TRACE(19);
#pragma unroll
        for (int c = 0; c < COLS; ++c) {
            const int v = col + c * NT;
            if (cls >= TS || v >= NV) continue;
            const int h = (4 * v) / D;
            const float so = scale_old[h];
            float4 o = acc[c];
            o.x *= so;
            o.y *= so;
            o.z *= so;
            o.w *= so;
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int sp = cls + u * TS;
                const float f = sp < nsp ? f_m[sp * G + h] : 0.f;
                o.x = fmaf(x[c][u].x, f, o.x);
                o.y = fmaf(x[c][u].y, f, o.y);
                o.z = fmaf(x[c][u].z, f, o.z);
                o.w = fmaf(x[c][u].w, f, o.w);
            }
            acc[c] = o;
        }
    }
    if constexpr (G <= 5 && NT == 512) if (dest < 0) KVDEC_TRACE(20);
    // combine the TS residue classes of each column
    if constexpr (TS > 1) {
        red[tid] = acc[0];
        __syncthreads();
        if (cls == 0) {
            float4 o = acc[0];
            for (int t = 1; t < TS; ++t) {
                const float4 y = red[t * NV + col];
                o.x += y.x;
                o.y += y.y;
                o.z += y.z;
                o.w += y.w;
            }
            acc[0] = o;
        }
    }
    if constexpr (G <= 5 && NT == 512) if (dest < 0) KVDEC_TRACE(21);
    if (cls == 0) {
#pragma unroll
        for (int c = 0; c < COLS; ++c) {
            const int v = col + c * NT;
            if (v >= NV) continue;
            const int h = (4 * v) / D;
            const int d0 = 4 * v - h * D;
            float M = run_m[h], L = run_l[h];
            float4 O = acc[c];
            if (dest < 0) {
                if (!rm.real(h)) continue;
                merge_acc_in(a, rm.row(h), d0, D, M, L, O);
                emit4(a, sa.to_acc, rm.row(h), d0, D, M, L, O);
            } else {
                st_dev4(rs, (dest * (G * D) + 4 * v) * 4, O);
                if (d0 == 0) {
                    st_dev(a.part_m + dest * G + h, M);
                    st_dev(a.part_l + dest * G + h, L);
                }
            }
        }
    }
}

// One arrival at a ticket that counts `expected` arrivals; true (for the
// whole workgroup) in the last one to arrive, which also resets the ticket.
__device__ __forceinline__ bool last_arrival(uint32_t* ticket, int expected, int& sm_last) {
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == (uint32_t)(expected - 1);
        if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = last;
    }
    __syncthreads();
    return sm_last != 0;
}

template <int D, int G, int NT>
__device__ __forceinline__ void arrive_and_merge(const SplitArgs& a, const SlotArg& sa, int s, int g, int split,
                                                 const RowMap& rm, int& sm_last);

// End of a split: merge the NS cell streams left in LDS (m2, l, o per
// stream and head) into the split's result; a single-split group writes its
// output directly, otherwise the split's record is published and the last
// workgroup of the (slot, KV head) merges all records.
template <int D, int G, int NS, int DP, int NT = kThreads>
__device__ __forceinline__ void finish_split(const SplitArgs& a, const SlotArg& sa, int s, int g, int split,
                                             const RowMap& rm, const float (*sm_m)[G], const float (*sm_l)[G],
                                             const float (*sm_o)[G][DP], int& sm_last) {
    const int tid = threadIdx.x;
    // Merge the NS streams: P adjacent threads per float4 column, each over
    // every P-th stream, combined by lane shuffles.  Result of this split in
    // log2 units.
    constexpr int NV = G * D / 4;
    constexpr int PQ = NT / NV;
    constexpr int P = (NS % 4 == 0 && PQ >= 4) ? 4 : ((NS % 2 == 0 && PQ >= 2) ? 2 : 1);
    const int part = tid % P;
    const int n_splits = sa.n_splits;  // record stride of the (slot, KV head)
    const bool single = live_splits(a, sa, s) == 1;
    const int64_t rec = sa.part_begin + (int64_t)g * n_splits + split;
    const __amdgpu_buffer_rsrc_t rs = part_rsrc(a);
    for (int v = tid / P; v < NV; v += NT / P) {
        const int h = (4 * v) / D, d0 = 4 * v - h * D;
        float M = kNegInf;
#pragma unroll
        for (int k = part; k < NS; k += P) M = fmaxf(M, sm_m[k][h]);
        // the P threads of a column are adjacent lanes of one quad: DPP
        if constexpr (P >= 2) M = fmaxf(M, dpp<0xB1>(M));  // lane ^ 1
        if constexpr (P >= 4) M = fmaxf(M, dpp<0x4E>(M));  // lane ^ 2
        float L = 0.f;
        float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = part; k < NS; k += P) {
            const float mk = sm_m[k][h];
            const float f = (mk == kNegInf) ? 0.f : exp2_fast(mk - M);
            const float4 ok = *reinterpret_cast<const float4*>(&sm_o[k][h][d0]);
            L = fmaf(sm_l[k][h], f, L);
            O.x = fmaf(ok.x, f, O.x);
            O.y = fmaf(ok.y, f, O.y);
            O.z = fmaf(ok.z, f, O.z);
            O.w = fmaf(ok.w, f, O.w);
        }
        if constexpr (P >= 2) {
            L += dpp<0xB1>(L);
            O.x += dpp<0xB1>(O.x);
            O.y += dpp<0xB1>(O.y);
            O.z += dpp<0xB1>(O.z);
            O.w += dpp<0xB1>(O.w);
        }
        if constexpr (P >= 4) {
            L += dpp<0x4E>(L);
            O.x += dpp<0x4E>(O.x);
            O.y += dpp<0x4E>(O.y);
            O.z += dpp<0x4E>(O.z);
            O.w += dpp<0x4E>(O.w);
        }
        if (part != 0) continue;
        if (single) {
            if (rm.real(h)) {
                merge_acc_in(a, rm.row(h), d0, D, M, L, O);
                emit4(a, sa.to_acc, rm.row(h), d0, D, M, L, O);
            }
        } else {
            st_dev4(rs, (rec * (G * D) + 4 * v) * 4, O);
            if (d0 == 0) {
                st_dev(a.part_m + rec * G + h, M);
                st_dev(a.part_l + rec * G + h, L);
            }
        }
    }
    if (single) return;
    arrive_and_merge<D, G, NT>(a, sa, s, g, split, rm, sm_last);
}

// After a split's record stores: count the arrival and, in the last
// workgroup of the (slot, KV head) -- or of its cluster, then of the cluster
// records -- merge the records into the outputs.
template <int D, int G, int NT>
__device__ __forceinline__ void arrive_and_merge(const SplitArgs& a, const SlotArg& sa, int s, int g, int split,
                                                 const RowMap& rm, int& sm_last) {
    // the splits taking part (all, or those holding entries in use) and the
    // merge shape the planner gives that many splits
    const int n_splits = live_splits(a, sa, s);
    const int chunk = merge_chunk_for(D, G, n_splits);
    const int ncl = merge_clusters(n_splits, chunk);
    // Records are published (stores complete) before the arrival is counted.
    wait_stores();
    __syncthreads();
    if constexpr (G <= 5) KVDEC_TRACE(15);
    uint32_t* gticket = a.tickets + kTicketStride * ((int64_t)(a.slot_base + s) * a.n_kv_heads + g);
    const int64_t srec0 = sa.part_begin + (int64_t)g * sa.n_splits;
    if (ncl <= 1) {
        // the last workgroup of the (slot, KV head) merges every split
        const bool last = last_arrival(gticket, n_splits, sm_last);
        if constexpr (G <= 5) KVDEC_TRACE(16);
        if (!last) return;
        merge_records<D, G, NT>(a, sa, rm, srec0, n_splits, -1, chunk);
#ifdef KVDEC_PHASE_TRACE
        wait_stores();
        if constexpr (G <= 5) KVDEC_TRACE(17);
#endif
        return;
    }
    // two levels: the last of each cluster of splits merges the cluster into
    // a cluster record; the last cluster merger merges the cluster records
    // (record slots of the plan's sa.n_clusters clusters; ncl <= that)
    const int CH = merge_chunk_max(D, G) == merge_chunk(D, G) ? merge_chunk(D, G) : chunk;
    const int cid = split / CH;
    const int c0 = cid * CH;
    const int cn = (n_splits - c0) < CH ? (n_splits - c0) : CH;
    const int64_t cidx = sa.cl_begin + (int64_t)g * sa.n_clusters + cid;
    if (!last_arrival(a.ctickets + kTicketStride * cidx, cn, sm_last)) return;
    merge_records<D, G, NT>(a, sa, rm, srec0 + c0, cn, a.crec_base + cidx, chunk);
    wait_stores();
    __syncthreads();
    if (!last_arrival(gticket, ncl, sm_last)) return;
    merge_records<D, G, NT>(a, sa, rm, a.crec_base + sa.cl_begin + (int64_t)g * sa.n_clusters, ncl, -1, chunk);
}


template <int D, int G, int KT, int VT, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void split_kernel(const SplitArgs a) {
    using Gm = Geo<D, G>;
    constexpr int DL = Gm::DL, R = Gm::R, CPW = Gm::CPW, NCW = Gm::NB;
    constexpr int STEP = W * CPW * NCW;  // cells per workgroup step (W waves)
    using FK = Fmt<KT, DL>;
    using FV = Fmt<VT, DL>;
    constexpr int NCK = DL / FK::EPC;  // K chunks per lane per cell
    constexpr int NCV = DL / FV::EPC;  // V chunks per lane per cell
    static_assert(NCK >= 1 && NCV >= 1 && NCK * FK::EPC == DL && NCV * FV::EPC == DL, "chunking");
    constexpr int NB = D / kBlock;     // scales per row
    // Cell streams per wave left after the in-register (DPP) merge step.
    constexpr bool kDppStep = R <= 8;
    constexpr int NSW = kDppStep ? CPW / 2 : CPW;
    constexpr int NS = W * NSW;        // streams per workgroup merged through LDS

    __shared__ float sm_m[NS][G];
    __shared__ float sm_l[NS][G];
    // f16 caches: the next step's K / V rows are loaded straight into LDS
    // (global_load_lds, 16 bytes per lane, lane l's data at slot l) while the
    // current step computes from registers -- a second step in flight that
    // costs no VGPRs.  The staging area (16 KiB per wave) is reused for the
    // stream merge after the loop.
    constexpr bool kDma = KT == KVDEC_F16 && VT == KVDEC_F16;
    constexpr int kMergeBytes = NS * G * (D + 16) * 4;
    constexpr int kDmaBytes = kDma ? W * 64 * NCW * (NCK + NCV) * 16 : 0;
    __shared__ __align__(16) unsigned char lds_raw[kMergeBytes > kDmaBytes ? kMergeBytes : kDmaBytes];
    // stream stride padded by 16 floats: streams written by one instruction land in different banks
    float (*sm_o)[G][D + 16] = reinterpret_cast<float (*)[G][D + 16]>(lds_raw);
    __shared__ int sm_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane % R;
    const int cl = lane / R;

    // Which (slot, KV head, split) this workgroup owns.
    const int wg = blockIdx.x;
    int s = 0;
    while (s + 1 < a.n_slots && a.slot[s + 1].wg_begin <= wg) ++s;
    const SlotArg sa = a.slot[s];
    const int local = wg - sa.wg_begin;
    // Consecutive workgroups take the same cell range of different KV heads,
    // so the workgroups resident together read neighbouring bytes of each
    // cell row.
    const int split = local / a.n_kv_heads;
    const int g = local - split * a.n_kv_heads;
    if (split >= live_splits(a, sa, s)) return;  // nothing in use: not part of the merge
    // Positions [pos_begin, pos_end) of the slot: split boundaries fall on
    // multiples of a.split_unit.
    const int64_t pos_begin = (((int64_t)split * sa.n_units) / sa.n_splits) * a.split_unit;
    const int64_t span_end = (((int64_t)(split + 1) * sa.n_units) / sa.n_splits) * a.split_unit;
    const int hq0 = g * G;  // first query head of the group
    const int64_t row0 = (int64_t)(a.slot_base + s) * a.n_q_heads + hq0;

    // Query rows of the group, f16 pairs, this lane's K d-slice only.
    h2 qh[G][DL / 2];
    {
        const float* qp = a.q + row0 * D;
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int c = 0; c < NCK; ++c) {
                const int e = (c * R + sub) * FK::EPC;
#pragma unroll
                for (int i = 0; i < FK::EPC / 2; ++i) {
                    const float2 x = *reinterpret_cast<const float2*>(qp + h * D + e + 2 * i);
                    qh[h][c * (FK::EPC / 2) + i] = h2{(_Float16)x.x, (_Float16)x.y};
                }
            }
        }
    }

    float m[G], l[G], o[G][DL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[h][i] = 0.f;
    }

    const uint8_t* kbase = a.k + (int64_t)g * a.k_hs;
    const uint8_t* vbase = a.v + (int64_t)g * a.v_hs;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    const int64_t slot_end = live_end(a, sa, s);
    const int64_t pos_end = span_end < slot_end ? span_end : slot_end;

    // One step: NCW cells per lane.  Buffers of a step in flight.
    struct Step {
        bool valid[NCW];
        Chunk<FK::CB> kc[NCW][NCK];
        Chunk<FV::CB> vc[NCW][NCV];
        float kd[NCW][NCK], vd[NCW][NCV];
    };

    // Issue the loads of the step starting at slot position `base`.  Load j
    // of the W waves covers W * CPW consecutive cells (wave w the w-th group
    // of CPW), so every wave's cells spread over the whole step instead of
    // one contiguous block per wave (Qwen3-8B-shaped layer 20.9 -> 20.3 us;
    // the last wave's loads land 0.5 us earlier).
    auto load_step = [&](int64_t base, Step& st) {
        int64_t cell[NCW];
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const int64_t pos = base + (j * W + wave) * CPW + cl;  // position in the slot
            if (a.plan) {
                const bool in = pos < pos_end;
                const int64_t c = in ? (int64_t)a.plan[sa.first + pos] : -1;
                st.valid[j] = c >= 0 && c < a.capacity;
                cell[j] = st.valid[j] ? c : 0;
            } else {
                st.valid[j] = pos < pos_end;
                cell[j] = sa.first + (st.valid[j] ? pos : 0);
            }
        }
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const uint8_t* kr = kbase + cell[j] * a.k_cs;
            const uint8_t* vr = vbase + cell[j] * a.v_cs;
#pragma unroll
            for (int c = 0; c < NCK; ++c)
                st.kc[j][c] = st.valid[j] ? load_chunk<FK::CB>(kr + (c * R + sub) * FK::CB) : zero_chunk<FK::CB>();
#pragma unroll
            for (int c = 0; c < NCV; ++c)
                st.vc[j][c] = st.valid[j] ? load_chunk<FV::CB>(vr + (c * R + sub) * FV::CB) : zero_chunk<FV::CB>();
            if constexpr (FK::scaled) {
#pragma unroll
                for (int c = 0; c < NCK; ++c) {
                    const int blk = ((c * R + sub) * FK::EPC) / kBlock;
                    st.kd[j][c] = st.valid[j] ? half_bits_to_float(a.ks[(cell[j] * a.n_kv_heads + g) * NB + blk]) : 0.f;
                }
            }
            if constexpr (FV::scaled) {
#pragma unroll
                for (int c = 0; c < NCV; ++c) {
                    const int blk = ((c * R + sub) * FV::EPC) / kBlock;
                    st.vd[j][c] = st.valid[j] ? half_bits_to_float(a.vs[(cell[j] * a.n_kv_heads + g) * NB + blk]) : 0.f;
                }
            }
        }
    };

    // Scores, online-softmax update and P.V of one loaded step.
    auto compute_step = [&](const Step& st) {
        float sc[NCW][G];
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            float acc[G];
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
            for (int c = 0; c < NCK; ++c) {
                h2 kp[FK::EPC / 2];
                to_pairs<KT>(st.kc[j][c], kp);
                if constexpr (FK::scaled) {
                    float part[G];
#pragma unroll
                    for (int h = 0; h < G; ++h) part[h] = 0.f;
#pragma unroll
                    for (int i = 0; i < FK::EPC / 2; ++i)
#pragma unroll
                        for (int h = 0; h < G; ++h)
                            part[h] = __builtin_amdgcn_fdot2(kp[i], qh[h][c * (FK::EPC / 2) + i], part[h], false);
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h] = fmaf(part[h], st.kd[j][c], acc[h]);
                } else {
#pragma unroll
                    for (int i = 0; i < FK::EPC / 2; ++i)
#pragma unroll
                        for (int h = 0; h < G; ++h)
                            acc[h] = __builtin_amdgcn_fdot2(kp[i], qh[h][c * (FK::EPC / 2) + i], acc[h], false);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float full = group_sum<R>(acc[h]);
                sc[j][h] = st.valid[j] ? full * a.scale_log2 : kNegInf;
            }
        }

        float p[NCW][G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mt = sc[0][h];
#pragma unroll
            for (int j = 1; j < NCW; ++j) mt = fmaxf(mt, sc[j][h]);
            const float mn = fmaxf(m[h], mt);
            const float alpha = (mn == kNegInf) ? 1.f : exp2_fast(m[h] - mn);
            l[h] *= alpha;
#pragma unroll
            for (int i = 0; i < DL; ++i) o[h][i] *= alpha;
            m[h] = mn;
#pragma unroll
            for (int j = 0; j < NCW; ++j) p[j][h] = (sc[j][h] == kNegInf) ? 0.f : exp2_fast(sc[j][h] - mn + kPOff);
        }

        if constexpr (VT == KVDEC_F16) {
            // Pairs of cells: (V[A][d], V[B][d]) . (pA, pB) in one packed dot.
#pragma unroll
            for (int jp = 0; jp < NCW / 2; ++jp) {
                const int A = 2 * jp, B = 2 * jp + 1;
                h2 pp[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    pp[h] = to_h2(p[A][h], p[B][h]);
                    l[h] = __builtin_amdgcn_fdot2(pp[h], ones, l[h], false);
                }
#pragma unroll
                for (int c = 0; c < NCV; ++c) {
#pragma unroll
                    for (int i = 0; i < FV::CB / 4; ++i) {
                        const h2 lo = as_h2(__builtin_amdgcn_perm(st.vc[B][c].w[i], st.vc[A][c].w[i], 0x05040100u));
                        const h2 hi = as_h2(__builtin_amdgcn_perm(st.vc[B][c].w[i], st.vc[A][c].w[i], 0x07060302u));
                        const int dd = c * FV::EPC + 2 * i;
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            o[h][dd] = __builtin_amdgcn_fdot2(lo, pp[h], o[h][dd], false);
                            o[h][dd + 1] = __builtin_amdgcn_fdot2(hi, pp[h], o[h][dd + 1], false);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
#pragma unroll
                for (int h = 0; h < G; ++h) l[h] += p[j][h];
#pragma unroll
                for (int c = 0; c < NCV; ++c) {
                    h2 vp[FV::EPC / 2];
                    to_pairs<VT>(st.vc[j][c], vp);
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float pd = p[j][h] * st.vd[j][c];
#pragma unroll
                        for (int i = 0; i < FV::EPC / 2; ++i) {
                            o[h][c * FV::EPC + 2 * i] = fmaf((float)vp[i].x, pd, o[h][c * FV::EPC + 2 * i]);
                            o[h][c * FV::EPC + 2 * i + 1] = fmaf((float)vp[i].y, pd, o[h][c * FV::EPC + 2 * i + 1]);
                        }
                    }
                }
            }
        }
    };

    // Short splits (one or two steps) take the plain path: staging the
    // second step of a two-step split measured slower (on short layers the
    // requests already in flight saturate the memory system).
    bool staged = false;
    if constexpr (kDma) staged = (pos_end - pos_begin) > 2 * STEP;
    if constexpr (kDma) if (staged) {
        static_assert(FK::CB == 16 && FV::CB == 16 && !FK::scaled && !FV::scaled, "16-byte f16 chunks");
        typedef __attribute__((address_space(3))) void lds_void;
        unsigned char* stage = lds_raw + wave * (64 * NCW * (NCK + NCV) * 16);
        // Slot of (cell j, chunk c) of this wave's staged step: K chunks, then V.
        auto slot_k = [&](int j, int c) { return stage + ((j * (NCK + NCV) + c) * 64) * 16; };
        auto slot_v = [&](int j, int c) { return stage + ((j * (NCK + NCV) + NCK + c) * 64) * 16; };
        bool staged_valid[NCW];
        auto stage_step = [&](int64_t base) {
            int64_t cell[NCW];
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
                const int64_t pos = base + (j * W + wave) * CPW + cl;
                if (a.plan) {
                    const int64_t c = pos < pos_end ? (int64_t)a.plan[sa.first + pos] : -1;
                    staged_valid[j] = c >= 0 && c < a.capacity;
                    cell[j] = staged_valid[j] ? c : 0;
                } else {
                    staged_valid[j] = pos < pos_end;
                    cell[j] = sa.first + (staged_valid[j] ? pos : 0);
                }
            }
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
                const uint8_t* kr = kbase + cell[j] * a.k_cs;
                const uint8_t* vr = vbase + cell[j] * a.v_cs;
#pragma unroll
                for (int c = 0; c < NCK; ++c)
                    if (staged_valid[j])
                        __builtin_amdgcn_global_load_lds((const void*)(kr + (c * R + sub) * 16), (lds_void*)slot_k(j, c),
                                                         16, 0, 0);
#pragma unroll
                for (int c = 0; c < NCV; ++c)
                    if (staged_valid[j])
                        __builtin_amdgcn_global_load_lds((const void*)(vr + (c * R + sub) * 16), (lds_void*)slot_v(j, c),
                                                         16, 0, 0);
            }
        };
        auto read_staged = [&](Step& st) {
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
                st.valid[j] = staged_valid[j];
#pragma unroll
                for (int c = 0; c < NCK; ++c) {
                    const uint4 x = *reinterpret_cast<const uint4*>(slot_k(j, c) + lane * 16);
                    st.kc[j][c] = staged_valid[j] ? Chunk<16>{{x.x, x.y, x.z, x.w}} : zero_chunk<16>();
                }
#pragma unroll
                for (int c = 0; c < NCV; ++c) {
                    const uint4 x = *reinterpret_cast<const uint4*>(slot_v(j, c) + lane * 16);
                    st.vc[j][c] = staged_valid[j] ? Chunk<16>{{x.x, x.y, x.z, x.w}} : zero_chunk<16>();
                }
            }
        };
        int64_t base = pos_begin;
        if (base < pos_end) {
            {
                Step st;
                load_step(base, st);                                 // step 0 -> registers
                if (base + STEP < pos_end) stage_step(base + STEP);  // step 1 -> LDS
                compute_step(st);
            }
            for (base += STEP; base < pos_end; base += STEP) {
                // this step was staged: wait for its LDS loads, move it to
                // registers, then stage the following step into the freed
                // slots before computing
                Step st;
                __builtin_amdgcn_s_waitcnt(0);
                __builtin_amdgcn_wave_barrier();
                read_staged(st);
                __builtin_amdgcn_s_waitcnt(0);
                __builtin_amdgcn_wave_barrier();
                if (base + STEP < pos_end) stage_step(base + STEP);
                compute_step(st);
            }
        }
        __syncthreads();  // every wave is done with its staging area before the merge reuses it
    }
    if (!staged) {
        for (int64_t base = pos_begin; base < pos_end; base += STEP) {
            Step st;
            load_step(base, st);
            compute_step(st);
        }
    }

    // Merge the cell streams.  Lanes with the same sub own the same d-slice
    // for different cells.  One in-register step pairs lane i with lane i ^ 8
    // (DPP row rotate by 8) when that partner holds the same slice; the
    // remaining NSW streams per wave go through LDS.
    if constexpr (kDppStep) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = dpp<0x128>(m[h]);
            const float lo = dpp<0x128>(l[h]);
            const float mn = fmaxf(m[h], mo);
            const float fa = (m[h] == kNegInf) ? 0.f : exp2_fast(m[h] - mn);
            const float fb = (mo == kNegInf) ? 0.f : exp2_fast(mo - mn);
            l[h] = l[h] * fa + lo * fb;
#pragma unroll
            for (int i = 0; i < DL; ++i) o[h][i] = o[h][i] * fa + dpp<0x128>(o[h][i]) * fb;
            m[h] = mn;
        }
    }
    const bool rep = kDppStep ? ((lane & 8) == 0) : true;
    const int kl = kDppStep ? (((lane & 7) | ((lane >> 4) << 3)) / R) : cl;
    if (rep) {
        const int k = wave * NSW + kl;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (sub == 0) {
                sm_m[k][h] = m[h];
                sm_l[k][h] = l[h] * kPOffInv;
            }
#pragma unroll
            for (int c = 0; c < NCV; ++c)
#pragma unroll
                for (int i = 0; i < FV::EPC; i += 4)
                    *reinterpret_cast<float4*>(&sm_o[k][h][(c * R + sub) * FV::EPC + i]) =
                        make_float4(o[h][c * FV::EPC + i] * kPOffInv, o[h][c * FV::EPC + i + 1] * kPOffInv,
                                    o[h][c * FV::EPC + i + 2] * kPOffInv, o[h][c * FV::EPC + i + 3] * kPOffInv);
        }
    }
    __syncthreads();

    const RowMap rm{row0, G, a.n_q_heads, G};
    finish_split<D, G, NS, D + 16, 64 * W>(a, sa, s, g, split, rm, sm_m, sm_l, sm_o, sm_last);
}

// Output of one column d of a row after the merge (the scalar form of emit4).
__device__ __forceinline__ void emit1(const SplitArgs& a, int to_acc, int64_t row, int d, int D, float M2, float L,
                                      float O) {
    if (to_acc) {
        float* acc = a.acc_out;
        if (d == 0) {
            acc[row] = M2;
            acc[a.acc_rows + row] = L;
        }
        acc[acc_o_offset(a.acc_rows) + row * D + d] = O;
        return;
    }
    const bool empty = !(L > 0.f);
    if (a.out) a.out[row * D + d] = empty ? 0.f : O / L;
    if (d == 0) {
        if (a.lse) a.lse[row] = empty ? kNegInf : (M2 + log2f(L)) * kLn2;
        if (a.pm) {
            a.pm[row] = empty ? kNegInf : M2 * kLn2;
            a.pl[row] = L;
        }
    }
    if (a.po) a.po[row * D + d] = O;
}

__device__ __forceinline__ void merge_acc_in1(const SplitArgs& a, int64_t row, int d, int D, float& M, float& L,
                                              float& O) {
    if (!a.acc_in) return;
    const float mb = a.acc_in[row], lb = a.acc_in[a.acc_rows + row];
    const float ob = a.acc_in[acc_o_offset(a.acc_rows) + row * D + d];
    const float mn = fmaxf(M, mb);
    const float fa = (M == kNegInf) ? 0.f : exp2_fast(M - mn);
    const float fb = (mb == kNegInf) ? 0.f : exp2_fast(mb - mn);
    L = L * fa + lb * fb;
    O = O * fa + ob * fb;
    M = mn;
}

// ---------------------------------------------------------------------------
// One-shot split kernel (head_dim 128, f16 K and V, G <= 5 query rows per KV
// head, contiguous cells) for splits short enough that a workgroup's whole
// share of the cache fits in its registers.  Every load of the split is
// issued at workgroup entry -- the query rows, then K, then V, all 16-byte
// loads into registers -- so each compute unit's whole share is requested at
// once and no load waits on an earlier step's arithmetic.  (Plain loads only:
// they complete in order, so each use waits for exactly its own data.)  Wave
// w owns a contiguous block of the split's cells:
//   * scores: 8 lanes per cell, 16 elements each (two 16-byte chunks of the
//     row), combined with DPP; all of the wave's scores are known before any
//     weight is formed, so the wave's maximum per head is exact and the wave
//     is a single softmax stream;
//   * weights 2^(s - m + 15), rounded to f16, go to LDS as pairs of
//     consecutive cells;
//   * V rows go to a per-wave LDS tile as their loads land, and P.V reads
//     them column-wise: lane l owns output columns 2l and 2l+1 of every head
//     and walks the wave's cells in pairs, so a wave's P.V needs no
//     reduction across lanes;
//   * the eight wave streams are merged through LDS, one output column per
//     thread, and the split's record is published as by the other kernels.
// ---------------------------------------------------------------------------
template <int G, int JM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void split_oneshot_kernel(const SplitArgs a) {
    constexpr int D = 128, W = 8;
    constexpr int R = 8;                 // lanes per cell for the scores
    constexpr int CPL = 64 / R;          // cells per wave load
    constexpr int NC = 2;                // 16-byte chunks per lane and cell row
    constexpr int CW = JM * CPL;         // most cells per wave
    constexpr int VSTR = 2 * D + 16;     // bytes per staged V row (padded against bank conflicts)
    constexpr int GP = (G + 3) / 4 * 4;  // dwords per weight-pair entry
    constexpr int VBYTES = W * CW * VSTR;
    constexpr int MBYTES = W * G * D * 4;
    static_assert(MBYTES <= VBYTES, "merge area inside the V tiles");

    // V tiles of the waves; after the last P.V, the waves' o rows for the merge
    __shared__ __align__(16) unsigned char v_lds[VBYTES];
    __shared__ __align__(16) uint32_t p_lds[W][CW / 2][GP];
    __shared__ __align__(16) uint32_t q_lds[W][G * D / 2];  // each wave's copy of the query rows, f16 pairs
    __shared__ float mg_m[W][G], mg_l[W][G];
    __shared__ int sm_last;

    KVDEC_TRACE(0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = lane % R;
    const int cl = lane / R;

    const int wg = blockIdx.x;
    int s = 0;
    while (s + 1 < a.n_slots && a.slot[s + 1].wg_begin <= wg) ++s;
    const SlotArg sa = a.slot[s];
    const int local = wg - sa.wg_begin;
    const int split = local / a.n_kv_heads;
    const int g = local - split * a.n_kv_heads;
    // The split's positions: a contiguous run, or (interleaved) the split
    // units split, split + n_splits, ...; position p of the split is slot
    // position pos(p).  The unit is the vector-ALU kernels' (the dispatch
    // checks), a constant, so the positions take shifts, not divisions.
    constexpr int U = kSplitUnit;
    int64_t pos_begin = 0;
    int n = 0;
    if (a.interleave) {
        const int nu = split < sa.n_units ? (sa.n_units - split + sa.n_splits - 1) / sa.n_splits : 0;
        if (nu > 0) {
            const int64_t last = ((int64_t)split + (int64_t)(nu - 1) * sa.n_splits) * U;
            n = (nu - 1) * U + (int)((sa.n - last) < U ? (sa.n - last) : U);
        }
    } else {
        pos_begin = (((int64_t)split * sa.n_units) / sa.n_splits) * U;
        const int64_t span_end = (((int64_t)(split + 1) * sa.n_units) / sa.n_splits) * U;
        const int64_t pos_end = span_end < sa.n ? span_end : sa.n;
        n = pos_end > pos_begin ? (int)(pos_end - pos_begin) : 0;
    }
    auto pos = [&](int p) -> int64_t {
        return a.interleave ? ((int64_t)split + (int64_t)(p / U) * sa.n_splits) * U + p % U : pos_begin + p;
    };
    // wave w: cells w * cw ... of the split, cw even and at most CW (the
    // planner keeps splits within W * CW cells; the clamp only keeps LDS
    // accesses in bounds)
    int cw = ((n + W - 1) / W + 1) & ~1;
    cw = cw < CW ? cw : CW;
    const int w0 = wave * cw;
    const int cnt = n - w0 <= 0 ? 0 : (n - w0 > cw ? cw : n - w0);
    const int hq0 = g * G;
    const int64_t row0 = (int64_t)(a.slot_base + s) * a.n_q_heads + hq0;
    unsigned char* vt = v_lds + wave * CW * VSTR;

    // Softmax state of one row per lane: the scores' reduce-scatter leaves
    // lane sub of each cell the row my_row of GS rows (the G real ones padded
    // to a power of two); lanes of a cell whose sub differs only in the kDup
    // bits hold the same row.
    constexpr int GS = scatter_rows<G>();
    constexpr int kDup = GS == 8 ? 0 : (GS == 4 ? 1 : (GS == 2 ? 3 : 7));
    const int my_row = scatter_row<GS>(sub);
    float m_r = kNegInf, l_r = 0.f, o[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = 0.f;

    if (cnt > 0) {
        // cell of the wave's row r; rows past the wave's cells read its first cell instead
        auto cell = [&](int r) -> int64_t { return sa.first + pos(w0 + (r < cnt ? r : 0)); };
        const uint8_t* kbase = a.k + (int64_t)g * a.k_hs;
        const uint8_t* vbase = a.v + (int64_t)g * a.v_hs;

        // 1. loads: the group's G query rows (contiguous, 2G floats per lane,
        // each element loaded once per wave), then the K and V chunks of the
        // lane's cells 8j + cl
        float2 qf[G];
        {
            const float2* qp = reinterpret_cast<const float2*>(a.q + row0 * D) + lane * G;
#pragma unroll
            for (int i = 0; i < G; ++i) qf[i] = qp[i];
        }
        __builtin_amdgcn_sched_barrier(0);
        Chunk<16> kc[JM][NC], vc[JM][NC];
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const uint8_t* kr = kbase + cell(j * CPL + cl) * a.k_cs;
#pragma unroll
            for (int c = 0; c < NC; ++c) kc[j][c] = load_chunk<16>(kr + (c * R + sub) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const uint8_t* vr = vbase + cell(j * CPL + cl) * a.v_cs;
#pragma unroll
            for (int c = 0; c < NC; ++c) vc[j][c] = load_chunk<16>(vr + (c * R + sub) * 16);
        }
        __builtin_amdgcn_sched_barrier(0);

        KVDEC_TRACE(1);
        // 2. query rows -> f16 pairs in the wave's LDS copy, then this lane's
        // pairs: elements (c * 8 + sub) * 8 .. + 8 of each row
#pragma unroll
        for (int i = 0; i < G; ++i)
            q_lds[wave][lane * G + i] = __builtin_bit_cast(uint32_t, h2{(_Float16)qf[i].x, (_Float16)qf[i].y});
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        h2 qh[G][NC * 4];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const uint4 x = *reinterpret_cast<const uint4*>(&q_lds[wave][h * (D / 2) + (c * R + sub) * 4]);
                qh[h][c * 4 + 0] = as_h2(x.x);
                qh[h][c * 4 + 1] = as_h2(x.y);
                qh[h][c * 4 + 2] = as_h2(x.z);
                qh[h][c * 4 + 3] = as_h2(x.w);
            }

        KVDEC_TRACE(2);
        // 3. scores (log2 units) of the lane's cells: the 8 lanes of a cell
        // hold partial dot products of the G rows, reduce-scattered so that
        // each lane gets the score of row my_row; then that row's maximum
        // over the wave's cells
        float sc[JM];
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            float acc[GS];
#pragma unroll
            for (int h = 0; h < GS; ++h) acc[h] = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const h2 kp = as_h2(kc[j][c].w[i]);
#pragma unroll
                    for (int h = 0; h < G; ++h) acc[h] = __builtin_amdgcn_fdot2(kp, qh[h][c * 4 + i], acc[h], false);
                }
            const float full = scatter_sum8<GS>(acc, sub);
            const bool live = j * CPL + cl < cnt && my_row < G;
            sc[j] = live ? full * a.scale_log2 : kNegInf;
        }
        {
            float mx = sc[0];
#pragma unroll
            for (int j = 1; j < JM; ++j) mx = fmaxf(mx, sc[j]);
            mx = fmaxf(mx, dpp<0x128>(mx));  // lane ^ 8: the other cell group of the row
            m_r = pair_max<32>(pair_max<16>(mx));
        }

        KVDEC_TRACE(3);
        // 4. weights, rounded to f16 (to nearest); l from the rounded values;
        // pairs of cells (8j + cl, 8j + cl + 1) to LDS from the even groups,
        // one lane per row
        const bool writer = (cl & 1) == 0 && (sub & kDup) == 0 && my_row < G;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const float p = (sc[j] == kNegInf) ? 0.f : exp2_fast(sc[j] - m_r + kPOff);
            const float pn = dpp<0x128>(p);
            const h2 pp = to_h2(p, pn);
            l_r += (float)pp.x;
            if (writer) p_lds[wave][j * (CPL / 2) + cl / 2][my_row] = __builtin_bit_cast(uint32_t, pp);
        }
        {
            float x = l_r;
            x += dpp<0x128>(x);
            l_r = pair_sum<32>(pair_sum<16>(x));
        }

        KVDEC_TRACE(4);
        // 5. per wave load j: its 8 V rows -> LDS, then P.V over them (lane
        // owns columns 2 lane, 2 lane + 1), the four row pairs at once (rows
        // past the wave's cells hold finite data of its first cell and carry
        // weight 0), so the block's LDS reads all leave before its products
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            if (j * CPL >= cnt) break;  // uniform over the wave
#ifdef KVDEC_PHASE_TRACE
            if (j == (cnt - 1) / CPL) {  // the wave's last V rows: wait for them, then stamp
                __builtin_amdgcn_s_waitcnt(0);
                KVDEC_TRACE_WAVE(22 + wave);
            }
#endif
#pragma unroll
            for (int c = 0; c < NC; ++c)
                *reinterpret_cast<uint4*>(vt + (j * CPL + cl) * VSTR + (c * R + sub) * 16) =
                    make_uint4(vc[j][c].w[0], vc[j][c].w[1], vc[j][c].w[2], vc[j][c].w[3]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint32_t va[CPL / 2], vb[CPL / 2];
            uint4 pw[CPL / 2][GP / 4];
#pragma unroll
            for (int qq = 0; qq < CPL / 2; ++qq) {
                const int pr = j * (CPL / 2) + qq;
                va[qq] = *reinterpret_cast<const uint32_t*>(vt + (2 * pr) * VSTR + 4 * lane);
                vb[qq] = *reinterpret_cast<const uint32_t*>(vt + (2 * pr + 1) * VSTR + 4 * lane);
#pragma unroll
                for (int x = 0; x < GP / 4; ++x) pw[qq][x] = *reinterpret_cast<const uint4*>(&p_lds[wave][pr][4 * x]);
            }
#pragma unroll
            for (int qq = 0; qq < CPL / 2; ++qq) {
                const h2 lo = as_h2(__builtin_amdgcn_perm(vb[qq], va[qq], 0x05040100u));
                const h2 hi = as_h2(__builtin_amdgcn_perm(vb[qq], va[qq], 0x07060302u));
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint4& q4 = pw[qq][h / 4];
                    const uint32_t wb = (h % 4 == 0) ? q4.x : (h % 4 == 1) ? q4.y : (h % 4 == 2) ? q4.z : q4.w;
                    const h2 w2 = as_h2(wb);
                    o[h][0] = __builtin_amdgcn_fdot2(lo, w2, o[h][0], false);
                    o[h][1] = __builtin_amdgcn_fdot2(hi, w2, o[h][1], false);
                }
            }
        }
    }

    KVDEC_TRACE_WAVE(5 + wave);
    // 6. merge the wave streams: thread t -> column t of the group's rows
    __syncthreads();  // every wave is done with its V tile
    float (*mg_o)[G][D] = reinterpret_cast<float (*)[G][D]>(v_lds);
    if (lane < R && (lane & kDup) == 0 && my_row < G) {  // cell group 0: one lane per row
        mg_m[wave][my_row] = m_r;
        mg_l[wave][my_row] = l_r * kPOffInv;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
        *reinterpret_cast<float2*>(&mg_o[wave][h][2 * lane]) = make_float2(o[h][0] * kPOffInv, o[h][1] * kPOffInv);
    __syncthreads();

    KVDEC_TRACE(13);
    const RowMap rm{row0, G, a.n_q_heads, G};
    const bool single = sa.n_splits == 1;
    const int64_t rec = sa.part_begin + (int64_t)g * sa.n_splits + split;
    const __amdgpu_buffer_rsrc_t rs = part_rsrc(a);
    for (int t = tid; t < G * D; t += 64 * W) {
        static_assert(W == 8 && D % 64 == 0, "stream factors in lanes 0..7, one row per wave");
        // A wave covers 64 columns of one row h (D is a multiple of 64): the
        // W streams' factors of the row are computed once, in lanes 0..W-1,
        // and read back as scalars; the sums keep the stream order.
        const int h = __builtin_amdgcn_readfirstlane(t / D), d = t - h * D;
        // every LDS read of the column first, so that their latencies overlap
        float ow[W];
#pragma unroll
        for (int w = 0; w < W; ++w) ow[w] = mg_o[w][h][d];
        const float mr = mg_m[lane % W][h], lr = mg_l[lane % W][h];
        const float mw = lane < W ? mr : kNegInf;
        float M = fmaxf(mw, dpp<0xB1>(mw));  // maximum over lanes 0..7
        M = fmaxf(M, dpp<0x4E>(M));
        M = fmaxf(M, dpp<0x141>(M));
        const float fw = (mw == kNegInf) ? 0.f : exp2_fast(mw - M);
        const float lw = lane < W ? lr : 0.f;
        M = lane_value(M, 0);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = lane_value(fw, w);
            L = fmaf(lane_value(lw, w), f, L);
            O = fmaf(ow[w], f, O);
        }
        if (single) {
            merge_acc_in1(a, rm.row(h), d, D, M, L, O);
            emit1(a, sa.to_acc, rm.row(h), d, D, M, L, O);
        } else {
            // (the builtin takes the 32 bits as an unsigned int: pass them, not a converted value)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O), rs, (int)(((rec * G + h) * D + d) * 4), 0, 0x10);
            if (d == 0) {
                st_dev(a.part_m + rec * G + h, M);
                st_dev(a.part_l + rec * G + h, L);
            }
        }
    }
    KVDEC_TRACE(14);
    if (single) return;
    arrive_and_merge<D, G, 64 * W>(a, sa, s, g, split, rm, sm_last);
}

// ---------------------------------------------------------------------------
// Wide-group kernel (G = 6..8 query heads per KV head): matrix-core path.
//
// With six or more query rows per KV head the VALU path runs out of issue
// slots before HBM does (int8 / 4-bit rows also need dequantisation), so the
// two contractions of a 32-cell step go to v_mfma_f32_16x16x32_f16, the G
// query rows padded to 16 with zero rows:
//   S^T[cell][head] = K^[cell][:] . q[head][:]   (A = K^ rows, B = q^T)
//   O[head][d]     += P[head][cell] . V^[cell][d] (A = P, B = V^)
// Operand layouts (measured on gfx950): A[i][k] sits in lane i + 16*(k/8),
// element k%8; B[k][j] in lane j + 16*(k/8); D[i][j] in lane j + 16*(i/4),
// element i%4.  The order of the contraction index is free, so
//  * for S, lane group q of a 16-cell block reads 16-byte chunks q, q+4, ...
//    of its cell's row and q is loaded in the same permuted element order,
//    so every chunk feeds whole MFMAs without any shuffle;
//  * for P.V, the 8 contraction slots of lane group q are cells 4q..4q+3 of
//    the step's two 16-cell blocks -- exactly the scores that lane holds
//    after the S product -- so P never moves between lanes.
// V^ is dequantised (d * code rounded to f16) into a per-wave LDS tile of 32
// rows and read back column-wise with ds_read_b64_tr_b16, whose 16-lane 4x4
// transpose delivers the B operand.  Each wave is one online-softmax stream;
// the waves (four, or eight for 16-row records at head_dim 128) are merged at
// the end like the VALU path's streams.
// ---------------------------------------------------------------------------
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));

// Elements per 16-byte chunk of a stored row.
template <int T>
struct Row16 {
    static constexpr int EPC = T == KVDEC_F16 ? 8 : T == KVDEC_Q8_B32 ? 16 : 32;
};

// Order of the elements of a 4-bit chunk in the matrix-core kernel's f16
// pairs: pair 4w + k of dword w holds elements 8w + a and 8w + a + 2 with
// a = 0, 4, 1, 5 for k = 0..3 -- even elements from the low nibbles, odd
// ones from the high nibbles, each pair one byte permute against the f16
// exponent byte.  Slot i of an 8-element group holds element q4_order(i).
__device__ __forceinline__ constexpr int q4_order(int i) { return (i & 3) * 2 + (i >> 2); }

// One 16-byte chunk -> its EPC values as f16 pairs (block-scaled kinds: d * code,
// rounded to f16).  4-bit chunks come out in q4_order within each 8 elements.
template <int T>
__device__ __forceinline__ void dequant16(const Chunk<16>& c, uint16_t scale_bits, h2 (&out)[Row16<T>::EPC / 2]) {
    if constexpr (T == KVDEC_Q4_B32) {
        // 1024 + u in each f16 (exponent byte 0x64 above the nibble), minus
        // 1032: u - 8 exactly
        const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = c.w[w] & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6 of the dword
            const uint32_t hi = (c.w[w] >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
            out[4 * w + 0] = as_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - bias;  // 0, 2
            out[4 * w + 1] = as_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - bias;  // 4, 6
            out[4 * w + 2] = as_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - bias;  // 1, 3
            out[4 * w + 3] = as_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - bias;  // 5, 7
        }
    } else {
        to_pairs<T>(c, out);
    }
    if constexpr (T != KVDEC_F16) {
        const _Float16 d = __builtin_bit_cast(_Float16, scale_bits);
        const h2 dd = {d, d};
#pragma unroll
        for (int i = 0; i < Row16<T>::EPC / 2; ++i) out[i] = out[i] * dd;
    }
}

// Workgroup order seen by the work decomposition.  The dispatcher hands
// workgroups to the 8 XCDs round-robin (workgroup b to XCD b % 8), and each
// XCD has its own L2.  Renumbering so that consecutive logical indices land
// on the same XCD puts the KV heads of one split -- which share the cache
// lines of the cells' block scales and plan entries -- behind one L2.  Only
// a bijection of [0, n): correctness never depends on the placement.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical_index(int b, int n) {
    const int per = n / kXcds, extra = n % kXcds;
    const int x = b % kXcds, k = b / kXcds;
    return (x < extra ? x * (per + 1) : extra * (per + 1) + (x - extra) * per) + k;
}

// Scale of the 32-element block holding chunk lq + 4j of a row, taken from
// the row's SB bytes of scales.  int8: 16 elements per chunk, so the block is
// 2j + lq/2 (dword j); 4-bit: 32 per chunk, block lq + 4j (half lq of dwords 2j, 2j+1).
template <int T, int SB>
__device__ __forceinline__ uint16_t scale_of(const Chunk<SB>& r, int j, int lq) {
    if constexpr (T == KVDEC_Q8_B32) {
        return (uint16_t)(r.w[j] >> (16 * (lq >> 1)));
    } else if constexpr (T == KVDEC_Q4_B32) {
        // halves 4j..4j+3 of the row as one 64-bit value (no lane-dependent
        // register index, which would go through scratch memory)
        const uint64_t x = (uint64_t)r.w[2 * j] | ((uint64_t)r.w[2 * j + 1] << 32);
        return (uint16_t)(x >> (16 * lq));
    } else {
        return 0;
    }
}

template <int D, int RM, int KT, int VT, bool IND, bool MQ, int W>
__global__ __launch_bounds__(64 * W) void split_mfma_kernel(const SplitArgs a) {
    // RM: rows of a split record (8 or 16); the G * n_q real query rows of
    // the (slot, KV head) are padded to RM and to the 16-row tile.
    static_assert(RM == 8 || RM == 16, "record rows");
    constexpr int G = RM;  // record rows, for the shared publish / merge code
    constexpr int EK = Row16<KT>::EPC, EV = Row16<VT>::EPC;
    constexpr int JK = D / EK / 4, JV = D / EV / 4;  // chunks per lane per row
    static_assert(JK >= 1 && JV >= 1 && JK * 4 * EK == D && JV * 4 * EV == D, "row chunking");
    constexpr int NKB = D / 32;                    // S MFMAs per 16-cell block
    constexpr int NNB = D / 16;                    // P.V MFMAs (16-column blocks of O)
    constexpr int NB = D / kBlock;                 // scales per row
    constexpr int SB = NB * 2;                     // bytes of one row of scales
    constexpr int VSTR = 2 * D + 32;               // bytes per staged V row (padded)
    constexpr int STAGE = W * 32 * VSTR;           // V staging of the W waves
    constexpr int MERGE = W * G * 4 * 2 + W * G * D * 4;
    constexpr int SC = 32 * W;                     // cells per workgroup step (32 per wave)
    constexpr int SMEM = STAGE > MERGE ? STAGE : MERGE;
    __shared__ __align__(16) unsigned char smem[SMEM];
    __shared__ int sm_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;  // row / column index inside a 16-lane group
    const int lq = lane >> 4;  // lane group

    // With live_records the splits in use are a prefix of each slot's
    // range: the dispatch order itself (workgroup b on XCD b % 8) spreads
    // them evenly over the XCDs, where per-XCD blocks of the renumbering
    // could leave one XCD all of them.
    const int wg = a.live_records ? (int)blockIdx.x : xcd_logical_index(blockIdx.x, a.n_workgroups);
    int s = 0;
    while (s + 1 < a.n_slots && a.slot[s + 1].wg_begin <= wg) ++s;
    const SlotArg sa = a.slot[s];
    const int local = wg - sa.wg_begin;
    const int split = local / a.n_kv_heads;
    const int g = local - split * a.n_kv_heads;
    if (split >= live_splits(a, sa, s)) return;  // nothing in use: not part of the merge
    const int64_t base0 = (((int64_t)split * sa.n_units) / sa.n_splits) * a.split_unit;
    const int64_t span_end = (((int64_t)(split + 1) * sa.n_units) / sa.n_splits) * a.split_unit;
    // Record row r = t * grp + hh is query row t of the slot, head g * grp + hh.
    const int grp = a.group;
    const int rows = grp * a.n_q;
    const RowMap rm{(int64_t)(a.slot_base + s) * a.n_q * a.n_q_heads + (int64_t)g * grp, grp, a.n_q_heads, rows};
    const bool real_row = li < rows;
    // Position of this lane's query row (multi-query): it sees cells whose
    // position is at most qpos; padding rows see nothing.
    int64_t qpos = INT64_MIN;
    if constexpr (MQ)
        if (real_row) qpos = a.q_pos[(int64_t)(a.slot_base + s) * a.n_q + li / grp];

    // B operand of S: q rows (zero rows past the real ones) in the permuted
    // order of the K chunks this lane group reads.  Loads are unconditional
    // (row clamped) so that they all leave before the first wait.
    h8 qb[NKB];
    {
        const float* qr = a.q + rm.row(real_row ? li : 0) * D;
#pragma unroll
        for (int j = 0; j < JK; ++j) {
#pragma unroll
            for (int sub = 0; sub < EK / 8; ++sub) {
                const int e0 = (lq + 4 * j) * EK + 8 * sub;
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float2 v = *reinterpret_cast<const float2*>(qr + e0 + e);
                    x[e] = v.x;
                    x[e + 1] = v.y;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // 4-bit K comes out of dequant16 in q4_order: q follows it
                    const float xe = KT == KVDEC_Q4_B32 ? x[q4_order(e)] : x[e];
                    qb[j * (EK / 8) + sub][e] = real_row ? (_Float16)xe : (_Float16)0.0f;
                }
            }
        }
    }

    // Online softmax of head li (identical over the 4 lane groups).  The
    // reference m_h moves only when a score exceeds it by more than kLazy,
    // so the O tile is rarely rescaled; weights 2^(s - m_h + kMPOff) then stay
    // below 2^15 and remain normal f16 numbers far below the maximum.
    constexpr float kLazy = 6.0f;
    constexpr float kMPOff = 9.0f;
    constexpr float kMPOffInv = 1.0f / 512.0f;
    float m_h = kNegInf, l_h = 0.f;
    f4v oacc[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) oacc[nb] = f4v{0.f, 0.f, 0.f, 0.f};

    const uint8_t* kbase = a.k + (int64_t)g * a.k_hs;
    const uint8_t* vbase = a.v + (int64_t)g * a.v_hs;
    unsigned char* vst = smem + wave * 32 * VSTR;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    const int64_t slot_end = live_end(a, sa, s);
    const int64_t pos_end = span_end < slot_end ? span_end : slot_end;
    // one step per SC positions: 32 cells per wave
    const int n_steps = pos_end > base0 ? (int)((pos_end - base0 + SC - 1) / SC) : 0;

    // Cells of a step: lane li owns cell li of the wave's two 16-cell blocks,
    // block mb of wave w at (mb * W + w) * 16 of the step: each wave's cells
    // spread over the step instead of one contiguous 32-cell block (4-bit
    // GQA-6 80.4 -> 77.9 us, 4-query layer 24.8 -> 24.2 us).
    // Loads never branch: an invalid cell reads row 0 of the cache instead,
    // its score is masked and its V row is zeroed where it is consumed.  Raw
    // plan entries are fetched two steps ahead and left untouched until the
    // step before their use, and the K / V loads of step i+1 leave while
    // step i computes, so no wait falls on data that is not needed yet.
    const int32_t* plan_s = IND ? a.plan + sa.first : nullptr;
    auto fetch = [&](int64_t base, int mb) -> int32_t {
        if constexpr (IND) {
            const int64_t pos = base + (mb * W + wave) * 16 + li;
            return plan_s[pos < pos_end ? pos : pos_end - 1];
        } else {
            return 0;
        }
    };
    auto resolve = [&](int64_t base, int mb, int32_t raw, int64_t& cell, bool& valid) {
        const int64_t pos = base + (mb * W + wave) * 16 + li;
        if constexpr (IND) {
            valid = pos < pos_end && raw >= 0 && raw < a.capacity;
            cell = valid ? raw : 0;
        } else {
            valid = pos < pos_end;
            cell = valid ? sa.first + pos : 0;
        }
    };
    Chunk<16> kc[2][JK], vc[2][JV];
    Chunk<SB> kr_s[2], vr_s[2];  // scale rows of the two cells (block-scaled kinds)
    auto load_k = [&](const int64_t (&cell)[2]) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const uint8_t* kr = kbase + cell[mb] * a.k_cs;
#pragma unroll
            for (int j = 0; j < JK; ++j) kc[mb][j] = load_chunk<16>(kr + (lq + 4 * j) * 16);
            if constexpr (KT != KVDEC_F16)
                kr_s[mb] = load_chunk<SB>(reinterpret_cast<const uint8_t*>(a.ks) + (cell[mb] * a.n_kv_heads + g) * SB);
        }
    };
    auto load_v = [&](const int64_t (&cell)[2]) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const uint8_t* vr = vbase + cell[mb] * a.v_cs;
#pragma unroll
            for (int j = 0; j < JV; ++j) vc[mb][j] = load_chunk<16>(vr + (lq + 4 * j) * 16);
            if constexpr (VT != KVDEC_F16)
                vr_s[mb] = load_chunk<SB>(reinterpret_cast<const uint8_t*>(a.vs) + (cell[mb] * a.n_kv_heads + g) * SB);
        }
    };

    // Multi-query: positions of a step's cells come from cell_pos (loaded a
    // step ahead, left untouched until used) or are cell index + pos_offset.
    auto fetch_pos = [&](const int64_t (&c)[2], int32_t (&raw)[2]) {
        if constexpr (MQ) {
            if (a.cell_pos) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) raw[mb] = a.cell_pos[c[mb]];
            }
        }
    };

    int32_t raw_next[2] = {0, 0};
    int32_t praw[2] = {0, 0};
    int64_t cell[2] = {0, 0};
    bool valid[2] = {false, false};
    if (n_steps > 0) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            resolve(base0, mb, fetch(base0, mb), cell[mb], valid[mb]);
            raw_next[mb] = fetch(base0 + SC, mb);
        }
        fetch_pos(cell, praw);
        load_k(cell);
        __builtin_amdgcn_sched_barrier(0);  // same issue order as in the loop: K, then V
        load_v(cell);
        if constexpr (MQ) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                int32_t t;
                asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(praw[mb]));
                praw[mb] = t;
            }
        }
        if constexpr (IND) {
            // Land the step-1 entries here, behind an opaque copy: entering the
            // loop with a load still pending on them would make the compiler
            // wait for every prefetched K / V load at the top of each step.
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                int32_t t;
                asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(raw_next[mb]));
                raw_next[mb] = t;
            }
        }
    }

    for (int st = 0; st < n_steps; ++st) {
        const int64_t base = base0 + (int64_t)st * SC;
        const uint64_t vm0 = __ballot(valid[0]), vm1 = __ballot(valid[1]);
        int32_t raw2[2];
        int64_t ncell[2];
        bool nvalid[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            raw2[mb] = fetch(base + 2 * SC, mb);
            resolve(base + SC, mb, raw_next[mb], ncell[mb], nvalid[mb]);
        }
        int32_t npraw[2] = {0, 0};
        fetch_pos(ncell, npraw);
        // Multi-query mask: bit e of vis[mb] = cell 4 * lq + e of block mb is
        // visible to this lane's query row.
        uint32_t vis[2] = {0xFu, 0xFu};
        if constexpr (MQ) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                uint32_t bits = 0;
                if (!IND && !a.cell_pos) {
                    // contiguous cells without explicit positions: the
                    // position of cell 4 * lq + e of the block is known here
                    const int64_t p0 = sa.first + base + (mb * W + wave) * 16 + 4 * lq + a.pos_offset;
#pragma unroll
                    for (int e = 0; e < 4; ++e) bits |= (p0 + e <= qpos ? 1u : 0u) << e;
                } else {
                    const int64_t mine = a.cell_pos ? (int64_t)praw[mb] : cell[mb] + a.pos_offset;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t p = __shfl(mine, 4 * lq + e);
                        bits |= (p <= qpos ? 1u : 0u) << e;
                    }
                }
                vis[mb] = bits;
            }
        }

        // S^T for the two blocks.
        f4v sacc[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int j = 0; j < JK; ++j) {
                h2 kp[EK / 2];
                dequant16<KT>(kc[mb][j], scale_of<KT, SB>(kr_s[mb], j, lq), kp);
#pragma unroll
                for (int sub = 0; sub < EK / 8; ++sub) {
                    h8 av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        av[2 * e] = kp[4 * sub + e].x;
                        av[2 * e + 1] = kp[4 * sub + e].y;
                    }
                    sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[j * (EK / 8) + sub], sacc[mb], 0, 0, 0);
                }
            }
        }
        load_k(ncell);  // K of the next step (its registers are free now)
        // phase fence for the scheduler: V data is consumed only below
        __builtin_amdgcn_sched_barrier(0);

        // Scores of head li for cells 4*lq + e of each block (log2 units).
        // bit e: cell 4 * lq + e of the block is valid (the ballot's bit of
        // the lane that loaded it) and visible to this lane's query row
        const uint32_t live0 = (uint32_t)(vm0 >> (4 * lq)) & vis[0] & 0xFu;
        const uint32_t live1 = (uint32_t)(vm1 >> (4 * lq)) & vis[1] & 0xFu;
        float sc[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sc[e] = ((live0 >> e) & 1u) ? sacc[0][e] * a.scale_log2 : kNegInf;
            sc[4 + e] = ((live1 >> e) & 1u) ? sacc[1][e] * a.scale_log2 : kNegInf;
        }
        float mt = sc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sc[e]);
        mt = pair_max<32>(pair_max<16>(mt));
        const bool bump = mt > m_h + kLazy;  // also the first finite score
        const float mn = bump ? mt : m_h;
        const float alpha = bump ? exp2_fast(m_h - mn) : 1.f;
        const bool rescale = bump && m_h != kNegInf;
        m_h = mn;
        // Each weight as an f16 pair hi + lo: hi is p rounded to nearest,
        // lo the residual p - hi (exact in f32) rounded again, so hi + lo
        // carries p to about 2^-22 of itself.  A single f16 weight would
        // re-weight two cells by up to 2^-11 of each weight -- on two cells
        // of near-equal score and values v1, v2 an error of up to
        // 2^-12 |v1 - v2| in the output.
        h8 pa, pl;
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float p0 = (sc[e] == kNegInf) ? 0.f : exp2_fast(sc[e] - mn + kMPOff);
            const float p1 = (sc[e + 1] == kNegInf) ? 0.f : exp2_fast(sc[e + 1] - mn + kMPOff);
            const h2 pp = to_h2(p0, p1);
            const h2 pr = to_h2(p0 - (float)pp.x, p1 - (float)pp.y);
            pa[e] = pp.x;
            pa[e + 1] = pp.y;
            pl[e] = pr.x;
            pl[e + 1] = pr.y;
            lsum = __builtin_amdgcn_fdot2(pp, ones, lsum, false);
            lsum = __builtin_amdgcn_fdot2(pr, ones, lsum, false);
        }
        lsum = pair_sum<32>(pair_sum<16>(lsum));
        l_h = l_h * alpha + lsum;
        // O rows held by this lane are heads 4*lq + e: rescale with their alphas.
        if (__ballot(rescale) != 0) {
            float ae[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ae[e] = __shfl(alpha, 4 * lq + e);
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[nb][e] *= ae[e];
        }

        __builtin_amdgcn_sched_barrier(0);
        // V^ rows of the step -> LDS (row = 16*block + cell), f16.
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int j = 0; j < JV; ++j) {
                const int c = lq + 4 * j;
                h2 vp[EV / 2];
                if constexpr (VT == KVDEC_F16) {
                    Chunk<16> x = vc[mb][j];
#pragma unroll
                    for (int w = 0; w < 4; ++w) x.w[w] = valid[mb] ? x.w[w] : 0u;
                    dequant16<VT>(x, 0, vp);
                } else {
                    dequant16<VT>(vc[mb][j], valid[mb] ? scale_of<VT, SB>(vr_s[mb], j, lq) : (uint16_t)0, vp);
                }
                uint4* dst = reinterpret_cast<uint4*>(vst + (16 * mb + li) * VSTR + c * EV * 2);
#pragma unroll
                for (int w = 0; w < EV / 8; ++w)
                    dst[w] = make_uint4(__builtin_bit_cast(uint32_t, vp[4 * w]), __builtin_bit_cast(uint32_t, vp[4 * w + 1]),
                                        __builtin_bit_cast(uint32_t, vp[4 * w + 2]),
                                        __builtin_bit_cast(uint32_t, vp[4 * w + 3]));
            }
        }
        load_v(ncell);  // V of the next step
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // O += P . V^: B operand by transposing 16-lane reads of the staged rows.
        typedef __attribute__((address_space(3))) fp16x4_t lds_h4;
        const int r_lo = 4 * lq + (li >> 2);  // staged row of block 0 read by this lane
        const int col = 4 * (li & 3);
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
            const int cb = (16 * nb + col) * 2;
            // generic -> LDS address space (C-style cast: the pointer is in smem)
            lds_h4* p0 = (lds_h4*)(vst + r_lo * VSTR + cb);
            lds_h4* p1 = (lds_h4*)(vst + (16 + r_lo) * VSTR + cb);
            const fp16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(p0);
            const fp16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(p1);
            h8 vb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vb[e] = (_Float16)v0[e];
                vb[4 + e] = (_Float16)v1[e];
            }
            oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, oacc[nb], 0, 0, 0);
            oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, vb, oacc[nb], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            raw_next[mb] = raw2[mb];
            praw[mb] = npraw[mb];
            cell[mb] = ncell[mb];
            valid[mb] = nvalid[mb];
        }
    }

    // Each wave is one stream: (m2, l, o) of heads < G -> LDS, then merge.
    __syncthreads();  // the V staging area is reused for the merge arrays
    float (*sm_m)[G] = reinterpret_cast<float (*)[G]>(smem);
    float (*sm_l)[G] = reinterpret_cast<float (*)[G]>(smem + W * G * 4);
    float (*sm_o)[G][D] = reinterpret_cast<float (*)[G][D]>(smem + W * G * 4 * 2);
    if (lq == 0 && li < G) {
        sm_m[wave][li] = m_h;
        sm_l[wave][li] = l_h * kMPOffInv;
    }
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int h = 4 * lq + e;
            // staged 4-bit V columns sit in q4_order within each 8 columns
            const int col = VT == KVDEC_Q4_B32 ? ((16 * nb + li) & ~7) + q4_order(li & 7) : 16 * nb + li;
            if (h < G) sm_o[wave][h][col] = oacc[nb][e] * kMPOffInv;
        }
    __syncthreads();
    finish_split<D, G, W, D, 64 * W>(a, sa, s, g, split, rm, sm_m, sm_l, sm_o, sm_last);
}

template <int D, int G, int KT, int VT>
int launch_valu(const SplitArgs& a, void* stream) {
    // one-shot splits: head_dim 128, f16 K and V, up to 5 query rows
    if constexpr (D == 128 && G <= 5 && KT == KVDEC_F16 && VT == KVDEC_F16) {
        if (a.oneshot > 0 && !a.plan) {
            if (a.split_unit != kSplitUnit) return (int)hipErrorInvalidValue;  // the kernel's unit is a constant
            const hipStream_t st = (hipStream_t)stream;
            if (a.oneshot <= 2)
                hipLaunchKernelGGL((split_oneshot_kernel<G, 2>), dim3(a.n_workgroups), dim3(512), 0, st, a);
            else if (a.oneshot <= 4)
                hipLaunchKernelGGL((split_oneshot_kernel<G, 4>), dim3(a.n_workgroups), dim3(512), 0, st, a);
            else
                hipLaunchKernelGGL((split_oneshot_kernel<G, 7>), dim3(a.n_workgroups), dim3(512), 0, st, a);
            return (int)hipGetLastError();
        }
    }
    // eight-wave workgroups: head_dim up to 128 (their stream-merge area fits LDS)
    if constexpr (D <= 128 && KT == KVDEC_F16 && VT == KVDEC_F16) {
        if (a.waves == 8) {
            hipLaunchKernelGGL((split_kernel<D, G, KT, VT, 8>), dim3(a.n_workgroups), dim3(512), 0,
                               (hipStream_t)stream, a);
            return (int)hipGetLastError();
        }
    }
    hipLaunchKernelGGL((split_kernel<D, G, KT, VT, 4>), dim3(a.n_workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                       a);
    return (int)hipGetLastError();
}

template <int D, int RM, int KT, int VT, bool MQ>
int launch_mfma(const SplitArgs& a, void* stream) {
    // eight-wave workgroups for 16-row records at head_dim 128 (at 256 the
    // f16 and int8 instances would spill registers)
    if constexpr (D == 128 && RM == 16) {
        if (a.waves == 8) {
            if (a.plan)
                hipLaunchKernelGGL((split_mfma_kernel<D, RM, KT, VT, true, MQ, 8>), dim3(a.n_workgroups), dim3(512), 0,
                                   (hipStream_t)stream, a);
            else
                hipLaunchKernelGGL((split_mfma_kernel<D, RM, KT, VT, false, MQ, 8>), dim3(a.n_workgroups), dim3(512),
                                   0, (hipStream_t)stream, a);
            return (int)hipGetLastError();
        }
    }
    if (a.plan)
        hipLaunchKernelGGL((split_mfma_kernel<D, RM, KT, VT, true, MQ, 4>), dim3(a.n_workgroups), dim3(kThreads), 0,
                           (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL((split_mfma_kernel<D, RM, KT, VT, false, MQ, 4>), dim3(a.n_workgroups), dim3(kThreads), 0,
                           (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

// Vector-ALU instances exist only where the picker can select them.
template <int D, int G, int KT, int VT>
SplitLaunchFn valu_fn() {
    if constexpr (uses_matrix_cores(G, 1, D))
        return nullptr;
    else
        return &launch_valu<D, G, KT, VT>;
}

// The instance for (G, n_q) at one head_dim and pair of storage kinds: the
// VALU kernel (mfma false; one query row and G <= 5, any G <= 8 for
// head_dim 64), or the matrix-core kernel with 8- or 16-row records
// (head_dim 128 / 256, G * n_q <= 16).
template <int D, int KT, int VT>
SplitLaunchFn pick_g(int g, int n_q, bool mfma) {
    if (g < 1 || n_q < 1) return nullptr;
    if (!mfma) {
        if (n_q != 1) return nullptr;
        switch (g) {
            case 1: return valu_fn<D, 1, KT, VT>();
            case 2: return valu_fn<D, 2, KT, VT>();
            case 3: return valu_fn<D, 3, KT, VT>();
            case 4: return valu_fn<D, 4, KT, VT>();
            case 5: return valu_fn<D, 5, KT, VT>();
            case 6: return valu_fn<D, 6, KT, VT>();
            case 7: return valu_fn<D, 7, KT, VT>();
            case 8: return valu_fn<D, 8, KT, VT>();
            default: return nullptr;
        }
    }
    if constexpr (D >= 128) {
        if (g * n_q > 16) return nullptr;
        const bool wide = record_rows_of(true, g, n_q) == 16;
        if (n_q == 1) return wide ? &launch_mfma<D, 16, KT, VT, false> : &launch_mfma<D, 8, KT, VT, false>;
        return wide ? &launch_mfma<D, 16, KT, VT, true> : &launch_mfma<D, 8, KT, VT, true>;
    }
    return nullptr;
}

// Every (head_dim, group, n_q) instance of one pair of storage kinds.
template <int KT, int VT>
SplitLaunchFn pick_dg(int head_dim, int g, int n_q, bool mfma) {
    switch (head_dim) {
        case 64: return pick_g<64, KT, VT>(g, n_q, mfma);
        case 128: return pick_g<128, KT, VT>(g, n_q, mfma);
        case 256: return pick_g<256, KT, VT>(g, n_q, mfma);
        default: return nullptr;
    }
}

}  // namespace
}  // namespace kvdec

"""Float64 CPU oracle for grouped-query decode attention over a KV cache --
single-query (n_q = 1) and multi-query with a positional mask -- with
block-scaled int8 / 4-bit caches, indirect cell plans and the log-sum-exp
merge of partial results.

Test infrastructure only: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP library and imports nothing from it.  Every function is written to be read
against its definition, not to be fast.

Sources (web pages, cited by title and section):

* "Rolling-KV -- overflow throughput evaluations (consolidated)", section 1
  (resident window plus a host tail re-read every step) and section 3 (the
  log-sum-exp channel that lets a window result and a tail result combine).
* "KVARN KV Performance optimizations" (beellama.cpp issue 140), "What was
  implemented" item 3 (duplicate filtering, first occurrence kept, capacity
  checks), item 4 (plans grouped by physical 128-cell record, one monotonic
  segment per record, -1 holes kept), item 7 (split decode for up to 8 query
  rows, which needs an attention mask) and item 9 (partial windows keep the
  running maximum, numerator and denominator and are merged afterwards).

Readings where the pages are silent:

* query head h reads KV head floor(h / G), G = n_q_heads / n_kv_heads;
* scores are ``scale * q . k``; exponentials are natural (e^x); a partial's m
  is in score units and its l and o are relative to e^m, o unnormalised;
* int8 blocks dequantise as ``d * q`` and 4-bit blocks as ``d * (u - 8)``,
  with one f16 scale ``d`` per 32 consecutive elements of one (cell, KV head)
  row; element 2i of a 4-bit row is the low nibble of byte i, 2i+1 the high;
* an empty set of cells gives output 0 and lse -inf; the empty partial is
  (-inf, 0, 0);
* an indirect entry -1 is a hole (skipped); any other entry is attended with
  multiplicity (the plan builder is what removes duplicates);
* no positional mask with one query: every attended cell is visible; with
  several query rows per slot, row t at position q_pos[s][t] sees the cells
  whose position (cell_pos[c], or the cell index c) is at most q_pos[s][t].

Pins (tests/test_oracle_pins.py): exhaustive f16 decoding against the IEEE
formula, the dequantisation table, closed forms (one cell, two cells,
constant scores, hard-max limit), a 50-digit mpmath brute force on tiny inputs,
torch's float64 scaled_dot_product_attention with repeated KV heads, merge
invariants (partition, associativity, empty identity), permutation, hole and
duplicate invariants, and hand-worked compact-plan examples.
"""

import math

import numpy as np

# KV storage kinds.
F16 = 0      # IEEE binary16, one value per element
Q8_B32 = 1   # int8 codes, one f16 scale per 32 elements
Q4_B32 = 2   # 4-bit codes (two per byte), one f16 scale per 32 elements

BLOCK = 32          # elements that share one f16 scale
RECORD_CELLS = 128  # cells per physical record of an indirect plan


def f16_bits_to_f64(bits):
    """IEEE binary16 bit patterns (uint16) to float64; exact for every pattern."""
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return a.view(np.float16).astype(np.float64)


def row_elems(kind, head_dim):
    """Stored code elements per (cell, KV head) row: f16 values, int8 codes, or
    bytes of packed 4-bit codes."""
    if kind == Q4_B32:
        return head_dim // 2
    return head_dim


def dequantize(kind, codes, scales=None):
    """Dequantise stored rows to float64.

    ``codes`` has shape [..., row_elems]; ``scales`` (uint16 f16 bit patterns)
    has shape [..., head_dim / 32] for the block-scaled kinds.  Returns float64
    [..., head_dim].
    """
    if kind == F16:
        return f16_bits_to_f64(codes)
    d = f16_bits_to_f64(scales)
    d_per_elem = np.repeat(d, BLOCK, axis=-1)
    if kind == Q8_B32:
        q = np.asarray(codes).astype(np.int8).astype(np.float64)
        return d_per_elem * q
    if kind == Q4_B32:
        b = np.asarray(codes).astype(np.uint8)
        low = (b & 0x0F).astype(np.float64) - 8.0   # element 2i
        high = (b >> 4).astype(np.float64) - 8.0    # element 2i + 1
        u = np.stack([low, high], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])
        return d_per_elem * u
    raise ValueError(f"unknown KV kind {kind}")


def attend_row(q, k_hat, v_hat, scale):
    """Softmax attention of one query row over n cells, in float64.

    q [D]; k_hat, v_hat [n, D].  Returns (out [D], lse).  With n = 0 the output
    is zero and lse is -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[0]
    if k_hat.shape[0] == 0:
        return np.zeros(d), -math.inf
    s = scale * (k_hat @ q)          # one score per cell
    m = s.max()
    w = np.exp(s - m)                 # weights relative to the maximum
    l = w.sum()
    out = (w @ v_hat) / l
    return out, m + math.log(l)


def partial_row(q, k_hat, v_hat, scale):
    """Online-softmax partial of one query row over a subset of cells:
    (m, l, o) with m the maximum score, l = sum e^(s - m) and o = sum
    e^(s - m) v (unnormalised).  The empty subset gives (-inf, 0, 0)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[0]
    if k_hat.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(d)
    s = scale * (k_hat @ q)
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ v_hat


def merge_partials(parts):
    """Log-sum-exp merge of partials [(m, l, o), ...] of disjoint cell subsets.

    M = max m_p;  L = sum l_p e^(m_p - M);  O = sum o_p e^(m_p - M);
    out = O / L;  lse = M + ln L.  Partials with m = -inf contribute nothing;
    if all are empty, out = 0 and lse = -inf.  Returns (out, lse, (M, L, O)).
    """
    parts = list(parts)
    d = len(parts[0][2])
    live = [p for p in parts if p[0] != -math.inf]
    if not live:
        return np.zeros(d), -math.inf, (-math.inf, 0.0, np.zeros(d))
    big_m = max(p[0] for p in live)
    big_l = 0.0
    big_o = np.zeros(d)
    for m, l, o in live:
        f = math.exp(m - big_m)
        big_l += l * f
        big_o = big_o + np.asarray(o, dtype=np.float64) * f
    return big_o / big_l, big_m + math.log(big_l), (big_m, big_l, big_o)


def _rows(cache, cells, kv_head):
    """Dequantised float64 rows [len(cells), D] of one KV head of a cache.

    ``cache`` is (kind, codes, scales): codes [n_cells][n_kv_heads][row_elems],
    scales [n_cells][n_kv_heads][D/32] or None.
    """
    kind, codes, scales = cache
    idx = np.asarray(cells, dtype=np.int64)
    c = np.asarray(codes)[idx, kv_head]
    s = None if scales is None else np.asarray(scales)[idx, kv_head]
    return dequantize(kind, c, s)


def decode_attention(q, regions, n_kv_heads, scale, return_partials=False):
    """Single-query grouped-query decode attention over one or more regions.

    q: [S][Hq][D] (any float dtype; used as float64).
    regions: list of (k_cache, v_cache, cells) where each cache is
        (kind, codes, scales) as in ``_rows`` and ``cells`` is a list of S
        integer sequences (the cells of each slot inside that region).  An
        entry of -1 is a hole and is skipped; every other entry is attended,
        with multiplicity.  The attended set of a slot is the union over the
        regions (e.g. a resident window and a host tail).

    Returns out [S][Hq][D] and lse [S][Hq] in float64, and with
    ``return_partials`` also the per-region partials [(m, l, o) arrays].
    """
    q = np.asarray(q, dtype=np.float64)
    n_slots, n_q_heads, head_dim = q.shape
    group = n_q_heads // n_kv_heads
    out = np.zeros((n_slots, n_q_heads, head_dim))
    lse = np.full((n_slots, n_q_heads), -math.inf)
    region_parts = [
        (np.full((n_slots, n_q_heads), -math.inf),
         np.zeros((n_slots, n_q_heads)),
         np.zeros((n_slots, n_q_heads, head_dim)))
        for _ in regions
    ]
    for s in range(n_slots):
        for g in range(n_kv_heads):
            ks, vs = [], []
            per_region = []
            for k_cache, v_cache, cells in regions:
                live = [int(c) for c in cells[s] if int(c) != -1]
                k_hat = _rows(k_cache, live, g)
                v_hat = _rows(v_cache, live, g)
                ks.append(k_hat)
                vs.append(v_hat)
                per_region.append((k_hat, v_hat))
            k_all = np.concatenate(ks, axis=0)
            v_all = np.concatenate(vs, axis=0)
            for h in range(g * group, (g + 1) * group):
                out[s, h], lse[s, h] = attend_row(q[s, h], k_all, v_all, scale)
                if return_partials:
                    for r, (k_hat, v_hat) in enumerate(per_region):
                        m, l, o = partial_row(q[s, h], k_hat, v_hat, scale)
                        region_parts[r][0][s, h] = m
                        region_parts[r][1][s, h] = l
                        region_parts[r][2][s, h] = o
    if return_partials:
        return out, lse, region_parts
    return out, lse


def decode_attention_multi(q, regions, n_kv_heads, scale, q_pos, cell_pos=None):
    """Multi-query decode attention with a positional (causal) mask: several
    query rows per slot, as in speculative verification, where split decoding
    serves up to 8 query rows and a multi-query call must carry an attention
    mask ("KVARN KV Performance optimizations", "What was implemented"
    item 7).

    q: [S][NQ][Hq][D], query row t of slot s at position q_pos[s][t].
    regions: as in ``decode_attention``.
    cell_pos: None (a cell's position is its cell index) or an integer array
        indexed by cell.
    Query row (s, t) attends to every cell of slot s (holes skipped,
    multiplicity kept, union over the regions) whose position is at most
    q_pos[s][t]; a row that sees no cell gets output 0 and lse -inf.

    Returns out [S][NQ][Hq][D] and lse [S][NQ][Hq] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    n_slots, n_q, n_q_heads, head_dim = q.shape
    group = n_q_heads // n_kv_heads
    qp = np.asarray(q_pos, dtype=np.int64).reshape(n_slots, n_q)
    out = np.zeros((n_slots, n_q, n_q_heads, head_dim))
    lse = np.full((n_slots, n_q, n_q_heads), -math.inf)
    for s in range(n_slots):
        for t in range(n_q):
            for g in range(n_kv_heads):
                ks, vs = [], []
                for k_cache, v_cache, cells in regions:
                    live = [int(c) for c in cells[s] if int(c) != -1]
                    pos = live if cell_pos is None else [int(cell_pos[c]) for c in live]
                    seen = [c for c, p in zip(live, pos) if p <= qp[s, t]]
                    ks.append(_rows(k_cache, seen, g))
                    vs.append(_rows(v_cache, seen, g))
                k_all = np.concatenate(ks, axis=0)
                v_all = np.concatenate(vs, axis=0)
                for h in range(g * group, (g + 1) * group):
                    out[s, t, h], lse[s, t, h] = attend_row(q[s, t, h], k_all, v_all, scale)
    return out, lse


def compact_plan(raw_cells_per_slot, capacity):
    """Compact indirect read plan, built per slot from a raw cell list.

    Steps, in the order of "KVARN KV Performance optimizations", items 3-4:
      1. drop -1 entries (holes); reject any other negative entry or any entry
         >= capacity (ValueError);
      2. remove duplicates, keeping the first occurrence;
      3. group the kept cells by physical record r = c // 128 and take the
         records in ascending order;
      4. emit one 128-entry segment per record: entry k is r*128 + k when that
         cell was kept, else -1.

    Returns (entries int32 [total], offsets int64 [S + 1]); slot s owns
    entries[offsets[s]:offsets[s+1]].
    """
    entries = []
    offsets = [0]
    for raw in raw_cells_per_slot:
        seen = set()
        kept = []
        for c in raw:
            c = int(c)
            if c == -1:
                continue
            if c < -1 or c >= capacity:
                raise ValueError(f"cell {c} outside [0, {capacity})")
            if c in seen:
                continue
            seen.add(c)
            kept.append(c)
        records = sorted({c // RECORD_CELLS for c in kept})
        for r in records:
            for k in range(RECORD_CELLS):
                cell = r * RECORD_CELLS + k
                entries.append(cell if cell in seen else -1)
        offsets.append(len(entries))
    return np.asarray(entries, dtype=np.int32), np.asarray(offsets, dtype=np.int64)

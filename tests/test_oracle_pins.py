"""Pins for the float64 oracle: every check here compares the oracle with
something other than itself (the IEEE binary16 formula, values worked by hand,
closed forms, a 50-digit brute force, torch's float64 attention, and the
invariants the log-sum-exp merge must satisfy).  CPU only."""

import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle as O
from long_context_decode_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- f16 decoding

def _half_formula(bits):
    """binary16 value from sign, exponent and fraction fields (IEEE 754)."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0:
        return sign * math.ldexp(f, -24)
    if e == 31:
        return sign * math.inf if f == 0 else math.nan
    return sign * math.ldexp(1024 + f, e - 25)


def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.f16_bits_to_f64(bits)
    want = np.array([_half_formula(int(b)) for b in range(65536)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ---------------------------------------------------------------- dequantisation

def _scale_bits(value):
    return np.array([value], dtype=np.float16).view(np.uint16)[0]


def test_q8_table():
    # d = 0.5: codes -127, -1, 0, 1, 127 -> -63.5, -0.5, 0, 0.5, 63.5
    codes = np.zeros(32, dtype=np.int8)
    codes[:5] = [-127, -1, 0, 1, 127]
    scales = np.array([_scale_bits(0.5)], dtype=np.uint16)
    x = O.dequantize(O.Q8_B32, codes, scales)
    assert list(x[:5]) == [-63.5, -0.5, 0.0, 0.5, 63.5]
    assert np.all(x[5:] == 0)
    # every int8 code is defined, -128 included
    codes = np.arange(-128, 128, dtype=np.int64).astype(np.int8).reshape(8, 32)
    scales = np.full((8, 1), _scale_bits(0.25), dtype=np.uint16)
    x = O.dequantize(O.Q8_B32, codes, scales).ravel()
    assert np.array_equal(x, np.arange(-128, 128) * 0.25)


def test_q4_table():
    # byte 0x1F: low nibble 0xF -> element 0 = (15 - 8) d, high nibble 0x1 ->
    # element 1 = (1 - 8) d
    d = 0.5
    codes = np.full(16, 0x88, dtype=np.uint8)  # u = 8 -> 0
    codes[0] = 0x1F
    scales = np.array([_scale_bits(d)], dtype=np.uint16)
    x = O.dequantize(O.Q4_B32, codes, scales)
    assert x[0] == 7 * d and x[1] == -7 * d
    assert np.all(x[2:] == 0)
    # all 16 nibble values in both positions
    u = np.arange(16, dtype=np.uint8)
    codes = (u | (u[::-1] << 4)).astype(np.uint8)  # 16 bytes = 32 elements
    x = O.dequantize(O.Q4_B32, codes, np.array([_scale_bits(1.0)], dtype=np.uint16))
    assert np.array_equal(x[0::2], np.arange(16) - 8.0)
    assert np.array_equal(x[1::2], np.arange(15, -1, -1) - 8.0)


def test_block_scale_positions():
    # a 96-element row has three blocks; each element must use its own block's scale
    for kind in (O.Q8_B32, O.Q4_B32):
        n = 96 if kind == O.Q8_B32 else 48
        codes = np.full(n, 1 if kind == O.Q8_B32 else 0x99, dtype=np.int8 if kind == O.Q8_B32 else np.uint8)
        scales = np.array([_scale_bits(v) for v in (1.0, 2.0, 4.0)], dtype=np.uint16)
        x = O.dequantize(kind, codes, scales)
        assert np.array_equal(x, np.repeat([1.0, 2.0, 4.0], 32))


def test_encoder_roundtrip_bound():
    # the harness encoder and the oracle's reader agree to half a quantum
    r = synth.rng(7)
    x = r.standard_normal((4, 3, 64), dtype=np.float32)
    for kind, qmax in ((O.Q8_B32, 127.0), (O.Q4_B32, 7.0)):
        codes, scales = synth.encode_blocks(kind, x)
        y = O.dequantize(kind, codes, scales)
        d = np.repeat(O.f16_bits_to_f64(scales), 32, axis=-1)
        amax = np.repeat(np.abs(x.reshape(4, 3, 2, 32)).max(-1), 32, axis=-1)
        # d = f16(amax / qmax) may round down, so the top code can clip by < 1 quantum
        assert np.all(np.abs(y - x) <= 0.5 * d + np.maximum(0, amax - qmax * d) + 1e-7)


# ---------------------------------------------------------------- closed forms

def _cache(rows):
    """f16 cache [n][1][D] holding the given rows (already f16-exact)."""
    bits = np.asarray(rows, dtype=np.float16).view(np.uint16)
    return (O.F16, bits[:, None, :], None)


def test_one_cell_returns_its_v_row():
    r = synth.rng(1)
    k = r.standard_normal((1, 8)).astype(np.float16)
    v = r.standard_normal((1, 8)).astype(np.float16)
    q = r.standard_normal((1, 1, 8))
    out, lse = O.decode_attention(q, [(_cache(k), _cache(v), [[0]])], 1, 0.3)
    assert np.array_equal(out[0, 0], v[0].astype(np.float64))
    s = 0.3 * float(np.dot(k[0].astype(np.float64), q[0, 0]))
    assert lse[0, 0] == pytest.approx(s, abs=1e-15)


def test_two_cells_sigmoid():
    r = synth.rng(2)
    k = r.standard_normal((2, 16)).astype(np.float16)
    v = r.standard_normal((2, 16)).astype(np.float16)
    q = r.standard_normal((1, 1, 16))
    out, lse = O.decode_attention(q, [(_cache(k), _cache(v), [[0, 1]])], 1, 0.25)
    kd, vd = k.astype(np.float64), v.astype(np.float64)
    s1, s2 = 0.25 * kd[0] @ q[0, 0], 0.25 * kd[1] @ q[0, 0]
    sig = 1.0 / (1.0 + math.exp(-(s2 - s1)))
    assert np.allclose(out[0, 0], vd[0] + sig * (vd[1] - vd[0]), atol=1e-14, rtol=0)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(s1) + math.exp(s2)), abs=1e-14)


def test_constant_scores_give_mean():
    r = synth.rng(3)
    n, d = 37, 32
    k = r.standard_normal((n, d)).astype(np.float16)
    v = r.standard_normal((n, d)).astype(np.float16)
    cells = [[i for i in range(n)] + [4, 4, 9]]  # multiplicity counts
    vd = v.astype(np.float64)
    want = (vd.sum(0) + 2 * vd[4] + vd[9]) / (n + 3)
    for q, scale in ((np.zeros((1, 1, d)), 1.0), (r.standard_normal((1, 1, d)), 0.0)):
        out, lse = O.decode_attention(q, [(_cache(k), _cache(v), cells)], 1, scale)
        assert np.allclose(out[0, 0], want, atol=1e-14, rtol=0)
        assert lse[0, 0] == pytest.approx(math.log(n + 3), abs=1e-13)
    # all K rows equal -> mean as well
    kk = np.repeat(k[:1], n, axis=0)
    out, _ = O.decode_attention(r.standard_normal((1, 1, d)), [(_cache(kk), _cache(v), [list(range(n))])], 1, 0.7)
    assert np.allclose(out[0, 0], vd.mean(0), atol=1e-14, rtol=0)


def test_hardmax_limit():
    r = synth.rng(4)
    n, d = 50, 16
    k = r.standard_normal((n, d)).astype(np.float16)
    v = r.standard_normal((n, d)).astype(np.float16)
    q = r.standard_normal((1, 1, d))
    s = k.astype(np.float64) @ q[0, 0]
    top = int(np.argmax(s))
    gap = np.sort(s)[-1] - np.sort(s)[-2]
    scale = 800.0 / gap  # second-best weight <= n * e^-800 -> 0
    out, _ = O.decode_attention(q, [(_cache(k), _cache(v), [list(range(n))])], 1, scale)
    assert np.array_equal(out[0, 0], v[top].astype(np.float64))


def test_empty_set():
    q = np.ones((1, 2, 8))
    cache = _cache(np.ones((4, 8)))
    out, lse = O.decode_attention(q, [(cache, cache, [[-1, -1]])], 1, 1.0)
    assert np.all(out == 0) and np.all(lse == -math.inf)
    m, l, o = O.partial_row(q[0, 0], np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert m == -math.inf and l == 0.0 and np.all(o == 0)


# ---------------------------------------------------------------- brute force

mpmath.mp.dps = 50


def _mp_half(bits):
    b = int(bits)
    sign = -1 if b >> 15 else 1
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    if e == 0:
        return sign * mpmath.mpf(f) * mpmath.mpf(2) ** -24
    return sign * mpmath.mpf(1024 + f) * mpmath.mpf(2) ** (e - 25)


def _mp_row(kind, codes, scales, head_dim):
    vals = []
    for i in range(head_dim):
        if kind == O.F16:
            vals.append(_mp_half(codes[i]))
            continue
        d = _mp_half(scales[i // 32])
        if kind == O.Q8_B32:
            c = int(codes[i])
            c = c - 256 if c > 127 else c
            vals.append(d * c)
        else:
            byte = int(codes[i // 2])
            u = (byte & 15) if i % 2 == 0 else (byte >> 4)
            vals.append(d * (u - 8))
    return vals


def _mp_attention(q, k_cache, v_cache, cells, n_kv_heads, scale):
    """Attention written out term by term with 50-digit arithmetic."""
    n_slots, n_q_heads, head_dim = q.shape
    group = n_q_heads // n_kv_heads
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for s in range(n_slots):
        for h in range(n_q_heads):
            g = h // group
            live = [c for c in cells[s] if c != -1]
            scores = []
            for c in live:
                krow = _mp_row(k_cache[0], k_cache[1][c, g], None if k_cache[2] is None else k_cache[2][c, g], head_dim)
                dot = mpmath.fsum(mpmath.mpf(float(q[s, h, i])) * krow[i] for i in range(head_dim))
                scores.append(mpmath.mpf(scale) * dot)
            if not live:
                lse[s, h] = -math.inf
                continue
            m = max(scores)
            w = [mpmath.exp(x - m) for x in scores]
            l = mpmath.fsum(w)
            for i in range(head_dim):
                acc = mpmath.fsum(
                    w[j] * _mp_row(v_cache[0], v_cache[1][c, g], None if v_cache[2] is None else v_cache[2][c, g], head_dim)[i]
                    for j, c in enumerate(live)
                )
                out[s, h, i] = float(acc / l)
            lse[s, h] = float(m + mpmath.log(l))
    return out, lse


@pytest.mark.parametrize("kind", [O.F16, O.Q8_B32, O.Q4_B32])
def test_brute_force_mpmath(kind):
    r = synth.rng(10 + kind)
    n_slots, hq, hkv, d, n_cells = 2, 4, 2, 32, 7
    q = synth.gen_q(r, n_slots, hq, d).astype(np.float64)
    kc, ks = synth.gen_cache(r, kind, n_cells, hkv, d)
    vc, vs = synth.gen_cache(r, kind, n_cells, hkv, d)
    cells = [[0, 3, 5, -1, 6], [1, 2, 2, 4]]
    scale = 1 / math.sqrt(d)
    got, glse = O.decode_attention(q, [((kind, kc, ks), (kind, vc, vs), cells)], hkv, scale)
    want, wlse = _mp_attention(q, (kind, kc, ks), (kind, vc, vs), cells, hkv, scale)
    assert np.allclose(got, want, atol=1e-13, rtol=1e-13)
    assert np.allclose(glse, wlse, atol=1e-13, rtol=1e-13)


# ---------------------------------------------------------------- library routine

def test_matches_torch_sdpa_float64():
    r = synth.rng(20)
    n_slots, hq, hkv, d, n = 2, 12, 2, 64, 300
    q = synth.gen_q(r, n_slots, hq, d).astype(np.float64)
    kc = synth.gen_f16_cache(r, n, hkv, d)
    vc = synth.gen_f16_cache(r, n, hkv, d)
    cells = [list(range(0, 300, 2)), list(range(7, 211))]
    scale = 0.11
    got, lse = O.decode_attention(q, [((O.F16, kc, None), (O.F16, vc, None), cells)], hkv, scale)
    kd = kc.view(np.float16).astype(np.float64)
    vd = vc.view(np.float16).astype(np.float64)
    for s in range(n_slots):
        idx = np.array(cells[s])
        K = torch.from_numpy(kd[idx]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)  # [Hq, n, D]
        V = torch.from_numpy(vd[idx]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        Q = torch.from_numpy(q[s])[:, None, :]  # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0, :].numpy()
        assert np.allclose(got[s], ref, atol=1e-13, rtol=0)
        sc = (torch.from_numpy(kd[idx]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0) @ Q.transpose(1, 2))[..., 0] * scale
        assert np.allclose(lse[s], torch.logsumexp(sc, dim=-1).numpy(), atol=1e-13, rtol=0)


# ---------------------------------------------------------------- invariants

def _random_problem(seed, n=200, d=32, hq=4, hkv=2):
    r = synth.rng(seed)
    q = synth.gen_q(r, 1, hq, d).astype(np.float64)
    kc = synth.gen_f16_cache(r, n, hkv, d)
    vc = synth.gen_f16_cache(r, n, hkv, d)
    return r, q, (O.F16, kc, None), (O.F16, vc, None)


def test_merge_of_partition_equals_unsplit():
    r, q, kcache, vcache = _random_problem(30)
    cells = list(range(200))
    want, wlse = O.decode_attention(q, [(kcache, vcache, [cells])], 2, 0.2)
    for trial in range(5):
        perm = r.permutation(200)
        cuts = np.sort(r.integers(0, 201, 4))
        pieces = np.split(perm, cuts)  # some pieces may be empty
        k_hat = O.dequantize(O.F16, kcache[1][:, 0])
        v_hat = O.dequantize(O.F16, vcache[1][:, 0])
        for h in (0, 1):
            parts = [O.partial_row(q[0, h], k_hat[p], v_hat[p], 0.2) for p in pieces]
            out, lse, _ = O.merge_partials(parts)
            assert np.allclose(out, want[0, h], atol=1e-12, rtol=0)
            assert lse == pytest.approx(wlse[0, h], abs=1e-12)


def test_merge_associative_commutative_identity():
    r, q, kcache, _ = _random_problem(31)
    k_hat = O.dequantize(O.F16, kcache[1][:, 1])
    a = O.partial_row(q[0, 2], k_hat[:50], k_hat[:50], 0.3)
    b = O.partial_row(q[0, 2], k_hat[50:120], k_hat[50:120], 0.3)
    c = O.partial_row(q[0, 2], k_hat[120:], k_hat[120:], 0.3)
    empty = (-math.inf, 0.0, np.zeros(32))
    ab = O.merge_partials([a, b])[2]
    bc = O.merge_partials([b, c])[2]
    left = O.merge_partials([ab, c])
    right = O.merge_partials([a, bc])
    flat = O.merge_partials([c, a, b])
    assert np.allclose(left[0], right[0], atol=1e-13) and np.allclose(left[0], flat[0], atol=1e-13)
    assert left[1] == pytest.approx(right[1], abs=1e-13)
    with_empty = O.merge_partials([empty, a, empty])
    alone = O.merge_partials([a])
    assert np.array_equal(with_empty[0], alone[0]) and with_empty[1] == alone[1]
    assert O.merge_partials([empty, empty])[1] == -math.inf


def test_permutation_holes_duplicates():
    r, q, kcache, vcache = _random_problem(32)
    cells = list(range(0, 200, 3))
    base, blse = O.decode_attention(q, [(kcache, vcache, [cells])], 2, 0.2)
    perm = list(np.asarray(cells)[r.permutation(len(cells))])
    out, lse = O.decode_attention(q, [(kcache, vcache, [perm])], 2, 0.2)
    assert np.allclose(out, base, atol=1e-13) and np.allclose(lse, blse, atol=1e-13)
    holed = []
    for c in cells:
        holed += [c, -1] if c % 2 else [-1, c]
    out, lse = O.decode_attention(q, [(kcache, vcache, [holed])], 2, 0.2)
    assert np.allclose(out, base, atol=1e-13) and np.allclose(lse, blse, atol=1e-13)
    # one repeated cell = that cell's weight doubled, written out by hand
    dup = cells + [cells[5]]
    out, _ = O.decode_attention(q, [(kcache, vcache, [dup])], 2, 0.2)
    k_hat = O.dequantize(O.F16, kcache[1][cells, 0])
    v_hat = O.dequantize(O.F16, vcache[1][cells, 0])
    s = 0.2 * k_hat @ q[0, 0]
    w = np.exp(s - s.max())
    w[5] *= 2
    assert np.allclose(out[0, 0], (w @ v_hat) / w.sum(), atol=1e-13)


def test_gqa_equals_mha_with_repeated_heads():
    r, q, kcache, vcache = _random_problem(33)
    cells = [list(range(13, 170))]
    gqa, glse = O.decode_attention(q, [(kcache, vcache, cells)], 2, 0.2)
    rep = lambda c: (c[0], np.repeat(c[1], 2, axis=1), None)  # KV head g -> query heads 2g, 2g+1
    mha, mlse = O.decode_attention(q, [(rep(kcache), rep(vcache), cells)], 4, 0.2)
    assert np.array_equal(gqa, mha) and np.array_equal(glse, mlse)


def test_window_plus_tail_equals_resident():
    r, q, kcache, vcache = _random_problem(34, n=300)
    resident, rlse = O.decode_attention(q, [(kcache, vcache, [list(range(300))])], 2, 0.2)
    # tail = cells 0..109 held in a separate host cache, window = 110..299
    tail_k = (O.F16, kcache[1][:110], None)
    tail_v = (O.F16, vcache[1][:110], None)
    out, lse, parts = O.decode_attention(
        q, [(kcache, vcache, [list(range(110, 300))]), (tail_k, tail_v, [list(range(110))])], 2, 0.2,
        return_partials=True)
    assert np.allclose(out, resident, atol=1e-13) and np.allclose(lse, rlse, atol=1e-13)
    for h in range(4):
        merged = O.merge_partials([(parts[i][0][0, h], parts[i][1][0, h], parts[i][2][0, h]) for i in range(2)])
        assert np.allclose(merged[0], resident[0, h], atol=1e-13)


# ---------------------------------------------------------------- compact plan

def _read_plan_examples():
    path = os.path.join(GOLDEN, "compact_plan_examples.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, _, rest = line.partition(":")
        vals = [int(x) for x in rest.split()]
        if key == "capacity":
            cur = {"capacity": vals[0], "slots": [], "expect": []}
            cases.append(cur)
        elif key == "slot":
            cur["slots"].append(vals)
            cur["expect"].append([])
        elif key == "record":
            cur["expect"][-1].append((vals[0], vals[1:]))
        elif key == "error":
            cur["error"] = True
    return cases


def test_compact_plan_hand_examples():
    cases = _read_plan_examples()
    assert len(cases) >= 4
    for case in cases:
        if case.get("error"):
            with pytest.raises(ValueError):
                O.compact_plan(case["slots"], case["capacity"])
            continue
        entries, offsets = O.compact_plan(case["slots"], case["capacity"])
        for s, expect in enumerate(case["expect"]):
            seg = entries[offsets[s]:offsets[s + 1]]
            assert len(seg) == 128 * len(expect)
            for i, (rec, kept_positions) in enumerate(expect):
                block = seg[128 * i:128 * (i + 1)]
                live = [k for k in range(128) if block[k] != -1]
                assert live == kept_positions
                assert all(block[k] == rec * 128 + k for k in live)


def test_compact_plan_invariants():
    r = synth.rng(40)
    lists, cap = synth.interleaved_record_lists([3000, 777, 128, 0, 1], r, shuffle=True, duplicates=50)
    entries, offsets = O.compact_plan(lists, cap)
    for s, raw in enumerate(lists):
        seg = entries[offsets[s]:offsets[s + 1]]
        assert len(seg) % 128 == 0
        live = seg[seg >= 0]
        assert sorted(live.tolist()) == sorted(set(int(c) for c in raw if c >= 0))
        assert np.all(np.diff(live) > 0)  # records ascending, monotonic inside
        for i in range(0, len(seg), 128):
            block = seg[i:i + 128]
            rec = block[block >= 0][0] // 128
            ks = np.nonzero(block >= 0)[0]
            assert np.array_equal(block[ks], rec * 128 + ks)
    # 215 holes for the four-slot GQA-6 workload (96 + 119)
    lists, cap = synth.interleaved_record_lists([131072, 65536, 20000, 777])
    entries, offsets = O.compact_plan(lists, cap)
    assert cap == 1700 * 128 and len(entries) == cap and int((entries == -1).sum()) == 215


# ---------------------------------------------------------------- multi-query (positional mask)

def _multi_problem(seed, kind=O.F16, n_slots=2, n_q=3, hq=4, hkv=2, d=32, n=60):
    r = synth.rng(seed)
    q = synth.gen_q(r, n_slots * n_q, hq, d).astype(np.float64).reshape(n_slots, n_q, hq, d)
    kc, ks = synth.gen_cache(r, kind, n, hkv, d)
    vc, vs = synth.gen_cache(r, kind, n, hkv, d)
    return r, q, (kind, kc, ks), (kind, vc, vs)


def test_multi_query_all_visible_equals_single_query():
    """Every cell visible: each query row is the single-query result of that row."""
    r, q, kcache, vcache = _multi_problem(40)
    cells = [list(range(0, 60, 3)) + [-1, 5, 5], list(range(10, 50))]
    got, glse = O.decode_attention_multi(q, [(kcache, vcache, cells)], 2, 0.17, q_pos=np.full((2, 3), 10 ** 6))
    for t in range(3):
        want, wlse = O.decode_attention(q[:, t], [(kcache, vcache, cells)], 2, 0.17)
        assert np.array_equal(got[:, t], want) and np.array_equal(glse[:, t], wlse)


def test_multi_query_matches_torch_sdpa_with_boolean_mask():
    """torch's float64 scaled_dot_product_attention with an explicit mask built
    from the cell positions (a random permutation as cell_pos)."""
    r, q, kcache, vcache = _multi_problem(41, n_q=4, hq=6, hkv=2, d=64, n=90)
    cell_pos = r.permutation(90) + 1000
    cells = [list(range(90)), list(range(20, 77))]
    q_pos = np.array([[1010, 1040, 1041, 1089], [1000, 1030, 1060, 1200]])
    got, glse = O.decode_attention_multi(q, [(kcache, vcache, cells)], 2, 0.125, q_pos=q_pos, cell_pos=cell_pos)
    kd = kcache[1].view(np.float16).astype(np.float64)
    vd = vcache[1].view(np.float16).astype(np.float64)
    for s in range(2):
        idx = np.array(cells[s])
        K = torch.from_numpy(kd[idx]).permute(1, 0, 2).repeat_interleave(3, dim=0)   # [Hq, n, D]
        V = torch.from_numpy(vd[idx]).permute(1, 0, 2).repeat_interleave(3, dim=0)
        Q = torch.from_numpy(q[s]).permute(1, 0, 2)                                  # [Hq, NQ, D]
        mask = torch.from_numpy(cell_pos[idx][None, :] <= q_pos[s][:, None])         # [NQ, n]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=0.125)
        assert np.allclose(got[s], ref.permute(1, 0, 2).numpy(), atol=1e-13, rtol=0)
        sc = (K @ Q.transpose(1, 2)).transpose(1, 2) * 0.125                         # [Hq, NQ, n]
        sc = sc.masked_fill(~mask[None], -math.inf)
        assert np.allclose(glse[s], torch.logsumexp(sc, dim=-1).T.numpy(), atol=1e-13, rtol=0)


@pytest.mark.parametrize("kind", [O.F16, O.Q4_B32])
def test_multi_query_brute_force_mpmath(kind):
    """Masked softmax written out term by term in 50-digit arithmetic: row t
    attends exactly to the cells whose index is at most q_pos[t]."""
    r, q, kcache, vcache = _multi_problem(42 + kind, n_slots=1, n_q=3, hq=2, hkv=1, d=32, n=7)
    cells = [[0, 3, 5, -1, 6, 2]]
    q_pos = np.array([[2, 5, 6]])
    got, glse = O.decode_attention_multi(q, [(kcache, vcache, cells)], 1, 0.25, q_pos=q_pos)
    visible = {2: [0, 2], 5: [0, 3, 5, 2], 6: [0, 3, 5, 6, 2]}  # by hand
    for t in range(3):
        want, wlse = _mp_attention(q[:, t], kcache, vcache, [visible[int(q_pos[0, t])]], 1, 0.25)
        assert np.allclose(got[:, t], want, atol=1e-13, rtol=1e-13)
        assert np.allclose(glse[:, t], wlse, atol=1e-13, rtol=1e-13)


def test_multi_query_causality_and_empty_rows():
    """Changing cells past a row's position leaves the row unchanged; changing
    a visible cell does not; a row before every cell sees nothing."""
    r, q, kcache, vcache = _multi_problem(43, n_slots=1, n_q=3, n=40)
    cells = [list(range(40))]
    q_pos = np.array([[-1, 20, 39]])
    base, blse = O.decode_attention_multi(q, [(kcache, vcache, cells)], 2, 0.2, q_pos=q_pos)
    assert np.all(base[0, 0] == 0) and np.all(blse[0, 0] == -math.inf)
    k2, v2 = kcache[1].copy(), vcache[1].copy()
    k2[21:] ^= 0x0155
    v2[21:] ^= 0x0155
    got, glse = O.decode_attention_multi(q, [((O.F16, k2, None), (O.F16, v2, None), cells)], 2, 0.2, q_pos=q_pos)
    assert np.array_equal(got[0, 1], base[0, 1]) and np.array_equal(glse[0, 1], blse[0, 1])
    assert not np.allclose(got[0, 2], base[0, 2])

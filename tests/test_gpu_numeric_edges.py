"""Numeric worst cases of the f16 arithmetic against the float64 oracle, on
every kernel, with block-scaled V whose (d, code) pairs are chosen so that
d * code lies as far as the data allows from the nearest f16 value -- half
an f16 ulp, which is what the matrix-core kernel's staged V^ can be off by:

* one-cell slots with |d * code| in [4, 8) (up to 2^-9 off): the output is
  the V row itself;
* two-cell slots with |d * code| in [4, 8) whose K rows are equal: the two
  scores are exactly equal, the softmax weights exactly 1/2 each;
* two-cell slots whose K rows differ in one code step (near-equal scores),
  V in the value range of N(0, 1) blocks (|d * code| in [2, 4)): the f16
  weights and the f16 staging of K^ move the two weights against each
  other, and that moves the output by up to that shift times |v1 - v2|;
* the same near ties on f16 K and V, with score gaps spread over many
  sizes and |V| in [2, 4).

The bound is the one of every parity case (2e-3 on out and lse)."""

import numpy as np
import pytest

import oracle as O
from gpu_cases import check, dev
from long_context_decode_kv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available()
    from long_context_decode_kv_amd import kvdec
    return kvdec


def f16_error(x):
    """|f16(x) - x| for float64 x (numpy rounds to nearest even)."""
    return np.abs(x.astype(np.float16).astype(np.float64) - x)


def adversarial_rows(kind, r, shape, vmin=4.0):
    """Block-scaled rows [..., D] with |d * code| in [vmin, 2 vmin) everywhere
    (vmin a power of two) and the code of every element picked among the
    valid ones for the largest f16 rounding error of d * code (random
    signs).  Returns (codes, scale_bits) in the stored layout."""
    *lead, D = shape
    nb = D // 32
    n = int(np.prod(lead)) * nb
    # scale ranges for which some magnitudes in `mags` keep d * code in range
    if kind == O.Q8_B32:
        lo, hi, mags = vmin / 64, vmin / 32, np.arange(1, 128)
    else:
        lo, hi, mags = vmin / 4, vmin * 2 / 7, np.arange(1, 8)
    d16 = r.uniform(lo, hi, size=(n, 16)).astype(np.float16)  # 16 candidate scales per block
    codes = np.zeros((n, 32), np.int64)
    scales = np.zeros(n, np.float16)
    for b in range(n):
        best = None
        for d in d16[b]:
            x = float(d) * mags
            ok = (x >= vmin) & (x < 2 * vmin)
            if not ok.any():
                continue
            m, e = mags[ok], f16_error(x[ok])
            top = np.argsort(-e)[:4]  # the four worst magnitudes of this scale
            score = e[top].mean()
            if best is None or score > best[0]:
                best = (score, d, m[top])
        _, d, m = best
        scales[b] = d
        codes[b] = m[r.integers(0, len(m), size=32)] * np.where(r.random(32) < 0.5, -1, 1)
    codes = codes.reshape(*lead, D)
    sb = scales.reshape(*lead, nb).view(np.uint16)
    if kind == O.Q8_B32:
        return codes.astype(np.int8), sb
    u = (codes + 8).astype(np.uint8).reshape(*lead, D // 2, 2)
    return (u[..., 0] | (u[..., 1] << 4)).astype(np.uint8), sb


def run(K, hq, hkv, d, kind, v_kind, q, kc, ks, vc, vs, n_slots, cells_per_slot):
    import torch
    cap = n_slots * cells_per_slot
    p = K.plan(hq, hkv, d, n_slots, cap, k_type=kind, v_type=v_kind, n_occupied=[cells_per_slot] * n_slots,
               cell_begin=[s * cells_per_slot for s in range(n_slots)])
    out = torch.full((n_slots, hq, d), float("nan"), device="cuda")
    lse = torch.full((n_slots, hq), float("nan"), device="cuda")
    K.attend(p, dev(q), dev(kc), dev(vc), K.workspace(p), out=out, lse=lse, k_scales=dev(ks), v_scales=dev(vs))
    torch.cuda.synchronize()
    want = O.decode_attention(q, [((kind, kc, ks), (v_kind, vc, vs),
                                   [np.arange(s * cells_per_slot, (s + 1) * cells_per_slot) for s in range(n_slots)])],
                              hkv, 1 / np.sqrt(d))
    return p.info(), out.cpu().numpy(), lse.cpu().numpy(), want


SHAPES = [  # (q heads, KV heads, head_dim, K kind, V kind): matrix-core kernel first
    (24, 4, 256, O.Q8_B32, O.Q8_B32),
    (24, 4, 256, O.Q4_B32, O.Q4_B32),
    (24, 4, 256, O.Q8_B32, O.Q4_B32),
    (32, 8, 128, O.Q8_B32, O.Q8_B32),
    (32, 8, 128, O.Q4_B32, O.Q4_B32),
]


def _ids(s):
    return f"hq{s[0]}-hkv{s[1]}-d{s[2]}-k{s[3]}-v{s[4]}"


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_one_cell_slots_v_in_4_8(K, shape):
    hq, hkv, d, kind, v_kind = shape
    r = synth.rng(7100 + hq + 3 * kind + v_kind)
    S = 64
    q = synth.gen_q(r, S, hq, d)
    kc, ks = synth.gen_quant_cache(r, kind, S, hkv, d)
    vc, vs = adversarial_rows(v_kind, r, (S, hkv, d))
    v_hat = O.dequantize(v_kind, vc, vs)
    assert np.all(np.abs(v_hat) >= 4) and np.all(np.abs(v_hat) < 8)
    assert f16_error(v_hat).max() > 0.9 * 2.0 ** -9  # the data reaches the worst rounding
    info, go, gl, (wo, wl) = run(K, hq, hkv, d, kind, v_kind, q, kc, ks, vc, vs, S, 1)
    assert info["matrix_cores"] == (1 if hq // hkv == 6 else 0)
    check(go, gl, wo, wl)
    assert np.abs(go - wo).max() <= 2.0 ** -9 + 1e-6  # at most the f16 rounding of one V^ value


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("equal", [True, False], ids=["equal-scores", "one-step-apart"])
def test_two_cell_slots(K, shape, equal):
    hq, hkv, d, kind, v_kind = shape
    r = synth.rng(7200 + hq + 3 * kind + v_kind + (0 if equal else 50))
    S = 32
    q = synth.gen_q(r, S, hq, d)
    kc, ks = synth.gen_quant_cache(r, kind, 2 * S, hkv, d)
    kc[1::2], ks[1::2] = kc[0::2], ks[0::2]  # cell 2s+1 gets cell 2s's K row
    if not equal:
        # one code of each second row one step toward zero: scores differ
        # by d * |q| for one element
        if kind == O.Q8_B32:
            c = kc[1::2, :, 0].astype(np.int16)
            kc[1::2, :, 0] = (c - np.sign(c)).astype(np.int8)
        else:
            low = (kc[1::2, :, 0] & 0x0F).astype(np.int16) - 8
            low = low - np.sign(low)
            kc[1::2, :, 0] = (kc[1::2, :, 0] & 0xF0) | (low + 8).astype(np.uint8)
    vc, vs = adversarial_rows(v_kind, r, (2 * S, hkv, d), vmin=4.0 if equal else 2.0)
    info, go, gl, (wo, wl) = run(K, hq, hkv, d, kind, v_kind, q, kc, ks, vc, vs, S, 2)
    check(go, gl, wo, wl)
    if equal:
        # the two weights are exactly equal: only the staging of V^ rounds
        assert np.abs(go - wo).max() <= 2.0 ** -9 + 1e-6
    del info


F16_KERNELS = [  # (q heads, KV heads, head_dim, kernel): one-shot, streamed, matrix cores
    (32, 8, 128, "oneshot"),
    (32, 8, 128, "streamed"),
    (24, 4, 256, "mfma"),
]


@pytest.mark.parametrize("shape", F16_KERNELS, ids=lambda s: f"hq{s[0]}-hkv{s[1]}-d{s[2]}-{s[3]}")
def test_two_cell_slots_f16_near_ties(K, shape):
    """f16 K and V: two cells per slot whose K rows differ in one element by
    1 to 4000 f16 steps (score gaps of many sizes), V values of either sign
    with magnitude in [2, 4); V is exact in f16, so only the weights round
    (to nearest on the vector kernels, at most 2^-11 of the smaller weight
    -- the larger one, the stream's maximum, is exact: at most
    2^-13 |v1 - v2| < 2^-10 in the output)."""
    import torch
    hq, hkv, d, kern = shape
    r = synth.rng(7300 + d + len(kern))
    S = 32
    q = synth.gen_q(r, S, hq, d)
    kc = synth.gen_f16_cache(r, 2 * S, hkv, d)
    kc[1::2] = kc[0::2]
    # the first element moved by 1..4000 steps of its bit pattern toward
    # zero (only where its magnitude bits exceed the steps: same sign, finite)
    steps = r.integers(1, 4001, size=kc[1::2, :, 0].shape).astype(np.int64)
    first = kc[1::2, :, 0].astype(np.int64)
    kc[1::2, :, 0] = np.where((first & 0x7FFF) > steps, first - steps, first).astype(np.uint16)
    mag = r.uniform(2, 4, size=(2 * S, hkv, d))
    vc = synth.f16_bits(np.where(r.random((2 * S, hkv, d)) < 0.5, -mag, mag))
    cap = 2 * S
    kw = {"oneshot": dict(kernel=K.KERNEL_ONESHOT), "streamed": dict(kernel=K.KERNEL_STREAMED), "mfma": {}}[kern]
    p = K.plan(hq, hkv, d, S, cap, n_occupied=[2] * S, cell_begin=[2 * s for s in range(S)], **kw)
    info = p.info()
    assert info["matrix_cores"] == (1 if kern == "mfma" else 0)
    if kern != "mfma":
        assert info["kernel"] == (K.KERNEL_ONESHOT if kern == "oneshot" else K.KERNEL_STREAMED)
    out = torch.full((S, hq, d), float("nan"), device="cuda")
    lse = torch.full((S, hq), float("nan"), device="cuda")
    K.attend(p, dev(q), dev(kc), dev(vc), K.workspace(p), out=out, lse=lse)
    torch.cuda.synchronize()
    want = O.decode_attention(q, [((O.F16, kc, None), (O.F16, vc, None), [np.arange(2 * s, 2 * s + 2) for s in range(S)])],
                              hkv, 1 / np.sqrt(d))
    check(out.cpu().numpy(), lse.cpu().numpy(), *want)

"""Seeded synthetic inputs for the decode-attention library's tests and benchmarks.

Input generation only: random draws, f16 rounding of the draws, the block
encoder that turns a float draw into stored int8 / 4-bit codes plus one f16
scale per 32 elements, and indirect cell lists.  None of the attention
arithmetic and none of the rule that reads codes back as values lives here.

Host-side draws use numpy's PCG64; the multi-GiB caches of the long-context
workloads are drawn on the device with a seeded torch generator and copied to
the host where a check needs them.
"""

import numpy as np

F16, Q8_B32, Q4_B32 = 0, 1, 2
BLOCK = 32
RECORD_CELLS = 128


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def gen_q(r, n_slots, n_q_heads, head_dim):
    """q ~ N(0, 1), float32 [S][Hq][D]."""
    return r.standard_normal((n_slots, n_q_heads, head_dim), dtype=np.float32)


def f16_bits(x):
    """Round float values to binary16 (round-to-nearest-even) and return the bit
    patterns as uint16."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def gen_f16_cache(r, n_cells, n_kv_heads, head_dim):
    """K or V ~ N(0, 1) rounded to f16: uint16 bits [cells][Hkv][D]."""
    x = r.standard_normal((n_cells, n_kv_heads, head_dim), dtype=np.float32)
    return f16_bits(x)


def encode_blocks(kind, x):
    """Encode float32 rows [..., D] (D a multiple of 32) into stored codes and
    one f16 scale per 32 elements.

    int8:  d = f16(max|x| / 127), code = clamp(rint(x / d), -127, 127)
    4-bit: d = f16(max|x| / 7),   u = clamp(rint(x / d), -8, 7) + 8, two
           codes per byte, element 2i in the low nibble of byte i.
    An all-zero block gets d = 0 and zero codes (u = 8 for 4-bit).
    Returns (codes, scale_bits).
    """
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    d_model = shape[-1]
    xb = x.reshape(*shape[:-1], d_model // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=-1)
    qmax = 127.0 if kind == Q8_B32 else 7.0
    d16 = (amax / qmax).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, 1.0, d32)[..., None]
    t = np.rint(xb / safe)
    t = np.where(d32[..., None] == 0, 0.0, t)
    if kind == Q8_B32:
        codes = np.clip(t, -127, 127).astype(np.int8).reshape(shape)
    elif kind == Q4_B32:
        u = (np.clip(t, -8, 7) + 8).astype(np.uint8).reshape(*shape[:-1], d_model // 2, 2)
        codes = (u[..., 0] | (u[..., 1] << 4)).astype(np.uint8)
    else:
        raise ValueError(kind)
    return codes, d16.view(np.uint16)


def gen_quant_cache(r, kind, n_cells, n_kv_heads, head_dim):
    """x ~ N(0, 1) encoded per 32-element block: (codes, scale_bits)."""
    x = r.standard_normal((n_cells, n_kv_heads, head_dim), dtype=np.float32)
    return encode_blocks(kind, x)


def gen_cache(r, kind, n_cells, n_kv_heads, head_dim):
    """(codes, scales-or-None) for any kind."""
    if kind == F16:
        return gen_f16_cache(r, n_cells, n_kv_heads, head_dim), None
    return gen_quant_cache(r, kind, n_cells, n_kv_heads, head_dim)


def plant_needles(r, q, k_codes, cells_per_slot, n_kv_heads):
    """"Peaked" variant: per (slot, KV head) one seeded attended cell c* gets
    K[c*, g, :] = f16(q[s, g*G, :]), so that cell dominates the softmax of the
    group's first query head.  Modifies f16 ``k_codes`` in place and returns
    the chosen cells [S][Hkv]."""
    n_slots, n_q_heads, _ = q.shape
    group = n_q_heads // n_kv_heads
    chosen = np.full((n_slots, n_kv_heads), -1, dtype=np.int64)
    for s in range(n_slots):
        live = [int(c) for c in cells_per_slot[s] if int(c) >= 0]
        if not live:
            continue
        for g in range(n_kv_heads):
            c = live[int(r.integers(0, len(live)))]
            k_codes[c, g, :] = f16_bits(q[s, g * group, :])
            chosen[s, g] = c
    return chosen


def interleaved_record_lists(lengths, r=None, shuffle=False, duplicates=0):
    """Raw cell lists for slots whose cells sit in 128-cell physical records
    handed out round-robin across the slots (record 0 to slot 0, record 1 to
    slot 1, ... skipping slots that have all their records).

    Slot s with n_s cells owns ceil(n_s / 128) records and occupies the first
    n_s cells of them, so its last record ends in holes.  Returns
    (lists, capacity_cells).  With ``shuffle`` each list is permuted; with
    ``duplicates`` > 0 that many repeated entries and -1 holes are sprinkled
    into each non-empty list.
    """
    need = [-(-n // RECORD_CELLS) for n in lengths]
    owner = []
    left = list(need)
    while any(left):
        for s in range(len(lengths)):
            if left[s]:
                owner.append(s)
                left[s] -= 1
    lists = [[] for _ in lengths]
    filled = [0] * len(lengths)
    for rec, s in enumerate(owner):
        take = min(RECORD_CELLS, lengths[s] - filled[s])
        lists[s].extend(range(rec * RECORD_CELLS, rec * RECORD_CELLS + take))
        filled[s] += take
    out = []
    for lst in lists:
        a = np.asarray(lst, dtype=np.int32)
        if duplicates and len(a):
            extra = a[r.integers(0, len(a), duplicates)]
            holes = np.full(duplicates, -1, dtype=np.int32)
            a = np.concatenate([a, extra, holes])
        if shuffle and len(a):
            a = a[r.permutation(len(a))]
        out.append(a)
    return out, len(owner) * RECORD_CELLS


# --------------------------------------------------------------------------
# Device-side draws for the multi-GiB workloads (torch is plumbing only).
# --------------------------------------------------------------------------

def device_generator(seed, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def device_f16_cache(seed, n_cells, n_kv_heads, head_dim, device="cuda", out=None):
    """K or V ~ N(0, 1) rounded to f16 on the device: a float16 tensor
    [cells][Hkv][D], drawn in chunks to bound scratch memory."""
    import torch
    g = device_generator(seed, device)
    if out is None:
        out = torch.empty((n_cells, n_kv_heads, head_dim), dtype=torch.float16, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(torch.float16)
    return out


def device_q(seed, n_slots, n_q_heads, head_dim, device="cuda"):
    import torch
    g = device_generator(seed, device)
    return torch.randn((n_slots, n_q_heads, head_dim), generator=g, device=device, dtype=torch.float32)


def device_quant_cache(seed, kind, n_cells, n_kv_heads, head_dim, device="cuda"):
    """x ~ N(0, 1) drawn on the device and encoded per 32-element block with
    the same rule as ``encode_blocks``: returns (codes, scale bits as int16)."""
    import torch
    g = device_generator(seed, device)
    nb = head_dim // BLOCK
    row = head_dim if kind == Q8_B32 else head_dim // 2
    codes = torch.empty((n_cells, n_kv_heads, row), dtype=torch.int8 if kind == Q8_B32 else torch.uint8,
                        device=device)
    scales = torch.empty((n_cells, n_kv_heads, nb), dtype=torch.float16, device=device)
    step = max(1, (1 << 24) // (n_kv_heads * head_dim))
    qmax = 127.0 if kind == Q8_B32 else 7.0
    for c0 in range(0, n_cells, step):
        n = min(step, n_cells - c0)
        x = torch.randn((n, n_kv_heads, nb, BLOCK), generator=g, device=device, dtype=torch.float32)
        d16 = (x.abs().amax(dim=-1) / qmax).to(torch.float16)
        d32 = d16.to(torch.float32)
        safe = torch.where(d32 == 0, torch.ones_like(d32), d32)[..., None]
        t = torch.round(x / safe)
        t = torch.where(d32[..., None] == 0, torch.zeros_like(t), t)
        if kind == Q8_B32:
            codes[c0:c0 + n] = t.clamp(-127, 127).to(torch.int8).reshape(n, n_kv_heads, row)
        else:
            u = (t.clamp(-8, 7) + 8).to(torch.uint8).reshape(n, n_kv_heads, row, 2)
            codes[c0:c0 + n] = u[..., 0] | (u[..., 1] << 4)
        scales[c0:c0 + n] = d16
    return codes, scales

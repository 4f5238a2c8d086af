"""Shared helpers of the GPU parity tests: build a seeded case, run it through
the C ABI (via the ctypes binding), and evaluate the float64 oracle on the
same host arrays."""

import math
import os

import numpy as np

import oracle as O
from long_context_decode_kv_amd import synth

TOL = 2e-3  # max |err| of out and lse against the float64 oracle
# Two GPU results over different split partitions of the same cells: the f16
# softmax weights are rounded (to nearest) against each stream's own
# maximum, so the two are re-weighted differently by up to 2^-11 per weight;
# lse and out then differ by far less than this bound.  (Each result is also
# held to TOL against the oracle.)
TOL_SPLITS = 1e-3


def dev(a):
    """numpy -> cuda tensor holding the same bytes (uint16 travels as int16)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


class Case:
    """Seeded problem: q, K/V caches (codes, scales) and the cells of each slot."""

    def __init__(self, seed, n_q_heads, n_kv_heads, head_dim, kind=O.F16, occupied=None, begins=None,
                 indirect_lengths=None, shuffle=False, duplicates=0, peaked=False, capacity=None, scale=None,
                 v_kind=None):
        r = synth.rng(seed)
        self.hq, self.hkv, self.d, self.kind = n_q_heads, n_kv_heads, head_dim, kind
        self.vkind = kind if v_kind is None else v_kind  # V storage kind (K uses `kind`)
        self.scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
        if indirect_lengths is not None:
            self.raw, cap = synth.interleaved_record_lists(indirect_lengths, r, shuffle=shuffle, duplicates=duplicates)
            self.capacity = cap if capacity is None else capacity
            entries, off = O.compact_plan(self.raw, self.capacity)
            self.oracle_cells = [entries[off[s]:off[s + 1]] for s in range(len(indirect_lengths))]
            self.n_slots = len(indirect_lengths)
            self.occupied = None
            self.begins = None
        else:
            self.raw = None
            self.n_slots = len(occupied)
            self.begins = list(begins) if begins is not None else [0] * self.n_slots
            self.occupied = list(occupied)
            need = max([b + n for b, n in zip(self.begins, self.occupied)] + [1])
            self.capacity = need if capacity is None else capacity
            self.oracle_cells = [np.arange(b, b + n) for b, n in zip(self.begins, self.occupied)]
        self.q = synth.gen_q(r, self.n_slots, n_q_heads, head_dim)
        self.kc, self.ks = synth.gen_cache(r, kind, self.capacity, n_kv_heads, head_dim)
        self.vc, self.vs = synth.gen_cache(r, self.vkind, self.capacity, n_kv_heads, head_dim)
        if peaked:
            assert kind == O.F16
            synth.plant_needles(r, self.q, self.kc, self.oracle_cells, n_kv_heads)

    # -- oracle
    def oracle(self):
        return O.decode_attention(self.q, [((self.kind, self.kc, self.ks), (self.vkind, self.vc, self.vs),
                                            self.oracle_cells)], self.hkv, self.scale)

    # -- GPU
    def plan(self, K, **kw):
        if self.raw is not None:
            return K.plan(self.hq, self.hkv, self.d, self.n_slots, self.capacity, k_type=self.kind,
                          v_type=self.vkind, scale=self.scale, cells=self.raw, **kw)
        return K.plan(self.hq, self.hkv, self.d, self.n_slots, self.capacity, k_type=self.kind, v_type=self.vkind,
                      scale=self.scale, n_occupied=self.occupied, cell_begin=self.begins, **kw)

    def upload(self):
        self.q_d = dev(self.q)
        self.kc_d, self.vc_d = dev(self.kc), dev(self.vc)
        self.ks_d = None if self.ks is None else dev(self.ks)
        self.vs_d = None if self.vs is None else dev(self.vs)
        return self

    def run(self, K, plan=None, ws=None, part=False, **kw):
        import torch
        if not hasattr(self, "q_d"):
            self.upload()
        p = plan if plan is not None else self.plan(K, **kw)
        w = ws if ws is not None else K.workspace(p)
        out = torch.full((self.n_slots, self.hq, self.d), float("nan"), device="cuda")
        lse = torch.full((self.n_slots, self.hq), float("nan"), device="cuda")
        pc = None
        if self.raw is not None:
            pc = dev(p.cells()[0])
        parts = None
        if part:
            parts = (torch.empty(self.n_slots, self.hq, device="cuda"), torch.empty(self.n_slots, self.hq, device="cuda"),
                     torch.empty(self.n_slots, self.hq, self.d, device="cuda"))
        K.attend(p, self.q_d, self.kc_d, self.vc_d, w, out=out, lse=lse, part=parts, k_scales=self.ks_d,
                 v_scales=self.vs_d, plan_cells=pc)
        torch.cuda.synchronize()
        res = (out.cpu().numpy(), lse.cpu().numpy())
        if part:
            return res + (tuple(t.cpu().numpy() for t in parts),)
        return res


# (test, max |out err|, out RMSE, max |lse err|) of every comparison in this
# process; the session summary prints the worst of them.
REPORT = []


def check(got_out, got_lse, want_out, want_lse, tol=TOL):
    """Element-wise comparison; returns (max |err| of out, of lse)."""
    assert got_out.shape == want_out.shape
    assert np.all(np.isfinite(got_out)), "non-finite output"
    err = float(np.max(np.abs(got_out - want_out))) if got_out.size else 0.0
    rmse = float(np.sqrt(np.mean((got_out.astype(np.float64) - want_out) ** 2))) if got_out.size else 0.0
    REPORT.append([os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], err, rmse, None])
    assert err <= tol, f"max |out err| = {err:.3e}"
    empty = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), "lse -inf pattern differs"
    lerr = float(np.max(np.abs(got_lse[~empty] - want_lse[~empty]))) if (~empty).any() else 0.0
    REPORT[-1][3] = lerr
    assert lerr <= tol, f"max |lse err| = {lerr:.3e}"
    return err, lerr

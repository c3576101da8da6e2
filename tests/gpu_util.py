"""Helpers shared by the GPU parity tests: build slot pools from the seeded
generator, run layers through libmoe, and measure errors against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import expert_offload_amd as moe
from expert_offload_amd import layer
from gen import inputs as gi
import oracle

DEV = torch.device("cuda:0")


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def max_rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (tensor-level relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (denom if denom > 0 else 1.0))


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


class ResidentLayer:
    """All E experts of one layer resident in a slot pool under a seeded slot permutation."""

    def __init__(self, wl: gi.Workload, layer_idx: int = 0, experts=None, blocks=None):
        self.wl = wl
        self.layer = layer_idx
        self.perm = gi.slot_permutation(wl, layer_idx)
        self.pool = layer.SlotPool(wl.qtype, wl.H, wl.I, wl.E, device=DEV)
        self.blocks = {} if blocks is None else blocks
        experts = range(wl.E) if experts is None else experts

        def put(l, e, b):
            self.blocks[e] = b
            self.pool.put(int(self.perm[e]), layer.pack_expert(wl.qtype, wl.H, wl.I, *b))

        missing = [(layer_idx, e) for e in experts if e not in self.blocks]
        gi.generate_blocks_parallel(wl, missing, put)
        for e in experts:
            if (layer_idx, e) not in missing:
                put(layer_idx, e, self.blocks[e])
        self.slot_table = dev(self.perm)

    def get_blocks(self, e):
        if e not in self.blocks:
            self.blocks[e] = gi.expert_blocks(self.wl, self.layer, e)
        return self.blocks[e]


WEIGHT_TOL = 1e-5
NEAR_TIE = 1e-5  # oracle logit gap below which fp32 rounding may reorder experts


def check_routed_layer(ids, w, logits, y, out, ref, tol, T, reref=None) -> None:
    """Checks one layer's GPU results on every token.

    - The exact top-k contract: the oracle's selection and weights applied
      to the logits the GPU selected on equal the GPU's ids and weights.
    - End to end, the ids equal the oracle's own, except tokens whose k-th
      and (k+1)-th oracle logits are closer than NEAR_TIE (counted).
    - y and out within `tol` (max relative error), against the oracle run
      on the GPU's logits (`reref(logits)`) when a near tie changed a
      selection.
    """
    k = ids.shape[1]
    ids, w, lo = ids[:T], w[:T], logits[:T]
    np.testing.assert_array_equal(ids, oracle.topk_select(lo, k))
    own_w = oracle.renormalize(oracle.softmax(lo.astype(np.float64)), ids)
    assert np.abs(w - own_w).max() <= WEIGHT_TOL
    ok = ref["gap"] >= NEAR_TIE
    np.testing.assert_array_equal(ids[ok], ref["ids"][ok])
    assert (~ok).sum() <= max(1, T // 100)
    if not np.array_equal(ids, ref["ids"]):
        note(f"   {int((ids != ref['ids']).any(axis=1).sum())} near-tie tokens chose differently; "
             "comparing against the oracle on the GPU's logits")
        assert reref is not None, "a near tie changed a selection and no re-reference was given"
        ref = reref(lo)
        np.testing.assert_array_equal(ids, ref["ids"])
    H = out.shape[1]
    e_y = max_rel_err(y[:T * k].reshape(T, k, H), ref["y_pairs"].reshape(T, k, H))
    e_out = max_rel_err(out[:T], ref["out"])
    note(f"   y max rel err {e_y:.2e}, out max rel err {e_out:.2e}")
    assert np.isfinite(out[:T]).all()
    assert e_y <= tol and e_out <= tol

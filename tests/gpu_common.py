"""Shared pieces of the GPU tests: tolerances and a replay driver for the native path.

The native replay walks the same operation script as oracle/replay.py but
through the C ABI only (native allocator, pa_copy_blocks, pa_kv_write,
pa_decode_attention); it shares no code with the oracle.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from paged_kv_cache_320_amd import PagedKVCache

# Accumulation error allowed per output element (fp32 accumulation in every case).
ATOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
MANTISSA_BITS = {"f32": 23, "f16": 10, "bf16": 7}


def tolerance(dtype: str, ref: np.ndarray) -> np.ndarray:
    """Per-element bound: the accumulation gate plus half an ulp of the output format.

    The output is rounded to its storage format (round to nearest even), which
    alone moves it by up to half an ulp of |ref|: for bf16 that exceeds 2e-3 once
    |out| >= 0.5, so the rounding term is added to the gate rather than hidden in it.
    """
    mag = np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
    half_ulp = np.exp2(np.floor(np.log2(mag)) - MANTISSA_BITS[dtype] - 1)
    if dtype == "f32":
        return ATOL[dtype] + 0 * half_ulp
    return ATOL[dtype] + half_ulp


def assert_close(got, want: np.ndarray, dtype: str, what: str = ""):
    g = got.detach().to("cpu", torch.float64).numpy() if isinstance(got, torch.Tensor) else got
    assert g.shape == want.shape, (g.shape, want.shape)
    mask = ~np.isnan(want)
    err = np.abs(g[mask] - want[mask])
    tol = tolerance(dtype, want[mask])
    bad = err > tol
    if bad.any():
        i = int(np.argmax(err - tol))
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements exceed the bound; "
                             f"worst err {err[i]:.3e} > tol {tol[i]:.3e} (ref {want[mask][i]:.4f})")
    return float(err.max()) if err.size else 0.0


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class StepOut:
    def __init__(self, out, slots, pairs, tables, lens, seq_ids):
        self.out, self.slots, self.pairs = out, slots, pairs
        self.tables, self.lens, self.seq_ids = tables, lens, seq_ids


class NativeReplay:
    def __init__(self, w, d, fill=float("nan"), partition_tokens: int = 0):
        self.w, self.d = w, d
        self.cache = PagedKVCache(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                  w.pool_dtype, free_order=d.free_order, fill=fill,
                                  k_scale=w.k_scale, v_scale=w.v_scale)
        self.slot_of = {}
        self.partition_tokens = partition_tokens
        self.steps = []

    def _dev(self, t):
        return t.to("cuda").contiguous()

    def run(self, ops, max_blocks=None):
        c = self.cache
        for op in ops:
            kind = op[0]
            if kind == "add":
                self.slot_of[op[1]] = c.add()
            elif kind in ("prefill", "suffix"):
                sid = self.slot_of[op[1]]
                ks = self.d.prefill_k if kind == "prefill" else self.d.suffix_k
                vs = self.d.prefill_v if kind == "prefill" else self.d.suffix_v
                c.append(sid, self._dev(ks[op[2]]), self._dev(vs[op[2]]))
            elif kind == "fork":
                self.slot_of[op[1]] = c.fork(self.slot_of[op[2]])
            elif kind == "free":
                c.free(self.slot_of.pop(op[1]))
            elif kind == "step":
                t = op[1]
                seqs = [self.slot_of[s] for s in range(self.w.num_seqs)]
                out, slots, pairs, tables, lens = c.step(
                    seqs, self._dev(self.d.step_k[t]), self._dev(self.d.step_v[t]),
                    self._dev(self.d.step_q[t]), max_blocks=max_blocks,
                    partition_tokens=self.partition_tokens)
                self.steps.append(StepOut(out, slots, pairs, tables, lens, seqs))
            else:
                raise ValueError(kind)
        return self.steps


def sample_pairs(lens, H, k, seed):
    """k (text, head) pairs: the shortest and longest texts plus a seeded random draw."""
    rng = np.random.default_rng(seed)
    S = len(lens)
    order = np.argsort(np.asarray(lens), kind="stable")
    picks = {(int(order[0]), 0), (int(order[-1]), H - 1), (0, 0), (S - 1, H - 1)}
    while len(picks) < min(k, S * H):
        picks.add((int(rng.integers(S)), int(rng.integers(H))))
    return sorted(picks)

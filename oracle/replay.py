"""Replays a workload's operation script through the oracle pieces.

One decode step («The KV Cache and PagedAttention» › "One Token at a Time",
«KV cache» › "How it works") for every text of the batch, in batch order:
  1. the allocator gives the new token its slot, copying a shared partly
     filled last block first (› "The Block Table", › "Shared, Copied on Write");
  2. the copies are made (whole blocks, before any new token is written, so
     a copy never carries a sharer's new token);
  3. the new tokens' keys and values are written into their slots;
  4. every text's query attends over its whole cache, new token included.

Two modes:
  pool=True   full byte-level pools (small workloads): attention gathers
              through the exported block tables.
  pool=False  no pools (multi-gigabyte workloads): each text keeps the
              ordered list of the token data written to it, and attention for
              the requested (text, head) pairs runs on that contiguous copy
              (for E4M3 pools, on the values that data is stored as).
              The allocator still runs, so its tables can be compared.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

from . import attention, cache_ops
from .allocator import BlockAllocator


class StepResult:
    def __init__(self):
        self.seq_ids: List[int] = []
        self.slots: List[int] = []
        self.pairs: List[tuple] = []
        self.tables: Optional[np.ndarray] = None
        self.lens: List[int] = []
        self.out: Optional[np.ndarray] = None  # [S, H, D] float64 (NaN where not computed)


class Replay:
    def __init__(self, w, d, pool: bool = True, max_blocks: Optional[int] = None):
        import torch
        self.w, self.d, self.pool = w, d, pool
        self.alloc = BlockAllocator(w.num_blocks, w.block_size, d.free_order)
        self.slot_of: Dict[object, int] = {}  # batch position -> sequence id
        self.tokens: Dict[int, list] = {}      # logical mode: seq id -> [(k, v) chunks]
        self.max_blocks = max_blocks
        self.fp8 = getattr(w, "pool_dtype", w.dtype) == "fp8"
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        if pool:
            shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
            if self.fp8:  # E4M3 codes; 0x7F (NaN) where nothing was written
                self.k = torch.full(shape, 0x7F, dtype=torch.uint8)
                self.v = torch.full(shape, 0x7F, dtype=torch.uint8)
            else:
                self.k = torch.full(shape, float("nan"), dtype=tdt)
                self.v = torch.full(shape, float("nan"), dtype=tdt)
        self.steps: List[StepResult] = []

    def _cache_write(self, k, v, slots):
        if self.fp8:
            cache_ops.kv_write_fp8(self.k, self.v, k.cpu(), v.cpu(), slots, self.w.block_size,
                                   self.w.k_scale, self.w.v_scale)
        else:
            cache_ops.kv_write(self.k, self.v, k.cpu(), v.cpu(), slots, self.w.block_size)

    def stored_values(self, x, scale: float) -> np.ndarray:
        """fp64 values the cache holds for written data x (E4M3 pools: quantized with
        `scale`, then dequantized; other pools: x itself)."""
        if not self.fp8:
            return attention.to_f64(x)
        from . import fp8
        return fp8.dequantize(cache_ops.quantize_rows(x, scale).numpy(), scale)

    def _write(self, sid: int, k, v, slots, pair):
        if self.pool:
            if pair[0] >= 0:
                cache_ops.copy_blocks(self.k, self.v, [pair])
            self._cache_write(k, v, slots)
        else:
            self.tokens[sid].append((k, v))

    def run(self, ops, decode_pairs=None) -> List[StepResult]:
        """Replay `ops`; `decode_pairs(step)` may restrict the (s, h) computed."""
        w, d, a = self.w, self.d, self.alloc
        for op in ops:
            kind = op[0]
            if kind == "add":
                sid = a.add()
                self.slot_of[op[1]] = sid
                self.tokens[sid] = []
            elif kind in ("prefill", "suffix"):
                sid = self.slot_of[op[1]]
                src_k = d.prefill_k if kind == "prefill" else d.suffix_k
                src_v = d.prefill_v if kind == "prefill" else d.suffix_v
                k, v = src_k[op[2]], src_v[op[2]]
                slots, pair = a.append(sid, k.shape[0])
                self._write(sid, k, v, slots, pair)
            elif kind == "fork":
                sid = a.fork(self.slot_of[op[2]])
                self.slot_of[op[1]] = sid
                self.tokens[sid] = list(self.tokens[self.slot_of[op[2]]])
            elif kind == "free":
                sid = self.slot_of.pop(op[1])
                a.free_seq(sid)
                self.tokens.pop(sid, None)
            elif kind == "step":
                self.steps.append(self._step(op[1], decode_pairs))
            else:
                raise ValueError(kind)
        return self.steps

    def _step(self, t: int, decode_pairs) -> StepResult:
        w, d, a = self.w, self.d, self.alloc
        r = StepResult()
        S = w.num_seqs
        r.seq_ids = [self.slot_of[s] for s in range(S)]
        for sid in r.seq_ids:
            slots, pair = a.append(sid, 1)
            r.slots.extend(slots)
            if pair[0] >= 0:
                r.pairs.append(pair)
        k_new, v_new, q = d.step_k[t], d.step_v[t], d.step_q[t].cpu()
        if self.pool:
            cache_ops.copy_blocks(self.k, self.v, r.pairs)
            self._cache_write(k_new, v_new, r.slots)
        else:
            for i, sid in enumerate(r.seq_ids):
                self.tokens[sid].append((k_new[i:i + 1], v_new[i:i + 1]))
        mb = self.max_blocks or max(len(a.blocks[sid]) for sid in r.seq_ids)
        tables, lens = a.export(r.seq_ids, mb)
        r.tables = np.asarray(tables, dtype=np.int32)
        r.lens = lens
        pairs = decode_pairs(t) if decode_pairs is not None else None
        if self.pool:
            r.out = attention.decode_attention(q, self.k, self.v, r.tables, lens,
                                               w.block_size, pairs=pairs,
                                               k_scale=getattr(w, "k_scale", 1.0),
                                               v_scale=getattr(w, "v_scale", 1.0))
        else:
            r.out = self.logical_attention(q, r.seq_ids, pairs)
        return r

    def logical_attention(self, q, seq_ids, pairs) -> np.ndarray:
        import torch
        w = self.w
        S, H, D = q.shape
        group = H // w.num_kv_heads
        out = np.full((S, H, D), np.nan)
        qd = attention.to_f64(q)
        scale = 1.0 / math.sqrt(D)
        if pairs is None:
            pairs = [(s, h) for s in range(S) for h in range(H)]
        by_seq: Dict[int, list] = {}
        for s, h in pairs:
            by_seq.setdefault(s, []).append(h)
        for s, heads in by_seq.items():
            chunks = self.tokens[seq_ids[s]]
            for h in heads:
                kvh = h // group
                kh = self.stored_values(torch.cat([c[0][:, kvh].cpu() for c in chunks]),
                                        w.k_scale) if chunks else np.zeros((0, D))
                vh = self.stored_values(torch.cat([c[1][:, kvh].cpu() for c in chunks]),
                                        w.v_scale) if chunks else np.zeros((0, D))
                out[s, h] = attention.softmax_attention(qd[s, h], kh, vh, scale)
        return out

"""The five workloads replayed through the native path and the oracle.

Tiny and scaled-down workloads: whole pools, tables, slots and copy pairs
bit-exact, every output element checked. Full-size workloads (the launch
configuration the bench times): tables, slots and copy pairs bit-exact at every
step, sampled slots of the pools bit-exact against the written tokens, and
sampled (text, head) outputs against the oracle computed one by one.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_common import NativeReplay, StepOut, assert_close, sample_pairs, say
from oracle import cache_ops
from oracle.replay import Replay

pytestmark = pytest.mark.gpu


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.element_size() == 1:
        return t
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


# Relative bound on max |error| / max |out| over the checked outputs: half an ulp of the
# output format (its rounding) plus 1e-3 of fp32 accumulation room; fp32 outputs 1e-5.
REL_GATE = {"f32": 1e-5, "f16": 2.0 ** -11 + 1e-3, "bf16": 2.0 ** -8 + 1e-3}


def relative_error(nat_steps, ora_steps, pairs_for):
    """max |got - want| / max |want| over every step's checked outputs."""
    num = den = 0.0
    for t, (n, o) in enumerate(zip(nat_steps, ora_steps)):
        got = n.out.cpu().to(torch.float64).numpy()
        want = o.out
        for s, h in pairs_for(t):
            num = max(num, float(np.abs(got[s, h] - want[s, h]).max()))
            den = max(den, float(np.abs(want[s, h]).max()))
    return num / den, num, den


def log_parity(record: dict):
    """Append one JSON line to $PA_PARITY_LOG (if set): the full-size parity figures."""
    import json
    import os
    path = os.environ.get("PA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def compare_steps(w, nat_steps, ora_steps, pairs_for=None, strict_gate=False):
    assert len(nat_steps) == len(ora_steps) == w.steps
    worst = 0.0
    for t, (n, o) in enumerate(zip(nat_steps, ora_steps)):
        assert n.slots == o.slots, f"step {t}: slots differ"
        assert n.pairs == [tuple(p) for p in o.pairs], f"step {t}: copy pairs differ"
        assert np.array_equal(n.tables, o.tables), f"step {t}: block tables differ"
        assert list(n.lens) == list(o.lens), f"step {t}: context lengths differ"
        got = n.out.cpu().to(torch.float64).numpy()
        want = o.out
        if pairs_for is not None:
            mask = np.zeros(want.shape[:2], bool)
            for s, h in pairs_for(t):
                mask[s, h] = True
            got = np.where(mask[..., None], got, np.nan)
        worst = max(worst, assert_close(got, want, w.dtype, f"{w.name} step {t}"))
        if strict_gate:
            m = ~np.isnan(want)
            err = float(np.abs(got[m] - want[m]).max())
            gate = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}[w.dtype]
            assert err <= gate, f"{w.name} step {t}: max abs error {err:.3e} > {gate}"
    return worst


def test_tiny_workload_whole_pool(native):
    w = wl.TINY
    say(f"workload {w.name}")
    d = wl.draw(w)
    ops = wl.script(w, d)
    nat = NativeReplay(w, d)
    ns = nat.run(ops)
    ora = Replay(w, d, pool=True)
    os_ = ora.run(ops)
    err = compare_steps(w, ns, os_, strict_gate=True)
    torch.cuda.synchronize()
    assert torch.equal(bits(nat.cache.k[0]), bits(ora.k)) and torch.equal(bits(nat.cache.v[0]), bits(ora.v))
    say(f"  max abs error {err:.3e}")


@pytest.mark.parametrize("dtype,B,cache", [("bf16", 4, ""), ("f16", 16, ""), ("f32", 8, ""),
                                           ("f16", 16, "fp8"), ("bf16", 4, "fp8")])
def test_scaled_sharing_whole_pool(native, dtype, B, cache):
    """Copy-on-write every step (parallel samples / beams), small enough for whole pools."""
    w = wl.SHARING_32x8.scaled(groups=3, samples=4, num_seqs=12, num_heads=4, num_kv_heads=4,
                               head_dim=64, block_size=B, num_blocks=160, prompt_len=6 * B + 3,
                               suffix_lo=0, suffix_hi=2 * B + 1, steps=4, dtype=dtype,
                               kv_std=1.0 if dtype == "f32" else 0.125, cache_dtype=cache,
                               k_scale=1 / 64 if cache else 1.0, v_scale=1 / 32 if cache else 1.0)
    say(f"workload {w.name} scaled dtype={dtype} B={B}")
    d = wl.draw(w)
    ops = wl.script(w, d)
    nat = NativeReplay(w, d)
    ns = nat.run(ops)
    ora = Replay(w, d, pool=True)
    os_ = ora.run(ops)
    compare_steps(w, ns, os_)
    assert sum(len(s.pairs) for s in ns) > 0, "the workload must exercise copy-on-write"
    torch.cuda.synchronize()
    assert torch.equal(bits(nat.cache.k[0]), bits(ora.k)) and torch.equal(bits(nat.cache.v[0]), bits(ora.v))


def check_sampled_slots(nat, ora, w, d, nsamples=256, seed=0):
    """Pool places of sampled (text, token) positions hold exactly the written token."""
    rng = np.random.default_rng(seed)
    a = ora.alloc
    live = list(a.blocks)
    for _ in range(nsamples):
        sid = live[int(rng.integers(len(live)))]
        L = a.context_len(sid)
        t = int(rng.integers(L))
        blk = a.blocks[sid][t // w.block_size]
        place = t % w.block_size
        # the t-th written token of this text, from the oracle's logical record
        chunks = ora.tokens[sid]
        k_tok = None
        for ck, cv in chunks:
            if t < ck.shape[0]:
                k_tok, v_tok = ck[t], cv[t]
                break
            t -= ck.shape[0]
        got_k = nat.cache.k[0][blk, :, place]
        got_v = nat.cache.v[0][blk, :, place]
        if w.pool_dtype == "fp8":
            # E4M3 pools: the stored codes are the oracle's quantization of the token
            assert torch.equal(got_k.cpu(), cache_ops.quantize_rows(k_tok, w.k_scale)) and \
                torch.equal(got_v.cpu(), cache_ops.quantize_rows(v_tok, w.v_scale))
        else:
            assert torch.equal(bits(got_k), bits(k_tok)) and torch.equal(bits(got_v), bits(v_tok))


FULL = [wl.OPT13B_7x2048, wl.OPT13B_MIXED256, wl.SHARING_32x8, wl.LONG_16x32K,
        wl.LLAMA70B_32x4096, wl.OPT13B_7x2048_FP8]


def run_full_size(w, nsample=48, strict_gate=True):
    """The workload's script through the native path (the bench's launch configuration:
    random placement, NaN in every place never written) and through the oracle in logical
    mode; every (text, head) output compared when there are at most 280, else a seeded
    sample. Returns (worst abs error, relative error, pairs checked per step)."""
    d = wl.draw(w, device="cuda")
    ops = wl.script(w, d)
    nat = NativeReplay(w, d)
    ns = nat.run(ops)
    torch.cuda.synchronize()
    say("  native path done")
    every = w.num_seqs * w.num_heads <= 280
    lens0 = wl.attended_at_step0(w, d)

    def pairs_for(t):
        if every:
            return [(s, h) for s in range(w.num_seqs) for h in range(w.num_heads)]
        return sample_pairs(lens0, w.num_heads, nsample, seed=t)

    ora = Replay(w, d, pool=False)
    os_ = ora.run(ops, decode_pairs=pairs_for)
    say("  oracle done")
    err = compare_steps(w, ns, os_, pairs_for=pairs_for, strict_gate=strict_gate)
    check_sampled_slots(nat, ora, w, d)
    if w.length_kind == "sharing":
        assert sum(len(s.pairs) for s in ns) > 0
    rel, num, den = relative_error(ns, os_, pairs_for)
    return err, rel, den, len(pairs_for(0))


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_size_workload(native, w):
    say(f"workload {w.name} (full size)")
    err, rel, den, npairs = run_full_size(w)
    say(f"  max abs error {err:.3e}; relative {rel:.3e} (max |out| {den:.3e})")
    log_parity({"workload": w.name, "variant": "plain", "steps": w.steps,
                "pairs_per_step": npairs, "max_abs_err": err, "max_abs_out": den,
                "rel_err": rel})


SHARP = [wl.OPT13B_7x2048, wl.OPT13B_MIXED256, wl.LONG_16x32K, wl.LLAMA70B_32x4096,
         wl.OPT13B_7x2048_FP8]


@pytest.mark.parametrize("base", SHARP, ids=lambda w: w.name)
def test_full_size_sharp(native, base):
    """Each full-size workload with a peaked softmax (queries x 32, values N(0, 1): scores
    of standard deviation ~2.8, outputs of order 1 made of few tokens), at its shapes and
    pool size (the 6.4 and 5.4 GB pools of the mixed and long workloads put blocks past
    4 GiB), random placement and NaN in every unwritten place. Gated on the absolute bound
    and on max |error| / max |out|: an output that attended a wrong, dropped or doubled
    block moves by far more than either."""
    w = wl.sharp(base)
    say(f"workload {w.name} (full size, sharp)")
    err, rel, den, npairs = run_full_size(w, nsample=64, strict_gate=False)
    gate = REL_GATE[w.dtype]
    say(f"  max abs error {err:.3e}; relative {rel:.3e} (max |out| {den:.3e}, gate {gate:.2e})")
    log_parity({"workload": w.name, "variant": "sharp", "steps": w.steps,
                "pairs_per_step": npairs, "max_abs_err": err, "max_abs_out": den,
                "rel_err": rel, "rel_gate": gate})
    assert den > 0.5, "the sharp variant must give outputs of order 1"
    assert rel <= gate, f"{w.name}: relative error {rel:.3e} > {gate:.2e}"


class SharedDecodes(NativeReplay):
    """The native replay, plus after every step the decode over shared blocks on the same
    pools, tables, lengths and queries, in the bench's launch configuration: prompt groups
    once per group (pa_decode_attention_prefix), and prompt groups with each forked pair's
    blocks once per pair (pa_decode_attention_prefix2)."""

    def run(self, ops, max_blocks=None):
        self.shared = {"prefix": [], "nested": [], "derived": []}
        for op in ops:
            super().run([op], max_blocks)
            if op[0] == "step":
                self._shared_decode(op[1])
        return self.steps

    def _shared_decode(self, t):
        from paged_kv_cache_320_amd import _lib as L
        w, st = self.w, self.steps[-1]
        S, H, Hkv, D, B = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
        bt = torch.from_numpy(np.ascontiguousarray(st.tables, dtype=np.int32)).cuda()
        cl = torch.from_numpy(np.asarray(st.lens, dtype=np.int32)).cuda()
        q = self._dev(self.d.step_q[t])
        kc, vc = self.cache.k[0], self.cache.v[0]
        mx = int(max(st.lens))
        G, J, P = w.groups, w.samples, w.prompt_len
        i32 = dict(dtype=torch.int32, device="cuda")
        gf, gc, gp = torch.arange(0, S, J, **i32), torch.full((G,), J, **i32), \
            torch.full((G,), P, **i32)
        pf, pc, pp = torch.arange(0, S, 2, **i32), torch.full((S // 2,), 2, **i32), \
            torch.full((S // 2,), mx, **i32)
        code = L.dtype_code(q)
        ws1 = torch.empty(L.pa_decode_prefix_workspace_bytes(S, H, Hkv, D, B, mx, G, P, code),
                          dtype=torch.uint8, device="cuda")
        out1 = torch.empty_like(q)
        L.pa_decode_attention_prefix(out1, q, kc, vc, bt, cl, mx, gf, gc, gp, P, ws1)
        ws2 = torch.empty(L.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, mx, G, P, S // 2,
                                                              mx, 2, code),
                          dtype=torch.uint8, device="cuda")
        out2 = torch.empty_like(q)
        L.pa_decode_attention_prefix2(out2, q, kc, vc, bt, cl, mx, gf, gc, gp, P, pf, pc, pp, mx,
                                      2, ws2)
        self.shared["prefix"].append(out1)
        self.shared["nested"].append(out2)
        # the groups read off the block tables by the allocator (pa_share_groups)
        outer, inner = self.cache.alloc.share_groups(st.seq_ids, J, inner_members=2)
        dv = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        assert len(outer[0]) == G and len(inner[0]) >= 1
        ws3 = torch.empty(L.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, mx, len(outer[0]),
                                                              mx, len(inner[0]), mx, 2, code),
                          dtype=torch.uint8, device="cuda")
        out3 = torch.empty_like(q)
        L.pa_decode_attention_prefix2(out3, q, kc, vc, bt, cl, mx, *map(dv, outer), mx,
                                      *map(dv, inner), mx, 2, ws3)
        self.shared["derived"].append(out3)


@pytest.mark.parametrize("variant", ["plain", "sharp"])
def test_full_size_sharing_shared_block_decodes(native, variant):
    """The sharing workload at full size (32 groups x 8 samples, 1,024-token prompts, pair
    forks with copy-on-write every step): both shared-block decodes against the oracle on
    sampled (text, head) pairs, every step, within the plain 2e-3 gate (plain variant) or
    the per-element bound and the relative bound (sharp variant: queries x 32, values
    N(0, 1))."""
    w = wl.SHARING_32x8 if variant == "plain" else wl.sharp(wl.SHARING_32x8)
    say(f"workload {w.name} (full size), shared-block decodes")
    d = wl.draw(w, device="cuda")
    ops = wl.script(w, d)
    nat = SharedDecodes(w, d)
    ns = nat.run(ops)
    torch.cuda.synchronize()
    lens0 = wl.attended_at_step0(w, d)

    def pairs_for(t):
        return sample_pairs(lens0, w.num_heads, 48, seed=100 + t)

    ora = Replay(w, d, pool=False)
    os_ = ora.run(ops, decode_pairs=pairs_for)
    for kind in ("plain", "prefix", "nested", "derived"):
        if kind == "plain":
            steps = ns
        else:
            steps = [StepOut(o, s.slots, s.pairs, s.tables, s.lens, s.seq_ids)
                     for o, s in zip(nat.shared[kind], ns)]
        err = compare_steps(w, steps, os_, pairs_for=pairs_for, strict_gate=variant == "plain")
        rel, num, den = relative_error(steps, os_, pairs_for)
        say(f"  {kind}: max abs error {err:.3e}; relative {rel:.3e} (max |out| {den:.3e})")
        log_parity({"workload": w.name, "variant": variant, "decode": kind, "steps": w.steps,
                    "pairs_per_step": len(pairs_for(0)), "max_abs_err": err,
                    "max_abs_out": den, "rel_err": rel})
        if variant == "sharp":
            assert den > 0.5 and rel <= REL_GATE[w.dtype], (kind, rel)

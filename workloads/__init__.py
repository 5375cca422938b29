"""Seeded synthetic inputs for the paged decode path.

This module only draws random numbers and fixes the shapes of each workload.
It holds no attention, cache-write or block-allocation arithmetic, so the
oracle and the HIP library can both consume its output without sharing any
of the method's code.

The workloads stand in for the pages' OPT-13B serving setting: OPT-13B keeps
keys and values of 5,120 numbers per token and layer in 16-bit floats
(«The KV Cache and PagedAttention» › "800 KB a Token"), vLLM's default block
holds 16 tokens and the explanatory drawings use 4 (› "Like Pages of Memory").
The pages' request traces (ShareGPT, Alpaca) are not available; lengths are
drawn from the fixed distributions named per workload instead.

Draw order for one workload, all from one seeded stream:
  free-list permutation -> lengths -> per sequence: prefill K then prefill V
  -> per step: new k, new v, then q.
Values are drawn as float32 N(0, 1), multiplied by the workload's standard
deviation and rounded to the storage dtype (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    kv_std: float
    q_std: float
    steps: int = 1
    # standard deviation of the values when it differs from the keys' (0: kv_std)
    v_std: float = 0.0
    # "fixed": every sequence attends `ctx_fixed` tokens at step 0.
    # "list": attended lengths at step 0 are `ctx_list`.
    # "uniform": attended lengths ~ U{ctx_lo..ctx_hi} (inclusive).
    # "sharing": groups sharing a prompt (see sharing_* fields).
    length_kind: str = "fixed"
    ctx_fixed: int = 0
    ctx_list: tuple = ()
    ctx_lo: int = 0
    ctx_hi: int = 0
    groups: int = 0
    samples: int = 0
    prompt_len: int = 0
    suffix_lo: int = 0
    suffix_hi: int = 0
    # key/value pool format when it differs from `dtype` ("fp8": OCP E4M3 codes with one
    # scale per pool; the drawn keys/values are `dtype` values quantized on write)
    cache_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0
    description: str = ""

    @property
    def pool_dtype(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def value_std(self) -> float:
        return self.v_std or self.kv_std

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Attended lengths count the step's new token, whose
# key and value are written before attention reads the cache («KV cache» ›
# "How it works": the new position's own key is compared as well).
TINY = Workload(
    name="tiny_4x4x64_f32_b4", seed=1, num_seqs=4, num_heads=4, num_kv_heads=4,
    head_dim=64, block_size=4, num_blocks=64, dtype="f32", kv_std=1.0, q_std=1.0,
    length_kind="list", ctx_list=(5, 13, 22, 37),
    description="4 sequences, 4 heads x 64, fp32, block 4, attended {5,13,22,37}")

OPT13B_7x2048 = Workload(
    name="opt13b_7x2048_f16_b16", seed=2, num_seqs=7, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=983, dtype="f16",
    kv_std=1.0 / math.sqrt(128.0), q_std=1.0, length_kind="fixed", ctx_fixed=2048,
    description="OPT-13B one layer: 40 heads x 128, fp16, block 16, 7 x 2048 tokens, "
                "983-block pool (12 GiB / 40 layers), random placement")

OPT13B_MIXED256 = Workload(
    name="opt13b_mixed256_f16_b16", seed=3, num_seqs=256, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=39250, dtype="f16",
    kv_std=1.0 / math.sqrt(128.0), q_std=1.0, length_kind="uniform", ctx_lo=16, ctx_hi=2048,
    description="OPT-13B one layer, 256 sequences, attended lengths U{16..2048}, "
                "39,250-block pool (15,700 x 40 token slots)")

SHARING_32x8 = Workload(
    name="sharing_32x8_bf16_b16", seed=4, num_seqs=256, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=12288, dtype="bf16",
    kv_std=1.0 / math.sqrt(128.0), q_std=1.0, steps=4, length_kind="sharing",
    groups=32, samples=8, prompt_len=1024, suffix_lo=0, suffix_hi=512,
    description="32 groups x 8 samples sharing a 1,024-token prompt, suffixes U{0..512}, "
                "4 steps of pair fork -> append (copy-on-write) -> write -> decode")

LONG_16x32K = Workload(
    name="long_16x32k_f16_b16", seed=5, num_seqs=16, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=32800, dtype="f16",
    kv_std=1.0 / math.sqrt(128.0), q_std=1.0, steps=4, length_kind="fixed", ctx_fixed=32768,
    description="16 sequences x 32,768 tokens, 4 generation steps (32,768..32,771)")

# Heads sharing key/value sets (P1 "What Came After": Llama 2 70B gives its 64 heads 8
# sets). One layer of that shape: 64 query heads, 8 key/value heads of 128, fp16, block 16,
# 32 texts x 4,096 tokens (the model's context length); not one of the five workloads above,
# it measures the shared-head path.
LLAMA70B_32x4096 = Workload(
    name="llama2_70b_32x4096_f16_b16", seed=6, num_seqs=32, num_heads=64, num_kv_heads=8,
    head_dim=128, block_size=16, num_blocks=32 * 257 + 64, dtype="f16",
    kv_std=1.0 / math.sqrt(128.0), q_std=1.0, length_kind="fixed", ctx_fixed=4096,
    description="Llama-2-70B-shaped layer: 64 query heads sharing 8 key/value heads of 128, "
                "fp16, block 16, 32 x 4,096 tokens")

GQA4_32x4096 = Workload(
    name="gqa4_32x4096_f16_b16", seed=7, num_seqs=32, num_heads=32, num_kv_heads=8,
    head_dim=128, block_size=16, num_blocks=32 * 257 + 64, dtype="f16",
    kv_std=1 / math.sqrt(128), q_std=1.0, steps=4, length_kind="fixed", ctx_fixed=4096,
    description="shared K/V heads, 4 query heads per K/V head: 32 query heads over 8 K/V "
                "heads x 128, fp16, block 16, 32 texts x 4096 tokens")
# The cache kept in 8-bit floating point (P1 "What Came After": one byte a number, about
# twice the tokens in the same memory): the OPT-13B 7 x 2,048 step with E4M3 pools. The
# scales 1/256 (exact reciprocals) map the drawn keys/values (std 0.088) well inside E4M3's
# range (448 * 1/256 = 1.75, about 20 standard deviations).
OPT13B_7x2048_FP8 = OPT13B_7x2048.scaled(
    name="opt13b_7x2048_fp8_b16", cache_dtype="fp8", k_scale=1 / 256, v_scale=1 / 256,
    description="OPT-13B one layer with an E4M3 cache: 40 heads x 128, fp16 queries, "
                "block 16, 7 x 2048 tokens, pool scales 1/256")

# Many short texts (a serving batch of fresh requests): 4,096 texts of 16..64 tokens, where
# the per-text costs of the decode launch (finding each wave's first text, finishing runs)
# weigh most.
SHORT_4096 = Workload(
    name="short4096_f16_b16", seed=8, num_seqs=4096, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=4096 * 7 + 64, dtype="f16",
    kv_std=1 / math.sqrt(128), q_std=1.0, length_kind="uniform", ctx_lo=16, ctx_hi=64,
    description="4,096 texts of U{16..64} attended tokens, OPT-13B shapes (40 x 128), fp16, "
                "block 16")

ALL = (TINY, OPT13B_7x2048, OPT13B_MIXED256, SHARING_32x8, LONG_16x32K)


def sharp(w: Workload) -> Workload:
    """The workload with a peaked softmax: queries x 32 (scores of standard deviation about
    2.8 instead of 0.088) and values N(0, 1), so that a dropped, doubled or misplaced block
    moves the output by far more than the accuracy bound. E4M3 pools keep the values inside
    the format's range with a value scale of 1/32 (largest code 448 / 32 = 14)."""
    kw = dict(name=w.name + "_sharp", q_std=32.0 * w.q_std, v_std=1.0,
              description=w.description + "; sharp: queries x 32, values N(0, 1)")
    if w.pool_dtype == "fp8":
        kw["v_scale"] = 1 / 32
    return w.scaled(**kw)


# --- Prompt-phase workloads ----------------------------------------------------
# The prompt phase takes each text's whole prompt at once («The KV Cache and
# PagedAttention» › "One Token at a Time"); a prompt may follow cached tokens, e.g.
# a shared prefix whose blocks are reused (› "What Came After").

@dataclasses.dataclass(frozen=True)
class PromptWorkload:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    kv_std: float
    q_std: float
    prompt_lo: int           # prompt lengths ~ U{prompt_lo..prompt_hi} (equal: fixed)
    prompt_hi: int
    prefix_len: int = 0      # cached tokens, the same for every text, before each prompt
    description: str = ""

    def scaled(self, **kw) -> "PromptWorkload":
        return dataclasses.replace(self, **kw)


OPT13B_PROMPT_7x2048 = PromptWorkload(
    name="opt13b_prompt_7x2048_f16_b16", seed=12, num_seqs=7, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=983, dtype="f16", kv_std=1 / math.sqrt(128),
    q_std=1.0, prompt_lo=2048, prompt_hi=2048,
    description="prompt phase of the OPT-13B 7 x 2048 batch: 7 fresh 2,048-token prompts, "
                "40 heads x 128, fp16, block 16")
OPT13B_PROMPT_MIXED64 = PromptWorkload(
    name="opt13b_prompt_mixed64_f16_b16", seed=13, num_seqs=64, num_heads=40, num_kv_heads=40,
    head_dim=128, block_size=16, num_blocks=8300, dtype="f16", kv_std=1 / math.sqrt(128),
    q_std=1.0, prompt_lo=16, prompt_hi=2048,
    description="64 fresh prompts of U{16..2048} tokens, OPT-13B shapes, fp16, block 16")
LLAMA70B_PROMPT_8x4096 = PromptWorkload(
    name="llama2_70b_prompt_8x4096_f16_b16", seed=14, num_seqs=8, num_heads=64, num_kv_heads=8,
    head_dim=128, block_size=16, num_blocks=8 * 256 + 64, dtype="f16",
    kv_std=1 / math.sqrt(128), q_std=1.0, prompt_lo=4096, prompt_hi=4096,
    description="shared K/V heads: 64 query heads over 8 K/V heads x 128, 8 fresh "
                "4,096-token prompts, fp16, block 16")
OPT13B_PREFIX_32x1024 = PromptWorkload(
    name="opt13b_prefix_32x1024p512_f16_b16", seed=15, num_seqs=32, num_heads=40,
    num_kv_heads=40, head_dim=128, block_size=16, num_blocks=64 + 32 * 32 + 64, dtype="f16",
    kv_std=1 / math.sqrt(128), q_std=1.0, prompt_lo=512, prompt_hi=512, prefix_len=1024,
    description="32 prompts of 512 new tokens after one shared, cached 1,024-token prefix "
                "(64 blocks held by all 32 texts), OPT-13B shapes, fp16, block 16")
PROMPT = (OPT13B_PROMPT_7x2048, OPT13B_PROMPT_MIXED64, LLAMA70B_PROMPT_8x4096,
          OPT13B_PREFIX_32x1024)
EXTRA = (LLAMA70B_32x4096, OPT13B_7x2048_FP8, GQA4_32x4096, SHORT_4096)
BY_NAME = {w.name: w for w in ALL + EXTRA + PROMPT}


def _np_dtype_cast(x32: np.ndarray, dtype: str):
    """Round float32 draws to the storage dtype; returns a torch CPU tensor.

    torch's CPU casts round to nearest even for fp16 and bf16.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype])


class Stream:
    """One seeded stream of draws, numpy PCG64 (host) or torch Philox (device).

    The host stream is used where the oracle must also see every value; the
    device stream fills the multi-gigabyte workloads in milliseconds, and the
    oracle then reads back only the slices it checks.
    """

    def __init__(self, seed: int, device: Optional[str] = None):
        self.device = device
        if device is None:
            self.rng = np.random.Generator(np.random.PCG64(seed))
        else:
            import torch
            self.gen = torch.Generator(device=device)
            self.gen.manual_seed(seed)
            self.rng = np.random.Generator(np.random.PCG64(seed))  # integers stay on host

    def permutation(self, n: int) -> np.ndarray:
        return self.rng.permutation(n).astype(np.int32)

    def integers(self, lo: int, hi_inclusive: int, size: int) -> np.ndarray:
        return self.rng.integers(lo, hi_inclusive + 1, size=size).astype(np.int64)

    def normal(self, shape: Sequence[int], std: float, dtype: str):
        """float32 N(0, std^2) rounded to `dtype`; a torch tensor (CPU or device)."""
        import torch
        if self.device is None:
            x = self.rng.standard_normal(size=tuple(shape), dtype=np.float32)
            if std != 1.0:
                x *= np.float32(std)
            return _np_dtype_cast(x, dtype)
        x = torch.randn(tuple(shape), generator=self.gen, device=self.device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(float(std))
        return x.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype])


@dataclasses.dataclass
class Draws:
    """Every random input of one workload (torch tensors, CPU or device).

    prefill_k[i] / prefill_v[i]: [n_i, H_kv, D] for prefill sequence i (the
      prompt of group i for the sharing workload).
    suffix_k / suffix_v (sharing only): per sample, [suffix_len, H_kv, D].
    step_k / step_v: per step, [S, H_kv, D]; step_q: per step, [S, H, D].
    """
    free_order: np.ndarray
    prefill_lens: List[int]
    prefill_k: list
    prefill_v: list
    step_k: list
    step_v: list
    step_q: list
    suffix_lens: List[int] = dataclasses.field(default_factory=list)
    suffix_k: list = dataclasses.field(default_factory=list)
    suffix_v: list = dataclasses.field(default_factory=list)


def draw(w: Workload, device: Optional[str] = None) -> Draws:
    """All inputs of workload `w`, in the fixed draw order of this module."""
    st = Stream(w.seed, device)
    free_order = st.permutation(w.num_blocks)
    Hk, D = w.num_kv_heads, w.head_dim
    suffix_lens: List[int] = []
    if w.length_kind == "fixed":
        attended = [w.ctx_fixed] * w.num_seqs
    elif w.length_kind == "list":
        attended = list(w.ctx_list)
        assert len(attended) == w.num_seqs
    elif w.length_kind == "uniform":
        attended = [int(x) for x in st.integers(w.ctx_lo, w.ctx_hi, w.num_seqs)]
    elif w.length_kind == "sharing":
        assert w.groups * w.samples == w.num_seqs
        suffix_lens = [int(x) for x in st.integers(w.suffix_lo, w.suffix_hi, w.num_seqs)]
        attended = []
    else:
        raise ValueError(w.length_kind)

    if w.length_kind == "sharing":
        prefill_lens = [w.prompt_len] * w.groups
    else:
        prefill_lens = [a - 1 for a in attended]
    pk, pv = [], []
    for n in prefill_lens:
        pk.append(st.normal((n, Hk, D), w.kv_std, w.dtype))
        pv.append(st.normal((n, Hk, D), w.value_std, w.dtype))
    sk, sv = [], []
    for n in suffix_lens:
        sk.append(st.normal((n, Hk, D), w.kv_std, w.dtype))
        sv.append(st.normal((n, Hk, D), w.value_std, w.dtype))
    step_k, step_v, step_q = [], [], []
    for _ in range(w.steps):
        step_k.append(st.normal((w.num_seqs, Hk, D), w.kv_std, w.dtype))
        step_v.append(st.normal((w.num_seqs, Hk, D), w.value_std, w.dtype))
        step_q.append(st.normal((w.num_seqs, w.num_heads, D), w.q_std, w.dtype))
    return Draws(free_order=free_order, prefill_lens=prefill_lens, prefill_k=pk, prefill_v=pv,
                 step_k=step_k, step_v=step_v, step_q=step_q, suffix_lens=suffix_lens,
                 suffix_k=sk, suffix_v=sv)


# --- Operation scripts -------------------------------------------------------
# A script is a list of tuples naming cache-manager operations on *slots*
# (positions in the decode batch), never physical blocks:
#   ("add", slot)                      new empty sequence placed at `slot`
#   ("prefill", slot, i)               append prefill tokens i (all of them)
#   ("suffix", slot, j)                append suffix tokens j (sharing workload)
#   ("fork", dst_slot, src_slot)       dst becomes a sharer of src's blocks
#   ("free", slot)                     release the sequence at `slot`
#   ("step", t)                        append one token to every slot in order,
#                                      write step t's k/v, decode step t's q
# Both the oracle model and the library replay the same script.

def script(w: Workload, d: Draws) -> list:
    ops: list = []
    if w.length_kind != "sharing":
        for s in range(w.num_seqs):
            ops.append(("add", s))
            ops.append(("prefill", s, s))
        for t in range(w.steps):
            ops.append(("step", t))
        return ops
    # Sharing: per group a prompt sequence is prefilled, forked into the
    # group's samples and released, so the prompt blocks are held by the
    # samples only; each sample then appends its own suffix. Every step
    # first replaces odd sample 2k+1 by a fresh fork of even sample 2k (beam
    # search keeping the better of two beams), so the pair shares a
    # partially filled last block when the step's token is appended.
    G, J = w.groups, w.samples
    for g in range(G):
        prompt_slot = ("prompt", g)
        ops.append(("add", prompt_slot))
        ops.append(("prefill", prompt_slot, g))
        for j in range(J):
            ops.append(("fork", g * J + j, prompt_slot))
        ops.append(("free", prompt_slot))
    for s in range(G * J):
        ops.append(("suffix", s, s))
    for t in range(w.steps):
        for g in range(G):
            for k in range(J // 2):
                a, b = g * J + 2 * k, g * J + 2 * k + 1
                ops.append(("free", b))
                ops.append(("fork", b, a))
        ops.append(("step", t))
    return ops


def attended_at_step0(w: Workload, d: Draws) -> List[int]:
    """Attended lengths at the first decode step (for sizing workspace/pools)."""
    if w.length_kind == "sharing":
        # after the first pair fork, odd samples inherit their even partner's length
        out = []
        for s in range(w.num_seqs):
            src = s - (s % 2)
            out.append(w.prompt_len + d.suffix_lens[src] + 1)
        return out
    return [n + 1 for n in d.prefill_lens]


@dataclasses.dataclass
class PromptDraws:
    """Every random input of a prompt workload (torch tensors, CPU or device).

    prefix_k / prefix_v: [prefix_len, H_kv, D], the cached tokens before every prompt;
    prompt_k / prompt_v[s]: [n_s, H_kv, D]; q: [sum n_s, H, D], texts' rows one after another.
    """
    free_order: np.ndarray
    prompt_lens: List[int]
    prefix_k: list
    prefix_v: list
    prompt_k: list
    prompt_v: list
    q: object


def draw_prompt(w: PromptWorkload, device: Optional[str] = None) -> PromptDraws:
    """Inputs of a prompt workload: free-list permutation -> prompt lengths -> prefix K,
    prefix V -> per text: prompt K, prompt V -> the packed queries."""
    st = Stream(w.seed, device)
    free_order = st.permutation(w.num_blocks)
    lens = [int(x) for x in st.integers(w.prompt_lo, w.prompt_hi, w.num_seqs)]
    Hk, D = w.num_kv_heads, w.head_dim
    xk = st.normal((w.prefix_len, Hk, D), w.kv_std, w.dtype)
    xv = st.normal((w.prefix_len, Hk, D), w.kv_std, w.dtype)
    pk, pv = [], []
    for n in lens:
        pk.append(st.normal((n, Hk, D), w.kv_std, w.dtype))
        pv.append(st.normal((n, Hk, D), w.kv_std, w.dtype))
    q = st.normal((sum(lens), w.num_heads, D), w.q_std, w.dtype)
    return PromptDraws(free_order=free_order, prompt_lens=lens, prefix_k=xk, prefix_v=xv,
                       prompt_k=pk, prompt_v=pv, q=q)


# --- Prefix-caching workloads -------------------------------------------------
# Requests that begin with one of a few shared system prompts and go on with their own
# tokens (› "What Came After": many requests begin the same way). Token ids are drawn
# as well as keys and values, so that the block hashes of the prefix cache can be formed.

@dataclasses.dataclass(frozen=True)
class PrefixWorkload:
    name: str
    seed: int
    prompt_lens: tuple       # shared system prompts
    num_requests: int
    user_lo: int             # each request's own tokens ~ U{user_lo..user_hi}
    user_hi: int
    batch: int               # requests per prompt-phase call
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str
    kv_std: float
    q_std: float
    vocab: int = 50000
    description: str = ""

    def scaled(self, **kw) -> "PrefixWorkload":
        return dataclasses.replace(self, **kw)


PREFIX_CHAT = PrefixWorkload(
    name="prefix_chat_f16_b16", seed=21, prompt_lens=(100, 64, 37), num_requests=24,
    user_lo=5, user_hi=60, batch=6, num_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
    num_blocks=64, dtype="f16", kv_std=0.5, q_std=1.0,
    description="24 requests after one of 3 shared system prompts (100, 64, 37 tokens), "
                "5-60 own tokens each, prompt phase in batches of 6; a 64-block pool, so "
                "cached blocks are also evicted")


@dataclasses.dataclass
class PrefixDraws:
    """sys_tokens[i] (int64 numpy), sys_k / sys_v[i]: [len_i, H_kv, D]; per request r:
    req_sys[r] (its system prompt), user_tokens[r], user_k / user_v[r]: [u_r, H_kv, D],
    q[r]: [len_i + u_r, H, D] (a query for every position of the request)."""
    free_order: np.ndarray
    sys_tokens: list
    sys_k: list
    sys_v: list
    req_sys: List[int]
    user_tokens: list
    user_k: list
    user_v: list
    q: list


def draw_prefix(w: PrefixWorkload, device: Optional[str] = None) -> PrefixDraws:
    """free-list permutation -> per system prompt: tokens, K, V -> per request: its
    system prompt, own length, tokens, K, V, queries."""
    st = Stream(w.seed, device)
    free_order = st.permutation(w.num_blocks)
    Hk, D = w.num_kv_heads, w.head_dim
    sys_t, sys_k, sys_v = [], [], []
    for n in w.prompt_lens:
        sys_t.append(st.integers(0, w.vocab - 1, n))
        sys_k.append(st.normal((n, Hk, D), w.kv_std, w.dtype))
        sys_v.append(st.normal((n, Hk, D), w.kv_std, w.dtype))
    req_sys, ut, uk, uv, qs = [], [], [], [], []
    for _ in range(w.num_requests):
        i = int(st.integers(0, len(w.prompt_lens) - 1, 1)[0])
        u = int(st.integers(w.user_lo, w.user_hi, 1)[0])
        req_sys.append(i)
        ut.append(st.integers(0, w.vocab - 1, u))
        uk.append(st.normal((u, Hk, D), w.kv_std, w.dtype))
        uv.append(st.normal((u, Hk, D), w.kv_std, w.dtype))
        qs.append(st.normal((w.prompt_lens[i] + u, w.num_heads, D), w.q_std, w.dtype))
    return PrefixDraws(free_order=free_order, sys_tokens=sys_t, sys_k=sys_k, sys_v=sys_v,
                       req_sys=req_sys, user_tokens=ut, user_k=uk, user_v=uv, q=qs)


def prefix_schedule(w: PrefixWorkload) -> list:
    """Batches of `batch` consecutive requests; after a batch's prompt phase its blocks
    are registered, then the requests of the batch before it finish (are freed)."""
    ops = []
    batches = [list(range(i, min(i + w.batch, w.num_requests)))
               for i in range(0, w.num_requests, w.batch)]
    for b, reqs in enumerate(batches):
        ops.append(("batch", reqs))
        if b > 0:
            ops.append(("finish", batches[b - 1]))
    ops.append(("finish", batches[-1]))
    return ops

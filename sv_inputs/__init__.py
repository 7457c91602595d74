"""Seeded synthetic inputs for speculative-sampling verification.

This module is shared by the oracle side and the HIP side of every test and of
the benchmark.  It holds random-number generation only: Gaussian logits, bf16
rounding, peaked tokens, draft tokens drawn from the draft distribution, and the
verification uniforms.  None of the verification arithmetic (softmax
normalisers, acceptance test, residual, inverse CDF, top-k) lives here.

Random streams: numpy's Philox counter-based generator (Salmon et al., SC'11,
the 4x64-10 variant numpy ships), keyed per (seed, tensor, row) so that any row
can be regenerated on its own.

Draft tokens are drawn with the Gumbel-max trick: argmax_x (d_x / T + G_x) with
G_x = -log(-log U_x) is an exact sample from softmax(d / T).  That keeps the
generator free of any normaliser or cumulative sum.  With T == 0 the draft token
is the argmax of the draft row (lowest index on ties).

Workloads follow the five configurations the verification step is measured on:
  tiny      B=2,  k=3,  V=1000,   fp32, t~N(0,2^2), d=t+N(0,0.5^2), T=1
  steady    B=32, k=3,  V=151936, bf16, t~N(0,3^2) +8 on 20 distinct tokens
            per row, d=t+N(0,1^2), T=1
  longtail  B in {1,2,4}, k=8, V=151936, bf16, t~N(0,2^2), d=t+N(0,0.6^2), T=1
  grpo      B=256 (32 prompts x 8 rollouts), k=3, V=128256, bf16,
            t~N(0,3^2), d=t+N(0,1.5^2), T=0.7; target and draft row 0 are
            shared by the 8 rollouts of a prompt
  wide      B=32, k=15, V=151936, fp32, t~N(0,3^2), d=t+N(0,2^2), T=1
            (and T=0 greedy with draft tokens = argmax of the draft row)
  plain     B=32, k=0, V=151936, bf16, as steady: one token sampled per sequence
and the distillation batches (kd_workload, kd_small, kd_rollout) below.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# tensor ids of the Philox key
_T_TARGET, _T_DRAFT_NOISE, _T_PEAKS, _T_DRAFT_TOK, _T_UNIFORM = 0, 1, 2, 3, 4
_PROMPT_ROW = 1 << 40  # key offset marking a row shared by a prompt group

F32, BF16 = 0, 1
DTYPE_NAME = {F32: "f32", BF16: "bf16"}


def _rng(seed: int, tensor: int, row: int) -> np.random.Generator:
    # Philox key is two 64-bit words: (seed, tensor << 48 | row)
    return np.random.Generator(np.random.Philox(key=[int(seed), (int(tensor) << 48) | int(row)]))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    k: int
    V: int
    dtype: int             # F32 or BF16
    temperature: float
    target: np.ndarray     # [B,k+1,V] float32, or uint16 bf16 patterns
    draft: np.ndarray      # [B,k,V]   same storage as target
    draft_tokens: np.ndarray  # [B,k] int32
    uniforms: np.ndarray   # [B,k+2] float32 in [0,1)
    seed: int = 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def target_f32(self) -> np.ndarray:
        return self.target if self.dtype == F32 else bf16_to_f32(self.target)

    def draft_f32(self) -> np.ndarray:
        return self.draft if self.dtype == F32 else bf16_to_f32(self.draft)

    def alg_bytes(self) -> int:
        """Logit bytes the step must read once: B(2k+1)V e when sampling,
        B(k+1)V e when greedy."""
        rows = self.B * (self.k + 1) + (self.B * self.k if self.temperature > 0 else 0)
        return rows * self.V * self.elem_bytes

    def subset(self, bs) -> "Workload":
        bs = np.asarray(bs)
        return dataclasses.replace(
            self, B=len(bs), target=np.ascontiguousarray(self.target[bs]),
            draft=np.ascontiguousarray(self.draft[bs]),
            draft_tokens=np.ascontiguousarray(self.draft_tokens[bs]),
            uniforms=np.ascontiguousarray(self.uniforms[bs]))


def _uniform24(rng: np.random.Generator, n) -> np.ndarray:
    """Uniforms on the 2^-24 grid in [0,1), exact in float32."""
    x = rng.integers(0, 1 << 24, size=n, dtype=np.uint32)
    return (x.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_max_token(rng: np.random.Generator, d_row: np.ndarray, T: float) -> int:
    """One exact draw from softmax(d_row / T) by the Gumbel-max trick (T > 0),
    or argmax(d_row) with lowest-index ties (T == 0)."""
    d = np.asarray(d_row, dtype=np.float64)
    if T == 0:
        return int(np.argmax(d))
    u = rng.random(d.shape[0]) + 2.0 ** -54          # in (0,1)
    g = -np.log(-np.log(u))
    return int(np.argmax(d / T + g))


def make_workload(name: str, B: int, k: int, V: int, dtype: int, T: float, seed: int,
                  sigma_t: float, sigma_d: float, peaks: int = 0, peak_boost: float = 0.0,
                  group: int = 0, draft_T: Optional[float] = None) -> Workload:
    """Rows are generated one by one from keyed Philox streams.

    group > 0: sequences come in groups of `group` rollouts of one prompt and row
    0 of target and draft is drawn from the prompt's stream (shared in the group).
    draft_T: temperature the draft tokens are drawn at (defaults to T; 0 = argmax).
    """
    dT = T if draft_T is None else draft_T
    K1 = k + 1
    store = np.float32 if dtype == F32 else np.uint16
    target = np.empty((B, K1, V), dtype=store)
    draft = np.empty((B, k, V), dtype=store)
    tokens = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(K1):
            if group and i == 0:
                rk = _PROMPT_ROW + (b // group)
            else:
                rk = b * K1 + i
            t = (_rng(seed, _T_TARGET, rk).standard_normal(V) * sigma_t).astype(np.float32)
            if peaks:
                idx = _rng(seed, _T_PEAKS, rk).choice(V, size=peaks, replace=False)
                t[idx] += np.float32(peak_boost)
            if i < k:
                n = (_rng(seed, _T_DRAFT_NOISE, rk).standard_normal(V) * sigma_d).astype(np.float32)
                d = t + n      # formed in fp32 before any rounding
            if dtype == BF16:
                target[b, i] = bf16_round(t)
                if i < k:
                    draft[b, i] = bf16_round(d)
            else:
                target[b, i] = t
                if i < k:
                    draft[b, i] = d
            if i < k:
                d_seen = draft[b, i] if dtype == F32 else bf16_to_f32(draft[b, i])
                tokens[b, i] = gumbel_max_token(_rng(seed, _T_DRAFT_TOK, b * K1 + i), d_seen, dT)
    uniforms = np.stack([_uniform24(_rng(seed, _T_UNIFORM, b), K1 + 1) for b in range(B)]) \
        if B else np.zeros((0, K1 + 1), np.float32)
    return Workload(name, B, k, V, dtype, float(T), target, draft, tokens, uniforms, seed)


# The five workloads (seed = 1000 + workload number; long-tail adds B).
def tiny(seed: int = 1001, B: int = 2, k: int = 3, V: int = 1000) -> Workload:
    return make_workload("tiny", B, k, V, F32, 1.0, seed, 2.0, 0.5)


def steady(seed: int = 1002, B: int = 32, k: int = 3, V: int = 151936) -> Workload:
    return make_workload("steady", B, k, V, BF16, 1.0, seed, 3.0, 1.0, peaks=20, peak_boost=8.0)


def longtail(B: int = 1, seed: Optional[int] = None, k: int = 8, V: int = 151936) -> Workload:
    return make_workload("longtail", B, k, V, BF16, 1.0, 1003 + B if seed is None else seed, 2.0, 0.6)


def grpo(seed: int = 1004, prompts: int = 32, rollouts: int = 8, k: int = 3, V: int = 128256) -> Workload:
    return make_workload("grpo", prompts * rollouts, k, V, BF16, 0.7, seed, 3.0, 1.5, group=rollouts)


def wide(seed: int = 1005, B: int = 32, k: int = 15, V: int = 151936, greedy: bool = False) -> Workload:
    if greedy:
        return make_workload("wide_greedy", B, k, V, F32, 0.0, seed, 3.0, 2.0, draft_T=0.0)
    return make_workload("wide", B, k, V, F32, 1.0, seed, 3.0, 2.0)


def fixed_rows(B: int, target_rows: np.ndarray, draft_rows: np.ndarray, T: float, seed: int,
               dtype: int = F32) -> Workload:
    """B independent sequences that all share the same fixed logits (for
    distribution tests at tiny V): target_rows [k+1,V], draft_rows [k,V] float32.
    Draft tokens are drawn per sequence and position from softmax(draft/T) by
    Gumbel-max, vectorised over sequences."""
    target_rows = np.asarray(target_rows, np.float32)
    draft_rows = np.asarray(draft_rows, np.float32)
    K1, V = target_rows.shape
    k = K1 - 1
    rng = _rng(seed, _T_DRAFT_TOK, 0)
    if dtype == BF16:
        tr, dr = bf16_round(target_rows), bf16_round(draft_rows)
        d_seen = bf16_to_f32(dr).astype(np.float64)
    else:
        tr, dr = target_rows, draft_rows
        d_seen = draft_rows.astype(np.float64)
    tokens = np.empty((B, k), np.int32)
    for i in range(k):
        if T == 0:
            tokens[:, i] = int(np.argmax(d_seen[i]))
            continue
        u = rng.random((B, V)) + 2.0 ** -54
        g = -np.log(-np.log(u))
        tokens[:, i] = np.argmax(d_seen[i][None, :] / T + g, axis=1)
    target = np.broadcast_to(tr, (B, K1, V)).copy()
    draft = np.broadcast_to(dr, (B, k, V)).copy()
    uniforms = _uniform24(_rng(seed, _T_UNIFORM, 0), (B, K1 + 1))
    return Workload("fixed", B, k, V, dtype, float(T), target, draft, tokens, uniforms, seed)


# ---------------------------------------------------------------- distillation
# Inputs of the reward-weighted drafter distillation over stored top-32 soft
# targets.  Rows are stored positions of rollout samples (L positions per
# sample, samples in groups of `group` rollouts of one prompt).  Per row: 32
# distinct token ids with stored target logits ~ N(10, 2^2) (bf16-representable
# values), and drafter logits ~ N(0, 3^2) except at the stored ids, where they
# are the stored value plus N(0, 1.5^2).  Rewards take the levels of the pages'
# GRPO example, {0, 0.3, 0.8, 1.0}, uniformly.
_T_KD_LOGITS, _T_KD_IDS, _T_KD_VALS, _T_KD_NOISE, _T_KD_REWARD = 10, 11, 12, 13, 14
KD_TOP = 32


@dataclasses.dataclass
class KDWorkload:
    name: str
    N: int
    V: int
    dtype: int             # of the drafter logits
    group: int
    L: int                 # stored positions per sample
    logits: np.ndarray     # [N,V] float32, or uint16 bf16 patterns
    topk_val: np.ndarray   # [N,32] float32
    topk_idx: np.ndarray   # [N,32] int32
    row_sample: np.ndarray  # [N] int32
    rewards: np.ndarray    # [S] float32
    w_max: float = float("inf")
    seed: int = 0

    @property
    def S(self) -> int:
        return int(self.rewards.size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def alg_bytes(self, grad_bytes: int = 0) -> int:
        """Drafter logit bytes read once, plus the gradient written once."""
        return self.N * self.V * (self.elem_bytes + grad_bytes)


def kd_workload(name: str, samples: int, group: int, L: int, V: int, dtype: int, seed: int,
                w_max: float = float("inf")) -> KDWorkload:
    N = samples * L
    store = np.float32 if dtype == F32 else np.uint16
    logits = np.empty((N, V), dtype=store)
    tv = np.empty((N, KD_TOP), np.float32)
    ti = np.empty((N, KD_TOP), np.int32)
    for n in range(N):
        ids = _rng(seed, _T_KD_IDS, n).choice(V, size=min(KD_TOP, V), replace=False).astype(np.int32)
        vals = bf16_to_f32(bf16_round(_rng(seed, _T_KD_VALS, n).standard_normal(ids.size).astype(np.float32) * 2 + 10))
        z = (_rng(seed, _T_KD_LOGITS, n).standard_normal(V) * 3.0).astype(np.float32)
        z[ids] = vals + (_rng(seed, _T_KD_NOISE, n).standard_normal(ids.size) * 1.5).astype(np.float32)
        logits[n] = z if dtype == F32 else bf16_round(z)
        tv[n] = -np.inf
        ti[n] = -1
        tv[n, :ids.size] = vals
        ti[n, :ids.size] = ids
    levels = np.array([0.0, 0.3, 0.8, 1.0], np.float32)
    rewards = levels[_rng(seed, _T_KD_REWARD, 0).integers(0, 4, size=samples)]
    row_sample = (np.arange(N) // L).astype(np.int32)
    return KDWorkload(name, N, V, dtype, group, L, logits, tv, ti, row_sample, rewards, float(w_max), seed)


def plain(seed: int = 1007, B: int = 32, V: int = 151936) -> Workload:
    """k = 0: plain temperature sampling of one token per sequence (the engine's
    non-speculative step), steady-state logits."""
    return make_workload("plain", B, 0, V, BF16, 1.0, seed, 3.0, 1.0, peaks=20, peak_boost=8.0)


def kd_small(seed: int = 1101, V: int = 20000, dtype: int = BF16) -> KDWorkload:
    """3 groups of 4 samples, 2 positions each: 24 rows, a ragged last tile."""
    return kd_workload("kd_small", 12, 4, 2, V, dtype, seed)


def kd_rollout(seed: int = 1106, prompts: int = 32, rollouts: int = 8, L: int = 16, V: int = 151936) -> KDWorkload:
    """The distillation batch of one GRPO step: 32 prompts x 8 rollouts, 16
    stored positions each (4096 rows), V = 151936, bf16 drafter logits."""
    return kd_workload("kd_rollout", prompts * rollouts, rollouts, L, V, BF16, seed)

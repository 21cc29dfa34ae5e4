"""Seeded synthetic inputs for the verify step and the E2E-TV loss.

This module is shared by the tests, the benchmark and the CPU oracle's
callers. It holds none of the method's arithmetic: it only draws logits,
draft tokens and target probabilities of the shapes and value distributions
of the five workloads below, and stores them in the workload's dtype.

The pages measure on model logits over public suites and live traffic; these
generators stand in for them (no suite item is reproduced or needed).

Every row is drawn from its own stream, ``numpy.random.default_rng([case, b,
k, role])`` with role 0 = target noise, 1 = draft noise, 2 = draft-token
draw, so any row can be rebuilt in isolation. Per-workload draws (the Zipf
permutation, ragged K, seeds) use ``default_rng([case, 99])``,
``default_rng([case, 98])`` and ``default_rng([case, 97])``.

Workloads (numbers are the defaults; tests shrink B, K and V):

1. B=1, K=4, V=4096, fp32. target ~ N(0, 2^2); draft = target + N(0, 0.5^2);
   draft tokens sampled from q at T=1; Philox seed 0; run at T=1 and at T=0 on
   the same tensors.
2. B=32, K=4, V=32000, bf16. target ~ N(0, 3^2) plus +8 on 1% of entries
   (peaked rows); draft = target + N(0, 1); T=1; seed 0.
3. B=64, K=7, V=151936, bf16, Zipf prior: target = -1.1 ln(rank(v)) + N(0,1)
   with one random rank permutation per workload; draft noise sigma
   (0.3, 1.0, 2.0)[b mod 3]; T in {0, 0.6, 1.0}, draft tokens drawn at that T.
4. Loss: N=512 branches, W=7, V=151936. Target logits from the workload-3
   Zipf generator; target probabilities = fp32 of their fp64 softmax;
   draft logits = bf16(target + N(0, sigma_n^2)), sigma_n = (0.3, 1, 2)[n mod 3].
   With the target given as logits, the same target rows are stored as bf16
   instead of probabilities.
5. B=256, K_b ~ U{1..8}, Kmax=8, padded layout, V=129280, bf16 Zipf, sigma_b as
   in 3; T_b = 0 for even b and 1.0 for odd b; per-request uint64 seeds.

Draft tokens are drawn from the stored draft row: Gumbel-max,
argmax(d / T + G), at T > 0 and argmax(d) at T = 0. Padding rows of the
padded layout (target rows k > K_b, draft rows k >= K_b) are filled with NaN
and padding tokens with -1, so that a kernel reading them shows up.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ZIPF_SLOPE = 1.1
SIGMAS = (0.3, 1.0, 2.0)
BF16_NAN = np.uint16(0x7FC0)


def to_bf16(x32):
    """float32 -> uint16 bfloat16 patterns, round to nearest even (storage)."""
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def from_bf16(u16):
    """uint16 bfloat16 patterns -> float32 (exact)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*words):
    return np.random.default_rng(list(words))


def zipf_prior(case, vocab):
    """-1.1 ln(rank(v)), rank = 1 + pi(v) for one permutation per workload."""
    perm = _rng(case, 99).permutation(vocab)
    return (-ZIPF_SLOPE * np.log1p(perm.astype(np.float64))).astype(np.float32)


@dataclass
class VerifyCase:
    case: int
    dtype: str                 # "f32" or "bf16"
    target: np.ndarray         # [B, Kmax+1, V] float32 or uint16
    draft: np.ndarray          # [B, Kmax, V]
    tokens: np.ndarray         # int32 [B, Kmax]
    k: np.ndarray              # int32 [B]
    temperature: np.ndarray    # float32 [B]
    seed: np.ndarray           # uint64 [B]
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.target.shape[0], self.draft.shape[1], self.target.shape[2]


def _store(x32, dtype):
    return x32.astype(np.float32) if dtype == "f32" else to_bf16(x32)


def _decode(stored, dtype):
    return stored if dtype == "f32" else from_bf16(stored)


def _draw_token(case, b, k, d_stored, dtype, temperature):
    d = _decode(d_stored, dtype).astype(np.float64)
    if temperature == 0.0:
        return int(np.argmax(d))
    u = _rng(case, b, k, 2).random(d.shape[0])
    gumbel = -np.log(-np.log(np.maximum(u, np.finfo(np.float64).tiny)))
    return int(np.argmax(d / float(np.float32(temperature)) + gumbel))


def _target_row(case, b, k, vocab, kind, prior):
    rng = _rng(case, b, k, 0)
    if kind == "gauss2":
        return (2.0 * rng.standard_normal(vocab, dtype=np.float32)).astype(np.float32)
    if kind == "gauss3_boost":
        x = 3.0 * rng.standard_normal(vocab, dtype=np.float32)
        x += np.float32(8.0) * (rng.random(vocab, dtype=np.float32) < 0.01)
        return x.astype(np.float32)
    return (prior + rng.standard_normal(vocab, dtype=np.float32)).astype(np.float32)


def _draft_row(case, b, k, vocab, t32, sigma):
    noise = _rng(case, b, k, 1).standard_normal(vocab, dtype=np.float32)
    return (t32 + np.float32(sigma) * noise).astype(np.float32)


def verify_case(case, temperature=None, batch=None, kmax=None, vocab=None,
                k_values=None, draw_temperature=None):
    """Build the inputs of verify workload ``case`` (1, 2, 3 or 5).

    ``temperature`` overrides the per-request temperature (workloads 1 and
    3 take it from their sweep); ``draw_temperature`` the temperature the
    draft tokens are drawn at (defaults to the run temperature, except
    workload 1, which draws at T=1 for both its runs). ``k_values`` forces
    per-request K (ragged tests).
    """
    spec = {
        1: dict(B=1, K=4, V=4096, dtype="f32", kind="gauss2", sig=(0.5,)),
        2: dict(B=32, K=4, V=32000, dtype="bf16", kind="gauss3_boost", sig=(1.0,)),
        3: dict(B=64, K=7, V=151936, dtype="bf16", kind="zipf", sig=SIGMAS),
        5: dict(B=256, K=8, V=129280, dtype="bf16", kind="zipf", sig=SIGMAS),
    }[case]
    B = spec["B"] if batch is None else batch
    K = spec["K"] if kmax is None else kmax
    V = spec["V"] if vocab is None else vocab
    dtype = spec["dtype"]
    prior = zipf_prior(case, V) if spec["kind"] == "zipf" else None

    if k_values is not None:
        kb = np.asarray(k_values, dtype=np.int32)
    elif case == 5:
        kb = _rng(case, 98).integers(1, K + 1, size=B).astype(np.int32)
    else:
        kb = np.full(B, K, dtype=np.int32)

    if case == 5:
        temps = np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)
        seeds = _rng(case, 97).integers(0, 2**64, size=B, dtype=np.uint64)
    else:
        t_run = 1.0 if temperature is None else temperature
        temps = np.full(B, t_run, dtype=np.float32)
        seeds = np.zeros(B, dtype=np.uint64)
    if temperature is not None:
        temps = np.full(B, temperature, dtype=np.float32)

    if dtype == "f32":
        target = np.full((B, K + 1, V), np.nan, dtype=np.float32)
        draft = np.full((B, K, V), np.nan, dtype=np.float32)
    else:
        target = np.full((B, K + 1, V), BF16_NAN, dtype=np.uint16)
        draft = np.full((B, K, V), BF16_NAN, dtype=np.uint16)
    tokens = np.full((B, K), -1, dtype=np.int32)

    for b in range(B):
        sigma = spec["sig"][b % len(spec["sig"])]
        if draw_temperature is not None:
            t_draw = draw_temperature
        elif case == 1:
            t_draw = 1.0
        else:
            t_draw = float(temps[b])
        for k in range(int(kb[b]) + 1):
            t32 = _target_row(case, b, k, V, spec["kind"], prior)
            target[b, k] = _store(t32, dtype)
            if k < kb[b]:
                draft[b, k] = _store(_draft_row(case, b, k, V, t32, sigma), dtype)
                tokens[b, k] = _draw_token(case, b, k, draft[b, k], dtype, t_draw)
    return VerifyCase(case, dtype, target, draft, tokens, kb, temps, seeds,
                      meta={"B": B, "Kmax": K, "V": V})


def redraw_tokens(case: VerifyCase, temperature: float) -> VerifyCase:
    """Same logits, draft tokens drawn at another temperature, and that
    temperature for every request (workload 3 sweeps T over one set of
    logits)."""
    tokens = np.full_like(case.tokens, -1)
    for b in range(case.tokens.shape[0]):
        for k in range(int(case.k[b])):
            tokens[b, k] = _draw_token(case.case, b, k, case.draft[b, k], case.dtype,
                                       temperature)
    temps = np.full_like(case.temperature, temperature)
    return VerifyCase(case.case, case.dtype, case.target, case.draft, tokens, case.k, temps,
                      case.seed, meta=dict(case.meta))


@dataclass
class LossCase:
    draft_logits: np.ndarray   # uint16 bf16 [N, W, V]
    target_probs: np.ndarray   # float32 [N, W, V]
    meta: dict = field(default_factory=dict)


def loss_branch(n, width, vocab, prior, case=4):
    """Rows of branch ``n``: (bf16 draft logits [W, V], fp32 probs [W, V])."""
    z = np.empty((width, vocab), dtype=np.uint16)
    p = np.empty((width, vocab), dtype=np.float32)
    sigma = SIGMAS[n % len(SIGMAS)]
    for k in range(width):
        t32 = _target_row(case, n, k, vocab, "zipf", prior)
        t64 = t32.astype(np.float64)
        e = np.exp(t64 - t64.max())
        p[k] = (e / e.sum()).astype(np.float32)
        z[k] = to_bf16(_draft_row(case, n, k, vocab, t32, sigma))
    return z, p


def loss_case(n_branches=512, width=7, vocab=151936, case=4, workers=1):
    """Build the inputs of the loss workload (defaults: workload 4)."""
    prior = zipf_prior(case, vocab)
    z = np.empty((n_branches, width, vocab), dtype=np.uint16)
    p = np.empty((n_branches, width, vocab), dtype=np.float32)
    if workers > 1 and n_branches > 1:
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(max_workers=workers) as pool:
            futs = {n: pool.submit(loss_branch, n, width, vocab, prior, case)
                    for n in range(n_branches)}
            for n, f in futs.items():
                z[n], p[n] = f.result()
    else:
        for n in range(n_branches):
            z[n], p[n] = loss_branch(n, width, vocab, prior, case)
    return LossCase(z, p, meta={"N": n_branches, "W": width, "V": vocab})


@dataclass
class LossLogitsCase:
    draft_logits: np.ndarray   # uint16 bf16 [N, W, V]
    target_logits: np.ndarray  # uint16 bf16 [N, W, V]
    meta: dict = field(default_factory=dict)


def loss_logits_branch(n, width, vocab, prior, case=4):
    """Rows of branch ``n`` with the target as logits: (bf16 draft logits
    [W, V], bf16 target logits [W, V]); the same rows as ``loss_branch``,
    the target stored in bf16 instead of as probabilities."""
    z = np.empty((width, vocab), dtype=np.uint16)
    t = np.empty((width, vocab), dtype=np.uint16)
    sigma = SIGMAS[n % len(SIGMAS)]
    for k in range(width):
        t32 = _target_row(case, n, k, vocab, "zipf", prior)
        t[k] = to_bf16(t32)
        z[k] = to_bf16(_draft_row(case, n, k, vocab, t32, sigma))
    return z, t


def loss_logits_case(n_branches=512, width=7, vocab=151936, case=4, workers=1):
    """The loss workload with the target given as bf16 logits (the
    temperature is a call argument, not part of the inputs)."""
    prior = zipf_prior(case, vocab)
    z = np.empty((n_branches, width, vocab), dtype=np.uint16)
    t = np.empty((n_branches, width, vocab), dtype=np.uint16)
    if workers > 1 and n_branches > 1:
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(max_workers=workers) as pool:
            futs = {n: pool.submit(loss_logits_branch, n, width, vocab, prior, case)
                    for n in range(n_branches)}
            for n, f in futs.items():
                z[n], t[n] = f.result()
    else:
        for n in range(n_branches):
            z[n], t[n] = loss_logits_branch(n, width, vocab, prior, case)
    return LossLogitsCase(z, t, meta={"N": n_branches, "W": width, "V": vocab})

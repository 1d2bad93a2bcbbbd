"""Per-step schedule of KV-cached MAR decoding (integer logic only).

TEST INFRASTRUCTURE ONLY: the independent reference for the GPU library's
``mar_plan_step`` / ``mar_layer_kind`` host functions.

Rules, from the method pages:
  * A periodic full refresh runs on every step with ``step % period == 0``
    (period 3), which includes the initial step; on such a step every layer
    runs full attention and rewrites its whole KV cache ("MARche" paper-notes
    page, Method flowchart and Key Design 3).
  * On the other steps layers 1 and 2 still run full attention, layer 2 picks
    the refreshing tokens, and layers 3.. run cache-aware attention over the
    active set (same page, Overall Architecture and Key Designs 1-2).
  * The active set is this step's generating tokens G, the previous step's
    (caching) tokens P and K refreshing tokens, inside a fixed total budget,
    so K = budget - |G| - |P| (same page, Key Design 1: a fixed active budget
    shared by the three groups).
  * LazyMAR's token gate applies only to layers after the first three and its
    condition cache re-stores the residual on every fully computed step
    ("LazyMAR" paper-notes page, Key designs and the cache-reuse-refresh policy).

Generation order: step t generates the tokens order[o_t : o_t + n_t] where
o_t = n_0 + ... + n_{t-1}; the previous step's tokens are
order[o_{t-1} : o_t].  So P followed by G is the contiguous slice
order[o_{t-1} : o_t + n_t].
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

FULL = "full"
CACHE = "cache"


@dataclass(frozen=True)
class StepPlan:
    step: int
    refresh: bool
    gen_begin: int
    n_gen: int
    prev_begin: int
    n_prev: int
    n_refresh: int  # K
    n_active: int   # |G| + |P| + K on cache steps; N on refresh steps
    n_cached: int


def is_refresh(step: int, period: int = 3, warmup: int = 0) -> bool:
    return step < warmup or step % period == 0


def plan_step(counts: Sequence[int], step: int, n_tokens: int, budget: int,
              period: int = 3, warmup: int = 0) -> StepPlan:
    if not 0 <= step < len(counts):
        raise ValueError("step out of range")
    gen_begin = 0
    for s in range(step):
        gen_begin += int(counts[s])
    n_gen = int(counts[step])
    n_prev = int(counts[step - 1]) if step > 0 else 0
    prev_begin = gen_begin - n_prev
    if is_refresh(step, period, warmup):
        return StepPlan(step, True, gen_begin, n_gen, prev_begin, n_prev, 0, n_tokens, 0)
    k = budget - n_gen - n_prev
    if k < 0:
        k = 0
    room = n_tokens - n_gen - n_prev
    if k > room:
        k = room
    a = n_gen + n_prev + k
    return StepPlan(step, False, gen_begin, n_gen, prev_begin, n_prev, k, a, n_tokens - a)


def layer_kind(plan: StepPlan, layer: int, n_full_layers: int = 2) -> str:
    """layer is 1-based."""
    if plan.refresh or layer <= n_full_layers:
        return FULL
    return CACHE


def selects_refresh(plan: StepPlan, layer: int, select_layer: int = 2) -> bool:
    return (not plan.refresh) and layer == select_layer


def gate_applies(plan: StepPlan, layer: int, ungated_layers: int = 3) -> bool:
    return (not plan.refresh) and layer > ungated_layers


def cfg_mode(plan: StepPlan) -> str:
    return "store" if plan.refresh else "reuse"

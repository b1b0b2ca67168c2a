"""Dynamic loss scaling of fp16 training (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and the benchmark's cpu_baseline leg may
import this module; the product path never does.

The LucilleAI page lists a GradScaler next to the trainer and AdamW, and an
optional feature of FP16 autocast plus GradScaler; it prints no constants or
rule. The reading followed here is the usual dynamic scaler:
  * the loss gradient is multiplied by the scale S before the backward, so
    every gradient holds S times its value; the clip and the update use the
    gradients divided by S;
  * a step whose gradients are not all finite is skipped (parameters and
    Adam moments unchanged), S is multiplied by `backoff` and the run of
    finite steps restarts at 0;
  * after each finite step the run grows by one; when it reaches `interval`,
    S is multiplied by `growth` and the run restarts at 0;
  * defaults S = 2^16, growth 2, backoff 0.5, interval 2000.
In exact arithmetic, and in floating point whenever nothing over- or
underflows, S cancels out: a power of two scales every value exactly, so the
training step itself is the plain one of model.train_step.
"""
from __future__ import annotations

from typing import Iterable, List, Tuple


def loss_scale_update(scale: float, good_steps: int, finite: bool, growth: float = 2.0, backoff: float = 0.5,
                      interval: int = 2000) -> Tuple[float, int]:
    """One step of the rule above: (S, run) after a step whose gradients were
    finite or not."""
    if not finite:
        return scale * backoff, 0
    good_steps += 1
    if good_steps >= interval:
        return scale * growth, 0
    return scale, good_steps


def loss_scale_trace(scale: float, finite_flags: Iterable[bool], growth: float = 2.0, backoff: float = 0.5,
                     interval: int = 2000, good_steps: int = 0) -> List[Tuple[float, int]]:
    """(S, run) after each step of a sequence of finite / non-finite steps."""
    out = []
    for f in finite_flags:
        scale, good_steps = loss_scale_update(scale, good_steps, bool(f), growth, backoff, interval)
        out.append((scale, good_steps))
    return out

"""Learning-rate schedule of the multi-step driver (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and the benchmark's cpu_baseline leg may
import this module; the product path never does.

The LucilleAI page's trainer usage names a cosine scheduler with warm-up steps
and a minimum learning rate, but prints no formula. The reading followed here
(stated once, evaluated in float64):
  * steps are 1-based; a step below 1 counts as step 1;
  * warm-up: lr = lr_max * step / warmup_steps for step <= warmup_steps;
  * decay: with progress p = (step - warmup_steps) / (total_steps - warmup_steps),
    lr = lr_min + (lr_max - lr_min) * (1 + cos(pi * p)) / 2, down to lr_min at
    total_steps and lr_min after it;
  * no decay phase when total_steps <= warmup_steps: lr_max after the warm-up.
"""
from __future__ import annotations

import math


def lr_schedule(step: int, warmup_steps: int, total_steps: int, lr_max: float, lr_min: float) -> float:
    s = max(int(step), 1)
    if warmup_steps > 0 and s <= warmup_steps:
        return lr_max * s / warmup_steps
    if total_steps <= warmup_steps or total_steps <= 0:
        return float(lr_max)
    if s >= total_steps:
        return float(lr_min)
    progress = (s - warmup_steps) / (total_steps - warmup_steps)
    return lr_min + (lr_max - lr_min) * 0.5 * (1.0 + math.cos(math.pi * progress))

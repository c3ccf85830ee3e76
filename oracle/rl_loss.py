"""fp64 CPU oracle for the per-token RL objective fed by the selected logp.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product path never does, and this module shares no code with it.

The pages say what the selected log-probability is for: it enters the
importance ratio, the clipping and the KL terms of PPO / GRPO ("vLLM
RL-Kernel v0.1.0: Bitwise Train-Rollout Consistency on ROCm", opening
section; "Announcing RL-Kernel for vime", section "Vision": PPO, GRPO and
related algorithms only need log probabilities for selected tokens), and
the k3 KL estimator is named as one of the per-token quantities compared
between rollout and training (the GB200 write-up on train-inference
consistency).  They print no formulas; the readings taken are the standard
ones:

    r_t    = exp(logp_t - logp_old_t)                       importance ratio
    c_t    = min(max(r_t, 1 - eps_low), 1 + eps_high)       clipped ratio
    Lclip  = -min(r_t A_t, c_t A_t)                         clipped surrogate
    d_t    = logp_ref_t - logp_t
    KL_t   = exp(d_t) - d_t - 1                             k3 estimator
    L_t    = scale * (Lclip + beta KL_t)
    g_t    = dL_t / dlogp_t
           = scale * ( (-r_t A_t if r_t A_t <= c_t A_t else 0) + beta (1 - exp(d_t)) )

(the clipped branch has zero derivative: where it is the smaller term, r
lies outside the clip range and c is constant).  Rows whose target is
ignore_index have L = g = 0.  The branch is decided on the comparison
r_t A_t <= c_t A_t; within a few ulps of the clip boundaries the GPU (fp32)
and this oracle (fp64) may decide differently, and both answers are valid.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


def token_loss(logp, logp_old, adv, y, eps_low, eps_high, beta=0.0, logp_ref=None, scale=1.0,
               ignore_index=IGNORE_INDEX):
    """Per-token loss and its derivative with respect to logp (float64 [T] each)."""
    logp = np.asarray(logp, dtype=np.float64)
    logp_old = np.asarray(logp_old, dtype=np.float64)
    adv = np.asarray(adv, dtype=np.float64)
    active = np.asarray(y) != ignore_index
    r = np.exp(logp - logp_old)
    c = np.minimum(np.maximum(r, 1.0 - eps_low), 1.0 + eps_high)
    unclipped = r * adv <= c * adv
    loss = -np.minimum(r * adv, c * adv)
    g = np.where(unclipped, -r * adv, 0.0)
    if beta != 0.0:
        if logp_ref is None:
            raise ValueError("beta != 0 needs logp_ref")
        d = np.asarray(logp_ref, dtype=np.float64) - logp
        loss = loss + beta * (np.exp(d) - d - 1.0)
        g = g + beta * (1.0 - np.exp(d))
    loss = np.where(active, scale * loss, 0.0)
    g = np.where(active, scale * g, 0.0)
    return loss, g

"""torch custom ops over the C ABI, with fake (meta) kernels.

``gdn::scan`` and ``gdn::recurrent_step`` let torch.export / torch.compile /
opcheck trace the recurrence.  Their fake kernels state the output contract of
the "gated_delta" page (gated_delta_fake): y is float32 for every operand dtype
(the recurrence runs against a float32 state, so the output is widened to it);
final_state is float32 [B, Hv, D, D].  The real kernels are the HIP
library's, called through ``linear_attention_recurrence_recurrent_amd.scan`` /
``recurrent_step`` (argument marshalling only).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import recurrent_step as _recurrent_step
from . import scan as _scan

__all__ = ["scan_op", "recurrent_step_op"]


@torch.library.custom_op("gdn::scan", mutates_args=())
def scan_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
            beta: torch.Tensor, s0: torch.Tensor, z: Optional[torch.Tensor] = None,
            w: Optional[torch.Tensor] = None, head_major: bool = False
            ) -> Tuple[torch.Tensor, torch.Tensor]:
    y, s = _scan(q, k, v, log_decay, beta, s0, z, w, head_major=head_major)
    return y, s


@scan_op.register_fake
def _scan_fake(q, k, v, log_decay, beta, s0, z=None, w=None, head_major=False):
    # y is float32 in v's layout; the final state is float32 like s0.
    return (torch.empty(v.shape, dtype=torch.float32, device=v.device),
            torch.empty(s0.shape, dtype=torch.float32, device=s0.device))


@torch.library.custom_op("gdn::recurrent_step", mutates_args=())
def recurrent_step_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
                      beta: torch.Tensor, s0: torch.Tensor, z: Optional[torch.Tensor] = None,
                      w: Optional[torch.Tensor] = None, head_major: bool = False
                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    y, s = _recurrent_step(q, k, v, log_decay, beta, s0, z, w, head_major=head_major)
    return y, s


@recurrent_step_op.register_fake
def _step_fake(q, k, v, log_decay, beta, s0, z=None, w=None, head_major=False):
    return (torch.empty(v.shape, dtype=torch.float32, device=v.device),
            torch.empty(s0.shape, dtype=torch.float32, device=s0.device))

"""The bitmask API of XGrammar's "Bitmask Operations" page, on this library.

Drop-in names and signatures for callers written against that page:

* ``bitmask_dtype`` -- int32 (the page keeps int32 because old PyTorch had
  no uint32; words are read as uint32).
* ``get_bitmask_shape(batch_size, vocab_size)`` -- (batch_size, ceil(vocab_size / 32)).
* ``allocate_token_bitmask(batch_size, vocab_size)`` -- a CPU int32 tensor of
  that shape holding the full mask (every token allowed).  The page only
  says the tensor is allocated; starting from the full mask, the state
  ``reset_token_bitmask`` restores, is the reading taken here.
* ``reset_token_bitmask(bitmask)`` -- back to the full mask (all bits set).
* ``apply_token_bitmask_inplace(logits, bitmask, *, vocab_size=None, indices=None)``
  -- masked logits become -inf.  Both tensors on the GPU: the HIP kernels;
  both on the CPU: the library's native host implementation (Notes:
  Device).  Mixed devices raise: the page leaves copying the bitmask to the
  GPU to the caller.
"""

from __future__ import annotations

import math
from typing import List, Optional, Tuple

import torch

from . import _binding

bitmask_dtype = torch.int32


def get_bitmask_shape(batch_size: int, vocab_size: int) -> Tuple[int, int]:
    return (int(batch_size), (int(vocab_size) + 31) // 32)


def allocate_token_bitmask(batch_size: int, vocab_size: int) -> torch.Tensor:
    return torch.full(get_bitmask_shape(batch_size, vocab_size), -1, dtype=bitmask_dtype)


def reset_token_bitmask(bitmask: torch.Tensor) -> None:
    if bitmask.dtype != bitmask_dtype:
        raise TypeError("bitmask must be int32")
    bitmask.fill_(-1)


def apply_token_bitmask_inplace(logits: torch.Tensor, bitmask: torch.Tensor, *,
                                vocab_size: Optional[int] = None,
                                indices: Optional[List[int]] = None) -> None:
    if logits.device != bitmask.device:
        raise ValueError(f"logits on {logits.device} and bitmask on {bitmask.device}: put both on the same "
                         "device (copy the bitmask to the GPU first)")
    if logits.is_cuda:
        _binding.mi_apply_bitmask_inplace(logits, bitmask, vocab_size, indices, -math.inf)
    else:
        _binding.mi_apply_bitmask_inplace_host(logits, bitmask, vocab_size, indices, -math.inf)

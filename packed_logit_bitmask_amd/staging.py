"""Mask staging: get the host-filled bitmask onto the GPU behind other work.

The grammar engine fills the bitmask on the host (XGrammar "Bitmask
Operations": the bitmask is allocated on the CPU and the caller copies it to
the GPU).  TensorRT-Edge-LLM's "Guided Decoder" keeps a host/device bitmask
pair, uploads on a stream and records an event instead of synchronising, so
the GPU is not idle while the host works.  ``MaskStager`` does the same
with HIP streams and events:

* ``depth`` pinned host buffers (page-locked, so the copy is a true async
  DMA) and as many device buffers, used round robin;
* ``host()`` returns the next host buffer to fill -- first waiting, on the
  host, until that buffer's previous upload has finished;
* ``upload()`` enqueues its copy on a side stream (default priority) and
  records an event;
* ``apply_inplace`` / ``apply_rows`` make the apply stream wait for that
  event (a device-side wait: the host does not block), launch the apply and
  record when it was enqueued, so the next upload into that device buffer
  waits for it.

A device-side wait costs the GPU a few microseconds even when the event has
long completed, so each wait is skipped when the host already sees the event
complete (the ordering it would enforce then already holds).

The apply itself is the library's kernel; this class only moves the mask.
"""

from __future__ import annotations

from typing import Optional

import torch

from .xgrammar_api import bitmask_dtype, get_bitmask_shape


class MaskStager:
    def __init__(self, batch_size: int, vocab_size: int, device="cuda", depth: int = 2,
                 copy_stream: Optional[torch.cuda.Stream] = None):
        if depth < 1:
            raise ValueError("depth must be >= 1")
        self.shape = get_bitmask_shape(batch_size, vocab_size)
        self.device = torch.device(device)
        self.depth = depth
        self.hosts = [torch.full(self.shape, -1, dtype=bitmask_dtype, pin_memory=True) for _ in range(depth)]
        self.devs = [torch.empty(self.shape, dtype=bitmask_dtype, device=self.device) for _ in range(depth)]
        self.copied = [None] * depth      # event: upload of slot k done (host buffer reusable)
        self.consumed = [None] * depth    # event: last apply that read device slot k was enqueued before this
        self.copy_stream = copy_stream or torch.cuda.Stream(device=self.device)
        self.k = -1

    def host(self) -> torch.Tensor:
        """Advance to the next slot and return its pinned host buffer to fill."""
        self.k = (self.k + 1) % self.depth
        ev = self.copied[self.k]
        if ev is not None:
            ev.synchronize()   # the previous copy out of this host buffer has landed
        return self.hosts[self.k]

    def upload(self) -> None:
        """Enqueue the host -> device copy of the current slot on the side stream."""
        k = self.k
        if k < 0:
            raise RuntimeError("upload() before host(): fill the buffer host() returns first")
        with torch.cuda.stream(self.copy_stream):
            if self.consumed[k] is not None and not self.consumed[k].query():
                self.copy_stream.wait_event(self.consumed[k])   # do not overwrite a mask still being applied
            self.devs[k].copy_(self.hosts[k], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(self.copy_stream)
        self.copied[k] = ev

    def _consume(self, stream):
        k = self.k
        if k < 0 or self.copied[k] is None:
            raise RuntimeError("apply before upload(): the current slot holds no mask yet")
        s = stream or torch.cuda.current_stream(self.device)
        if not self.copied[k].query():
            s.wait_event(self.copied[k])      # device-side wait for this slot's upload
        return k, s

    def _done(self, k, s):
        ev = torch.cuda.Event()
        ev.record(s)
        self.consumed[k] = ev                 # the next upload into slot k waits for this

    def apply_inplace(self, logits: torch.Tensor, vocab_size: Optional[int] = None, indices=None,
                      fill_value: float = float("-inf"), stream: Optional[torch.cuda.Stream] = None):
        """Apply the current slot's mask to ``logits`` on ``stream`` (default: current)."""
        from ._binding import mi_apply_bitmask_inplace

        k, s = self._consume(stream)
        mi_apply_bitmask_inplace(logits, self.devs[k], vocab_size, indices, fill_value, stream=s)
        self._done(k, s)
        return logits

    def apply_rows(self, logits: torch.Tensor, row_needs_mask=None, vocab_size: Optional[int] = None,
                   fill_value: float = float("-inf"), report: bool = False,
                   stream: Optional[torch.cuda.Stream] = None):
        """Gated apply of the current slot's mask (see ``mi_apply_bitmask_rows``)."""
        from ._binding import mi_apply_bitmask_rows

        k, s = self._consume(stream)
        rep = mi_apply_bitmask_rows(logits, self.devs[k], row_needs_mask, vocab_size, fill_value,
                                    report=report, stream=s)
        self._done(k, s)
        return rep

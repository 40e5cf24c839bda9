"""Per-layer anchor cache (groups, KV ids, residual), resident or offloaded.

At an anchor step each attention layer produces its query grouping (perm),
the selected KV ids of every group and the residual; the reuse steps that
follow read them back, layer by layer.  The ai.info page ("Main Findings",
cache transfers; "Key Contributions") describes keeping inactive entries in
CPU memory and prefetching the next layer's entry while the current layer
computes.  This module provides both placements behind one interface:

* resident (the default): the entries stay in device memory.  One MI355X
  holds 288 GB of HBM; a layer of the 40-head, N = 75600 video workload at
  density 0.2 needs 2.2 GB (perm 12 MB, ids 1.43 GB, residual 774 MB), so
  the 40 layers of such a model fit beside its weights.
* offloaded: the entries live in pinned host memory.  ``get(layer)`` hands out
  device copies staged in one of two device slots; the copy of layer l + 1 is
  started on a side stream as soon as layer l is handed out, so it overlaps
  layer l's attention.  Events order everything: a slot is refilled only after
  the work enqueued on the compute stream before the refill was requested
  (which includes every use of the slot's previous layer), and the compute
  stream waits for the copy of the layer it is given.  An entry handed out is
  valid for work enqueued on the current stream before the next get().

Only device memory, pinned host memory, copies, streams and events are used
here (PyTorch plumbing); every computation stays in the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass
class Entry:
    perm: torch.Tensor      # int32 [B, H, N]
    kv_idx: torch.Tensor    # int32 [B, H, G, K]
    residual: torch.Tensor  # bf16 [B, H, N, D]

    def tensors(self):
        return (self.perm, self.kv_idx, self.residual)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors())


def _like(t: torch.Tensor, device=None, pin=False) -> torch.Tensor:
    return torch.empty(t.shape, dtype=t.dtype, device=device if device is not None else t.device,
                       pin_memory=pin)


class AnchorCache:
    """Anchor metadata of ``layers`` attention layers.

    put(layer, perm, kv_idx, residual)  store a layer's entry (at an anchor)
    get(layer) -> Entry                 the layer's entry on the device, valid
                                        for work enqueued on the current stream
                                        before the next get()
    """

    def __init__(self, layers: int, offload: bool = False, device=None):
        self.layers = layers
        self.offload = offload
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self._host: list[Entry | None] = [None] * layers       # pinned host copies (offloaded)
        self._dev: list[Entry | None] = [None] * layers        # device entries (resident)
        if offload:
            self._side = torch.cuda.Stream(device=self.device)   # default priority
            self._slots: list[Entry | None] = [None, None]
            self._slot_layer = [-1, -1]
            self._copied = [None, None]      # event: the copy into the slot is done
            self._last_slot = -1             # slot of the entry handed out last
            self._stored: list[torch.cuda.Event | None] = [None] * layers

    # ---- anchor step ---------------------------------------------------
    def put(self, layer: int, perm: torch.Tensor, kv_idx: torch.Tensor, residual: torch.Tensor) -> None:
        if not self.offload:
            e = self._dev[layer]
            if e is None:
                e = Entry(_like(perm), _like(kv_idx), _like(residual))
                self._dev[layer] = e
            for dst, src in zip(e.tensors(), (perm, kv_idx, residual)):
                dst.copy_(src)
            return
        e = self._host[layer]
        if e is None:
            e = Entry(*(_like(t, device="cpu", pin=True) for t in (perm, kv_idx, residual)))
            self._host[layer] = e
        # write back on the side stream once the producers on the current
        # stream are done; the sources must stay alive until `stored` fires
        ready = torch.cuda.Event()
        ready.record(torch.cuda.current_stream(self.device))
        self._side.wait_event(ready)
        with torch.cuda.stream(self._side):
            for dst, src in zip(e.tensors(), (perm, kv_idx, residual)):
                dst.copy_(src, non_blocking=True)
                src.record_stream(self._side)
            done = torch.cuda.Event()
            done.record(self._side)
        self._stored[layer] = done
        # a stored layer invalidates whatever a slot holds of it
        for s in range(2):
            if self._slot_layer[s] == layer:
                self._slot_layer[s] = -1

    # ---- reuse steps -----------------------------------------------------
    def get(self, layer: int) -> Entry:
        if not self.offload:
            e = self._dev[layer]
            if e is None:
                raise KeyError(f"layer {layer} has no anchor entry")
            return e
        s = self._slot_of(layer)
        if s < 0:
            s = self._prefetch(layer, avoid=self._last_slot)
        torch.cuda.current_stream(self.device).wait_event(self._copied[s])
        self._last_slot = s
        # start the next layer's copy into the other slot now, so that it
        # overlaps the work the caller enqueues on this layer
        nxt = (layer + 1) % self.layers
        if nxt != layer and self._host[nxt] is not None and self._slot_of(nxt) < 0:
            self._prefetch(nxt, avoid=s)
        return self._slots[s]

    def _slot_of(self, layer: int) -> int:
        for s in range(2):
            if self._slot_layer[s] == layer:
                return s
        return -1

    def _prefetch(self, layer: int, avoid: int) -> int:
        """Copies the host entry of `layer` into the slot other than `avoid`.

        Everything that may still read the slot's old contents was enqueued on
        the current stream before this call (the slot was handed out by an
        earlier get()), so the copy waits for an event recorded here."""
        h = self._host[layer]
        if h is None:
            raise KeyError(f"layer {layer} has no anchor entry")
        s = 1 - avoid if avoid >= 0 else 0
        if self._slots[s] is None:
            self._slots[s] = Entry(*(_like(t, device=self.device) for t in h.tensors()))
        free = torch.cuda.Event()
        free.record(torch.cuda.current_stream(self.device))
        self._side.wait_event(free)
        if self._stored[layer] is not None:
            self._side.wait_event(self._stored[layer])
        with torch.cuda.stream(self._side):
            for dst, src in zip(self._slots[s].tensors(), h.tensors()):
                dst.copy_(src, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(self._side)
        self._copied[s] = ev
        self._slot_layer[s] = layer
        return s

    def entry_bytes(self, layer: int) -> int:
        e = self._host[layer] if self.offload else self._dev[layer]
        return e.nbytes() if e is not None else 0

"""PagedKVCache: device K/V pools + the host block allocator, driven step by step.

Orchestration only — every decision (slots, copies) comes from the C++ host
allocator and every byte moved on the device is moved by the library's HIP
kernels.  The pattern of one decode step, all on one HIP stream:

    slots, pairs = allocator.append_batch(seqs)      # host C++
    kv_copy_blocks(pairs)  (every layer)             # copy-on-write first
    kv_cache_write(slots, k_new, v_new)  (per layer)
    pa_decode(q, block tables)           (per layer)

Host-to-device uploads go through a small ring of pinned buffers so the host
can run ahead of the device; a ring slot is reused only after the copy that
last read it has completed (an event wait that normally returns at once).
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib


class _PinnedRing:
    """Pinned host staging buffers for asynchronous uploads."""

    def __init__(self, nbytes: int, depth: int = 8):
        self.bufs = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        self.events = [None] * depth
        self.next = 0

    def upload(self, array: np.ndarray, out: torch.Tensor, stream) -> torch.Tensor:
        array = np.ascontiguousarray(array)
        nbytes = array.nbytes
        if nbytes == 0:
            return out
        i = self.next
        self.next = (i + 1) % len(self.bufs)
        if self.bufs[i].numel() < nbytes:
            if self.events[i] is not None:
                self.events[i].synchronize()
            self.bufs[i] = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        elif self.events[i] is not None:
            self.events[i].synchronize()
        host = self.bufs[i][:nbytes]
        host.numpy()[:] = array.view(np.uint8).reshape(-1)
        out.view(torch.uint8).view(-1)[:nbytes].copy_(host, non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        self.events[i] = ev
        return out


class PagedKVCache:
    """K/V pools for ``num_layers`` layers sharing one block allocator."""

    def __init__(self, num_blocks, num_kv_heads, head_dim, block_size, num_layers=1,
                 initial_order=None, device="cuda", poison=True, stream=None):
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.block_size = block_size
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.alloc = _lib.BlockAllocator(num_blocks, block_size, initial_order)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        fill = float("nan") if poison else 0.0
        self.k = [torch.full(shape, fill, dtype=torch.float16, device=self.device)
                  for _ in range(num_layers)]
        self.v = [torch.full(shape, fill, dtype=torch.float16, device=self.device)
                  for _ in range(num_layers)]
        self._ring = _PinnedRing(1 << 20)
        self._dev_bufs = {}
        self._workspace = None

    # -- sequences -------------------------------------------------------------
    def new_sequence(self) -> int:
        return self.alloc.create()

    def fork(self, seq: int) -> int:
        return self.alloc.fork(seq)

    def free(self, seq: int):
        self.alloc.free(seq)

    def length(self, seq: int) -> int:
        return self.alloc.length(seq)

    # -- device staging -------------------------------------------------------
    def _buf(self, name, numel, dtype):
        t = self._dev_bufs.get(name)
        if t is None or t.numel() < numel or t.dtype != dtype:
            t = torch.empty(max(numel, 1), dtype=dtype, device=self.device)
            self._dev_bufs[name] = t
        return t[:numel]

    def upload(self, name, array: np.ndarray, dtype) -> torch.Tensor:
        out = self._buf(name, array.size, dtype)
        return self._ring.upload(array, out, self.stream).view(array.shape)

    def _copy_pairs(self, pairs: np.ndarray):
        if len(pairs):
            dev = self.upload("pairs", np.ascontiguousarray(pairs, dtype=np.int32), torch.int32)
            _lib.kv_copy_blocks(self.k, self.v, dev, stream=self.stream)

    # -- reserving slots (copy-on-write copies are issued here) -------------------
    def reserve(self, seq: int, n: int) -> torch.Tensor:
        """Slots for ``n`` more tokens of one sequence, as a device int64 tensor."""
        slots, pairs = self.alloc.append(seq, n)
        self._copy_pairs(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        return self.upload("slots", slots, torch.int64)

    def reserve_many(self, seqs, counts) -> torch.Tensor:
        """Slots for ``counts[i]`` more tokens of each ``seqs[i]`` (e.g. a batched prefill),
        concatenated in order, as one device int64 tensor; copies are issued first."""
        all_slots, all_pairs = [], []
        for seq, n in zip(seqs, counts):
            slots, pairs = self.alloc.append(int(seq), int(n))
            all_slots.append(slots)
            all_pairs.extend(pairs)
        self._copy_pairs(np.asarray(all_pairs, dtype=np.int32).reshape(-1, 2))
        flat = np.concatenate(all_slots) if all_slots else np.empty(0, dtype=np.int64)
        return self.upload("many_slots", flat, torch.int64)

    def reserve_step(self, seqs) -> torch.Tensor:
        """One slot per listed sequence (a decode step); device int64 [len(seqs)]."""
        slots, pairs = self.alloc.append_batch(seqs)
        self._copy_pairs(pairs)
        return self.upload("step_slots", slots, torch.int64)

    def write(self, slots: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, layer: int = 0):
        _lib.kv_cache_write(self.k[layer], self.v[layer], k_new, v_new, slots, stream=self.stream)

    # -- attention ---------------------------------------------------------------
    def block_tables(self, seqs, max_blocks=None, pad_value=None):
        """Device int32 tables [n, max_blocks], device int32 lengths [n], host max length."""
        seqs = np.asarray(seqs, dtype=np.int32)
        lens_host = np.array([self.alloc.length(int(s)) for s in seqs], dtype=np.int32)
        max_len = int(lens_host.max()) if len(lens_host) else 0
        if max_blocks is None:
            max_blocks = max(1, -(-max_len // self.block_size))
        pad = self.num_blocks if pad_value is None else pad_value
        tables, lens = self.alloc.export(seqs, max_blocks, pad)
        return (self.upload("tables", tables, torch.int32), self.upload("lens", lens, torch.int32),
                max_len)

    def workspace(self, num_seqs, num_q_heads, max_context_len, partition_size):
        need = _lib.pa_decode_workspace_size(num_seqs, num_q_heads, self.head_dim, max_context_len,
                                             partition_size)
        if need == 0:
            return None
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._workspace

    def attend(self, q, tables, lens, max_context_len, scale, partition_size=512, layer=0, out=None):
        s, hq, d = q.shape
        if out is None:
            out = torch.empty((s, hq, d), dtype=torch.float32, device=self.device)
        ws = self.workspace(s, hq, max_context_len, partition_size)
        _lib.pa_decode(out, q, self.k[layer], self.v[layer], tables, lens, scale, max_context_len,
                       partition_size=partition_size, workspace=ws, stream=self.stream)
        return out

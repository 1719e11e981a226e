"""PagedKVCache: device K/V pools + the host block allocator, driven step by step.

Orchestration only — every decision (slots, copies) comes from the C++ host
allocator and every byte moved on the device is moved by the library's HIP
kernels.  The pattern of one decode step, all on one HIP stream:

    slots, pairs = allocator.append_batch(seqs)      # host C++
    kv_copy_blocks(pairs)  (every layer)             # copy-on-write first
    kv_cache_write(slots, k_new, v_new)  (per layer)
    pa_decode(q, block tables)           (per layer)

Host-to-device uploads of one step (slots, copy pairs, tables, lengths,
schedule) are packed into one pinned buffer and sent with a single copy: each
small copy is a serialised operation on the stream, so one copy instead of
four or five shortens every step.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib


class _Staging:
    """Uploads several small host arrays with ONE host-to-device copy.

    The arrays are packed (16-byte aligned) into a pinned host buffer taken from a
    ring, copied asynchronously into a device buffer, and returned as typed views
    of that buffer.  A pinned ring slot is reused only after the copy that last
    read it has completed; the device buffer is reused in stream order, so views
    stay valid until the next ``upload`` on the same stream.
    """

    def __init__(self, device, depth: int = 4, nbytes: int = 1 << 20):
        self.device = device
        self.host = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        self.events = [None] * depth
        self.next = 0
        self.dev = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def upload(self, arrays, stream):
        arrays = [np.ascontiguousarray(a) for a in arrays]
        offsets, total = [], 0
        for a in arrays:
            offsets.append(total)
            total += (a.nbytes + 15) // 16 * 16
        i = self.next
        self.next = (i + 1) % len(self.host)
        if self.events[i] is not None:
            self.events[i].synchronize()
        if self.host[i].numel() < total:
            self.host[i] = torch.empty(total, dtype=torch.uint8, pin_memory=True)
        if self.dev.numel() < total:
            self.dev = torch.empty(total, dtype=torch.uint8, device=self.device)
        buf = self.host[i].numpy()
        for a, off in zip(arrays, offsets):
            buf[off:off + a.nbytes] = a.reshape(-1).view(np.uint8)
        if total:
            self.dev[:total].copy_(self.host[i][:total], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
            self.events[i] = ev
        views = []
        for a, off in zip(arrays, offsets):
            t = self.dev[off:off + a.nbytes].view(_TORCH_DTYPE[a.dtype.str[1:]])
            views.append(t.view(a.shape))
        return views


_TORCH_DTYPE = {"i4": torch.int32, "i8": torch.int64, "f4": torch.float32, "f2": torch.float16}


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
        self._staging = _Staging(self.device)
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
    def upload(self, *arrays):
        """Copy host arrays to the device in one transfer; returns device views."""
        return self._staging.upload(arrays, self.stream)

    def _copy_pairs_dev(self, pairs_dev):
        if pairs_dev is not None and pairs_dev.shape[0]:
            _lib.kv_copy_blocks(self.k, self.v, pairs_dev, stream=self.stream)

    # -- reserving slots (copy-on-write copies are issued here) -------------------
    def reserve(self, seq: int, n: int) -> torch.Tensor:
        """Slots for ``n`` more tokens of one sequence, as a device int64 tensor."""
        return self.reserve_many([seq], [n])

    def reserve_many(self, seqs, counts) -> torch.Tensor:
        """Slots for ``counts[i]`` more tokens of each ``seqs[i]`` (e.g. a batched prefill),
        concatenated in order, as one device int64 tensor; copies are issued first."""
        all_slots, all_pairs = [], []
        for seq, n in zip(seqs, counts):
            slots, pairs = self.alloc.append(int(seq), int(n))
            all_slots.append(slots)
            all_pairs.extend(pairs)
        flat = np.concatenate(all_slots) if all_slots else np.empty(0, dtype=np.int64)
        pairs = np.asarray(all_pairs, dtype=np.int32).reshape(-1, 2)
        slots_dev, pairs_dev = self.upload(flat.astype(np.int64), pairs)
        self._copy_pairs_dev(pairs_dev)
        return slots_dev

    def reserve_step(self, seqs) -> torch.Tensor:
        """One slot per listed sequence (a decode step); device int64 [len(seqs)]."""
        slots, pairs = self.alloc.append_batch(seqs)
        slots_dev, pairs_dev = self.upload(slots, pairs)
        self._copy_pairs_dev(pairs_dev)
        return slots_dev

    def decode_step(self, seqs, max_blocks=None, longest_first=True):
        """One decode step's host work with a single upload: reserve one slot per
        sequence (issuing copy-on-write copies), then export tables, lengths and the
        schedule.  Returns (device slots, DecodeBatch)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        slots, pairs = self.alloc.append_batch(seqs)
        tables, lens, max_len, order = self._tables(seqs, max_blocks, None, longest_first)
        arrays = [slots, pairs, tables, lens] + ([order] if order is not None else [])
        views = self.upload(*arrays)
        self._copy_pairs_dev(views[1])
        batch = DecodeBatch(views[2], views[3], max_len, views[4] if order is not None else None,
                            lens)
        return views[0], batch

    def write(self, slots: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, layer: int = 0):
        _lib.kv_cache_write(self.k[layer], self.v[layer], k_new, v_new, slots, stream=self.stream)

    # -- attention ---------------------------------------------------------------
    def _tables(self, seqs, max_blocks, pad_value, longest_first):
        lens = self.alloc.lengths(seqs)
        max_len = int(lens.max()) if len(lens) else 0
        if max_blocks is None:
            max_blocks = max(1, -(-max_len // self.block_size))
        pad = self.num_blocks if pad_value is None else pad_value
        tables, _ = self.alloc.export(seqs, max_blocks, pad)
        order = None
        if longest_first and len(lens) > 1:
            order = np.argsort(-lens, kind="stable").astype(np.int32)
        return tables, lens, max_len, order

    def batch(self, seqs, max_blocks=None, pad_value=None, longest_first=True) -> "DecodeBatch":
        """Upload the block tables, lengths and schedule of ``seqs`` for one decode launch.

        The returned device tensors stay valid until the next upload.
        """
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        tables, lens, max_len, order = self._tables(seqs, max_blocks, pad_value, longest_first)
        if order is None:
            t, l_ = self.upload(tables, lens)
            return DecodeBatch(t, l_, max_len, None, lens)
        t, l_, o = self.upload(tables, lens, order)
        return DecodeBatch(t, l_, max_len, o, lens)

    def workspace(self, num_seqs, num_q_heads, max_context_len, partition_size):
        need = _lib.pa_decode_workspace_size(num_seqs, num_q_heads, self.head_dim, max_context_len,
                                             partition_size)
        if need == 0:
            return None
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._workspace

    def attend(self, q, batch: "DecodeBatch", scale, partition_size="auto", layer=0, out=None):
        """Decode attention for ``batch``; ``partition_size`` "auto" applies
        ``choose_partition`` to the batch's host-side lengths."""
        s, hq, d = q.shape
        if partition_size == "auto":
            partition_size = choose_partition(batch.lens_host, hq, self.num_kv_heads,
                                              self.block_size)
        if out is None:
            out = torch.empty((s, hq, d), dtype=torch.float32, device=self.device)
        ws = self.workspace(s, hq, batch.max_len, partition_size)
        _lib.pa_decode(out, q, self.k[layer], self.v[layer], batch.tables, batch.lens, scale,
                       batch.max_len, partition_size=partition_size, workspace=ws,
                       stream=self.stream, work_order=batch.order)
        return out


def head_tile(num_q_heads: int, num_kv_heads: int) -> int:
    """Query heads one wave serves (the library's choice for fp16 queries: groups of
    4 or more run 4, 8 or 16 heads per wave on the matrix cores)."""
    group = num_q_heads // num_kv_heads
    for gt in (16, 8, 4):
        if group % gt == 0:
            return gt
    return 2 if group % 2 == 0 else 1


def choose_partition(lens_host, num_q_heads, num_kv_heads, block_size, gpu_waves=2048) -> int:
    """Split-context policy (measured on MI355X): one pass per request when there are
    enough (request, head tile) work items to fill the GPU; otherwise the largest of
    1024 / 512 tokens that yields a GPU's worth of items, else 512."""
    lens = np.asarray(lens_host, dtype=np.int64)
    if lens.size == 0:
        return 0
    tiles = num_q_heads // head_tile(num_q_heads, num_kv_heads)
    if lens.size * tiles >= gpu_waves and int(lens.max()) <= 8192:
        return 0
    for part in (1024, 512):
        if part % block_size:
            continue
        if tiles * int(np.sum((lens + part - 1) // part)) >= gpu_waves:
            return part
    return max(512, block_size)


class DecodeBatch:
    """Device views of one decode launch: tables, lengths, schedule; host lengths."""

    __slots__ = ("tables", "lens", "max_len", "order", "lens_host")

    def __init__(self, tables, lens, max_len, order, lens_host):
        self.tables = tables
        self.lens = lens
        self.max_len = max_len
        self.order = order
        self.lens_host = lens_host

"""PagedKVCache: device K/V pools + the host block allocator, driven step by step.

Orchestration only — every decision (slots, copies) comes from the C++ host
allocator and every byte moved on the device is moved by the library's HIP
kernels.  The pattern of one decode step, all on one HIP stream:

    slots, pairs = allocator.append_batch(seqs)      # host C++
    kv_copy_blocks(pairs)  (every layer)             # copy-on-write first
    kv_cache_write(slots, k_new, v_new)  (per layer)
    pa_decode(q, block tables)           (per layer)

Host-to-device uploads of one step (slots, copy pairs, tables, lengths, the
launch's work items) are packed into one pinned buffer and sent with a single
copy: each small copy is a serialised operation on the stream, so one copy
instead of four or five shortens every step.

With ``host_blocks`` > 0 the cache also has a host tier: K/V pools in pinned
host memory to which whole requests can be swapped out and back in
(``swap_out`` / ``swap_in``); the allocator picks the blocks and a library
kernel on the cache's stream moves them over the host link.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _lib


class _Stamp:
    """Which upload a set of device views came from: ring slot and its generation.
    ``current()`` is False once a later upload has reused that slot's device buffer."""

    __slots__ = ("staging", "slot", "gen")

    def __init__(self, staging, slot, gen):
        self.staging, self.slot, self.gen = staging, slot, gen

    def current(self) -> bool:
        return self.staging.gen[self.slot] == self.gen


class _RingMarks:
    """Bookkeeping of a staging ring of ``depth`` slots (no device work).

    Upload u uses slot u % depth.  A completion mark (an event) follows every
    ``mark_every``-th upload only, since each is a barrier packet that costs the
    GPU a few microseconds between kernels.  Slot i, last read by upload u, may
    be written again once the first mark at or after u has completed; that mark
    exists because it comes at most mark_every - 1 uploads after u, before the
    slot's next use."""

    def __init__(self, depth, mark_every):
        if not 0 < mark_every < depth:
            raise ValueError("need 0 < mark_every < depth")
        self.depth, self.mark_every = depth, mark_every
        self.count = 0                      # uploads issued so far
        self.marks = []                     # (upload index, handle), oldest first
        self.last_use = [-1] * depth        # upload that last read each slot, or -1

    def next_slot(self):
        """(slot of the next upload, handle of the mark to wait for first, or None)."""
        i = self.count % self.depth
        used = self.last_use[i]
        if used < 0:
            return i, None
        while self.marks and self.marks[0][0] < used:
            self.marks.pop(0)
        return i, self.marks[0][1]

    def issued(self, slot, read, make_mark):
        """Account for the upload just issued in ``slot`` (``read``: it launched a
        copy that reads the slot); ``make_mark()`` records and returns a mark when
        one is due.  Returns the upload's index."""
        u = self.count
        self.count += 1
        if read:
            self.last_use[slot] = u
        if u % self.mark_every == self.mark_every - 1:
            self.marks.append((u, make_mark()))
        return u


class _Staging:
    """Uploads several small host arrays with ONE host-to-device copy.

    The arrays are packed (16-byte aligned) into a pinned host buffer taken from a
    ring, copied asynchronously into the device buffer of the same ring slot, and
    returned as typed views of that buffer.  A pinned slot is reused only after the
    copy that last read it has completed; a device slot is reused in stream order,
    ``depth`` uploads later.  So the views of one upload (say a decode step's
    tables) stay valid while up to ``depth - 1`` other uploads (a prefill, a swap)
    run in between; each upload's stamp (``last_stamp``) tells whether they still are.
    Completion marks follow every ``mark_every``-th upload only (``_RingMarks``).
    """

    def __init__(self, device, depth: int = 8, nbytes: int = 1 << 20, mark_every: int = 4):
        self.device = device
        self.ring = _RingMarks(depth, mark_every)
        self.host = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        self.dev = [torch.empty(nbytes, dtype=torch.uint8, device=device) for _ in range(depth)]
        self.gen = [0] * depth
        self.last_stamp = None

    def _slot(self, nbytes):
        """Next ring slot, once the copy that last read its pinned buffer is done."""
        i, wait = self.ring.next_slot()
        if wait is not None:
            wait.synchronize()
        if self.host[i].numel() < nbytes:
            self.host[i] = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        return i

    def _send(self, i, total, stream, write=None, mark=None):
        """Copy ``total`` bytes of ring slot i's pinned buffer to its device buffer.
        ``write`` (a callable taking the device buffer's address and the pinned slot)
        replaces the plain copy with one launch that also writes the step's new tokens.
        ``mark``, a ``_lib.KernelTimer``, takes the launch's kernel times."""
        if self.dev[i].numel() < total:
            self.dev[i] = torch.empty(total, dtype=torch.uint8, device=self.device)
        self.gen[i] += 1
        self.last_stamp = _Stamp(self, i, self.gen[i])
        dev = self.dev[i]
        if total:
            # A library kernel reads the pinned buffer over the bus: no copy-engine
            # hand-off between the step's kernels.
            nbytes = (total + 15) // 16 * 16
            if mark is not None:
                _lib.time_next_call(mark)
            if write is None:
                _lib._check(_lib.lib().pkv_upload(dev.data_ptr(), self.host[i].data_ptr(),
                                                  nbytes, stream.cuda_stream))
            else:
                write(dev.data_ptr(), self.host[i].data_ptr(), nbytes)

        def mark():
            ev = torch.cuda.Event()
            ev.record(stream)
            return ev

        self.ring.issued(i, total > 0, mark)
        return dev

    def upload(self, arrays, stream):
        arrays = [np.ascontiguousarray(a) for a in arrays]
        offsets, total = [], 0
        for a in arrays:
            offsets.append(total)
            total += (a.nbytes + 15) // 16 * 16
        i = self._slot(total)
        buf = self.host[i].numpy()
        for a, off in zip(arrays, offsets):
            buf[off:off + a.nbytes] = a.reshape(-1).view(np.uint8)
        dev = self._send(i, total, stream)
        views = []
        for a, off in zip(arrays, offsets):
            t = dev[off:off + a.nbytes].view(_TORCH_DTYPE[a.dtype.str[1:]])
            views.append(t.view(a.shape))
        return views

    def fill_and_upload(self, fill, stream, write=None, mark=None):
        """``fill(host_ptr, capacity)`` writes the host buffer in place and returns the
        bytes used, or None with ``needed`` bytes to retry with.  Returns
        (result of fill, device buffer, pinned host buffer) after one asynchronous copy.
        ``write(result)``, if given, returns the fused copy-and-write for ``_send`` (or
        None for a plain copy)."""
        i = self._slot(0)
        while True:
            host = self.host[i]
            res = fill(host.data_ptr(), host.numel())
            if res is not None:
                break
            self.host[i] = torch.empty(max(fill.needed, 2 * host.numel()), dtype=torch.uint8,
                                       pin_memory=True)
        fused = write(res) if write is not None else None
        return res, self._send(i, int(res.total_bytes), stream, fused, mark), self.host[i]


_TORCH_DTYPE = {"i4": torch.int32, "i8": torch.int64, "f4": torch.float32, "f2": torch.float16}


class DeviceArray:
    """A typed region of a device buffer: its address for the library, and a torch
    view built only when asked for (``tensor()``)."""

    __slots__ = ("base", "offset", "dtype", "shape", "ptr", "_t", "stamp")

    def __init__(self, base, offset, dtype, shape, stamp=None):
        self.base, self.offset, self.dtype, self.shape = base, int(offset), dtype, tuple(shape)
        self.ptr = base.data_ptr() + self.offset
        self._t = None
        self.stamp = stamp          # the staging upload holding it, if any

    @classmethod
    def of(cls, t):
        a = cls.__new__(cls)
        a.base, a.offset, a.dtype, a.shape, a.ptr, a._t = t, 0, t.dtype, tuple(t.shape), t.data_ptr(), t
        a.stamp = None
        return a

    def tensor(self):
        if self._t is None:
            n = int(np.prod(self.shape)) * torch.empty(0, dtype=self.dtype).element_size()
            self._t = self.base[self.offset:self.offset + n].view(self.dtype).view(self.shape)
        return self._t

    def cpu(self):
        return self.tensor().cpu()


class PagedKVCache:
    """K/V pools for ``num_layers`` layers sharing one block allocator.

    ``num_q_heads`` and ``q_dtype`` describe the queries that will attend (they
    decide the kernel and so the schedule that ``decode_step`` and ``batch``
    prepare); defaults: one query head per KV head, fp16.  ``prefix_groups``
    lets ``decode_step`` group requests that share leading physical blocks
    (forked samples and beams) so that ``attend`` reads those blocks once per
    group (``pa_decode_grouped``); the planner uses groups only where they pay.
    """

    def __init__(self, num_blocks, num_kv_heads, head_dim, block_size, num_layers=1,
                 initial_order=None, device="cuda", poison=True, stream=None,
                 num_q_heads=None, q_dtype=None, host_blocks=0, host_order=None,
                 prefix_groups=True):
        self.prefix_groups = bool(prefix_groups)
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.block_size = block_size
        self.num_q_heads = int(num_q_heads) if num_q_heads else num_kv_heads
        self.q_dtype = q_dtype if q_dtype is not None else torch.float16
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.alloc = _lib.BlockAllocator(num_blocks, block_size, initial_order)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        fill = float("nan") if poison else 0.0
        self.k = [torch.full(shape, fill, dtype=torch.float16, device=self.device)
                  for _ in range(num_layers)]
        self.v = [torch.full(shape, fill, dtype=torch.float16, device=self.device)
                  for _ in range(num_layers)]
        self.host_blocks = int(host_blocks)
        self.host_k, self.host_v = [], []
        if self.host_blocks:
            self.alloc.add_host_tier(self.host_blocks, host_order)
            hshape = (self.host_blocks, num_kv_heads, block_size, head_dim)
            for pools in (self.host_k, self.host_v):
                for _ in range(num_layers):
                    t = torch.empty(hshape, dtype=torch.float16, pin_memory=True)
                    if poison:
                        t.fill_(float("nan"))
                    pools.append(t)
        self._staging = _Staging(self.device)
        self._plan_staging = _Staging(self.device, nbytes=1 << 16)   # re-plans in attend
        self._workspace = None
        self._stream_ptr = self.stream.cuda_stream
        self._epoch = 0
        self._pending = []            # (epoch, event) of deferred frees, oldest first

    # -- sequences -------------------------------------------------------------
    def new_sequence(self) -> int:
        return self.alloc.create()

    def fork(self, seq: int) -> int:
        return self.alloc.fork(seq)

    def free(self, seq: int, deferred: bool = False):
        """Release a sequence.  Immediate reuse is safe for work on this cache's stream
        (it runs in order).  ``deferred=True`` keeps its blocks out of circulation until
        the device work enqueued on the stream so far has finished (an event marks it),
        so that work on other streams, or a host running ahead, cannot reuse them early."""
        if not deferred:
            self.alloc.free(seq)
            return
        self._epoch += 1
        ev = torch.cuda.Event()
        ev.record(self.stream)
        self._pending.append((self._epoch, ev))
        self.alloc.free_deferred(seq, self._epoch)

    def retire(self, wait: bool = False) -> int:
        """Return the blocks of deferred frees whose device work has finished (all of
        them, waiting, with ``wait=True``) to the free list; how many came back."""
        done = None
        while self._pending and (wait or self._pending[0][1].query()):
            if wait:
                self._pending[0][1].synchronize()
            done = self._pending.pop(0)[0]
        return self.alloc.retire(done) if done is not None else 0

    def length(self, seq: int) -> int:
        return self.alloc.length(seq)

    # -- the host tier -----------------------------------------------------------
    def _epoch_for(self, deferred):
        if not deferred:
            return 0
        self._epoch += 1
        return self._epoch

    def _after_copy(self, deferred, epoch):
        if deferred:
            ev = torch.cuda.Event()
            ev.record(self.stream)
            self._pending.append((epoch, ev))

    def swap_out(self, seqs, deferred: bool = False, events=None) -> int:
        """Move the requests' blocks to the host tier (each distinct block once, blocks
        shared inside the set stay shared) and free their device blocks.  The copy runs
        on the cache's stream, so work queued later on it may reuse the blocks at once;
        ``deferred=True`` keeps them out of circulation until the copy has finished
        (for work on other streams).  ``events`` (start, end), if given, are recorded
        on the stream around the copy kernels.  Returns the number of blocks copied."""
        if self._pending:
            self.retire()
        epoch = self._epoch_for(deferred)
        pairs = self.alloc.swap_out(np.asarray(seqs, dtype=np.int32), deferred, epoch)
        self._move(pairs, self.host_k, self.host_v, self.k, self.v, events)
        self._after_copy(deferred, epoch)
        return int(pairs.shape[0])

    def swap_in(self, seqs, deferred: bool = False, events=None) -> int:
        """Move swapped-out requests back to device blocks (the inverse of ``swap_out``;
        the new blocks are whatever the free list gives).  Returns the blocks copied."""
        if self._pending:
            self.retire()
        epoch = self._epoch_for(deferred)
        pairs = self.alloc.swap_in(np.asarray(seqs, dtype=np.int32), deferred, epoch)
        self._move(pairs, self.k, self.v, self.host_k, self.host_v, events)
        self._after_copy(deferred, epoch)
        return int(pairs.shape[0])

    def _move(self, pairs, dst_k, dst_v, src_k, src_v, events=None):
        if pairs.shape[0] == 0:
            return
        for first in range(0, pairs.shape[0], 65535):       # the kernel's per-call limit
            (pairs_dev,) = self.upload(pairs[first:first + 65535])
            if events is not None and first == 0:
                events[0].record(self.stream)
            _lib.kv_swap_blocks(dst_k, dst_v, src_k, src_v, pairs_dev, stream=self.stream)
        if events is not None:
            events[1].record(self.stream)

    def is_swapped(self, seq: int) -> bool:
        return self.alloc.is_swapped(seq)

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
        if self._pending:
            self.retire()
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
        if self._pending:
            self.retire()
        slots, pairs = self.alloc.append_batch(seqs)
        slots_dev, pairs_dev = self.upload(slots, pairs)
        self._copy_pairs_dev(pairs_dev)
        return slots_dev

    def decode_step(self, seqs, max_blocks=None, partition_size="auto", k_new=None, v_new=None,
                    layer=0, marks=None):
        """One decode step's host work in one library call and one upload: reserve one
        slot per sequence (issuing copy-on-write copies), export tables and lengths and
        plan the launch (``kv_decode_step_host``).  With ``k_new``/``v_new`` ([S, kv_heads,
        head_dim] fp16 device tensors) the new tokens are written into ``layer`` too; a
        step without copy-on-write copies does the upload and the write in one launch
        (``pkv_upload_write``).  Returns (device slots, DecodeBatch).

        The slots and the batch's device arrays sit in one slot of the cache's
        staging ring, which later uploads (steps, batches, prefills, swaps,
        reserves) reuse only after the ring's other slots: up to 7 of them may run
        between this call and ``attend``; after more, ``attend`` and ``write``
        raise instead of reading another call's bytes.

        ``marks`` (for timing) is a dict of ``_lib.KernelTimer``: "upload" takes
        the kernel times of the upload (fused with the write on steps without
        copies), and on steps with copy-on-write copies "copy" and "write" those
        of the copy and the write (``_lib.time_next_call``); ``marks["pairs"]`` is
        set to the number of copied blocks."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        if self._pending:
            self.retire()
        key = (self.num_q_heads, self.q_dtype, partition_size)
        part = -1 if partition_size == "auto" else int(partition_size)
        qd = _lib.PKV_F16 if self.q_dtype == torch.float16 else _lib.PKV_F32
        alloc = self.alloc

        flags = _lib.PKV_STEP_GROUPS if self.prefix_groups else 0

        def fill(ptr, cap):
            lay = alloc.decode_step_host(seqs, max_blocks or 0, self.num_blocks, self.num_q_heads,
                                         self.num_kv_heads, self.head_dim, qd, part, ptr, cap,
                                         flags=flags)
            if lay is None:
                fill.needed = alloc.needed
            return lay

        n = int(seqs.shape[0])
        if k_new is not None:
            want = (n, self.num_kv_heads, self.head_dim)
            for x in (k_new, v_new):
                if (x is None or tuple(x.shape) != want or x.dtype != torch.float16 or not x.is_cuda
                        or not x.is_contiguous()):
                    raise ValueError(f"k_new/v_new must be contiguous device fp16 {want}")

        def fused(lay):
            if k_new is None or lay.num_pairs:
                return None                  # copy-on-write copies go between upload and write

            def launch(dev_ptr, host_ptr, nbytes):
                _lib._check(_lib.lib().pkv_upload_write(
                    dev_ptr, host_ptr, nbytes, self.k[layer].data_ptr(), self.v[layer].data_ptr(),
                    self.num_blocks, k_new.data_ptr(), v_new.data_ptr(),
                    host_ptr + lay.slots_offset, n, self.num_kv_heads, self.head_dim,
                    self.block_size, self._stream_ptr))
            return launch

        lay, dev, host = self._staging.fill_and_upload(
            fill, self.stream, fused, None if marks is None else marks["upload"])
        lens_host = host[lay.lens_offset:lay.lens_offset + 4 * n].numpy().view(np.int32).copy()
        if marks is not None:
            marks["pairs"] = int(lay.num_pairs)
        if lay.num_pairs:
            if marks is not None:
                _lib.time_next_call(marks["copy"])
            _lib.kv_copy_blocks(self.k, self.v, DeviceArray(dev, lay.pairs_offset, torch.int32,
                                                            (lay.num_pairs, 2)).tensor(),
                                stream=self.stream)
        plan = {name: int(getattr(lay.plan, name)) for name, _ in _lib.DecodePlan._fields_}
        slots = DeviceArray(dev, lay.slots_offset, torch.int64, (n,), self._staging.last_stamp)
        if k_new is not None and lay.num_pairs:
            if marks is not None:
                _lib.time_next_call(marks["write"])
            self.write(slots, k_new, v_new, layer=layer)
        batch = DecodeBatch(DeviceArray(dev, lay.tables_offset, torch.int32, (n, lay.max_blocks)),
                            DeviceArray(dev, lay.lens_offset, torch.int32, (n,)),
                            int(lay.max_context_len), lens_host,
                            DeviceArray(dev, lay.items_offset, torch.int32, (plan["num_items"],)),
                            plan, key)
        batch.stamp = self._staging.last_stamp
        if lay.num_group_items:
            batch.groups_dev = DeviceArray(dev, lay.groups_offset, torch.int32,
                                           (lay.num_groups, _lib.GROUP_STRIDE))
            batch.group_items_dev = DeviceArray(dev, lay.group_items_offset, torch.int32,
                                                (lay.num_group_items,))
            batch.shared_dev = DeviceArray(dev, lay.shared_lens_offset, torch.int32, (n,))
        return slots, batch

    def write(self, slots, k_new: torch.Tensor, v_new: torch.Tensor, layer: int = 0):
        """Store k_new/v_new ([T, kv_heads, head_dim] fp16) at ``slots`` (int64 [T])."""
        if not isinstance(slots, DeviceArray):
            _lib.kv_cache_write(self.k[layer], self.v[layer], k_new, v_new, slots,
                                stream=self.stream)
            return
        if slots.stamp is not None and not slots.stamp.current():
            raise RuntimeError("slots are stale: later uploads have reused their staging buffer")
        t = slots.shape[0]
        want = (t, self.num_kv_heads, self.head_dim)
        for x in (k_new, v_new):
            if (tuple(x.shape) != want or x.dtype != torch.float16 or not x.is_cuda
                    or not x.is_contiguous()):
                raise ValueError(f"k_new/v_new must be contiguous device fp16 {want}")
        _lib._check(_lib.lib().kv_cache_write(
            self.k[layer].data_ptr(), self.v[layer].data_ptr(), self.num_blocks, k_new.data_ptr(),
            v_new.data_ptr(), slots.ptr, t, self.num_kv_heads, self.head_dim, self.block_size,
            self._stream_ptr))

    # -- attention ---------------------------------------------------------------
    def _tables(self, seqs, max_blocks, pad_value):
        lens = self.alloc.lengths(seqs)
        max_len = int(lens.max()) if len(lens) else 0
        if max_blocks is None:
            max_blocks = max(1, -(-max_len // self.block_size))
        pad = self.num_blocks if pad_value is None else pad_value
        tables, _ = self.alloc.export(seqs, max_blocks, pad)
        return tables, lens, max_len

    def _plan(self, lens, num_q_heads, q_dtype, partition_size):
        """Host schedule (library planner): work items as int32 bits, plan dict."""
        part = -1 if partition_size == "auto" else int(partition_size)
        qd = _lib.PKV_F16 if q_dtype == torch.float16 else _lib.PKV_F32
        items, info = _lib.plan(lens, num_q_heads, self.num_kv_heads, self.head_dim,
                                self.block_size, qd, part)
        return items.view(np.int32), info

    def batch(self, seqs, max_blocks=None, pad_value=None, partition_size="auto") -> "DecodeBatch":
        """Upload the block tables, lengths and launch schedule of ``seqs`` for decode
        (with prefix groups where they pay, as ``decode_step`` plans them).

        The returned device arrays live in one slot of the cache's staging ring: they
        stay valid while fewer than 8 later uploads have been made (``attend``
        refuses a batch whose slot was reused).
        """
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        tables, lens, max_len = self._tables(seqs, max_blocks, pad_value)
        key = (self.num_q_heads, self.q_dtype, partition_size)
        if self.prefix_groups and self.q_dtype == torch.float16:
            part = -1 if partition_size == "auto" else int(partition_size)
            items, info, groups, gitems, shared = _lib.plan_groups(
                tables, lens, self.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size,
                _lib.PKV_F16, part)
            if len(groups):
                t, l_, it, g, gi, sh = self.upload(tables, lens, items.view(np.int32), groups,
                                                   gitems.view(np.int32), shared)
                batch = DecodeBatch(DeviceArray.of(t), DeviceArray.of(l_), max_len, lens,
                                    DeviceArray.of(it), info, key)
                batch.groups_dev, batch.group_items_dev = DeviceArray.of(g), DeviceArray.of(gi)
                batch.shared_dev = DeviceArray.of(sh)
                batch.stamp = self._staging.last_stamp
                return batch
        items, info = self._plan(lens, *key)
        t, l_, it = self.upload(tables, lens, items)
        batch = DecodeBatch(DeviceArray.of(t), DeviceArray.of(l_), max_len, lens,
                            DeviceArray.of(it), info, key)
        batch.stamp = self._staging.last_stamp
        return batch

    def workspace(self, num_seqs, num_q_heads, max_context_len, partition_size):
        need = _lib.pa_decode_workspace_size(num_seqs, num_q_heads, self.head_dim, max_context_len,
                                             partition_size)
        if need == 0:
            return None
        if self._workspace is None or self._workspace.numel() < need:
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._workspace

    def prefill(self, q, seqs, q_lens, scale, layer=0, out=None, timing=None):
        """Causal attention of new tokens (``pa_prefill``): ``q`` [T, Hq, D] fp16 holds
        the last ``q_lens[i]`` tokens of each ``seqs[i]`` in order, whose K/V are
        already written.  Tables, lengths, query offsets and the work list go up in
        one upload.  Returns out [T, Hq, D] fp32.  ``timing``, a ``_lib.KernelTimer``,
        takes the prefill kernel's start and end."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        tables, lens, _ = self._tables(seqs, None, None)
        starts = _prefill_starts(q_lens)
        items = _lib.prefill_plan(np.diff(starts), lens, q.shape[1], self.num_kv_heads)
        t_d, l_d, s_d, i_d = self.upload(tables, lens, starts, items.view(np.int32))
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        if timing is not None:
            _lib.time_next_call(timing)
        _lib.pa_prefill(out, q, s_d, self.k[layer], self.v[layer], t_d, l_d, scale, i_d,
                        stream=self.stream)
        return out

    def check_tables(self, batch: "DecodeBatch") -> dict:
        """Debug check of a batch's device tables and lengths against this pool
        (pkv_check_tables): ids outside the pool, lengths the tables cannot hold,
        and the first offender.  Waits for the cache's stream."""
        return _lib.check_tables(batch.tables, batch.lens, self.block_size, self.num_blocks,
                                 stream=self.stream)

    def attend(self, q, batch: "DecodeBatch", scale, partition_size=None, layer=0, out=None,
               timing=None):
        """Decode attention for ``batch`` with the schedule planned for it.

        ``partition_size`` None keeps the batch's plan; "auto" or a number plans
        again (the library's policy, or that split), as does a query shape or dtype
        other than the one the batch was planned for.  ``timing``, a
        ``_lib.KernelTimer``, takes the decode kernels' start and end
        (``_lib.time_next_call``).
        """
        s, hq, d = q.shape
        if batch.stamp is not None and not batch.stamp.current():
            raise RuntimeError(
                "DecodeBatch is stale: its tables and work list were in a staging buffer that "
                f"{len(self._staging.dev)} later uploads (decode steps, batches, prefills, swaps, "
                "reserves) have reused; make the batch again")
        key = (hq, q.dtype, batch.plan_key[2] if partition_size is None else partition_size)
        if key == batch.plan_key:
            items, info = batch.items_dev, batch.plan
        else:
            items_h, info = self._plan(batch.lens_host, *key)
            (items,) = self._plan_staging.upload([items_h], self.stream)
            items = DeviceArray.of(items)
        if out is None:
            out = torch.empty((s, hq, d), dtype=torch.float32, device=self.device)
        if (q.dtype not in (torch.float16, torch.float32) or not q.is_cuda or not q.is_contiguous()
                or d != self.head_dim or s != batch.num_seqs):
            raise ValueError("q must be a contiguous device fp16/fp32 [S, Hq, head_dim] tensor "
                             "for the batch's S requests")
        if (tuple(out.shape) != (s, hq, d) or out.dtype != torch.float32 or not out.is_cuda
                or not out.is_contiguous()):
            raise ValueError("out must be a contiguous device fp32 [S, Hq, head_dim] tensor")
        part = info["partition_size"]
        grouped = key == batch.plan_key and batch.group_items_dev is not None
        # a grouped launch keeps one spare partial slot per request
        ws = self.workspace(s, hq, batch.max_len + (part if grouped else 0), part)
        if timing is not None:
            _lib.time_next_call(timing)
        if grouped:
            g, gi = batch.groups_dev, batch.group_items_dev
            _lib._check(_lib.lib().pa_decode_grouped(
                out.data_ptr(), q.data_ptr(), _lib.PKV_F16, self.k[layer].data_ptr(),
                self.v[layer].data_ptr(), self.num_blocks, batch.tables_dev.ptr,
                batch.tables_dev.shape[1], batch.lens_dev.ptr, s, hq, self.num_kv_heads, d,
                self.block_size, float(scale), batch.max_len, part, items.ptr, items.shape[0],
                info["waves_per_cu"], g.ptr, g.shape[0], gi.ptr, gi.shape[0], batch.shared_dev.ptr,
                info["fuse_groups"], ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0,
                self._stream_ptr))
            return out
        _lib._check(_lib.lib().pa_decode(
            out.data_ptr(), q.data_ptr(), _lib.PKV_F16 if q.dtype == torch.float16 else _lib.PKV_F32,
            self.k[layer].data_ptr(), self.v[layer].data_ptr(), self.num_blocks,
            batch.tables_dev.ptr, batch.tables_dev.shape[1], batch.lens_dev.ptr, s, hq,
            self.num_kv_heads, d, self.block_size, float(scale), batch.max_len, part, items.ptr,
            items.shape[0], info["waves_per_cu"], ws.data_ptr() if ws is not None else None,
            ws.numel() if ws is not None else 0, self._stream_ptr))
        return out


def _prefill_starts(q_lens):
    return np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))]).astype(np.int32)


class DecodeBatch:
    """One decode launch: device tables, lengths and work items (``*_dev``: addresses
    for the library; ``tables``/``lens``/``items``: torch views, built on demand), the
    host lengths, the plan and the (num_q_heads, q dtype, partition request) it was
    made for."""

    __slots__ = ("tables_dev", "lens_dev", "max_len", "lens_host", "items_dev", "plan",
                 "plan_key", "num_seqs", "groups_dev", "group_items_dev", "shared_dev", "stamp")

    def __init__(self, tables, lens, max_len, lens_host, items, plan, plan_key):
        self.tables_dev, self.lens_dev, self.items_dev = tables, lens, items
        self.stamp = None          # the upload that holds the device arrays (cache-made batches)
        self.groups_dev = self.group_items_dev = self.shared_dev = None   # prefix groups
        self.max_len = max_len
        self.lens_host = lens_host
        self.plan = plan
        self.plan_key = plan_key
        self.num_seqs = tables.shape[0]

    @property
    def tables(self):
        return self.tables_dev.tensor()

    @property
    def lens(self):
        return self.lens_dev.tensor()

    @property
    def items(self):
        return self.items_dev.tensor()

"""One rank's optimizer over its FlatParameter shard: owns the fp32 master, m,
v and the device step state, and issues the library calls of one step in the
order the pages give (reduce or statistics, then the fused AdamW step).  No
arithmetic happens here; every part of the step runs in libzeroflat.
"""
import torch

from . import (ZERO_AVG, StepState, _current_raw_stream, zero_adamw_hparams_t,
               zero_adamw_shard_step, zero_grad_accumulate_shard, zero_grad_reduce_shard,
               zero_grad_reduce_shard_int8, zero_offload_step, zero_unscale_norm)


class ShardOptimizer:
    def __init__(self, master, hp, loss_scale=65536.0, dynamic=False, window=1000,
                 min_scale=1.0, quant_block=0):
        if master.dtype != torch.float32 or not master.is_cuda or not master.is_contiguous():
            raise ValueError("master must be a contiguous float32 CUDA tensor")
        self.master = master
        self.exp_avg = torch.zeros_like(master)
        self.exp_avg_sq = torch.zeros_like(master)
        self.hp = dict(hp)
        self.state = StepState(loss_scale, dynamic, window, min_scale, device=master.device)
        self.quant_block = quant_block
        self._red = None
        self._h = (None, None)   # (hp items, their C struct)

    @property
    def numel(self):
        return self.master.numel()

    def _hparams(self):
        """The C hyper-parameter struct, rebuilt only when self.hp changed."""
        key = tuple(self.hp.items())
        if self._h[0] != key:
            self._h = (key, zero_adamw_hparams_t(**self.hp))
        return self._h[1]

    def reduced_buffer(self):
        if self._red is None:
            self._red = torch.empty_like(self.master)
        return self._red

    def step_from_rank_buffers(self, grad_bufs, elem_offset, allgather_buf, slot_offset,
                               op=ZERO_AVG, q_buf=None, q_scales=None, q_slot_offset=0,
                               q_scale_offset=0, stream=None):
        """Reduce-Scatter's reduce over the N rank buffers, then the step."""
        red = self.reduced_buffer()
        if stream is None:
            stream = _current_raw_stream()   # one lookup for both calls
        zero_grad_reduce_shard(grad_bufs, elem_offset, self.numel, op, red, self.state,
                               stream=stream)
        self._apply(red, allgather_buf, slot_offset, q_buf, q_scales, q_slot_offset,
                    q_scale_offset, stream)

    def step_from_int8_grads(self, q_slices, scale_slices, allgather_buf, slot_offset,
                             op=ZERO_AVG, block=256, q_buf=None, q_scales=None, q_slot_offset=0,
                             q_scale_offset=0, stream=None):
        """Reduce over the N ranks' INT8-quantised gradient slices for this rank
        (ZeRO++'s quantised Reduce-Scatter), then the step."""
        red = self.reduced_buffer()
        if stream is None:
            stream = _current_raw_stream()
        zero_grad_reduce_shard_int8(q_slices, scale_slices, self.numel, op, red, self.state,
                                    block=block, stream=stream)
        self._apply(red, allgather_buf, slot_offset, q_buf, q_scales, q_slot_offset,
                    q_scale_offset, stream)

    def micro_step(self, grad_bufs, elem_offset, op=ZERO_AVG, first=False, last=False,
                   stream=None):
        """One micro-step of gradient accumulation into the fp32 gradient shard:
        the first overwrites it (reduce), later ones add to it, and the last one
        also takes the step statistics over the accumulated shard."""
        red = self.reduced_buffer()
        st = self.state if last else None
        if first:
            zero_grad_reduce_shard(grad_bufs, elem_offset, self.numel, op, red, st, stream=stream)
        else:
            zero_grad_accumulate_shard(grad_bufs, elem_offset, self.numel, op, red, st,
                                       stream=stream)

    def step_from_accumulated(self, allgather_buf, slot_offset, q_buf=None, q_scales=None,
                              q_slot_offset=0, q_scale_offset=0, stream=None):
        """The step on the shard accumulated by micro_step (statistics already taken)."""
        if self._red is None:
            raise RuntimeError("no accumulated gradient: call micro_step first")
        self._apply(self._red, allgather_buf, slot_offset, q_buf, q_scales, q_slot_offset,
                    q_scale_offset, stream)

    def step_from_reduced(self, grad_shard, allgather_buf, slot_offset, q_buf=None,
                          q_scales=None, q_slot_offset=0, q_scale_offset=0, stream=None):
        """Statistics over an already reduced (fp32/fp16/bf16) shard, then the step."""
        if stream is None:
            stream = _current_raw_stream()
        zero_unscale_norm(grad_shard, self.state, n=self.numel, stream=stream)
        self._apply(grad_shard, allgather_buf, slot_offset, q_buf, q_scales, q_slot_offset,
                    q_scale_offset, stream)

    def _apply(self, grad, allgather_buf, slot_offset, q_buf, q_scales, q_slot_offset,
               q_scale_offset, stream):
        zero_adamw_shard_step(grad, self.master, self.exp_avg, self.exp_avg_sq, allgather_buf,
                              slot_offset, self._hparams(), self.state, q_buf=q_buf,
                              q_scales=q_scales,
                              q_slot_offset=q_slot_offset, q_scale_offset=q_scale_offset,
                              q_block=self.quant_block or 256, finalize=True, stream=stream)


class OffloadShardOptimizer:
    """ZeRO-Offload for one rank's shard: the fp32 master, m and v live in host
    memory and the update runs on host cores; the device keeps the gradient
    shard, the step state and the All-Gather buffer.  Pinned staging buffers
    carry the gradient to the host and the 16-bit parameters back; with a
    16-bit gradient and `in_place_staging`, one buffer serves both ways (each
    chunk's parameters overwrite its gradients in place)."""

    def __init__(self, master_host, hp, loss_scale=65536.0, dynamic=False, window=1000,
                 min_scale=1.0, device="cuda", n_threads=0, chunk=0, in_place_staging=True):
        if master_host.dtype != torch.float32 or master_host.is_cuda or \
                not master_host.is_contiguous():
            raise ValueError("master must be a contiguous float32 host tensor")
        self.master = master_host
        self.exp_avg = torch.zeros_like(master_host)
        self.exp_avg_sq = torch.zeros_like(master_host)
        self.hp = dict(hp)
        self.state = StepState(loss_scale, dynamic, window, min_scale, device=device)
        self.n_threads = n_threads
        self.chunk = chunk
        self.in_place_staging = in_place_staging
        self._stage = {}

    @property
    def numel(self):
        return self.master.numel()

    def _staging(self, role, dtype):
        """The pinned buffer for one direction ("grad" down, "param" up)."""
        key = (role, dtype)
        if key not in self._stage:
            self._stage[key] = torch.empty(self.numel, dtype=dtype, pin_memory=True)
        return self._stage[key]

    def _staging_pair(self, grad_dtype, param_dtype):
        g = self._staging("grad", grad_dtype)
        if self.in_place_staging and g.element_size() == 2:
            return g, g.view(param_dtype)
        return g, self._staging("param", param_dtype)

    def step_from_reduced(self, grad_shard, allgather_buf, slot_offset, stream=None):
        """Statistics over the device gradient shard, then the offloaded step."""
        zero_unscale_norm(grad_shard, self.state, n=self.numel, stream=stream)
        g_stage, lp_stage = self._staging_pair(grad_shard.dtype, allgather_buf.dtype)
        zero_offload_step(grad_shard, self.master, self.exp_avg, self.exp_avg_sq, g_stage, lp_stage,
                          allgather_buf, slot_offset, self.hp, self.state, chunk=self.chunk,
                          n_threads=self.n_threads, stream=stream)


class MultiShardOptimizer:
    """One rank's shards of several FlatParameters (one per FSDP unit) under a
    single optimizer.  One step state serves every unit, so the global gradient
    norm, the clip coefficient, the overflow skip and the loss scale cover all
    of them, as one optimizer over all the model's parameters does.  A step
    takes the statistics of every unit first, then runs each unit's AdamW, and
    updates the loss scaler once, after the last unit."""

    def __init__(self, masters, hp, loss_scale=65536.0, dynamic=False, window=1000,
                 min_scale=1.0):
        if not masters:
            raise ValueError("need at least one master shard")
        for k, mst in enumerate(masters):
            if mst.dtype != torch.float32 or not mst.is_cuda or not mst.is_contiguous():
                raise ValueError("masters[%d] must be a contiguous float32 CUDA tensor" % k)
        self.master = list(masters)
        self.exp_avg = [torch.zeros_like(mst) for mst in masters]
        self.exp_avg_sq = [torch.zeros_like(mst) for mst in masters]
        self.hp = dict(hp)
        self.state = StepState(loss_scale, dynamic, window, min_scale, device=masters[0].device)
        self._red = [None] * len(masters)

    def __len__(self):
        return len(self.master)

    def _check(self, *lists):
        for x in lists:
            if len(x) != len(self.master):
                raise ValueError("one entry per unit expected (%d units)" % len(self.master))

    def _reduced(self, u):
        if self._red[u] is None:
            self._red[u] = torch.empty_like(self.master[u])
        return self._red[u]

    def step_from_rank_buffers(self, grad_bufs, elem_offsets, allgather_bufs, slot_offsets,
                               op=ZERO_AVG, quant=None, stream=None):
        """grad_bufs[u]: unit u's N rank gradient buffers; the reduce of each
        unit with its statistics, then the step of every unit (with the INT8
        payloads of `quant`, see _apply)."""
        self._check(grad_bufs, elem_offsets, allgather_bufs, slot_offsets)
        for u, (bufs, off) in enumerate(zip(grad_bufs, elem_offsets)):
            zero_grad_reduce_shard(bufs, off, self.master[u].numel(), op, self._reduced(u),
                                   self.state, stream=stream)
        self._apply(self._red, allgather_bufs, slot_offsets, stream, quant)

    def micro_step(self, grad_bufs, elem_offsets, op=ZERO_AVG, first=False, last=False,
                   stream=None):
        """One micro-step of gradient accumulation for every unit, as
        ShardOptimizer.micro_step: the first overwrites each unit's fp32
        gradient shard, later ones add to it, and the last one takes every
        unit's statistics into the shared state."""
        self._check(grad_bufs, elem_offsets)
        st = self.state if last else None
        for u, (bufs, off) in enumerate(zip(grad_bufs, elem_offsets)):
            fn = zero_grad_reduce_shard if first else zero_grad_accumulate_shard
            fn(bufs, off, self.master[u].numel(), op, self._reduced(u), st, stream=stream)

    def step_from_accumulated(self, allgather_bufs, slot_offsets, quant=None, stream=None):
        """The step of every unit on the shards accumulated by micro_step."""
        self._check(allgather_bufs, slot_offsets)
        if any(r is None for r in self._red):
            raise RuntimeError("no accumulated gradient: call micro_step first")
        self._apply(self._red, allgather_bufs, slot_offsets, stream, quant)

    def step_from_reduced(self, grad_shards, allgather_bufs, slot_offsets, quant=None,
                          stream=None):
        """Statistics over every unit's reduced (fp32/fp16/bf16) shard, then the
        step of every unit."""
        self._check(grad_shards, allgather_bufs, slot_offsets)
        for u, g in enumerate(grad_shards):
            zero_unscale_norm(g, self.state, n=self.master[u].numel(), stream=stream)
        self._apply(grad_shards, allgather_bufs, slot_offsets, stream, quant)

    def _apply(self, grads, allgather_bufs, slot_offsets, stream, quant=None):
        """quant: None, or per unit None or (q_buf, q_scales, q_slot_offset,
        q_scale_offset) for that unit's blockwise-INT8 All-Gather payload."""
        if quant is not None:
            self._check(quant)
        last = len(grads) - 1
        for u, g in enumerate(grads):
            q = quant[u] if quant is not None and quant[u] is not None else (None, None, 0, 0)
            zero_adamw_shard_step(g, self.master[u], self.exp_avg[u], self.exp_avg_sq[u],
                                  allgather_bufs[u], slot_offsets[u], self.hp, self.state,
                                  q_buf=q[0], q_scales=q[1], q_slot_offset=q[2],
                                  q_scale_offset=q[3], finalize=u == last, stream=stream)

"""One decode step of the sparse-MLA path with simulated DCP shards on one GPU.

Chains the three library calls with buffers allocated once up front (no allocation,
no host synchronisation inside ``run``, so ``capture`` can record a step as a HIP graph):

    for each shard r:  sparse_mla_convert_index(ids -> shard-local slots, -1 in place)
                       sparse_mla_decode(q, shard cache, slots -> partial out, lse)
    sparse_mla_merge_lse(partials -> out, lse)

With one shard the merge is skipped and decode writes the final output directly.  The
flow follows page "FlashMLA sparse fp8 path gains DCP and MTP", "Implementation
breakdown" steps 1-3 (localise ids, return LSE in the kernel's (H, T) layout, merge
partials in (T, H)); here every shard runs on the same device.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from . import _binding as B


class DcpDecodeStep:
    def __init__(self, *, T: int, H: int, K: int, dcp_size: int, block_size: int, softmax_scale: float,
                 out_dtype: torch.dtype = torch.bfloat16, partial_dtype: torch.dtype = torch.float32,
                 lse_layout: str = "HT", device="cuda", num_splits: int = 0, interleave: int = 1):
        self.T, self.H, self.K, self.D, self.interleave = T, H, K, dcp_size, interleave
        self.block_size, self.scale, self.num_splits = block_size, float(softmax_scale), num_splits
        dev = torch.device(device)
        self.slots = torch.empty((dcp_size, T, K), dtype=torch.int32, device=dev)
        self.valid = torch.empty((dcp_size, T), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, H, B.LATENT_DIM), dtype=out_dtype, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        if dcp_size > 1:
            self.parts = torch.empty((dcp_size, T, H, B.LATENT_DIM), dtype=partial_dtype, device=dev)
            if lse_layout == "HT":  # kernel-native (H, T) per shard, read back as (T, H) by the merge
                self.lse_store = torch.empty((dcp_size, H, T), dtype=torch.float32, device=dev)
                self.lse_parts = self.lse_store.transpose(1, 2)
            else:
                self.lse_store = torch.empty((dcp_size, T, H), dtype=torch.float32, device=dev)
                self.lse_parts = self.lse_store
        if num_splits == 0 and dcp_size > 1:  # plan the shard decodes for their ~K / D valid entries
            num_splits = shard_splits(T, H, K, dcp_size, torch.cuda.get_device_properties(dev).multi_processor_count)
            self.num_splits = num_splits
        need = B.sparse_mla_decode_workspace_size(T, H, K, num_splits)
        self.workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev) if need else None

    def run(self, q: torch.Tensor, ids: torch.Tensor, req: torch.Tensor,
            shards: Sequence[Tuple[torch.Tensor, torch.Tensor]], decode_events: Optional[list] = None
            ) -> Tuple[torch.Tensor, torch.Tensor]:
        """shards[r] = (kv_cache_r [num_slots_r, 656] uint8, block_table_r [R, W_r] int32).

        decode_events: if a list is given, a (start, end) pair of timing events recorded on the
        launch stream around every decode call is appended to it.
        """
        if len(shards) != self.D:
            raise ValueError("one (cache, block table) pair per shard")
        stream = torch.cuda.current_stream(q.device)
        for r, (cache, bt) in enumerate(shards):
            B.convert_index(ids, req, bt, self.block_size, dcp_size=self.D, dcp_rank=r, interleave=self.interleave,
                            out=self.slots[r], valid=self.valid[r])
            if decode_events is not None:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[0].record(stream)
            self.decode_shard(q, cache, r)
            if decode_events is not None:
                ev[1].record(stream)
                decode_events.append(ev)
        if self.D > 1:
            B.merge_lse(self.parts, self.lse_parts, out=self.out, lse=self.lse)
        return self.out, self.lse

    def decode_shard(self, q: torch.Tensor, cache: torch.Tensor, r: int) -> None:
        """The decode of shard r alone, from the slots and counts its last conversion left."""
        if self.D == 1:
            B.decode(q, cache, self.slots[r], self.scale, out=self.out, lse=self.lse, num_splits=self.num_splits,
                     workspace=self.workspace, valid_count=self.valid[r])
        else:
            B.decode(q, cache, self.slots[r], self.scale, out=self.parts[r], lse=self.lse_parts[r],
                     num_splits=self.num_splits, workspace=self.workspace, valid_count=self.valid[r])

    def capture(self, q: torch.Tensor, ids: torch.Tensor, req: torch.Tensor,
                shards: Sequence[Tuple[torch.Tensor, torch.Tensor]]) -> "torch.cuda.CUDAGraph":
        """Record one run() over these tensors as a HIP graph.

        Each replay re-runs the whole step (every conversion, decode and the merge) on the same
        storage: change the inputs' contents in place between replays, never their storage.
        Results land in self.out / self.lse.  The graph holds kernel nodes only (no memset or
        copy nodes), and one graph must not be replayed on two streams at once, since the
        replays share this step's buffers.
        """
        self.run(q, ids, req, shards)  # outside the capture: first-use work of the binding and torch
        torch.cuda.synchronize(q.device)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(q, ids, req, shards)
        return graph


def shard_splits(T: int, H: int, K: int, dcp_size: int, cus: int) -> int:
    """Top-k ranges per row for the decode of one DCP shard.  The library's automatic plan splits
    rows that are too few to cover the CUs, keeping at least 256 list entries per range; a shard
    row holds only about K / dcp_size valid entries (the others are -1), so the same rule is
    applied to that count.  A range never exceeds the 4096 entries one workgroup compacts, and a
    call takes at most 64 ranges."""
    items = T * -(-H // 64)
    splits = 1
    if 0 < items < cus:
        splits = min(-(-cus // items), max(1, -(-K // dcp_size) // 256))
    return min(max(splits, -(-K // 4096), 1), 64)


def device_shards(workload, device="cuda") -> List[Tuple[torch.Tensor, torch.Tensor]]:
    """(cache, block table) device tensors of every shard of a workload (the unsharded cache
    as the single shard when the workload has no DCP split)."""
    if workload.dcp_size == 1 or not workload.shards:
        return [(workload.cache.to_device(device), torch.from_numpy(workload.block_table).to(device))]
    return [(sh.cache.to_device(device), torch.from_numpy(sh.block_table).to(device)) for sh in workload.shards]

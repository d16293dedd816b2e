"""The caller-side exchange of the split step across data-parallel ranks.

The clip coefficient and the skip decision need the squared gradient norm over every
rank's shard [GPT-NeoX article
"GPT-NeoX：如何为开源社区打开千亿级大模型训练的“民主化”之门", 技术深度解析: ZeRO stage 1 shards the
optimizer state over the data-parallel ranks].  Each rank runs `neox_zero1_step_local`,
then `gather_sumsq` all-gathers the ranks' fp64 squared norms into one array in rank
order, then each rank runs `neox_zero1_step_apply(h, array, nranks=world)`, whose
finalize adds them in a fixed order, so every rank takes the same decisions.  This
module moves data only; the sum is the library's.

On MI355X ranks the tensors live in HBM and the group is RCCL ("nccl"); a gloo group
takes CPU tensors.
"""
import torch
import torch.distributed as dist


def gather_sumsq(local: torch.Tensor, group=None) -> torch.Tensor:
    """local: one-element float64 tensor (this rank's squared norm).  Returns a new
    contiguous float64 tensor of world-size elements on the same device, element r being
    rank r's value."""
    if local.dtype != torch.float64 or local.numel() != 1:
        raise ValueError("local must be a one-element float64 tensor")
    world = dist.get_world_size(group)
    parts = [torch.empty_like(local) for _ in range(world)]
    dist.all_gather(parts, local.contiguous(), group=group)
    return torch.cat(parts).contiguous()

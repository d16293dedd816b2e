"""The caller-side exchange of the split step across data-parallel ranks.

The clip coefficient and the skip decision need the squared gradient norm over every
rank's shard [GPT-NeoX article
"GPT-NeoX：如何为开源社区打开千亿级大模型训练的“民主化”之门", 技术深度解析: ZeRO stage 1 shards the
optimizer state over the data-parallel ranks].  Each rank runs
`neox_zero1_step_local`, then `global_sumsq` all-gathers the ranks' fp64 values and adds
them in rank order, so every rank holds the same bits and takes the same skip and clip
decisions; then each rank runs `neox_zero1_step_apply` on the result.  A non-finite
value from any rank (an overflow there) makes the sum non-finite on every rank.

On MI355X ranks the tensors live in HBM and the group is RCCL ("nccl"); a gloo group
takes CPU tensors.  This is communication glue outside the step's kernels.
"""
import torch
import torch.distributed as dist


def global_sumsq(local: torch.Tensor, group=None) -> torch.Tensor:
    """local: one-element float64 tensor (this rank's squared norm).  Returns a new
    one-element tensor on the same device with the rank-order sum over the group."""
    if local.dtype != torch.float64 or local.numel() != 1:
        raise ValueError("local must be a one-element float64 tensor")
    world = dist.get_world_size(group)
    parts = [torch.empty_like(local) for _ in range(world)]
    dist.all_gather(parts, local, group=group)
    out = parts[0].clone()
    for p in parts[1:]:
        out += p
    return out

"""MI355X-native Hydra/Medusa draft-and-verify round (libhydra, HIP for gfx950).

The four stages and the commit of the kept branch are the C entry points of
include/hydra.h, bound under the same names in
``speculative_decoding_hydra_amd.hydra``; ``HydraRound`` allocates the buffers
of a round and calls them in order.
"""
from .hydra import (  # noqa: F401
    DevicePlan, HydraError, PackedWeight, PlanRows, TreePlan, hydra_draft_heads, hydra_draft_heads_attn,
    hydra_draft_heads_attn_workspace_size, hydra_draft_heads_sketch,
    hydra_draft_heads_sketch_workspace_size, hydra_draft_heads_workspace_size,
    hydra_fold_embedding, hydra_pack_weight, hydra_packed_weight_size, hydra_plan_cartesian, hydra_plan_rows, hydra_plan_sparse, hydra_vocab_projection,
    hydra_vocab_projection_workspace_size, hydra_vocab_topk, tree_accept, tree_accept_noalloc,
    tree_accept_workspace_size, tree_attention_verify, tree_attention_verify_workspace_size, tree_build,
    tree_build_workspace_size, tree_commit, tree_decoder_layer, tree_decoder_layer_workspace_size, tree_rope,
    tree_rope_qk, tree_verify_layers, tree_verify_layers_workspace_size,
)
from .round import HydraRound, make_plan, round_from_inputs, run_round  # noqa: F401

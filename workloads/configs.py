"""The five workloads: shapes, formats and activation types.

"R x C" in a shape is output rows x input columns (N x K).
"""
from .gen import FMT_Q8_0, FMT_Q4_0, FMT_MXFP4

CONFIGS = {
    0: dict(name="q8_0_2048x2048_m1_f32x", fmt=FMT_Q8_0, xt="f32",
            mats=[("w", 2048, 2048)], ms=[1]),
    1: dict(name="q4_0_qwen3_4b_like_layer_m1", fmt=FMT_Q4_0, xt="bf16",
            mats=[("gate_up", 19456, 2560), ("down", 2560, 9728)], ms=[1]),
    2: dict(name="q8_0_full_decode_sweep_m1", fmt=FMT_Q8_0, xt="bf16",
            mats=None, ms=[1]),
    3: dict(name="q4_0_cobatch_8b_like", fmt=FMT_Q4_0, xt="bf16",
            mats=[("qkv", 6144, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)],
            ms=[2, 4, 8]),
    4: dict(name="mxfp4_moe_32x_top4", fmt=FMT_MXFP4, xt="bf16",
            n_experts=32, top_k=4,
            mats=[("gate_up", 3584, 2048), ("down", 2048, 1792)], ms=[1, 4]),
}

C2_LAYERS = 36
C2_LAYER_MATS = [("qkv", 6144, 2560), ("o", 2560, 4096), ("gate_up", 19456, 2560), ("down", 2560, 9728)]
C2_LM_HEAD = ("lm_head", 151936, 2560)


def c2_sweep_shapes():
    """[(matrix_index, name, n, k)] for the 145 launches of the full decode sweep,
    in dependency order: per layer qkv, o, gate_up, down; the LM head last."""
    out = []
    for layer in range(C2_LAYERS):
        for r, (nm, n, k) in enumerate(C2_LAYER_MATS):
            out.append((4 * layer + r, f"l{layer}.{nm}", n, k))
    out.append((4 * C2_LAYERS, C2_LM_HEAD[0], C2_LM_HEAD[1], C2_LM_HEAD[2]))
    return out

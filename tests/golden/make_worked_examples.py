"""Writes the hand-derived worked examples in this folder (closed forms, Python ``math`` only).

Nothing here runs the oracle or the HIP path: every expected value below is derived by hand
in the comments and evaluated with ``math`` so that the fixtures can pin the oracle.

Attention examples follow the causal ("autoregressive", "Inside Large World Model: UC
Berkeley Multimodal Model that can Understand 1 Hour Long Videos", "Core Architecture")
softmax attention with the masked-sequence-packing mask ("LWM：突破 100 万 Token 的开源大模型"
§概述 (b)).  RoPE examples follow "theta-scaled RoPE" ("[论文解读] World Model on Million-Length
Video And Language With Blockwise RingAttention" §提出的方法) with inv_freq_i = theta^(-2i/D).
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def attention_cases():
    r2 = math.sqrt(2.0)
    # D = 2, scale 1/sqrt(2): with q_i = (1, 0) and k_j = (sqrt(2) ln w_j, 0) the score of key j
    # is ln w_j, so the softmax weights are w = (1, 2, 3).
    k = [[0.0, 0.0], [r2 * math.log(2.0), 0.0], [r2 * math.log(3.0), 0.0]]
    q = [[1.0, 0.0]] * 3
    v = [[6.0, 0.0], [0.0, 3.0], [0.0, -6.0]]
    causal = {
        "name": "causal_three_tokens",
        "derivation": "row0: only key0 -> O=v0, lse=0; row1: weights 1,2 -> O=(v0+2v1)/3=(2,2), "
                      "lse=ln3; row2: weights 1,2,3 -> O=(v0+2v1+3v2)/6=(1,-2), lse=ln6",
        "q": q, "k": k, "v": v, "seg": None, "scale": None,
        "o": [[6.0, 0.0], [2.0, 2.0], [1.0, -2.0]],
        "lse": [0.0, math.log(3.0), math.log(6.0)],
    }
    packed = dict(causal)
    packed.update({
        "name": "packed_segment_boundary",
        "derivation": "seg=(0,0,1): rows 0,1 as in the causal case; row2 only sees key2 -> O=v2=(0,-6), "
                      "lse=score(2,2)=ln3",
        "seg": [0, 0, 1],
        "o": [[6.0, 0.0], [2.0, 2.0], [0.0, -6.0]],
        "lse": [0.0, math.log(3.0), math.log(3.0)],
    })
    unit = dict(causal)
    unit.update({
        "name": "explicit_unit_scale",
        "derivation": "scale=1 with k_j=(ln w_j, 0): same weights 1,2,3 as the causal case",
        "k": [[0.0, 0.0], [math.log(2.0), 0.0], [math.log(3.0), 0.0]],
        "scale": 1.0,
    })
    return [causal, packed, unit]


def rope_cases():
    return [
        {"name": "d2_pos1", "derivation": "D=2: inv_freq=1, rotate (1,0) by 1 rad",
         "x": [1.0, 0.0], "pos": 1, "theta": 10000.0, "layout": "half",
         "y": [math.cos(1.0), math.sin(1.0)]},
        {"name": "d4_half_pos2", "derivation": "D=4, theta=1e4: inv_freq=(1, 0.01); pairs (0,2),(1,3); "
                                              "(1,0) by 2 rad and (1,0) by 0.02 rad",
         "x": [1.0, 1.0, 0.0, 0.0], "pos": 2, "theta": 10000.0, "layout": "half",
         "y": [math.cos(2.0), math.cos(0.02), math.sin(2.0), math.sin(0.02)]},
        {"name": "d4_interleaved_pos2", "derivation": "pairs (0,1),(2,3): (1,0) by 2 rad, (0,1) by 0.02 rad",
         "x": [1.0, 0.0, 0.0, 1.0], "pos": 2, "theta": 10000.0, "layout": "interleaved",
         "y": [math.cos(2.0), math.sin(2.0), -math.sin(0.02), math.cos(0.02)]},
        {"name": "d2_inverse_pos3", "derivation": "rotate (0,1) by -3 rad -> (sin3, cos3)",
         "x": [0.0, 1.0], "pos": 3, "theta": 5.0e7, "layout": "half", "inverse": True,
         "y": [math.sin(3.0), math.cos(3.0)]},
    ]


if __name__ == "__main__":
    for name, cases, cite in (
        ("worked_attention.json", attention_cases(),
         "causal softmax attention ('Inside Large World Model...' Core Architecture) with the packing "
         "mask ('LWM：突破 100 万 Token 的开源大模型' §概述 (b)); values derived by hand"),
        ("worked_rope.json", rope_cases(),
         "theta-scaled RoPE ('[论文解读] World Model on Million-Length Video And Language With Blockwise "
         "RingAttention' §提出的方法); values derived by hand"),
    ):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump({"source": cite, "cases": cases}, f, indent=1)
            f.write("\n")

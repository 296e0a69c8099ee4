"""The synthetic workloads, by name.

Each entry states the shapes and value distributions of one workload.  The
second argument of every N(mu, s) is a standard deviation.  Where a recipe
says "built like the tiny workload" it means: target logits ~ N(0, 2).  The
Zipf-like alternative (reading "B") is available for the large linear
workload through ``logits="zipf"``.
"""

CONFIGS = {
    # B=1, gamma=4, V=32, fp32; target ~ N(0,2); draft = target + N(0,1);
    # uniforms [1,5]; T = 1.0.
    "tiny": dict(kind="linear", B=1, gamma=4, V=32, dtype="f32",
                 logits="normal", target_std=2.0, draft_noise=1.0,
                 temperature=1.0, seed=0),
    # B=8, gamma=5, V=32000, fp32; target = N(0,3) - 1.1 ln(rank) over one
    # seeded permutation of the vocabulary; draft = target + N(0,0.5); T = 1.
    "zipf32k": dict(kind="linear", B=8, gamma=5, V=32000, dtype="f32",
                    logits="zipf", target_std=3.0, zipf_slope=1.1,
                    draft_noise=0.5, temperature=1.0, seed=0),
    # B=64, gamma=7, V=128256, bf16; target ~ N(0,2); draft noise N(0,0.8);
    # T = 0.7; uniforms [64,8].  Also used in greedy mode.
    "b64g7v128k": dict(kind="linear", B=64, gamma=7, V=128256, dtype="bf16",
                       logits="normal", target_std=2.0, draft_noise=0.8,
                       temperature=0.7, seed=0),
    # B=32, complete binary candidate tree of 63 nodes (parent(i)=(i-1)/2,
    # root parent -1), bf16 target [32,63,128256] ~ N(0,2); node token =
    # argmax of its parent's target row with probability 0.7, else uniform.
    "tree63": dict(kind="tree", B=32, N=63, V=128256, dtype="bf16",
                   logits="normal", target_std=2.0, match_prob=0.7,
                   tree="binary", seed=0),
    # Stochastic tree verification: B=32, complete binary tree of 63 nodes,
    # bf16 target rows [32,63,128256] ~ N(0,2), draft rows = target + N(0,0.8),
    # T = 0.7 (the large linear workload's distributions); every node's token
    # is drawn independently from its parent's draft row; uniforms [32,63].
    "tree_sample63": dict(kind="tree_sample", B=32, N=63, V=128256, dtype="bf16",
                          logits="normal", target_std=2.0, draft_noise=0.8,
                          temperature=0.7, tree="binary", seed=0),
    # B=64, gamma=5, d=4096: target features bf16 [64*6,4096] ~ N(0,1);
    # LM head bf16 [4096,128256] ~ N(0,0.02); draft features = target
    # features (rows i<gamma) + N(0,0.3); T = 1.
    "eagle_lmhead": dict(kind="lmhead", B=64, gamma=5, d=4096, V=128256,
                         feat_std=1.0, w_std=0.02, draft_noise=0.3,
                         temperature=1.0, seed=0),
}


def get_config(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg

"""Selection-quality report: how well the pre-downsampled block scores rank
key blocks against the exact post-downsample attention map.

The pith.science review of "Efficient Long-Context Modeling in Diffusion
Language Models via Block Approximate Sparse Attention" has the diagonal
covariance correction stand in for the full covariance, and the compact
scores stand in for the post-downsample map ("Core claim", abstract); the
referee report notes that neither approximation is measured.  For one
workload this compares three block scores -- the corrected diagonal score
the selection pass uses, the same second-cumulant score with full block
covariances, and the uncorrected pooled logit -- with two reference maps --
the block log-mean-exp of the logits and the block mean of the softmax
probabilities -- row by row: recall of the kept sets at the workload's
sparsity and Spearman's rank correlation.  Everything runs on the GPU
through the C ABI.

    python -m block_sparse_attention_ba_amd.quality [workload ...]
"""

from __future__ import annotations

import json
import sys

SCORES = ("diag", "full", "mean")
REFS = ("lme", "prob")


def _timed(fn, stream, reps: int = 3):
    import torch
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    out = None
    for a, b in evs:
        a.record(stream)
        out = fn()
        b.record(stream)
    torch.cuda.synchronize()
    return out, min(a.elapsed_time(b) for a, b in evs)


def measure(q, k, v, block: int, sparsity: float) -> dict:
    """Quality of the three block scores against both reference maps for
    bf16 Q/K/V [B,H,N,D] on the GPU.  Returns mean recall and mean rho over
    all (b, h, query-block) rows for each (score, reference) pair, the
    fraction of rows whose kept set equals the reference's, and the device
    time of the diagnostic calls."""
    import torch

    from block_sparse_attention_ba_amd import api

    B, H, N, D = (int(x) for x in q.shape)
    n = api.num_blocks(N, block)
    keep = api.keep_count(n, sparsity)
    stream = torch.cuda.current_stream(q.device)
    ws = torch.empty(api.score_full_workspace_bytes(B, H, N, D, block), dtype=torch.uint8, device=q.device)
    (_, _, _, s_diag) = api.select(q, k, block, sparsity, return_score=True)
    (s_full, s_mean), full_ms = _timed(lambda: api.score_full(q, k, block, workspace=ws), stream)
    del ws
    _, lse = api.dense(q, k, v, out_dtype=torch.bfloat16)
    (m_lme, m_prob), map_ms = _timed(lambda: api.block_map(q, k, block, lse=lse), stream)
    scores = {"diag": s_diag, "full": s_full, "mean": s_mean}
    refs = {"lme": m_lme, "prob": m_prob}
    pairs = {}
    agree_ms = 0.0
    for sname in SCORES:
        for rname in REFS:
            (recall, rho), ms = _timed(lambda: api.rank_agreement(scores[sname], refs[rname], keep), stream, 1)
            agree_ms += ms
            pairs[f"{sname}_vs_{rname}"] = {
                "recall": round(float(recall.mean()), 5),
                "rho": round(float(rho.mean()), 5),
                "rows_exact": round(float((recall == 1.0).float().mean()), 5),
            }
    map_flops = 2.0 * B * H * N * N * D
    return {
        "keep": keep, "n_blocks": n, "rows": B * H * n, "pairs": pairs,
        "block_map_ms": round(map_ms, 4), "block_map_tflops": round(map_flops / map_ms / 1e9, 1),
        "score_full_ms": round(full_ms, 4), "rank_agreement_ms_total": round(agree_ms, 4),
    }


def main(argv):
    import numpy as np
    import torch

    from block_sparse_attention_ba_amd import api, workloads

    api.load()
    names = argv or ["tiny", "llada8b", "long_b64", "long_b128", "shift", "video"]
    dev = torch.device("cuda:0")
    for name in names:
        w = workloads.WORKLOADS[name]
        print(f"[quality] generating {name} ...", file=sys.stderr, flush=True)
        x = workloads.make_inputs(name)

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        q, k, v = up(x["q"]), up(x["k"]), up(x["v"])
        del x
        for sp in w.sparsities:
            if sp == 0.0:
                continue  # every block kept: nothing to rank
            res = measure(q, k, v, w.block, sp)
            print(json.dumps({"workload": name, "shape": f"B{w.B} H{w.H} N{w.N} D{w.D} b{w.block}",
                              "sparsity": sp, **res}), flush=True)
        del q, k, v
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main(sys.argv[1:])

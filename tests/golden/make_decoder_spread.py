"""Writes decoder_tree_spread.json: how far two valid fixed-order fp32 models
of the config-5 decoder drift apart, per position, over the 768 positions the
teacher-forced parity test scores.

Both models are the oracle (oracle/decoder.py): one folds every reduction in
ascending order, the other in descending order (matmul over k, the RMSNorm
sum of squares, attention's dot products and its sums over keys) -- the two
orders of the chapter "Batch-invariant kernels: why temperature-0 decoding is
still nondeterministic", Case 4 (forward and reverse), applied to the whole
model.  Both are exact definitions of the same mathematics; their per-position
distance, max |a - b| / max |a| over the vocabulary, is the spread a correct
implementation with a third tree can be expected to show against either.

Inputs are the parity test's: decoder weights (seed 0), prompt row 0 of the
[64, 512] seed-1 prompts, then 256 more ids (seed 5).

    python tests/golden/make_decoder_spread.py        # about a minute on 8 cores
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from invariant_reductions_amd import inputs          # noqa: E402  (seeded generators only)
from oracle import decoder as odec                    # noqa: E402

P, S = 512, 256


def main() -> None:
    cfg = inputs.LLAMA_4L
    w = inputs.decoder_weights(cfg, seed=0)
    seq = np.concatenate([inputs.prompts(64, P, cfg["vocab"], seed=1)[0], inputs.prompts(1, S, cfg["vocab"], seed=5)[0]])
    cos_t, sin_t = inputs.rope_tables(P + S + 8, cfg["head_dim"])
    a, _, ta = odec.forward(w, cfg, seq, cos_t, sin_t)
    b, _, tb = odec.forward(w, cfg, seq, cos_t, sin_t, descending=True)
    a64 = a.astype(np.float64)
    rel = np.abs(a64 - b).max(1) / np.abs(a64).max(1)
    out = {
        "source": "oracle/decoder.py forward, ascending vs descending reduction order (tests/golden/make_decoder_spread.py)",
        "workload": "config 5 decoder, seed-0 weights, prompt row 0 of seed-1 prompts [64, 512] + 256 seed-5 ids",
        "positions": int(rel.size),
        "max": float(rel.max()),
        "argmax": int(rel.argmax()),
        "median": float(np.median(rel)),
        "p90": float(np.quantile(rel, 0.9)),
        "greedy_token_mismatches": int((ta != tb).sum()),
        "per_position": [float(f"{x:.6e}") for x in rel],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decoder_tree_spread.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"spread over {rel.size} positions: max {rel.max():.4e} at {rel.argmax()}, median {np.median(rel):.4e}, "
          f"greedy mismatches {out['greedy_token_mismatches']}")


if __name__ == "__main__":
    main()

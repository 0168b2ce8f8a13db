"""Write tests/golden/hash_tables.json: per-workload hash metadata from the oracle.

The primes and offsets follow the EngramLayout rule, and the multipliers follow
compute_hash_multipliers. Both rules are on the vLLM page
"vllm.models.deepseek_v41.common.engram" and both are computed by the oracle
only. A real model ships these tables as checkpoint metadata, so here they are
stored data that the HIP path reads as input.

Run from the repository root:  python tests/golden/make_hash_tables.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle                      # noqa: E402
from workloads import SPECS        # noqa: E402  (sizes only)


def tables() -> dict:
    out = {}
    for spec in SPECS:
        primes, offsets = oracle.engram_layout(len(spec.layer_ids), spec.max_ngram,
                                               spec.n_heads, spec.engram_vocab_size)
        mult = oracle.hash_multipliers(spec.layer_ids, spec.max_ngram,
                                       spec.compressed_vocab)
        out[str(spec.index)] = {
            "name": spec.name,
            "layer_ids": list(spec.layer_ids),
            "max_ngram": spec.max_ngram,
            "n_heads": spec.n_heads,
            "pad_id": spec.pad_id,
            "compressed_vocab": spec.compressed_vocab,
            "engram_vocab_size": spec.engram_vocab_size,
            "primes": primes.tolist(),
            "offsets": offsets.tolist(),
            "multipliers": mult.tolist(),
        }
    return out


if __name__ == "__main__":
    path = os.path.join(ROOT, "tests", "golden", "hash_tables.json")
    with open(path, "w") as f:
        json.dump(tables(), f, indent=1)
        f.write("\n")
    print("wrote", path)

"""Writes tests/golden/blockhash_vs_radix.json: reused prompt tokens on the workload
traces under the token-level radix tree and under a 16-token block-hash chain.

TEST INFRASTRUCTURE ONLY: calls nothing but the oracle (oracle.episode for the tree,
oracle.blockhash for the block cache) and the seeded input generators. Comparison
requested by the page "49 · RadixAttention, eviction và cache churn", §3 (vLLM's
block-hash prefix caching at 16-token granularity against token-level matching).

Usage: python -m oracle.blockhash_report   (a few minutes; the scattered-chat decode
trace is the slow one)
"""
from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.blockhash import run_block_episode  # noqa: E402
from oracle.episode import run_episode  # noqa: E402
from workloads import config  # noqa: E402

TRACES = [(2, ""), (3, "A"), (3, "B"), (4, ""), (4, "cyclic"), (4, "grouped"), (4, "cyclic_lpf")]
OUT = os.path.join(ROOT, "tests", "golden", "blockhash_vs_radix.json")


def compare(n, variant):
    w = config(n, variant)
    r = run_episode(w)
    b = run_block_episode(w)
    rr, rt, pt = r.hits()
    br, bt, pt2 = b.hits()
    assert pt == pt2
    return {"workload": w.name, "prompt_tokens": pt,
            "radix": {"full_hits": rr, "reused_tokens": rt, "token_hit_rate": rt / pt,
                      "evicted_tokens": r.evicted_tokens_total},
            "block16": {"full_hits": br, "reused_tokens": bt, "token_hit_rate": bt / pt,
                        "evicted_tokens": 16 * b.evicted_blocks}}


def main():
    rows = []
    for n, v in TRACES:
        rows.append(compare(n, v))
        print(json.dumps(rows[-1]), flush=True)
    with open(OUT, "w") as f:
        json.dump({"source": "page '49 · RadixAttention, eviction và cache churn', §3; "
                             "written by oracle/blockhash_report.py",
                   "traces": rows}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

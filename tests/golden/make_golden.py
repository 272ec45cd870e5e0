"""Writes tests/golden/tiny_fp32_prefill.json: the oracle's selection for the
seeded tiny fp32 workload (4 q-heads / 2 kv-heads, d 64, prompt 512, C = 196).
Calls only the oracle and the seeded input generator.  The stored values are
a regression fixture for the oracle itself, not an external pin."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from kv_cache_compression_obs_amd import synth  # noqa: E402
from oracle import Config, prefill_compress_one  # noqa: E402


def main():
    w = synth.workload("tiny_fp32")
    cfg = Config(n_q_heads=4, n_kv_heads=2, d_qk=64, d_v=64, L_sink=4, K=64, L_recent=128,
                 W=16, pool=7)
    inp = synth.prefill_inputs(w, seed=1)
    q, k, v = (synth.to_f64(inp[n])[0] for n in ("q_obs", "k", "v"))
    res = prefill_compress_one(cfg, q, k, v)
    out = {
        "_about": "oracle output for synth.prefill_inputs(tiny_fp32, seed=1); written by make_golden.py",
        "sel": res.sel.tolist(),
        "slot_pos": res.slot_pos.tolist(),
        "raw_sum": [float(x) for x in res.raw.sum(axis=1)],
        "kth_pooled": [float(sorted(res.pooled[h], reverse=True)[cfg.K - 1]) for h in range(2)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_prefill.json")
    with open(path, "w") as f:
        json.dump(out, f)
        f.write("\n")


if __name__ == "__main__":
    main()

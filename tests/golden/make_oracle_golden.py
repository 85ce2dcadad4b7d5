"""Writes the stored oracle results of the two full-size configurations whose
fp64 oracle takes minutes: every sample of the batch-64 denoise, and the
18-layer Gemma-2B prefix pass over 816 real tokens followed by the 10-step
expert denoise from its cache.

Calls only the fp64 oracle (oracle/) and the seeded input generators
(vla_flow_matching_amd/synth.py); nothing here touches the HIP path.  The
GPU tests regenerate the same seeded inputs and compare against these files
(and recompute a few samples live, so a stale file fails the test).

    python tests/golden/make_oracle_golden.py b64       # pi0_bf16_b64_oracle.npz
    python tests/golden/make_oracle_golden.py prefill   # gemma2b_prefill_816_oracle.npz

Method: page 1 (vllm-omni modeling_pi0.py), sample_actions / denoise_step
for the loop and the prefix-only branch of PaliGemmaWithExpertModel.forward
(_compute_layer_prefix_only) for the cache, as the oracle implements them.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import oracle  # noqa: E402
from vla_flow_matching_amd import synth  # noqa: E402

B64_FILE = os.path.join(HERE, "pi0_bf16_b64_oracle.npz")
PREFILL_FILE = os.path.join(HERE, "gemma2b_prefill_816_oracle.npz")

# prefix pass: Gemma-2B decoder stack, 816 real tokens; the expert that
# denoises from its cache
PREFILL_SEED = 21
EXPERT_SEED = 22
# cache rows stored per layer (K and V): the first and last token, the
# boundaries of the three 256-token camera blocks and the text, and seeded
# random rows in between
PREFILL_ROWS_FIXED = [0, 1, 127, 128, 255, 256, 511, 512, 767, 768, 814, 815]
PREFILL_ROWS_RANDOM = 20


def prefill_rows(L: int = 816) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([PREFILL_SEED, 7])))
    extra = rng.choice(np.setdiff1d(np.arange(L), PREFILL_ROWS_FIXED), PREFILL_ROWS_RANDOM, replace=False)
    return np.sort(np.concatenate([PREFILL_ROWS_FIXED, extra])).astype(np.int64)


def prefill_workloads():
    pw = synth.PREFILL_WORKLOADS["paligemma_bf16_b1"].replace(name="gemma2b_bf16_816_golden", seed=PREFILL_SEED)
    ew = synth.WORKLOADS["pi0_bf16_b1"].replace(name="pi0_bf16_b1_on_gemma2b_cache", seed=EXPERT_SEED)
    return pw, ew


def make_b64() -> None:
    w = synth.WORKLOADS["pi0_bf16_b64"]
    blob = synth.make_weights(w.shape, seed=w.seed, dtype=w.dtype)
    inputs = synth.make_inputs(w)
    orc = oracle.Oracle(w.shape, blob)
    outs = []
    t0 = time.time()
    for b in range(w.batch):
        outs.append(orc.denoise_batch(inputs, w.num_steps, samples=[b])[0])
        print(f"b64 sample {b} done ({time.time() - t0:.0f} s)", flush=True)
    np.savez_compressed(B64_FILE, actions=np.stack(outs).astype(np.float32), workload=np.array(w.name),
                        num_steps=np.array(w.num_steps))
    print("wrote", B64_FILE)


def make_prefill() -> None:
    pw, ew = prefill_workloads()
    t0 = time.time()
    pblob = synth.make_prefill_weights(pw.shape, seed=pw.seed, dtype=pw.dtype)
    pin = synth.make_prefill_inputs(pw)
    cache = oracle.PrefillOracle(pw.shape, pblob).prefill_batch(pin)  # [depth][2][1][L][1][dh]
    del pblob
    print(f"prefill done ({time.time() - t0:.0f} s)", flush=True)
    cache = cache.reshape(cache.shape[0], 2, 1, pw.prefix_len, -1)
    eblob = synth.make_weights(ew.shape, seed=ew.seed, dtype=ew.dtype)
    ein = synth.make_inputs(ew)
    ein["prefix_kv"] = cache.reshape(cache.shape[:4] + (1, -1))
    ein["valid_len"] = pin["valid_len"]
    actions = oracle.Oracle(ew.shape, eblob).denoise_batch(ein, ew.num_steps)
    print(f"denoise done ({time.time() - t0:.0f} s)", flush=True)
    rows = prefill_rows(pw.prefix_len)
    np.savez_compressed(PREFILL_FILE, rows=rows, cache_rows=cache[:, :, 0, rows, :].astype(np.float32),
                        actions=actions.astype(np.float32), prefill_seed=np.array(PREFILL_SEED),
                        expert_seed=np.array(EXPERT_SEED))
    print("wrote", PREFILL_FILE)


if __name__ == "__main__":
    which = sys.argv[1:] or ["b64", "prefill"]
    for name in which:
        {"b64": make_b64, "prefill": make_prefill}[name]()

"""One worker process of the multi-process contention test
(test_gpu_contention.py): runs its own seeded decode workload through
dsa_decode_step many times on the shared GPU, checks every repetition bit for
bit against its first result and that result against the oracle (scores
within the score gate, indices exact on its own scores, attention within
tolerance), and saves the last result for the parent to compare with a
single-process run.

    python contention_worker.py --worker W --steps N --out FILE.npz
"""
import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def workload(w: int):
    from sparse_attention_14_amd import inputs
    if w % 2 == 0:
        return inputs.small(inputs.DECODE_128K_FP8, name=f"c{w}", wid=700 + w, batch=2, seq_len=(12000, 24000))
    return inputs.small(inputs.PAGED_DECODE, name=f"c{w}", wid=700 + w, batch=3, seq_len=(5000, 15000))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--worker", type=int, required=True)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    import numpy as np
    import torch

    import oracle
    from sparse_attention_14_amd import device, inputs

    from gpu_util import TOL, check_attention, check_scores, gpu_decode_step

    p = inputs.make_problem(workload(a.worker))
    dp = device.upload(p)
    print(f"worker {a.worker}: case {p.name} batch {p.n_q} lens {p.q_len.tolist()}", flush=True)
    first = gpu_decode_step(dp)
    ws = first[4]
    for s in range(a.steps):
        r = gpu_decode_step(dp, ws=ws)
        for x, y, what in zip(first[:4], r[:4], ("out", "lse", "scores", "indices")):
            if not torch.equal(x.view(torch.int32), y.view(torch.int32)):
                raise SystemExit(f"worker {a.worker}: step {s}: {what} differs from the first step")
    out, lse, scores, idx = (t.cpu().numpy() for t in first[:4])
    ref_scores = oracle.index_scores(p.q_idx, p.q_idx_dtype, p.w_idx, p.keys, p.q_seq, p.q_len)
    check_scores(p, scores, ref_scores)
    ref_idx, _ = oracle.topk(scores.astype(np.float64), p.q_len, p.topk)
    if not np.array_equal(idx, ref_idx):
        raise SystemExit(f"worker {a.worker}: kept indices differ from the oracle's top-k of its scores")
    ref_o, ref_l, _ = oracle.mla_attend(p.q_mla, p.q_mla_dtype, p.latent, p.kv_lora, idx, p.q_seq, p.softmax_scale)
    check_attention(out, lse, ref_o, ref_l, TOL[p.latent.dtype])
    np.savez(a.out, out=out, lse=lse, scores=scores, idx=idx)
    print(f"worker {a.worker}: ok after {a.steps + 1} steps", flush=True)


if __name__ == "__main__":
    main()

"""Every request and KV head of a full-size workload against the oracle.

Not collected by pytest (it takes minutes at full size); run it directly on
a GPU host:  python tests/full_coverage.py gemma3_mixed 0 48
It builds the workload's caches, runs the step once (three request
micro-batches, as the bench does), then checks layers [first, last) of every
request with the same checks as the parity tests: min-max bounds
value-exact, scores within tolerance, top-K exact on the GPU's own scores
and within the near-tie band against the oracle's, outputs within
max-abs 1e-2 / rel-L2 5e-3.  Prints one line per layer."""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)
import torch  # noqa: E402

from gpu_harness import Stats, assert_output_bar, check_layer  # noqa: E402
from non_uniform_sparse_amd.pipeline import DecodeStep  # noqa: E402
from non_uniform_sparse_amd.workloads import make_workload  # noqa: E402


def main(name: str, l0: int, l1: int) -> None:
    wl = make_workload(name)
    step = DecodeStep(wl, device="cuda", microbatches=3)
    qs = step.queries()
    step.run(qs)
    torch.cuda.synchronize()
    tot = Stats()
    for l in range(l0, l1):
        t = time.time()
        st = Stats()
        check_layer(step, l, qs[l], range(wl.cfg.b), st)
        for k in ("minmax_checked", "scores_checked", "topk_heads", "out_rows"):
            setattr(tot, k, getattr(tot, k) + getattr(st, k))
        tot.band_events += st.band_events
        tot.score_err_max = max(tot.score_err_max, st.score_err_max)
        tot.out_max_abs = max(tot.out_max_abs, st.out_max_abs)
        tot.out_sq_err += st.out_sq_err
        tot.out_sq_ref += st.out_sq_ref
        print(f"layer {l}: {time.time() - t:.1f}s heads {st.topk_heads} "
              f"max-abs {st.out_max_abs:.2e} score err/A {st.score_err_max:.2e} "
              f"band {len(st.band_events)}", flush=True)
    assert_output_bar(tot, f"{name} layers {l0}..{l1 - 1} all requests")


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]), int(sys.argv[3]))

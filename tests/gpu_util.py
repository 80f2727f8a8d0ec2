"""Shared pieces of the GPU parity tests: the library (loaded or the test fails), cached
workloads, and the near-tie rules for discrete outputs."""

import functools
import sys

import numpy as np

from oracle.formats import bf16_round
from speculative_verify_decode_amd import binding as B
from speculative_verify_decode_amd import synth
from speculative_verify_decode_amd.runner import StepRunner

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_lib():
    # On a machine with a GPU the HIP path must load: a missing library is a failure, not a skip.
    return B.lib()


@functools.lru_cache(maxsize=2)
def workload(name):
    say(f"[gpu-test] generating workload {name}")
    return synth.make_workload(name)


def runner(wk):
    require_lib()
    return StepRunner(wk, DEV)


def route_flags(z, k, rel=1e-4):
    """Rows whose top k+1 logits hold an adjacent gap below rel * (1 + max|z|)."""
    z = np.asarray(z, dtype=np.float64)
    srt = -np.sort(-z, axis=1)[:, : k + 1]
    gaps = srt[:, :-1] - srt[:, 1:]
    thr = rel * (1.0 + np.abs(z).max(axis=1, keepdims=True))
    return np.any(gaps < thr, axis=1)


def valid_topk(z_row, ids_row, k, slack):
    """The chosen ids are a top-k of z up to `slack` (for flagged rows)."""
    kth = -np.sort(-z_row)[k - 1]
    return len(set(ids_row.tolist())) == k and np.all(z_row[ids_row] >= kth - slack)


def check_route_stage_a(z_ref, gpu_ids, k):
    """Expert ids bit-exact on every row that is not a near tie; flagged rows must still
    hold a valid top-k.  Returns the flagged row indices."""
    flagged = route_flags(z_ref, k)
    from oracle import topk_route
    ref_ids, _ = topk_route(z_ref, k)
    for t in range(z_ref.shape[0]):
        if flagged[t]:
            slack = 1e-4 * (1 + np.abs(z_ref[t]).max())
            assert valid_topk(z_ref[t], gpu_ids[t], k, slack), (t, gpu_ids[t], ref_ids[t])
        else:
            assert np.array_equal(gpu_ids[t], ref_ids[t]), (t, gpu_ids[t], ref_ids[t], z_ref[t])
    return np.nonzero(flagged)[0]


def head_flags(exact_logits, rel=2.0 ** -20):
    """Rows where an exact logit within one bf16 step of the row's rounded maximum lies
    within `rel` (relative) of a bf16 rounding midpoint: a last-bit difference in the
    accumulation may legitimately move it across."""
    lg = np.asarray(exact_logits, dtype=np.float64)
    rb = bf16_round(lg)
    m = rb.max(axis=1, keepdims=True)
    _, e = np.frexp(np.abs(lg))
    ulp = np.ldexp(1.0, e - 8)
    mid_dist = np.abs(np.abs(lg) / ulp - np.floor(np.abs(lg) / ulp) - 0.5) * ulp
    near_mid = mid_dist < rel * np.abs(lg) + 1e-30
    near_top = rb >= m - 2 * ulp
    return np.any(near_mid & near_top, axis=1)


def teacher_forcer(gpu_ids, rel, record):
    """A route_override for the oracle: rows whose own top-k gap is below rel*(1+max|z|)
    take the GPU's ids (and are recorded); the rest keep the oracle's ids."""
    def f(z, ids):
        flagged = route_flags(z, ids.shape[1], rel)
        out = np.array(ids, copy=True)
        out[flagged] = gpu_ids[flagged]
        record.append(np.nonzero(flagged)[0])
        return out
    return f


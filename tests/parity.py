"""Parity helpers: run the HIP library through the C-ABI and the fp64 oracle on
the same seeded inputs, and compare at the stated tolerances.

Tolerances (bf16 storage, fp32 accumulation): max |d logit| <= 2e-2 and
max |d prob| <= 2e-3; argmax identical, except that a question may pick the
other option when the oracle's gap between the two picks is no larger than the
two options' measured logit errors together (a near tie, reported)."""
import sys
import time

import numpy as np

from oracle import head as O

TOL_LOGIT = 2e-2
TOL_PROB = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_outputs(case, records=None):
    t = time.time()
    out = O.forward(case.weights, case.head, case.batch, lambda ids: case.table[np.asarray(ids, np.int64)],
                    records=records)
    say(f"  oracle {case.spec.name} records={'all' if records is None else list(records)}: {time.time() - t:.1f}s")
    return out


def select(batch, records, lg, pr, am):
    """Outputs of a subset of records from whole-batch outputs."""
    L, P, A = [], [], []
    for r in records:
        q0, q1 = int(batch.q_offsets[r]), int(batch.q_offsets[r + 1])
        o0, o1 = int(batch.o_offsets[q0]), int(batch.o_offsets[q1])
        L.append(lg[o0:o1])
        P.append(pr[o0:o1])
        A.append(am[q0:q1])
    return np.concatenate(L), np.concatenate(P), np.concatenate(A)


def local_offsets(batch, records):
    offs = [0]
    for r in records:
        for q in range(int(batch.q_offsets[r]), int(batch.q_offsets[r + 1])):
            offs.append(offs[-1] + int(batch.o_offsets[q + 1] - batch.o_offsets[q]))
    return np.array(offs)


def compare(name, gpu, ref, o_offsets, tol_logit=TOL_LOGIT, tol_prob=TOL_PROB):
    lg, pr, am = gpu
    lo, po, ao = ref
    assert lg.shape == lo.shape and am.shape == ao.shape
    assert np.isfinite(lg).all() and np.isfinite(pr).all()
    dl = np.abs(lg - lo)
    dp = np.abs(pr - po)
    margins = O.top2_margin(lo, o_offsets)
    say(f"  {name}: NO={len(lo)} NQ={len(ao)} max|dlogit|={dl.max():.3e} max|dprob|={dp.max():.3e} "
        f"min oracle top-2 margin={margins.min():.3e}")
    assert dl.max() <= tol_logit, f"{name}: max |d logit| {dl.max()}"
    assert dp.max() <= tol_prob, f"{name}: max |d prob| {dp.max()}"
    near = 0
    for q in range(len(ao)):
        if am[q] != ao[q]:
            o0 = o_offsets[q]
            gap = lo[o0 + ao[q]] - lo[o0 + am[q]]
            err = dl[o0 + ao[q]] + dl[o0 + am[q]]
            assert gap <= err, f"{name}: question {q} argmax {am[q]} != {ao[q]} with oracle gap {gap} > {err}"
            near += 1
    if near:
        say(f"  {name}: {near} near-tie argmax differences (oracle gap within the measured logit error)")
    return dl.max(), dp.max()

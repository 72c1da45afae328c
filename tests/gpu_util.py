"""Helpers shared by the GPU parity tests: host<->device copies, the oracle
acceptance check with a readable failure message, the oracle's whole product
over all host cores, and guard canaries."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

TOL = 1e-4   # |gpu - ref| <= TOL * sum_k |a_ik b_kj|, per element


def torch():
    import torch as t
    return t


def dev(a):
    t = torch()
    a = np.ascontiguousarray(a)
    return t.from_numpy(a).to("cuda")


def host(t_):
    torch().cuda.synchronize()
    return t_.detach().cpu().numpy()


def assert_close(gpu, ref, bound, what=""):
    ok, worst, idx = oracle.check(gpu, ref, bound, TOL)
    if not ok:
        g = np.asarray(gpu, np.float64)
        msg = "%s: worst |gpu-ref|/bound = %.3g at %s (gpu %r, ref %r, bound %r)" % (
            what, worst, idx, g[idx], np.asarray(ref)[idx], np.asarray(bound)[idx])
        raise AssertionError(msg)
    return worst


def guarded(rows, cols, pad=64, fill=np.float32(1.2345e9)):
    """A device buffer with `pad` canary elements before and after a rows x cols
    output; returns (whole buffer, output view)."""
    t = torch()
    n = rows * cols
    buf = t.full((n + 2 * pad,), float(fill), dtype=t.float32, device="cuda")
    view = buf[pad:pad + n].view(rows, cols) if n else buf[pad:pad].view(rows, cols)
    return buf, view


def canaries_intact(buf, pad=64, fill=np.float32(1.2345e9)):
    h = host(buf)
    return bool(np.all(h[:pad] == fill) and np.all(h[-pad:] == fill))


def oracle_product(layout, A, B):
    """The oracle's whole product op(A).op(B) (layout "nn", "tn" with A stored
    K x M, or "nt" with B stored N x K), its output rows split into blocks
    over every usable host core: threads calling the C oracle, which runs
    without the interpreter lock.  Each cell is the same plain dot product
    as in one call.  Returns (C, bound) as fp64 arrays."""
    fn = {"nn": oracle.gemm_nn, "tn": oracle.gemm_tn, "nt": oracle.gemm_nt}[layout]
    M = A.shape[1] if layout == "tn" else A.shape[0]
    cores = len(os.sched_getaffinity(0))
    blocks = [b for b in np.array_split(np.arange(M), cores) if b.size]

    def part(r):
        return fn(A[:, r[0]:r[-1] + 1] if layout == "tn" else A[r[0]:r[-1] + 1], B)
    with ThreadPoolExecutor(max_workers=len(blocks)) as pool:
        parts = list(pool.map(part, blocks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])

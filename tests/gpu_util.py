"""Helpers shared by the GPU parity tests: host<->device copies, the oracle
acceptance check with a readable failure message, and guard canaries."""
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

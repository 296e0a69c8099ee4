"""Comparison rules between the HIP library and the CPU oracle.

* Greedy and tree outputs: bit-exact.
* Sampling: outputs must equal the oracle's, except where the first
  differing decision sits at an oracle decision margin below MARGIN:
  - an accept test at drafted position i with |u_i - r_i| < MARGIN, or
  - the final draw, when the token the GPU drew has positive oracle mass and
    its oracle CDF interval lies within MARGIN of the threshold u.
  Such explained disagreements are counted per sequence and, summed over all
  runs of a test, must stay below MAX_RATE of the verified positions.
"""
import numpy as np
import torch

MARGIN = 1e-6
MAX_RATE = 1e-4


def to_dev(arr, device="cuda"):
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def classify_sample(gpu_acc, gpu_out, ora_acc, ora_out, infos, margin=MARGIN):
    """Returns dict(exact, explained, unexplained=[(b, why)], sequences)."""
    gpu_acc = np.asarray(gpu_acc)
    gpu_out = np.asarray(gpu_out)
    res = dict(exact=0, explained=0, unexplained=[], sequences=len(ora_acc), details=[])
    for b in range(len(ora_acc)):
        jg, jo = int(gpu_acc[b]), int(ora_acc[b])
        if jg == jo and np.array_equal(gpu_out[b], ora_out[b]):
            res["exact"] += 1
            continue
        info = infos[b]
        if jg < 0 or np.any(gpu_out[b, : max(jg, 0) + 1] < 0):
            res["unexplained"].append((b, f"invalid GPU output j={jg} out={gpu_out[b].tolist()}"))
            continue
        if jg != jo:
            i = min(jg, jo)
            tests = {t[0]: t for t in info["tests"]}
            _, u, r = tests[i]
            if abs(u - r) < margin:
                res["explained"] += 1
                res["details"].append((b, "accept", i, abs(u - r)))
            else:
                res["unexplained"].append((b, f"accept at {i}: gpu j={jg} oracle j={jo} |u-r|={abs(u - r):.3e}"))
            continue
        if not np.array_equal(gpu_out[b, :jg], ora_out[b, :jo]) or np.any(gpu_out[b, jg + 1:] != -1):
            res["unexplained"].append((b, "accepted prefix or padding differs"))
            continue
        y = int(gpu_out[b, jg])
        F, t, w = info["draw"]["F"], info["draw"]["t"], info["w"]
        if not (0 <= y < len(F)) or not w[y] > 0:
            res["unexplained"].append((b, f"draw: token {y} has no oracle mass"))
            continue
        lo = F[y - 1] if y > 0 else 0.0
        hi = F[y]
        dist = 0.0 if lo <= t < hi else min(abs(t - lo), abs(t - hi))
        if dist < margin:
            res["explained"] += 1
            res["details"].append((b, "draw", y, dist))
        else:
            res["unexplained"].append((b, f"draw: gpu {y} oracle {int(ora_out[b, jo])} distance {dist:.3e}"))
    return res

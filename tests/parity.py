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

MARGIN = 1e-6
MAX_RATE = 1e-4


def to_dev(arr, device="cuda"):
    import torch
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


def _draw_distance(info, y):
    F, t, w = info["draw"]["F"], info["draw"]["t"], info["w"]
    if not (0 <= y < len(F)) or not w[y] > 0:
        return None
    lo = F[y - 1] if y > 0 else 0.0
    hi = F[y]
    return 0.0 if lo <= t < hi else min(abs(t - lo), abs(t - hi))


def classify_tree_sample(gpu_acc, gpu_path, gpu_tok, ora_acc, ora_path, ora_tok, infos, parents, margin=MARGIN):
    """Tree sampling: equal outputs, or a first differing decision at an
    oracle margin below `margin`: an accept test (|u - r|, for the first
    child of a node and for a child tried after rejected siblings alike) or
    the final draw (as in classify_sample).  parents [B][N]."""
    res = dict(exact=0, explained=0, unexplained=[], sequences=len(ora_acc), details=[])
    for b in range(len(ora_acc)):
        ja, jo = int(gpu_acc[b]), int(ora_acc[b])
        gp, gt = np.asarray(gpu_path[b]), np.asarray(gpu_tok[b])
        if ja == jo and np.array_equal(gp, ora_path[b]) and np.array_equal(gt, ora_tok[b]):
            res["exact"] += 1
            continue
        if ja < 0 or jo < 0:
            res["unexplained"].append((b, f"validity differs: gpu {ja} oracle {jo}"))
            continue
        gpu_set = set(int(c) for c in gp[:ja])
        why = None
        for (c, u, r) in infos[b]["tests"]:
            if (u < r) != (c in gpu_set):
                if abs(u - r) < margin:
                    why = ("explained", (b, "accept", c, abs(u - r)))
                else:
                    why = ("unexplained", (b, f"test of node {c}: |u-r|={abs(u - r):.3e}"))
                break
        if why is None:
            if ja != jo or not np.array_equal(gp, ora_path[b]):
                why = ("unexplained", (b, "paths differ with every oracle test agreeing"))
            elif not np.array_equal(gt[:ja], ora_tok[b][:jo]) or np.any(gt[ja + 1:] != -1):
                why = ("unexplained", (b, "path tokens or padding differ"))
            else:
                dist = _draw_distance(infos[b], int(gt[ja]))
                if dist is not None and dist < margin:
                    why = ("explained", (b, "draw", int(gt[ja]), dist))
                else:
                    why = ("unexplained", (b, f"draw: gpu {int(gt[ja])} oracle {int(ora_tok[b][jo])} {dist}"))
        if why[0] == "explained":
            res["explained"] += 1
            res["details"].append(why[1])
        else:
            res["unexplained"].append(why[1])
    return res

"""Helpers for the GPU tests: device copies, bit views and the parity bar."""
import math
import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")
SM = float(np.float32(1.0 / math.sqrt(128)))
MAX_ABS = 2e-2        # attention parity: max-abs error
REL_L2 = 5e-3         # attention parity: relative L2 error


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(a):
    """uint16 bf16 bits (numpy) -> int16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    return t.cpu().numpy().view(np.uint16)


def f64(t):
    return oracle.bf16_bits_to_f64(bits(t))


def errs(got, ref):
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    e, r = errs(got, ref)
    say("%s: max-abs %.3e rel-L2 %.3e" % (what, e, r))
    assert e <= max_abs and r <= rel_l2, "%s: max-abs %.3e rel-L2 %.3e" % (what, e, r)
    return e, r


def assert_bf16_output(got, ref, what, rel_l2=REL_L2):
    """Bar for a result that the kernel rounds once to bf16 from an fp32 sum
    (the W8A16 linear layer): each element within 2^-7 |ref| (twice the
    half-ulp bound 2^-8 |ref| of one bf16 rounding) plus 10^-4 of the
    largest |ref| for the fp32 accumulation, and rel-L2 <= rel_l2.  An
    absolute bar does not fit here: outputs of magnitude 8 or more already
    round by up to 2^-5."""
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    d = np.abs(got - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 1e-4 * float(np.abs(ref).max())
    worst = float((d / bound).max()) if d.size else 0.0
    e, r = errs(got, ref) if d.size else (0.0, 0.0)
    say("%s: max-abs %.3e rel-L2 %.3e, worst error / element bound %.3f" % (what, e, r, worst))
    assert worst <= 1.0 and r <= rel_l2, "%s: max-abs %.3e rel-L2 %.3e worst/bound %.3f" % (what, e, r, worst)
    return e, r


def cache_tensors(H, cap):
    kc = torch.zeros((H, cap, 128), dtype=torch.int8, device=DEV)
    vc = torch.zeros((H, cap, 128), dtype=torch.int8, device=DEV)
    ks = torch.zeros((H, cap), dtype=torch.float32, device=DEV)
    vs = torch.zeros((H, cap), dtype=torch.float32, device=DEV)
    return kc, vc, ks, vs


def cache_from_oracle(kc, vc, ks, vs):
    return dev(kc), dev(vc), dev(ks), dev(vs)

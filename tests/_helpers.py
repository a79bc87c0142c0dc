"""Helpers for the GPU parity tests: host <-> device copies and the acceptance tolerances.

Tolerances (stated once, used by every GEMM parity test):
  * fp16 / bf16 output: |gpu - ref| <= 1e-2 + 1e-2 * |ref| for every element;
  * fp32 output:        |gpu - ref| <= 1e-4 * sqrt(K) * max |ref|.
ref is the fp64 oracle value.
"""

import numpy as np
import torch


def dev16(bits, dtype):
    """uint16 bit patterns (numpy) -> fp16/bf16 CUDA tensor holding the same bytes."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def host64(t):
    """CUDA tensor -> float64 numpy array (exact for fp16 / bf16 / fp32)."""
    return t.float().cpu().numpy().astype(np.float64)


def bits16(t):
    """fp16/bf16 CUDA tensor -> its uint16 bit patterns (numpy)."""
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# unit roundoff of the output types (half an ulp relative to the value) and half their smallest
# subnormal step
_U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "f32": 2.0 ** -24}
_TINY_OUT = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134, "f32": 2.0 ** -150}


def check_bound(gpu, ref, absprod, K, out, what=""):
    """A bound derived from the arithmetic instead of a fixed tolerance. Products of fp16 or bf16
    values are exact in fp32; an fp32 sum of K of them, in any order and whether each addition
    rounds to nearest or toward zero, errs by at most 2 K 2^-24 sum|a b| (absprod, from
    oracle.gemm.abs_products_rows); rounding to the output type then adds at most its unit roundoff
    times the value, or half its smallest subnormal step:
        |gpu - ref| <= (1 + u) 2 K 2^-24 absprod + u |ref| + tiny."""
    u, tiny = _U_OUT[out], _TINY_OUT[out]
    bound = (1 + u) * 2.0 * K * 2.0 ** -24 * absprod + u * np.abs(ref) + tiny
    err = np.abs(gpu - ref)
    ok = err <= bound
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements beyond the derived bound; first at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    return float(np.max(err / bound))


def check_tol(gpu, ref, K, f32_out=False, what=""):
    err = np.abs(gpu - ref)
    if f32_out:
        bound = 1e-4 * np.sqrt(K) * np.max(np.abs(ref))
        ok = err <= bound
    else:
        bound = 1e-2 + 1e-2 * np.abs(ref)
        ok = err <= bound
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements out of tolerance; first at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r}")
    return float(np.max(err))


def check_gemm(gpu, a, b, dtype, K, out, rows=None, what=""):
    """Both bars against the oracle for a GEMM result: the generic tolerance and the derived bound.
    gpu: the result (all rows, or the sampled ``rows``) as fp64; a, b: the input bit patterns;
    out: the output type ("f16", "bf16" or "f32")."""
    from oracle import gemm as og
    rows = np.arange(np.asarray(a).shape[0]) if rows is None else np.asarray(rows)
    ref = og.gemm_rows(a, b, dtype, rows)
    check_tol(gpu, ref, K, f32_out=out == "f32", what=what)
    return check_bound(gpu, ref, og.abs_products_rows(a, b, dtype, rows), K, out, what=what)

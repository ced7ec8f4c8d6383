"""Helpers shared by the GPU parity tests (marshalling and tolerance checks)."""
import sys

import numpy as np
import torch

import token_choice_routing_amd as tcr
from token_choice_routing_amd.layer import to_device, to_host
from workloads import bf16_bits_to_f32

# Tolerances of the layer output: max-abs error relative to the oracle's RMS.
TOL_BF16 = 2e-2
TOL_F32 = 1e-5
FLIP_GAP = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def vals(a):
    """float64 values of a host array (uint16 = bf16 bit patterns)."""
    a = np.asarray(a)
    return bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_close_rms(got, ref, tol, what=""):
    got, ref = vals(got), np.asarray(ref, dtype=np.float64)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    scale = rms(ref)
    say(f"  {what}: max|err| = {err:.3e}, RMS(ref) = {scale:.3e}, ratio = {err / max(scale, 1e-300):.3e} (tol {tol:g})")
    assert err <= tol * scale, f"{what}: max abs error {err} > {tol} * RMS {scale}"


def output_floor(ref, bf16):
    """max |round(ref) - ref| / RMS(ref): the least whole-tensor error ratio any output in
    the layer's storage type can have (ref rounded once to bf16, or to float32)."""
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    if bf16:
        from workloads import bf16_round
        r = bf16_bits_to_f32(bf16_round(ref.astype(np.float32))).astype(np.float64)
    else:
        r = ref.astype(np.float32).astype(np.float64)
    return float(np.abs(r - ref).max()) / max(rms(ref), 1e-300)


def assert_layer_close(got, ref, tol, bf16, what=""):
    """Layer-output tolerance: max |got - ref| <= tol * RMS(ref) over the whole tensor,
    the stated rule, wherever the rule is reachable with room to spare: the exact output
    rounded once to the output type (output_floor) stays below 0.9 tol. Where it does not
    (the modality-skewed workload: vision rows ~17x larger than text rows, floor 3.9%;
    copy null slots, whose copied tokens dominate the largest outputs), no output in that
    type meets the whole-tensor rule, and each token row is held to tol * RMS(row)
    instead. The floors of the benchmark workloads are computed on the CPU in
    tests/test_tolerance_floor.py. Both ratios are printed."""
    fl = output_floor(ref, bf16)
    if fl >= 0.9 * tol:
        say(f"  {what}: output floor {fl:.3e} >= 0.9 tol: per-row rule")
        assert_rows_close(got, ref, tol, what)
        return
    assert_close_rms(got, ref, tol, what)
    g, r = vals(got), np.asarray(ref, dtype=np.float64)
    if r.size:
        rr = np.sqrt((r * r).mean(axis=1))
        ratio = np.abs(g - r).max(axis=1) / np.where(rr > 0, rr, 1.0)
        say(f"  {what}: output floor {fl:.3e}; per-row max|err|/RMS(row) = {ratio.max():.3e}")


def assert_rows_close(got, ref, tol, what=""):
    """Layer-output tolerance, one token row at a time: max_j |got - ref| <= tol * RMS_j(ref)
    for every row; a row whose reference is exactly zero must be exactly zero. The
    whole-tensor ratio max|err| / RMS(ref) is printed as well."""
    got, ref = vals(got), np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return
    err = np.abs(got - ref)
    row_rms = np.sqrt((ref * ref).mean(axis=1))
    row_err = err.max(axis=1)
    zero = row_rms == 0
    assert (row_err[zero] == 0).all(), f"{what}: an all-zero reference row is not exactly zero"
    ratio = np.where(zero, 0.0, row_err / np.where(zero, 1.0, row_rms))
    worst = int(np.argmax(ratio))
    say(f"  {what}: per-row max|err|/RMS(row) = {ratio.max():.3e} (row {worst}), "
        f"whole-tensor max|err|/RMS = {err.max() / max(rms(ref), 1e-300):.3e} (tol {tol:g})")
    assert ratio.max() <= tol, f"{what}: row {worst} error {row_err[worst]} > {tol} * RMS(row) {row_rms[worst]}"


def bf16_tensor(a_f32):
    from workloads import bf16_round
    return to_device(bf16_round(np.asarray(a_f32, dtype=np.float32)))


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def route_from_logits(logits_f32, N, M, K, null_kind=0):
    T = logits_f32.shape[0]
    dims = tcr.make_dims(T, 64, N, M, K, 64, 0, tcr.MOE_F32, null_kind)
    topk = empty((T, K), torch.int32)
    w = empty((T, K), torch.float32)
    nr = empty((T,), torch.int32)
    tcr.moe_route(dims, None, None, logits_in=to_device(np.ascontiguousarray(logits_f32, dtype=np.float32)),
                  topk_idx=topk, topk_w=w, n_real=nr)
    torch.cuda.synchronize()
    return to_host(topk), to_host(w), to_host(nr)

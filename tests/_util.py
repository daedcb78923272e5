"""Shared test helpers: seeded inputs, cached oracle results, comparisons."""
import functools

import numpy as np

import synth
from oracle import smconv_oracle as so


@functools.lru_cache(maxsize=None)
def config(name):
    w = synth.workload(name)
    return w, synth.make_coords(w)


@functools.lru_cache(maxsize=None)
def oracle_map(name):
    _, coords = config(name)
    return oracle_map_of(coords)


def oracle_map_of(coords):
    nbr, mask = so.build_kernel_map(coords)
    perm = so.mask_sort(mask)
    pin, pout, toff = so.compact_pairs(nbr, mask, perm)
    return dict(nbr=nbr, mask=mask, perm=perm, pair_in=pin, pair_out=pout, tap_off=toff)


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bf16_bits_of(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def assert_map_equal(got, want, label=""):
    for key in ("nbr", "mask", "perm", "pair_in", "pair_out", "tap_off"):
        g, w = np.asarray(got[key]), np.asarray(want[key])
        assert g.shape == w.shape, f"{label} {key}: shape {g.shape} != {w.shape}"
        if not np.array_equal(g.astype(np.int64), w.astype(np.int64)):
            bad = np.nonzero(g.astype(np.int64) != w.astype(np.int64))
            first = tuple(int(b[0]) for b in bad)
            raise AssertionError(f"{label} {key}: {len(bad[0])} mismatches, first at {first}: "
                                 f"got {g[first]} want {w[first]}")


def check_bf16_output(y_bits, acc_ref, label="", max_ulp=1):
    """GPU bf16 output vs the oracle accumulator.

    Required: |y - bf16(ref)| <= 2e-2 (1 + |bf16(ref)|) elementwise. Also
    checked: at most ``max_ulp`` bf16 ulps from the oracle's rounding, which
    is what a float32 accumulator differing from the float64 one only by
    summation order can produce.
    """
    ref = so.round_to_bf16(acc_ref)
    got = so.bf16_bits_to_f64(y_bits)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = 2e-2 * (1 + np.abs(ref))
    worst = np.argmax(err - bound)
    assert (err <= bound).all(), (f"{label}: bf16 tolerance exceeded at {np.unravel_index(worst, err.shape)}:"
                                  f" got {got.flat[worst]} ref {ref.flat[worst]}")
    rb = so.bf16_bits(ref).astype(np.int32)
    gb = np.asarray(y_bits, np.uint16).astype(np.int32)
    # ordered integer view of bf16 bit patterns: distance in ulps
    def ordered(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    ulp = np.abs(ordered(gb) - ordered(rb))
    assert ulp.max() <= max_ulp, f"{label}: {ulp.max()} bf16 ulps from the oracle (max {max_ulp})"


def check_f32_acc(acc_gpu, acc_ref, label=""):
    """|acc_gpu - acc_ref| <= 1e-3 (1 + |acc_ref|) elementwise, and relative L2 <= 1e-3."""
    acc_gpu = np.asarray(acc_gpu, np.float64)
    d = np.abs(acc_gpu - acc_ref)
    assert (d <= 1e-3 * (1 + np.abs(acc_ref))).all(), f"{label}: fp32 accumulator tolerance"
    nr = np.linalg.norm(acc_ref)
    if nr > 0:
        assert np.linalg.norm(acc_gpu - acc_ref) / nr <= 1e-3, f"{label}: relative L2"

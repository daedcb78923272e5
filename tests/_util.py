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
    perm = so.mask_sort(mask)[None, :]          # one group, plain order: [1, N]
    pin, pout, toff = so.compact_pairs(nbr, mask)
    return dict(nbr=nbr, mask=mask, perm=perm, pair_in=pin, pair_out=pout, tap_off=toff,
                group_rows=np.asarray([len(mask)], np.int64))


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
    """Every part of the map present in got (nbr, mask, perm, pair lists, tap_off)
    equals want, bit for bit."""
    for key in ("nbr", "mask", "perm", "group_rows", "pair_in", "pair_out", "tap_off"):
        if key not in got or key not in want:
            continue
        g, w = np.asarray(got[key]), np.asarray(want[key])
        assert g.shape == w.shape, f"{label} {key}: shape {g.shape} != {w.shape}"
        if not np.array_equal(g.astype(np.int64), w.astype(np.int64)):
            bad = np.nonzero(g.astype(np.int64) != w.astype(np.int64))
            first = tuple(int(b[0]) for b in bad)
            raise AssertionError(f"{label} {key}: {len(bad[0])} mismatches, first at {first}: "
                                 f"got {g[first]} want {w[first]}")


def fp32_sum_bound(abs_ref, n_terms):
    """Rigorous bound on |float32 sum - exact| for sums of n_terms products.

    Any summation order: |fl(sum) - sum| <= gamma_n * sum|terms|, gamma_n =
    n u / (1 - n u), u = 2^-24; abs_ref is sum|x||w| per output.
    """
    u = 2.0 ** -24
    g = n_terms * u / (1 - n_terms * u)
    return g * abs_ref


def check_bf16_output(y_bits, acc_ref, label="", abs_ref=None, n_terms=None):
    """GPU bf16 output vs the oracle accumulator (float64, exact products).

    Required: |y - bf16(ref)| <= 2e-2 (1 + |bf16(ref)|) elementwise.
    With abs_ref (sum |x||w| per output) also a tight, rigorous check: the
    output is a float32 sum of n_terms products rounded to bf16, so
    |y - exact| <= gamma_n abs_ref + 2^-8 max(|y|, |exact|) + 2^-133.
    """
    ref = so.round_to_bf16(acc_ref)
    got = so.bf16_bits_to_f64(y_bits)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = 2e-2 * (1 + np.abs(ref))
    worst = np.argmax(err - bound)
    assert (err <= bound).all(), (f"{label}: bf16 tolerance exceeded at "
                                  f"{np.unravel_index(worst, err.shape)}: got {got.flat[worst]} "
                                  f"ref {ref.flat[worst]}")
    if abs_ref is not None:
        tight = (fp32_sum_bound(abs_ref, n_terms) + 2.0 ** -8 * np.maximum(np.abs(got), np.abs(acc_ref))
                 + 2.0 ** -133)
        e = np.abs(got - acc_ref)
        worst = np.argmax(e - tight)
        assert (e <= tight).all(), (f"{label}: outside the float32+bf16 rounding bound at "
                                    f"{np.unravel_index(worst, e.shape)}: got {got.flat[worst]} "
                                    f"exact {acc_ref.flat[worst]} bound {tight.flat[worst]}")


def check_f32_acc(acc_gpu, acc_ref, label="", abs_ref=None, n_terms=None):
    """|acc_gpu - acc_ref| <= 1e-3 (1 + |acc_ref|) elementwise, and relative L2 <= 1e-3.

    With abs_ref, also the rigorous float32 summation bound gamma_n sum|x||w|.
    """
    acc_gpu = np.asarray(acc_gpu, np.float64)
    d = np.abs(acc_gpu - acc_ref)
    assert (d <= 1e-3 * (1 + np.abs(acc_ref))).all(), f"{label}: fp32 accumulator tolerance"
    if abs_ref is not None:
        b = fp32_sum_bound(abs_ref, n_terms) + 2.0 ** -126
        worst = np.argmax(d - b)
        assert (d <= b).all(), (f"{label}: outside the float32 summation bound at "
                                f"{np.unravel_index(worst, d.shape)}: {d.flat[worst]} > {b.flat[worst]}")
    nr = np.linalg.norm(acc_ref)
    if nr > 0:
        assert np.linalg.norm(acc_gpu - acc_ref) / nr <= 1e-3, f"{label}: relative L2"

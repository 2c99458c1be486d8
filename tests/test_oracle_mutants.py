"""Each planted mistake in the oracle (a -DFM_ORACLE_MUTANT=<n> build of
oracle/fm_oracle.c) must be caught by at least one of the pins that guard the
function it lives in.  This shows the pins are strong enough to notice a
dropped term, a misplaced chunk, a wrong slice, an unstable sort, a wrong
gather index, a dropped gate weight and wrong activation forms.  The
every-element forms in oracle/full.py get the same treatment, with their
mistakes planted by wrapping the correct function for one test."""
import numpy as np
import pytest

import oracle as oracle_pkg
import oracle_pins as pins

MUTANTS = {
    1: ("dropped last K term in the GEMM", [pins.pin_gemm_numpy, pins.pin_gemm_bruteforce]),
    2: ("AllGather places chunks by arrival slot", [pins.pin_ag_concat,
                                                    pins.pin_ag_arrival_invariance,
                                                    pins.pin_golden_mlp]),
    3: ("ReduceScatter adds into the wrong slice", [pins.pin_rs_sum_of_slices,
                                                    pins.pin_rs_split_k_bruteforce,
                                                    pins.pin_golden_mlp]),
    4: ("gate weight dropped from the combine", [pins.pin_moe_layer1_token_loop,
                                                 pins.pin_moe_identical_experts_chain,
                                                 pins.pin_golden_moe]),
    5: ("unstable placement inside an expert", [pins.pin_route_numpy, pins.pin_golden_moe]),
    6: ("pair id used as the gathered token", [pins.pin_moe_layer0_bruteforce,
                                               pins.pin_golden_moe]),
    7: ("GELU without its factor 1/2", [pins.pin_act_gelu]),
    8: ("SiLU with sigmoid(-x)", [pins.pin_act_silu]),
}


@pytest.mark.parametrize("mid", sorted(MUTANTS), ids=[MUTANTS[m][0] for m in sorted(MUTANTS)])
def test_pins_catch_mutant(mid):
    mut = oracle_pkg.load(mutant=mid)
    assert mut._L.or_mutant_id() == mid
    what, guards = MUTANTS[mid]
    caught = []
    for pin in guards:
        try:
            pin(mut)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {mid} ({what})"


# Planted mistakes in the every-element forms (oracle/full.py), each made by
# wrapping the correct function for one test: the pin_full_* pins must catch
# every one.
def _pair_id_as_token(orig):
    # X[pair id] in place of X[pair id // topk] (rows past T wrap around)
    return lambda dt, X, W1, sp, off, topk: orig(dt, np.concatenate([X] * topk), W1, sp, off, 1)


def _gate_weight_dropped(orig):
    return lambda dt, H, W2, ids, wts, sp, off, seed, e0: orig(
        dt, H, W2, ids, np.ones_like(np.asarray(wts)), sp, off, seed, e0)


def _wrong_slice(orig):
    def f(dt, A, W, seeds):
        r = orig(dt, A, W, seeds)
        return r[1:] + r[:1]
    return f


def _other_format(orig):
    return lambda dt, bits: orig(1 - dt, bits)


def _chunks_by_arrival(orig):
    return lambda dt, chunks, W: orig(dt, list(chunks)[::-1], W)


def _transposed_product(orig):
    # the contraction's second operand read transposed where it is square
    def f(dt, A, B):
        return orig(dt, A, B.T.copy() if B.shape[0] == B.shape[1] else B)
    return f


FULL_MUTANTS = {
    "pair id used as the gathered token": ("moe_layer0", _pair_id_as_token),
    "gate weight dropped from the combine": ("moe_layer1", _gate_weight_dropped),
    "ReduceScatter slices rotated": ("gemm_rs", _wrong_slice),
    "inputs decoded in the other 16-bit format": ("decode", _other_format),
    "AllGather stacks chunks in reverse": ("ag_gemm", _chunks_by_arrival),
    "square second operand transposed": ("gemm", _transposed_product),
}


@pytest.mark.parametrize("what", sorted(FULL_MUTANTS))
def test_full_form_pins_catch_mutant(monkeypatch, what):
    from oracle import full
    attr, make = FULL_MUTANTS[what]
    monkeypatch.setattr(full, attr, make(getattr(full, attr)))
    o = oracle_pkg.load()
    caught = []
    for pin in pins.ALL_PINS:
        if not pin.__name__.startswith("pin_full_"):
            continue
        try:
            with np.errstate(invalid="ignore"):
                pin(o)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {what}"

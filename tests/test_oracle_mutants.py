"""Each planted mistake in the oracle (a -DFM_ORACLE_MUTANT=<n> build of
oracle/fm_oracle.c) must be caught by at least one of the pins that guard the
function it lives in.  This shows the pins are strong enough to notice a
dropped term, a misplaced chunk, a wrong slice, an unstable sort, a wrong
gather index, a dropped gate weight and wrong activation forms."""
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

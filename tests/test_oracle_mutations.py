"""Mutation check of the oracle's pins, on the CPU.

Each case plants one plausible mistake in the oracle (by patching one of its
functions for the duration of the case) and runs the pins that should catch
it; the case passes when at least one of them fails.  A mistake that no pin
catches would mean the oracle is not pinned at that point.  Nothing here runs
on the GPU or touches the HIP library.
"""
import numpy as np
import pytest

from oracle import bf16, e4m3, gemm, quant

import test_oracle_codecs as codecs_pins
import test_oracle_gemm as gemm_pins
import test_oracle_quant as quant_pins

# some planted mistakes overflow on purpose (bf16 truncation through fp32)
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _fails(pins):
    """True when at least one pin raises."""
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_orig_dequant = quant.dequantize_rows


def _encode_ties_away(t):
    """E4M3 encode with ties away from zero instead of ties to even."""
    t = np.asarray(t, np.float64)
    a = np.abs(t)
    pos = e4m3.DECODE_TABLE[:0x7F]
    hi = np.minimum(np.searchsorted(pos, a, side="left"), 0x7E)
    lo = np.where(pos[hi] == a, hi, np.maximum(hi - 1, 0))
    pick_hi = (pos[hi] - a) <= (a - pos[lo])
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(t).astype(np.uint8) << 7)


MUTATIONS = {
    # quotient x * RN(1/s) instead of the correctly rounded x / s
    "reciprocal_quotient": ("oracle.quant.encode_scaled",
                            lambda x, s: e4m3.encode(np.clip(
                                (np.asarray(x, np.float32) * (np.float32(1) / np.asarray(s, np.float32))).astype(
                                    np.float32), -448, 448)),
                            [quant_pins.test_division_cases_bit_exact]),
    # scale amax * RN(1/448) instead of amax / 448
    "reciprocal_scale": ("oracle.quant.block_scale",
                         lambda amax, ue8m0: (lambda s: quant.ue8m0_round_up(s) if ue8m0 else s)(
                             (np.maximum(np.asarray(amax, np.float32), quant.AMAX_FLOOR) *
                              (np.float32(1) / np.float32(448))).astype(np.float32)),
                         [quant_pins.test_division_cases_bit_exact]),
    # quotient rounded straight to E4M3 (float64), skipping the fp32 rounding
    "no_fp32_quotient": ("oracle.quant.encode_scaled",
                         lambda x, s: e4m3.encode(np.clip(
                             np.asarray(x, np.float64) / np.asarray(s, np.float64), -448, 448)),
                         [quant_pins.test_division_cases_bit_exact]),
    # ties away from zero in the E4M3 encoder
    "e4m3_ties_away": ("oracle.e4m3.encode", _encode_ties_away,
                       [codecs_pins.test_encode_ties_to_even_at_every_midpoint,
                        quant_pins.test_golden_quant_examples]),
    # UE8M0 scale rounded down instead of up
    "ue8m0_round_down": ("oracle.quant.ue8m0_round_up",
                         lambda s: (np.asarray(s, np.float32).view(np.uint32) & np.uint32(0x7F800000)).view(
                             np.float32),
                         [quant_pins.test_scale_closed_forms, quant_pins.test_golden_quant_examples]),
    # amax floor dropped (an all-zero block divides by zero)
    "no_amax_floor": ("oracle.quant.block_scale",
                      lambda amax, ue8m0: (np.asarray(amax, np.float32) / np.float32(448)).astype(np.float32),
                      [quant_pins.test_scale_closed_forms, quant_pins.test_golden_quant_examples]),
    # bf16 rounding by truncation (overflow to inf in the fp32 cast is part of the mistake)
    "bf16_truncate": ("oracle.bf16.round_to_bf16_bits",
                      lambda x: (np.asarray(x, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(
                          np.uint16),
                      [codecs_pins.test_bf16_hand_picked_cases, codecs_pins.test_bf16_matches_torch_on_fp32_values]),
    # bf16 rounding through fp32 first (double rounding)
    "bf16_via_fp32": ("oracle.bf16.round_to_bf16_bits",
                      lambda x, _f=bf16.round_to_bf16_bits: _f(np.asarray(x, np.float64).astype(np.float32)),
                      [codecs_pins.test_bf16_hand_picked_cases]),
    # K-block scales applied in reverse K order
    "kblock_scale_order": ("oracle.gemm.dequantize_rows",
                           lambda c, s: _orig_dequant(c, np.asarray(s)[:, ::-1]),
                           [gemm_pins.test_single_nonzero_k_block, gemm_pins.test_identity_b_picks_the_right_scales]
                           + [lambda s=s: gemm_pins.test_brute_force_matches_exact_rationals(s) for s in range(6)]),
    # B scale of the 128-row block picked by row % 128 instead of row // 128
    "b_scale_index": ("oracle.gemm._b_row_scales",
                      lambda sfb, rows: np.asarray(sfb, np.float64)[np.asarray(rows) % np.asarray(sfb).shape[0]],
                      [gemm_pins.test_identity_b_picks_the_right_scales]),
    # a spurious factor on the sum
    "spurious_factor": ("oracle.gemm.gemm_nt_fp64",
                        lambda a, sfa, b, sfb, _f=gemm.gemm_nt_fp64: _f(a, sfa, b, sfb) * (1 + 2.0 ** -12),
                        [gemm_pins.test_all_ones_gives_k,
                         gemm_pins.test_unit_scales_reduce_to_int64_matmul_and_torch_rounding]),
    # a dropped K block (the last one)
    "dropped_kblock": ("oracle.gemm.dequantize_rows",
                       lambda c, s: np.concatenate([_orig_dequant(c, s)[:, :-128],
                                                    np.zeros((np.asarray(c).shape[0], 128))], axis=1),
                       [gemm_pins.test_all_ones_gives_k]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    target, replacement, pins = MUTATIONS[name]
    monkeypatch.setattr(target, replacement)
    assert _fails(pins), f"no pin catches the planted mistake {name!r}"


def test_pins_pass_without_mutation():
    # the same pins, unpatched, must pass (so a failure above is the mutation's)
    seen = set()
    for _, _, pins in MUTATIONS.values():
        for pin in pins:
            if id(pin) not in seen:
                seen.add(id(pin))
                pin()

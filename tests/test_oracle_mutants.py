"""The pins must reject plausible mistakes in the oracle.

Each case compiles a copy of oracle/gspn_oracle.c with one deliberate error
(a dropped term, a wrong sign or index, a transposed operand, a wrong scan
order), points the oracle module at it, and requires that at least one pin
of the oracle's pin tests fails.  Everything runs on the CPU.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_backward as bpins
import test_oracle_ex as xpins
import test_oracle_ex_backward as xbpins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")

MUTANTS = [
    ("taps mirrored in the mix", "                        long q = p + k - 1;",
     "                        long q = p - k + 1;"),
    ("out-of-line taps kept in the sum", "? sigmoid(raw[k]) : 0.0", "? sigmoid(raw[k]) : sigmoid(raw[k])"),
    ("eps added instead of clamping", "double S = sum > eps ? sum : eps;", "double S = sum + eps;"),
    ("clamp missing", "double S = sum > eps ? sum : eps;", "double S = sum;"),
    ("lambda dropped", "double bx = lp[r * W + c] * xp[r * W + c];", "double bx = xp[r * W + c];"),
    ("u dropped", "op[r * W + c] = up[r * W + c] * h;", "op[r * W + c] = h;"),
    ("BU scans downwards, LR leftwards", "int forward = (dir == DIR_TD || dir == DIR_LR);",
     "int forward = (dir == DIR_TD || dir == DIR_BU);"),
    ("propagation term dropped", "h = mix + bx;", "h = bx;"),
    ("sigmoid sign flipped", "exp(-z)", "exp(z)"),
    ("only three directions summed", "for (int d = 0; d < 4; ++d)", "for (int d = 0; d < 3; ++d)"),
    ("taps read mirrored along the line", "raw[k] = wp[k * npix + i * L + p];",
     "raw[k] = wp[k * npix + i * L + (L - 1 - p)];"),
    ("taps read from the transposed plane", "raw[k] = wp[k * npix + i * L + p];",
     "raw[k] = wp[k * npix + p * NL + i];"),
    # gradient (oracle.prop2d_backward)
    ("adjoint uses the forward tap map", "long q = p - k + 1;", "long q = p + k - 1;"),
    ("adjoint seed without u", "double v = up[r * W + c] * gyp[r * W + c];",
     "double v = gyp[r * W + c];"),
    ("normalisation Jacobian without the mean term", "(gwn[k] - dot) / T", "gwn[k] / T"),
    ("clamp branch differentiated as unclamped", "gwn[k] / eps;", "(gwn[k] - dot) / eps;"),
    ("sigmoid derivative dropped", "gz = gsk * s[k] * (1.0 - s[k]);", "gz = gsk * s[k];"),
    ("tap gradient paired with the older adjoint line", "gwn[k] = gn[p] * hl[iprev * L + q];",
     "gwn[k] = g[p] * hl[iprev * L + q];"),
    ("gu without gy", "gu[pl * npix + e] = gyp[e] * hs[e];", "gu[pl * npix + e] = hs[e];"),
    ("gx scaled by x", "gx[pl * npix + e] = lp[e] * gs[e];", "gx[pl * npix + e] = xp[e] * gs[e];"),
    # tap groups and chunked scans (oracle.prop2d_ex)
    ("reverse segments restart at their first spatial line",
     "return i == NL - 1 || (i + 1) % Lc == 0;", "return i == NL - 1 || i % Lc == 0;"),
    ("forward segments restart one line late", "if (fwd) return i % Lc == 0;",
     "if (fwd) return i == 0 || i % Lc == 1;"),
    ("segment length rounded down", "long Lc = (NL + k_chunk - 1) / k_chunk;",
     "long Lc = NL > k_chunk ? NL / k_chunk : 1;"),
    ("channel groups interleaved", "ch / cpg) * 3 * npix;", "ch % G) * 3 * npix;"),
    ("segments never restart", "if (!restart) {", "if (step > 0) {"),
    # gradient of the extended operator (oracle.prop2d_ex_backward)
    ("restart lines keep tap gradients", "int reads_before = !restarts_segment(i, NL, seg, fwd);",
     "int reads_before = step > 0;"),
    ("adjoint flows back across segment starts",
     "int after_reads_i = step < NL - 1 && !restarts_segment(after, NL, seg, fwd);",
     "int after_reads_i = step < NL - 1;"),
    ("adjoint cut at the wrong line",
     "step < NL - 1 && !restarts_segment(after, NL, seg, fwd);",
     "step < NL - 1 && !restarts_segment(i, NL, seg, fwd);"),
    ("group tap gradient overwritten, not summed", "gtg[(long)k * npix + i * L + p] += gs_k",
     "gtg[(long)k * npix + i * L + p] = gs_k"),
    ("gradient's forward ignores restarts", "int restart = restarts_segment(i, NL, seg, fwd);",
     "int restart = step == 0;"),
    ("grouped gu from the adjoint sum", "gu[pl * npix + e] = gys[e] * hsum[e];",
     "gu[pl * npix + e] = gys[e] * gsum[e];"),
]


def _checks():
    yield lambda: pins.test_normalize_closed_forms()
    yield lambda: pins.test_normalize_invariants(5, 7)
    yield lambda: pins.test_worked_2x2()
    for d in range(4):
        yield lambda d=d: pins.test_scan_matches_dense_map(3, 5, d)
        yield lambda d=d: pins.test_single_position_lines_are_running_sums(d)
        yield lambda d=d: pins.test_identity_and_shift_taps(d)
        yield lambda d=d: pins.test_row_stochastic_constant_propagates(d, 6, 9)
    yield lambda: pins.test_direction_symmetries(4, 7)
    yield lambda: pins.test_prop2d_is_sum_of_directions()
    yield lambda: bpins.test_backward_matches_directional_finite_differences(3, 5, 0)
    yield lambda: bpins.test_backward_adjoint_identities(3, 4)
    yield lambda: bpins.test_backward_clamp_branch()
    yield lambda: bpins.test_backward_first_line_and_dropped_taps_have_zero_gradient()
    yield lambda: xpins.test_ex_reduces_to_prop2d(3, 5)
    yield lambda: xpins.test_grouped_taps_equal_expanded_per_channel_taps(6, 2)
    yield lambda: xpins.test_groups_are_contiguous_channel_blocks()
    yield lambda: xpins.test_chunked_scan_equals_global_scans_of_segments(7, 9, 3)
    yield lambda: xpins.test_one_line_segments_reduce_to_4_u_lambda_x(7)
    yield lambda: xbpins.test_ex_backward_reduces_to_per_channel_backward()
    yield lambda: xbpins.test_ex_backward_matches_finite_differences(2, 3)
    yield lambda: xbpins.test_ex_backward_shared_taps_sum_the_replicated_gradients(2, 3)
    yield lambda: xbpins.test_ex_backward_one_line_segments_closed_form()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique: " + old
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", str(mut), "-o", str(lib), "-lm"])
    oracle.use_library(str(lib))
    failed = 0
    try:
        for check in _checks():
            try:
                check()
            except AssertionError:
                failed += 1
    finally:
        oracle.use_library(None)
    assert failed > 0, "no pin rejects the mutant: " + name


def test_unmutated_oracle_passes_every_check():
    for check in _checks():
        check()

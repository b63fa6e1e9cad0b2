"""The pins are strong enough: every plausible slip planted in a copy of the
oracle's C source fails at least one pin.  CPU only; the committed oracle is
never modified (each mutant is compiled from a patched copy in a temp dir)."""
import subprocess

import pytest

import oracle
import pins

# (name, original text, replacement) -- each a single plausible mistake.
MUTANTS = [
    ("offset_xy_swapped", "p->offset_scale * offk[1];", "p->offset_scale * offk[0];"),
    ("offset_scale_dropped_y", "+ p->offset_scale * offk[1]", "+ offk[1]"),
    ("pad_sign", "ho * p->stride_h - p->pad_h", "ho * p->stride_h + p->pad_h"),
    ("dilation_dropped", "i * p->dil_h", "i"),
    ("stride_dropped", "wo * p->stride_w", "wo"),
    ("point_order_transposed", "int64_t i = q / p->kw, j = q % p->kw;",
     "int64_t i = q % p->kh, j = q / p->kh;"),
    ("bilinear_weight_flipped", "wy[a] = 1.0 - fabs(py - (double)cy[a]);",
     "wy[a] = fabs(py - (double)cy[a]);"),
    ("second_corner_dropped", "cx[1] = cx[0] + 1;", "cx[1] = cx[0];"),
    ("softmax_not_normalised", "m[k] /= sum;", "m[k] /= 1.0;"),
    ("softmax_skipped", "if (!p->softmax) {", "if (1) {"),
    ("edge_clamp_not_zero_pad", "return 0.0;\n    return x[",
     "{ yy = yy < 0 ? 0 : (yy >= p->h ? p->h - 1 : yy);"
     " xx = xx < 0 ? 0 : (xx >= p->w ? p->w - 1 : xx); }\n    return x["),
    ("group_channel_base_dropped", "feat(p, x, n, cy[a], cx[e], g * Cg + c)",
     "feat(p, x, n, cy[a], cx[e], c)"),
    ("grad_kink_sign", "const double dsy[2] = {-1.0, 1.0}", "const double dsy[2] = {1.0, -1.0}"),
    ("grad_offset_scale_dropped", "go[0] = s * m[k] * gpx;", "go[0] = m[k] * gpx;"),
    ("grad_offset_pair_swapped", "go[1] = s * m[k] * gpy;", "go[1] = s * m[k] * gpx;"),
    ("softmax_jacobian_dropped", "gmr[k] = m[k] * (gm[k] - dot);", "gmr[k] = gm[k];"),
    ("grad_input_mask_dropped", "m[k] * wy[a] * wx[e] * gyr[c];", "wy[a] * wx[e] * gyr[c];"),
    ("grad_mask_gy_dropped", "gm[k] += gyr[c] * b;", "gm[k] += b;"),
    ("grad_input_corner_weight", "m[k] * wy[a] * wx[e] * gyr[c];", "m[k] * wy[a] * gyr[c];"),
    ("out_size_off_by_one", "return span / stride + 1;", "return span / stride;"),
    ("removed_point_is_the_first", "q >= (p->kh / 2) * p->kw + p->kw / 2", "q >= 0"),
    ("removed_point_is_the_last", "q >= (p->kh / 2) * p->kw + p->kw / 2", "q >= p->kh * p->kw - 1"),
    ("points_after_centre_not_shifted", "        ++q;", "        q += 0;"),
    ("centre_still_counted", "- (p->remove_center ? 1 : 0)", "- 0"),
    # the backward's branches for samples infinitely far away and NaN locations
    ("far_grad_offset_not_zero", "go[0] = s * m[k] * 0.0;", "go[0] = s * m[k];"),
    ("far_needs_both_axes", "if (!(fabs(py) < 1e15 && fabs(px) < 1e15))",
     "if (!(fabs(py) < 1e15 || fabs(px) < 1e15))"),
    ("nan_grad_mask_not_poisoned", "gm[k] = go[0] = go[1] = NAN;", "go[0] = go[1] = NAN;"),
    ("nan_grad_offset_zero", "gm[k] = go[0] = go[1] = NAN;", "gm[k] = NAN; go[0] = go[1] = 0.0;"),
    # the linear layer and the steps before and after the core
    ("linear_weight_transposed", "in[q * nin + c] * w[o * nin + c]", "in[q * nin + c] * w[c * nout + o]"),
    ("linear_bias_dropped", "double acc = b ? b[o] : 0.0;", "double acc = 0.0;"),
    ("linear_last_input_dropped", "for (int64_t c = 0; c < nin; ++c)\n                acc +=",
     "for (int64_t c = 0; c + 1 < nin; ++c)\n                acc +="),
    ("generation_branches_swapped", "ref_linear(npix, cgd, p->groups * K, guide, w_mask, b_mask, mask);",
     "ref_linear(npix, cgd, p->groups * K, guide, w_off, b_off, mask);"),
    ("generation_offset_bias_dropped", "guide, w_off, b_off, off);", "guide, w_off, NULL, off);"),
    ("projection_skipped", "ref_linear(npix, p->c, p->c, y, w_out, b_out, out);",
     "memcpy(out, y, sizeof(double) * (size_t)(npix * p->c));"),
    ("nan_location_taken_as_far", "if (isnan(py) || isnan(px))\n        return -1;",
     "if (isnan(py) || isnan(px))\n        return 0;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = oracle.SOURCE_PATH.read_text()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found in the oracle source"
    mutated = src.replace(old, new, 1)
    assert mutated != src
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib_{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                    "-o", str(so), str(c), "-lm"], check=True)
    return oracle.Oracle(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    orc = _build_mutant(tmp_path, name, old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same build recipe on the unmodified source passes all pins."""
    src = oracle.SOURCE_PATH.read_text()
    c = tmp_path / "same.c"
    so = tmp_path / "lib_same.so"
    c.write_text(src)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                    "-o", str(so), str(c), "-lm"], check=True)
    orc = oracle.Oracle(so)
    for pin in pins.ALL_PINS:
        pin(orc)

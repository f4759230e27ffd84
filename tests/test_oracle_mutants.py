"""Plant plausible mistakes in a copy of the oracle's C source and check that
at least one pin catches each of them.  Runs on the CPU only (gcc)."""
import os

import pytest

import oracle
from oracle import build as obuild
from tests import pins

MUTANTS = {
    "x_transposed": ("x[(int64_t)b * Ks + k]", "x[k * B + b]"),
    "A_transposed": ("A_r[n * Ks + k]", "A_r[k * N + n]"),
    "dropped_last_k": ("for (int64_t k = 0; k < Ks; ++k)", "for (int64_t k = 0; k < Ks - 1; ++k)"),
    "wrong_sign": ("sum += p;", "sum -= p;"),
    "abs_dropped": ("sum_abs += fabs(p);", "sum_abs += p;"),
    "own_term_from_slot": ("(r == rank) ? y64[i] :", "(r == r + 1) ? y64[i] :"),
    "own_term_dropped": ("(r == rank) ? y64[i] :", "(r == rank) ? 0.0 :"),
    "peer_stride": ("? y64[i] : (double)slots[(int64_t)r * NB + i]",
                    "? y64[i] : (double)slots[(int64_t)r * N + i]"),
    "fold_stride": ("            acc = acc + slots[(int64_t)r * NB + i];\n        out[i] = acc;",
                    "            acc = acc + slots[(int64_t)r * W + i];\n        out[i] = acc;"),
    "y_index": ("y64[n * B + b] = sum;", "y64[(int64_t)b * N + n] = sum;"),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "fold_reversed": ("for (int r = 0; r < W; ++r)\n            acc = acc + slots",
                      "for (int r = W - 1; r >= 0; --r)\n            acc = acc + slots"),
    "fold_starts_at_slot0": ("float acc = 0.0f;\n        for (int r = 0; r < W; ++r)",
                             "float acc = slots[i];\n        for (int r = 1; r < W; ++r)"),
    "fold_in_double": ("        float acc = 0.0f;\n        for", "        double acc = 0.0;\n        for"),
    "out_skips_first_rank": ("for (int r = 0; r < W; ++r) {\n            double term",
                             "for (int r = 1; r < W; ++r) {\n            double term"),
    "rms_mean_over_n_minus_1": ("sqrt(ssq / (double)N + eps)", "sqrt(ssq / (double)(N - 1) + eps)"),
    "rms_eps_dropped": ("sqrt(ssq / (double)N + eps)", "sqrt(ssq / (double)N)"),
    "rms_sqrt_dropped": ("1.0 / sqrt(ssq / (double)N + eps)", "1.0 / (ssq / (double)N + eps)"),
    "rms_bias_subtracted": ("out[n * B + b] + add", "out[n * B + b] - add"),
    "rms_weight_dropped": ("* inv64[b] * wn", "* inv64[b]"),
    "rms_one_column": ("double v = (double)z[n * B + b];", "double v = (double)z[n * B];"),
    "rms_z_in_double": ("float add = bias ? bias[n] : 0.0f;\n            z[n * B + b] = out[n * B + b] + add;",
                        "float add = bias ? bias[n] : 0.0f;\n            z[n * B + b] = (float)((double)out[n * B + b] + (double)add + 1e-9);"),
    "scale_other_order": ("float v = z[n * B + b] * inv[b];\n            if (w)\n                v = v * w[n];",
                          "float v = w ? z[n * B + b] * (inv[b] * w[n]) : z[n * B + b] * inv[b];"),
    "scale_in_double": ("float v = z[n * B + b] * inv[b];\n            if (w)\n                v = v * w[n];",
                        "float v = (float)((double)z[n * B + b] * (double)inv[b] * (w ? (double)w[n] : 1.0));"),
    "rne_truncates": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)(u >> 16);"),
    "rne_ties_away": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)((u + 0x8000u) >> 16);"),
    "two_shot_no_tile_round": ("return (per_rank + 15) / 16 * 16;", "return per_rank;"),
    "two_shot_round_down": ("return (per_rank + 15) / 16 * 16;", "return per_rank / 16 * 16 + 16 * (per_rank < 16);"),
    "two_shot_owner_off_by_one": ("int64_t owner = n / cr;", "int64_t owner = (n + 1) / cr;"),
    "two_shot_copies_slot": ("out[i] = gathered[i];", "out[i] = slots[(int64_t)rank * NB + i];"),
    "two_shot_fold_reversed": ("for (int r = 0; r < W; ++r)\n                    acc = acc + slots",
                               "for (int r = W - 1; r >= 0; --r)\n                    acc = acc + slots"),
    "two_shot_skips_own": ("for (int r = 0; r < W; ++r)\n                    acc = acc + slots",
                           "for (int r = 0; r < W; ++r)\n                    if (r != rank) acc = acc + slots"),
    "moe_weight_transposed": ("bf16_bits_to_double(xr[k]) * bf16_bits_to_double(wr[k])",
                              "bf16_bits_to_double(xr[k]) * bf16_bits_to_double(Wd[(int64_t)e * H * F + (k % H) * F + n % F])"),
    "moe_expert_ignored": ("const uint16_t *wr = Wd + ((int64_t)e * H + n) * F;",
                           "const uint16_t *wr = Wd + ((int64_t)0 * H + n) * F;"),
    "moe_len_transposed": ("int64_t n_rows = len[e * W + s];", "int64_t n_rows = len[(s * ne + e) % (W * ne)];"),
    "moe_in_off_transposed": ("int64_t src = in_off[e * W + s];", "int64_t src = in_off[(s * ne + e) % (W * ne)];"),
    "moe_dst_transposed": ("int64_t dst = dst_off[s * ne + e];", "int64_t dst = dst_off[(e * W + s) % (W * ne)];"),
    "moe_dropped_last_row": ("for (int64_t i = 0; i < n_rows; ++i) {", "for (int64_t i = 0; i < n_rows - 1; ++i) {"),
    "moe_dropped_last_k": ("for (int64_t k = 0; k < F; ++k) {", "for (int64_t k = 0; k < F - 1; ++k) {"),
    "moe_dest_rank_ignored": ("int64_t orow = (int64_t)s * rows_out + dst + i;", "int64_t orow = dst + i;"),
    "moe_first_row_only": ("const uint16_t *xr = X + (src + i) * F;", "const uint16_t *xr = X + src * F;"),
    "moe_abs_dropped": ("acc_abs += fabs(q);", "acc_abs += q;"),
    "moe_overlap_unchecked": ("if (written[orow])\n                    return -2;\n", ""),
    "bf16_fold_in_bf16": ("            sum = sum + v;\n",
                          "            sum = sum + v;\n            { uint32_t t; memcpy(&t, &sum, 4);"
                          " t = (t + 0x7FFFu + ((t >> 16) & 1u)) & 0xFFFF0000u; memcpy(&sum, &t, 4); }\n"),
    "bf16_fold_reversed": ("            uint32_t word = (uint32_t)slots[(int64_t)r * NB + i] << 16;",
                           "            uint32_t word = (uint32_t)slots[(int64_t)(W - 1 - r) * NB + i] << 16;"),
    "bf16_fold_widen_shift": ("            uint32_t word = (uint32_t)slots[(int64_t)r * NB + i] << 16;",
                              "            uint32_t word = (uint32_t)slots[(int64_t)r * NB + i] << 15;"),
    "bf16_fold_stride": ("            uint32_t word = (uint32_t)slots[(int64_t)r * NB + i] << 16;",
                         "            uint32_t word = (uint32_t)slots[(int64_t)r * W + i] << 16;"),
    "bf16_fold_starts_at_slot0": ("        float sum = 0.0f;\n        for (int r = 0; r < W; ++r) {",
                                  "        float sum = 0.0f;\n        for (int r = 0; r < W; ++r) {\n            if (r == 0) sum = -0.0f;"),
    "bf16_fold_skips_last": ("        for (int r = 0; r < W; ++r) {\n            uint32_t word",
                             "        for (int r = 0; r < W - 1; ++r) {\n            uint32_t word"),
    "bf16_out_truncates": ("        out[i] = f32_to_bf16_rne(in[i]);",
                           "        { uint32_t t; memcpy(&t, &in[i], 4); out[i] = (uint16_t)(t >> 16); }"),
    "nan_branch_dropped": ("if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)\n        return (uint16_t)((u >> 16) | 0x0040u);\n", ""),
}


@pytest.fixture(scope="module")
def source():
    with open(obuild.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique/found"
    src = tmp_path / f"mutant_{name}.c"
    src.write_text(source.replace(old, new))
    lib = obuild.build(str(src), str(tmp_path / f"libmutant_{name}.so"),
                       extra_flags=["-Wno-error"])
    failed = pins.failing_pins(oracle.load(lib))
    assert failed, f"no pin catches mutant {name}"


def test_unmutated_copy_passes(source, tmp_path):
    src = tmp_path / "copy.c"
    src.write_text(source)
    lib = obuild.build(str(src), str(tmp_path / "libcopy.so"))
    assert pins.failing_pins(oracle.load(lib)) == []
    assert os.path.exists(lib)

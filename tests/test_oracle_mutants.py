"""Plant mistakes in copies of the oracle (on the CPU) and check that the pins
in test_oracle.py catch every one of them.

Each mutant is a one-token edit of oracle.c of the kind a slip would make: a
dropped scale, a transposed operand, a wrong sign, an off-by-one, a missing
normalisation, a head offset forgotten.  The mutant is compiled with gcc into a
temporary directory and swapped in for the real library while the pins run.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_scale": ("s_buf[j] = scale * dot;", "s_buf[j] = dot;"),
    "transposed_qk": ("load_elem(kb, dtype, key_rows[j] * k_stride + head_off + c);",
                      "load_elem(kb, dtype, key_rows[j] * k_stride + head_off + (d - 1 - c));"),
    "wrong_sign_exp": ("s_buf[j] = exp(s_buf[j] - mx);", "s_buf[j] = exp(mx - s_buf[j]);"),
    "no_normalise": ("double p = s_buf[j] / denom;", "double p = s_buf[j];"),
    "no_head_offset_v": ("out[c] += p * load_elem(vb, dtype, key_rows[j] * v_stride + head_off + c);",
                         "out[c] += p * load_elem(vb, dtype, key_rows[j] * v_stride + c);"),
    "offset_off_by_one": ("int64_t start = cu_seqlens[b];",
                          "int64_t start = cu_seqlens[b] - (b > 0);"),
    "pack_skip_first": ("for (int32_t n = 0; n < N; ++n) {\n            if (keep",
                        "for (int32_t n = 1; n < N; ++n) {\n            if (keep"),
    "pack_keep_is_one": ("if (keep[(int64_t)b * N + n] != 0) {", "if (keep[(int64_t)b * N + n] == 1) {"),
    "unpack_off_by_one": ("for (int64_t t = 0; t < T; ++t)", "for (int64_t t = 1; t < T; ++t)"),
    "padded_ignores_mask": ("const uint8_t* ok = keep + (int64_t)b * N;", "const uint8_t* ok = NULL;"),
    "bf16_decode_shift": ("uint32_t w = ((uint32_t)bits) << 16;", "uint32_t w = ((uint32_t)bits) << 15;"),
    "repack_gather_not_composed": ("gather_out[t_out] = gather_in[t];", "gather_out[t_out] = (int32_t)t;"),
    "repack_skips_image_start": ("for (int64_t t = cu_in[b]; t < cu_in[b + 1]; ++t) {",
                                 "for (int64_t t = cu_in[b] + 1; t < cu_in[b + 1]; ++t) {"),
    "repack_keep_is_one": ("            if (keep[t] != 0) {", "            if (keep[t] == 1) {"),
    "rows_image_lookup_off_by_one": ("        while (!(cu_seqlens[b] <= row && row < cu_seqlens[b + 1]))",
                                     "        while (!(cu_seqlens[b] <= row && row <= cu_seqlens[b + 1]))"),
    "rows_keys_from_row_on": ("            rows_buf[j] = first + j;",
                              "            rows_buf[j] = row + j;"),
}

PINS = [
    pins.test_bf16_decode_exhaustive_matches_torch,
    pins.test_pack_golden,
    lambda: pins.test_pack_matches_flatnonzero(0, 0.5),
    pins.test_unpack_roundtrip_and_sentinel,
    pins.test_attn_golden_worked_example,
    pins.test_attn_length_one_returns_v_row,
    pins.test_attn_zero_query_or_zero_scale_gives_mean_of_v,
    pins.test_attn_constant_v_and_identical_keys,
    pins.test_attn_probability_rows_sum_to_one,
    pins.test_attn_bounded_by_v_and_no_leakage,
    lambda: pins.test_attn_brute_force_tiny([4, 1, 5], 2, 8),
    lambda: pins.test_attn_matches_torch_sdpa_fp64("bf16"),
    pins.test_padded_kept_rows_equal_ragged_and_dropped_rows_match_masked_sdpa,
    lambda: pins.test_repack_equals_pack_of_the_composed_mask(0, 0.5, 0.5),
    pins.test_repack_keep_all_is_identity_and_keep_none_is_empty,
    pins.test_repack_brute_force_per_image,
    pins.test_attn_rows_match_torch_sdpa_on_sampled_rows,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found: %s" % name
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        csrc = os.path.join(tmp, "oracle.c")
        with open(csrc, "w") as f:
            f.write(text.replace(old, new))
        lib = os.path.join(tmp, "liboracle_mutant.so")
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", csrc, "-o", lib, "-lm"])
        saved = oracle._load()
        oracle._lib = oracle._bind(lib)
        caught = []
        try:
            for pin in PINS:
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught.append(getattr(pin, "__name__", "lambda"))
        finally:
            oracle._lib = saved
        assert caught, "no pin caught mutant %s" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


# ---- the ViT block reference (Python): the same idea, one-token slips in a
# copy of oracle/vit_block.py, loaded in place of the module while the block
# pins run.
import importlib.util  # noqa: E402
import sys  # noqa: E402

from oracle import vit_block  # noqa: E402

BLOCK_SRC = vit_block.__file__
BLOCK_MUTANTS = {
    "ln_unbiased_variance": ("var = ((x - mean) ** 2).mean(axis=1, keepdims=True)",
                             "var = ((x - mean) ** 2).sum(axis=1, keepdims=True) / (x.shape[1] - 1)"),
    "ln_eps_outside_root": ("return (x - mean) / np.sqrt(var + eps) * gamma + beta",
                            "return (x - mean) / (np.sqrt(var) + eps) * gamma + beta"),
    "no_first_residual": ("x1 = x + a @ W[\"w_proj\"] + P[\"b_proj\"]", "x1 = a @ W[\"w_proj\"] + P[\"b_proj\"]"),
    "k_from_v_block": ("k = qkv[s:e, C + h * d:C + (h + 1) * d]",
                       "k = qkv[s:e, 2 * C + h * d:2 * C + (h + 1) * d]"),
    "transposed_proj": ("x1 = x + a @ W[\"w_proj\"] + P[\"b_proj\"]", "x1 = x + a @ W[\"w_proj\"].T + P[\"b_proj\"]"),
    "gelu_erf_scale": ("np.vectorize(math.erf)(x / math.sqrt(2.0))", "np.vectorize(math.erf)(x / 2.0)"),
    "ln2_on_x": ("h2 = layernorm(x1, P[\"ln2_gamma\"]", "h2 = layernorm(x, P[\"ln2_gamma\"]"),
    "second_residual_from_x": ("return x1 + m @ W[\"w_fc2\"] + P[\"b_fc2\"]",
                               "return x + m @ W[\"w_fc2\"] + P[\"b_fc2\"]"),
    "block_gelu_tanh": ("eps: float = 1e-6, gelu_form: str = \"erf\"", "eps: float = 1e-6, gelu_form: str = \"tanh\""),
}
BLOCK_PINS = [
    pins.test_layernorm_golden,
    pins.test_gelu_forms_against_the_normal_cdf_table,
    pins.test_block_attention_step_matches_the_c_oracle,
    pins.test_block_with_zero_weights_is_the_identity,
    pins.test_block_matches_torch_transformer_encoder_layer_fp64,
    lambda: pins.test_block_brute_force_tiny("erf"),
    lambda: pins.test_block_brute_force_tiny("tanh"),
]


@pytest.mark.parametrize("name", sorted(BLOCK_MUTANTS))
def test_block_pins_catch_planted_mistake(name):
    old, new = BLOCK_MUTANTS[name]
    text = open(BLOCK_SRC).read()
    assert text.count(old) == 1, "mutation site not found: %s" % name
    tmp = tempfile.mkdtemp(prefix="block_mutant_")
    try:
        path = os.path.join(tmp, "vit_block_mutant.py")
        with open(path, "w") as f:
            f.write(text.replace(old, new))
        spec = importlib.util.spec_from_file_location("vit_block_mutant", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        saved = pins.vb
        pins.vb = mod
        caught = []
        try:
            for pin in BLOCK_PINS:
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught.append(getattr(pin, "__name__", "lambda"))
        finally:
            pins.vb = saved
        assert caught, "no pin caught mutant %s" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
        sys.modules.pop("vit_block_mutant", None)

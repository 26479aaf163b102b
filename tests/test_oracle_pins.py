"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""
import os
import subprocess

import pytest

import oracle
import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle.load())


# Plausible mistakes planted in a copy of oracle.c; each must make some pin fail.
MUTATIONS = [
    ("rope_term_dropped", "for (int d = 0; d < ORC_D_QK; ++d)\n                    acc += qh[d]",
     "for (int d = 0; d < ORC_D_LATENT; ++d)\n                    acc += qh[d]"),
    ("scale_block_interleaved", "4 * (d / 128)", "4 * (d % 4)"),
    ("v_reads_shifted_dims", "o[d] += w * xb[(size_t)t * ORC_D_QK + d];",
     "o[d] += w * xb[(size_t)t * ORC_D_QK + d + ORC_D_ROPE];"),
    ("softmax_scale_dropped", "sco[t] = sc * acc;", "sco[t] = acc;"),
    ("lse_base2", "m + log(L)", "m + log2(L)"),
    ("mask_off_by_one", "i >= ctx_len[b]", "i > ctx_len[b]"),
    ("row_in_page_wrong", "return page * ORC_PAGE + i % ORC_PAGE;", "return page * ORC_PAGE + (i + 1) % ORC_PAGE;"),
    ("logical_page_wrong", "int64_t lp = i / ORC_PAGE;", "int64_t lp = i % max_pages;"),
    ("e4m3_bias", "e - 7)", "e - 8)"),
    ("e4m3_subnormal", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    ("softmax_sign", "exp(sco[t] - m)", "exp(m - sco[t])"),
    ("normalisation_dropped", "o[d] /= L;", "o[d] /= 1.0;"),
    ("scales_read_from_rope", "row + ORC_D_LATENT + 4 * (d / 128)", "row + ORC_D_LATENT + 16 + 4 * (d / 128)"),
    ("rope_offset_wrong", "row + ORC_D_LATENT + 16 + 2 * k", "row + ORC_D_LATENT + 2 * k"),
    ("bf16_row_pairs_swapped", "u16_le(row + 2 * d)", "u16_le(row + 2 * (d ^ 1))"),
    ("q_request_head_transposed", "q[((size_t)b * H + h) * ORC_D_QK + d]", "q[((size_t)h * B + b) * ORC_D_QK + d]"),
    ("page_bound_unchecked", "if (page < 0 || page >= pool_pages)", "if (page < 0)"),
    ("masked_rows_not_zeroed", "memset(dst, 0, (size_t)rb);", "memset(dst, 1, (size_t)rb);"),
    ("empty_lse_zero", "lse[(size_t)b * H + h] = -INFINITY;", "lse[(size_t)b * H + h] = 0.0;"),
    # the cache producer
    ("e4m3_ties_away", "double m = nearbyint((a / ldexp(1.0, e - 1) - 1.0) * 8.0);",
     "double m = round((a / ldexp(1.0, e - 1) - 1.0) * 8.0);"),
    ("e4m3_no_saturation", "if (E > 15 || (E == 15 && m > 6.0)) {", "if (E > 15) {"),
    ("e4m3_subnormal_truncated", "nearbyint(a * 512.0)", "floor(a * 512.0)"),
    ("bf16_truncates", "a = nearbyint(a / ldexp(1.0, ulp_exp)) * ldexp(1.0, ulp_exp);",
     "a = trunc(a / ldexp(1.0, ulp_exp)) * ldexp(1.0, ulp_exp);"),
    ("append_scale_off", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 447.0f : 1.0f"),
    ("append_zero_block_scale", "? amax / 448.0f : 1.0f;", "? amax / 448.0f : 0.5f;"),
    ("append_page_unchecked", "if (page < 0 || pool_pages <= page)", "if (page < 0)"),
    ("append_row_in_page_wrong", "(page * ORC_PAGE + p % ORC_PAGE) * rb", "(page * ORC_PAGE + p / ORC_PAGE) * rb"),
    # the top-k indexer
    ("indexer_relu_dropped", "(dot > 0.0 ? dot : 0.0)", "dot"),
    ("indexer_tie_order_reversed", "return (a[1] < b[1]) ? -1 : (a[1] > b[1]);", "return (a[1] > b[1]) ? -1 : (a[1] < b[1]);"),
    ("indexer_weight_dropped", "acc += (double)w[(size_t)b * HI + j] * ", "acc += 1.0 * "),
    ("indexer_padding_zero", ": -1;", ": 0;"),
    ("indexer_select_page_unchecked", "if (!(page >= 0 && page < pool_pages))", "if (page < 0)"),
    ("indexer_ctx_inclusive", "for (int64_t s = 0; s < ctx; ++s) {", "for (int64_t s = 0; s <= ctx && s < npos; ++s) {"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mutated), "-o", str(so), "-lm"], check=True)
    lib = oracle.load(str(so))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"

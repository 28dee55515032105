"""Mutation check of the oracle's pins (CPU).

Each mutant is the oracle's C source with one plausible mistake planted by a
textual edit: a wrong tie rule, a dropped term or sign, a transposed operand,
an off-by-one exponent bias, a wrong bit or byte order, a wrong counter.  Each
is compiled on its own and the oracle's pin tests run against it in a child
process (FP4Q_ORACLE_LIB points the oracle loader at the mutant).  Every
mutant must make at least one pin fail; a surviving mutant is a hole in the
pins.  Every edit must match the source exactly once, so a change to the
oracle that silently disarms a mutant fails here too.

Not planted: rewrites that are equal in exact arithmetic and differ only in
rounding order (for example the order of the RHT butterfly stages); that
order is a reading of the pages and is not pinned by them.  Likewise not
planted in the matrix product: one permutation of the K elements applied to
both operands alike (say, reading the two nibbles of a byte the other way
round), which leaves every result unchanged.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp4_oracle.c")
PINS = ["codecs", "encode", "quantize", "philox_rht", "gemm"]

# name -> (pin file expected to catch it, run first; [(exact text, replacement), ...])
MUTANTS = {
    # element grids
    "grid_subnormal_step": ("codecs", [("if (e == 0) return m * 0.5;", "if (e == 0) return m * 1.0;")]),
    "grid_exponent_bias": ("codecs", [("return ldexp(1.0 + m * 0.5, e - 1);", "return ldexp(1.0 + m * 0.5, e);")]),
    "uniform_grid_as_e1m2": ("codecs", [("if (grid == ORC_UNIFORM) return (double)k;",
                              "if (grid == ORC_UNIFORM) return (double)k * 0.25;")]),
    # scale codecs
    "e4m3_bias": ("codecs", [("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)")]),
    "e4m3_subnormal_step": ("codecs", [("if (e == 0) v = m * ldexp(1.0, -9);", "if (e == 0) v = m * ldexp(1.0, -10);")]),
    "e4m3_encode_ties_to_odd": ("codecs", [("(d == bestd && (c & 1) == 0)", "(d == bestd && (c & 1) == 1)")]),
    "e4m3_encode_truncates": ("codecs", [("double d = fabs(orc_e4m3_decode(c) - (double)t);",
                               "double d = (double)t - orc_e4m3_decode(c); if (d < 0) continue;")]),
    "e4m3_overflow_to_nan": ("codecs", [("if (t >= 448.0f) return 0x7E;", "if (t >= 448.0f) return 0x7F;")]),
    "e8m0_bias": ("codecs", [("return ldexp(1.0, (int)code - 127);", "return ldexp(1.0, (int)code - 128);")]),
    "bf16_ties_away": ("quantize", [("if (rest > 0x8000 || (rest == 0x8000 && (keep & 1))) keep += 1;",
                        "if (rest >= 0x8000) keep += 1;")]),
    # Philox4x32-10
    "philox_multipliers_swapped": ("philox_rht", [("const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;",
                                    "const uint32_t M0 = 0xCD9E8D57u, M1 = 0xD2511F53u;")]),
    "philox_key_bump_after_round": ("philox_rht", [("if (round > 0) {", "if (round < 9) {")]),
    "philox_wrong_word": ("philox_rht", [("uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;",
                           "uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[3] ^ k0;")]),
    "philox_nine_rounds": ("philox_rht", [("round < 10;", "round < 9;")]),
    "philox_byte_order_transposed": ("philox_rht", [("return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;",
                                      "return (w[j & 3] >> (8 * (j >> 2))) & 0xFFu;")]),
    # RHT16
    "rht_sign_bits_high_half": ("philox_rht", [("return w[0] & 0xFFFFu;", "return w[0] >> 16;")]),
    "rht_missing_quarter": ("philox_rht", [("float v = orc_mul32(a[j], 0.25f);", "float v = a[j];")]),
    "rht_difference_reversed": ("philox_rht", [("float d = orc_sub32(a[i], a[i + h]);", "float d = orc_sub32(a[i + h], a[i]);")]),
    "rht_signs_after_butterfly": ("philox_rht", [
        ("if (!inverse && ((signs >> j) & 1)) a[j] = -a[j];", "if (inverse && ((signs >> j) & 1)) a[j] = -a[j];"),
        ("if (inverse && ((signs >> j) & 1)) v = -v;", "if (!inverse && ((signs >> j) & 1)) v = -v;")]),
    # tensor scale
    "ts_wrong_denominator": ("quantize", [("float denom = rn32(orc_grid_max(cfg->grid) * 448.0);",
                              "float denom = rn32(orc_grid_max(cfg->grid) * 256.0);")]),
    "ts_zero_tensor_gives_zero": ("quantize", [("if (amax == 0.0) return 1.0f;", "if (amax == 0.0) return 0.0f;")]),
    "ts_counts_infinities": ("quantize", [("if (!isfinite(y[j])) continue;", "if (isnan(y[j])) continue;")]),
    "ts_signed_amax": ("quantize", [("double a = fabs((double)y[j]);", "double a = (double)y[j];")]),
    # block scale
    "nvfp4_scale_drops_ts": ("quantize", [("float denom = orc_mul32((float)orc_grid_max(cfg->grid), ts);",
                              "float denom = orc_mul32((float)orc_grid_max(cfg->grid), 1.0f);")]),
    "nvfp4_inv_drops_ts": ("quantize", [("float S = orc_mul32((float)d, ts);", "float S = (float)d;")]),
    "nvfp4_inv_no_overflow_clamp": ("quantize", [("if (isinf(inv)) inv = FLT_MAX;", "")]),
    "nvfp4_zero_scale_keeps_values": ("quantize", [("if (S == 0.0f) return 0.0f;", "if (S == 0.0f) return 1.0f;")]),
    "mx_emax_off_by_one": ("quantize", [("e = (ex - 1) - 2;", "e = (ex - 1) - 1;")]),
    "mx_ceil_log2": ("quantize", [("e = (ex - 1) - 2;", "e = ex - 2;")]),
    "mx_no_low_clamp": ("quantize", [("if (e < -127) e = -127;", "")]),
    "mx_inv_sign": ("quantize", [("return (float)ldexp(1.0, -e);", "return (float)ldexp(1.0, e);")]),
    "block_signed_amax": ("quantize", [("else if (fabsf(y[j]) > amax) amax = fabsf(y[j]);",
                           "else if (y[j] > amax) amax = y[j];")]),
    "block_inf_counts_as_finite": ("quantize", [("if (!isfinite(y[j])) finite = 0;", "if (isnan(y[j])) finite = 0;")]),
    # element encode
    "bracket_lo_strict": ("encode", [("if (orc_grid(grid, k) <= vc) klo = k;", "if (orc_grid(grid, k) < vc) klo = k;")]),
    "rtn_tie_to_odd": ("encode", [("(klo % 2 == 0) ? klo : khi", "(klo % 2 == 1) ? klo : khi")]),
    "rtn_tie_down": ("encode", [("if (vc < mid) return (unsigned)klo;", "if (vc <= mid) return (unsigned)klo;")]),
    "rtn_tie_up": ("encode", [("if (vc > mid) return (unsigned)khi;", "if (vc >= mid) return (unsigned)khi;")]),
    "sr_up_on_equal": ("encode", [("(double)(2 * aux + 1) < 512.0 * f", "(double)(2 * aux + 1) <= 512.0 * f")]),
    "sr_threshold_half_step_low": ("encode", [("(double)(2 * aux + 1) < 512.0 * f", "(double)(2 * aux) < 512.0 * f")]),
    "sr_direction_flipped": ("encode", [("? (unsigned)khi : (unsigned)klo;", "? (unsigned)klo : (unsigned)khi;")]),
    "guided_bit_inverted": ("encode", [("((unsigned)klo & 1u) == (aux & 1u)", "((unsigned)klo & 1u) != (aux & 1u)")]),
    # quantize: random bytes, guide, packing
    "sr_counter_ignores_row0": ("quantize", [("uint64_t g = (uint64_t)(gi / 16) + cfg->sr_offset;",
                                 "uint64_t g = (uint64_t)(li / 16) + cfg->sr_offset;")]),
    "sr_offset_in_elements": ("quantize", [("uint64_t g = (uint64_t)(gi / 16) + cfg->sr_offset;",
                               "uint64_t g = (uint64_t)((gi + (int64_t)cfg->sr_offset) / 16);")]),
    "sr_group_of_32": ("quantize", [("uint64_t g = (uint64_t)(gi / 16) + cfg->sr_offset;",
                        "uint64_t g = (uint64_t)(gi / 32) + cfg->sr_offset;")]),
    "sr_counter_in_high_words": ("quantize", [("uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0, 0};",
                                  "uint32_t ctr[4] = {0, 0, (uint32_t)g, (uint32_t)(g >> 32)};")]),
    "guided_recomputes_scale": ("quantize", [("ok = orc_guided_params(cfg, scode, ts, &inv) && finite;",
                                 "orc_block_params(cfg, amax, ts, &scode, &inv); ok = finite;")]),
    "guided_bits_msb_first": ("quantize", [("aux = (gbits[li / 8] >> (li % 8)) & 1u;",
                               "aux = (gbits[li / 8] >> (7 - li % 8)) & 1u;")]),
    "guided_nvfp4_nan_scale_missed": ("quantize", [("if ((code & 0x7F) == 0x7F) return 0;", "if (code == 0xFF) return 0;")]),
    "sign_dropped": ("quantize", [("code = (signbit(y[j]) ? 8u : 0u) | k;", "code = k;")]),
    "negative_zero_loses_sign": ("quantize", [("code = (signbit(y[j]) ? 8u : 0u) | k;", "code = (y[j] < 0.0f ? 8u : 0u) | k;")]),
    "nibble_order_swapped": ("quantize", [("codes[li / 2] |= (uint8_t)(code << (4 * (li % 2)));",
                              "codes[li / 2] |= (uint8_t)(code << (4 * (1 - li % 2)));")]),
    "emitted_bit_not_lsb": ("quantize", [("if (emit) emit[li / 8] |= (uint8_t)((code & 1u) << (li % 8));",
                             "if (emit) emit[li / 8] |= (uint8_t)(((code >> 2) & 1u) << (li % 8));")]),
    # dequantize and guide cache
    "dequant_sign_dropped": ("quantize", [("} else if (code & 8) {", "} else if (code & 0) {")]),
    "dequant_block_of_16_always": ("quantize", [("unsigned s = scales[i / B];", "unsigned s = scales[i / 16];")]),
    "dequant_drops_ts": ("quantize", [("val = orc_mul32(gd, ts);", "val = gd;")]),
    "dequant_nan_payload": ("quantize", [("uint32_t qnan = 0x7FC00000u;", "uint32_t qnan = 0x7FC00001u;")]),
    "mismatch_nonadjacent_counts_sign": ("quantize", [("counts[1] += (rc & 7u) != (gc & 7u);",
                                                         "counts[1] += rc != gc;")]),
    "mismatch_counts_nonfinite_blocks": ("quantize", [("if (!finite || !orc_guided_params(cfg, rscales[r * nblk + b], ts, &inv)) continue;",
                                                       "if (!orc_guided_params(cfg, rscales[r * nblk + b], ts, &inv)) continue;")]),
    "mismatch_guide_from_wrong_bit": ("quantize", [("gbits[i / 8] |= (uint8_t)((r & 1u) << (i % 8));",
                                                    "gbits[i / 8] |= (uint8_t)(((r >> 1) & 1u) << (i % 8));")]),
    # MXFP4 matrix product
    "gemm_sign_from_wrong_bit": ("gemm", [("return (code & 8) ? -v : v;", "return (code & 4) ? -v : v;")]),
    "gemm_scale_per_16": ("gemm", [("orc_e8m0_decode(scales[i / 32])", "orc_e8m0_decode(scales[i / 16])")]),
    "gemm_nan_scale_ignored": ("gemm", [("orc_e8m0_decode(scales[i / 32])", "ldexp(1.0, (int)scales[i / 32] - 127)")]),
    "gemm_uniform_grid": ("gemm", [("orc_grid(ORC_E2M1, (int)(code & 7))", "orc_grid(ORC_UNIFORM, (int)(code & 7))")]),
    "gemm_a_transposed": ("gemm", [("av[m * K + k] * bv", "av[k * M + m] * bv")]),
    "gemm_b_reversed": ("gemm", [("bv[n * K + k];", "bv[n * K + (K - 1 - k)];")]),
    "gemm_drops_last_block": ("gemm", [("for (int64_t k = 0; k < K; ++k) {\n                const double prod",
                                        "for (int64_t k = 0; k < K - 32; ++k) {\n                const double prod")]),
    "gemm_absdot_signed": ("gemm", [("mag += fabs(prod);", "mag += prod;")]),
    "guide_pack_wrong_bit": ("quantize", [("bits[i / 8] |= (uint8_t)((code & 1u) << (i % 8));",
                              "bits[i / 8] |= (uint8_t)(((code >> 1) & 1u) << (i % 8));")]),
}


def _mutate(src, edits):
    for old, new in edits:
        n = src.count(old)
        assert n == 1, f"mutation site {old!r} found {n} times"
        src = src.replace(old, new)
    return src


def _run_mutant(name, hint, edits, tmp):
    from oracle import build as ob
    src = _mutate(open(SRC).read(), edits)
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *ob.CFLAGS, "-w", c, "-o", so, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, FP4Q_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    order = ([hint] if hint else []) + [p for p in PINS if p != hint]
    files = [f"tests/test_oracle_{p}.py" for p in order]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *files], cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-1500:]


@pytest.fixture(scope="module")
def outcomes():
    tmp = tempfile.mkdtemp(prefix="fp4q_mutants_")
    workers = max(1, min(7, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        futs = {n: ex.submit(_run_mutant, n, h, e, tmp) for n, (h, e) in MUTANTS.items()}
        res = {n: f.result() for n, f in futs.items()}
    subprocess.run(["rm", "-rf", tmp], check=False)
    return res


def test_unmutated_oracle_passes_the_pins():
    from oracle import build as ob
    with tempfile.TemporaryDirectory() as tmp:
        rc, out = _run_mutant("unmutated", None, [], tmp)
    assert rc == 0, out
    assert ob.SRC == SRC


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(outcomes, name):
    rc, out = outcomes[name]
    assert rc == 1, f"mutant {name} was not caught by any pin (exit {rc}):\n{out}"

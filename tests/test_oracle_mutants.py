"""Planted mistakes in the oracle, on the CPU: does the pin suite see them?

Each entry of MUTANTS edits one passage of oracle/lco.c (the passage must
occur exactly once, so an edit to the oracle that moves it makes this test
fail rather than silently test nothing), the edited source is compiled into a
temporary directory with the oracle's own flags, and the pins
(tests/test_oracle_pins.py) run against that library in a child process.
Every mutant must make at least one pin fail.  The mutants are the plausible
slips of each function: a dropped term, a wrong sign, index or operand, an
off-by-one, another rounding or summation order, another tie or parity rule.
Mutants that cannot change any result (a commutative swap, a count the
diagnostics never take on that path) are not listed.  FLAG_MUTANTS compile
the unedited source with other floating-point flags (contraction into fused
multiply-adds), on hosts whose CPU has them.

Nothing here touches the GPU or the files in oracle/.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lco.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, passage of lco.c, replacement)
MUTANTS = [
    # bf16 conversion
    ("bf16_truncates", "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
     "return (uint16_t)(u >> 16);"),
    ("bf16_ties_away", "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
     "return (uint16_t)((u + 0x8000u) >> 16);"),
    ("bf16_nan_kept", "return 0x7FC0; /* NaN */", "return (uint16_t)(u >> 16); /* NaN */"),
    # 1-bit compression and the vote
    ("zero_parity_flipped", "  return (int)(t & 1);\n}", "  return (int)((t + 1) & 1);\n}"),
    ("negative_zero_is_minus", "if (c < 0.0f) return 0;", "if (signbit(c)) return 0;"),
    ("pack_bit_order_reversed",
     "        bits[i * words + j / 64] |= (uint64_t)1 << (j % 64);",
     "        bits[i * words + j / 64] |= (uint64_t)1 << (63 - j % 64);"),
    ("vote_ge", "if (2 * count > W) return 1;", "if (2 * count >= W) return 1;"),
    ("tie_parity_flipped", "return (t & 1) ? 1 : -1;", "return (t & 1) ? -1 : 1;"),
    ("tie_zero_inverted", "if (tie_mode == LCO_TIE_ZERO) return 0;",
     "if (tie_mode != LCO_TIE_ZERO) return 0;"),
    ("vote_counts_minus", "if (counts) counts[j] = (uint8_t)v;",
     "if (counts) counts[j] = (uint8_t)(W - v);"),
    # the mean-|x| tree, level by level
    ("m1_quad_sequential", "acc[l] = acc[l] + ((e[0] + e[1]) + (e[2] + e[3]));",
     "acc[l] = acc[l] + (((e[0] + e[1]) + e[2]) + e[3]);"),
    ("m1_quad_pairing", "acc[l] = acc[l] + ((e[0] + e[1]) + (e[2] + e[3]));",
     "acc[l] = acc[l] + ((e[0] + e[2]) + (e[1] + e[3]));"),
    ("m1_rounds_reversed", "int64_t idx = 1024 * r + 4 * l + k;",
     "int64_t idx = 1024 * (3 - r) + 4 * l + k;"),
    ("m1_lanes_contiguous", "int64_t idx = 1024 * r + 4 * l + k;",
     "int64_t idx = 16 * l + 4 * r + k;"),
    ("m1_drops_last_element", "e[k] = idx < n ? fabs((double)a[idx]) : 0.0;",
     "e[k] = idx < n - 1 ? fabs((double)a[idx]) : 0.0;"),
    ("m1_folds_adjacent", "for (int q = 0; q < s; q++) a[q] = a[q] + a[q + s];",
     "for (int q = 0; q < s; q++) a[q] = a[2 * q] + a[2 * q + 1];"),
    ("m1_block_sequential",
     "  return (wv[0] + wv[1]) + (wv[2] + wv[3]);\n}\n\n/* Finalize",
     "  return ((wv[0] + wv[1]) + wv[2]) + wv[3];\n}\n\n/* Finalize"),
    ("m1_group_sequential",
     "  return (wv[0] + wv[1]) + (wv[2] + wv[3]);\n}\n\ndouble lco_m1_finalize",
     "  return ((wv[0] + wv[1]) + wv[2]) + wv[3];\n}\n\ndouble lco_m1_finalize"),
    ("m1_group_drops_partial", "acc[l] = l < cnt ? P[l] : 0.0;",
     "acc[l] = l < cnt - 1 ? P[l] : 0.0;"),
    ("m1_final_sequential", "p[g % LCO_M1_WAVE] = p[g % LCO_M1_WAVE] + G;", "p[0] = p[0] + G;"),
    ("m1_final_lanes_contiguous", "p[g % LCO_M1_WAVE] = p[g % LCO_M1_WAVE] + G;",
     "p[(g * LCO_M1_WAVE) / ng] = p[(g * LCO_M1_WAVE) / ng] + G;"),
    ("m1_final_plain_sum", "return fold64(p) / (double)nT;",
     "double s = 0.0;\n  for (int l = 0; l < LCO_M1_WAVE; l++) s = s + p[l];\n"
     "  return s / (double)nT;"),
    ("m1_divides_padded_count", "return fold64(p) / (double)nT;",
     "return fold64(p) / (double)(nb * LCO_M1_BLOCK);"),
    # Eq. (1)
    ("q1_rounds_half_away", "double r = rint((double)c * scale);",
     "double r = round((double)c * scale);"),
    ("q1_truncates", "double r = rint((double)c * scale);",
     "double r = trunc((double)c * scale);"),
    ("q1_asymmetric_clamp", "if (r < -(double)qmax) r = -(double)qmax;",
     "if (r < -(double)qmax - 1) r = -(double)qmax - 1;"),
    ("q1_fp32_scale", "double scale = (double)qmax / m1;",
     "double scale = (double)((float)qmax / (float)m1);"),
    ("q1_qmax_off", "  int32_t qmax = (1 << (qbits - 1)) - 1;\n  if (m1 == 0.0) return 0;",
     "  int32_t qmax = (1 << (qbits - 1));\n  if (m1 == 0.0) return 0;"),
    # the step: c, aggregation, theta, momentum, averaging
    ("c_uses_beta2", "float c = (cfg->beta1 * m[i * ldc + col]) + (omega1 * G);",
     "float c = (cfg->beta2 * m[i * ldc + col]) + (omega1 * G);"),
    ("c_omega_is_beta", "const float omega1 = 1.0f - cfg->beta1;\n  const float omega2",
     "const float omega1 = cfg->beta1;\n  const float omega2"),
    ("c_row_omega_is_beta", "float omega1 = 1.0f - cfg->beta1;\n  for (int64_t k",
     "float omega1 = cfg->beta1;\n  for (int64_t k"),
    ("step_ignores_tie_mode", "s = vote_sign(W, count, t, cfg->tie_mode);",
     "s = vote_sign(W, count, t, LCO_TIE_PARITY);"),
    ("l1_zero_sum_is_plus", "s = (int8_t)((sum > 0) - (sum < 0));",
     "s = (int8_t)((sum >= 0) - (sum < 0));"),
    ("avg_halved", "sf = (float)net / (float)W;", "sf = (float)net / (float)(2 * W);"),
    ("l1_norm_index_transposed",
     "q = lco_q1(c, m1[(int64_t)i * cfg->n_tensors + T], cfg->qbits);",
     "q = lco_q1(c, m1[(int64_t)T * cfg->W + i], cfg->qbits);"),
    ("tensor_boundary_off_by_one",
     "    const int64_t col = j - j0;\n    while (T + 1 < cfg->n_tensors && cfg->off[T + 1] <= j) T++;",
     "    const int64_t col = j - j0;\n    while (T + 1 < cfg->n_tensors && cfg->off[T + 1] < j) T++;"),
    ("theta_no_decay", "th[col] = x - (cfg->lr * (sf + (cfg->wd * x)));",
     "th[col] = x - (cfg->lr * sf);"),
    ("theta_distributed", "th[col] = x - (cfg->lr * (sf + (cfg->wd * x)));",
     "th[col] = (x - (cfg->lr * sf)) - (cfg->lr * (cfg->wd * x));"),
    ("theta_wrong_direction", "th[col] = x - (cfg->lr * (sf + (cfg->wd * x)));",
     "th[col] = x + (cfg->lr * (sf + (cfg->wd * x)));"),
    ("theta_bf16_no_decay", "float y = x - (cfg->lr * (sf + (cfg->wd * x)));",
     "float y = x - (cfg->lr * sf);"),
    ("momentum_sign", "m[i * ldc + col] = (cfg->beta2 * m[i * ldc + col]) + (omega2 * G);",
     "m[i * ldc + col] = (cfg->beta2 * m[i * ldc + col]) - (omega2 * G);"),
    ("momentum_uses_beta1", "m[i * ldc + col] = (cfg->beta2 * m[i * ldc + col]) + (omega2 * G);",
     "m[i * ldc + col] = (cfg->beta1 * m[i * ldc + col]) + (omega2 * G);"),
    ("avg_every_step", "const int avg_step = (t % cfg->sync_every) == 0;\n  const int64_t words",
     "const int avg_step = 1;\n  const int64_t words"),
    ("avg_all_tensors", "if (avg_step && cfg->sync_m && cfg->sync_m[T]) {\n      float acc = m[col];",
     "if (avg_step && cfg->sync_m) {\n      float acc = m[col];"),
    ("avg_divides_by_W_plus_1",
     "float avg = acc / (float)W;\n      for (int32_t i = 0; i < W; i++) m[i * ldc + col] = avg;",
     "float avg = acc / (float)(W + 1);\n      for (int32_t i = 0; i < W; i++) m[i * ldc + col] = avg;"),
    ("avg_reciprocal",
     "float avg = acc / (float)W;\n      for (int32_t i = 0; i < W; i++) m[i * ldc + col] = avg;",
     "float avg = acc * (1.0f / (float)W);\n      for (int32_t i = 0; i < W; i++) m[i * ldc + col] = avg;"),
    ("avg_summed_in_reverse",
     "float acc = m[col];\n      for (int32_t i = 1; i < W; i++) acc = acc + m[i * ldc + col];",
     "float acc = m[(W - 1) * ldc + col];\n"
     "      for (int32_t i = W - 2; i >= 0; i--) acc = acc + m[i * ldc + col];"),
    # fused diagnostics
    ("stats_match_counts_zero_sign", "if (s != 0 && s == ref) st[1] += 1;",
     "if (s == ref) st[1] += 1;"),
    ("stats_flip_is_match", "if (s != 0 && s == -ref) st[2] += 1;",
     "if (s != 0 && s != -ref) st[2] += 1;"),
    ("stats_sample_variance", "double var = (S2 / (double)W) - (mean * mean);",
     "double var = (S2 - ((double)W * (mean * mean))) / (double)(W > 1 ? W - 1 : 1);"),
    ("stats_variance_not_floored", "if (var < 0.0) var = 0.0;", "if (var < 0.0) var = -var;"),
    # receive side and wire formats
    ("vote_bits_tie_is_plus", "if (s > 0) sign_bits[j / 64] |= (uint64_t)1 << (j % 64);",
     "if (s >= 0) sign_bits[j / 64] |= (uint64_t)1 << (j % 64);"),
    ("apply_ignores_zero_plane", "float sf = zer ? 0.0f : (pos ? 1.0f : -1.0f);",
     "float sf = pos ? 1.0f : -1.0f;"),
    ("apply_no_decay", "th[j] = x - (cfg->lr * (sf + (cfg->wd * x)));", "th[j] = x - (cfg->lr * sf);"),
    ("pack_codes_fields_reversed",
     "int64_t bit = (j / 32) * 32 * qbits + (j % 32) * qbits;  /* bit offset in row */",
     "int64_t bit = (j / 32) * 32 * qbits + (31 - j % 32) * qbits;  /* bit offset in row */"),
    ("unpack_no_sign_extension",
     "int32_t q = (field & (1u << (qbits - 1))) ? (int32_t)field - (1 << qbits)\n"
     "                                                 : (int32_t)field;",
     "int32_t q = (int32_t)field;"),
    ("unpack_bits_zero_is_nonpositive", "if (S[j] == 0) zb |= 1ull << k;",
     "if (S[j] <= 0) zb |= 1ull << k;"),
    # the max-norm stochastic baseline and its generator
    ("splitmix_counter_from_zero", "uint64_t z = seed + (counter + 1u) * 0x9E3779B97F4A7C15ull;",
     "uint64_t z = seed + counter * 0x9E3779B97F4A7C15ull;"),
    ("splitmix_shift", "z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;",
     "z = (z ^ (z >> 28)) * 0x94D049BB133111EBull;"),
    ("sr_halves_swapped", "return (j & 1) ? (uint32_t)(r >> 32) : (uint32_t)r;",
     "return (j & 1) ? (uint32_t)r : (uint32_t)(r >> 32);"),
    ("sr_pair_mask_dropped", "(uint64_t)d + ((uint64_t)j & ~(uint64_t)1);",
     "(uint64_t)d + (uint64_t)j;"),
    ("sr_counter_off_by_one", "(uint64_t)d + ((uint64_t)j & ~(uint64_t)1);",
     "(uint64_t)d + ((uint64_t)j & ~(uint64_t)1) + 1u;"),
    ("sr_step_minus_one", "uint64_t ctr = ((uint64_t)t * (uint64_t)W + (uint64_t)i)",
     "uint64_t ctr = ((uint64_t)(t - 1) * (uint64_t)W + (uint64_t)i)"),
    ("sr_worker_major", "uint64_t ctr = ((uint64_t)t * (uint64_t)W + (uint64_t)i)",
     "uint64_t ctr = ((uint64_t)i * (uint64_t)W + (uint64_t)t)"),
    ("qinf_threshold_reversed", "double q = fl + (u < frac ? 1.0 : 0.0);",
     "double q = fl + (u > frac ? 1.0 : 0.0);"),
    ("qinf_threshold_inclusive", "double q = fl + (u < frac ? 1.0 : 0.0);",
     "double q = fl + (u <= frac ? 1.0 : 0.0);"),
    ("qinf_rounds_to_nearest", "double q = fl + (u < frac ? 1.0 : 0.0);", "double q = rint(y);"),
    ("qinf_u_24_bits", "double u = (double)r * 0x1.0p-32;", "double u = (double)(r >> 8) * 0x1.0p-24;"),
    ("qinf_loose_clamp", "if (q > (double)qmax) q = (double)qmax;",
     "if (q > (double)qmax + 1) q = (double)qmax + 1;"),
    ("minf_sums", "if (a > mx) mx = a;", "if (a > mx) mx = mx + a;"),
    ("linf_step_uses_mean_norm", "else lco_minf_all(cfg, ld, m, g, m1);",
     "else lco_m1_all(cfg, ld, m, g, m1);"),
    ("quant_linf_next_step_draws", "lco_sr_u32(cfg->seed, cfg->d, cfg->W, t, i, j));",
     "lco_sr_u32(cfg->seed, cfg->d, cfg->W, t + 1, i, j));"),
]


# (name, extra compiler flags) for the unedited source: the oracle's
# arithmetic contracted into fused multiply-adds (needs an FMA-capable host)
FLAG_MUTANTS = [
    ("contracted_to_fma", ["-ffp-contract=fast", "-mfma"]),
]


def _host_has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return any(line.startswith("flags") and " fma " in line + " " for line in f)
    except OSError:
        return False


def _cflags():
    sys.path.insert(0, ROOT)
    from oracle import build
    return build.CFLAGS


def _apply(src, find, repl):
    n = src.count(find)
    assert n == 1, f"passage occurs {n} times in lco.c: {find!r}"
    return src.replace(find, repl)


def _run_mutant(name, find, repl, src, cflags, tmp, extra=()):
    d = os.path.join(tmp, name)
    os.makedirs(d)
    c_path = os.path.join(d, "lco.c")
    with open(c_path, "w") as f:
        f.write(src if find is None else _apply(src, find, repl))
    # lco.h sits beside the original; the mutant includes it from there
    lib = os.path.join(d, "liblco.so")
    cc = subprocess.run(["gcc", *cflags, *extra, "-I", os.path.join(ROOT, "oracle"), "-o", lib,
                         c_path, "-lm"], capture_output=True, text=True)
    if cc.returncode != 0:
        return name, "does not compile", cc.stderr[-800:]
    code = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        from oracle import lco
        lco.LIB_PATH = {lib!r}
        import pytest
        sys.exit(pytest.main([{PINS!r}, "-x", "-q", "-p", "no:cacheprovider"]))
    """)
    try:
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=300, cwd=ROOT)
    except subprocess.TimeoutExpired:
        return name, "timed out", ""
    if r.returncode == 0:
        return name, "survived", r.stdout[-400:]
    m = re.search(r"FAILED \S+::(\S+)", r.stdout)
    return name, "caught", m.group(1) if m else r.stdout[-400:]


def test_mutant_passages_are_unique():
    with open(SRC) as f:
        src = f.read()
    names = [m[0] for m in MUTANTS]
    assert len(set(names)) == len(names)
    for name, find, repl in MUTANTS:
        assert find != repl, name
        assert src.count(find) == 1, f"{name}: passage occurs {src.count(find)} times"


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(SRC) as f:
        src = f.read()
    cflags = _cflags()
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    jobs = [(n, f, r, ()) for n, f, r in MUTANTS]
    if _host_has_fma():
        jobs += [(n, None, None, tuple(fl)) for n, fl in FLAG_MUTANTS]
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run_mutant(j[0], j[1], j[2], src, cflags, str(tmp_path),
                                                    j[3]), jobs))
    for name, status, detail in results:
        print(f"{name:34s} {status:10s} {detail if status == 'caught' else ''}")
    bad = [(n, s, dt) for n, s, dt in results if s != "caught"]
    assert not bad, "\n".join(f"{n}: {s}\n{dt}" for n, s, dt in bad)

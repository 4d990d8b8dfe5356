"""Mutation check of the oracle's pins, on the CPU alone.

Each mutant below is one plausible mistake planted in a copy of
``oracle/adacomp_oracle.c``: a dropped term, a wrong sign, index, operand or
comparison, a wrong reading of the optimizer or message formulas.  The copy
is compiled into pytest's ``tmp_path`` (the oracle's own library is never
touched) and the pin suite ``test_oracle_pins.py`` runs against it in a child
process through ``ADACOMP_ORACLE_LIB``.  The check passes when every mutant
fails at least one pin, and when the unmutated copy, built and loaded the same
way, passes them all.

The method each group of mutants breaks: "AdaComp (Adaptive Residual Gradient
Compression)", AIMech curated page -- the definition paragraph and the
Mechanism claim on local-bin soft threshold and mean-g_max quantization
(Algorithm 2) for the compressor; the Application claim (Table 2) for the word
widths; the Mechanism claim on self-adjusting sparsity (Figures 4-6) for the
hard local-selection baseline; the arXiv abstract of the paper for the SGD
with momentum and Adam steps that consume the decoded sum.
"""
import os
import pathlib
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import oracle

ROOT = pathlib.Path(__file__).resolve().parents[1]
SRC = ROOT / "oracle" / "adacomp_oracle.c"
PINS = ROOT / "tests" / "test_oracle_pins.py"

# name -> list of (text in the oracle source, replacement, which occurrence)
MUTANTS = {
    # accumulated gradient and the probe H (definition paragraph)
    "G_subtracts_dW": [("G[j] = r[j] + dw[j];", "G[j] = r[j] - dw[j];", 0)],
    "H_drops_dW": [("H[j] = G[j] + dw[j];", "H[j] = G[j];", 0)],
    "H_rounded_once": [("H[j] = G[j] + dw[j];",
                        "H[j] = (float)((double)r[j] + 2.0 * (double)dw[j]);", 0)],
    # local bin maxima
    "gmax_signed": [("if (fabsf(G[j]) > m) m = fabsf(G[j]);", "if (G[j] > m) m = G[j];", 0)],
    "gmax_over_H": [("if (fabsf(G[j]) > m) m = fabsf(G[j]);",
                     "if (fabsf(H[j]) > m) m = fabsf(H[j]);", 0)],
    "last_bin_dropped": [("(sg->numel + sg->bin_len - 1u) / sg->bin_len",
                          "sg->numel / sg->bin_len", 0)],
    # the layer-wide scale s
    "mean_over_elements": [("acc / (double)B", "acc / (double)N", 0)],
    "mean_in_float": [("double acc = 0.0;", "float acc = 0.0f;", 0)],
    "mean_drops_last_bin": [("for (uint64_t b = 0; b < B; ++b) acc += (double)gmax[b];",
                             "for (uint64_t b = 0; b + 1 < B; ++b) acc += (double)gmax[b];", 0)],
    # soft-threshold selection
    "threshold_strict": [("fabsf(H[j]) >= gmax[b]", "fabsf(H[j]) > gmax[b]", 0)],
    "threshold_on_G": [("fabsf(H[j]) >= gmax[b]", "fabsf(G[j]) >= gmax[b]", 0)],
    "zero_G_sent": [(" && G[j] != 0.0f", "", 0)],
    # ternary quantization and residue update
    "residue_adds_gq": [("r[j] = G[j] - gq;", "r[j] = G[j] + gq;", 0)],
    "residue_unsent_stale": [("r[j] = G[j];", "r[j] = r[j];", 0)],
    "gq_sign_of_H": [("float gq = G[j] > 0.0f ? s : -s;", "float gq = H[j] > 0.0f ? s : -s;", 0)],
    # sparse-index words (Table 2)
    "sign_bit_inverted": [("uint32_t sign = G[j] < 0.0f ? 1u : 0u;",
                           "uint32_t sign = G[j] > 0.0f ? 1u : 0u;", 0)],
    "sign_bit_position": [("(sign << (8u * wb - 1u))", "(sign << (8u * wb - 2u))", 0)],
    "index_not_in_bin": [("(uint32_t)(j - lo)", "(uint32_t)j", 0)],
    "word_width_boundary": [("bin_len < 64u ? 1u : 2u", "bin_len <= 64u ? 1u : 2u", 0)],
    "count_region_unpadded": [("count_at = round_up16(count_at + B * wb);",
                               "count_at = count_at + B * wb;", 0)],
    "directory_offset_wrong": [("put_u64(dir + 8, entry_at);", "put_u64(dir + 8, count_at);", 0)],
    "header_survivors_wrong": [("put_u64(msg + 24, total_surv);",
                                "put_u64(msg + 24, total_surv - 1u);", 0)],
    # plan hash (FNV-1a 32)
    "hash_fnv1_order": [("h ^= buf[k];\n            h *= 16777619u;",
                         "h *= 16777619u;\n            h ^= buf[k];", 0)],
    "hash_skips_flags": [("for (int k = 0; k < 24; ++k)", "for (int k = 0; k < 20; ++k)", 0)],
    "hash_zero_basis": [("uint32_t h = 2166136261u;", "uint32_t h = 0u;", 0)],
    # message capacity
    "capacity_always_16bit": [("at = round_up16(at + segs[i].numel * word_bytes(segs[i].bin_len));",
                               "at = round_up16(at + segs[i].numel * 2u);", 0)],
    "capacity_off_by_one": [("at = round_up16(at + segs[i].numel * word_bytes(segs[i].bin_len));",
                             "at = round_up16(at + (segs[i].numel + 1u) * word_bytes(segs[i].bin_len));",
                             0)],
    # hard local selection (Figures 4-6 baseline)
    "ls_flag_ignored": [("const int ls = (sg->flags & ORACLE_FLAG_LS) != 0u;", "const int ls = 0;", 0)],
    "ls_last_maximum": [("for (uint64_t j = lo; j < hi && first_max == hi; ++j)",
                         "for (uint64_t j = lo; j < hi; ++j)", 0)],
    "ls_sends_zero_bins": [("if (ls && gmax[b] > 0.0f)", "if (ls)", 0)],
    "ls_maximum_of_H": [("if (fabsf(G[j]) == gmax[b]) first_max = j;",
                         "if (fabsf(H[j]) >= gmax[b]) first_max = j;", 0)],
    # decode-accumulate
    "decode_sign_flipped": [("float q = sign ? -s : s;", "float q = sign ? s : -s;", 0)],
    "decode_bin_base_dropped": [("uint64_t j = b * sg->bin_len + idx;", "uint64_t j = idx;", 0)],
    "decode_no_zero_fill": [("if (!accumulate)", "if (accumulate)", 0)],
    "decode_order_reversed": [("const uint8_t *m = msgs[k];", "const uint8_t *m = msgs[K - 1u - k];", 0)],
    "decode_skips_count_check": [("if (seen != get_u32(dir + 4)) return ORACLE_BAD_MESSAGE;", "", 0)],
    "decode_skips_hash_check": [(" ||\n            get_u32(m + 8) != nseg || get_u32(m + 12) != hash)",
                                 " ||\n            get_u32(m + 8) != nseg)", 0)],
    # SGD with momentum on the decoded sum
    "sgd_no_scale": [("float g = scale * sum[j];", "float g = sum[j];", 0)],
    "sgd_decay_sign": [("if (weight_decay != 0.0f) g = g + weight_decay * w[j];",
                        "if (weight_decay != 0.0f) g = g - weight_decay * w[j];", 0)],
    "sgd_dampening": [("m[j] = momentum * m[j] + g;", "m[j] = momentum * m[j] + (1.0f - momentum) * g;", 0)],
    "sgd_step_on_g": [("w[j] = w[j] - lr * m[j];", "w[j] = w[j] - lr * g;", 0)],
    "sgd_nesterov": [("w[j] = w[j] - lr * m[j];", "w[j] = w[j] - lr * (g + momentum * m[j]);", 0)],
    # Adam on the decoded sum
    "adam_no_scale": [("float g = scale * sum[j];", "float g = sum[j];", 1)],
    "adam_decay_sign": [("if (weight_decay != 0.0f) g = g + weight_decay * w[j];",
                         "if (weight_decay != 0.0f) g = g - weight_decay * w[j];", 1)],
    "adam_decoupled_decay": [
        ("if (weight_decay != 0.0f) g = g + weight_decay * w[j];", "", 1),
        ("w[j] = w[j] - lr * (mh / (sqrtf(vh) + eps));",
         "w[j] = w[j] - lr * (mh / (sqrtf(vh) + eps)) - lr * weight_decay * w[j];", 0)],
    "adam_no_bias_correction_m": [("const float mh = m[j] / c1;", "const float mh = m[j];", 0)],
    "adam_no_bias_correction_v": [("const float vh = v[j] / c2;", "const float vh = v[j];", 0)],
    "adam_eps_inside_sqrt": [("(sqrtf(vh) + eps)", "sqrtf(vh + eps)", 0)],
    "adam_c2_uses_b1": [("pow((double)b2, (double)t)", "pow((double)b1, (double)t)", 0)],
    "adam_step_off_by_one": [("pow((double)b1, (double)t)", "pow((double)b1, (double)(t + 1u))", 0)],
    "adam_v_of_abs_g": [("omb2 * (g * g)", "omb2 * fabsf(g)", 0)],
    "adam_m_of_g_squared": [("m[j] = b1 * m[j] + omb1 * g;", "m[j] = b1 * m[j] + omb1 * (g * g);", 0)],
    # Not planted: the precision in which the bias corrections c1 and c2 are
    # formed.  The pages fix none, and the readings differ by float rounding
    # only, inside the bound of the float64 Adam comparison.
}


def mutate(src: str, edits) -> str:
    for old, new, occ in edits:
        at = -1
        for _ in range(occ + 1):
            at = src.find(old, at + 1)
            assert at >= 0, f"oracle source no longer holds {old!r} (occurrence {occ})"
        src = src[:at] + new + src[at + len(old):]
    return src


def build(src_text: str, out_dir: pathlib.Path) -> pathlib.Path:
    out_dir.mkdir(parents=True, exist_ok=True)
    c = out_dir / "adacomp_oracle.c"
    c.write_text(src_text)
    lib = out_dir / "libadacomp_oracle.so"
    flags = [f for f in oracle.CFLAGS if f not in ("-Wall", "-Wextra")]
    subprocess.run(["gcc", *flags, "-w", "-o", str(lib), str(c), "-lm"], check=True)
    return lib


def run_pins(lib: pathlib.Path):
    env = dict(os.environ, ADACOMP_ORACLE_LIB=str(lib), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", str(PINS), "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=str(ROOT), env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-2000:]


def test_each_mutant_breaks_the_source_it_names():
    """Every mutant changes the source (its text is still found)."""
    src = SRC.read_text()
    for name, edits in MUTANTS.items():
        assert mutate(src, edits) != src, name


def test_every_mutant_fails_a_pin(tmp_path):
    src = SRC.read_text()
    control = build(src, tmp_path / "control")
    code, tail = run_pins(control)
    assert code == 0, "the unmutated copy fails its pins:\n" + tail

    libs = {name: build(mutate(src, edits), tmp_path / name) for name, edits in MUTANTS.items()}
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = dict(zip(libs, pool.map(run_pins, libs.values())))
    survivors = [name for name, (code, _) in results.items() if code == 0]
    assert not survivors, f"mutants that pass every pin: {survivors}"
    # a pytest usage or collection error would also be a nonzero exit: demand a failed test
    not_failed = [name for name, (code, _) in results.items() if code != 1]
    for name in not_failed:
        tail = results[name][1]
        assert "failed" in tail or "Error" in tail, f"{name}: exit {results[name][0]}\n{tail}"

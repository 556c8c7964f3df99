"""The oracle pins must fail on plausible mistakes.

Each case plants one mistake in a temporary copy of oracle/kvoracle.c (on the
CPU), builds it, and runs tests/test_oracle_pins.py against that build through
KVORACLE_LIB. The pins pass on the real oracle (test_oracle_pins.py) and must
fail on every mutant here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvoracle.c")

MUTANTS = {
    # query head -> kv head mapping interleaved instead of contiguous groups
    "grouping": ("int kvh = h / g;\n        int n = ctx_lens[b];", "int kvh = h % n_kv;\n        int n = ctx_lens[b];"),
    "multi_grouping": ("int kvh = h / g;\n        int hi", "int kvh = h % n_kv;\n        int hi"),
    # the softmax scale dropped
    "scale": ("double s = scale * dot;", "double s = dot;"),
    # append writes the slot after the right one
    "slot": ("int t = L % BLOCK;\n        for (int h = 0; h < n_kv; ++h) {\n            size_t dst",
             "int t = (L + 1) % BLOCK;\n        for (int h = 0; h < n_kv; ++h) {\n            size_t dst"),
    # window off by one
    "window": ("? n - window : 0;", "? n - window + 1 : 0;"),
    # the per-layer window list indexed from the second entry
    "layer_window_shift": ("if (pos == layer) return windows[i];", "if (pos == layer + 1) return windows[i];"),
    # released blocks: the next query's own token left out of its window
    "released_own_token": ("first = L + 1 - window;", "first = L - window;"),
    # released blocks: a block released as soon as its first token leaves the window
    "released_first_token": ("while (n * 16 + 15 < first) ++n;", "while (n * 16 < first) ++n;"),
    # INT4 rounding ties to even instead of half away from zero
    "round_even": ("c = (int)roundf(v);", "c = (int)rintf(v);"),
    # INT4 codes not clamped above 15 (fp16 rounding of s can push the quotient past 15.5)
    "no_clamp_high": ("            else if (v >= 15.0f)\n                c = 15;\n", ""),
    # INT4 codes not clamped below 0 (an fp16 min rounded up can push the quotient below -0.5)
    "no_clamp_low": ("if (isnan(v) || v <= 0.0f)", "if (isnan(v))"),
    # no clamp at all
    "no_clamp": ("            if (isnan(v) || v <= 0.0f)\n                c = 0;\n            else if (v >= 15.0f)\n"
                 "                c = 15;\n            else\n                c = (int)roundf(v); /* half away from zero */",
                 "            c = isnan(v) ? 0 : (int)roundf(v);"),
    # a negative-zero min kept as -0 (stored min bits 0x8000)
    "signed_zero_min": ("if (mn == 0.0f) mn = 0.0f;", ""),
    # a negative-zero max kept as -0 (an all -0 group gets s = -0, bits 0x8000)
    "signed_zero_max": ("if (mx == 0.0f) mx = 0.0f;", ""),
    # INT4 symmetric (min dropped)
    "no_min": ("float v = (x[i * xs] - mf) / sf;", "float v = x[i * xs] / sf;"),
    # INT4 codes from the unrounded min instead of the stored fp16 min
    "unrounded_min": ("mf = kvo_f16_to_f32(*m16);", "mf = mn;"),
    # K grouped along channels instead of tokens
    "k_orientation": ("q4_group(k + c, BLOCK, (size_t)d,", "q4_group(k + c, BLOCK, 1,"),
    # nibble order swapped
    "nibble": ("    if (c & 1)\n        row[c / 2]", "    if (!(c & 1))\n        row[c / 2]"),
    # partial-block keys not read from the bf16 tail
    "tail": ("Kd[row + c] = bf16_bits_to_float(kt[row_index(n_kv, d, slot, h, t) + c]);",
             "Kd[row + c] = 0.0;"),
    # fp16 rounding half-up instead of ties-to-even
    "f16_round": ("    double r = rint(a / q) * q;\n    if (r == 0.0)", "    double r = floor(a / q + 0.5) * q;\n    if (r == 0.0)"),
    # fp16 subnormal quantum wrong
    "f16_subnormal": ("if (ex < -14) ex = -14;", "if (ex < -15) ex = -15;"),
    # rotation direction flipped
    "rope_sign": ("float nx = xc - ys, ny = xs + yc;", "float nx = xc + ys, ny = yc - xs;"),
    # RoPE frequency exponent halved
    "rope_freq": ("double theta = pow(base, -(2.0 * i) / d);", "double theta = pow(base, -(1.0 * i) / d);"),
    # half-split pairing wrong
    "rope_pair": ("*c1 = i + d / 2;", "*c1 = d - 1 - i;"),
    # several query tokens: no causal mask among the new tokens
    "multi_causal": ("int hi = ctx_lens[b] - q_len + i + 1;", "int hi = ctx_lens[b];"),
    # several query tokens: a token does not see itself
    "multi_self": ("int hi = ctx_lens[b] - q_len + i + 1;", "int hi = ctx_lens[b] - q_len + i;"),
    # block copy in the wrong direction
    "copy_dir": ("memcpy(regions[r] + (size_t)dst[i] * block_bytes[r], regions[r] + (size_t)src[i] * block_bytes[r],",
                 "memcpy(regions[r] + (size_t)src[i] * block_bytes[r], regions[r] + (size_t)dst[i] * block_bytes[r],"),
    # KV deviation without the V term
    "dev_no_v": ("acc += dk * dk + dv * dv;", "acc += dk * dk;"),
    # KV deviation looked up in the first sequence's table for every row
    "dev_table": ("int p = tables[(size_t)row_seq[i] * max_blocks + pos / BLOCK];",
                  "int p = tables[pos / BLOCK];"),
    # recompute count rounded to nearest instead of up
    "count_round": ("double c = ceil(ratio * (double)num_tokens);", "double c = floor(ratio * (double)num_tokens + 0.5);"),
    # top-k ties go to the higher row
    "topk_tie": ("return (a->i > b->i) - (a->i < b->i);", "return (a->i < b->i) - (a->i > b->i);"),
    # top-k keeps the smallest values
    "topk_order": ("if (a->v > b->v) return -1;\n    if (a->v < b->v) return 1;",
                   "if (a->v < b->v) return -1;\n    if (a->v > b->v) return 1;"),
    # recompute ratio without its floor
    "ratio_floor": ("if (r < floor_ratio) r = floor_ratio;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in kvoracle.c"
    mut = tmp_path / "kvoracle.c"
    mut.write_text(src.replace(old, new), encoding="utf-8")
    lib = tmp_path / "libkvoracle.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-fopenmp", "-ffp-contract=off",
                    "-fPIC", "-shared", str(mut), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, KVORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}"

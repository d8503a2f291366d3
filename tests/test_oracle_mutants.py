"""Planted mistakes in copies of the oracle.  Each mutant below changes one
spot of oracle/kvq_oracle.c the way a plausible slip would -- a rounding tie,
a sign, an index, a dropped or wrong factor, an off-by-one limit -- and must
fail at least one pin of tests/test_oracle_pins.py, while the unchanged
source, built the same way, passes them all.  This checks the pins, not the
library: CPU only, each copy compiled with gcc into a temporary directory and
loaded by the pin suite in its own process (KVQ_ORACLE_LIB)."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvq_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (what the slip is, the exact text it changes, the text it leaves)
MUTANTS = [
    ("E2M1 ties to the odd code",
     "    double d = fabs(a - kvqo_e2m1_value(c));\n    if (d < bestd || (d == bestd && (c & 1) == 0)) {",
     "    double d = fabs(a - kvqo_e2m1_value(c));\n    if (d < bestd || (d == bestd && (c & 1) == 1)) {"),
    ("E4M3 ties to the odd code",
     "    double d = fabs(a - kvqo_e4m3_value(c));\n    if (d < bestd || (d == bestd && (c & 1) == 0)) {",
     "    double d = fabs(a - kvqo_e4m3_value(c));\n    if (d < bestd || (d == bestd && (c & 1) == 1)) {"),
    ("E4M3 saturates to the NaN code", "  if (s >= 448.0f) return 0x7E;", "  if (s > 448.0f) return 0x7F;"),
    ("E4M3 subnormal exponent", "(m / 8.0) * ldexp(1.0, -6)", "(m / 8.0) * ldexp(1.0, -7)"),
    ("E2M1 exponent bias", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("NVFP4 block maximum mapped to 4 instead of 6", "    float den = 6.0f * gs;", "    float den = 4.0f * gs;"),
    ("NVFP4 elements rounded under the raw scale", "kvqo_e2m1_encode(xb[i] / S)",
     "kvqo_e2m1_encode(xb[i] / (s_raw * gs))"),
    ("NVFP4 nibble order", "(uint8_t)(c[2 * j] | (c[2 * j + 1] << 4))", "(uint8_t)(c[2 * j + 1] | (c[2 * j] << 4))"),
    ("INT4 scale amax / 8", "  float s = amax / 7.0f;", "  float s = amax / 8.0f;"),
    ("INT4 ties away from zero", "float rr = nearbyintf(r);", "float rr = roundf(r);"),
    # (a clamp at -8 instead of -7 would be no mistake: with s = amax / 7 no
    # quotient reaches 7.5 in magnitude, so neither clamp ever acts)
    ("INT4 clamp at 6", "        if (v > 7) v = 7;", "        if (v > 6) v = 6;"),
    ("INT4 nibble sign extension", "    int q = (nib & 8) ? nib - 16 : nib;", "    int q = (nib & 8) ? nib - 8 : nib;"),
    ("NVFP4 dequantization drops the global scale", "kvqo_e4m3_value(scales[i / 16]) * (double)gs;",
     "kvqo_e4m3_value(scales[i / 16]);"),
    ("V section placed right after the K codes",
     "  size_t half = (size_t)P * (row_code_bytes(D) + row_scale_bytes(fmt, D));",
     "  size_t half = (size_t)P * row_code_bytes(D);"),
    ("store row offset one off", "    int off = slot % P;", "    int off = (slot + 1) % P;"),
    ("decode without the softmax scale", "    s[t - t0] = sm_scale * dot;", "    s[t - t0] = dot;"),
    ("decode query heads interleaved instead of grouped", "      int g = h / G;\n      int64_t L = seq_lens[b];",
     "      int g = h % Hkv;\n      int64_t L = seq_lens[b];"),
    ("decode reads the values from the key rows",
     "    read_token(pool, fmt, P, Hkv, D, gs, pages, t, g, 1, row);\n    for (int c = 0; c < D; c++) acc[c] += p * row[c];",
     "    read_token(pool, fmt, P, Hkv, D, gs, pages, t, g, 0, row);\n    for (int c = 0; c < D; c++) acc[c] += p * row[c];"),
    ("split merge weight inverted", "        double w = exp(ms[i] - M);", "        double w = exp(M - ms[i]);"),
    ("decode lse without its maximum", "        lse[(size_t)b * Hq + h] = M + log(denom);",
     "        lse[(size_t)b * Hq + h] = log(denom);"),
    ("bf16 ties to odd", "(((lo >> 16) & 1) == 0 ? lo : hi)", "(((lo >> 16) & 1) == 1 ? lo : hi)"),
    ("Hadamard butterfly sign", "      x[i + h] = a - b;", "      x[i + h] = b - a;"),
    ("Hadamard scale 1/D instead of 1/sqrt(D)", "  const float s = (float)(1.0 / sqrt((double)D));",
     "  const float s = (float)(1.0 / (double)D);"),
    ("extend causal limit one key short", "      const int64_t nk = prefix_len + i + 1;",
     "      const int64_t nk = prefix_len + i;"),
    ("fused extend causal limit one key short", "      const int64_t nk = q_pos[j] + 1;",
     "      const int64_t nk = q_pos[j];"),
    ("global scale over 448 instead of 6 * 448", "amax / 2688.0f", "amax / 448.0f"),
    ("FP8 values stored by token instead of by channel",
     "  return kv ? (size_t)P * D + (size_t)c * P + off : (size_t)off * D + c;",
     "  return kv ? (size_t)P * D + (size_t)off * D + c : (size_t)off * D + c;"),
]


def _pins_pass(name: str, text: str, tmp: str) -> tuple[bool, str]:
    """Build one copy of the oracle source and run the pin suite against it."""
    import oracle
    stem = os.path.join(tmp, "".join(ch if ch.isalnum() else "_" for ch in name))
    with open(stem + ".c", "w") as f:
        f.write(text)
    oracle.compile_source(stem + ".c", stem + ".so")
    env = dict(os.environ, KVQ_ORACLE_LIB=stem + ".so", OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=900)
    lines = (r.stdout + r.stderr).strip().splitlines()
    return r.returncode == 0, "\n".join(lines[-3:])


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(SRC).read()
    jobs = [("unchanged", src)]
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"mutation site of '{name}' is not unique in the oracle source"
        jobs.append((name, src.replace(old, new)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = dict(zip([n for n, _ in jobs], ex.map(lambda j: _pins_pass(j[0], j[1], str(tmp_path)), jobs)))
    ok, tail = results["unchanged"]
    assert ok, f"the unchanged oracle fails its pins when built this way:\n{tail}"
    survivors = [f"{n}: {results[n][1]}" for n, _, _ in MUTANTS if results[n][0]]
    assert not survivors, "planted mistakes no pin catches:\n" + "\n".join(survivors)

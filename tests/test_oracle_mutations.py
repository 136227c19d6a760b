"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, a swapped operand,
a wrong index or order) in a copy of the oracle's C source, builds that copy
on the CPU, and runs the pin tests against it in a subprocess; the pins must
fail.  The real oracle is never modified.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zero_oracle.c")
ADAM = "tests/test_oracle_adam.py"
RS = "tests/test_oracle_reduce_stats.py"
F16 = "tests/test_oracle_f16.py"
CLIP = "tests/test_oracle_clip.py"
AG = "tests/test_oracle_allgather.py"
QWZ = "tests/test_oracle_qwz.py"
LM = "tests/test_oracle_layout_memory.py"

MUTATIONS = [
    ("step sign", "*master - lr * (mh", "*master + lr * (mh", ADAM),
    ("drop 1-b1", "omb1 * g;", "g;", ADAM),
    ("eps inside sqrt", "sqrtf(vh) + eps", "sqrtf(vh + eps)", ADAM),
    ("no bias correction on m", "m1 / bc1", "m1", ADAM),
    ("no bias correction on v", "v1 / bc2", "v1", ADAM),
    ("b1 and b2 swapped", "s[0] = (float)beta1;", "s[0] = (float)beta2;", ADAM),
    ("g instead of g^2", "omb2 * (g * g)", "omb2 * g", ADAM),
    ("bias power t-1", "pow(beta1, (double)step)", "pow(beta1, (double)(step - 1))", ADAM),
    ("no unscale", "const float g = x * inv;", "const float g = x;", ADAM),
    ("lr squared", "s[6] = (float)lr;", "s[6] = (float)(lr * lr);", ADAM),
    ("p16 from the wrong variable", "*p16 = zo_f32_to_f16(th1);", "*p16 = zo_f32_to_f16(mh);", ADAM),
    ("skip ignored", "if (overflow) return ZO_OK; /* skipped", "if (0) return ZO_OK; /* skipped", ADAM),
    ("whole-step skip ignored", "if (*overflow) return ZO_OK; /* skipped", "if (0) return ZO_OK; /* skipped", ADAM),
    ("1-b in float", "s[1] = (float)(1.0 - beta1);", "s[1] = 1.0f - (float)beta1;", ADAM),
    ("reduce drops slice 0", "float acc = zo_f16_to_f32(slices[0][j]);", "float acc = 0.0f;", RS),
    ("reduce in reverse order",
     "for (int32_t r = 1; r < n_slices; ++r)\n      acc = acc + zo_f16_to_f32(slices[r][j]);",
     "for (int32_t r = n_slices - 1; r >= 1; --r)\n      acc = zo_f16_to_f32(slices[r][j]) + acc;", RS),
    ("flag misses NaN", "if (!isfinite(x)) *flag = 1u;", "if (isinf(x)) *flag = 1u;", RS),
    ("sumsq of |g|", "neumaier_add(sum, comp, d * d);", "neumaier_add(sum, comp, fabs(d));", RS),
    ("sumsq without unscale", "const float g = x * s;          /*", "const float g = x;          /*", RS),
    ("encode truncates", "nearbyint(a / spacing)", "floor(a / spacing)", F16),
    ("encode rounds half up", "nearbyint(a / spacing)", "floor(a / spacing + 0.5)", F16),
    ("decode subnormal scale", "mag = ldexpf((float)f, -24);", "mag = ldexpf((float)f, -25);", F16),
    ("layout floor", "rows = psi / unit + (psi % unit != 0 ? 1 : 0);", "rows = psi / unit;", LM),
    ("layout offset", "const int64_t offset = (int64_t)rank * shard;", "const int64_t offset = (int64_t)rank * (shard - 1);", LM),
    ("memory stage 2", "case 2: return 2.0 * psi + (2.0 * psi + K * psi) / n;", "case 2: return 2.0 * psi + (K * psi) / n;", LM),
    ("clip norm without sqrt", "const double norm = sqrt(sumsq);", "const double norm = sumsq;", CLIP),
    ("clip factor inverted", "return norm > max_norm ? max_norm / norm : 1.0;",
     "return norm > max_norm ? norm / max_norm : 1.0;", CLIP),
    ("clip below the bound", "return norm > max_norm ? max_norm / norm : 1.0;", "return max_norm / norm;", CLIP),
    ("allgather rank order reversed", "if (flat < psi) replica[flat] = shards[r][j];",
     "if (flat < psi) replica[flat] = shards[n_ranks - 1 - r][j];", AG),
    ("allgather offset stride", "const int64_t flat = (int64_t)r * shard_len + j;",
     "const int64_t flat = (int64_t)r * (shard_len - (shard_len > 1)) + j;", AG),
    ("qwz truncates", "q = rintf(zo_f16_to_f32(x16[j]) / scale); /* ties to even */",
     "q = truncf(zo_f16_to_f32(x16[j]) / scale); /* ties to even */", QWZ),
    ("qwz rounds half away", "q = rintf(zo_f16_to_f32(x16[j]) / scale); /* ties to even */",
     "q = roundf(zo_f16_to_f32(x16[j]) / scale); /* ties to even */", QWZ),
    ("qwz scale 255", "const float scale = amax / 127.0f;", "const float scale = amax / 255.0f;", QWZ),
    ("qwz dequant wrong block", "scales[j / ZO_QWZ_BLOCK]", "scales[j / (ZO_QWZ_BLOCK / 2) / 2 + (j % 2)]", QWZ),
    ("memory stage 1", "case 1: return 2.0 * psi + 2.0 * psi + K * psi / n;", "case 1: return 2.0 * psi + K * psi / n;", LM),
    ("bias correction in float", "s[5] = (float)(1.0 - pow(beta2, (double)step));",
     "s[5] = 1.0f - powf((float)beta2, (float)step);", ADAM),
    ("v decays with b1", "const float v1 = b2 * *v + omb2 * (g * g);", "const float v1 = b1 * *v + omb2 * (g * g);", ADAM),
    ("sqrt before bias correction", "sqrtf(vh) + eps", "sqrtf(v1) / bc2 + eps", ADAM),
    ("reduce accumulates in double", "float acc = zo_f16_to_f32(slices[0][j]);",
     "double acc = zo_f16_to_f32(slices[0][j]);", RS),
    ("qwz scale from the signed maximum", "const float a = fabsf(zo_f16_to_f32(x16[j]));",
     "const float a = zo_f16_to_f32(x16[j]);", QWZ),
    # (a clamp at +-128 would change nothing: with scale = max/127 rounded to
    # nearest, |x/scale| never rounds beyond 127 for finite values)
    ("qwz clamp at 126", "if (q > 127.0f) q = 127.0f;", "if (q > 126.0f) q = 126.0f;", QWZ),
    ("allgather copies the padding", "if (flat < psi) replica[flat] = shards[r][j];",
     "if (flat < psi + 1 && flat < (int64_t)n_ranks * shard_len) replica[flat < psi ? flat : psi - 1] = shards[r][j];", AG),
]


def _run_mutation(case, workdir):
    name, old, new, test_file = case
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new, 1)
    d = os.path.join(workdir, name.replace(" ", "_").replace("/", "_"))
    os.makedirs(d, exist_ok=True)
    c_path = os.path.join(d, "zero_oracle.c")
    with open(c_path, "w") as f:
        f.write(mutated)
    so = os.path.join(d, "liboracle.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-I", os.path.join(ROOT, "oracle"), "-o", so, c_path, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, ZERO_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        test_file], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_pins_catch_planted_mistakes():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda c: _run_mutation(c, tmp), MUTATIONS))
    # exit code 1 = the pin tests ran and failed; anything else (a crash, a
    # collection error, a pass) does not count as caught
    survived = [(name, rc) for name, rc in results if rc != 1]
    assert not survived, f"mutations not caught by the pins: {survived}"

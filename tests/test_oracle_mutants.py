"""Plants plausible mistakes in a copy of the oracle's C source (on the CPU only), builds
each mutant and checks that the pin suite rejects it: the pins constrain every part of the
step, so a dropped term, a wrong index or sign, or a transposed operand cannot pass."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "rope interleaved pairs": ("double a = u[i], b = u[i + half];\n        u[i] = a * c - b * s;\n        u[i + half] = b * c + a * s;",
                               "double a = u[2 * i], b = u[2 * i + 1];\n        u[2 * i] = a * c - b * s;\n        u[2 * i + 1] = b * c + a * s;"),
    "rope sign": ("u[i + half] = b * c + a * s;", "u[i + half] = b * c - a * s;"),
    "rope frequency": ("pow(theta, -2.0 * (double)i / (double)hd)", "pow(theta, -(double)i / (double)hd)"),
    "gqa modulo map": ("int g = (int)(((int64_t)hh * nKV) / nH);", "int g = hh % nKV;"),
    "attention scale": ("double scale = 1.0 / sqrt((double)hd);", "double scale = 1.0;"),
    "attention reads one row too many": ("c->kv + kv_index(c, l, 1, g, 0), pos + 1, hd,", "c->kv + kv_index(c, l, 1, g, 0), pos + 2, hd,"),
    "kv append at row 0": ("float* kr = c->kv + kv_index(c, l, 0, g, pos);", "float* kr = c->kv + kv_index(c, l, 0, g, 0);"),
    "rmsnorm n-1": ("double r = 1.0 / sqrt(ss / (double)n + eps);", "double r = 1.0 / sqrt(ss / (double)(n - 1) + eps);"),
    "rmsnorm eps outside root": ("double r = 1.0 / sqrt(ss / (double)n + eps);", "double r = 1.0 / (sqrt(ss / (double)n) + eps);"),
    "int8 scale of row 0": ("acc *= (double)m->s[j];", "acc *= (double)m->s[0];"),
    "int4 group scale of group 0": ("acc += (double)m->s[j * ng + b] * part;", "acc += (double)m->s[j * ng] * part;"),
    "quant scale not rounded to fp16": ("float sc = (float)orc_round((double)ratio, ORC_FMT_F16);", "float sc = ratio;"),
    "quant truncation": ("float n = nearbyintf(t);", "float n = truncf(t);"),
    "residual dropped": ("gemv(c, &c->wo[l], c->o, c->acc);\n        for (int i = 0; i < H; ++i) c->x[i] = orc_round(c->x[i] + c->acc[i], act);",
                         "gemv(c, &c->wo[l], c->o, c->acc);\n        for (int i = 0; i < H; ++i) c->x[i] = orc_round(c->acc[i], act);"),
    "gate and up swapped": ("c->a[j] = orc_swiglu(c->g[j], c->u[j], act);", "c->a[j] = orc_swiglu(c->u[j], c->g[j], act);"),
    "mlp norm uses attention gains": ("load_gains(c, c->mlp_norm[l], H, gain);", "load_gains(c, c->attn_norm[l], H, gain);"),
    "mlp norm dropped": ("load_gains(c, c->mlp_norm[l], H, gain);\n        orc_rmsnorm(c->x, gain, H, d->rms_eps, act, c->h);",
                         "load_gains(c, c->mlp_norm[l], H, gain);\n        for (int i = 0; i < H; ++i) c->h[i] = c->x[i];"),
    "down residual dropped": ("gemv(c, &c->wd[l], c->a, c->acc);\n        for (int i = 0; i < H; ++i) c->x[i] = orc_round(c->x[i] + c->acc[i], act);",
                              "gemv(c, &c->wd[l], c->a, c->acc);\n        for (int i = 0; i < H; ++i) c->x[i] = orc_round(c->acc[i], act);"),
    "down reads the gate": ("gemv(c, &c->wd[l], c->a, c->acc);", "gemv(c, &c->wd[l], c->g, c->acc);"),
    "attention norm uses mlp gains": ("load_gains(c, c->attn_norm[l], H, gain);", "load_gains(c, c->mlp_norm[l], H, gain);"),
    "final norm dropped": ("load_gains(c, c->final_norm, H, gain);\n    orc_rmsnorm(c->x, gain, H, d->rms_eps, act, c->h);",
                           "load_gains(c, c->final_norm, H, gain);\n    for (int i = 0; i < H; ++i) c->h[i] = c->x[i];"),
    "value head for key": ("c->v[i] = orc_round(c->v[i], act);", "c->v[i] = orc_round(c->k[i], act);"),
    "swiglu sign": ("return orc_round(g / (1.0 + exp(-g)) * u, act_fmt);", "return orc_round(g / (1.0 + exp(g)) * u, act_fmt);"),
    "argmax last tie": ("if (best < 0 || v[i] > bv)", "if (best < 0 || v[i] >= bv)"),
    "ties away from zero": ("double r = nearbyint(scaled);", "double r = round(scaled);"),
    "bf16 mantissa 7": ("case ORC_FMT_BF16: return round_fmt(x, 8, -126, 3.3895313892515355e38);",
                        "case ORC_FMT_BF16: return round_fmt(x, 7, -126, 3.3895313892515355e38);"),
}


def _run(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation pattern for {name!r} not found exactly once"
    cpath = os.path.join(tmp, name.replace(" ", "_") + ".c")
    so = cpath[:-2] + ".so"
    open(cpath, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so, cpath, "-lm"],
                   check=True)
    env = dict(os.environ, AMK_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(min(4, os.cpu_count() or 1)) as ex:
        codes = dict(zip(MUTANTS, ex.map(lambda n: _run(n, str(tmp_path)), MUTANTS)))
    survivors = [n for n, rc in codes.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    assert all(rc == 1 for rc in codes.values()), codes     # failures, not crashes

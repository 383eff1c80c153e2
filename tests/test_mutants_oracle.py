"""The oracle's pins catch plausible mistakes in the oracle.

Each mutant below is a copy of oracle/ with one planted slip: a dropped term,
a wrong sign, index or constant, a swapped operand, a rounding rule changed.
The C oracle is rebuilt from the mutated source. The pin tests
(tests/test_oracle_*.py) then run in a child process against that copy, and
at least one of them must fail. An unmutated copy must pass, so that a
broken harness cannot look like caught mutants.

Mistakes are planted on the CPU only, in the oracle only; nothing here
touches the GPU or the HIP library.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
PINS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))

C = "oracle.c"
MUTANTS = [
    # ---- bf16 rounding and conversion
    ("bf16 ties round up, not to even", C,
     "u += 0x7fffu + keep_lsb;", "u += 0x8000u;"),
    ("bf16 truncates", C, "u += 0x7fffu + keep_lsb;", "u += 0u;"),
    ("Inf taken for NaN", C, "if ((u & 0x7fffffffu) > 0x7f800000u)",
     "if ((u & 0x7fffffffu) >= 0x7f800000u)"),
    ("NaN keeps its payload", C, "return (uint16_t)0x7fc0u;", "return (uint16_t)(u >> 16);"),
    ("bf16 widened with the wrong shift", C, "uint32_t u = ((uint32_t)h) << 16;",
     "uint32_t u = ((uint32_t)h) << 15;"),
    # ---- data-parallel average
    ("bf16 average not divided by N", C,
     "acc = acc + bf16_bits_to_float(ranks[q][i]);\n        out[i] = acc / n;",
     "acc = acc + bf16_bits_to_float(ranks[q][i]);\n        out[i] = acc;"),
    ("bf16 average over ranks in descending order", C,
     "acc = acc + bf16_bits_to_float(ranks[q][i]);",
     "acc = acc + bf16_bits_to_float(ranks[n_ranks - 1 - q][i]);"),
    ("fp32 average multiplies by 1/N", C,
     "acc = acc + ranks[q][i];\n        out[i] = acc / n;",
     "acc = acc + ranks[q][i];\n        out[i] = acc * (1.0f / n);"),
    ("fp32 average over ranks in descending order", C,
     "acc = acc + ranks[q][i];", "acc = acc + ranks[n_ranks - 1 - q][i];"),
    ("fp32 accumulation overwrites", C,
     "acc[i] = acc[i] + bf16_bits_to_float(micro[i]);",
     "acc[i] = bf16_bits_to_float(micro[i]);"),
    # ---- global-norm clip
    ("sum of squares without the square", C, "s = s + x * x;", "s = s + x;"),
    ("clip coefficient without the 1e-6", C, "(double)max_norm / (norm + 1e-6)",
     "(double)max_norm / norm"),
    ("clip coefficient not clamped at 1", C, "return c < 1.0f ? c : 1.0f;", "return c;"),
    ("clip divides by the sum of squares", C, "double norm = sqrt(sumsq);",
     "double norm = sumsq;"),
    ("clip scale divides by the coefficient", C, "g[i] = g[i] * c;", "g[i] = g[i] / c;"),
    ("clip scale by the reciprocal of the coefficient", C, "g[i] = g[i] * c;",
     "g[i] = g[i] * (1.0f / c);"),
    ("clip scale skips the last element", C,
     "for (int64_t i = 0; i < count; ++i)\n        g[i] = g[i] * c;",
     "for (int64_t i = 0; i + 1 < count; ++i)\n        g[i] = g[i] * c;"),
    # ---- Adam step scalars
    ("decay without lr", C,
     "s.decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);",
     "s.decay = (float)(1.0 - (double)h->weight_decay);"),
    ("second bias correction with beta1", C, "s.bias2 = (float)(1.0 - pow(b2, t));",
     "s.bias2 = (float)(1.0 - pow(b1, t));"),
    ("step counted from 0", C,
     "double b1 = (double)h->beta1, b2 = (double)h->beta2, t = (double)h->step;",
     "double b1 = (double)h->beta1, b2 = (double)h->beta2, t = (double)(h->step + 1);"),
    # ---- Adam element update (fp32)
    ("AdamW and L2 weight decay swapped", C,
     "if (h->decoupled)\n                pi = pi * s.decay;",
     "if (!h->decoupled)\n                pi = pi * s.decay;"),
    ("L2 decay term dropped", C,
     "pi = pi * s.decay;\n            else\n                g = g + wd * pi;",
     "pi = pi * s.decay;\n            else\n                g = g;"),
    ("first moment with beta2", C, "float mi = b1 * m[i] + s.one_minus_b1 * g;",
     "float mi = b2 * m[i] + s.one_minus_b2 * g;"),
    ("second moment with 1 - beta1", C, "float vi = b2 * v[i] + s.one_minus_b2 * (g * g);",
     "float vi = b2 * v[i] + s.one_minus_b1 * (g * g);"),
    ("no bias correction of m", C, "float m_hat = mi / s.bias1;", "float m_hat = mi;"),
    ("no bias correction of v", C, "float v_hat = vi / s.bias2;", "float v_hat = vi;"),
    ("eps inside the square root", C, "float denom = sqrtf(v_hat) + eps;",
     "float denom = sqrtf(v_hat + eps);"),
    ("update added instead of subtracted", C, "pi = pi - lr * (m_hat / denom);",
     "pi = pi + lr * (m_hat / denom);"),
    # ---- fp64 reference evaluation
    ("fp64 Adam with eps inside the root", C,
     "pi = pi - lr * ((mi / bias1) / (sqrt(vi / bias2) + eps));",
     "pi = pi - lr * ((mi / bias1) / (sqrt(vi / bias2 + eps)));"),
    # ---- the per-rank chain (average, clip, Adam, cast)
    ("rank step skips the clip", C,
     "    orc_average_bf16(n_ranks, ranks, count, tmp_grad);\n"
     "    if (clip_coef < 1.0f)\n        orc_scale_f32(tmp_grad, count, clip_coef);",
     "    orc_average_bf16(n_ranks, ranks, count, tmp_grad);"),
    ("rank step casts the old master", C,
     "    orc_adam_f32(h, count, tmp_grad, p, m, v);\n    orc_f32_to_bf16(p, param_out, count);\n}\n\n"
     "void orc_rank_step_f32",
     "    orc_f32_to_bf16(p, param_out, count);\n    orc_adam_f32(h, count, tmp_grad, p, m, v);\n}\n\n"
     "void orc_rank_step_f32"),
    # ---- layout
    ("padding rounds down", "layout.py", "padded = -(-n // parts) * parts",
     "padded = (n // parts) * parts"),
    ("owned slice ignores the unit offset", "layout.py",
     "b = U.flat_off + self.rank * U.shard", "b = self.rank * U.shard"),
    ("FSDP2 chunk is floor(rows / N) + 1", "layout.py", "chunk = -(-rows // n_ranks)",
     "chunk = rows // n_ranks + 1"),
    ("FSDP2 valid rows start one row early", "layout.py",
     "first = min(layout.rank * chunk, rows)", "first = min(layout.rank * chunk, max(rows - 1, 0))"),
    # ---- closed forms
    ("ZeRO-2 bytes as ZeRO-1", "closed_forms.py",
     '"zero2": lambda psi, n: 2 * psi + Fr(14 * psi, n),',
     '"zero2": lambda psi, n: 4 * psi + Fr(12 * psi, n),'),
    ("ZeRO-3 traffic as DDP's", "closed_forms.py", '"zero3": lambda psi: 3 * psi,',
     '"zero3": lambda psi: 2 * psi,'),
    ("Megatron bytes with a 2-byte gradient", "closed_forms.py",
     '"megatron_do": lambda psi, n: 6 * psi + Fr(12 * psi, n),',
     '"megatron_do": lambda psi, n: 4 * psi + Fr(12 * psi, n),'),
    ("unsharded Megatron at 16 bytes", "closed_forms.py", "return 18 * psi", "return 16 * psi"),
    ("bus bandwidth factor (N-1)/N", "closed_forms.py",
     "return Fr(algbw) * Fr(2 * (n - 1), n)", "return Fr(algbw) * Fr(n - 1, n)"),
    ("ring volume 2 S instead of 2 (N-1)/N S", "closed_forms.py",
     "return Fr(2 * (n - 1), n) * Fr(size_bytes)", "return Fr(2 * n, n) * Fr(size_bytes)"),
    # ---- ring simulation
    ("reduce-scatter sends the wrong chunk", "ring.py", "c = (q - k - 1) % N", "c = (q - k) % N"),
    ("all-gather forwards the wrong chunk", "ring.py", "ci = (q - k) % N", "ci = (q - k - 1) % N"),
    # ---- strategy simulation
    ("ZeRO-3 logs one parameter gather, not two", "strategies.py",
     '        cl.comm_log.append(("all_gather_backward", P))\n', ""),
    ("Megatron main gradient not reset each step", "strategies.py",
     "            cl.ranks[q].grads[:] = 0.0\n", ""),
    ("ZeRO-1 keeps only its gradient shard", "strategies.py",
     'if s in ("zero1", "zero1_allreduce"):', 'if s in ("zero1_allreduce",):'),
    ("gathered shards land one element late", "strategies.py",
     "full[b:b + n] = shard[s:s + n]", "full[b + 1:b + n] = shard[s:s + n - 1]"),
    ("clip norm over rank 0's shard only", "strategies.py",
     "c = _clip_coefficient(cfg, g_mean_full)", "c = _clip_coefficient(cfg, shards[0])"),
    ("sharded strategies skip the clip scale", "strategies.py",
     "        if c < 1.0:\n            _c.scale(g, c)\n", ""),
    # ---- linear layer
    ("linear gather keeps the last rows", "linear.py", "return full[:rows]",
     "return full[full.shape[0] - rows:]"),
    ("linear reduce-scatter sums instead of averaging", "linear.py",
     "total = sum(dws) / n", "total = sum(dws)"),
    ("linear reduce-scatter takes the wrong rows", "linear.py", "first = lay.rank * c",
     "first = lay.rank * (c - 1)"),
    ("fp32 dot-product bound without the factor K", "linear.py",
     "return k * u / (1 - k * u)", "return u / (1 - k * u)"),
]


def _copy_oracle(dst_root: str) -> str:
    dst = os.path.join(dst_root, "oracle")
    shutil.copytree(ORACLE, dst, ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.tmp"))
    return dst


def _build_c(dst: str) -> None:
    from oracle.build import CFLAGS
    subprocess.run(["gcc", *CFLAGS, os.path.join(dst, "oracle.c"), "-o",
                    os.path.join(dst, "liboracle.so"), "-lm"], check=True,
                   capture_output=True, timeout=120)


# The pass over all 2^32 cast patterns takes half a minute; the selected
# million patterns of the same file catch every planted cast mistake, so
# the mutant runs leave the exhaustive pass out.
SLOW_PINS = ["tests/test_oracle_bf16.py::test_rne_matches_torch_on_every_fp32_pattern"]


def _run_pins(root: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ZS_ORACLE_MUTANT_ROOT=root, PYTHONDONTWRITEBYTECODE="1")
    deselect = [a for p in SLOW_PINS for a in ("--deselect", p)]
    return subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu", *deselect],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _first_failure(out: str) -> str:
    for line in out.splitlines():
        if line.startswith("FAILED "):
            return line[len("FAILED "):].split(" - ")[0]
    return "?"


def _try(i, mutant, base):
    name, fname, find, repl = mutant
    root = os.path.join(base, f"m{i:02d}")
    dst = _copy_oracle(root)
    path = os.path.join(dst, fname)
    src = open(path).read()
    if src.count(find) != 1:
        return name, "pattern", f"occurs {src.count(find)} times in {fname}, not once"
    open(path, "w").write(src.replace(find, repl))
    _build_c(dst)
    r = _run_pins(root)
    return name, r.returncode, _first_failure(r.stdout)


def test_pins_catch_every_planted_mistake(tmp_path):
    assert len(PINS) >= 8 and not any("mutant" in p for p in PINS)
    clean = str(tmp_path / "clean")
    _build_c(_copy_oracle(clean))
    r = _run_pins(clean)
    assert r.returncode == 0, "the unmutated copy must pass its pins:\n" + r.stdout[-2000:]
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda a: _try(*a), [(i, m, str(tmp_path))
                                                   for i, m in enumerate(MUTANTS)]))
    survivors = [name for name, rc, _ in results if rc != 1]
    report = "\n".join(f"  {name}: rc {rc}, caught by {who}" for name, rc, who in results)
    assert not survivors, f"mutants not caught by a failing pin: {survivors}\n{report}"

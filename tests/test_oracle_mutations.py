"""The oracle's pins catch planted mistakes (CPU only).

Each mutant below is a copy of oracle/oracle.c with one plausible slip
planted in it -- a dropped term, a wrong sign, a transposed operand, an
off-by-one, a wrong tie-break, a wrong rounding rule.  The copy is compiled
with gcc exactly as the oracle is, and the pin suite (test_oracle_pins.py)
is run against it in a child process (MOE_ORACLE_LIB points the oracle
wrapper at the copy).  A mutant the pins let through is a hole in the pins,
so every mutant must make the suite fail; the unmodified source, built the
same way, must pass it.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.c, replacement); each text occurs exactly once
MUTANTS = [
    ("bf16 decode shift", "uint32_t b = (uint32_t)h << 16;", "uint32_t b = (uint32_t)h << 15;"),
    ("fp16 exponent bias", "v = ldexp((double)(man | 0x400), ex - 25);", "v = ldexp((double)(man | 0x400), ex - 24);"),
    ("bf16 rounding ties away", "b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;", "b = (b + 0x8000u) & 0xFFFF0000u;"),
    ("4-bit nibble order", "int q = j < 16 ? (byte & 0xF) : (byte >> 4);", "int q = j < 16 ? (byte >> 4) : (byte & 0xF);"),
    ("4-bit offset", "return half_value(dh) * (float)(q - 8);", "return half_value(dh) * (float)(q - 7);"),
    ("int8 up plane takes the gate scales", "v->s[1] = slab + 3 * n + 4 * (int64_t)I;", "v->s[1] = slab + 3 * n;"),
    ("router gate transposed", "x_value(G, x_dtype, (int64_t)e * H + h)", "x_value(G, x_dtype, (int64_t)h * E + e)"),
    ("logits summed in fp32", "            double acc = 0.0;\n            for (int h = 0; h < H; ++h)",
     "            float acc = 0.0f;\n            for (int h = 0; h < H; ++h)"),
    ("bias sign", "log(b[e] / b_edge)", "log(b_edge / b[e])"),
    ("hot set one too large", "if (rank < n_hot) hot[e] = 1;", "if (rank <= n_hot) hot[e] = 1;"),
    ("bias cap ignored", "bias[e] = (float)(v > (double)cap ? v : (double)cap);", "bias[e] = (float)v;"),
    ("top-k ties to the higher id", "if (best < 0 || s[e] > s[best]) best = e;", "if (best < 0 || s[e] >= s[best]) best = e;"),
    ("top-k bias subtracted", "            if (bias) v = v + bias[e];\n            s[e] = v;",
     "            if (bias) v = v - bias[e];\n            s[e] = v;"),
    ("softmax drops a term", "for (int j = 0; j < k; ++j) sum += exp((double)z[(int64_t)t * E + id[j]] - m);",
     "for (int j = 1; j < k; ++j) sum += exp((double)z[(int64_t)t * E + id[j]] - m);"),
    ("softmax exponent sign", "(float)(exp((double)z[(int64_t)t * E + id[j]] - m) / sum)",
     "(float)(exp(m - (double)z[(int64_t)t * E + id[j]]) / sum)"),
    ("damped weights unbiased", "if (bias) v = v + bias[id[j]];", ""),
    ("flat bias hot set off by one", "bias[e] = rank < n_hot ? 0.0f : value;", "bias[e] = rank <= n_hot ? 0.0f : value;"),
    ("affinity misses slot 0", "if (e2s[e] >= 0) v = v + lambda;", "if (e2s[e] > 0) v = v + lambda;"),
    ("silu sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("gate and up swapped", "double hv = silu(g) * u;", "double hv = silu(u) * g;"),
    ("int8 gate and up swapped", "h[n] = (float)(silu((double)g) * (double)u);", "h[n] = (float)(silu((double)u) * (double)g);"),
    ("h not rounded to bf16", "if (w_type != ORC_W_F32) hv = (double)round_bf16((float)hv);", ""),
    ("down projection transposed (square)", "acc += (double)weight(&v, 2, m, n) * h[n];",
     "acc += (double)weight(&v, 2, m % I, n % H) * h[n];"),
    ("int8 truncating quantiser", "float c = rintf(v[i] / s);", "float c = truncf(v[i] / s);"),
    ("int8 quantiser rounds half away", "float c = rintf(v[i] / s);", "float c = roundf(v[i] / s);"),
    ("int8 scale over 128", "float s = amax > 0.0f ? amax / 127.0f : 1.0f;", "float s = amax > 0.0f ? amax / 128.0f : 1.0f;"),
    ("int8 activation scale dropped", "float g = ((float)ag * sx) * row_scale_i8(&v, 0, n);",
     "float g = (float)ag * row_scale_i8(&v, 0, n);"),
    ("int8 h scale dropped", "o[m] = (double)(((float)ad * sh) * row_scale_i8(&v, 2, m));",
     "o[m] = (double)((float)ad * row_scale_i8(&v, 2, m));"),
    ("routing weight dropped", "double c = wt * o[m];", "double c = o[m];"),
    ("split passes swapped", "                if (resident) yg[m] += c;", "                if (!resident) yg[m] += c;"),
    ("empty slots last", "if (ea != eb) return !ea;", "if (ea != eb) return ea;"),
    ("most recently used evicted", "if (last[a] != last[b]) return last[a] < last[b];",
     "if (last[a] != last[b]) return last[a] > last[b];"),
    ("LFU order ignores counts", "if (policy == ORC_LFU && freq[a] != freq[b]) return freq[a] < freq[b];", ""),
    ("hit does not refresh", "            last[s] = now;\n            if (policy == ORC_LFU) freq[s] += 1;",
     "            if (policy == ORC_LFU) freq[s] += 1;"),
    ("LFU counts every routing id", "        need[ids[i]] = 1;",
     "        need[ids[i]] = 1;\n        if (policy == ORC_LFU && e2s[ids[i]] >= 0) freq[e2s[ids[i]]] += 1;"),
    ("needed slots evictable", "if (s2e[s] < 0 || !need[s2e[s]]) cand[ncand++] = s;", "cand[ncand++] = s;"),
    ("misses in descending id", "    for (int e = 0; e < E; ++e) {\n        if (!need[e]) continue;",
     "    for (int e = E - 1; e >= 0; --e) {\n        if (!need[e]) continue;"),
    ("inserted slot keeps old count", "                last[s] = now;\n                freq[s] = 1;", "                last[s] = now;"),
    ("STATIC evicts", "    if (policy != ORC_STATIC) {\n        for (int s = 0; s < S; ++s)",
     "    if (1) {\n        for (int s = 0; s < S; ++s)"),
    ("step not advanced", "*step = now + 1;", "*step = now;"),
    ("gather reads the slot's row", "host_store + (int64_t)miss[2 * i] * slab_bytes",
     "host_store + (int64_t)miss[2 * i + 1] * slab_bytes"),
    ("residual truncates", "const float v = round_bf16(bf16_value(((const uint16_t*)x)[i]) + y[i]);",
     "const float v = bf16_value(((const uint16_t*)x)[i]) + y[i];"),
    ("repick loads keep the old use count", "        last[s] = *step;\n        freq[s] = 0;", "        last[s] = *step;"),
    ("repick fills slots from the top", "while (s < S && s2e[s] >= 0 && in_new[s2e[s]]) ++s;",
     "while (s < S && s2e[S - 1 - s] >= 0 && in_new[s2e[S - 1 - s]]) ++s;"),
    ("repick moves kept members", "if (!in_new[e] || e2s[e] >= 0) continue;", "if (!in_new[e]) continue;"),
    ("static set ties to the higher id", "if (cnt[o] > cnt[e] || (cnt[o] == cnt[e] && o < e)) ++rank;",
     "if (cnt[o] > cnt[e] || (cnt[o] == cnt[e] && o > e)) ++rank;"),
]


def _build(src_text: str, out_dir: str, name: str) -> str:
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                           "-I" + os.path.join(ROOT, "oracle"), "-o", so, c, "-lm"])
    return so


def _run_pins(so: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, MOE_ORACLE_LIB=so, PYTHONDONTWRITEBYTECODE="1")
    # the one slow pin (a c2-sized layer split) is left out: others cover the same lines
    cmd = [sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider", "-k", "not c2-4"]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_every_planted_mistake_fails_a_pin():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutant '{name}': its text occurs {src.count(old)} times in oracle.c"
    with tempfile.TemporaryDirectory() as d:
        control = _run_pins(_build(src, d, "control"))
        assert control.returncode == 0, "the unmodified oracle fails its pins:\n" + control.stdout[-2000:]

        def one(i):
            name, old, new = MUTANTS[i]
            r = _run_pins(_build(src.replace(old, new), d, f"m{i}"))
            return name, r

        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(one, range(len(MUTANTS))))
    survivors = [name for name, r in results if r.returncode == 0]
    broken = [(name, r.returncode) for name, r in results if r.returncode not in (0, 1)]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
    assert not broken, f"mutants that crashed the pin run instead of failing a pin: {broken}"

"""The fp64 oracle under the compiler's run-time checkers, on the CPU: built
with the address and undefined-behaviour sanitizers, and separately with the
thread sanitizer (its streams run on pthread workers), a small store +
retrieve of every read order and a read-only retrieve run clean."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tmref.c")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
int tmref_forward_read(int, int, int, int, int, int, int, const float*, const float*, const float*,
                       const float*, const float*, const float*, double*, double*, int, int);
int tmref_retrieve(int, int, int, int, int, int, const double*, const float*, double*, int);
long tmref_param_count(int, int, int);

static float frand(unsigned* s) { *s = *s * 1664525u + 1013904223u; return (float)(*s >> 8) / 16777216.0f - 0.5f; }

int main(void) {
    const int d = 8, depth = 3, ex = 2, b = 4, B = 2, H = 2, T = 12;
    const long P = tmref_param_count(d, depth, ex);
    const long nt = (long)B * T * H;
    float* k = malloc(sizeof(float) * nt * d);
    float* v = malloc(sizeof(float) * nt * d);
    float* q = malloc(sizeof(float) * nt * d);
    float* g[3];
    unsigned s = 7;
    for (long i = 0; i < nt * d; i++) { k[i] = frand(&s); v[i] = frand(&s); q[i] = frand(&s); }
    for (int j = 0; j < 3; j++) {
        g[j] = malloc(sizeof(float) * nt);
        for (long i = 0; i < nt; i++) g[j][i] = 0.3f + 0.4f * (frand(&s) + 0.5f);
    }
    double* st = malloc(sizeof(double) * B * H * 2 * P);
    double* y = malloc(sizeof(double) * nt * d);
    for (int read = 0; read < 3; read++) {
        for (long i = 0; i < B * H * 2 * P; i++) st[i] = i < B * H * P ? 0.1 * frand(&s) : 0.0;
        if (tmref_forward_read(d, depth, ex, b, B, H, T, k, v, q, g[0], g[1], g[2], st, y, read, 4) != 0)
            return 2;
    }
    if (tmref_retrieve(d, depth, ex, B, H, T, st, q, y, 4) != 0) return 3;
    printf("ok %g\n", y[0]);
    free(k); free(v); free(q); free(st); free(y);
    for (int j = 0; j < 3; j++) free(g[j]);
    return 0;
}
"""


def build_and_run(flags, tmp, name):
    drv = os.path.join(tmp, "driver.c")
    with open(drv, "w") as f:
        f.write(DRIVER)
    exe = os.path.join(tmp, name)
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11"] + flags + ["-o", exe, drv, SRC, "-lm", "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("flags,name", [
    (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"], "asan_ubsan"),
    (["-fsanitize=thread"], "tsan"),
])
def test_oracle_runs_clean_under_sanitizers(flags, name):
    with tempfile.TemporaryDirectory() as tmp:
        r = build_and_run(flags, tmp, name)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout + r.stderr
    assert "ERROR" not in r.stderr and "WARNING: ThreadSanitizer" not in r.stderr, r.stderr

"""The oracle's C source under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A small driver includes oracle/gla_oracle.c, reads seeded inputs from a file, runs the
forward pass in every direction (with an initial and a final state) and the backward
pass, and writes the results back.  It is built with gcc and the two sanitizers, with
every report fatal, on ragged non-square shapes.  The results must equal those of the
oracle library the other tests load.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import gla_inputs
import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "gla_oracle.c")

DRIVER = r'''
#include <stdio.h>
#include <stdlib.h>
#include "%s"

static double *take(FILE *f, long n) {
    double *p = malloc((size_t)n * sizeof(double));
    if (!p || fread(p, sizeof(double), (size_t)n, f) != (size_t)n) exit(3);
    return p;
}

int main(int argc, char **argv) {
    int B, H, gh, gw, dk, dv;
    if (argc != 9) return 2;
    B = atoi(argv[3]); H = atoi(argv[4]); gh = atoi(argv[5]); gw = atoi(argv[6]);
    dk = atoi(argv[7]); dv = atoi(argv[8]);
    const long nk = (long)B * H * gh * gw * dk, nv = (long)B * H * gh * gw * dv;
    const long ns = (long)B * H * dk * dv;
    FILE *in = fopen(argv[1], "rb");
    if (!in) return 4;
    double *q = take(in, nk), *k = take(in, nk), *v = take(in, nv), *g = take(in, nk);
    double *dout = take(in, nv), *s0 = take(in, ns), *dsf = take(in, ns);
    fclose(in);
    FILE *out = fopen(argv[2], "wb");
    if (!out) return 5;
    double *o = malloc(nv * sizeof(double)), *sf = malloc(ns * sizeof(double));
    double *dq = malloc(nk * sizeof(double)), *dkk = malloc(nk * sizeof(double));
    double *dvv = malloc(nv * sizeof(double)), *dg = malloc(nk * sizeof(double));
    double *ds0 = malloc(ns * sizeof(double));
    for (int d = 0; d < 4; ++d) {
        if (gla_oracle_f64(q, k, v, g, o, B, H, gh, gw, dk, dv, d, s0, sf, 2) < 1) return 6;
        fwrite(o, sizeof(double), nv, out);
        fwrite(sf, sizeof(double), ns, out);
        if (gla_oracle_bwd_f64(q, k, v, g, dout, s0, dsf, dq, dkk, dvv, dg, ds0, B, H, gh, gw, dk, dv,
                               d, 2) < 1) return 7;
        fwrite(dq, sizeof(double), nk, out);
        fwrite(dkk, sizeof(double), nk, out);
        fwrite(dvv, sizeof(double), nv, out);
        fwrite(dg, sizeof(double), nk, out);
        fwrite(ds0, sizeof(double), ns, out);
    }
    fclose(out);
    free(q); free(k); free(v); free(g); free(dout); free(s0); free(dsf);
    free(o); free(sf); free(dq); free(dkk); free(dvv); free(dg); free(ds0);
    return 0;
}
'''


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("shape", [(1, 2, 5, 7, 3, 5), (2, 1, 3, 9, 8, 4), (1, 1, 1, 1, 2, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_oracle_under_sanitizers(tmp_path, shape):
    B, H, gh, gw, dk, dv = shape
    q, k, v, g = (t.double().numpy() for t in gla_inputs.make_inputs(B, H, gh, gw, dk, dv, "f32", "light",
                                                                       seed=61))
    dout = gla_inputs.make_output_grad(v.shape, "f32", seed=62).double().numpy()
    rng = np.random.default_rng(63)
    s0 = rng.standard_normal((B, H, dk, dv))
    dsf = rng.standard_normal((B, H, dk, dv))
    driver = tmp_path / "driver.c"
    driver.write_text(DRIVER % SRC)
    exe = tmp_path / "driver"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", str(driver), "-o", str(exe),
                    "-lm"], check=True, capture_output=True, text=True)
    with open(tmp_path / "in.bin", "wb") as f:
        for a in (q, k, v, g, dout, s0, dsf):
            f.write(np.ascontiguousarray(a, dtype=np.float64).tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), str(tmp_path / "in.bin"), str(tmp_path / "out.bin"), *map(str, shape)],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    got = np.fromfile(tmp_path / "out.bin", dtype=np.float64)
    want = []
    for d in range(4):
        o, sf = oracle.gla_forward(q, k, v, g, d, s0=s0, want_state=True)
        want += [o.ravel(), sf.ravel()]
        grads = oracle.gla_backward(q, k, v, g, dout, d, s0=s0, ds_final=dsf, want_ds0=True)
        want += [x.ravel() for x in grads]
    want = np.concatenate(want)
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)

"""The boundary from C: a C99 program that includes include/phobos_sgemm.h
and links libphobos_sgemm.so, calling the entry points that need no GPU
(argument checks, configuration choice, the tuner's candidates and cache, the
host-resident planner, status strings).  It shows the header is plain C and
the library's exported names and types match it outside Python."""
import os
import subprocess

import fp32_gemm_02_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "phobos_sgemm.h"

static int failures = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAILED line %d: %s\n", __LINE__, #cond); ++failures; } } while (0)

int main(int argc, char** argv) {
    const char* cache = argc > 1 ? argv[1] : "tune.jsonl";
    float x = 0.0f;
    sgemm_config c;
    sgemm_config cands[64];
    sgemm_plan plan;
    int32_t n = -1;
    int i, k;
    FILE* f;

    EXPECT(sgemm_version() == PHOBOS_SGEMM_VERSION);
    /* argument checks, before any HIP call (BLAS-style numbering) */
    EXPECT(sgemm(-1, 4, 4, 1.0f, &x, 4, &x, 4, 0.0f, &x, 4, NULL) == -1);
    EXPECT(sgemm(4, 4, 8, 1.0f, &x, 4, &x, 4, 0.0f, &x, 4, NULL) == -6);
    EXPECT(sgemm(4, 4, 4, 1.0f, NULL, 4, &x, 4, 0.0f, &x, 4, NULL) == -5);
    EXPECT(sgemm(0, 4, 4, 1.0f, NULL, 4, NULL, 4, 0.0f, NULL, 4, NULL) == SGEMM_OK);
    EXPECT(sgemm_supertiled(4, 4, 4, 1.0f, &x, 4, &x, 4, 0.0f, &x, 4, 0, 4, 4, NULL) == -12);
    EXPECT(sgemm_tc(4, 4, 4, 1.0f, &x, 4, &x, 4, 0.0f, &x, 4, 99, NULL) == -12);
    EXPECT(flash_attention(4, 4, 32, &x, 64, &x, 64, &x, 64, &x, 64, 1.0f, NULL) == -3);
    EXPECT(strcmp(sgemm_status_string(SGEMM_OK), "success") == 0);
    EXPECT(sgemm_status_string(SGEMM_ERR_IO) != NULL);
    /* the compiled configurations and the built-in choice */
    k = sgemm_config_count();
    EXPECT(k > 0);
    for (i = 0; i < k; ++i) EXPECT(sgemm_config_at(i, &c) == SGEMM_OK && c.bm >= 32);
    EXPECT(sgemm_get_config(4096, 4096, 4096, 4096, 4096, 4096, &c) == SGEMM_OK);
    EXPECT(c.bm == 256 && c.bn == 256 && c.bk == 32 && c.wm == 4 && c.wn == 2);
    EXPECT(sgemm_tune_candidates(4096, 4096, 4096, cands, 64) > 0);
    /* the tuning cache: one entry in, the choice follows it, saved back out */
    f = fopen(cache, "w");
    EXPECT(f != NULL);
    if (f) {
        fprintf(f, "{\"M\": 777, \"N\": 555, \"K\": 333, \"lda\": 333, \"ldb\": 555, \"ldc\": 555, "
                   "\"bm\": 128, \"bn\": 128, \"bk\": 16, \"wm\": 2, \"wn\": 2}\n");
        fclose(f);
    }
    EXPECT(sgemm_tune_cache_load(cache, &n) == SGEMM_OK && n == 1);
    EXPECT(sgemm_get_config(777, 555, 333, 333, 555, 555, &c) == SGEMM_OK && c.bm == 128 &&
           c.bn == 128 && c.bk == 16);
    EXPECT(sgemm_tune_cache_save(cache, &n) == SGEMM_OK && n == 1);
    EXPECT(sgemm_tune_forget() == 1);
    EXPECT(sgemm_tune_cache_load(NULL, NULL) == -1);
    /* the host-resident planner runs on the host alone */
    EXPECT(sgemm_plan_supertiles(16384, 16384, 16384, 1.0f, (int64_t)2 << 30, NULL, &plan) ==
           SGEMM_OK);
    EXPECT(plan.TM >= 256 && plan.TN >= 256 && plan.TK >= 256 && plan.a_slots >= 1);
    printf("%d failures\n", failures);
    return failures != 0;
}
"""


def test_c_program_compiles_links_and_runs(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(g.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                         "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                         "-L" + libdir, "-lphobos_sgemm", "-Wl,-rpath," + libdir],
                        capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe), str(tmp_path / "tune.jsonl")], capture_output=True,
                         text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout

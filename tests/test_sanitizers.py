"""Sanitizer runs on the CPU: the C oracles under AddressSanitizer +
UndefinedBehaviorSanitizer and under ThreadSanitizer (their worker pools are
pthreads), and the C ABI's host-side argument validation under ASan + UBSan.

Each builds a small driver in a temporary directory, runs it and requires a
clean exit with no sanitizer report.  The oracle driver calls every oracle
entry point on small inputs (segment layouts with padding and negative IDs,
row subsets, probabilities, sensitivity sums, several threads).  The
validation driver calls every vdx_* entry point with arguments that fail
each check in turn and with valid ones (which end at the device check here,
where no GPU is visible); the launchers are replaced by stubs, since no
kernel runs.  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SOURCES = [os.path.join(ROOT, "oracle", f) for f in
                  ("attn_oracle.c", "natten_oracle.c", "attn_bwd_oracle.c", "rope_oracle.c")]
API_SOURCE = os.path.join(ROOT, "spatiotemporal_attention_amd", "csrc", "vdx_attn_api.hip")

ORACLE_DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int vdx_oracle_attn_fwd(const uint16_t *, const uint16_t *, const uint16_t *, const int32_t *,
                        const int32_t *, int64_t, int64_t, int64_t, int64_t, double, const int64_t *,
                        int64_t, double *, double *, double *, double *, int);
int vdx_oracle_natten3d_fwd(const uint16_t *, const uint16_t *, const uint16_t *, int64_t, int64_t,
                            int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double,
                            const int64_t *, int64_t, double *, double *, double *, int);
int vdx_oracle_attn_bwd(const uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *,
                        const int32_t *, const int32_t *, int64_t, int64_t, int64_t, int64_t, double,
                        double *, double *, double *, double *, double *, double *, int);
int vdx_oracle_attn_bwd_dq_rows(const uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *,
                                const int32_t *, const int32_t *, int64_t, int64_t, int64_t, int64_t,
                                double, const int64_t *, int64_t, double *, double *, int);
int vdx_oracle_rope3d(const uint16_t *, const int32_t *, const float *, const float *, const float *,
                      const float *, const float *, const float *, int64_t, int64_t, int64_t, int64_t,
                      int64_t, int64_t, int, int64_t, int64_t, int64_t, int64_t, uint16_t *, double *);
void vdx_oracle_round_bf16(const double *, int64_t, uint16_t *);

static uint32_t st = 12345u;
static uint16_t rnd_bf16(void) {
    st = st * 1664525u + 1013904223u;
    float f = ((int32_t)(st >> 8) - (1 << 23)) / (float)(1 << 23) * 2.0f;
    uint32_t w;
    memcpy(&w, &f, 4);
    return (uint16_t)(w >> 16);
}

int main(int argc, char **argv) {
    const int threads = argc > 1 ? atoi(argv[1]) : 4;
    enum { B = 2, S = 37, H = 2, D = 16, N = B * S * H * D };
    uint16_t *q = malloc(N * 2), *k = malloc(N * 2), *v = malloc(N * 2), *g = malloc(N * 2), *y = malloc(N * 2);
    double *o = malloc(N * 8), *t1 = malloc(N * 8), *t2 = malloc(N * 8), *t3 = malloc(N * 8);
    double *o2 = malloc(N * 8), *o3 = malloc(N * 8), *lse = malloc(B * H * S * 8), *pr = malloc(B * H * S * S * 8);
    int32_t seg[B * S], pos[B * S * 3];
    for (int i = 0; i < N; ++i) { q[i] = rnd_bf16(); k[i] = rnd_bf16(); v[i] = rnd_bf16(); g[i] = rnd_bf16(); }
    for (int i = 0; i < B * S; ++i) {
        seg[i] = (i % S) < 5 ? 0 : ((i % S) < 20 ? -3 : 7);
        pos[3 * i] = i % 3; pos[3 * i + 1] = (i / 3) % 4; pos[3 * i + 2] = (i % 5) - 1;
    }
    int64_t rows[3 * 6] = {0, 0, 0, 0, 1, 36, 1, 0, 4, 1, 1, 5, 1, 1, 20, 0, 0, 19};
    int rc = 0;
    rc |= vdx_oracle_attn_fwd(q, k, v, seg, seg, B, S, H, D, 0.3, NULL, 0, o, lse, pr, t1, threads);
    rc |= vdx_oracle_attn_fwd(q, k, v, NULL, NULL, B, S, H, D, 0.3, rows, 6, o2, lse, NULL, t2, threads) << 1;
    rc |= vdx_oracle_natten3d_fwd(q, k, v, 1, 3, 4, 6, 2, D, 3, 3, 5, 0.25, NULL, 0, o3, lse, t3, threads) << 2;
    rc |= vdx_oracle_attn_bwd(q, k, v, g, seg, seg, B, S, H, D, 0.3, o, o2, o3, t1, t2, t3, threads) << 3;
    rc |= vdx_oracle_attn_bwd_dq_rows(q, k, v, g, seg, seg, B, S, H, D, 0.3, rows, 6, o, t1, threads) << 4;
    float ct[3 * 2], stt[3 * 2], ch[4 * 3], sh[4 * 3], cw[4 * 3], sw[4 * 3];
    for (int i = 0; i < 6; ++i) { ct[i] = 0.5f; stt[i] = 0.25f; }
    for (int i = 0; i < 12; ++i) { ch[i] = cw[i] = 0.75f; sh[i] = sw[i] = -0.5f; }
    rc |= vdx_oracle_rope3d(q, pos, ct, stt, ch, sh, cw, sw, 3, 4, 4, 4, 6, 6, 1, B, S, H, D, y, o) << 5;
    rc |= vdx_oracle_rope3d(q, pos, ct, stt, ch, sh, cw, sw, 3, 4, 4, 4, 6, 6, 0, B, S, H, D, y, NULL) << 6;
    double vals[5] = {1.0 - 1.0 / 512, 3e-39, -2.5, 0.0, 1e38};
    uint16_t rb[5];
    vdx_oracle_round_bf16(vals, 5, rb);
    printf("rc=%d %04x\n", rc, rb[0]);
    free(q); free(k); free(v); free(g); free(y); free(o); free(t1); free(t2); free(t3); free(o2); free(o3);
    free(lse); free(pr);
    return rc;
}
"""

API_DRIVER = r"""
#include <stdio.h>
#include "vdx_attn.h"

int main(void) {
    char* A = (char*)0x10000;
    int bad = 0;
    /* forward */
    if (vdx_attn_fwd(0, A, A, 0, 0, A, (float*)A, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_NULL_PTR) bad |= 1;
    if (vdx_attn_fwd(A, A, A, (int*)A, 0, A, (float*)A, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_SEG_PAIR) bad |= 2;
    if (vdx_attn_fwd(A, A, A, 0, 0, A, (float*)A, 2147483647, 2147483647, 2147483647, 128, 0.1f, 0) != VDX_ERR_SHAPE) bad |= 4;
    if (vdx_attn_fwd(A, A, A, 0, 0, A, (float*)A, 1, 64, 1, 96, 0.1f, 0) != VDX_ERR_HEAD_DIM) bad |= 8;
    if (vdx_attn_fwd(A, A, A, 0, 0, A, (float*)A, 1, 64, 1, 64, -1.0f, 0) != VDX_ERR_SCALE) bad |= 16;
    if (vdx_attn_fwd(A + 2, A, A, 0, 0, A, (float*)A, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_ALIGN) bad |= 32;
    if (vdx_attn_fwd(A, A, A, 0, 0, A, (float*)A, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_DEVICE) bad |= 64;
    if (vdx_attn_fwd_ws(A, A, A, (int*)A, (int*)A, A, (float*)A, 0, 0, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_WORKSPACE)
        bad |= 131072;
    if (vdx_attn_fwd_ws(A, A, A, (int*)A, (int*)A, A, (float*)A, A, vdx_attn_fwd_workspace_size(1, 64, 1), 1, 64, 1,
                        64, 0.1f, 0) != VDX_ERR_DEVICE)
        bad |= 262144;
    if (vdx_attn_fwd_workspace_size(0, 5, 5) != 0) bad |= 524288;
    {
        vdx_rope3d rw = {(const int*)A, {(float*)A, (float*)A, (float*)A}, {(float*)A, (float*)A, (float*)A},
                         {4, 5, 6}, {20, 22, 22}, 1};
        if (vdx_rope3d_attn_fwd_ws(A, A, A, (int*)A, (int*)A, &rw, A, A, (float*)A, 0, 0, 1, 64, 1, 64, 0.1f, 0) !=
            VDX_ERR_WORKSPACE)
            bad |= 1048576;
    }
    /* neighbourhood */
    if (vdx_natten3d_fwd(A, A, A, A, (float*)A, 1, 4, 8, 32, 2, 128, 4, 3, 3, 0.1f, 0) != VDX_ERR_WINDOW) bad |= 128;
    if (vdx_natten3d_fwd(A, A, A, A, (float*)A, 1, 4, 8, 32, 2, 128, 3, 3, 3, 0.1f, 0) != VDX_ERR_DEVICE) bad |= 256;
    /* backward */
    if (vdx_attn_bwd(A, A, A, 0, 0, A, (float*)A, A, A, A, A, A, 1, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_WORKSPACE) bad |= 512;
    if (vdx_attn_bwd_workspace_size(-1, 5, 5) != 0 || vdx_attn_bwd_workspace_size(2147483647, 2147483647, 2147483647) != 0)
        bad |= 1024;
    if (vdx_attn_bwd_noalloc(A, A, A, 0, 0, A, (float*)A, A, A, A, A, 1, 1 << 20, 4, 128, 0.1f, 0) != VDX_ERR_SCRATCH)
        bad |= 2048;
    if (vdx_attn_bwd_noalloc(A, A, A, 0, 0, A, (float*)A, A, A, A, A, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_DEVICE)
        bad |= 4096;
    /* rotary embedding */
    vdx_rope3d r = {(const int*)A, {(float*)A, (float*)A, (float*)A}, {(float*)A, (float*)A, (float*)A},
                    {4, 5, 6}, {20, 22, 22}, 1};
    if (vdx_rope3d_apply(A, A, 0, 1, 64, 1, 64, 0) != VDX_ERR_ROPE) bad |= 8192;
    if (vdx_rope3d_apply(A, A, &r, 1, 64, 1, 64, 0) != VDX_ERR_DEVICE) bad |= 16384;
    r.dims[1] = 23;
    if (vdx_rope3d_attn_fwd(A, A, A, 0, 0, &r, A, A, (float*)A, 1, 64, 1, 64, 0.1f, 0) != VDX_ERR_ROPE) bad |= 32768;
    for (int s = -2; s < 14; ++s)
        if (vdx_status_str(s) == 0) bad |= 65536;
    printf("bad=%d abi=%d\n", bad, vdx_abi_version());
    return bad;
}
"""

LAUNCH_STUBS = r"""
#include <hip/hip_runtime_api.h>
#include "attn_fwd_launch.h"
namespace vdx {
hipError_t launch_attn_fwd(const AttnArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_attn_fwd_sched(const AttnArgs&, void*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_rope3d_attn_fwd_sched(const AttnArgs&, const Rope3DDev&, void*, hipStream_t) {
    return hipErrorInvalidValue;
}
size_t attn_fwd_workspace_bytes(int64_t B, int64_t S) {
    const int64_t nq = (S + 255) / 256, nk = (S + 63) / 64;
    return 256 + (size_t)((16 * B * nk + 255) / 256 * 256) + (size_t)((4 * B * nq + 255) / 256 * 256) + (size_t)(4 * B * nq);
}
hipError_t launch_rope3d_attn_fwd(const AttnArgs&, const Rope3DDev&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_rope3d_apply(const void*, void*, const Rope3DDev&, int, int, int, int, hipStream_t) {
    return hipErrorInvalidValue;
}
int64_t max_masked_seq() { return (int64_t)30720 * 64; }
int64_t queries_per_workgroup() { return 256; }
hipError_t launch_natten_fwd(const NattenArgs&, hipStream_t) { return hipErrorInvalidValue; }
int64_t natten_workgroups(const NattenArgs& a) { return (int64_t)a.B * a.H * a.NT * a.NH * a.NW / 256 + 1; }
size_t attn_bwd_workspace_bytes(int64_t B, int64_t S, int64_t H) {
    return (size_t)(8 * B * H * ((S + 63) / 64 * 64) + 16 * B * ((S + 127) / 128));
}
hipError_t launch_attn_bwd(const BwdArgs&, hipStream_t) { return hipErrorInvalidValue; }
int64_t bwd_max_masked_seq() { return (int64_t)14000 * 64; }
int64_t bwd_rows_per_workgroup() { return 128; }
}  // namespace vdx
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    return r


def _no_report(r):
    text = r.stdout + r.stderr
    return not any(s in text for s in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                                       "ERROR: LeakSanitizer"))


@pytest.fixture(scope="module")
def gcc():
    path = shutil.which("gcc")
    if path is None:
        pytest.skip("no C compiler")
    return path


@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_oracle_under_sanitizer(tmp_path, gcc, san):
    drv = tmp_path / "driver.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_san"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={san}",
           "-fno-sanitize-recover=all", "-pthread", str(drv), *ORACLE_SOURCES, "-o", str(exe), "-lm"]
    r = _run(cmd)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = _run([str(exe), "4"], env=env)
    assert r.returncode == 0 and _no_report(r), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "rc=0" in r.stdout


def test_host_validation_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc")
    csrc = os.path.dirname(API_SOURCE)
    (tmp_path / "stubs.cpp").write_text(LAUNCH_STUBS)
    (tmp_path / "driver.c").write_text(API_DRIVER)
    exe = tmp_path / "api_san"
    # -Xarch_host before each -fsanitize= keeps the device side of the .hip
    # file uninstrumented (only host code is checked here)
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
           API_SOURCE, str(tmp_path / "stubs.cpp"),
           "-x", "c++", str(tmp_path / "driver.c"), "-o", str(exe)]
    r = _run(cmd)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([str(exe)], env=env)
    if "a GPU is visible" in r.stdout:  # pragma: no cover
        pytest.skip("a GPU is visible")
    assert r.returncode == 0 and _no_report(r), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "bad=0" in r.stdout

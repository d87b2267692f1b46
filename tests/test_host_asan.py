"""The runtime's host code under AddressSanitizer (CPU, no GPU): the library
is rebuilt with host-side ASan (device code unchanged) and, in a child process
that preloads the ASan runtime, the C-ABI checks of test_abi.py run against
it, followed by a sweep of the workspace and cache sizing over many
configurations (the workspace planner walks every batch size and window
length, the GEMM scratch sizing every row count) and of spec_verify_init's
argument errors.  Any invalid host memory access ends the child with an ASan
report."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

DRIVER = r'''
import sys
import pytest
import speculative_decoding_verify_spec_amd as S
import synth
S.LIB_PATH = sys.argv[1]
assert S.lib()._name == sys.argv[1]
rc = pytest.main(["-q", "-m", "not gpu", "-p", "no:cacheprovider", sys.argv[2]])
if rc != 0:
    sys.exit(int(rc))
n = bad = 0
for shape in (synth.TOY, synth.MINI8B, synth.LLAMA8B):
    for mb in (1, 3, 16, 128):
        for rows in (1, 4, 8, 17, 128):
            for ctx in (64, 2112, 32832):
                for pages in (0, 96):
                    cfg = S.make_config(shape, mb, ctx, rows, kv_pages=pages)
                    ws = S.spec_workspace_bytes(cfg)
                    kv = S.spec_kv_cache_bytes(cfg)
                    w = [256] * shape.n_weights()
                    if ws == 0:  # a configuration the library rejects, by every call
                        assert kv == 0, (shape, mb, rows, ctx, pages)
                        assert S.spec_verify_init(cfg, w, 256, 256, 1 << 30, None, check=False)[0] == S.SPEC_ERR_SHAPE
                        bad += 1
                        continue
                    assert ws % 256 == 0 and kv > 0, (shape, mb, rows, ctx, pages)
                    st, h = S.spec_verify_init(cfg, w, 256, 256, ws - 1, None, check=False)
                    assert st == S.SPEC_ERR_CAPACITY and h is None
                    n += 1
assert n > 100
print(f"sized {n} configurations, {bad} rejected", flush=True)
'''


@pytest.mark.skipif(not ASAN_RT, reason="clang's ASan runtime is not installed")
def test_abi_and_sizing_under_host_asan(tmp_path):
    sys.path.insert(0, ROOT)
    from speculative_decoding_verify_spec_amd import build

    lib = build.build_host_asan(os.path.join(ROOT, "_build", "asan"))
    with open(lib, "rb") as fh:
        assert b"__asan_report_load" in fh.read(), "the library is not instrumented"
    drv = tmp_path / "drive.py"
    drv.write_text(DRIVER)
    # the ASan runtime goes first in the preload list; whatever the environment
    # already preloads stays after it
    pre = " ".join(x for x in (ASAN_RT[-1], os.environ.get("LD_PRELOAD", "")) if x)
    env = dict(os.environ, LD_PRELOAD=pre, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, str(drv), lib, os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out
    assert r.returncode == 0
    assert "sized" in out

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The fp64 oracle, built with gcc -fsanitize=address,undefined, runs every form on small ragged inputs (rotation,
  incoming state, several chunk sizes, the normalizations, the gradients, the epilogue) in a child process that
  preloads gcc's sanitizer runtime. Any out-of-bounds access, use after free or undefined operation aborts the
  child.
* The library's host side (argument checks, planning, workspace layouts, options, timers, status strings), built
  host-only with the sanitizers on the host pass, is driven in a child process over every entry point's rejection
  paths and every workspace query: calls that never reach a device.
Each child must exit 0 with no sanitizer report.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(cmd):
    path = subprocess.run(cmd, capture_output=True, text=True).stdout.strip()
    return path if path and os.path.isabs(path) and os.path.exists(path) else None


def _run_child(script, preload, tmp_path):
    env = dict(os.environ, **SAN_OPTS, LD_PRELOAD=preload, PYTHONPATH=ROOT)
    p = subprocess.run([sys.executable, "-c", textwrap.dedent(script)], env=env, capture_output=True, text=True,
                       cwd=str(tmp_path), timeout=600)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-shared", "-fPIC", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle",
                    "retention_oracle.c"), "-o", lib, "-lm"], check=True)
    out = _run_child("""
        import numpy as np
        import oracle
        oracle._LIB_PATH = %r
        oracle._lib = None
        rng = np.random.default_rng(3)
        for (B, N, H, dk, dv, C, pos0) in [(1, 1, 1, 2, 2, 1, 0), (2, 37, 3, 8, 4, 16, 5), (1, 70, 2, 16, 8, 64, 0),
                                            (1, 33, 1, 4, 6, 8, 1000)]:
            q = rng.standard_normal((B, N, H, dk)); k = rng.standard_normal((B, N, H, dk))
            v = rng.standard_normal((B, N, H, dv))
            s0 = rng.standard_normal((B, H, dk, dv)); z0 = rng.standard_normal((B, H, dk))
            g = np.linspace(0.8, 0.99, H); th = 10000.0 ** (-2.0 * np.arange(dk // 2) / dk)
            o1 = oracle.parallel(q, k, v, g, theta=th, pos0=pos0)
            o2, s2 = oracle.recurrent(q, k, v, g, theta=th, pos0=pos0)
            o3, s3 = oracle.chunkwise(q, k, v, g, C, theta=th, pos0=pos0)
            assert np.allclose(o1, o2) and np.allclose(o1, o3) and np.allclose(s2, s3)
            o4, s4 = oracle.chunkwise(q, k, v, g, C, theta=th, pos0=pos0, state_in=s0)
            rows = [0, N - 1, N // 2]
            oracle.parallel_rows(q, k, v, g, rows, theta=th, pos0=pos0)
            for norm in range(8):
                f = dict(scale=bool(norm & 1), decay=bool(norm & 2), scores=bool(norm & 4))
                oracle.parallel_normalized(q, k, v, g, theta=th, pos0=pos0, **f)
                oracle.normalized(q, k, v, g, C, theta=th, pos0=pos0, state_in=s0, z_in=z0, **f)
                oracle.normalized(q, k, v, g, 0, theta=th, pos0=pos0, state_in=s0, z_in=z0, **f)
            do = rng.standard_normal((B, N, H, dv))
            oracle.grad(q, k, v, do, g, theta=th, pos0=pos0)
            gate = rng.standard_normal((B, N, H, dv))
            oracle.msr_epilogue(o1, gate, np.ones(H * dv), np.zeros(H * dv), 1e-5)
            oracle.msr_epilogue(o1)
        print("oracle ok")
    """ % lib, asan, tmp_path)
    assert "oracle ok" in out


def test_host_abi_under_sanitizers(tmp_path):
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found or not _runtime(["which", "hipcc"]):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from linear_recurrent_sequence_amd import build as B
    csrc = os.path.join(ROOT, "linear_recurrent_sequence_amd", "csrc")
    flags = [f for f in B.COMMON if f != "--offload-arch=gfx950"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(csrc, "*.hip"))):
        o = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        objs.append(o)
        # the device pass as in the library's own build (no sanitizer there); nothing here reaches a device
        cmd = (["hipcc", "--offload-arch=gfx950"] + flags + B.EXTRA.get(os.path.basename(src), []) + san +
               ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                '-DRET_SOURCE_DIGEST="sanitized"', "-c", src, "-o", o])
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-3000:]
    lib = str(tmp_path / "libretention_san.so")
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"] + san + ["-o", lib] + objs, check=True,
                   capture_output=True)
    out = _run_child("""
        import ctypes
        lib = ctypes.CDLL(%r)
        from linear_recurrent_sequence_amd import retention as R
        lib.ret_source_digest.restype = ctypes.c_char_p
        lib.ret_status_string.restype = ctypes.c_char_p
        lib.ret_last_error.restype = ctypes.c_char_p
        assert lib.ret_abi_version() > 0 and lib.ret_source_digest() == b"sanitized"
        for s in range(-2, 12):
            assert lib.ret_status_string(s)
        o = R.Options()
        lib.ret_options_default(ctypes.byref(o))
        t = lib.ret_timer_create
        t.restype = ctypes.c_void_p
        tm = ctypes.c_void_p(t())
        ms, n = ctypes.c_double(), ctypes.c_int64()
        lib.ret_timer_reset(tm)
        lib.ret_timer_query(tm, b"ret_chunk_wide", ctypes.byref(ms), ctypes.byref(n))
        lib.ret_timer_query(tm, None, ctypes.byref(ms), ctypes.byref(n))
        lib.ret_timer_destroy(tm)
        lib.ret_timer_destroy(None)
        sz = ctypes.c_size_t
        for f in (lib.ret_chunkwise_workspace_bytes, lib.ret_chunkwise_bwd_workspace_bytes):
            f.restype = sz
        lib.ret_chunkwise_workspace_bytes_ex.restype = sz
        lib.ret_chunkwise_bwd_workspace_bytes_ex.restype = sz
        lib.ret_chunkwise_normalized_workspace_bytes.restype = sz
        total = 0
        for dt in (0, 1):
            for dk in (16, 32, 64, 128, 256, 512, 7, 0, -1):
                for dv in (16, 64, 128, 256, 384, 512, 5):
                    for (B_, N, H, C) in [(1, 1, 1, 64), (8, 2048, 8, 64), (1, 65536, 8, 128), (1, 8192, 16, 128),
                                          (3, 333, 2, 512), (1, 100, 3, 0), (1 << 20, 1 << 20, 64, 64)]:
                        total += lib.ret_chunkwise_workspace_bytes(B_, N, H, dk, dv, C, dt)
                        total += lib.ret_chunkwise_bwd_workspace_bytes(B_, N, H, dk, dv, C, dt)
                        total += lib.ret_chunkwise_normalized_workspace_bytes(B_, N, H, dk, dv, C, dt, None)
                        for variant in (0, 3, 4, 5):
                            o.variant = variant
                            o.segments = 3
                            total += lib.ret_chunkwise_workspace_bytes_ex(B_, N, H, dk, dv, C, dt, ctypes.byref(o))
                            total += lib.ret_chunkwise_bwd_workspace_bytes_ex(B_, N, H, dk, dv, C, dt,
                                                                              ctypes.byref(o))
                            total += lib.ret_chunkwise_normalized_workspace_bytes(B_, N, H, dk, dv, C, dt,
                                                                                  ctypes.byref(o))
        lib.ret_options_default(ctypes.byref(o))
        # rejections before any device work: null buffers, bad shapes, bad dtypes, unsupported sizes
        g = (ctypes.c_float * 4)(0.9, 0.9, 0.9, 0.9)
        th = (ctypes.c_double * 256)()
        nul, z64, zs = None, ctypes.c_int64(0), ctypes.c_size_t(0)
        st = []
        st.append(lib.ret_parallel_fwd(nul, nul, nul, nul, 1, 8, 1, 64, 64, 1, 1, g, th, z64, nul))
        st.append(lib.ret_chunkwise_fwd(nul, nul, nul, nul, 1, 8, 1, 64, 64, 1, 1, g, th, z64, 64, nul, nul, nul,
                                        zs, nul))
        st.append(lib.ret_chunkwise_fwd(nul, nul, nul, nul, -1, 8, 1, 64, 64, 1, 1, g, th, z64, 64, nul, nul, nul,
                                        zs, nul))
        st.append(lib.ret_chunkwise_fwd_ex(nul, nul, nul, nul, 1, 8, 1, 64, 64, 1, 1, g, th, z64, 0, nul, nul, nul,
                                           zs, nul, ctypes.byref(o)))
        st.append(lib.ret_recurrent_step(nul, nul, nul, nul, nul, 1, 1, 64, 64, 1, 1, g, th, z64, nul))
        st.append(lib.ret_recurrent_step_positions(nul, nul, nul, nul, nul, 1, 1, 64, 64, 1, 1, g, th, nul, nul))
        st.append(lib.ret_msr_epilogue(nul, nul, nul, nul, nul, ctypes.c_int64(1), 1, 64, 1, 1, 1,
                                       ctypes.c_float(1e-5), nul))
        st.append(lib.ret_chunkwise_bwd(nul, nul, nul, nul, nul, nul, nul, 1, 8, 1, 64, 64, 1, 1, g, th, z64, 64,
                                        nul, zs, nul))
        st.append(lib.ret_chunkwise_normalized_fwd(nul, nul, nul, nul, 1, 8, 1, 64, 64, 1, 1, g, th, z64, 64, 7,
                                                   nul, nul, nul, nul, nul, zs, nul, nul))
        st.append(lib.ret_recurrent_step_normalized(nul, nul, nul, nul, nul, nul, 1, 1, 64, 64, 1, 1, g, th, z64,
                                                    7, nul, nul))
        st.append(lib.ret_chunkwise_fwd_noalloc(nul, nul, nul, nul, 1, 8, 1, 64, 64, 1, 1, g, th, z64, 64, nul,
                                                nul, nul))
        st.append(lib.ret_chunkwise_check(nul, nul))
        assert all(s != 0 for s in st[:-1]), st
        assert lib.ret_last_error()
        print("host abi ok", total > 0)
    """ % lib, found[-1], tmp_path)
    assert "host abi ok True" in out

"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer (host only; no GPU).

* The oracle (oracle.c) and the input generator (synth.c), built with gcc
  -fsanitize=address,undefined, run every oracle pin plus a small workload of each
  configuration through every oracle function.
* The library's host code (argument checks, workspace sizing, launch set-up in
  api.hip and the launchers), built with hipcc with the sanitizers on the host side
  only, runs the C-ABI error and sizing checks of test_abi.py (no kernel is launched).

Each runs in a child process with the sanitizer runtime preloaded (it must come
first in the process); any report aborts the child and fails the test.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run_child(script, preload, tmp_path, timeout=600):
    path = tmp_path / "child.py"
    path.write_text(textwrap.dedent(script))
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, str(path)], env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, f"child exited {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r.stdout


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    libs = {}
    for name, src in (("oracle", "oracle/oracle.c"), ("synth", "synth/synth.c")):
        out = tmp_path / f"lib{name}_san.so"
        subprocess.run(["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-std=c11", os.path.join(ROOT, src), "-o",
                        str(out), "-lm"], check=True)
        libs[name] = str(out)
    preload = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    out = _run_child(f"""
        import sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, "tests")!r})
        import numpy as np
        import synth, oracle
        synth._LIB_PATH = {libs["synth"]!r}
        lib = oracle.load_variant({libs["oracle"]!r})
        oracle._lib = lib
        import oracle_pins
        for pin in oracle_pins.ALL_PINS:
            pin(lib)
        for cfg, kw in ((1, {{}}), (2, dict(n=3000, batch=2)), (3, dict(n=2100, batch=2)),
                        (4, dict(n=2000, batch=2, steps=3)), (5, dict(n=4000, batch=3, steps=3))):
            wl = synth.config(cfg, **kw)
            for step in range(wl.steps):
                if step:
                    wl.advance()
                c = oracle.Cache.of(wl)
                kps = wl.k_per_seq()
                idx, kth, s, o = oracle.decode_step(c, wl.q, kps, wl.k_max())
                oracle.dense(c, wl.q)
                sm = oracle.quest_summaries(c)
                u = oracle.quest_bounds(sm, c.sl, wl.q)
                oracle.quest_select(u, c.sl, (kps + 15) // 16, int(((kps + 15) // 16).max()))
                ch = np.tile(np.arange(16, dtype=np.int32) * 8, (wl.num_kv_heads, 1))
                oracle.label_scores(c, wl.q, ch)
                draws = np.arange(wl.batch * wl.num_q_heads * 5, dtype=np.uint32).reshape(wl.batch, wl.num_q_heads, 5)
                smp, w = oracle.sample_residual(idx, kps, c.sl, draws * np.uint32(797003437), np.full(wl.batch, 5, np.int32))
                oracle.attend_sampled(c, wl.q, idx, smp, w)
        print("sanitized oracle and generator ok")
    """, preload, tmp_path)
    assert "ok" in out


def test_library_host_code_under_asan_ubsan(tmp_path):
    from sparse_attention_decode_index_amd import build as b
    out = tmp_path / "libsparse_decode_san.so"
    flags = [f for f in b.HIPCC_FLAGS if f != "-O3"]
    host_san = []
    for f in SAN[:3]:
        host_san += ["-Xarch_host", f]
    subprocess.run([b.hipcc(), *flags, "-O1", "-g", *host_san, "-shared-libsan", f"-I{b.INCLUDE}",
                    *[os.path.join(b.CSRC, s) for s in b.SOURCES], "-o", str(out)], check=True,
                   capture_output=True)
    clang = os.path.join(os.path.dirname(b.hipcc()), "..", "lib", "llvm", "bin", "clang")
    preload = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.exists(preload), preload
    res = _run_child(f"""
        import sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, "tests")!r})
        import sparse_attention_decode_index_amd as sdi
        sdi._lib = sdi.load_library({str(out)!r})
        import pytest
        rc = pytest.main(["-q", "-p", "no:cacheprovider", {os.path.join(ROOT, "tests", "test_abi.py")!r},
                          "-k", "not missing_library"])
        sys.exit(int(rc))
    """, preload, tmp_path)
    assert "passed" in res

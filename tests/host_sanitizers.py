"""Run the CPU test suite with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code (CPU only; no GPU is touched).

    python tests/host_sanitizers.py

Copies the source tree to a temporary directory and, there,
* builds libkda.so with the sanitizers on the host side of every source
  (each ``-fsanitize=`` behind ``-Xarch_host``, so the gfx950 code objects
  are built as usual): the C ABI's validation, workspace carve-up and launch
  plumbing in kda_api.cpp and the host halves of the kernel sources;
* builds the C oracle with the same sanitizers (clang, without OpenMP);
* runs ``pytest tests -m "not gpu"`` there with the sanitizer runtime
  preloaded into the Python process (leak checking off: the interpreter and
  its libraries keep memory until exit by design).
Exits with pytest's status; a sanitizer report aborts the run.
"""
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["address", "undefined"]
COPY = ["gated_delta_rule_97_amd", "include", "oracle", "tests", "workloads", "pytest.ini"]


def run(cmd, **kw):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def main():
    rt = subprocess.run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.exists(rt):
        sys.exit(f"no ASan runtime at {rt}")
    tmp = tempfile.mkdtemp(prefix="kda_san_")
    try:
        for name in COPY:
            src = os.path.join(ROOT, name)
            dst = os.path.join(tmp, name)
            if os.path.isdir(src):
                shutil.copytree(src, dst, ignore=shutil.ignore_patterns("_build", "*.so", "__pycache__"))
            else:
                shutil.copy2(src, dst)
        pkg = os.path.join(tmp, "gated_delta_rule_97_amd")
        sys.path.insert(0, pkg)
        import build as kbuild  # the copy's build script
        host_san = []
        for s in SAN:
            host_san += ["-Xarch_host", f"-fsanitize={s}"]
        kbuild.FLAGS = kbuild.FLAGS + host_san + ["-Xarch_host", "-fno-omit-frame-pointer",
                                                  "-Xarch_host", "-fno-sanitize-recover=all"]
        kbuild.LINK_FLAGS = ["-fsanitize=" + ",".join(SAN), "-shared-libsan"]
        kbuild.build()
        orc = os.path.join(tmp, "oracle")
        run([os.path.join(LLVM, "clang"), "-O1", "-g", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
             "-ffp-contract=off", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", os.path.join(orc, "kda_oracle.c"), "-o",
             os.path.join(orc, "libkda_oracle.so"), "-lm"])
        env = dict(os.environ)
        env["LD_PRELOAD"] = rt
        env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:abort_on_error=1"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-q", "-s", "-p", "no:cacheprovider"],
                           cwd=tmp, env=env)
        print(f"sanitized CPU suite: exit status {r.returncode}", flush=True)
        return r.returncode
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    sys.exit(main())

"""Build and run the sanitizer drivers (CPU only, no GPU needed).

    python tests/sanitizers/build_and_run.py [oracle|abi]

oracle: oracle/moe_oracle.c + oracle_driver.c with gcc, AddressSanitizer and
        UndefinedBehaviorSanitizer (leak checking on), no OpenMP.
abi:    libmoe's C-ABI layer (csrc/capi.hip) compiled by hipcc with both
        sanitizers on its host code only (-Xarch_host before each flag; the
        GPU code is built as usual), linked with the library's other objects
        from the regular build (_build/), and abi_driver.cpp compiled and
        linked by the same clang with both sanitizers.
Each prints the driver's last line and returns its exit status; the build
products go to _build/sanitize/.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(ROOT, "sparse_moe_layer_bias_amd", "csrc")
INC = os.path.join(ROOT, "include")


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    if r.returncode != 0:
        raise RuntimeError("%s failed (%d):\n%s\n%s" % (cmd[0], r.returncode, r.stdout[-3000:],
                                                         r.stderr[-3000:]))
    return r


def oracle():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-mfma",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-Wall", "-Wno-unknown-pragmas", os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    return r.returncode, (r.stdout + r.stderr).strip()


def abi():
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OUT, exist_ok=True)
    base = ["-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INC, "-I", CSRC, "-Xclang",
            "-target-feature", "-Xclang", "-packed-fp32-ops"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        o = os.path.join(OUT, f + ".o")
        extra = ["-O1", "-g", *san] if f == "capi.hip" else ["-O3"]
        _run([HIPCC, *extra, *base, "-c", os.path.join(CSRC, f), "-o", o])
        return o

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    capi_o, objs = objs[srcs.index("capi.hip")], [o for o in objs if "capi.hip" not in o]
    lib = os.path.join(OUT, "libmoe_sanitize.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", capi_o, *objs, "-o", lib])
    exe = os.path.join(OUT, "abi_driver")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", INC,
          os.path.join(HERE, "abi_driver.cpp"), lib, "-Wl,-rpath," + OUT, "-o", exe])
    # the HIP runtime's own allocations at exit are not this code's: no leak check
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    return r.returncode, (r.stdout + r.stderr).strip()


if __name__ == "__main__":
    which = sys.argv[1:] or ["oracle", "abi"]
    rc = 0
    for w in which:
        code, out = {"oracle": oracle, "abi": abi}[w]()
        print("%s: rc=%d\n%s" % (w, code, out[-2000:]))
        rc = rc or code
    sys.exit(rc)

"""Build libflux3.so (the HIP kernels and the C ABI) for gfx950, in-tree.

python -m latent_flow_matching_flux_amd.build               the library
python -m latent_flow_matching_flux_amd.build --sanitize    a CPU-side check:
    the host code (validation, workspace carving, launch set-up) built with
    AddressSanitizer and UndefinedBehaviorSanitizer into _build/sanitize/,
    then tests/test_abi_cpu.py run against that copy (no GPU is touched:
    those tests only make calls that fail validation before any enqueue).
    The device code is built as usual; the sanitizers apply to host code only.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libflux3.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay disabled: the compiler must not emit them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]
# host-only sanitizers (each flag bound to the host compilation)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]

SOURCES = ["rope.hip", "ln_modulate.hip", "gemm.hip", "attention.hip", "modulation.hip", "quant.hip",
           "sampler.hip", "noalloc.hip", "abi.cpp"]


def _compile(src, defines=(), build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *extra, *[f"-D{d}" for d in defines], *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, defines=(), out=LIB, build_dir=BUILD, sanitize=False):
    """Compile every source and link libflux3.so.  `defines` (NAME=VALUE
    strings) select compile-time kernel parameters; `out`/`build_dir` place
    the result elsewhere than the package directory; `sanitize` instruments
    the host code with AddressSanitizer and UndefinedBehaviorSanitizer."""
    os.makedirs(build_dir, exist_ok=True)
    extra = HOST_SANITIZE if sanitize else ()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda src: _compile(src, defines, build_dir, extra), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = out + ".tmp"
    link = ["-shared-libsan", *HOST_SANITIZE] if sanitize else []
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def sanitizer_runtime():
    """The clang AddressSanitizer runtime the instrumented library links."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def sanitize_check():
    """Builds the instrumented copy and runs the host-side ABI tests on it;
    returns pytest's exit status (non-zero also when a sanitizer reports)."""
    bdir = os.path.join(BUILD, "sanitize")
    lib = build(verbose=False, out=os.path.join(bdir, "libflux3_san.so"), build_dir=bdir,
                sanitize=True)
    env = dict(os.environ)
    env["FLUX3_LIB"] = lib
    env["LD_PRELOAD"] = sanitizer_runtime()
    # python itself is not instrumented: its own allocations are not leaks
    # of the library; any other report ends the run with a non-zero status
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_cpu.py")]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        sys.exit(sanitize_check())
    print(build(verbose=True))

"""Build libpa.so (gfx950) in-tree with hipcc.

    python -m paged_kv_cache_store_amd.build

Every HIP source under csrc/ is compiled for gfx950 only and linked into
paged_kv_cache_store_amd/libpa.so next to this file. Flags:
* -O3, -fPIC, --offload-arch=gfx950;
* packed-fp32 instructions disabled (-target-feature -packed-fp32-ops);
* IEEE-correct float32 division kept explicit
  (-fhip-fp32-correctly-rounded-divide-sqrt): the fp8 store depends on it.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["api.hip", "store_kv.hip", "decode.hip", "prefill.hip", "rmsnorm.hip", "block_manager.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link libpa.so (or `out`); returns the library path.
    `defines` are extra -D macros (tuning variants of the kernels)."""
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.rsplit(".", 1)[0] + ".o")
            cmd = [HIPCC, *DEVICE_FLAGS, *["-D" + d for d in defines], "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            cmds.append(cmd)
            objs.append(obj)
        # one compiler process per source, at most as many as usable cores
        workers = max(1, min(len(cmds), len(os.sched_getaffinity(0)), 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(_run, cmds))
        out_tmp = os.path.join(tmp, "libpa.so")
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp])
        shutil.move(out_tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

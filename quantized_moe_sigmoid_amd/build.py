"""Build libcolimoe.so (the HIP library) in-tree with hipcc for gfx950.

Every csrc/*.hip file is compiled to its own object in parallel, then the objects
are linked into the shared library. Two variants come out of the same sources:
  libcolimoe.so       the product library;
  libcolimoe_taps.so  the same code compiled with COLI_TAPS, which adds the test-only
                      entry points of include/coli_moe_taps.h (pre-SiLU gate/up taps).
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libcolimoe.so")
TAPS_LIB_PATH = os.path.join(HERE, "libcolimoe_taps.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (v_pk_*_f32 are not generated)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 division correctly rounded: Q8_0 codes are defined by x / d
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _jobs() -> int:
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit():
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def _compile(src: str, obj: str, defines, verbose: bool):
    cmd = ["hipcc", *HIP_FLAGS, *defines, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")


def _link(objs, out: str, verbose: bool):
    tmp = out + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, taps: bool = True) -> str:
    """Compile both variants (the taps one unless taps=False); returns the product path."""
    variants = [("prod", [], LIB_PATH)]
    if taps:
        variants.append(("taps", ["-DCOLI_TAPS"], TAPS_LIB_PATH))
    jobs = []
    for name, defines, _ in variants:
        d = os.path.join(OBJ_DIR, name)
        os.makedirs(d, exist_ok=True)
        for src in sources():
            jobs.append((src, os.path.join(d, os.path.basename(src) + ".o"), defines))
    # the largest translation units first, so the pool ends evenly
    jobs.sort(key=lambda j: -os.path.getsize(j[0]))
    with ThreadPoolExecutor(_jobs()) as ex:
        for f in [ex.submit(_compile, s, o, dfs, verbose) for s, o, dfs in jobs]:
            f.result()
    for name, _, out in variants:
        d = os.path.join(OBJ_DIR, name)
        _link([os.path.join(d, os.path.basename(s) + ".o") for s in sources()], out, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

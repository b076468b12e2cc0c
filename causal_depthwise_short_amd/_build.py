"""Build libcconv.so (and the flat-copy roofline library) for gfx950 with hipcc, in-tree.

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel), then linked
into a shared library next to this file. All device code is built with packed-fp32
instructions disabled and without floating-point contraction (FMAs are written explicitly).
"""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}",
]

LIBS = {
    "libcconv.so": [
        "cconv_api.hip", "cconv_fwd.hip", "cconv_fwd_extra.hip", "cconv_bwd.hip", "cconv_bwd_extra.hip",
        "cconv_update.hip", "cconv_seq.hip",
    ],
    "libcconv_roofline.so": ["roofline_copy.hip"],
}


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> list[Path]:
    """Compile and link every library. Returns the paths of the built libraries."""
    BUILD.mkdir(exist_ok=True)
    sources = sorted({s for srcs in LIBS.values() for s in srcs})
    jobs = min(len(sources), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = dict(zip(sources, ex.map(lambda s: _compile(CSRC / s), sources)))
    out = []
    for lib, srcs in LIBS.items():
        target = PKG / lib
        tmp = target.with_suffix(".so.tmp")
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[str(objs[s]) for s in srcs], "-o", str(tmp)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {lib} failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, target)
        out.append(target)
        if verbose:
            print(f"built {target}")
    return out


if __name__ == "__main__":
    build(verbose=True)

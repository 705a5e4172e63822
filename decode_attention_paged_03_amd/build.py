"""Build libpa.so (the HIP library) in-tree with hipcc for gfx950.

    python -m decode_attention_paged_03_amd.build [-v] [--asm DIR]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = [os.path.join(CSRC, "pa_kernels.hip"), os.path.join(CSRC, "pa_append.hip"),
           os.path.join(CSRC, "pa_noalloc.hip"), os.path.join(CSRC, "pa_api.cpp")]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # no operand canonicalisation around fmaxf; NaN inputs still propagate through
          # the arithmetic (that is hardware behaviour), the kernels test for none
          "-fno-honor-nans"]


def build(verbose: bool = False, asm_dir: str | None = None, defines=(), out: str = LIB,
          build_dir: str | None = None) -> str:
    """Compile the library; ``defines`` (e.g. ["PA_WAVES=8"]) override compile-time tunables."""
    objs = []
    build_dir = build_dir or os.path.join(PKG, "_build")
    extra = [f"-D{d}" for d in defines]
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        src = SOURCES[0]
        cmd = [HIPCC, *COMMON, *extra, "--cuda-device-only", "-S", src, "-o",
               os.path.join(asm_dir, "pa_kernels.s"), "-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, check=True, capture_output=True, text=True)
        with open(os.path.join(asm_dir, "resource_usage.txt"), "w") as f:
            f.write(r.stderr)
    return out


_FIELDS = (("TotalSGPRs", "sgpr"), ("VGPRs", "vgpr"), ("AGPRs", "agpr"),
           ("ScratchSize [bytes/lane]", "scratch"), ("Occupancy [waves/SIMD]", "waves/simd"),
           ("SGPRs Spill", "sgpr_spill"), ("VGPRs Spill", "vgpr_spill"),
           ("LDS Size [bytes/block]", "lds"))


def parse_resource_usage(text: str) -> dict:
    """{mangled kernel name: {field: int}} from clang's -Rpass-analysis=kernel-resource-usage
    remarks."""
    import re
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\d+) \[", line)
        if m and cur is not None:
            for name, key in _FIELDS:
                if m.group(1) == name:
                    cur[key] = int(m.group(2))
    return out


def short_kernel_name(mangled: str) -> str:
    """'pa_decode_balanced<128,4,1,12,0,1>' from an Itanium-mangled kernel name in this
    library (integer and bool template arguments only)."""
    import re
    m = re.search(r"N_1(\d+)(pa_\w+)", mangled) or re.search(r"(\d+)(pa_\w+)", mangled)
    if not m:
        return mangled
    n = int(m.group(1))
    name = m.group(2)[:n]
    rest = m.group(2)[n:]
    if not rest.startswith("I"):
        return name
    args = re.findall(r"L[ib](\d+)E", rest[:rest.find("EE") + 2] if "EE" in rest else rest)
    return f"{name}<{','.join(args)}>"


def resource_table(text: str) -> str:
    """One line per kernel: registers, scratch, occupancy and LDS."""
    rows = sorted((short_kernel_name(name), f) for name, f in parse_resource_usage(text).items())
    cols = [key for _, key in _FIELDS]
    lines = [f"{'kernel':<40} " + " ".join(f"{c:>10}" for c in cols)]
    for short, f in rows:
        lines.append(f"{short:<40} " + " ".join(f"{f.get(c, -1):>10}" for c in cols))
    return "\n".join(lines)


if __name__ == "__main__":
    asm = None
    if "--asm" in sys.argv:
        asm = sys.argv[sys.argv.index("--asm") + 1]
    print(build(verbose="-v" in sys.argv, asm_dir=asm))

"""Build libfa355.so (attention) and libfa355_micro.so (machine microbenchmarks)
in-tree with hipcc for gfx950.

    python -m exact_io_aware_19_amd.build [--verbose]

Each source is compiled separately (parallel), then linked into its shared library
next to this file.  Kernel resource usage (VGPR/AGPR/LDS/spills) is written to
``_build/resource_usage.txt`` for inspection.
"""

import argparse
import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libfa355.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_api.cpp"]
# sources of the attention library's kernels (a profile taken on other ones is stale)
KERNEL_SOURCES = SOURCES + ["common.hpp", "fa_kernels.hpp"]
MICRO_SOURCES = ["micro.hip"]
MICRO_LIB_PATH = os.path.join(PKG_DIR, "libfa355_micro.so")

COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm required to build the HIP library)")


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    else:
        cmd = [_hipcc(), "-x", "hip", *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose:
        print(" ".join(cmd))
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stderr}")
    return obj, r.stderr


# Sources whose kernels issue MFMAs as inline assembly (the compiler inserts no wait
# states around those): their device assembly is checked after the build.
ASM_CHECKED = ["fa_bwd.hip"]
_MFMA_AGPR_B = re.compile(r"v_mfma_\S+\s+\S+,\s*\S+,\s*a\[(\d+):(\d+)\]")
_AGPR_WRITE = re.compile(r"v_accvgpr_write_b32\s+a(\d+),")


def check_inline_mfma_operands(asm_text, window=8):
    """Find inline-asm MFMAs whose B operand (accumulation registers) was written by a
    v_accvgpr_write among the `window` instructions before it.  The compiler does not
    know an inline-asm product is an MFMA, so it inserts no wait states after such a
    write and the product reads stale operands.  Returns the offending snippets."""
    lines = asm_text.splitlines()
    bad = []
    for i, line in enumerate(lines):
        m = _MFMA_AGPR_B.search(line)
        if not m or i == 0 or "ASMSTART" not in lines[i - 1]:
            continue
        lo, hi = int(m.group(1)), int(m.group(2))
        seen = 0
        for j in range(i - 1, -1, -1):
            t = lines[j].strip()
            if not t or t.startswith(";") or t.startswith("."):
                continue
            seen += 1
            if seen > window:
                break
            w = _AGPR_WRITE.search(t)
            if w and lo <= int(w.group(1)) <= hi:
                bad.append("\n".join(lines[j:i + 1]))
                break
    return bad


def _device_asm(src):
    out = os.path.join(BUILD_DIR, src + ".s")
    cmd = [_hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device assembly of {src} failed:\n{r.stderr}")
    with open(out) as f:
        return f.read()


def _link(objs, path, verbose):
    tmp = path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(path)} failed:\n{r.stderr}")
    os.replace(tmp, path)
    if verbose:
        print(f"built {path}")


def _resource_table(remarks):
    """Markdown table of the compiler's per-kernel resource remarks (registers, scratch,
    static LDS, occupancy); kernel names demangled with c++filt when it is there."""
    rows, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: +(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)", line)
        if not m:
            continue
        key, val = m.groups()
        if key == "Function Name":
            cur = {"name": val}
            rows.append(cur)
        elif cur is not None:
            cur[key] = val
    names = [r["name"] for r in rows]
    filt = shutil.which("c++filt")
    if filt and names:
        r = subprocess.run([filt], input="\n".join(names), capture_output=True, text=True)
        if r.returncode == 0 and len(r.stdout.splitlines()) == len(names):
            names = r.stdout.splitlines()
    out = ["| kernel | VGPRs | AGPRs | SGPRs | spilled VGPRs | scratch bytes/lane | static LDS bytes | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|"]
    for r, n in sorted(zip(rows, names), key=lambda x: x[1]):
        n = n.replace("void ", "", 1).replace("fa355::(anonymous namespace)::", "").split("(")[0]
        out.append("| `%s` | %s | %s | %s | %s | %s | %s | %s |" % (
            n, r.get("VGPRs"), r.get("AGPRs"), r.get("TotalSGPRs"), r.get("VGPRs Spill"),
            r.get("ScratchSize [bytes/lane]"), r.get("LDS Size [bytes/block]"), r.get("Occupancy [waves/SIMD]")))
    return "\n".join(out) + "\n"


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + MICRO_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs) + len(ASM_CHECKED)) as ex:
        asm = {s: ex.submit(_device_asm, s) for s in ASM_CHECKED}
        results = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
        for s, fut in asm.items():
            bad = check_inline_mfma_operands(fut.result())
            if bad:
                raise RuntimeError(f"{s}: {len(bad)} inline-asm MFMA(s) read accumulation registers written just "
                                   f"before them (no wait states); first:\n{bad[0]}")
    usage = "\n".join(err for _, err in results.values() if "resource usage" in err.lower() or "remark" in err)
    with open(os.path.join(BUILD_DIR, "resource_usage.txt"), "w") as f:
        f.write(usage)
    with open(os.path.join(BUILD_DIR, "resource_usage.md"), "w") as f:
        f.write(_resource_table(usage))
    _link([results[s][0] for s in SOURCES], LIB_PATH, verbose)
    _link([results[s][0] for s in MICRO_SOURCES], MICRO_LIB_PATH, verbose)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    build(verbose=args.verbose)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Build libw4a8.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Every translation unit is compiled in parallel, then linked into
``bit_group_quantized_act_amd/libw4a8.so`` (replaced atomically).  The benchmark's HBM read probe
(csrc/stream_probe.hip) is built into its own ``libw4a8_probe.so``, outside the layer's C ABI.
Flags:
  --offload-arch=gfx950                       MI355X only, no other targets
  -fhip-fp32-correctly-rounded-divide-sqrt    IEEE fp32 division (the prepass is bit-exact)
  -target-feature -packed-fp32-ops            no packed fp32 VALU instructions in device code
  -amdgpu-mfma-vgpr-form                      MFMA results in VGPRs, where the VALU epilogue reads
                                              them (no accumulator-register copies)
The GEMM kernels are also compiled to device assembly, and the build fails if any of them uses
scratch (see NO_SCRATCH).
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libw4a8.so")
PROBE_LIB = os.path.join(HERE, "libw4a8_probe.so")
PROBE_SOURCE = "stream_probe.hip"
SOURCES = ["api.hip", "pack.hip", "prep.hip", "gemv.hip", "gemm.hip", "tail.hip", "a16.hip",
           "attn.hip", "w8.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4a8)")


def _quiet(stderr: str) -> str:
    # hipcc's host pass does not know the device-only target feature; that warning is noise.
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


# The GEMM's stage wait counts the vector memory accesses it issues itself; a register spill
# would add scratch accesses to that count and make the wait too weak.  Its device assembly is
# therefore built too and every GEMM kernel must show a zero private segment (no scratch).
NO_SCRATCH = {"gemm.hip": "gemm_kernel"}


def check_no_scratch(asm_path: str, kernel_substr: str) -> None:
    name = None
    bad = []
    with open(asm_path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith(".amdhsa_kernel "):
                name = line.split()[1]
            elif line.startswith(".amdhsa_private_segment_fixed_size") and name \
                    and kernel_substr in name and int(line.split()[1]) != 0:
                bad.append((name, int(line.split()[1])))
            elif line.startswith(".end_amdhsa_kernel"):
                name = None
    if bad:
        raise RuntimeError("kernels use scratch (register spills), which their wait counts do not "
                           "allow: " + ", ".join(f"{n} ({b} bytes)" for n, b in bad))


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source and link libw4a8.so.  Always rebuilds.  Returns the path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = HIPCC_FLAGS + list(extra_flags or [])
    procs = []
    objs = []
    asm_checks = []
    for src, kernel in NO_SCRATCH.items():
        asm = os.path.join(BUILD_DIR, src.replace(".hip", ".device.s"))
        asm_checks.append((asm, kernel))
        cmd = [cc] + flags + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
        procs.append((src + " (device assembly)",
                      subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                       text=True)))
    probe_tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    procs.append((PROBE_SOURCE, subprocess.Popen(
        [cc] + flags + ["-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_tmp],
        stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    tmp = LIB + ".tmp%d" % os.getpid()
    try:
        failed = []
        for src, p in procs:
            out, err = p.communicate()
            err = _quiet(err)
            if p.returncode != 0:
                failed.append(f"{src}:\n{err}")
            elif verbose and err.strip():
                print(err)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        for asm, kernel in asm_checks:
            check_no_scratch(asm, kernel)
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + _quiet(r.stderr))
        os.replace(tmp, LIB)
        os.replace(probe_tmp, PROBE_LIB)
    finally:
        # a failed build leaves no partial library behind
        for leftover in (tmp, probe_tmp):
            if os.path.exists(leftover):
                os.remove(leftover)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

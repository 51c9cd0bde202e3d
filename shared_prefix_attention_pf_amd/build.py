"""Build libpf.so (the C-ABI library) in-tree with hipcc for gfx950.

    python shared_prefix_attention_pf_amd/build.py

Compiles every source under csrc/ into shared_prefix_attention_pf_amd/libpf.so.
Packed fp32 VALU instructions are disabled for all device code.
"""
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpf.so")
SOURCES = ["pf_api.cpp", "pf_prep.hip", "pf_attn_bf16.hip", "pf_attn_f32.hip", "pf_logprob.hip"]
ARCH = os.environ.get("PF_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpf.so)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", INCLUDE, "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA builtins produce VGPR results (they feed VALU code); the long-lived
        # accumulators are placed in AGPRs explicitly by the kernels
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
    ]


def check_wait_states(cc: str, tmp: str, verbose: bool = False) -> None:
    """Generate the gfx950 assembly of the bf16 and fp32 attention kernels and
    check that no instruction touches an inline-asm MFMA's destination within
    its latency (see asm_check.py), and that nothing spills to scratch.
    Raises on a violation."""
    sys.path.insert(0, PKG)
    import asm_check  # noqa: E402  (module beside this file)
    for name, wait_states, own_m0 in (("pf_attn_bf16", asm_check.WAIT_STATES, True),
                                      ("pf_attn_f32", asm_check.WAIT_STATES_16PASS, False)):
        src = os.path.join(CSRC, name + ".hip")
        asm = os.path.join(tmp, name + ".s")
        cmd = [cc] + common_flags() + ["--cuda-device-only", "-S", src, "-o", asm]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        with open(asm) as fh:
            lines = fh.readlines()
        bad = asm_check.check(lines, wait_states)
        bad += asm_check.check_no_stack(lines)
        # the bf16 kernels set M0 in their own staging asm; the fp32 kernels
        # stage through builtins, for which the compiler sets M0 itself
        if own_m0:
            bad += asm_check.check_m0(lines)
        if bad:
            for no, msg in bad[:20]:
                print(f"{name}.s:{no}: {msg}", file=sys.stderr)
            raise RuntimeError(f"{len(bad)} MFMA wait-state violation(s) in {name}.hip")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="pf_build_") as tmp:
        check_wait_states(cc, tmp, verbose)
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            if resource_usage and src.endswith(".hip"):
                cmd.append("-Rpass-analysis=kernel-resource-usage")
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libpf.so")
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        shutil.copyfile(tmp_lib, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--usage" in sys.argv))

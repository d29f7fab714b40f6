"""Builds tests/c_abi_parity (a C program that uses libspecverify.so through its
C ABI alone and checks it against the oracle) with gcc; called by the
repository's build step so that GPU runs find it ready."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_parity.c")
BIN = os.path.join(HERE, "c_abi_parity")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "lossless_draft_verification_02_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", orc,
           SRC, "-o", BIN,
           "-L", pkg, "-lspecverify", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../lossless_draft_verification_02_amd:$ORIGIN/../oracle:" + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build())

"""Builds tests/c_abi/plora_c_abi_test: plain C against include/plora.h,
linked to the in-tree libplora.so, the HIP runtime and the fp64 oracle
(test infrastructure)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "plora_c_abi_test")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    libdir = os.path.join(ROOT, "packed_adapter_lora_amd")
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-fopenmp", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "plora_c_abi_test.c"), os.path.join(ROOT, "oracle", "plora_oracle.c"),
           "-L", libdir, "-lplora", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../packed_adapter_lora_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm",
           "-o", BIN + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())

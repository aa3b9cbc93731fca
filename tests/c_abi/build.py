"""Compile tests/c_abi/abi_demo.c (plain C11 with gcc) against the library's header,
libdecode_attention.so, the HIP runtime and the C oracle.  Test infrastructure."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "abi_demo")
LIBDIR = os.path.join(ROOT, "decode_attention_07_amd")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-fopenmp",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include",
           os.path.join(HERE, "abi_demo.c"), os.path.join(ROOT, "oracle", "decode_oracle.c"),
           "-L", LIBDIR, "-ldecode_attention", "-Wl,-rpath,$ORIGIN/../../decode_attention_07_amd",
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm",
           "-o", BIN + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())

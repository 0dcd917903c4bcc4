"""Build the plain C consumer of the C ABI (tests/c_abi_check.c) into tests/_bin/.

It links the library, the CPU oracle and the shared generators through their shared objects
(found next to the binary through a relative rpath, so the tree can move) and the HIP
runtime.  gcc compiles it as C11: the public header must stay valid C.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BIN = os.path.join(HERE, "_bin", "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compile_cmd(out: str, syntax_only: bool = False) -> list:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi_check.c")]
    if syntax_only:
        return cmd + ["-fsyntax-only"]
    rpath = ":".join("$ORIGIN/../../" + d for d in ("fp8_gemv_amd", "oracle", "synth"))
    return cmd + ["-L", os.path.join(ROOT, "fp8_gemv_amd"), "-lfp8_gemv",
                  "-L", os.path.join(ROOT, "oracle"), "-loracle",
                  "-L", os.path.join(ROOT, "synth"), "-lsynth",
                  "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
                  "-Wl,-rpath," + rpath, "-o", out]


def build() -> str:
    """Compile the checker (the three shared objects must be built first); returns its path."""
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    tmp = BIN + ".tmp"
    subprocess.check_call(compile_cmd(tmp))
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())

"""Build the CPU oracle (test infrastructure only) with gcc into oracle/liboracle.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


# The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only; loaded by the sanitizer test with the runtime preloaded).
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O1" if sanitize else "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", *(SAN_FLAGS if sanitize else []), SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

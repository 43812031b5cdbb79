"""Build the oracle library (plain C, gcc) in place: oracle/libmsk_oracle.so.
The oracle is test infrastructure; building it is not using it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    out = os.path.join(HERE, "libmsk_oracle.so")
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99",
           os.path.join(HERE, "msk_oracle.c"), "-o", out + ".tmp", "-lm"]
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build()

"""Build the CPU oracle library (test infrastructure only).

``build_oracle()`` compiles ``kvpub_oracle.c`` with gcc into
``oracle/libkvpub_oracle.so``.  ``build_oracle(plant=k)`` builds a copy with
mistake number ``k`` planted (see the ``KVO_PLANT`` blocks in the C file);
the test suite uses those copies to show that its pins catch such mistakes.
The flags keep IEEE binary32 semantics: no FMA contraction, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvpub_oracle.c")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fPIC", "-shared", "-Wall", "-Wextra"]


def lib_path(plant=0):
    name = "libkvpub_oracle.so" if not plant else f"libkvpub_oracle_plant{plant}.so"
    if plant:
        return os.path.join(HERE, "_plants", name)
    return os.path.join(HERE, name)


def build_oracle(plant=0, cc="gcc"):
    out = lib_path(plant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [cc, *CFLAGS, SRC, "-o", out + ".tmp"]
    if plant:
        cmd.insert(1, f"-DKVO_PLANT={int(plant)}")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_oracle())

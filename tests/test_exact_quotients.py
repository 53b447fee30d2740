"""The activation quantizer's division-free quotients equal the IEEE quotients on their whole
domain (host check of tests/exact_quotients.c: every bf16 block max, every bf16 row max with an
outer scale of at least 2^-96, both 4/6 candidates -- about 10^9 cases)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_division_free_quotients_are_exact(tmp_path):
    exe = str(tmp_path / "exact_quotients")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-o", exe,
                    os.path.join(HERE, "exact_quotients.c"), "-lm"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=600).stdout.split()
    vals = dict(zip(out[0::2], map(int, out[1::2])))
    assert vals["pairs"] > 10 ** 9
    assert vals["div6"] == 0 and vals["div"] == 0 and vals["small"] == 0, vals

"""Host check of the plan-time divisors (FastDiv in the library's internal
header): floor(n / d) as one multiply and shift must equal integer division for
every n in [0, 2^31) and d >= 1.  The header is compiled with the host C++
compiler; n runs over the values around every multiple boundary that can go
wrong (k d - 1, k d), the top of the range and a seeded random sample."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shared_base_residual_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include "internal.h"
using rattn::FastDiv;
static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32() {  // splitmix64
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static long bad = 0, checked = 0;
static void check(int n, const FastDiv &f) {
    ++checked;
    if (rattn::fdiv(n, f) != n / f.d) {
        if (bad < 5) printf("mismatch n=%d d=%d got %d\n", n, f.d, rattn::fdiv(n, f));
        ++bad;
    }
}
int main() {
    const int big[] = {4095, 4096, 4097, 65535, 65536, 65537, 1 << 20, (1 << 20) + 1, 1000003,
                       (1 << 30) - 1, 1 << 30, (1 << 30) + 1, 2147483646, 2147483647};
    for (int di = 0; di < 4096 + 14; ++di) {
        const int d = di < 4096 ? di + 1 : big[di - 4096];
        const FastDiv f = rattn::make_fastdiv(d);
        for (int n = 0; n < 600; ++n) check(n, f);
        for (int64_t k = 1; k * d < 2147483647ll && k < 4000; k += (k < 64 ? 1 : 37)) {
            check((int)(k * d - 1), f);
            if (k * d <= 2147483647ll) check((int)(k * d), f);
        }
        for (int t = 0; t < 64; ++t) check(2147483647 - t, f);
        for (int t = 0; t < 256; ++t) check((int)(next32() >> 1), f);
    }
    const FastDiv z = rattn::make_fastdiv(0);  // an empty dimension divides by 1
    if (z.d != 1 || rattn::fdiv(12345, z) != 12345) ++bad;
    printf("checked %ld bad %ld\n", checked, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fastdiv.cpp"
    exe = tmp_path / "fastdiv"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " bad 0" in r.stdout

"""Host logic of the weight stream order (mk_stream_pos in the library's
internal header), compiled with the host C++ compiler: for every checked
element size, row count and row length, stream positions map one-to-one onto
(row, chunk); inside whole four-row groups each 4-chunk slot carries one
chunk index of four distinct rows; int8 rows are grouped at every length,
float32/bf16 rows of 4 chunks and rows after the last whole group run row
after row."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_megakernel_persistent_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include "mk_internal.h"
int main(void) {
    int bad = 0, cases = 0;
    for (int eb = 1; eb <= 4; eb *= 2)
    for (int rbp = 1; rbp <= 20; ++rbp)
        for (int rows = 0; rows <= 23; ++rows) {
            const int n = rows * rbp;
            char *seen = (char *)calloc(n > 0 ? n : 1, 1);
            const int full = mk_row_groups(rbp, eb) ? rows / 4 : 0;
            /* int8 rows are grouped at every length; wider ones never below 8 chunks */
            if (eb == 1 ? !mk_row_groups(rbp, eb) : (mk_row_groups(rbp, eb) && rbp < 8)) ++bad;
            for (int qq = 0; qq < n; ++qq) {
                int r, k;
                mk_stream_pos(qq, rows, rbp, eb, r, k);
                if (r < 0 || r >= rows || k < 0 || k >= rbp || seen[r * rbp + k]) { ++bad; continue; }
                seen[r * rbp + k] = 1;
                if (qq < full * 4 * rbp) {
                    int r0, k0;  /* the slot's first piece */
                    mk_stream_pos(qq & ~3, rows, rbp, eb, r0, k0);
                    if (k != k0 || r - r0 != (qq & 3) || r0 % 4 != 0) ++bad;
                } else {
                    const int rr = qq - full * 4 * rbp;
                    if (r != full * 4 + rr / rbp || k != rr % rbp) ++bad;
                }
            }
            free(seen);
            ++cases;
        }
    printf("%d cases, %d bad\n", cases, bad);
    return bad != 0;
}
"""


def test_stream_order_is_a_permutation_with_four_row_groups(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "t"
    cc = subprocess.run(["g++", "-O1", "-D__host__=", "-D__device__=", "-I", CSRC, str(src), "-o", str(exe)],
                        capture_output=True, text=True)
    if cc.returncode != 0:
        pytest.fail(cc.stderr)
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 bad" in run.stdout

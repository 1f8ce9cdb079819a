"""The global -> LDS copy plan of the backward's dK/dV kernel, walked on the CPU.

The kernel stages each 32-query chunk (q, dout, their transposes, the row
normalisers, D and the visibility words) with 50 copy instructions of 64 lanes x
16 bytes whose per-lane source offsets are fixed for the kernel (the header
csrc/bwd_plan.h, compiled here with the host compiler).  This test replays every
copy of a stage and checks that each byte the kernel's compute step reads holds
the byte of the source it expects, and that no LDS byte receives two different
source bytes.  The expected layout is written out below from the compute step's
reads, not from the plan.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dflash_block_draft_amd", "csrc")

DUMP = r"""
#include <cstdio>
#include <cstdlib>
#include "bwd_plan.h"
using namespace dflash;
int main(int argc, char** argv) {
  const int Lqp = atoi(argv[1]);
  const unsigned q0 = strtoul(argv[2], 0, 10), tile = strtoul(argv[3], 0, 10);
  const int c = atoi(argv[4]);
  printf("%d %d %d %d %d %d %d %d %d %d %d %d %d\n", kA_Q, kA_O, kA_QT, kA_OT, kA_L, kA_D, kA_B, kA_Stage,
         kA_Blocks, kSQ, kSO, kSQT, kQC);
  for (int blk = 0; blk < kA_Blocks; ++blk) {
    const int reg = a_region(blk);
    for (int lane = 0; lane < 64; ++lane)
      printf("%d %d %d %u\n", blk, lane, reg, a_voff(blk, lane, Lqp) + a_soff(reg, q0, tile, c));
  }
  return 0;
}
"""

REG_Q, REG_O, REG_QT, REG_OT, REG_L, REG_D, REG_B = range(7)


@pytest.fixture(scope="module")
def dump_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("bwd_plan")
    src, exe = d / "dump.cpp", d / "dump"
    src.write_text(DUMP)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return str(exe)


def _plan(exe, Lqp, q0, tile, c):
    out = subprocess.run([exe, str(Lqp), str(q0), str(tile), str(c)], check=True, capture_output=True,
                         text=True).stdout.split("\n")
    consts = [int(x) for x in out[0].split()]
    rows = np.array([[int(x) for x in l.split()] for l in out[1:] if l.strip()], dtype=np.int64)
    return consts, rows


def _expected(consts, Lqp, q0, tile, c):
    """(LDS byte, region, source byte) of every byte the compute step reads."""
    A_Q, A_O, A_QT, A_OT, A_L, A_D, A_B, _, _, SQ, SO, SQT, QC = consts
    exp = []
    for r in range(QC):                                   # q rows: 192 bf16 = 384 bytes
        exp += [(A_Q + r * SQ + x, REG_Q, (q0 + r) * 384 + x) for x in range(384)]
        exp += [(A_O + r * SO + x, REG_O, (q0 + r) * 256 + x) for x in range(256)]
    for d in range(192):                                  # q^T rows: this chunk's 32 queries
        exp += [(A_QT + d * SQT + x, REG_QT, d * Lqp * 2 + q0 * 2 + x) for x in range(64)]
    for d in range(128):
        exp += [(A_OT + d * SQT + x, REG_OT, d * Lqp * 2 + q0 * 2 + x) for x in range(64)]
    exp += [(A_L + x, REG_L, q0 * 4 + x) for x in range(4 * QC)]
    exp += [(A_D + x, REG_D, q0 * 4 + x) for x in range(4 * QC)]
    for t in range(2):                                    # the workgroup's two k-tiles
        for r in range(QC):
            exp += [(A_B + (t * QC + r) * 8 + x, REG_B, tile + t * 128 * 8 + c * QC * 8 + r * 8 + x)
                    for x in range(8)]
    return exp


@pytest.mark.parametrize("Lqp,qt,c,tile", [(128, 0, 0, 0), (384, 1, 3, 7 * 1024), (4096, 17, 2, 123 * 1024)])
def test_dkdv_copy_plan_delivers_every_read_byte(dump_exe, Lqp, qt, c, tile):
    q0 = qt * 128 + c * 32
    consts, rows = _plan(dump_exe, Lqp, q0, tile, c)
    stage = consts[7]
    assert consts[8] * 1024 == stage and rows.shape[0] == consts[8] * 64
    written = {}
    for blk, lane, reg, off in rows:
        for x in range(16):
            dst = blk * 1024 + lane * 16 + x
            assert 0 <= dst < stage
            src = (reg, off + x)
            assert written.setdefault(dst, src) == src, f"LDS byte {dst} gets two sources"
    for dst, reg, off in _expected(consts, Lqp, q0, tile, c):
        assert written.get(dst) == (reg, off), f"LDS byte {dst}: want {(reg, off)}, plan gives {written.get(dst)}"

"""The global -> LDS copy plan of the backward's dK/dV kernel, walked on the CPU.

The kernel stages each 32-query chunk in two parts (q and dout rows, exponent
offsets, -D and visibility words; the transposed q and dout) with 12 copy
instructions per wave of 64 lanes x 16 bytes, whose per-lane source offsets are
fixed for the kernel (the header csrc/bwd_plan.h, compiled here with the host
compiler).  This test replays the copies of all four waves and checks that

  * no LDS byte of a slot receives two different source bytes, and lanes with
    nothing to copy read past the end of every resource;
  * every 16-byte operand read of the compute (the header's read addresses, the
    ones the kernel uses) finds the bytes of the operand the MFMA needs there,
    with the operand written out below from the MFMA's lane layout, not from the
    plan: lane l of a 32x32x16 MFMA supplies row/column l % 32 and the 8
    reduction indices 8 (l / 32) .. +8 of a 16-wide chunk.
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
  const int Lqp = atoi(argv[1]), nqt = atoi(argv[2]);
  printf("%d %d %d %d %d %d %d %d %d %u\n", kF_Q, kF_O, kF_LD, kF_B, kF_Slot, kT_QT, kT_OT, kT_Slot,
         kCopiesPerStep, kPastEnd);
  for (int w = 0; w < kKvWaves; ++w)
    for (int j = 0; j < kCopiesPerStep; ++j)
      for (int l = 0; l < 64; ++l)
        printf("C %d %d %d %d %d %d %u\n", w, j, l, f_part(j) ? 1 : 0, src_region(j), dst_base(w, j) + 16 * l,
               voff(w, j, l, Lqp, nqt));
  for (int l = 0; l < 64; ++l) {
    const int li = l % 32, hi = l / 32;
    for (int s = 0; s < 12; ++s) printf("R q %d %d %d\n", l, s, rd_q(s, li, hi));
    for (int s = 0; s < 8; ++s) printf("R o %d %d %d\n", l, s, rd_o(s, li, hi));
    for (int nt = 0; nt < 6; ++nt)
      for (int kk = 0; kk < 2; ++kk) printf("R qt %d %d %d\n", l, 2 * nt + kk, rd_qt(nt, kk, li, hi));
    for (int nt = 0; nt < 4; ++nt)
      for (int kk = 0; kk < 2; ++kk) printf("R ot %d %d %d\n", l, 2 * nt + kk, rd_ot(nt, kk, li, hi));
    for (int g = 0; g < 4; ++g) printf("R nl %d %d %d\n", l, g, rd_nl(g, hi));
    for (int g = 0; g < 4; ++g) printf("R nd %d %d %d\n", l, g, rd_nd(g, hi));
  }
  for (int t = 0; t < 2; ++t)
    for (int k = 0; k < 64; ++k) printf("R w %d %d %d\n", t, k, rd_word(t, k));
  return 0;
}
"""

SRC_Q, SRC_O, SRC_LD, SRC_B, SRC_QT, SRC_OT = range(6)


@pytest.fixture(scope="module")
def dump_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("bwd_plan")
    src, exe = d / "dump.cpp", d / "dump"
    src.write_text(DUMP)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return str(exe)


def _plan(exe, Lqp, nqt):
    out = subprocess.run([exe, str(Lqp), str(nqt)], check=True, capture_output=True, text=True).stdout
    lines = out.split("\n")
    consts = [int(x) for x in lines[0].split()]
    copies, reads = [], {}
    for l in lines[1:]:
        f = l.split()
        if not f:
            continue
        if f[0] == "C":
            copies.append(tuple(int(x) for x in f[1:]))
        else:
            reads[(f[1], int(f[2]), int(f[3]))] = int(f[4])
    return consts, copies, reads


def _slots(consts, copies):
    """LDS byte -> (source region, source byte) per part, from replaying every copy."""
    past_end = consts[9]
    parts = {0: {}, 1: {}}
    for w, j, l, fpart, reg, dst, vo in copies:
        if vo >= past_end:
            continue                                   # reads zeros: nothing lands that a read may use
        slot = parts[1 if fpart else 0]
        for x in range(16):
            src = (reg, vo + x)
            assert slot.setdefault(dst + x, src) == src, f"LDS byte {dst + x} gets two sources"
    return parts[1], parts[0]


@pytest.mark.parametrize("Lqp,nqt", [(128, 1), (384, 3), (4096, 32)])
def test_dkdv_copy_plan_delivers_every_operand(dump_exe, Lqp, nqt):
    consts, copies, reads = _plan(dump_exe, Lqp, nqt)
    F_Q, F_O, F_LD, F_B, F_SLOT, T_QT, T_OT, T_SLOT, NCOPY, PAST_END = consts
    assert len(copies) == 4 * NCOPY * 64
    F, T = _slots(consts, copies)
    assert all(0 <= b < F_SLOT for b in F) and all(0 <= b < T_SLOT for b in T)

    def check(slot, lds, region, src0, what):
        for x in range(16):
            got = slot.get(lds + x)
            assert got == (region, src0 + x), f"{what}: LDS byte {lds + x} holds {got}, want {(region, src0 + x)}"

    for l in range(64):
        li, hi = l % 32, l // 32
        # S = Q K^T: A operand = q row li, dims 16s + 8hi .. +8 (bf16); chunk offset q0 * 384
        for s in range(12):
            check(F, reads[("q", l, s)], SRC_Q, li * 384 + (16 * s + 8 * hi) * 2, f"q lane {l} chunk {s}")
        for s in range(8):
            check(F, reads[("o", l, s)], SRC_O, li * 256 + (16 * s + 8 * hi) * 2, f"dout lane {l} chunk {s}")
        # dK += dS^T Q: B operand = Q^T row d = 32nt + li, chunk positions 16kk + 8hi .. +8
        for nt in range(6):
            for kk in range(2):
                d = 32 * nt + li
                check(T, reads[("qt", l, 2 * nt + kk)], SRC_QT, d * Lqp * 2 + (16 * kk + 8 * hi) * 2,
                      f"q^T lane {l} tile {nt} half {kk}")
        for nt in range(4):
            for kk in range(2):
                d = 32 * nt + li
                check(T, reads[("ot", l, 2 * nt + kk)], SRC_OT, d * Lqp * 2 + (16 * kk + 8 * hi) * 2,
                      f"dout^T lane {l} tile {nt} half {kk}")
        # accumulator rows 4g .. 4g+3 <-> queries 8g + 4hi .. +3: their offsets, then their -D
        for g in range(4):
            check(F, reads[("nl", l, g)], SRC_LD, (8 * g + 4 * hi) * 4, f"offsets lane {l} group {g}")
            check(F, reads[("nd", l, g)], SRC_LD, 128 + (8 * g + 4 * hi) * 4, f"-D lane {l} group {g}")
    # the word of key k of k-tile t: k-tiles nqt * 1024 bytes apart, 4 bytes per key
    for t in range(2):
        for k in range(64):
            lds = reads[("w", t, k)]
            for x in range(4):
                assert F.get(lds + x) == (SRC_B, t * nqt * 1024 + k * 4 + x), f"word of tile {t} key {k}"


def test_dkdv_plan_is_the_same_for_every_wave(dump_exe):
    """Each wave issues the same 12 copy instructions (the same regions, in the
    same order), so the kernel's wait counts are one constant for all waves."""
    _, copies, _ = _plan(dump_exe, 256, 2)
    regs = {}
    for w, j, l, fpart, reg, dst, vo in copies:
        regs.setdefault(w, {})[j] = (fpart, reg)
    assert all(regs[w] == regs[0] for w in range(4))


DUMP_Q = r"""
#include <cstdio>
#include <cstdlib>
#include "bwd_plan.h"
using namespace dflash;
int main(int argc, char** argv) {
  const int Lkp = atoi(argv[1]);
  printf("%d %d %d\n", kQF_Slot, kQT_Slot, kQCopiesPerStep);
  for (int w = 0; w < 4; ++w)
    for (int j = 0; j < kQCopiesPerStep; ++j)
      for (int l = 0; l < 64; ++l)
        printf("C %d %d %d %d %d %d %u\n", w, j, l, q_f_part(j) ? 1 : 0, q_src_region(j), q_dst_base(w, j) + 16 * l,
               q_voff(w, j, l, Lkp));
  for (int l = 0; l < 64; ++l) {
    const int li = l % 32, hi = l / 32;
    for (int s = 0; s < 12; ++s) printf("R k %d %d %d\n", l, s, rd_k(s, li, hi));
    for (int s = 0; s < 8; ++s) printf("R v %d %d %d\n", l, s, rd_v(s, li, hi));
    for (int mt = 0; mt < 6; ++mt)
      for (int kk = 0; kk < 2; ++kk) printf("R kt %d %d %d\n", l, 2 * mt + kk, rd_kt(mt, kk, li, hi));
  }
  for (int q = 0; q < 128; ++q) printf("R w %d 0 %d\n", q, rd_qword(q));
  return 0;
}
"""

SRC_KN, SRC_KR, SRC_V, SRC_BITS, SRC_KTN, SRC_KTR = range(6)


@pytest.fixture(scope="module")
def dump_q_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("bwd_plan_q")
    src, exe = d / "dump.cpp", d / "dump"
    src.write_text(DUMP_Q)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return str(exe)


@pytest.mark.parametrize("Lkp", [64, 320, 9216])
def test_dq_copy_plan_delivers_every_operand(dump_q_exe, Lkp):
    """The dQ kernel's staging of a 32-key step: k_nope, k_rope and v rows, the
    tile's 128 visibility words (F part), the transposed k rows (T part)."""
    out = subprocess.run([dump_q_exe, str(Lkp)], check=True, capture_output=True, text=True).stdout.split("\n")
    F_SLOT, T_SLOT, NCOPY = (int(x) for x in out[0].split())
    copies, reads = [], {}
    for l in out[1:]:
        f = l.split()
        if not f:
            continue
        if f[0] == "C":
            copies.append(tuple(int(x) for x in f[1:]))
        else:
            reads[(f[1], int(f[2]), int(f[3]))] = int(f[4])
    assert len(copies) == 4 * NCOPY * 64
    parts = {0: {}, 1: {}}
    regs = {}
    for w, j, l, fpart, reg, dst, vo in copies:
        regs.setdefault(w, {})[j] = (fpart, reg)
        slot = parts[fpart]
        for x in range(16):
            src = (reg, vo + x)
            assert slot.setdefault(dst + x, src) == src, f"LDS byte {dst + x} gets two sources"
    assert all(regs[w] == regs[0] for w in range(4)), "every wave issues the same copy sequence"
    F, T = parts[1], parts[0]
    assert all(0 <= b < F_SLOT for b in F) and all(0 <= b < T_SLOT for b in T)

    def check(slot, lds, region, src0, n, what):
        for x in range(n):
            got = slot.get(lds + x)
            assert got == (region, src0 + x), f"{what}: LDS byte {lds + x} holds {got}, want {(region, src0 + x)}"

    for l in range(64):
        li, hi = l % 32, l // 32
        # S^T = K Q^T: A operand = key row li, dims 16s + 8hi .. +8 (k_nope dims < 128, then k_rope)
        for s in range(12):
            if s < 8:
                check(F, reads[("k", l, s)], SRC_KN, li * 256 + (16 * s + 8 * hi) * 2, 16, f"k_nope lane {l} chunk {s}")
            else:
                check(F, reads[("k", l, s)], SRC_KR, li * 128 + (16 * (s - 8) + 8 * hi) * 2, 16, f"k_rope lane {l} chunk {s}")
        for s in range(8):
            check(F, reads[("v", l, s)], SRC_V, li * 256 + (16 * s + 8 * hi) * 2, 16, f"v lane {l} chunk {s}")
        # dQ^T += K^T dS^T: A operand = K^T row d = 32mt + li, positions 16kk + 8hi .. +8 of the step's keys
        for mt in range(6):
            for kk in range(2):
                d = 32 * mt + li
                reg, row = (SRC_KTN, d) if d < 128 else (SRC_KTR, d - 128)
                check(T, reads[("kt", l, 2 * mt + kk)], reg, row * Lkp * 2 + (16 * kk + 8 * hi) * 2, 16,
                      f"k^T lane {l} tile {mt} half {kk}")
    for q in range(128):                                  # query row q's 64-bit visibility word
        check(F, reads[("w", q, 0)], SRC_BITS, q * 8, 8, f"word of query {q}")

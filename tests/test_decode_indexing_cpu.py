"""CPU model of the decode kernel's indexing (no GPU).

The decode runs one group of waves per (row, k-head) and, for small heads,
several groups per workgroup, each with its own slice of LDS.  This test
restates the kernel's shape rules and index arithmetic (DecodeShape, the
k-heads-per-workgroup choice, decode_kernel and decode_group in
decode_kernel.hip) for every head size and conv width the kernel is compiled
for, over k-head counts and GQA ratios, and checks:

  * the grid gives every (row, k-head) to exactly one group;
  * every state element of every v-head of the group is loaded and stored by
    exactly one lane, inside the page's state region;
  * LDS accesses (conv outputs, key rows, partial sums, v rows) stay inside the
    group's slice, and the slices inside the launch's allocation;
  * conv channels and output columns stay inside their arrays.

A change of that arithmetic in the kernel must be mirrored here before the
kernel runs on a GPU.
"""
import itertools

import pytest


def shape(DK, DV):
    LPR = DV // 4                      # lanes per key row (a float4 each)
    RPI = 64 // LPR                    # key rows per memory instruction
    NWMAX = DK * DV // 1024
    NW = 1 if NWMAX < 1 else min(NWMAX, 4)
    KPW = DK // NW                     # key rows per wave
    JPL = KPW // RPI                   # key rows per lane
    return dict(LPR=LPR, RPI=RPI, NW=NW, KPW=KPW, JPL=JPL, NT=64 * NW)


def kpg_for(dk):
    return {64: 2, 32: 8, 16: 8}.get(dk, 1)


CASES = [(d, Hk, G) for d in (16, 32, 64, 128) for Hk in (1, 2, 3, 4, 8, 16, 24)
         for G in (1, 2, 3, 4)]


@pytest.mark.parametrize("d,Hk,G", CASES)
def test_decode_indexing_stays_in_bounds(d, Hk, G):
    DK = DV = d
    sh = shape(DK, DV)
    LPR, RPI, NW, KPW, JPL, NT = (sh[k] for k in ("LPR", "RPI", "NW", "KPW", "JPL", "NT"))
    assert LPR * RPI == 64 and DK % NW == 0 and KPW % RPI == 0 and JPL >= 1
    K = kpg_for(DK)
    KPG = K if K > 1 and Hk % K == 0 else 1
    Hv = Hk * G
    C = 2 * Hk * DK + Hv * DV
    per_group = 2 * DK + G * DV + 4 * NW * DV          # floats of one group's LDS slice
    lds_floats = KPG * per_group                        # the host's allocation
    state_bytes = Hv * DK * DV * 4
    nvc = 2 * DK + G * DV                               # conv channels of a group

    # the grid: rows x Hk / KPG workgroups, each covering KPG consecutive k-heads
    per_row = Hk // KPG
    groups = sorted(b * KPG + sub for b in range(per_row) for sub in range(KPG))
    assert groups == list(range(Hk))

    for sub in range(KPG):
        g = sub  # any k-head of the row; offsets below depend on g only through h0
        h0 = g * G
        base = sub * per_group
        assert base + per_group <= lds_floats

        def chan(vc):
            if vc < DK:
                return g * DK + vc
            if vc < 2 * DK:
                return Hk * DK + g * DK + (vc - DK)
            return 2 * Hk * DK + h0 * DV + (vc - 2 * DK)

        seen = {h: set() for h in range(G)}
        for tid in range(NT):
            wave, lane = tid >> 6, tid & 63
            c4 = lane % LPR
            key0 = wave * KPW + lane // LPR
            # conv outputs: channel pairs vc, vc + 1 from 2 tid on, NT pairs apart
            for vc in range(2 * tid, nvc, 2 * NT):
                assert vc + 1 < nvc
                c = chan(vc)
                assert 0 <= c and c + 1 < C and chan(vc + 1) == c + 1
            # key rows of the lane, and their state elements for every head
            for m in range(JPL):
                key = key0 + RPI * m
                assert 0 <= key < DK                     # ys[DK + key], ys[key]
                for hh in range(G):
                    h = h0 + hh
                    off = (h * DK + key) * DV * 4 + 4 * c4 * 4
                    assert 0 <= off and off + 16 <= state_bytes
                    assert (key, c4) not in seen[hh]
                    seen[hh].add((key, c4))
            # partial sums of a head pair, v rows and outputs
            if lane < LPR:
                for rh in (0, 2 * NW * DV):             # red, red + RH
                    for idx in (rh + wave * DV + 4 * c4, rh + (NW + wave) * DV + 4 * c4):
                        assert 0 <= idx and idx + 4 <= 4 * NW * DV
            for hh in range(G):
                v = 2 * DK + hh * DV + 4 * c4
                assert v + 4 <= nvc
                assert hh * DV + 4 * c4 + 4 <= G * DV    # out_row columns of the group
        for hh in range(G):
            assert seen[hh] == set(itertools.product(range(DK), range(LPR)))
    # the padding-row loop zeroes exactly the KPG groups' outputs
    zeroed = sorted(e for t in range(KPG * NT) for e in range(t, KPG * G * DV, KPG * NT))
    assert zeroed == list(range(KPG * G * DV))

"""CPU bounds model of the varlen prefill's producer loads (no GPU).

The prefill kernel's conv waves (q and k rows) and state waves (each lane its
own v channel) read raw inputs with buffer loads whose range check returns
zero past a resource's end, so every load either lies inside the rows of its
own sequence (or its slot's window) or is refused by the range check.  A wrong row base or range here once let a wave read past
the end of x.  This test replays the producers' row / range / offset
arithmetic for every head size and conv width the kernel is compiled for,
over ragged lengths, and checks:

  * every load the range check lets through lies inside the sequence's rows
    of x (token rows [tb, tb + L)), inside one row, on a channel pair the
    wave owns, and at the row its token needs (so no needed row is refused);
  * window loads stay inside the window region, and the window resource is
    empty when the sequence starts cold (a cold page is never read);
  * gate loads stay inside the sequence's tokens, and the waves that do not
    use the gates load none.

The loop issues the loads of chunk c + 1 while it prepares chunk c, with no
branch, so it also loads a chunk past the last one (c = nchunks - 1); those
rows lie past the sequence's end, where the ranges are empty.  The
arithmetic is restated from the kernel's `issue` / `issue_first`
(prefill_kernel.hip); a change there must be mirrored here before the
kernel runs on a GPU.
"""
import numpy as np
import pytest

CT, NPROD = 16, 8
INT32_MAX = 2**31 - 1
OUT_OF_RANGE = 0xFFFFFFF0


def shape(dk, swr=4):
    """Column slice of a workgroup: up to `swr` 16-column blocks of the head
    (4, or 8 for whole 128-column heads), one state wave per block.  Eight
    conv waves: two per 4 tokens, one for the q pairs and one for the k
    pairs."""
    nb = dk // 16
    sw = min(nb, swr)
    isz = 16 * sw
    tpw = 2 * CT // NPROD
    nfin = 1 if sw <= 4 else 0   # a finish wave of its own in the smaller workgroups
    return dict(ISZ=isz, SW=sw, NSL=nb // sw, TPW=tpw, QKP=dk // 2, NFIN=nfin,
                TYPE=[((pw + 1) & 1) if nfin else (pw & 1) for pw in range(NPROD)],
                RATIO_PW=5 if nfin else 1)


def range_bytes(n):
    """The kernel's clamp to [0, INT32_MAX] (a negative range would be a huge
    unsigned record count, which passes every offset)."""
    return min(max(n, 0), INT32_MAX)


def check_sequence(dk, W, Hk, Hv, L, tb, warm, total_rows, swr=4):
    """All input loads (conv waves' q/k rows and gates, state waves' v rows)
    of all workgroups of one sequence."""
    sh = shape(dk, swr)
    C = 2 * Hk * dk + Hv * dk
    rowb = 2 * C
    HR, TPW = W - 1, sh["TPW"]
    NR = HR + TPW      # rows of a conv wave (4 tokens)
    NRV = HR + 4       # rows of a state-wave lane (4 tokens)
    lane = np.arange(64)
    q4, m16 = lane // 16, lane % 16
    nchunks = (L + CT - 1) // CT
    x_lo, x_hi = tb * rowb, (tb + L) * rowb          # the sequence's bytes of x
    assert x_hi <= total_rows * rowb
    n_checked = 0

    def through(res_base, res_range, off, row_needed, size):
        """Loads of `size` bytes at byte offsets `off` of the resource: the ones
        the range check lets through must lie in the sequence's rows, and
        every needed row must get through."""
        off = np.asarray(off, np.int64) % 2**32                  # a VGPR offset is unsigned
        ok_ = off + size <= res_range
        addr = res_base + off
        assert ((addr >= x_lo) & (addr + size <= x_hi))[ok_].all()
        need = (row_needed >= 0) & (row_needed < L)
        assert (ok_ | ~need).all(), "a row inside the sequence was refused"
        return int(ok_.sum())

    def window(r, off, size):
        """Window loads at rows r < 0 (offsets off), else OUT_OF_RANGE."""
        win_range = HR * rowb if warm else 0
        ow = np.where(r < 0, (HR + r) * rowb + off, OUT_OF_RANGE)
        inwin = ow + size <= win_range
        assert ((ow >= 0) & (ow + size <= HR * rowb))[inwin].all()
        if warm:
            assert (inwin | (r >= 0)).all(), "a window row was refused"
        else:
            assert not inwin.any(), "a cold page was read"

    for h in range(Hv):
        g = h // (Hv // Hk)
        for sl in range(sh["NSL"]):
            def chan(ch):
                ch = np.asarray(ch)
                return np.where(ch < dk, g * dk + ch,
                                np.where(ch < 2 * dk, Hk * dk + g * dk + (ch - dk),
                                         2 * Hk * dk + h * dk + sl * sh["ISZ"] + (ch - 2 * dk)))
            qkp = np.minimum(lane, sh["QKP"] - 1)
            for pw in range(NPROD):
                ty = sh["TYPE"][pw]                                      # 0: q, 1: k
                t0 = (pw >> 1) * TPW
                ox = chan(ty * dk + 2 * qkp) * 2
                # every owned channel pair lies inside one row of x
                assert (ox >= 0).all() and (ox + 4 <= rowb).all()
                k = np.arange(nchunks + 1)                               # one past the last chunk
                rbase = k * CT + t0 - HR
                # issue(k): rows from min(rbase, L); issue_first's window
                # path (rbase < 0): rows from 0
                xb = np.where(rbase >= 0, np.minimum(rbase, L), 0)
                base = (tb + xb) * rowb                                  # resource base (bytes of x)
                # the record count is an unsigned 32-bit field: a negative range
                # would pass every offset
                rng = np.array([range_bytes((L - b) * rowb) for b in xb]) % 2**32
                main = rbase >= 0
                for i in range(NR):
                    row = rbase[:, None] + i                              # token row of load i
                    n_checked += through(base[main, None], rng[main, None],
                                         (ox[None, :] + i * rowb)[np.zeros(main.sum(), int)],
                                         row[main], 4)
                if (~main).any():
                    # the first chunk of the waves of tokens 0-3: rows before the
                    # start come from the window
                    assert pw < 2 and rbase[0] == -HR and (~main).sum() == 1
                    for i in range(NR):
                        r = np.full(64, i - HR)
                        window(r, ox, 4)
                        n_checked += through(base[0], rng[0],
                                             np.where(r >= 0, r * rowb + ox, OUT_OF_RANGE),
                                             np.where(r >= 0, r, -1), 4)
                # gates: token k CT + lane % CT of head h, for the ratio wave only
                ht = Hv * 4
                use = pw == sh["RATIO_PW"]
                grec = np.array([range_bytes((L - kk * CT) * ht) if use else 0 for kk in k])
                grec = grec % 2**32
                goff = (lane % CT) * ht
                okg = goff[None, :] + 4 <= grec[:, None]
                tok = k[:, None] * CT + (lane % CT)[None, :]
                assert ((tok >= 0) & (tok < L))[okg].all()
                if use:
                    assert (okg | (tok >= L)).all()
                else:
                    assert not okg.any()
            # state waves: lane (q4, m16) of state wave sw loads the rows of its
            # v channel (16-bit loads) that tokens 4 q4 .. 4 q4 + 3 need
            for sw in range(sh["SW"]):
                vo = chan(2 * dk + 16 * sw + m16) * 2
                assert (vo >= 0).all() and (vo + 2 <= rowb).all()
                assert len(set(vo.tolist())) == 16                       # one column per m16
                k = np.arange(1, nchunks + 1)                            # issue_v(k + 1) after chunk k
                xb = np.minimum(k * CT - HR, L)
                assert (xb >= 0).all()
                base = (tb + xb) * rowb
                rng = np.array([range_bytes((L - b) * rowb) for b in xb]) % 2**32
                for i in range(NRV):
                    off = (4 * q4 + i) * rowb + vo
                    row = xb[:, None] + (4 * q4 + i)[None, :]
                    n_checked += through(base[:, None], rng[:, None], off[None, :], row, 2)
                # chunk 0: rows before the start from the window
                rng0 = range_bytes(L * rowb) % 2**32
                for i in range(NRV):
                    r = 4 * q4 + i - HR
                    window(r, vo, 2)
                    n_checked += through(tb * rowb, rng0, np.where(r >= 0, r * rowb + vo, OUT_OF_RANGE),
                                         np.where(r >= 0, r, -1), 2)
    return n_checked


C3_LENGTHS = [3561, 2795, 2344, 1479, 1615, 658, 781, 571]


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("W", [2, 3, 4])
def test_producer_loads_short_and_ragged(dk, W):
    lengths = list(range(1, 80)) + [1000]
    Hk, Hv = 1, 2
    total = sum(lengths)
    tb = 0
    n = 0
    for i, L in enumerate(lengths):
        n += check_sequence(dk, W, Hk, Hv, L, tb, warm=bool(i % 2), total_rows=total)
        tb += L
    assert n > 0


@pytest.mark.parametrize("W", [2, 4])
def test_producer_loads_workload_lengths(W):
    # the 8-sequence workload's lengths (16 v-heads / 8 k-heads at dk 128),
    # the last sequence ending exactly at the end of x
    lengths = C3_LENGTHS
    total = sum(lengths)
    tb = 0
    for i, L in enumerate(lengths):
        check_sequence(128, W, 2, 4, L, tb, warm=i < 4, total_rows=total)
        tb += L


@pytest.mark.parametrize("W", [2, 4])
def test_producer_loads_whole_head_workgroups(W):
    # head size 128 in whole-head workgroups (64 sequences x 1000 tokens
    # at 32 v-heads uses them); ragged lengths and the 1000-token rows
    lengths = list(range(1, 40)) + [1000, 1000]
    total = sum(lengths)
    tb = 0
    for i, L in enumerate(lengths):
        check_sequence(128, W, 2, 4, L, tb, warm=bool(i % 2), total_rows=total, swr=8)
        tb += L


def test_producer_loads_long_sequence():
    # one 65,536-token sequence after a 3-token one, at the end of x
    check_sequence(128, 4, 1, 2, 3, 0, warm=True, total_rows=65539)
    check_sequence(128, 4, 1, 2, 65536, 3, warm=False, total_rows=65539)


@pytest.mark.parametrize("dk,swr", [(16, 4), (64, 4), (128, 4), (128, 8)])
def test_every_token_group_has_a_q_and_a_k_wave(dk, swr):
    # the two conv waves of 4 tokens (2 g, 2 g + 1) split q and k between them,
    # and the ratio wave exists
    sh = shape(dk, swr)
    for g in range(NPROD // 2):
        assert sorted(sh["TYPE"][2 * g: 2 * g + 2]) == [0, 1]
    assert 0 <= sh["RATIO_PW"] < NPROD

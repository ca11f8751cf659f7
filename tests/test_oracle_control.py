"""Pins of the dynamic-gamma oracle: the page's thresholds at their edges,
the history window, error rounds, temperature coupling and the round-to-
outcome reading."""

import numpy as np

from oracle import control as C


def word(bits, count):
    return (bits & 0xFFFF) | (count << 16)


def test_thresholds_at_their_edges():
    # rate exactly 0.6 is "30-60%": 4; just above: 8; exactly 0.3: 4; below: 2
    assert C.gamma_of(word(0b111, 5)) == 4          # 3/5 = 0.6
    assert C.gamma_of(word(0b1111, 6)) == 8         # 4/6 > 0.6
    assert C.gamma_of(word(0b111, 10)) == 4         # 3/10 = 0.3
    assert C.gamma_of(word(0b11, 7)) == 2           # 2/7 < 0.3
    assert C.gamma_of(word(0xFFFF, 16)) == 8
    assert C.gamma_of(word(0, 16)) == 2
    assert C.gamma_of(word(0, 0)) == 4              # nothing seen yet
    # full windows: k/16 for every k
    for k in range(17):
        g = C.gamma_of(word((1 << k) - 1, 16))
        rate = k / 16
        assert g == (8 if rate > 0.6 else (4 if rate >= 0.3 else 2))


def test_rounds_become_outcomes():
    w = C.push(0, 3, 5)                 # accepted 3 of 5: 1 1 1 0 (newest in bit 0)
    assert w == word(0b1110, 4)
    w = C.push(w, 2, 2)                 # all accepted: no rejection outcome
    assert w == word(0b111011, 6)
    assert C.push(w, -1, 4) == w        # flagged round: nothing
    w = 0
    for _ in range(10):
        w = C.push(w, 4, 8)             # 1111 0 per round
    # newest first: 0, 1111, 0, 1111, 0, 1111, 0
    assert (w >> 16) == 16 and (w & 0xFFFF) == 0b0111101111011110
    assert C.gamma_of(w) == 8                        # 12 / 16


def test_long_rounds_keep_the_newest_sixteen():
    # 20 accepted then a rejection: the newest 16 are fifteen ones, then the zero
    assert C.push(word(0x1234, 9), 20, 30) == word(0xFFFE, 16)
    # 40 of 40 accepted: sixteen ones, no zero
    assert C.push(word(0, 16), 40, 40) == word(0xFFFF, 16)
    # exactly 16 outcomes (15 ones, a zero) replace the whole window
    assert C.push(word(0xFFFF, 16), 15, 16) == word(0xFFFE, 16)


def test_window_forgets_old_outcomes():
    w = 0
    for _ in range(4):
        w = C.push(w, 0, 8)             # four rejections
    for _ in range(3):
        w = C.push(w, 8, 8)             # then 24 acceptances push them out
    assert C.gamma_of(w) == 8 and (w & 0xFFFF) == 0xFFFF


def test_temperature_coupling_and_offsets():
    hist = np.array([word(0xFFFF, 16), word(0, 16), word(0x00FF, 16)])
    h, g, off = C.gamma_update(hist, np.array([2, 0, -1]), np.array([8, 2, 4]),
                               temp_target=np.array([0.5, 0.9, 1.0]), couple_temperature=True)
    assert list(g) == [8, 1, 1]
    assert list(off) == [0, 8, 9, 10]
    h, g, off = C.gamma_update(hist, np.array([2, 0, -1]), np.array([8, 2, 4]))
    assert list(g) == [8, 2, 4] and list(off) == [0, 8, 10, 14]
    # 0.8 itself (as the float32 a caller passes) is not above 0.8
    assert C.gamma_of(word(0, 16), np.float32(0.8), True) == 2

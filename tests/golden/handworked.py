"""Input of the hand-worked golden record and a parser of its expected bytes
(c128_handworked.txt, derived in make_handworked.py)."""
import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def build_handworked():
    base, state = synth.alloc_state(16)
    synth.fill_state(state, 4242, 1.0, 1.0)  # scores stay random
    sign = np.where(np.arange(512) % 3 == 0, 1.0, -1.0).astype(np.float32)
    state[:, :, :512] = sign[None, None, :]
    w = np.ones(512, np.float32)
    for g in range(7):
        w[64 * g: 64 * (g + 1)] = 2.0 ** (g - 3)
    bt = synth.permutation(16, 4242, 1).astype(np.int32).reshape(1, 16)
    positions = np.array([127, 126], np.int32)
    slot = np.array([int(bt[0, 15]) * 8 + 7, int(bt[0, 15]) * 8 + 6], np.int32)
    kc_base, kc = synth.alloc_k_cache(1, 2)
    return synth.Workload("handworked", state, bt, np.zeros(2, np.int32), positions, slot, w, 0.0,
                          synth.rope_table(256), kc, np.array([0, 1], np.int32), 4242, base,
                          kc_base)


DOUBLE_ROUNDING_W = 1.0 + 2.0 ** -4 + 2.0 ** -10  # exact in fp32


def build_double_rounding():
    """The hand-worked input with every rms weight 1 except the first quantisation block, where
    w = 1 + 2^-4 + 2^-10.  Every kv row is +-1 and eps is 0, so the normalised values are
    exactly +-w.  In the first block bf16 rounds w to 1.0625, the block's UE8M0 exponent is -8
    (absmax 1.0625 over 448 lies in (2^-9, 2^-8]) and 1.0625 * 2^8 = 272 falls midway between the
    E4M3 neighbours 256 and 288: ties go to the even code, 256 (0x78, 0xF8 negative).  Coded from
    the fp32 value without the bf16 step, 272.25 would round to 288 (0x79)."""
    wl = build_handworked()
    w = np.ones(512, np.float32)
    w[:64] = DOUBLE_ROUNDING_W
    wl.rms_w = w
    return wl


def expected_record():
    scales, codes, rope = [], [], []
    for line in open(os.path.join(HERE, "c128_handworked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        if key == "scales":
            scales += [int(v) for v in vals]
        elif key == "codes":
            codes += [int(v, 16) for v in vals]
        elif key == "rope":
            rope += [int(v, 16) for v in vals]
    return (np.array(codes, np.uint8), np.array(scales, np.uint8), np.array(rope, np.uint16))

"""Host checks of the bias-table indexing that the forward kernel relies on (CPU only).

The forward's per-element time bias for tiles whose time differences are below 2^24 looks the
bias up by the bit pattern of the difference as a float32: ((bits >> 18) & 0x1ffc) is a byte
offset from the bucket table's entry for distance 0, and offsets from 4064 on land in a table of
192 float classes (exponent and first three fraction bits), entry k holding the bucket of
((8 + k % 8) << (k // 8)) >> 3.  That is exact only if every integer distance of a class lies in
one bucket; this test checks it for every distance below 2^24 and both signs against the bucket
rule written as sorted start points (page 1, section 2.1.2: rab^{p,t} indexed by bucketized
|t_i - t_j|).
"""
import numpy as np

import oracle.brute as brute

K_FLOAT_CLASSES = 192
K_FLOAT_CLASS_BASE = 127 * 8 * 4


def float_class_table():
    k = np.arange(K_FLOAT_CLASSES, dtype=np.int64)
    member = ((8 + (k & 7)) << (k >> 3)) >> 3
    return brute.bucket_table_lookup(member)


def lookup(diff):
    """Bucket the kernel reads for signed int32 differences |diff| < 2^24."""
    bits = np.asarray(diff, dtype=np.int32).astype(np.float32).view(np.uint32).astype(np.int64)
    off = (bits >> 18) & 0x1FFC
    table = float_class_table()
    out = np.empty(off.shape, dtype=np.int64)
    zero = off == 0  # +0.0 / -0.0: the bucket table's first entry, distance 0
    out[zero] = 0
    idx = (off[~zero] - K_FLOAT_CLASS_BASE) // 4
    assert idx.min() >= 0 and idx.max() < K_FLOAT_CLASSES
    out[~zero] = table[idx]
    return out


def test_float_class_lookup_matches_buckets_below_2_24():
    d = np.arange(0, 1 << 24, dtype=np.int64)
    want = brute.bucket_table_lookup(d)
    np.testing.assert_array_equal(lookup(d), want)
    np.testing.assert_array_equal(lookup(-d), want)


def test_float_class_offsets_stay_inside_the_table():
    d = np.array([1, 2, 3, 15, 16, (1 << 23) + 12345, (1 << 24) - 1], dtype=np.int64)
    bits = d.astype(np.float32).view(np.uint32).astype(np.int64)
    off = (bits >> 18) & 0x1FFC
    assert off.min() >= K_FLOAT_CLASS_BASE
    assert off.max() < K_FLOAT_CLASS_BASE + 4 * K_FLOAT_CLASSES

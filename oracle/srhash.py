"""Counter-based random words for stochastic rounding (test infrastructure).

The pages say only that stochastic rounding picks the upper or lower
representable neighbour with a probability set by the distance (lhc.media
page, paragraph on requantising into MXFP8 with stochastic rounding).  The
random source is fixed here so that any implementation agrees bit for bit: a
counter-based hash keyed by (seed, stream, element index).

Mixer: ``fmix32``, the 32-bit finaliser of Austin Appleby's MurmurHash3
(public domain), implemented from its published description: xor-shift right
by 16, multiply by 0x85EBCA6B, xor-shift right by 13, multiply by 0xC2B2AE35,
xor-shift right by 16 (all modulo 2**32).  It is a bijection on 32-bit words.

Random bits of element i (i = row * cols + col, the 64-bit row-major index of
the element in the logical source matrix handed to the call):

    j    = i >> 1                                   (one 32-bit word per pair)
    key  = fmix32(fmix32(fmix32(fmix32(lo32(seed)) ^ hi32(seed)) ^ stream) ^ hi32(j))
    word = fmix32(lo32(j) ^ key)
    r_i  = (word >> (16 * (i & 1))) & 0xFFFF        (16 random bits)

Reading taken: 16 random bits per element (one hash per two elements).  A
32-bit word per element costs about 15 vector ALU operations on the GPU, twice
the whole per-element budget of an HBM-rate requantiser; with 16 bits the
rounding probability is floor(frac * 2**16) / 2**16, i.e. a bias below 2**-16
of one grid step.
"""
import numpy as np

M32 = 0xFFFFFFFF


def fmix32(h):
    """MurmurHash3 32-bit finaliser on a uint32 (scalar int or uint32 array)."""
    h = np.asarray(h, dtype=np.uint64) & M32
    h = h ^ (h >> 16)
    h = (h * 0x85EBCA6B) & M32
    h = h ^ (h >> 13)
    h = (h * 0xC2B2AE35) & M32
    h = h ^ (h >> 16)
    return h


def stream_key(seed, stream_id, hi_j):
    """Per-(seed, stream, high word of j) key."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    k = fmix32(seed & M32)
    k = fmix32(k ^ np.uint64(seed >> 32))
    k = fmix32(k ^ np.uint64(int(stream_id) & M32))
    return fmix32(k ^ (np.asarray(hi_j, dtype=np.uint64) & M32))


def random16(seed, stream_id, idx):
    """16-bit random words r_i for the 64-bit element indices ``idx``."""
    i = np.asarray(idx, dtype=np.uint64)
    j = i >> np.uint64(1)
    key = stream_key(seed, stream_id, j >> np.uint64(32))
    word = fmix32((j & np.uint64(M32)) ^ key)
    shift = (i & np.uint64(1)) * np.uint64(16)
    return ((word >> shift) & np.uint64(0xFFFF)).astype(np.int64)

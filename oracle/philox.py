"""Counter-based Gaussian streams for the probes P and the DP noise.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix only the *law* of these random numbers:
  * [RC] section 中核メカニズム, item 1: P in R^{p x k} has i.i.d. Gaussian
    entries;
  * [DPSGD] section DP-SGDのアルゴリズム, step 4: the noise is N(0, sigma^2 C^2 I).
They say nothing about the generator, so the generator is Philox4x32-10 from
its published definition (Salmon et al., SC'11) and the Gaussian transform is
Box-Muller from its mathematics.  The readings that fix the bit streams
(24-bit uniforms, lane order, counter layout) are stated next to the code.
"""

import numpy as np

MASK32 = 0xFFFFFFFF
# Philox4x32 round multipliers and Weyl key increments (Salmon et al., SC'11).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10

# Counter word c2 used by the DP-noise stream: it can never equal a sample
# index, so probe and noise streams of one layer are disjoint.
NOISE_C2 = 0xFFFFFFFF
# Each Philox call yields four 32-bit words = four normals ("lanes").
PROBE_LANES = 4


def philox4x32_10(c0, c1, c2, c3, seed):
    """Philox4x32 with 10 rounds on the 128-bit counter (c0, c1, c2, c3).

    The key is the 64-bit ``seed`` split as (low word, high word).  One round
    multiplies c0 and c2 by the two round constants (full 32x32 -> 64-bit
    products), mixes the high halves with the other two words and the key, and
    the key is bumped by the Weyl constants between rounds (the first round
    uses the unbumped key).  Returns an array [..., 4] of uint32.
    """
    x0 = np.asarray(c0, dtype=np.uint64) & MASK32
    x1 = np.asarray(c1, dtype=np.uint64) & MASK32
    x2 = np.asarray(c2, dtype=np.uint64) & MASK32
    x3 = np.asarray(c3, dtype=np.uint64) & MASK32
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    k0 = np.uint64(seed & MASK32)
    k1 = np.uint64((seed >> 32) & MASK32)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    mask = np.uint64(MASK32)
    s32 = np.uint64(32)
    for rnd in range(PHILOX_ROUNDS):
        if rnd:
            k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
            k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
        prod0 = x0 * m0  # < 2^64: exact in uint64
        prod1 = x2 * m1
        hi0, lo0 = prod0 >> s32, prod0 & mask
        hi1, lo1 = prod1 >> s32, prod1 & mask
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def uniforms_from_words(w_a, w_b):
    """Two 32-bit words -> (u1, u2) from their top 24 bits.

    Reading (pages silent): m = word >> 8; u1 = (m_a + 1) 2^-24 lies in (0, 1]
    so that log(u1) is finite; u2 = m_b 2^-24 lies in [0, 1).  Both are exact
    in fp32 and fp64, so the uniforms agree bit for bit on any device.
    """
    m_a = (np.asarray(w_a, dtype=np.uint64) >> np.uint64(8)).astype(np.float64)
    m_b = (np.asarray(w_b, dtype=np.uint64) >> np.uint64(8)).astype(np.float64)
    u1 = (m_a + 1.0) * 2.0 ** -24
    u2 = m_b * 2.0 ** -24
    return u1, u2


def box_muller(words):
    """Four Philox words [..., 4] -> four standard normals [..., 4] (fp64).

    Words (0, 1) give lanes 0 and 1, words (2, 3) give lanes 2 and 3:
    rho = sqrt(-2 ln u1), lanes = (rho cos 2 pi u2, rho sin 2 pi u2).
    """
    words = np.asarray(words)
    out = np.empty(words.shape, dtype=np.float64)
    for a in (0, 2):
        u1, u2 = uniforms_from_words(words[..., a], words[..., a + 1])
        rho = np.sqrt(-2.0 * np.log(u1))
        out[..., a] = rho * np.cos(2.0 * np.pi * u2)
        out[..., a + 1] = rho * np.sin(2.0 * np.pi * u2)
    return out


def normals_from_counters(c0, c1, c2, c3, seed):
    """Four N(0, 1) draws per counter: Philox4x32-10 then Box-Muller."""
    return box_muller(philox4x32_10(c0, c1, c2, c3, seed))


def probe_matrix(seed, layer, sample, p, k):
    """The Hutchinson probe P_i in R^{p x k} with i.i.d. N(0, 1) entries.

    [RC] section 中核メカニズム, item 1 (Gaussian random projection P of
    shape p x k).  Counter layout (a reading; the pages give none): entry
    (row r, column j) of sample ``sample`` in layer ``layer`` is lane r mod 4
    of the counter (r // 4, j, sample, layer).  A shared probe (one P for
    the whole batch) is the ``sample = 0`` matrix.
    """
    ngroups = (p + PROBE_LANES - 1) // PROBE_LANES
    g = np.arange(ngroups, dtype=np.uint64)[:, None]
    j = np.arange(k, dtype=np.uint64)[None, :]
    z = normals_from_counters(g, j, sample, layer, seed)  # [ngroups, k, 4]
    P = z.transpose(0, 2, 1).reshape(ngroups * PROBE_LANES, k)
    return P[:p].copy()


def rademacher_probe_matrix(seed, layer, sample, p, k):
    """A {+1, -1} probe P_i in R^{p x k} (Rademacher: independent fair signs).

    [RC] section 意義と主張 names {+-1}-valued sketching matrices as a way to
    cut the overhead further.  Reading (the pages give no generator): the
    same counters and lanes as the Gaussian probe -- entry (r, j) uses lane
    r mod 4 of the counter (r // 4, j, sample, layer) -- and the entry is +1
    when the top bit of that 32-bit word is 0, -1 when it is 1.
    """
    ngroups = (p + PROBE_LANES - 1) // PROBE_LANES
    g = np.arange(ngroups, dtype=np.uint64)[:, None]
    j = np.arange(k, dtype=np.uint64)[None, :]
    w = philox4x32_10(g, j, sample, layer, seed)  # [ngroups, k, 4] uint32
    sign = 1.0 - 2.0 * (w >> np.uint32(31)).astype(np.float64)
    P = sign.transpose(0, 2, 1).reshape(ngroups * PROBE_LANES, k)
    return P[:p].copy()


def noise_vector(seed, layer, n, offset=0):
    """DP noise xi[e] ~ N(0, 1) for flat parameter indices e in [offset, offset+n).

    [DPSGD] section DP-SGDのアルゴリズム, step 4 (Gaussian noise on the
    clipped sum).  Counter layout (a reading): element e is lane e mod 4 of
    the counter (low word of e // 4, high word of e // 4, 0xFFFFFFFF, layer).
    The element index of theta[o][q] (o < p output rows, q < d inputs) is
    e = o * d + q.
    """
    if n == 0:
        return np.zeros(0, dtype=np.float64)
    e = np.arange(offset, offset + n, dtype=np.uint64)
    grp = e >> np.uint64(2)
    first = int(grp[0])
    last = int(grp[-1])
    groups = np.arange(first, last + 1, dtype=np.uint64)
    z = normals_from_counters(groups & np.uint64(MASK32), groups >> np.uint64(32),
                              NOISE_C2, layer, seed)  # [ngroups, 4]
    lane = (e & np.uint64(3)).astype(np.int64)
    return z[(grp - np.uint64(first)).astype(np.int64), lane]

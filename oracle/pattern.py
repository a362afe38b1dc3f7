"""Oracle: block-selection rules and their CSR encoding (test infrastructure only).

Notation follows [P1] section 3.1: sequence length N, block size ``block_size``
(the page's 32), M = N / block_size blocks, query block ``row_i``.

Readings of the pages taken here (each one is also listed in the design notes):

* The log-stride exponent runs k = 1 .. ceil(log2(M)) ([P1] section 3.1 prints
  "k=1,2,...,ceil(log2(128))=7").  ceil(log2 M) is computed with integers.
* A stride floor(2^k / block_size) that is 0 adds the query block itself: it
  changes nothing.
* Targets outside [0, M) are dropped ([P1] section 3.1 intersects with
  [0, 127]).
* The three global anchors (block 0, M/2 and M-1) are added as *columns* of
  every row; the anchor rows themselves are not made dense ([P1] section 3.1
  lists them in the set of K blocks each token connects to).
* The selected set of a row is a set: duplicates collapse, CSR columns ascend.

Further rules (the pattern configuration examples of the Ascend CANN
SparseFlashAttention article: a sliding window with dilation and BigBird's
local + global + random blocks; BigBird also in [P1] section 2.2):

* Dilated window: S(i) = {i + dilation * t : |t| <= window} in [0, M), plus the
  global blocks given.
* BigBird: local {i - r .. i + r}, the global blocks given (columns only, as
  for the log-linear anchors) and ``num_random`` further blocks.  The pages
  name no generator; the draw is SplitMix64 (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", 2014, in the form of Vigna's
  reference code) read as a counter-based generator: output n of the
  sequence started at ``seed``.  Candidate c of row i is output
  i * 2**32 + c + 1 modulo M; blocks already in the row are skipped; the draw
  stops after ``num_random`` new blocks, a full row, or 64 M + 1024
  candidates.
* Causal: row i keeps only blocks j <= i.

Pins (tests/test_oracle.py): the hand-derived rows and row-size histogram of
the page's worked example N=4096, block 32 (tests/golden/), the hand-derived
tiny case, a closed-form offset description of every log-linear row, the
O(log M) row bound, own-block membership and symmetry; the ±4 block band that
the page's ±256-token window produces at block 64 (closed form 2080/4096
coverage); CSR round trips; SplitMix64's published first outputs from seed 0;
a dilated window of dilation 1 equal to a plain band, hand-derived dilated
rows; BigBird row contents (local and global blocks present, exactly
``num_random`` others, a full row when more are asked than exist), seed
dependence and the uniformity of the draw; causal filtering against the
lower triangle.
"""

from __future__ import annotations

import numpy as np


def ceil_log2(m: int) -> int:
    """ceil(log2(m)) for an integer m >= 1, without floating point."""
    if m < 1:
        raise ValueError("ceil_log2 needs m >= 1")
    return (m - 1).bit_length()


def loglinear_block_sets(seq_len: int, block_size: int, *, local_radius: int = 1,
                         k_max: int | None = None, global_blocks=None) -> list[set[int]]:
    """Selected K blocks of every query block under the log-linear rule.

    [P1] section 3.1 ("block partitioning and index mapping"), for the query
    block row_i of a token:

    1. Local: row_i - 1, row_i, row_i + 1, kept inside [0, M).
    2. Log-stride: for k = 1 .. ceil(log2 M) add row_i - floor(2^k / block_size)
       and row_i + floor(2^k / block_size) (the 2^k is a token distance, so it
       is divided by the block size to become a block distance), kept inside
       [0, M).
    3. Global: blocks 0, M/2 and M - 1.

    ``local_radius``, ``k_max`` and ``global_blocks`` generalise the printed
    constants (1, ceil(log2 M) and {0, M/2, M-1}); the defaults are the page's.
    """
    if block_size <= 0 or seq_len <= 0 or seq_len % block_size != 0:
        raise ValueError("seq_len must be a positive multiple of block_size")
    M = seq_len // block_size
    if k_max is None:
        k_max = ceil_log2(M)
    if global_blocks is None:
        global_blocks = [0, M // 2, M - 1]
    for g in global_blocks:
        if not 0 <= g < M:
            raise ValueError(f"global block {g} outside [0, {M})")

    sets: list[set[int]] = []
    for row_i in range(M):
        selected: set[int] = set()
        # 1. local blocks
        for j in range(row_i - local_radius, row_i + local_radius + 1):
            if 0 <= j < M:
                selected.add(j)
        # 2. log-stride blocks: token stride 2^k turned into a block stride
        for k in range(1, k_max + 1):
            stride = (2 ** k) // block_size
            for j in (row_i - stride, row_i + stride):
                if 0 <= j < M:
                    selected.add(j)
        # 3. global anchor blocks
        for g in global_blocks:
            selected.add(int(g))
        sets.append(selected)
    return sets


_GOLDEN = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1


def splitmix64_at(seed: int, n: int) -> int:
    """Output number n (n >= 1) of SplitMix64 started at state ``seed``.

    The generator adds the golden-ratio constant 0x9e3779b97f4a7c15 to its
    state per step and returns a mix of the new state: xor-shift 30, multiply
    by 0xbf58476d1ce4e5b9, xor-shift 27, multiply by 0x94d049bb133111eb,
    xor-shift 31 (all modulo 2**64).  After n steps the state is
    seed + n * golden, so any output can be formed directly.
    """
    z = (seed + n * _GOLDEN) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def dilated_block_sets(seq_len: int, block_size: int, *, window: int, dilation: int,
                       global_blocks=()) -> list[set[int]]:
    """Dilated sliding window over blocks: {i + dilation * t : |t| <= window}."""
    if block_size <= 0 or seq_len <= 0 or seq_len % block_size != 0:
        raise ValueError("seq_len must be a positive multiple of block_size")
    if window < 0 or dilation < 1:
        raise ValueError("window >= 0 and dilation >= 1 required")
    M = seq_len // block_size
    sets = []
    for i in range(M):
        selected = set()
        for t in range(-window, window + 1):
            j = i + dilation * t
            if 0 <= j < M:
                selected.add(j)
        for g in global_blocks:
            if not 0 <= g < M:
                raise ValueError(f"global block {g} outside [0, {M})")
            selected.add(int(g))
        sets.append(selected)
    return sets


def bigbird_block_sets(seq_len: int, block_size: int, *, num_random: int, seed: int,
                       local_radius: int = 1, global_blocks=()) -> list[set[int]]:
    """Local + global + random blocks per row (see the module notes for the draw)."""
    if block_size <= 0 or seq_len <= 0 or seq_len % block_size != 0:
        raise ValueError("seq_len must be a positive multiple of block_size")
    if num_random < 0:
        raise ValueError("num_random >= 0 required")
    M = seq_len // block_size
    sets = []
    for i in range(M):
        selected = set()
        for j in range(i - local_radius, i + local_radius + 1):
            if 0 <= j < M:
                selected.add(j)
        for g in global_blocks:
            if not 0 <= g < M:
                raise ValueError(f"global block {g} outside [0, {M})")
            selected.add(int(g))
        added = 0
        c = 0
        while added < num_random and len(selected) < M and c < 64 * M + 1024:
            j = splitmix64_at(seed, (i << 32) + c + 1) % M
            c += 1
            if j in selected:
                continue
            selected.add(j)
            added += 1
        sets.append(selected)
    return sets


def causal_block_sets(sets: list[set[int]]) -> list[set[int]]:
    """Row i keeps only blocks j <= i."""
    return [{j for j in s if j <= i} for i, s in enumerate(sets)]


def block_mask_from_sets(sets: list[set[int]]) -> np.ndarray:
    """[M, M] uint8 block mask with mask[i, j] = 1 iff j is selected by row i."""
    M = len(sets)
    mask = np.zeros((M, M), dtype=np.uint8)
    for i, s in enumerate(sets):
        for j in s:
            mask[i, j] = 1
    return mask


def csr_from_block_mask(mask: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """CSR of a block mask: row_ptr int32[M+1], col_idx int32[nnz].

    row_ptr[0] = 0, row_ptr[i+1] = row_ptr[i] + |S(i)|, and col_idx lists S(i)
    in ascending order.  This is the per-query-block index table of [P1]
    section 3.2 ("precomputed on the CPU before launch"), stored as CSR because
    the number of K blocks differs from row to row.
    """
    mask = np.asarray(mask)
    if mask.ndim != 2 or mask.shape[0] != mask.shape[1]:
        raise ValueError("block mask must be square")
    M = mask.shape[0]
    row_ptr = np.zeros(M + 1, dtype=np.int64)
    cols: list[int] = []
    for i in range(M):
        row_cols = np.nonzero(mask[i])[0]
        cols.extend(int(c) for c in row_cols)
        row_ptr[i + 1] = row_ptr[i] + len(row_cols)
    return row_ptr.astype(np.int32), np.asarray(cols, dtype=np.int32)


def block_mask_from_csr(row_ptr, col_idx, M: int) -> np.ndarray:
    """Decode a CSR back into an [M, M] uint8 block mask."""
    mask = np.zeros((M, M), dtype=np.uint8)
    for i in range(M):
        for t in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            mask[i, int(col_idx[t])] = 1
    return mask


def local_global_token_mask(seq_len: int, local_window: int, global_tokens) -> np.ndarray:
    """Token-level [N, N] bool mask of the local + global rule.

    [P3] "sparse pattern: Local + Global" states the rule: a token attends to
    every token at distance at most ``local_window`` from it, and a global
    token both attends to and is attended by every position.  Here the band
    is the set {(i, j) : |i - j| <= local_window}, formed by comparing the
    row and column position vectors; each global token then sets its whole
    row and column.  Negative global indices count from the end.
    """
    pos = np.arange(seq_len)
    mask = np.abs(pos[:, None] - pos[None, :]) <= local_window
    rows = np.asarray([int(g) % seq_len for g in global_tokens], dtype=np.int64)
    mask[rows, :] = True
    mask[:, rows] = True
    return mask


def token_mask_to_block_mask(token_mask: np.ndarray, block_size: int) -> np.ndarray:
    """Block mask of a token mask under the more-than-half rule.

    [P3] "Block-Sparse": a (query block, key block) tile is computed when more
    than half of its token pairs are set.  The token mask is padded with unset
    entries up to a whole number of blocks, reshaped to
    [blocks, block_size, blocks, block_size], and the set pairs of each tile
    are counted; a tile is kept when twice its count exceeds the number of
    real token pairs it covers (a partial last block covers fewer).
    """
    n = token_mask.shape[0]
    nb = -(-n // block_size)
    padded = np.zeros((nb * block_size, nb * block_size), dtype=np.int64)
    padded[:n, :n] = token_mask
    counts = padded.reshape(nb, block_size, nb, block_size).sum(axis=(1, 3))
    extent = np.minimum(block_size, n - block_size * np.arange(nb))  # tokens per block
    pairs = extent[:, None] * extent[None, :]
    return (2 * counts > pairs).astype(np.uint8)

"""Constants of the input generator (kept free of any library loading)."""

F32, BF16, F16 = 0, 1, 2
TABLE_SIZE = 65536 + 1

# buffer ids inside a stream tag
BUF_GRAD, BUF_MASTER, BUF_M, BUF_V, BUF_MISC = 1, 2, 3, 4, 5


def outlier_threshold(p):
    """Low-20-bit threshold giving an outlier probability of about p."""
    return int(round(p * (1 << 20)))


def tag(buf, cfg=0, step=0, micro=0, k=0):
    """Pack (buffer, config, step, micro-batch, contributing rank) into one
    64-bit stream tag: 8 | 8 | 16 | 8 | 24 bits."""
    assert 0 <= buf < 256 and 0 <= cfg < 256 and 0 <= step < 65536
    assert 0 <= micro < 256 and 0 <= k < (1 << 24)
    return (buf << 56) | (cfg << 48) | (step << 32) | (micro << 24) | k

"""Chosen hashes for draw tests: the inverse of MurmurHash3's 32-bit finaliser (each step
undone in reverse order), so a test can pick the counter whose hash is a given value."""
M32 = 0xFFFFFFFF


def inv_fmix32(h: int) -> int:
    """The input whose fmix32 is h."""
    h ^= h >> 16                              # x ^ (x >> 16) is its own inverse
    h = (h * pow(0xC2B2AE35, -1, 1 << 32)) & M32
    x = h                                     # undo x ^ (x >> 13): fixed point, 3 rounds
    for _ in range(3):
        x = h ^ (x >> 13)
    h = (x * pow(0x85EBCA6B, -1, 1 << 32)) & M32
    return h ^ (h >> 16)


def counter_for_hash(key: int, h: int) -> int:
    """The element counter whose draw under worker key `key` hashes to h."""
    return inv_fmix32(h) ^ key

"""Oracle for the block keys of the prefix cache of compressed maps.

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module.  It
shares no code with the HIP library.

The MapFlow page (163.com article "跨模型上下文交接还要重算KV?北大提出MapFlow",
section "让复用真正省时,还需要解决存储和执行问题", paragraph "第二") manages the
sender's compressed state by shared prefix.  In a causal sender, row-block i
depends only on tokens [0, (i + 1) B), so the state of row-block i is keyed by
a chained hash of the first i + 1 blocks of tokens.  The page fixes no hash;
the library uses 64-bit FNV-1a (the Fowler-Noll-Vo "1a" variant: per byte,
xor then multiply by the FNV prime, starting from the offset basis), chained
as follows: key[i] = FNV-1a over the 8 little-endian bytes of key[i - 1]
(the parent key, 0 at a sequence start) followed by the B tokens of block i,
each 4 bytes little-endian.  Pure-Python integer arithmetic, straight from
that definition.
"""
from __future__ import annotations

from typing import List, Sequence

FNV_OFFSET_BASIS_64 = 0xCBF29CE484222325
FNV_PRIME_64 = 0x100000001B3
MASK_64 = (1 << 64) - 1


def fnv1a_64(data: bytes, h: int = FNV_OFFSET_BASIS_64) -> int:
    """FNV-1a over `data`, continuing from state h."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME_64) & MASK_64
    return h


def prefix_block_keys(tokens: Sequence[int], B: int, parent: int = 0) -> List[int]:
    """One key per full block of B tokens; key i covers tokens [0, (i + 1) B)."""
    keys = []
    prev = parent
    for i in range(len(tokens) // B):
        data = prev.to_bytes(8, "little")
        for t in tokens[i * B:(i + 1) * B]:
            data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
        prev = fnv1a_64(data)
        keys.append(prev)
    return keys

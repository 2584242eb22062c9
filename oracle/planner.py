"""Pipeline chunk rule (oracle, test infrastructure only).

[pipe], section "Summary" (the formula) and "What changed" (the rounding): a
prompt of n tokens read in chunks of C over S pipeline stages takes
(S - 1 + n/C) stage-chunks of (b + a*C), which is smallest at
C = sqrt(n * (b/a) / (S - 1)).  The chunk is rounded up to the 256-token grid,
kept at least 512 and at most the buffers' chunk, then evened out over the
chunks it takes so that there is no short last chunk.  A prompt that would be
read in one chunk keeps the one-chunk path.  With one stage the rule does not
apply: the largest chunk the buffers allow is used.

Reading taken for "evened out": k = ceil(n / C0) chunks, C = roundup_256(ceil(n / k)).
Pinned by: the page's table of chosen chunks (1024, 1024, 2048, 3328 at
2,013 / 3,865 / 10,041 / 28,998 tokens on four stages).
"""
from __future__ import annotations

import math


def _roundup(v: int, g: int = 256) -> int:
    return -(-int(v) // g) * g


def pipeline_chunk(n: int, cap: int, stages: int, b_over_a: float = 1024.0) -> int:
    """Chunk size for an n-token prompt over `stages` stages, at most `cap`."""
    if n <= 0:
        return 0
    if stages <= 1:
        return min(n, cap)
    c0 = _roundup(math.ceil(math.sqrt(n * b_over_a / (stages - 1))))
    c0 = max(512, min(cap, c0))
    k = -(-n // c0)
    if k <= 1:
        return min(n, cap)
    return min(cap, _roundup(-(-n // k)))

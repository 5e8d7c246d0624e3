"""Host checks of the parity helpers that pick which tokens the full-size GPU
tests compare with the oracle (no GPU needed)."""
import numpy as np

from parity import tile_edge_tokens, tile_spans
from synthetic import Workload


def test_prefill_tiles_are_balanced_and_cover_every_row():
    # 300 rows -> two tiles of 150; 0 rows -> none; 44 -> one; 513 -> 171, 171, 171
    spans = tile_spans("stream", 256, [300, 0, 44, 513], 1000, has_shared=True)
    routed = [s for s in spans if s[0] < 4]
    assert routed == [(0, 0, 150), (0, 150, 150), (2, 300, 44), (3, 344, 171), (3, 515, 171), (3, 686, 171)]
    shared = [s for s in spans if s[0] == 4]
    assert shared == [(4, 0, 250), (4, 250, 250), (4, 500, 250), (4, 750, 250)]


def test_other_paths_take_full_tiles_and_a_ragged_last_one():
    spans = tile_spans("stream_decode", 32, [70, 32], 5, has_shared=False)
    assert spans == [(0, 0, 32), (0, 32, 32), (0, 64, 6), (1, 70, 32)]
    assert tile_spans("tiled", 128, [129], 0, False) == [(0, 0, 128), (0, 128, 1)]


def test_tile_edge_tokens_follow_the_permutation():
    # 6 tokens, top-2 over 3 experts; slots t*k+j; expert-contiguous perm
    w = Workload("t", 6, 64, 3, 2, 64, 64, "softmax", 1, 1, 1.0, "bf16", "zero")
    idx = np.array([[0, 1], [1, 2], [0, 2], [2, 1], [0, 1], [2, 0]])
    flat = idx.reshape(-1)
    perm = np.concatenate([np.nonzero(flat == e)[0] for e in range(3)])
    counts = np.bincount(flat, minlength=3)
    tok, n = tile_edge_tokens(w, "stream_decode", 2, counts, perm, 6)
    # expert 0 slots (tokens 0, 2, 4, 5): tiles [0,2] -> tokens 0, 2; [4, 5] -> 4, 5
    # expert 1 slots (tokens 0, 1, 3, 4): tiles -> 0, 1 and 3, 4; expert 2 (1, 2, 3, 5): 1, 2 and 3, 5
    # shared: token pairs (0,1), (2,3), (4,5)
    assert n == 2 + 2 + 2 + 3
    assert tok.tolist() == [0, 1, 2, 3, 4, 5]
    tok, _ = tile_edge_tokens(w, "stream_decode", 4, counts, perm, 6)
    # 4-row tiles: expert 0 -> first/last 0, 5; expert 1 -> 0, 4; expert 2 -> 1, 5; shared (0..3), (4, 5)
    assert tok.tolist() == [0, 1, 3, 4, 5]

"""Layout description and validation in plain Python (TEST INFRASTRUCTURE ONLY).

Follows the MiniMaxH3Transformer3DModel page (`forward` parameters
token_tags, timestep_indices, video/audio/text_indices; class description on
padding rows). For a packed sequence of S rows it derives, with set
operations, the per-row AdaLN table row (tag * n_tvals + tidx, -1 for padding
rows), the attention document of each row (1 for tag -1, else 0), the number
of padding rows and, for every 64-row tile, which documents it holds; and it
decides the status code of a malformed layout.

Status codes and their precedence (the first that applies is returned):
  -10 tag not in {-1, 0 .. n_tags-1}
  -11 timestep index outside [0, n_tvals) on a non-padding row
  -12 an index outside [0, S), a row addressed twice, or an index whose row
      carries another modality's tag
  -13 an index addresses a padding row, or a non-padding row is addressed by
      no index tensor
  -14 padding rows present although the caller promised a padless sequence
"""
from __future__ import annotations

import numpy as np

OK, E_TAG, E_TVAL, E_INDEX, E_PAD, E_NEEDS_MASK = 0, -10, -11, -12, -13, -14
TILE = 64


def describe(tags, tidx, video_idx, audio_idx, text_idx, num_tags: int, num_tvals: int,
             tag_video: int, tag_audio: int, tag_text: int, assume_padless: bool = False):
    tags = [int(t) for t in tags]
    tidx = [int(t) for t in tidx]
    S = len(tags)
    errors = set()
    for t in tags:
        if t != -1 and not (0 <= t < num_tags):
            errors.add(E_TAG)
    for t, k in zip(tags, tidx):
        if t != -1 and not (0 <= k < num_tvals):
            errors.add(E_TVAL)
    seen = {}
    for idx, want in ((video_idx, tag_video), (audio_idx, tag_audio), (text_idx, tag_text)):
        for i in idx:
            i = int(i)
            if not (0 <= i < S):
                errors.add(E_INDEX)
                continue
            seen[i] = seen.get(i, 0) + 1
            if tags[i] == -1:
                errors.add(E_PAD)
            elif tags[i] != want:
                errors.add(E_INDEX)
    if any(c > 1 for c in seen.values()):
        errors.add(E_INDEX)
    for i, t in enumerate(tags):
        if t != -1 and i not in seen:
            errors.add(E_PAD)
    pads = {i for i, t in enumerate(tags) if t == -1}
    if assume_padless and pads:
        errors.add(E_NEEDS_MASK)
    status = OK
    for code in (E_TAG, E_TVAL, E_INDEX, E_PAD, E_NEEDS_MASK):
        if code in errors:
            status = code
            break
    table_row = [(-1 if t == -1 else t * num_tvals + k) for t, k in zip(tags, tidx)]
    doc = [1 if i in pads else 0 for i in range(S)]
    n_tiles = (S + TILE - 1) // TILE
    tile_flags = []
    for tt in range(n_tiles):
        members = range(tt * TILE, min(S, (tt + 1) * TILE))
        has_real = any(i not in pads for i in members)
        has_pad = any(i in pads for i in members)
        tile_flags.append((1 if has_real else 0) | (2 if has_pad else 0))
    return dict(status=status, table_row=np.array(table_row, np.int32), doc=np.array(doc, np.int32),
                num_pad=len(pads), tile_flags=np.array(tile_flags, np.int32))

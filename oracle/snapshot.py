"""Prefix-cache snapshots of the recurrent state, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Automatic prefix caching on a recurrent hybrid (dflash-caddtree-integrations
README, "What's in here", the gdn_apc row: prefix caching under speculative
decoding, with a warm start bitwise equal to a cold one) keeps the committed
state a sequence reached after a shared prefix, and restores it into another
sequence's slot instead of recomputing the prefix.  Both directions are whole
slot copies: every value head's D_v x D_k fp32 state.

copy_slots: for each entry i, dst[dst_slot[i]] = src[src_slot[i]]; an entry
with a slot outside its cache is skipped.
"""
from __future__ import annotations

import numpy as np


def copy_slots(src: np.ndarray, src_slot, dst: np.ndarray, dst_slot) -> np.ndarray:
    """src [S_src][H][Dv][Dk], dst [S_dst][H][Dv][Dk]; returns the new dst."""
    out = np.array(dst, copy=True)
    for s, d in zip(np.asarray(src_slot), np.asarray(dst_slot)):
        if 0 <= s < src.shape[0] and 0 <= d < out.shape[0]:
            out[d] = src[s]
    return out

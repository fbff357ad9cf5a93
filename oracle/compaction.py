"""Removing evicted entries from a slot set.

After eviction the survivors form the new cache (MomentKV Algorithm 1, step
14: R <- R minus j*; InertiaKV §3: eviction is irreversible). The oracle keeps
survivors in their old slot order (a stable compaction). Slot order carries
no meaning for the method, so comparisons with the HIP path go by token
position, never by slot.
"""
from __future__ import annotations

import numpy as np


def compact(arrays: dict, evicted, slot_axis: dict | None = None) -> dict:
    """Drop the evicted slots from every array in `arrays`.

    arrays: name -> array whose slot axis is given by slot_axis[name] (default 0).
    evicted: slot indices to remove.
    """
    slot_axis = slot_axis or {}
    out = {}
    for name, a in arrays.items():
        ax = slot_axis.get(name, 0)
        a = np.asarray(a)
        keep = np.ones(a.shape[ax], dtype=bool)
        keep[np.asarray(evicted, dtype=np.int64)] = False
        out[name] = np.compress(keep, a, axis=ax)
    return out

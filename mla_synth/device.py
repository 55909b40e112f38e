"""Upload a :class:`mla_synth.Case` to GPU tensors (plumbing only: copies, no
arithmetic)."""
import numpy as np
import torch


def _t(x, device):
    if x is None:
        return None
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def upload(case, device="cuda"):
    """Returns a dict of device tensors: rows (uint8 [n_rows, row_stride]),
    scale (float32 or None), seq_start / seq_cap / seq_len (int32; seq_len is
    the cached length before any append), q_nope, q_rope, w_uk, w_uv and, for
    appending workloads, h, w_dkv, w_kr (float32, or int16 holding bf16 bits)."""
    out = {
        "rows": _t(case.rows, device),
        "scale": _t(case.scale, device),
        "seq_start": _t(case.seq_start.astype(np.int32), device),
        "seq_cap": _t(case.seq_cap.astype(np.int32), device),
        "seq_len": _t(case.lens.astype(np.int32), device),
    }
    for k in ("q_nope", "q_rope", "w_uk", "w_uv", "h", "w_dkv", "w_kr"):
        out[k] = _t(getattr(case, k), device)
    return out

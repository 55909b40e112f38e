"""Test helpers: run the HIP path through the binding, and the oracle on the
same seeded case. The two sides share only mla_synth's inputs."""
import math

import numpy as np
import torch

import mla_synth
from mla_synth.device import upload
from oracle import codecs
from oracle import mla as omla

DT = {"f32": 0, "bf16": 1, "fp8": 2}


def act_to_f64(x, dtype):
    if x is None:
        return None
    return codecs.bf16_decode(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def case_dims(m, case):
    return m.dims(case.H, case.d_c, case.d_rope, case.d_nope, case.d_v, case.d_model,
                  case.softmax_scale, case.rope_base)


def paged_layout(case, block_tokens, seed, spare_blocks=3):
    """The case's cache rearranged into blocks of block_tokens rows in a
    shuffled order: returns (rows, scale, block_table) with rows [n_blocks *
    block_tokens, row_stride] (unused blocks filled with 0xAB bytes), scale
    likewise (or None), block_table int32 [B, max_blocks] (-1 past a
    sequence's blocks). Token t of sequence b moves from row seq_start[b] + t
    to row block_table[b, t // bt] * bt + t % bt."""
    rng = np.random.default_rng(seed)
    bt = block_tokens
    nblk = [(int(c) + bt - 1) // bt for c in case.seq_cap]
    total = sum(nblk) + spare_blocks
    max_blocks = max(max(nblk), 1)
    ids = rng.permutation(total).astype(np.int32)
    table = np.full((case.B, max_blocks), -1, dtype=np.int32)
    rows = np.full((total * bt, case.row_stride), 0xAB, dtype=np.uint8)
    scale = None if case.scale is None else np.full(total * bt, 7.0, dtype=np.float32)
    k = 0
    for b in range(case.B):
        for j in range(nblk[b]):
            blk = int(ids[k])
            k += 1
            table[b, j] = blk
            n = min(bt, int(case.seq_cap[b]) - j * bt)
            src = int(case.seq_start[b]) + j * bt
            rows[blk * bt:blk * bt + n] = case.rows[src:src + n]
            if scale is not None:
                scale[blk * bt:blk * bt + n] = case.scale[src:src + n]
    return rows, scale, table


class DeviceRun:
    """Holds the device tensors of one case and runs the C-ABI entry points.
    ``paged`` = (rows, scale, block_table, block_tokens) from paged_layout()
    runs the same case on a paged copy of its cache."""

    def __init__(self, m, case, device="cuda", paged=None):
        self.m, self.case = m, case
        self.t = upload(case, device)
        self.d = case_dims(m, case)
        if paged is None:
            self.cache = m.cache(self.t["rows"], case.row_stride, DT[case.latent_dtype],
                                 DT[case.rope_dtype], self.t["seq_start"], self.t["seq_cap"],
                                 self.t["seq_len"], self.t["scale"])
        else:
            rows, scale, table, bt = paged
            self.t["rows"] = torch.from_numpy(rows).to(device)
            self.t["scale"] = None if scale is None else torch.from_numpy(scale).to(device)
            self.t["block_table"] = torch.from_numpy(table).to(device)
            self.cache = m.cache(self.t["rows"], case.row_stride, DT[case.latent_dtype],
                                 DT[case.rope_dtype], None, self.t["seq_cap"], self.t["seq_len"],
                                 self.t["scale"], block_table=self.t["block_table"], block_tokens=bt)
        self.ws = None

    def plan(self, lens=None, n_workers=0):
        lens = self.case.lens + self.case.n_new if lens is None else lens
        return self.m.mla_plan_create(self.d, lens, n_workers)

    def workspace(self, plan):
        # one token per sequence or none: the one-size query covers decode and append
        need = self.m.mla_workspace_bytes(self.d, plan)
        if self.case.n_new > 1:
            need = max(need, self.m.mla_append_workspace_bytes(self.d, self.case.B, self.case.n_new))
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.t["rows"].device)
            self.m.mla_workspace_init(self.ws)
        return self.ws

    def append(self, plan=None):
        c = self.case
        ws = self.workspace(plan or self.plan())
        self.m.mla_append(self.d, self.cache, self.t["h"], c.n_new, self.t["w_dkv"], self.t["w_kr"],
                          DT[c.act_dtype], ws)

    def decode(self, plan=None, q_pos=None, o_dtype="f32", n_workers=0):
        c = self.case
        plan = plan or self.plan(n_workers=n_workers)
        ws = self.workspace(plan)
        o = torch.empty((c.B, c.H, c.d_v), dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16,
                        device=self.t["rows"].device)
        self.m.mla_decode(self.d, self.cache, plan, self.t["q_nope"], self.t["q_rope"], q_pos,
                          self.t["w_uk"], self.t["w_uv"], DT[c.act_dtype], o, DT[o_dtype], ws)
        return o

    def decode_multi(self, q_len, q_nope, q_rope, plan=None, q_pos=None, o_dtype="f32", n_workers=0):
        """mla_decode_multi with host query arrays [B, q_len, H, *] (storage dtype)."""
        c = self.case
        plan = plan or self.plan(n_workers=n_workers)
        need = self.m.mla_decode_multi_workspace_bytes(self.d, plan, q_len)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.t["rows"].device)
            self.m.mla_workspace_init(self.ws)
        dev = self.t["rows"].device
        qn = torch.from_numpy(np.ascontiguousarray(q_nope).view(np.int16)).to(dev)
        qr = torch.from_numpy(np.ascontiguousarray(q_rope).view(np.int16)).to(dev)
        o = torch.empty((c.B, q_len, c.H, c.d_v), dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16,
                        device=dev)
        self.m.mla_decode_multi(self.d, self.cache, plan, q_len, qn, qr, q_pos, self.t["w_uk"], self.t["w_uv"],
                                DT[c.act_dtype], o, DT[o_dtype], self.ws)
        return o

    def append_decode(self, plan=None, o_dtype="f32"):
        c = self.case
        plan = plan or self.plan()
        ws = self.workspace(plan)
        o = torch.empty((c.B, c.H, c.d_v), dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16,
                        device=self.t["rows"].device)
        self.m.mla_append_decode(self.d, self.cache, plan, self.t["h"], c.n_new, self.t["w_dkv"],
                                 self.t["w_kr"], self.t["q_nope"], self.t["q_rope"], None,
                                 self.t["w_uk"], self.t["w_uv"], DT[c.act_dtype], o, DT[o_dtype], ws)
        return o

    def status(self):
        return self.m.mla_device_error(self.ws, reset=True)


# ---------------------------------------------------------------- oracle side


def oracle_cache(case, rows=None, scale=None, seqs=None):
    """Decode the case's stored rows to fp64 (C, R). ``seqs`` limits decoding to
    those sequences' rows (others stay zero) to bound memory."""
    rows = case.rows if rows is None else rows
    scale = case.scale if scale is None else scale
    n = rows.shape[0]
    C = np.zeros((n, case.d_c))
    R = np.zeros((n, case.d_rope))
    bs = range(case.B) if seqs is None else seqs
    for b in bs:
        s0 = int(case.seq_start[b])
        s1 = s0 + int(case.seq_cap[b])
        sc = None if scale is None else scale[s0:s1]
        C[s0:s1], R[s0:s1] = omla.decode_rows(rows[s0:s1], case.latent_dtype, case.rope_dtype,
                                             case.d_c, case.d_rope, sc)
    return C, R


def oracle_append(case):
    """The oracle's own append of the case's new tokens; returns the dict of
    oracle.mla.append."""
    return omla.append(act_to_f64(case.h, case.act_dtype), act_to_f64(case.w_dkv, case.act_dtype),
                       act_to_f64(case.w_kr, case.act_dtype), case.seq_start, case.lens,
                       case.rope_base, case.latent_dtype, case.rope_dtype)


def oracle_decode(case, pairs=None, absorbed=False, with_append=True, q_pos=None, seqs=None, C=None, R=None):
    """Oracle output for the case (after its own append when the case appends)."""
    if C is None:
        C, R = oracle_cache(case, seqs=seqs)
    lens = case.lens.astype(np.int64)
    if case.n_new and with_append:
        ap = oracle_append(case)
        rows = ap["rows"].reshape(-1)
        C[rows] = ap["c"].reshape(len(rows), -1)
        R[rows] = ap["k_rope"].reshape(len(rows), -1)
        lens = ap["seq_len"]
    fn = omla.decode_absorbed if absorbed else omla.decode
    return fn(C, R, case.seq_start, lens, act_to_f64(case.q_nope, case.act_dtype),
              act_to_f64(case.q_rope, case.act_dtype), act_to_f64(case.w_uk, case.act_dtype),
              act_to_f64(case.w_uv, case.act_dtype), case.softmax_scale, case.rope_base,
              q_pos=q_pos, pairs=pairs)


def oracle_full(case, with_append=True, rows=None, scale=None):
    """Every output [B, H, d_v] of the case from the oracle's all-heads
    absorbed form (pinned equal to the definition), one sequence at a time:
    only that sequence's rows are decoded to fp64, so full-size workloads fit
    in host memory. When the case appends, the oracle's own appended rows
    stand at their positions (end to end, as the GPU appends them itself).
    ``rows`` / ``scale`` replace the case's stored rows (e.g. read back)."""
    rows = case.rows if rows is None else rows
    scale = case.scale if scale is None else scale
    lens = case.lens.astype(np.int64)
    ap = oracle_append(case) if (case.n_new and with_append) else None
    qn = act_to_f64(case.q_nope, case.act_dtype)
    qr = act_to_f64(case.q_rope, case.act_dtype)
    wuk = act_to_f64(case.w_uk, case.act_dtype)
    wuv = act_to_f64(case.w_uv, case.act_dtype)
    out = np.zeros((case.B, case.H, case.d_v))
    for b in range(case.B):
        L = int(lens[b])
        s0 = int(case.seq_start[b])
        sc = None if scale is None else scale[s0:s0 + L]
        C, R = omla.decode_rows(rows[s0:s0 + L], case.latent_dtype, case.rope_dtype, case.d_c, case.d_rope, sc)
        if ap is not None:
            C = np.concatenate([C, ap["c"][b]])
            R = np.concatenate([R, ap["k_rope"][b]])
            L += case.n_new
        out[b] = omla.decode_absorbed_heads(C, R, qn[b], qr[b], wuk, wuv, case.softmax_scale, case.rope_base, L - 1)
    return out


def oracle_decode_multi(case, q_nope, q_rope, triples=None, absorbed=True, q_pos=None, C=None, R=None):
    """Oracle output of a several-token decode (queries [B, q_len, H, *] in
    storage dtype)."""
    if C is None:
        C, R = oracle_cache(case)
    return omla.decode_multi(C, R, case.seq_start, case.lens.astype(np.int64), act_to_f64(q_nope, case.act_dtype),
                             act_to_f64(q_rope, case.act_dtype), act_to_f64(case.w_uk, case.act_dtype),
                             act_to_f64(case.w_uv, case.act_dtype), case.softmax_scale, case.rope_base,
                             q_pos=q_pos, triples=triples, absorbed=absorbed)


def rel_rms_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(math.sqrt(float(np.mean(ref ** 2))), 1e-300))


def max_abs_err(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


# Tolerances stated by the workloads: fp32 max |err| <= 1e-4; bf16 cache
# max|err| / rms <= 2e-2; fp8 cache max|err| / rms <= 6e-2.
TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2
TOL_FP8_REL = 6e-2


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def make(name="custom", **kw):
    return mla_synth.make_case(name, **kw)

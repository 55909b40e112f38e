"""Python binding of libmla (MLA decode with weight absorption on MI355X).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. Functions carry the C names of include/mla.h and take torch tensors
on the current HIP device (contiguous), or plain Python values. PyTorch
supplies device memory and the current stream; the library allocates no
device memory. A missing library raises; there is no fallback.
"""
import ctypes
import os

__all__ = [
    "F32", "BF16", "FP8_E4M3", "MLAError", "MlaDims", "MlaCache", "Plan", "load", "lib_path",
    "dims", "cache", "mla_plan_create", "mla_plan_create_multi", "mla_append_workspace_bytes",
    "mla_decode_workspace_bytes", "mla_workspace_bytes", "mla_append", "mla_decode", "mla_append_decode",
    "mla_decode_multi", "mla_decode_multi_workspace_bytes", "mla_decode_noalloc",
    "mla_merge_query_weight", "mla_merge_output_weight", "mla_decode_merged", "mla_decode_merged_workspace_bytes",
    "mla_workspace_init", "mla_device_error", "mla_status_str", "mla_abi_version",
    "mla_prof_begin", "mla_prof_end", "mla_calib_copy", "mla_calib_read", "EXPORTED",
    "workspace", "decode", "append", "append_decode",
]

F32, BF16, FP8_E4M3 = 0, 1, 2
STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_CAPACITY",
          4: "MLA_ERR_HIP", 5: "MLA_ERR_WORKSPACE", 6: "MLA_ERR_PLAN", 7: "MLA_ERR_RANGE"}

# Every extern "C" entry point of include/mla.h.
EXPORTED = [
    "mla_append_workspace_bytes", "mla_append", "mla_plan_create", "mla_plan_create_multi", "mla_plan_destroy",
    "mla_plan_num_items", "mla_plan_item", "mla_plan_num_ranges", "mla_plan_range", "mla_decode_workspace_bytes", "mla_workspace_bytes", "mla_decode",
    "mla_decode_multi_workspace_bytes", "mla_decode_multi", "mla_decode_noalloc", "mla_append_decode",
    "mla_workspace_init", "mla_device_error", "mla_status_str",
    "mla_abi_version", "mla_prof_begin", "mla_prof_end", "mla_prof_kernel_name",
    "mla_prof_num_kernels", "mla_calib_copy", "mla_calib_read", "mla_merge_query_weight",
    "mla_merge_output_weight", "mla_decode_merged", "mla_decode_merged_workspace_bytes",
]


class MLAError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class MlaDims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float)]


class MlaCache(ctypes.Structure):
    _fields_ = [("latent_dtype", ctypes.c_int), ("rope_dtype", ctypes.c_int),
                ("rows", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
                ("scale", ctypes.c_void_p), ("n_rows", ctypes.c_int64), ("batch", ctypes.c_int32),
                ("seq_start", ctypes.c_void_p), ("seq_cap", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("block_tokens", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


_LIB = None
_P = ctypes.c_void_p


def lib_path():
    """The in-tree libmla.so, or the build MLA_LIBRARY names (e.g. a host-only
    AddressSanitizer build from build.build_host_asan)."""
    return os.environ.get("MLA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")


def load():
    """Load libmla.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = lib_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    sig = {
        "mla_append_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32, ctypes.c_int32]),
        "mla_append": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_int, _P,
                                      ctypes.c_size_t, _P]),
        "mla_plan_create": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P]),
        "mla_plan_create_multi": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]),
        "mla_plan_destroy": (None, [_P]),
        "mla_plan_num_items": (ctypes.c_int32, [_P]),
        "mla_plan_item": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P]),
        "mla_plan_num_ranges": (ctypes.c_int32, [_P]),
        "mla_plan_range": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P]),
        "mla_decode_workspace_bytes": (ctypes.c_size_t, [_P, _P]),
        "mla_workspace_bytes": (ctypes.c_size_t, [_P, _P]),
        "mla_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P,
                                      ctypes.c_int, _P, ctypes.c_size_t, _P]),
        "mla_decode_multi_workspace_bytes": (ctypes.c_size_t, [_P, _P, ctypes.c_int32]),
        "mla_decode_multi": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_int, _P,
                                            ctypes.c_int, _P, ctypes.c_size_t, _P]),
        "mla_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int, _P,
                                              _P]),
        "mla_append_decode": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                             _P, _P, ctypes.c_int, _P, ctypes.c_int, _P,
                                             ctypes.c_size_t, _P]),
        "mla_merge_query_weight": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, ctypes.c_int, _P, _P]),
        "mla_merge_output_weight": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, ctypes.c_int, _P, _P]),
        "mla_decode_merged": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, _P,
                                             ctypes.c_int, _P, ctypes.c_int, _P, ctypes.c_size_t, _P]),
        "mla_decode_merged_workspace_bytes": (ctypes.c_size_t, [_P, _P, ctypes.c_int32]),
        "mla_workspace_init": (ctypes.c_int, [_P, ctypes.c_size_t, _P]),
        "mla_device_error": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32]),
        "mla_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "mla_abi_version": (ctypes.c_int32, []),
        "mla_prof_begin": (ctypes.c_int, [ctypes.c_int32]),
        "mla_prof_end": (ctypes.c_int, [_P, _P, ctypes.c_int32]),
        "mla_prof_kernel_name": (ctypes.c_char_p, [ctypes.c_int32]),
        "mla_prof_num_kernels": (ctypes.c_int32, []),
        "mla_calib_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
        "mla_calib_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def _check(st, where):
    if st != 0:
        raise MLAError(st, where)


def _ptr(t):
    """Device pointer of a contiguous tensor (or None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def dims(n_heads, d_c, d_rope, d_nope, d_v, d_model=0, softmax_scale=None, rope_base=10000.0):
    """mla_dims; softmax_scale None passes 0, which the library reads as (d_nope + d_rope)^-1/2."""
    return MlaDims(n_heads, d_c, d_rope, d_nope, d_v, d_model, 0.0 if softmax_scale is None else softmax_scale,
                   rope_base)


def cache(rows, row_stride, latent_dtype, rope_dtype, seq_start, seq_cap, seq_len, scale=None,
          block_table=None, block_tokens=0):
    """Describe a cache held in torch tensors: rows is uint8 [n_rows, row_stride];
    seq_* are int32 [batch]; scale is float32 [n_rows] for fp8 latents. A paged
    cache passes block_table, int32 [batch, max_blocks], and block_tokens (then
    seq_start may be None)."""
    batch = seq_cap.numel()
    c = MlaCache(latent_dtype, rope_dtype, _ptr(rows), row_stride, _ptr(scale),
                 rows.numel() // row_stride, batch, _ptr(seq_start), _ptr(seq_cap),
                 _ptr(seq_len), _ptr(block_table), block_tokens,
                 0 if block_table is None else block_table.shape[-1])
    c._keep = (rows, scale, seq_start, seq_cap, seq_len, block_table)
    return c


class Plan:
    """Owns an mla_plan*; destroyed with the object."""

    def __init__(self, handle, batch):
        self.handle = handle
        self.batch = batch

    @property
    def n_items(self):
        return load().mla_plan_num_items(self.handle)

    def items(self):
        lib = load()
        b, t0, t1 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        out = []
        for k in range(self.n_items):
            _check(lib.mla_plan_item(self.handle, k, ctypes.byref(b), ctypes.byref(t0), ctypes.byref(t1)),
                   "mla_plan_item")
            out.append((b.value, t0.value, t1.value))
        return out

    def ranges(self):
        """[(first item, end item)] of every workgroup range."""
        lib = load()
        k0, k1 = ctypes.c_int32(), ctypes.c_int32()
        out = []
        for j in range(lib.mla_plan_num_ranges(self.handle)):
            _check(lib.mla_plan_range(self.handle, j, ctypes.byref(k0), ctypes.byref(k1)), "mla_plan_range")
            out.append((k0.value, k1.value))
        return out

    def __del__(self):
        if self.handle and _LIB is not None:
            _LIB.mla_plan_destroy(self.handle)
            self.handle = None


def mla_plan_create(d, host_lens, n_workers=0):
    lens = [int(x) for x in host_lens]
    arr = (ctypes.c_int32 * len(lens))(*lens)
    h = ctypes.c_void_p()
    _check(load().mla_plan_create(ctypes.byref(d), arr, len(lens), n_workers, ctypes.byref(h)),
           "mla_plan_create")
    return Plan(h, len(lens))


def mla_plan_create_multi(d, host_lens, q_len, n_workers=0):
    lens = [int(x) for x in host_lens]
    arr = (ctypes.c_int32 * len(lens))(*lens)
    h = ctypes.c_void_p()
    _check(load().mla_plan_create_multi(ctypes.byref(d), arr, len(lens), q_len, n_workers, ctypes.byref(h)),
           "mla_plan_create_multi")
    return Plan(h, len(lens))


def mla_append_workspace_bytes(d, batch, n_new):
    return load().mla_append_workspace_bytes(ctypes.byref(d), batch, n_new)


def mla_decode_workspace_bytes(d, plan):
    return load().mla_decode_workspace_bytes(ctypes.byref(d), plan.handle)


def mla_workspace_bytes(d, plan):
    return load().mla_workspace_bytes(ctypes.byref(d), plan.handle)


def mla_append(d, c, h, n_new, w_dkv, w_kr, act_w_dtype, ws, stream=None):
    _check(load().mla_append(ctypes.byref(d), ctypes.byref(c), _ptr(h), n_new, _ptr(w_dkv),
                             _ptr(w_kr), act_w_dtype, _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "mla_append")


def mla_decode(d, c, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws, stream=None):
    _check(load().mla_decode(ctypes.byref(d), ctypes.byref(c), plan.handle, _ptr(q_nope),
                             _ptr(q_rope), _ptr(q_pos), _ptr(w_uk), _ptr(w_uv), q_w_dtype, _ptr(o),
                             o_dtype, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "mla_decode")


def mla_decode_multi_workspace_bytes(d, plan, q_len):
    return load().mla_decode_multi_workspace_bytes(ctypes.byref(d), plan.handle, q_len)


def mla_decode_multi(d, c, plan, q_len, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws, stream=None):
    _check(load().mla_decode_multi(ctypes.byref(d), ctypes.byref(c), plan.handle, q_len, _ptr(q_nope),
                                   _ptr(q_rope), _ptr(q_pos), _ptr(w_uk), _ptr(w_uv), q_w_dtype, _ptr(o),
                                   o_dtype, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "mla_decode_multi")


def mla_decode_noalloc(d, c, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, dev_status=None,
                       stream=None):
    _check(load().mla_decode_noalloc(ctypes.byref(d), ctypes.byref(c), plan.handle, _ptr(q_nope), _ptr(q_rope),
                                     _ptr(q_pos), _ptr(w_uk), _ptr(w_uv), q_w_dtype, _ptr(o), o_dtype,
                                     _ptr(dev_status), _stream(stream)), "mla_decode_noalloc")


def mla_merge_query_weight(d, d_x, w_q, w_uk, w_dtype, a, stream=None):
    _check(load().mla_merge_query_weight(ctypes.byref(d), d_x, _ptr(w_q), _ptr(w_uk), w_dtype, _ptr(a),
                                         _stream(stream)), "mla_merge_query_weight")


def mla_merge_output_weight(d, d_out, w_o, w_uv, w_dtype, bm, stream=None):
    _check(load().mla_merge_output_weight(ctypes.byref(d), d_out, _ptr(w_o), _ptr(w_uv), w_dtype, _ptr(bm),
                                          _stream(stream)), "mla_merge_output_weight")


def mla_decode_merged_workspace_bytes(d, plan, d_out):
    return load().mla_decode_merged_workspace_bytes(ctypes.byref(d), plan.handle, d_out)


def mla_decode_merged(d, c, plan, d_x, x, q_rope, q_pos, a, d_out, bm, w_dtype, y, y_dtype, ws, stream=None):
    _check(load().mla_decode_merged(ctypes.byref(d), ctypes.byref(c), plan.handle, d_x, _ptr(x), _ptr(q_rope),
                                    _ptr(q_pos), _ptr(a), d_out, _ptr(bm), w_dtype, _ptr(y), y_dtype, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)), "mla_decode_merged")


def mla_append_decode(d, c, plan, h, n_new, w_dkv, w_kr, q_nope, q_rope, q_pos, w_uk, w_uv,
                      act_w_dtype, o, o_dtype, ws, stream=None):
    _check(load().mla_append_decode(ctypes.byref(d), ctypes.byref(c), plan.handle, _ptr(h), n_new,
                                    _ptr(w_dkv), _ptr(w_kr), _ptr(q_nope), _ptr(q_rope), _ptr(q_pos),
                                    _ptr(w_uk), _ptr(w_uv), act_w_dtype, _ptr(o), o_dtype, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)),
           "mla_append_decode")


def mla_workspace_init(ws, stream=None):
    _check(load().mla_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "mla_workspace_init")


def mla_device_error(ws, reset=True, stream=None):
    code = ctypes.c_int32()
    _check(load().mla_device_error(_ptr(ws), _stream(stream), ctypes.byref(code), int(reset)),
           "mla_device_error")
    return code.value


def mla_status_str(s):
    return load().mla_status_str(s).decode()


def mla_abi_version():
    return load().mla_abi_version()


def mla_prof_begin(max_records=100000):
    _check(load().mla_prof_begin(max_records), "mla_prof_begin")


def mla_prof_end():
    """Returns {kernel name: (total ms, launches)} for kernels that ran."""
    lib = load()
    n = lib.mla_prof_num_kernels()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib.mla_prof_end(ms, cnt, n), "mla_prof_end")
    return {lib.mla_prof_kernel_name(k).decode(): (ms[k], cnt[k]) for k in range(n) if cnt[k]}


def mla_calib_copy(dst, src, n_bytes, stream=None):
    _check(load().mla_calib_copy(_ptr(dst), _ptr(src), n_bytes, _stream(stream)), "mla_calib_copy")


def mla_calib_read(src, n_bytes, sink, stream=None):
    _check(load().mla_calib_read(_ptr(src), n_bytes, _ptr(sink), _stream(stream)), "mla_calib_read")


# ------------------------------------------------------------------ tensor-level calls
# The same entry points with the dtype codes read off the tensors, the output
# (and, if not given, a workspace) allocated with torch on the inputs' device.
# Nothing is computed here.

def _code(t, what):
    import torch
    codes = {torch.float32: F32, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise ValueError(f"{what}: dtype {t.dtype} is not float32 or bfloat16")
    return codes[t.dtype]


def _expect(t, what, shape, dtype=None):
    """t must have exactly `shape` (and `dtype` if given)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype} (one dtype for activations and weights)")


def _check_decode_args(d, plan, q_nope, q_rope, w_uk, w_uv, q_len=1):
    B, H = plan.batch, d.n_heads
    lead = (B, H) if q_len == 1 else (B, q_len, H)
    _code(q_nope, "q_nope")
    _expect(q_nope, "q_nope", lead + (d.d_nope,))
    _expect(q_rope, "q_rope", lead + (d.d_rope,), q_nope.dtype)
    _expect(w_uk, "w_uk", (H, d.d_nope, d.d_c), q_nope.dtype)
    _expect(w_uv, "w_uv", (H, d.d_v, d.d_c), q_nope.dtype)


def _check_append_args(d, c, h, w_dkv, w_kr):
    _code(h, "h")
    if h.dim() != 3 or h.shape[0] != c.batch or h.shape[2] != d.d_model:
        raise ValueError(f"h: shape {tuple(h.shape)}, expected ({c.batch}, n_new, {d.d_model})")
    _expect(w_dkv, "w_dkv", (d.d_c, d.d_model), h.dtype)
    _expect(w_kr, "w_kr", (d.d_rope, d.d_model), h.dtype)


def _temp_ws_stream(stream):
    """A workspace the call allocates itself is freed on return; with an
    explicit stream its kernels may still be queued there, so that case
    needs a caller-owned workspace."""
    if stream is not None:
        raise ValueError("pass ws (a workspace the caller keeps alive) when giving an explicit stream")


def workspace(d, plan, device=None):
    """A fresh workspace of mla_workspace_bytes(d, plan) bytes, status word cleared."""
    import torch
    ws = torch.empty(mla_workspace_bytes(d, plan), dtype=torch.uint8, device=device or "cuda")
    mla_workspace_init(ws)
    return ws


def decode(d, c, plan, q_nope, q_rope, w_uk, w_uv, out=None, q_pos=None, ws=None, stream=None):
    """mla_decode on tensors: returns out ([B, H, d_v], float32 unless given).
    q_nope, q_rope, w_uk and w_uv share one dtype (float32 or bfloat16)."""
    import torch
    _check_decode_args(d, plan, q_nope, q_rope, w_uk, w_uv)
    qw = _code(q_nope, "q_nope")
    if out is None:
        out = torch.empty((plan.batch, d.n_heads, d.d_v), dtype=torch.float32, device=q_nope.device)
    _expect(out, "out", (plan.batch, d.n_heads, d.d_v))
    if q_pos is not None:
        _expect(q_pos, "q_pos", (plan.batch,), torch.int32)
    if ws is None:
        _temp_ws_stream(stream)
        ws = workspace(d, plan, q_nope.device)
    mla_decode(d, c, plan, q_nope, q_rope, q_pos, w_uk, w_uv, qw, out, _code(out, "out"), ws, stream)
    return out


def append(d, c, h, w_dkv, w_kr, ws=None, stream=None):
    """mla_append on tensors: h is [B, n_new, d_model]; h, w_dkv and w_kr share
    one dtype."""
    import torch
    _check_append_args(d, c, h, w_dkv, w_kr)
    n_new = h.shape[1]
    if ws is None:
        _temp_ws_stream(stream)
        ws = torch.empty(mla_append_workspace_bytes(d, h.shape[0], n_new), dtype=torch.uint8, device=h.device)
        mla_workspace_init(ws)
    mla_append(d, c, h, n_new, w_dkv, w_kr, _code(h, "h"), ws, stream)


def append_decode(d, c, plan, h, w_dkv, w_kr, q_nope, q_rope, w_uk, w_uv, out=None, q_pos=None, ws=None,
                  stream=None):
    """mla_append_decode on tensors (the plan holds the lengths after the
    append); every activation and weight shares h's dtype."""
    import torch
    _check_append_args(d, c, h, w_dkv, w_kr)
    _check_decode_args(d, plan, q_nope, q_rope, w_uk, w_uv)
    if q_nope.dtype != h.dtype:
        raise ValueError(f"q_nope: dtype {q_nope.dtype}, expected {h.dtype} (one dtype for activations and weights)")
    n_new = h.shape[1]
    if out is None:
        out = torch.empty((plan.batch, d.n_heads, d.d_v), dtype=torch.float32, device=q_nope.device)
    _expect(out, "out", (plan.batch, d.n_heads, d.d_v))
    if q_pos is not None:
        _expect(q_pos, "q_pos", (plan.batch,), torch.int32)
    if ws is None:
        _temp_ws_stream(stream)
        need = max(mla_workspace_bytes(d, plan), mla_append_workspace_bytes(d, h.shape[0], n_new))
        ws = torch.empty(need, dtype=torch.uint8, device=q_nope.device)
        mla_workspace_init(ws)
    mla_append_decode(d, c, plan, h, n_new, w_dkv, w_kr, q_nope, q_rope, q_pos, w_uk, w_uv, _code(h, "h"), out,
                      _code(out, "out"), ws, stream)
    return out

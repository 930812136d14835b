"""ctypes binding of libpsa.so (argument marshalling only).

Every computation runs in the HIP library; this module converts numpy page
tables and torch tensors into the plain pointers and sizes the C ABI
(include/psa.h) takes.  It raises ``PsaError`` for any non-OK status and
``OSError`` when the library has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpsa.so")

PSA_BF16, PSA_F32 = 0, 1
PREFIX_ONLY, DISTINCT_ONLY, FORCE_MATVEC, DEBUG_POISON, NO_XCD_ORDER, NO_TILE_PAIRS = 0x1, 0x2, 0x4, 0x8, 0x10, 0x20
NO_PAGE_SHARING = 0x40
STATUS = {0: "PSA_OK", 1: "PSA_ERR_INVALID_ARGUMENT", 2: "PSA_ERR_UNSUPPORTED", 3: "PSA_ERR_OUT_OF_RANGE",
          4: "PSA_ERR_WORKSPACE_TOO_SMALL", 5: "PSA_ERR_HIP", 6: "PSA_ERR_ALLOC"}

# every symbol include/psa.h and include/psa_debug.h declare
EXPORTS = ["psa_build_plan", "psa_plan_get_info", "psa_plan_upload", "psa_decode_attention", "psa_merge",
           "psa_flatten_prefix_tree", "psa_batch_owned_view", "psa_free_batch", "psa_destroy_plan",
           "psa_last_error", "psa_version", "psa_plan_debug_items", "psa_plan_debug_queries",
           "psa_decode_attention_traced", "psa_debug_read_peak", "psa_debug_mfma_peak", "psa_debug_issue_probe",
           "psa_identify_prefix_groups", "psa_prefix_groups_view", "psa_free_prefix_groups",
           "psa_decode_attention_noalloc", "psa_plan_debug_members"]


class PsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        self.message = message


class psa_config(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("num_pages", C.c_int32), ("kv_dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("sm_scale", C.c_float)]


_I32P = C.POINTER(C.c_int32)
_I64P = C.POINTER(C.c_int64)


class psa_batch(C.Structure):
    _fields_ = [("num_groups", C.c_int32), ("group_prefix_len", _I32P), ("group_page_off", _I64P),
                ("group_pages", _I32P), ("num_queries", C.c_int32), ("query_group", _I32P),
                ("query_distinct_len", _I32P), ("query_page_off", _I64P), ("query_pages", _I32P),
                ("query_prefix_len", _I32P)]


class psa_plan_opts(C.Structure):
    _fields_ = [("flags", C.c_uint32), ("prefix_chunk_tokens", C.c_int32), ("distinct_chunk_tokens", C.c_int32),
                ("mfma_min_rows", C.c_int32), ("mfma_tile_rows", C.c_int32)]


class psa_plan_info(C.Structure):
    _fields_ = [("workspace_bytes", C.c_size_t), ("num_items", C.c_int64), ("num_prefix_items", C.c_int64),
                ("num_matvec_items", C.c_int64), ("num_partial_slots", C.c_int64), ("logical_tokens", C.c_int64),
                ("processed_tokens", C.c_int64), ("saved_tokens", C.c_int64), ("algorithmic_bytes", C.c_double),
                ("algorithmic_flops", C.c_double), ("prefix_flops", C.c_double), ("prefix_kv_bytes", C.c_double),
                ("distinct_kv_bytes", C.c_double), ("image_bytes", C.c_size_t), ("unique_kv_bytes", C.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class psa_tree(C.Structure):
    _fields_ = [("num_nodes", C.c_int32), ("node_parent", _I32P), ("node_len", _I32P), ("node_page_off", _I64P),
                ("node_pages", _I32P), ("num_queries", C.c_int32), ("query_node", _I32P),
                ("query_distinct_len", _I32P), ("query_page_off", _I64P), ("query_pages", _I32P)]


_lib = None


def lib():
    """The loaded library; raises OSError if it is missing (build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} not found: build it with `python -m prefix_shared_decode_amd.build`")
        # torch brings its own HIP runtime (same soname, libamdhip64.so.7).
        # Loading it first makes the library bind to that runtime; loaded the
        # other way round, the process holds two HIP and two HSA runtimes and
        # the library's finds no device once torch has opened it.
        import torch  # noqa: F401

        L = C.CDLL(LIB_PATH)
        vp = C.c_void_p
        L.psa_build_plan.argtypes = [C.POINTER(psa_config), C.POINTER(psa_batch), C.POINTER(psa_plan_opts),
                                     C.POINTER(vp)]
        L.psa_plan_get_info.argtypes = [vp, C.POINTER(psa_plan_info)]
        L.psa_plan_upload.argtypes = [vp, vp, C.c_size_t, vp]
        L.psa_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.psa_decode_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.psa_merge.argtypes = [C.c_int64, C.c_int32] + [vp] * 9 + [vp]
        L.psa_flatten_prefix_tree.argtypes = [C.POINTER(psa_tree), C.c_int32, C.POINTER(vp)]
        L.psa_batch_owned_view.argtypes = [vp, C.POINTER(psa_batch), _I64P]
        L.psa_free_batch.argtypes = [vp]
        L.psa_free_batch.restype = None
        L.psa_identify_prefix_groups.argtypes = [C.c_int32, _I64P, _I32P, C.POINTER(vp)]
        L.psa_prefix_groups_view.argtypes = [vp, C.POINTER(C.c_int32), C.POINTER(_I32P), C.POINTER(_I32P),
                                             C.POINTER(_I32P), C.POINTER(C.c_int64)]
        L.psa_free_prefix_groups.argtypes = [vp]
        L.psa_free_prefix_groups.restype = None
        L.psa_destroy_plan.argtypes = [vp]
        L.psa_destroy_plan.restype = None
        L.psa_last_error.restype = C.c_char_p
        L.psa_version.restype = C.c_int32
        L.psa_plan_debug_items.argtypes = [vp, _I32P, C.c_int64]
        L.psa_plan_debug_queries.argtypes = [vp, _I32P, _I32P, C.c_int64]
        L.psa_plan_debug_members.argtypes = [vp, _I32P, C.c_int64, _I64P]
        L.psa_decode_attention_traced.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, C.c_size_t, vp, C.c_int64, vp]
        L.psa_debug_read_peak.argtypes = [vp, C.c_size_t, vp, C.c_int64, vp]
        L.psa_debug_mfma_peak.argtypes = [vp, C.c_int64, C.c_int32, vp]
        L.psa_debug_issue_probe.argtypes = [C.c_int32, vp, C.c_int64, C.c_int32, vp]
        for name in EXPORTS:
            fn = getattr(L, name)
            if fn.restype is C.c_int and name not in ("psa_version",):
                fn.restype = C.c_int
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise PsaError(status, lib().psa_last_error().decode(errors="replace"))


def _arr(x, dtype):
    a = np.ascontiguousarray(np.asarray(x, dtype=dtype))
    return a


def _ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype)) if a.size else C.cast(None, C.POINTER(ctype))


class _Keep:
    """Keeps numpy arrays alive while a C struct points at them."""

    def __init__(self):
        self.arrays = []

    def __call__(self, x, dtype, ctype):
        a = _arr(x, dtype)
        if a.size == 0:
            a = np.zeros(1, dtype=dtype)
        self.arrays.append(a)
        return a.ctypes.data_as(C.POINTER(ctype))


def make_config(num_q_heads, num_kv_heads, head_dim, num_pages, kv_dtype="bf16", out_dtype="f32",
                page_size=16, sm_scale=0.0):
    dt = {"bf16": PSA_BF16, "f32": PSA_F32}
    return psa_config(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, dt[kv_dtype], dt[out_dtype],
                      float(sm_scale))


def _batch_struct(batch, keep):
    G = len(batch["group_prefix_len"])
    N = len(batch["query_group"])
    return psa_batch(G, keep(batch["group_prefix_len"], np.int32, C.c_int32),
                     keep(batch["group_page_off"] if G else [0], np.int64, C.c_int64),
                     keep(batch["group_pages"], np.int32, C.c_int32), N,
                     keep(batch["query_group"], np.int32, C.c_int32),
                     keep(batch["query_distinct_len"], np.int32, C.c_int32),
                     keep(batch["query_page_off"] if N else [0], np.int64, C.c_int64),
                     keep(batch["query_pages"], np.int32, C.c_int32),
                     keep(batch["query_prefix_len"], np.int32, C.c_int32)
                     if batch.get("query_prefix_len") is not None else None)


class Plan:
    """Owner of a psa_plan* (destroyed with the object)."""

    def __init__(self, handle, cfg):
        self.handle = handle
        self.cfg = cfg

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.psa_destroy_plan(h)

    def info(self):
        return psa_plan_get_info(self)

    def items(self):
        """Work list as an [num_units * 4, 8] int32 array (psa_debug.h)."""
        n = 4 * self.info()["num_items"]
        out = np.zeros((max(n, 1), 8), dtype=np.int32)
        _check(lib().psa_plan_debug_items(self.handle, out.ctypes.data_as(_I32P), n))
        return out[:n]

    def members(self):
        """The member array MFMA tile rows index (psa_debug.h)."""
        cnt = np.zeros(1, dtype=np.int64)
        n = self.num_queries  # a query is a member of at most one group
        out = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib().psa_plan_debug_members(self.handle, out.ctypes.data_as(_I32P), n, cnt.ctypes.data_as(_I64P)))
        return out[:int(cnt[0])]

    def queries(self):
        """(expected partials, first slot) per query (psa_debug.h)."""
        n = self.num_queries
        e = np.zeros(max(n, 1), dtype=np.int32)
        s = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib().psa_plan_debug_queries(self.handle, e.ctypes.data_as(_I32P), s.ctypes.data_as(_I32P), n))
        return e[:n], s[:n]


def psa_build_plan(cfg, batch, flags=0, prefix_chunk_tokens=0, distinct_chunk_tokens=0, mfma_min_rows=0,
                   mfma_tile_rows=0):
    """Plan for ``batch`` (dict of page-table arrays, see include/psa.h)."""
    keep = _Keep()
    b = _batch_struct(batch, keep)
    opts = psa_plan_opts(flags, prefix_chunk_tokens, distinct_chunk_tokens, mfma_min_rows, mfma_tile_rows)
    h = C.c_void_p()
    _check(lib().psa_build_plan(C.byref(cfg), C.byref(b), C.byref(opts), C.byref(h)))
    plan = Plan(h.value, cfg)
    plan.num_queries = len(batch["query_group"])
    return plan


def psa_plan_get_info(plan):
    info = psa_plan_info()
    _check(lib().psa_plan_get_info(plan.handle, C.byref(info)))
    return info.as_dict()


def _stream_ptr(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ptr(t, name):
    if t is None:
        return None
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def psa_plan_upload(plan, workspace, stream=None):
    _check(lib().psa_plan_upload(plan.handle, _dev_ptr(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream_ptr(stream)))


def _check_io(plan, q, k_pool, v_pool, out, out_m, out_l):
    import torch

    cfg = plan.cfg
    kvt = torch.bfloat16 if cfg.kv_dtype == PSA_BF16 else torch.float32
    ot = torch.bfloat16 if cfg.out_dtype == PSA_BF16 else torch.float32
    n = plan.num_queries
    want_q = (n, cfg.num_q_heads, cfg.head_dim)
    want_p = (cfg.num_pages, cfg.num_kv_heads, cfg.page_size, cfg.head_dim)
    for name, t, shape, dt in (("q", q, want_q, kvt), ("k_pool", k_pool, want_p, kvt), ("v_pool", v_pool, want_p, kvt),
                               ("out", out, want_q, ot)):
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"{name}: expected {shape} {dt}, got {tuple(t.shape)} {t.dtype}")
    for name, t in (("out_m", out_m), ("out_l", out_l)):
        if t is not None and (tuple(t.shape) != (n, cfg.num_q_heads) or t.dtype != torch.float32):
            raise ValueError(f"{name}: expected {(n, cfg.num_q_heads)} float32")


def psa_decode_attention(plan, q, k_pool, v_pool, out, workspace, out_m=None, out_l=None, stream=None, trace=None):
    """One fused decode launch; shapes/dtypes are checked against the plan's config.

    trace: optional int64 device tensor of >= 4 * num_items entries; the launch
    then records per-unit timing (include/psa_debug.h psa_decode_attention_traced).
    """
    import torch

    _check_io(plan, q, k_pool, v_pool, out, out_m, out_l)
    args = (plan.handle, _dev_ptr(q, "q"), _dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"),
            _dev_ptr(out, "out"), _dev_ptr(out_m, "out_m"), _dev_ptr(out_l, "out_l"),
            _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size())
    if trace is None:
        _check(lib().psa_decode_attention(*args, _stream_ptr(stream)))
    else:
        if trace.dtype != torch.int64:
            raise ValueError("trace: expected an int64 tensor")
        _check(lib().psa_decode_attention_traced(*args, _dev_ptr(trace, "trace"), trace.numel(), _stream_ptr(stream)))


def psa_decode_attention_noalloc(plan, q, k_pool, v_pool, out, image, out_m=None, out_l=None, stream=None):
    """psa_decode_attention with the library's static scratch (allocates nothing);
    ``image`` is a device buffer into which psa_plan_upload copied this plan."""
    _check_io(plan, q, k_pool, v_pool, out, out_m, out_l)
    _check(lib().psa_decode_attention_noalloc(
        plan.handle, _dev_ptr(q, "q"), _dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"), _dev_ptr(out, "out"),
        _dev_ptr(out_m, "out_m"), _dev_ptr(out_l, "out_l"), _dev_ptr(image, "image"),
        image.numel() * image.element_size(), _stream_ptr(stream)))


def psa_debug_read_peak(buf, sink, stream=None):
    """One streaming read of device tensor ``buf`` (include/psa_debug.h); ``sink``
    is a uint32/int32 device tensor of >= 2048 * 256 entries."""
    _check(lib().psa_debug_read_peak(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(), _dev_ptr(sink, "sink"),
                                     sink.numel(), _stream_ptr(stream)))


def psa_debug_mfma_peak(out, iters, stream=None):
    """One launch of dependent bf16 MFMA chains (include/psa_debug.h); ``out`` is a
    float32 device tensor of >= 2048 * 256 entries.  Returns the flops it does."""
    _check(lib().psa_debug_mfma_peak(_dev_ptr(out, "out"), out.numel(), int(iters), _stream_ptr(stream)))
    return 2048.0 * 4 * iters * 16384


# instructions per iteration of each issue-probe pattern (include/psa_debug.h)
ISSUE_PATTERNS = {0: ("mfma, 16 chains", 16), 1: ("mfma, 8 chains", 16), 2: ("mfma, 4 chains", 16),
                  3: ("mfma, 2 chains", 16), 4: ("mfma, 1 chain", 16), 5: ("v_fma_f32", 16), 6: ("v_exp_f32", 8),
                  7: ("mfma (8 chains) + 2 fma + 1/2 exp", 16)}


def psa_debug_issue_probe(pattern, cycles, iters, stream=None):
    """One launch of an issue-rate pattern (include/psa_debug.h); ``cycles`` is an
    int64 device tensor of >= 1024 entries."""
    _check(lib().psa_debug_issue_probe(int(pattern), _dev_ptr(cycles, "cycles"), cycles.numel(), int(iters),
                                       _stream_ptr(stream)))


def psa_merge(o_a, m_a, l_a, o_b, m_b, l_b, o, m, l, stream=None):
    """Eq. 1 merge of two partial sets; o_* are [rows, head_dim] fp32, m_*/l_* [rows]."""
    rows, d = o_a.shape[0], o_a.shape[-1]
    rows = int(o_a.numel() // d)
    _check(lib().psa_merge(rows, d, *[_dev_ptr(t, "merge operand") for t in (o_a, m_a, l_a, o_b, m_b, l_b, o, m, l)],
                           _stream_ptr(stream)))


def psa_flatten_prefix_tree(tree, page_size=16):
    """Flatten a tree (dict of arrays, include/psa.h psa_tree) to a batch dict + saved tokens."""
    keep = _Keep()
    M = len(tree["node_parent"])
    N = len(tree["query_node"])
    t = psa_tree(M, keep(tree["node_parent"], np.int32, C.c_int32), keep(tree["node_len"], np.int32, C.c_int32),
                 keep(tree["node_page_off"] if M else [0], np.int64, C.c_int64),
                 keep(tree["node_pages"], np.int32, C.c_int32), N, keep(tree["query_node"], np.int32, C.c_int32),
                 keep(tree["query_distinct_len"], np.int32, C.c_int32),
                 keep(tree["query_page_off"] if N else [0], np.int64, C.c_int64),
                 keep(tree["query_pages"], np.int32, C.c_int32))
    h = C.c_void_p()
    _check(lib().psa_flatten_prefix_tree(C.byref(t), page_size, C.byref(h)))
    try:
        v = psa_batch()
        saved = C.c_int64()
        _check(lib().psa_batch_owned_view(h, C.byref(v), C.byref(saved)))

        def grab(ptr, n, dtype):
            if n == 0:
                return np.zeros(0, dtype=dtype)
            return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)

        G, NQ = v.num_groups, v.num_queries
        goff = grab(v.group_page_off, G + 1, np.int64)
        qoff = grab(v.query_page_off, NQ + 1, np.int64)
        batch = {
            "page_size": page_size,
            "group_prefix_len": grab(v.group_prefix_len, G, np.int32),
            "group_page_off": goff if G else np.zeros(1, np.int64),
            "group_pages": grab(v.group_pages, int(goff[-1]) if G else 0, np.int32),
            "query_group": grab(v.query_group, NQ, np.int32),
            "query_distinct_len": grab(v.query_distinct_len, NQ, np.int32),
            "query_page_off": qoff if NQ else np.zeros(1, np.int64),
            "query_pages": grab(v.query_pages, int(qoff[-1]) if NQ else 0, np.int32),
        }
        return batch, int(saved.value)
    finally:
        lib().psa_free_batch(h)


def psa_identify_prefix_groups(requests):
    """Prefix-sharing groups of token sequences (include/psa.h): returns a dict
    with group_prefix_len, group_first_request, request_group (numpy int32)
    and saved_tokens."""
    lens = [len(r) for r in requests]
    off = np.zeros(len(requests) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens) if lens else []
    toks = np.concatenate([np.asarray(r, dtype=np.int32) for r in requests]) if sum(lens) else np.zeros(1, np.int32)
    toks = np.ascontiguousarray(toks, dtype=np.int32)
    h = C.c_void_p()
    _check(lib().psa_identify_prefix_groups(len(requests), off.ctypes.data_as(_I64P), toks.ctypes.data_as(_I32P),
                                            C.byref(h)))
    try:
        ng = C.c_int32()
        gl, gf, rg = _I32P(), _I32P(), _I32P()
        saved = C.c_int64()
        _check(lib().psa_prefix_groups_view(h, C.byref(ng), C.byref(gl), C.byref(gf), C.byref(rg), C.byref(saved)))

        def grab(ptr, n):
            return np.ctypeslib.as_array(ptr, shape=(n,)).astype(np.int32, copy=True) if n else np.zeros(0, np.int32)

        return {"group_prefix_len": grab(gl, ng.value), "group_first_request": grab(gf, ng.value),
                "request_group": grab(rg, len(requests)), "saved_tokens": int(saved.value)}
    finally:
        lib().psa_free_prefix_groups(h)

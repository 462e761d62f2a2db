"""Python binding of libtreeattn (prefix-tree attention on MI355X).

Argument marshalling only: every step of the computation runs in the C++
host code or the HIP kernels of libtreeattn.so.  torch supplies device memory
and the current stream.  If the library is not built it is built once (hipcc);
if it still cannot be loaded, importing the binding fails -- there is no
fallback implementation.

Names follow the C ABI in include/tt.h: tree_build / tree_info / tree_export /
tree_plan_upload, tree_attn_fwd, tree_attn_bwd, tree_weighted_nll.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# TT_LIB_PATH selects another build of the same library (e.g. an instrumented one)
LIB_PATH = os.environ.get("TT_LIB_PATH") or os.path.join(_PKG, "libtreeattn.so")

TT_OK, TT_EINVAL, TT_ENOMEM, TT_EWORKSPACE, TT_EUNSUPPORTED, TT_EDEVICE, TT_EOVERFLOW = 0, -1, -2, -3, -4, -5, -6
TT_F32, TT_BF16 = 0, 1
TT_ACCUMULATE_DKDV = 1
TT_BWD_REUSE_ROTATED = 2
TT_ALLOW_GENERIC = 1

EXPORTED = ("tree_build", "tree_free", "tree_info", "tree_export", "tree_plan_bytes", "tree_plan_upload",
            "tree_plan_copy",
            "tree_attn_workspace_bytes", "tree_attn_fwd", "tree_attn_bwd", "tree_nll_workspace_bytes",
            "tree_weighted_nll", "tt_last_error", "tt_timing_enable", "tt_timing_collect",
            "tree_target_weights", "tree_path_build", "tree_path_free", "tree_path_info", "tree_path_segments",
            "tree_path_plan_bytes", "tree_path_plan_upload", "tree_path_workspace_bytes", "tree_attn_path",
            "tt_probe_mfma", "tree_weighted_nll_noalloc")


class TTError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libtreeattn error {code}: {msg}")
        self.code = code


_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)


class TreeInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_nodes", "n_seqs", "n_roots", "n_leaves", "max_depth", "seq_tokens", "leaf_tokens", "n_targets",
        "pairs", "dense_pairs", "block_q", "block_k", "n_tiles", "n_full_tiles")]


class TreeArrays(ctypes.Structure):
    _fields_ = [("token", _i32p), ("depth", _i32p), ("end", _i32p), ("parent", _i32p), ("n_pass", _i32p),
                ("weight", _f32p), ("seq_pos_to_dfs", _i32p), ("tgt_row_ptr", _i32p), ("tgt_dfs", _i32p),
                ("tgt_token", _i32p), ("tgt_w", _f32p)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("tree", ctypes.c_void_p), ("plan", ctypes.c_void_p),
                ("q_off", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
                ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("scale", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint32)]


class AttnBwdArgs(ctypes.Structure):
    _fields_ = [("a", AttnArgs), ("d_o", ctypes.c_void_p), ("d_q", ctypes.c_void_p),
                ("d_k", ctypes.c_void_p), ("d_v", ctypes.c_void_p), ("flags", ctypes.c_uint32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("max_ms", ctypes.c_double)]


class NllArgs(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("d_model", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_tgt", ctypes.c_int32),
                ("hidden", ctypes.c_void_p), ("w_vocab", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("logits_dtype", ctypes.c_int),
                ("tgt_row_ptr", ctypes.c_void_p), ("tgt_id", ctypes.c_void_p), ("tgt_w", ctypes.c_void_p),
                ("loss", ctypes.c_void_p), ("logp", ctypes.c_void_p),
                ("d_hidden", ctypes.c_void_p), ("d_w_vocab", ctypes.c_void_p), ("dw_dtype", ctypes.c_int),
                ("d_logits", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


_LIB = None


class PathInfo(ctypes.Structure):
    _fields_ = [("n_segments", ctypes.c_int32), ("max_path", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("order", ctypes.c_int32), ("fwd_calls", ctypes.c_int64), ("bwd_calls", ctypes.c_int64),
                ("pad_rows", ctypes.c_int64), ("query_rows", ctypes.c_int64), ("pad_pairs", ctypes.c_int64)]


class PathArgs(ctypes.Structure):
    _fields_ = [("path", ctypes.c_void_p), ("plan", ctypes.c_void_p), ("h_q", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("d_o", ctypes.c_void_p), ("d_q", ctypes.c_void_p),
                ("d_k", ctypes.c_void_p), ("d_v", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32)]


def _setup(lib):
    lib.tree_build.argtypes = [_i32p, _i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                ctypes.POINTER(ctypes.c_void_p)]
    lib.tree_build.restype = ctypes.c_int
    lib.tree_free.argtypes = [ctypes.c_void_p]
    lib.tree_free.restype = None
    lib.tree_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(TreeInfo)]
    lib.tree_export.argtypes = [ctypes.c_void_p, ctypes.POINTER(TreeArrays)]
    lib.tree_plan_bytes.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    lib.tree_plan_upload.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.tree_plan_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    lib.tree_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.tree_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.tree_attn_bwd.argtypes = [ctypes.POINTER(AttnBwdArgs), ctypes.c_void_p]
    lib.tree_nll_workspace_bytes.argtypes = [ctypes.POINTER(NllArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.tree_weighted_nll.argtypes = [ctypes.POINTER(NllArgs), ctypes.c_void_p]
    lib.tree_weighted_nll_noalloc.argtypes = [ctypes.POINTER(NllArgs), ctypes.c_void_p]
    lib.tree_target_weights.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_float)]
    lib.tree_path_build.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    lib.tree_path_free.argtypes = [ctypes.c_void_p]
    lib.tree_path_free.restype = None
    lib.tree_path_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(PathInfo)]
    lib.tree_path_segments.argtypes = [ctypes.c_void_p] + [_i32p] * 5
    lib.tree_path_plan_bytes.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    lib.tree_path_plan_upload.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.tree_path_workspace_bytes.argtypes = [ctypes.POINTER(PathArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.tree_attn_path.argtypes = [ctypes.POINTER(PathArgs), ctypes.c_void_p]
    lib.tt_last_error.restype = ctypes.c_char_p
    lib.tt_timing_enable.argtypes = [ctypes.c_int]
    lib.tt_timing_enable.restype = ctypes.c_int
    lib.tt_timing_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.tt_timing_collect.restype = ctypes.c_int
    lib.tt_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_double)]
    lib.tt_probe_mfma.restype = ctypes.c_int
    for _n in ("tree_info", "tree_export", "tree_plan_bytes", "tree_plan_upload", "tree_plan_copy", "tree_attn_workspace_bytes",
               "tree_attn_fwd", "tree_attn_bwd", "tree_nll_workspace_bytes", "tree_weighted_nll",
               "tree_path_plan_bytes", "tree_path_plan_upload", "tree_path_workspace_bytes", "tree_attn_path",
               "tree_weighted_nll_noalloc"):
        getattr(lib, _n).restype = ctypes.c_int


def lib():
    """The loaded libtreeattn (built once with hipcc if it is missing; raises if it cannot be loaded)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib_ = ctypes.CDLL(LIB_PATH)
        _setup(lib_)
        _LIB = lib_
    return _LIB


def _check(rc):
    if rc != TT_OK:
        raise TTError(rc, lib().tt_last_error().decode())


def last_error():
    return lib().tt_last_error().decode()


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


# ------------------------------------------------------------------ kernel timing
def timing_enable(on=True):
    """Bracket every kernel the library launches (this thread) with HIP events."""
    _check(lib().tt_timing_enable(1 if on else 0))


def timing_collect():
    """{kernel name: (launches, total_ms, max_ms)} since the last collect; waits for the events."""
    buf = (KernelTime * 64)()
    n = ctypes.c_int()
    _check(lib().tt_timing_collect(buf, 64, ctypes.byref(n)))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms), float(buf[i].max_ms))
            for i in range(min(n.value, 64))}


def probe_mfma(n_blocks=1024, iters=2000, reps=3):
    """Sustained dense bf16 MFMA rate (TFLOP/s) of tt_probe_mfma on the current
    stream: one warm-up launch, then the best of `reps` timed launches."""
    import torch
    out = torch.empty(n_blocks * 512, dtype=torch.float32, device="cuda")
    fl = ctypes.c_double()
    best = None
    for r in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(lib().tt_probe_mfma(n_blocks, iters, ctypes.c_void_p(out.data_ptr()), _stream(), ctypes.byref(fl)))
        e1.record()
        e1.synchronize()
        if r:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    return fl.value / (best * 1e-3) / 1e12


# ------------------------------------------------------------------ tree
class Tree:
    """Host prefix tree (library-owned); see tree_build in include/tt.h."""

    def __init__(self, seqs=None, tokens=None, offsets=None, block_q=0, block_k=0):
        if seqs is not None:
            offsets = np.zeros(len(seqs) + 1, dtype=np.int64)
            for i, s in enumerate(seqs):
                offsets[i + 1] = offsets[i] + len(s)
            tokens = (np.concatenate([np.asarray(s, dtype=np.int32) for s in seqs])
                      if len(seqs) else np.zeros(0, dtype=np.int32))
        self._tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        self._offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        self.handle = ctypes.c_void_p()
        n_seqs = len(self._offsets) - 1
        _check(lib().tree_build(_ptr(self._tokens, ctypes.c_int32), _ptr(self._offsets, ctypes.c_int64),
                               n_seqs, block_q, block_k, ctypes.byref(self.handle)))
        inf = TreeInfo()
        _check(lib().tree_info(self.handle, ctypes.byref(inf)))
        self.info = {n: int(getattr(inf, n)) for n, _ in TreeInfo._fields_}
        self.N = self.info["n_nodes"]

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _LIB is not None:
            try:
                _LIB.tree_free(h)
            except Exception:  # interpreter shutdown
                pass
            self.handle = None

    def export(self):
        N, T, S = self.N, self.info["n_targets"], self.info["seq_tokens"]
        out = {k: np.zeros(N, dtype=np.int32) for k in ("token", "depth", "end", "parent", "n_pass")}
        out["weight"] = np.zeros(N, dtype=np.float32)
        out["seq_pos_to_dfs"] = np.zeros(S, dtype=np.int32)
        out["tgt_row_ptr"] = np.zeros(N + 1, dtype=np.int32)
        out["tgt_dfs"] = np.zeros(T, dtype=np.int32)
        out["tgt_token"] = np.zeros(T, dtype=np.int32)
        out["tgt_w"] = np.zeros(T, dtype=np.float32)
        arr = TreeArrays(**{k: _ptr(v, ctypes.c_float if v.dtype == np.float32 else ctypes.c_int32)
                            for k, v in out.items()})
        _check(lib().tree_export(self.handle, ctypes.byref(arr)))
        return out

    def target_weights(self, seq_scale=None, token_mask=None):
        """Target weights [n_targets] (tgt_dfs order) for per-sequence scalars and per-token masks."""
        out = np.zeros(self.info["n_targets"], dtype=np.float32)
        sc = None if seq_scale is None else np.ascontiguousarray(seq_scale, dtype=np.float32)
        mk = None if token_mask is None else np.ascontiguousarray(token_mask, dtype=np.uint8)
        if sc is not None and sc.shape != (self.info["n_seqs"],):
            raise ValueError("seq_scale must have one entry per sequence")
        if mk is not None and mk.shape != (self.info["seq_tokens"],):
            raise ValueError("token_mask must have one entry per input token")
        _check(lib().tree_target_weights(self.handle, None if sc is None else _ptr(sc, ctypes.c_float),
                                         None if mk is None else _ptr(mk, ctypes.c_uint8),
                                         _ptr(out, ctypes.c_float)))
        return out

    def plan_bytes(self):
        n = ctypes.c_size_t()
        _check(lib().tree_plan_bytes(self.handle, ctypes.byref(n)))
        return n.value

    def plan_host(self):
        """The plan image as host int32 words (no GPU needed)."""
        buf = np.zeros(self.plan_bytes() // 4, dtype=np.int32)
        _check(lib().tree_plan_copy(self.handle, buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes))
        return buf

    def schedule(self):
        """Decoded tile schedule: dict {(qb, kb): full}, per-k-block (qlo, qhi, minend), orders."""
        p = self.plan_host()
        H = dict(N=1, BQ=2, BK=3, NQB=4, NKB=5, NTILES=6, DEPTH=8, END=9, QB_PTR=10, QB_TILES=11,
                 QB_ORDER=12, KB_QLO=13, KB_QHI=14, KB_MINEND=15, KB_ORDER=16)
        nqb, nkb = int(p[H["NQB"]]), int(p[H["NKB"]])
        ptr = p[p[H["QB_PTR"]]:p[H["QB_PTR"]] + nqb + 1]
        tl = p[p[H["QB_TILES"]]:p[H["QB_TILES"]] + int(p[H["NTILES"]])]
        tiles = {}
        for qb in range(nqb):
            for e in range(ptr[qb], ptr[qb + 1]):
                tiles[(qb, int(tl[e] & 0x3FFFFFFF))] = bool(tl[e] & 0x40000000)
        sec = lambda name, n: p[p[H[name]]:p[H[name]] + n].copy()  # noqa: E731
        return dict(tiles=tiles, qb_ptr=ptr.copy(), depth=sec("DEPTH", self.N), end=sec("END", self.N),
                    qb_order=sec("QB_ORDER", nqb), kb_qlo=sec("KB_QLO", nkb), kb_qhi=sec("KB_QHI", nkb),
                    kb_minend=sec("KB_MINEND", nkb),
                    kb_order=sec("KB_ORDER", -(-nkb // max(1, 256 // int(p[H["BK"]])))),
                    bq=int(p[H["BQ"]]), bk=int(p[H["BK"]]))

    def upload_plan(self, device="cuda"):
        """Device plan as a torch uint8 tensor, copied on the current stream."""
        import torch
        buf = torch.empty(self.plan_bytes(), dtype=torch.uint8, device=device)
        _check(lib().tree_plan_upload(self.handle, ctypes.c_void_p(buf.data_ptr()), buf.numel(), _stream()))
        torch.cuda.current_stream().synchronize()  # the host image must outlive the copy
        return buf


# ------------------------------------------------------------------ attention
def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return TT_F32
    if t.dtype == torch.bfloat16:
        return TT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p()


def _fail(msg):
    raise ValueError(msg)


def _check_tensor(t, name, dtypes=None, shape=None):
    """Type, dtype, shape and contiguity of one tensor argument (ValueError)."""
    import torch
    if not isinstance(t, torch.Tensor):
        _fail(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        _fail(f"{name} has dtype {t.dtype}; expected {' or '.join(str(d) for d in dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        _fail(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if not t.is_contiguous():
        _fail(f"{name} must be contiguous (a strided view is read as if it were dense)")


def _check_devices(**named):
    """Every given tensor on one CUDA (HIP) device (checked after the layouts)."""
    ref = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            _fail(f"{name} must be on a CUDA (HIP) device, not {t.device}")
        if ref is None:
            ref = (name, t.device)
        elif t.device != ref[1]:
            _fail(f"{name} is on {t.device} but {ref[0]} is on {ref[1]}")


def _check_plan(tree, plan):
    import torch
    _check_tensor(plan, "plan", (torch.uint8,))
    if plan.numel() < tree.plan_bytes():
        _fail(f"plan holds {plan.numel()} bytes; this tree's plan needs {tree.plan_bytes()}")


def _check_workspace(ws):
    import torch
    if ws is not None:
        _check_tensor(ws, "workspace", (torch.uint8,))


def _check_attn(tree, plan, q, k, v, workspace):
    """q [n_q, h_q, d], k and v [n_k, h_kv, d], one dtype (float32 or bfloat16)."""
    import torch
    _check_tensor(q, "q", (torch.float32, torch.bfloat16))
    if q.dim() != 3:
        _fail(f"q must be [n_q, h_q, d]; got shape {tuple(q.shape)}")
    _check_tensor(k, "k", (q.dtype,))
    if k.dim() != 3 or k.shape[2] != q.shape[2]:
        _fail(f"k must be [n_k, h_kv, {q.shape[2]}]; got shape {tuple(k.shape)}")
    _check_tensor(v, "v", (q.dtype,), shape=k.shape)
    _check_plan(tree, plan)
    _check_workspace(workspace)


def _attn_args(tree, plan, q, k, v, o, lse, q_off, scale, rope_base, allow_generic=False):
    n_q, h_q, d = q.shape
    n_k, h_kv, _ = k.shape
    return AttnArgs(tree=tree.handle, plan=ctypes.c_void_p(plan.data_ptr()), q_off=q_off, n_q=n_q, n_k=n_k,
                    h_q=h_q, h_kv=h_kv, d=d, dtype=_dt(q), scale=scale, rope_base=rope_base,
                    q=_p(q), k=_p(k), v=_p(v), o=_p(o), lse=_p(lse), workspace=None, workspace_bytes=0,
                    flags=TT_ALLOW_GENERIC if allow_generic else 0)


def attn_workspace_bytes(tree, plan, q, k, v, for_bwd, q_off=0, rope_base=10000.0):
    a = _attn_args(tree, plan, q, k, v, None, None, q_off, 0.0, rope_base)
    n = ctypes.c_size_t()
    _check(lib().tree_attn_workspace_bytes(ctypes.byref(a), int(for_bwd), ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device, workspace):
    import torch
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return workspace


def tree_attn_fwd(tree, plan, q, k, v, q_off=0, scale=0.0, rope_base=10000.0, o=None, lse=None, workspace=None,
                  allow_generic=False):
    """O, LSE of tree attention for query rows [q_off, q_off + q.shape[0]) against key rows [0, k.shape[0]).

    allow_generic: run bf16 shapes the matrix-core kernels do not take on the
    vector kernels instead of raising (TT_ALLOW_GENERIC)."""
    import torch
    _check_attn(tree, plan, q, k, v, workspace)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    _check_tensor(o, "o", (q.dtype,), shape=q.shape)
    _check_tensor(lse, "lse", (torch.float32,), shape=q.shape[:2])
    _check_devices(q=q, k=k, v=v, o=o, lse=lse, plan=plan, workspace=workspace)
    a = _attn_args(tree, plan, q, k, v, o, lse, q_off, scale, rope_base, allow_generic)
    n = ctypes.c_size_t()
    _check(lib().tree_attn_workspace_bytes(ctypes.byref(a), 0, ctypes.byref(n)))
    ws = _workspace(n.value, q.device, workspace)
    a.workspace = ctypes.c_void_p(ws.data_ptr())
    a.workspace_bytes = ws.numel()
    _check(lib().tree_attn_fwd(ctypes.byref(a), _stream()))
    return o, lse


def tree_attn_bwd(tree, plan, q, k, v, o, lse, d_o, q_off=0, scale=0.0, rope_base=10000.0, d_q=None, d_k=None,
                  d_v=None, accumulate=False, workspace=None, reuse_rotated=False, allow_generic=False):
    """dQ, dK, dV (dK/dV are float32 and added into when accumulate=True).

    reuse_rotated: `workspace` is the one tree_attn_fwd used for these same
    arguments, unmodified since; the backward then takes its rotated q and k."""
    if reuse_rotated and workspace is None:
        raise ValueError("reuse_rotated needs the forward's workspace")
    import torch
    _check_attn(tree, plan, q, k, v, workspace)
    _check_tensor(o, "o", (q.dtype,), shape=q.shape)
    _check_tensor(lse, "lse", (torch.float32,), shape=q.shape[:2])
    _check_tensor(d_o, "d_o", (q.dtype,), shape=q.shape)
    gdt = torch.float32 if accumulate else k.dtype
    for name, t in (("d_k", d_k), ("d_v", d_v)):
        if t is not None:
            _check_tensor(t, name, (gdt,), shape=k.shape)
    if d_q is not None:
        _check_tensor(d_q, "d_q", (q.dtype,), shape=q.shape)
    _check_devices(q=q, k=k, v=v, o=o, lse=lse, d_o=d_o, d_q=d_q, d_k=d_k, d_v=d_v, plan=plan, workspace=workspace)
    if d_q is None:
        d_q = torch.empty_like(q)
    if d_k is None:
        d_k = (torch.zeros(k.shape, dtype=torch.float32, device=k.device) if accumulate else torch.empty_like(k))
    if d_v is None:
        d_v = (torch.zeros(v.shape, dtype=torch.float32, device=v.device) if accumulate else torch.empty_like(v))
    a = _attn_args(tree, plan, q, k, v, o, lse, q_off, scale, rope_base, allow_generic)
    n = ctypes.c_size_t()
    _check(lib().tree_attn_workspace_bytes(ctypes.byref(a), 1, ctypes.byref(n)))
    ws = _workspace(n.value, q.device, workspace)
    a.workspace = ctypes.c_void_p(ws.data_ptr())
    a.workspace_bytes = ws.numel()
    b = AttnBwdArgs(a=a, d_o=_p(d_o), d_q=_p(d_q), d_k=_p(d_k), d_v=_p(d_v),
                    flags=(TT_ACCUMULATE_DKDV if accumulate else 0) | (TT_BWD_REUSE_ROTATED if reuse_rotated else 0))
    _check(lib().tree_attn_bwd(ctypes.byref(b), _stream()))
    return d_q, d_k, d_v


# ------------------------------------------------------------------ path mode
class Path:
    """Depth-first walk plan over a tree's segments; see tree_path_build in include/tt.h."""

    def __init__(self, tree, chunk=2048, order=0):
        self.tree = tree  # the walk reads the tree: keep it alive
        self.plan = None  # device plan of the walk, uploaded on first use
        self.handle = ctypes.c_void_p()
        _check(lib().tree_path_build(tree.handle, int(chunk), int(order), ctypes.byref(self.handle)))
        inf = PathInfo()
        _check(lib().tree_path_info(self.handle, ctypes.byref(inf)))
        self.info = {n: int(getattr(inf, n)) for n, _ in PathInfo._fields_}

    def plan_bytes(self):
        n = ctypes.c_size_t()
        _check(lib().tree_path_plan_bytes(self.handle, ctypes.byref(n)))
        return n.value

    def upload_plan(self, device="cuda"):
        """The walk's device plan (uploaded once per path and device, kept on the object)."""
        import torch
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if self.plan is None or self.plan.device != dev:
            buf = torch.empty(max(self.plan_bytes(), 16), dtype=torch.uint8, device=dev)
            _check(lib().tree_path_plan_upload(self.handle, ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                               _stream()))
            torch.cuda.current_stream().synchronize()  # the host image must outlive the copy
            self.plan = buf
        return self.plan

    def segments(self):
        """Segment table (row0, len, depth0, parent) and the walk's events, as host arrays."""
        S = self.info["n_segments"]
        out = {k: np.zeros(S, dtype=np.int32) for k in ("row0", "len", "depth0", "parent")}
        out["events"] = np.zeros(2 * S, dtype=np.int32)
        _check(lib().tree_path_segments(self.handle, *(_ptr(out[k], ctypes.c_int32) for k in
                                                      ("row0", "len", "depth0", "parent", "events"))))
        return out

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _LIB is not None:
            try:
                _LIB.tree_path_free(h)
            except Exception:  # interpreter shutdown
                pass
            self.handle = None


def _path_args(path, q, k, v, d_o, scale, rope_base, plan=None, allow_generic=False):
    _, h_q, d = q.shape
    h_kv = k.shape[1]
    return PathArgs(path=path.handle, plan=_p(plan), h_q=h_q, h_kv=h_kv, d=d, dtype=_dt(q), scale=scale,
                    rope_base=rope_base, q=_p(q), k=_p(k), v=_p(v), d_o=_p(d_o),
                    flags=TT_ALLOW_GENERIC if allow_generic else 0)


def path_workspace_bytes(path, q, k, v, backward, scale=0.0, rope_base=10000.0):
    a = _path_args(path, q, k, v, q if backward else None, scale, rope_base)
    n = ctypes.c_size_t()
    _check(lib().tree_path_workspace_bytes(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def tree_attn_path(path, q, k, v, d_o=None, scale=0.0, rope_base=10000.0, o=None, lse=None, d_q=None, d_k=None,
                   d_v=None, workspace=None, allow_generic=False):
    """Path-mode walk of one layer: (o, lse), or (o, lse, d_q, d_k, d_v) when d_o is given."""
    import torch
    N = path.tree.N
    _check_tensor(q, "q", (torch.float32, torch.bfloat16))
    if q.dim() != 3 or q.shape[0] != N:
        _fail(f"q must be [{N}, h_q, d] (one row per tree row); got shape {tuple(q.shape)}")
    _check_tensor(k, "k", (q.dtype,))
    if k.dim() != 3 or k.shape[0] != N or k.shape[2] != q.shape[2]:
        _fail(f"k must be [{N}, h_kv, {q.shape[2]}]; got shape {tuple(k.shape)}")
    _check_tensor(v, "v", (q.dtype,), shape=k.shape)
    _check_workspace(workspace)
    for name, t, shp, dts in (("o", o, q.shape, (q.dtype,)), ("lse", lse, q.shape[:2], (torch.float32,)),
                              ("d_o", d_o, q.shape, (q.dtype,)), ("d_q", d_q, q.shape, (q.dtype,)),
                              ("d_k", d_k, k.shape, (q.dtype,)), ("d_v", d_v, k.shape, (q.dtype,))):
        if t is not None:
            _check_tensor(t, name, dts, shape=shp)
    _check_devices(q=q, k=k, v=v, o=o, lse=lse, d_o=d_o, d_q=d_q, d_k=d_k, d_v=d_v, workspace=workspace)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    if d_o is not None:
        d_q = torch.empty_like(q) if d_q is None else d_q
        d_k = torch.empty_like(k) if d_k is None else d_k
        d_v = torch.empty_like(v) if d_v is None else d_v
    plan = path.upload_plan(q.device)
    a = _path_args(path, q, k, v, d_o, scale, rope_base, plan, allow_generic)
    a.o, a.lse, a.d_q, a.d_k, a.d_v = _p(o), _p(lse), _p(d_q), _p(d_k), _p(d_v)
    n = ctypes.c_size_t()
    _check(lib().tree_path_workspace_bytes(ctypes.byref(a), ctypes.byref(n)))
    ws = _workspace(n.value, q.device, workspace)
    a.workspace = ctypes.c_void_p(ws.data_ptr())
    a.workspace_bytes = ws.numel()
    _check(lib().tree_attn_path(ctypes.byref(a), _stream()))
    return (o, lse) if d_o is None else (o, lse, d_q, d_k, d_v)


# ------------------------------------------------------------------ weighted NLL
def tree_weighted_nll(tgt_row_ptr, tgt_id, tgt_w, logits=None, hidden=None, w_vocab=None, want_logp=True,
                      grad=True, dw_dtype=None, d_logits=None, workspace=None):
    """Weighted tree NLL (logits mode or fused lm-head mode).

    Returns dict(loss=<0-d float32 tensor>, logp, d_logits | d_hidden, d_w_vocab)."""
    import torch
    fused = hidden is not None
    if fused == (logits is not None):
        _fail("give exactly one of logits or hidden (with w_vocab)")
    if fused:
        _check_tensor(hidden, "hidden", (torch.bfloat16,))
        if hidden.dim() != 2:
            _fail(f"hidden must be [n_rows, d_model]; got shape {tuple(hidden.shape)}")
        _check_tensor(w_vocab, "w_vocab", (torch.bfloat16,))
        if w_vocab.dim() != 2 or w_vocab.shape[0] != hidden.shape[1]:
            _fail(f"w_vocab must be [{hidden.shape[1]}, vocab]; got shape {tuple(w_vocab.shape)}")
    else:
        if w_vocab is not None:
            _fail("w_vocab needs hidden (fused mode)")
        _check_tensor(logits, "logits", (torch.float32, torch.bfloat16))
        if logits.dim() != 2:
            _fail(f"logits must be [n_rows, vocab]; got shape {tuple(logits.shape)}")
        if d_logits is not None:
            _check_tensor(d_logits, "d_logits", (logits.dtype,), shape=logits.shape)
    ref = hidden if fused else logits
    _check_tensor(tgt_row_ptr, "tgt_row_ptr", (torch.int32,), shape=(ref.shape[0] + 1,))
    _check_tensor(tgt_id, "tgt_id", (torch.int32,))
    if tgt_id.dim() != 1:
        _fail(f"tgt_id must be one-dimensional; got shape {tuple(tgt_id.shape)}")
    _check_tensor(tgt_w, "tgt_w", (torch.float32,), shape=tgt_id.shape)
    _check_workspace(workspace)
    _check_devices(hidden=hidden, w_vocab=w_vocab, logits=logits, d_logits=d_logits, tgt_row_ptr=tgt_row_ptr,
                   tgt_id=tgt_id, tgt_w=tgt_w, workspace=workspace)
    dev = ref.device
    n_rows = ref.shape[0]
    vocab = w_vocab.shape[1] if fused else logits.shape[1]
    d_model = hidden.shape[1] if fused else 0
    n_tgt = tgt_id.shape[0]
    out = {"loss": torch.empty((), dtype=torch.float32, device=dev)}
    out["logp"] = torch.empty(n_tgt, dtype=torch.float32, device=dev) if want_logp and n_tgt else None
    a = NllArgs(n_rows=n_rows, d_model=d_model, vocab=vocab, n_tgt=n_tgt,
                hidden=_p(hidden) if fused else None, w_vocab=_p(w_vocab) if fused else None,
                logits=None if fused else _p(logits), logits_dtype=_dt(logits) if not fused else TT_BF16,
                tgt_row_ptr=_p(tgt_row_ptr), tgt_id=_p(tgt_id), tgt_w=_p(tgt_w),
                loss=_p(out["loss"]), logp=_p(out["logp"]), dw_dtype=TT_F32)
    if grad:
        if fused:
            out["d_hidden"] = torch.empty_like(hidden)
            dwt = dw_dtype or torch.float32
            out["d_w_vocab"] = torch.empty(w_vocab.shape, dtype=dwt, device=dev)
            a.d_hidden = _p(out["d_hidden"])
            a.d_w_vocab = _p(out["d_w_vocab"])
            a.dw_dtype = _dt(out["d_w_vocab"])
        else:
            out["d_logits"] = d_logits if d_logits is not None else torch.empty_like(logits)
            a.d_logits = _p(out["d_logits"])
    n = ctypes.c_size_t()
    _check(lib().tree_nll_workspace_bytes(ctypes.byref(a), ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    a.workspace = ctypes.c_void_p(ws.data_ptr())
    a.workspace_bytes = ws.numel()
    _check(lib().tree_weighted_nll(ctypes.byref(a), _stream()))
    return out

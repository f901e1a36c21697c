"""Python binding of librattn: fused residual attention over a shared base KV cache
on AMD Instinct MI355X (gfx950).

Thin marshalling over the C ABI declared in ``include/rattn.h`` (same names):
shapes are read from the torch tensors, pointers and the current HIP stream are
passed through ctypes, and the workspace is a torch allocation.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, importing succeeds but every call raises.

Tensor layouts (row-major, contiguous, on the GPU):
  q        [N, q_len, H_q, d]
  k_base   [H_kv, L, d], or a paged pool [n_phys, H_kv, page, d] with block_table [ceil(L/page)] int32
  lk, lv   [N, L, r] (or [1, L, r] with shared_lr)
  bk, bv   [N, r, H_kv*d]
  k_priv   [N, H_kv, S, d]
  out      [N, q_len, H_q, d] fp32,  lse [N, q_len, H_q] fp32
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librattn.so")

RATTN_F32, RATTN_BF16 = 0, 1
RATTN_KEYS_DTYPE, RATTN_KEYS_INT8 = 0, 1
RATTN_VALUES_DTYPE, RATTN_VALUES_FWHT3 = 0, 1
RATTN_OP_DECODE, RATTN_OP_PREFILL, RATTN_OP_RECONSTRUCT = 0, 1, 2
STATUS = {0: "RATTN_OK", -1: "RATTN_E_NULL", -2: "RATTN_E_SHAPE", -3: "RATTN_E_UNSUPPORTED",
          -4: "RATTN_E_WORKSPACE", -5: "RATTN_E_ALIGN", -6: "RATTN_E_HIP", -7: "RATTN_E_SCRATCH",
          -8: "RATTN_E_POOL"}
NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTS = ("rattn_workspace_bytes", "rattn_decode", "rattn_prefill_chunk", "rattn_gather_base",
           "rattn_decode_plan", "rattn_prefill_plan", "rattn_status_str", "rattn_version", "rattn_last_hip_error",
           "rattn_attention_stages", "rattn_decode_noalloc", "rattn_lr_project", "rattn_pagepool_create",
           "rattn_pagepool_destroy", "rattn_pagepool_free_pages", "rattn_pagepool_refcount", "rattn_pagepool_alloc",
           "rattn_pagepool_retain", "rattn_pagepool_release", "rattn_pagepool_plan_append", "rattn_append_kv",
           "rattn_quantize_keys", "rattn_decode_reconstruct", "rattn_quantize_values", "rattn_values_codebook", "rattn_check_block_table")
STAGE_SPLIT, STAGE_COMBINE, STAGE_ALL = 1, 2, 3


class RattnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = f"{what}: {STATUS.get(status, status)}"
        if status == -6 and _lib is not None:
            msg += f" (hipError {_lib.rattn_last_hip_error()})"
        super().__init__(msg)


class Desc(ctypes.Structure):
    _fields_ = [
        ("n_agents", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("prefix_len", ctypes.c_int64), ("priv_len", ctypes.c_int64),
        ("page_size", ctypes.c_int32), ("shared_lr", ctypes.c_int32),
        ("n_phys_pages", ctypes.c_int64), ("dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("k_format", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_format", ctypes.c_int32),
    ]


ARG_NAMES = ("q", "k_base", "v_base", "block_table", "lk", "lv", "bk", "bv", "k_priv", "v_priv", "out", "lse",
             "v_scale")


class Args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ARG_NAMES]


class LrDesc(ctypes.Structure):
    _fields_ = [("n_sets", ctypes.c_int32), ("shared_x", ctypes.c_int32), ("shared_a", ctypes.c_int32),
                ("d_in", ctypes.c_int32), ("rank", ctypes.c_int32), ("n_tokens", ctypes.c_int64),
                ("pos0", ctypes.c_int64), ("cache_len", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_prefix_splits", ctypes.c_int32), ("prefix_split_len", ctypes.c_int64),
                ("n_priv_splits", ctypes.c_int32), ("priv_split_len", ctypes.c_int64),
                ("row_blocks", ctypes.c_int32), ("agents_per_block", ctypes.c_int32),
                ("resid_cols", ctypes.c_int32), ("work_items", ctypes.c_int32),
                ("heads_per_item", ctypes.c_int32), ("waves", ctypes.c_int32), ("masked", ctypes.c_int32),
                ("blocks_per_group", ctypes.c_int32), ("path", ctypes.c_int32), ("rows_per_item", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded librattn (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"librattn is not built ({LIB_PATH} missing): run "
                               "`python -m shared_base_residual_amd.build`")
        # torch first: its HIP runtime is then the one librattn binds to (one
        # runtime per process; loading librattn first would bind the system
        # runtime, under which torch's own device calls then fail)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.rattn_workspace_bytes.argtypes = [ctypes.POINTER(Desc), I, ctypes.POINTER(ctypes.c_size_t)]
        L.rattn_decode.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args), P, ctypes.c_size_t, P]
        L.rattn_prefill_chunk.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args), P, ctypes.c_size_t, P]
        L.rattn_gather_base.argtypes = [ctypes.POINTER(Desc), P, P, P, P]
        L.rattn_decode_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(PlanInfo)]
        L.rattn_prefill_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(PlanInfo)]
        L.rattn_attention_stages.argtypes = [ctypes.POINTER(Desc), I, ctypes.POINTER(Args), P, ctypes.c_size_t, P,
                                             ctypes.c_uint]
        L.rattn_decode_noalloc.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args), P]
        I64, I32P = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
        L.rattn_lr_project.argtypes = [ctypes.POINTER(LrDesc), P, P, P, P, P, P]
        L.rattn_pagepool_create.argtypes = [I64, ctypes.POINTER(P)]
        L.rattn_pagepool_destroy.argtypes = [P]
        L.rattn_pagepool_destroy.restype = None
        L.rattn_pagepool_free_pages.argtypes = [P]
        L.rattn_pagepool_free_pages.restype = I64
        L.rattn_pagepool_refcount.argtypes = [P, ctypes.c_int32, I32P]
        L.rattn_pagepool_alloc.argtypes = [P, I64, I32P]
        L.rattn_pagepool_retain.argtypes = [P, I32P, I64]
        L.rattn_pagepool_release.argtypes = [P, I32P, I64]
        L.rattn_pagepool_plan_append.argtypes = [P, I32P, I64, I64, I64, ctypes.c_int32, I32P, I32P]
        L.rattn_append_kv.argtypes = [ctypes.POINTER(Desc), P, P, P, I64, I64, P, P, ctypes.c_int32,
                                      ctypes.c_int32, P]
        L.rattn_quantize_keys.argtypes = [P, I64, ctypes.c_int32, P, P, P]
        L.rattn_decode_reconstruct.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Args), P, P, ctypes.c_size_t, P]
        L.rattn_quantize_values.argtypes = [P, I64, ctypes.c_int32, ctypes.c_int32, P, P, P]
        L.rattn_values_codebook.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.rattn_check_block_table.argtypes = [ctypes.POINTER(Desc), P, P, P]
        for f in ("rattn_decode_reconstruct", "rattn_quantize_keys", "rattn_lr_project", "rattn_pagepool_create", "rattn_pagepool_refcount", "rattn_pagepool_alloc",
                  "rattn_pagepool_retain", "rattn_pagepool_release", "rattn_pagepool_plan_append",
                  "rattn_append_kv"):
            getattr(L, f).restype = I
        L.rattn_status_str.argtypes = [I]
        L.rattn_status_str.restype = ctypes.c_char_p
        for f in ("rattn_workspace_bytes", "rattn_decode", "rattn_prefill_chunk", "rattn_gather_base",
                  "rattn_decode_plan", "rattn_prefill_plan", "rattn_version", "rattn_last_hip_error",
                  "rattn_attention_stages", "rattn_decode_noalloc", "rattn_lr_project", "rattn_pagepool_create",
           "rattn_pagepool_destroy", "rattn_pagepool_free_pages", "rattn_pagepool_refcount", "rattn_pagepool_alloc",
           "rattn_pagepool_retain", "rattn_pagepool_release", "rattn_pagepool_plan_append", "rattn_append_kv",
           "rattn_quantize_keys", "rattn_decode_reconstruct", "rattn_quantize_values", "rattn_values_codebook", "rattn_check_block_table"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def make_desc(*, n_agents, n_q_heads, n_kv_heads, head_dim, rank, q_len, prefix_len, priv_len=0, page_size=0,
              shared_lr=False, n_phys_pages=0, dtype=RATTN_BF16, sm_scale=0.0, k_format=RATTN_KEYS_DTYPE,
              k_scale=0.0, v_format=RATTN_VALUES_DTYPE) -> Desc:
    return Desc(n_agents, n_q_heads, n_kv_heads, head_dim, rank, q_len, prefix_len, priv_len, page_size,
                int(bool(shared_lr)), n_phys_pages, dtype, sm_scale, k_format, k_scale, v_format)


def workspace_bytes(desc: Desc, op: int = RATTN_OP_DECODE) -> int:
    n = ctypes.c_size_t(0)
    st = lib().rattn_workspace_bytes(ctypes.byref(desc), op, ctypes.byref(n))
    if st:
        raise RattnError(st, "rattn_workspace_bytes")
    return n.value


def decode_plan(desc: Desc) -> dict:
    info = PlanInfo()
    st = lib().rattn_decode_plan(ctypes.byref(desc), ctypes.byref(info))
    if st:
        raise RattnError(st, "rattn_decode_plan")
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def prefill_plan(desc: Desc) -> dict:
    info = PlanInfo()
    st = lib().rattn_prefill_plan(ctypes.byref(desc), ctypes.byref(info))
    if st:
        raise RattnError(st, "rattn_prefill_plan")
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def plan(desc: Desc, op: int = RATTN_OP_DECODE) -> dict:
    return prefill_plan(desc) if op == RATTN_OP_PREFILL else decode_plan(desc)


def kernel_of(desc: Desc, op: int = RATTN_OP_DECODE) -> tuple:
    """The kernel instantiation a call runs: ("split", dtype, d, residual columns,
    masked, twelve-wave form) or ("prefill", dtype, d, residual columns)."""
    p = plan(desc, op)
    dt = "bf16" if desc.dtype == RATTN_BF16 else "f32"
    if desc.k_format == RATTN_KEYS_INT8:
        dt += "-k8"
    if desc.v_format == RATTN_VALUES_FWHT3:
        dt += "v3"
    if p["path"] == 1:
        return ("prefill", dt, desc.head_dim, p["resid_cols"])
    return ("split", dt, desc.head_dim, p["resid_cols"], bool(p["masked"]), p["waves"] > 8)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def describe(q, k_base, lk=None, bk=None, *, block_table=None, k_priv=None, prefix_len=None, shared_lr=None,
             sm_scale=0.0, op=RATTN_OP_DECODE, k_scale=None, v_base=None) -> Desc:
    """Descriptor read off the tensors' shapes.  A uint8 k_base holds int8 key
    codes (excess-128, RATTN_KEYS_INT8) whose scale ``k_scale`` must be given;
    a uint8 v_base holds 3-bit value codes (RATTN_VALUES_FWHT3)."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [N, q_len, H_q, d]")
    N, QL, HQ, D = q.shape
    paged = block_table is not None
    if k_base is not None:
        if paged:
            n_phys, HK, ps = k_base.shape[0], k_base.shape[1], k_base.shape[2]
        else:
            HK, ps, n_phys = k_base.shape[0], 0, 0
    else:
        HK = k_priv.shape[1]
        ps, n_phys = 0, 0
    if prefix_len is None:
        if lk is not None:
            prefix_len = lk.shape[1]
        elif k_base is not None and not paged:
            prefix_len = k_base.shape[1]
        else:
            raise ValueError("prefix_len must be given for a paged base cache without a low-rank cache")
    r = bk.shape[1] if bk is not None else 0
    if shared_lr is None:
        shared_lr = lk is not None and lk.shape[0] == 1 and N > 1
    S = k_priv.shape[2] if k_priv is not None else 0
    if q.dtype == torch.bfloat16:
        dt = RATTN_BF16
    elif q.dtype == torch.float32:
        dt = RATTN_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    kf, ks = RATTN_KEYS_DTYPE, 0.0
    if k_base is not None and k_base.dtype == torch.uint8:
        if k_scale is None:
            raise ValueError("int8 keys (uint8 k_base) need k_scale")
        kf, ks = RATTN_KEYS_INT8, float(k_scale)
    vf = RATTN_VALUES_FWHT3 if v_base is not None and v_base.dtype == torch.uint8 else RATTN_VALUES_DTYPE
    return make_desc(n_agents=N, n_q_heads=HQ, n_kv_heads=HK, head_dim=D, rank=r, q_len=QL,
                     prefix_len=prefix_len, priv_len=S, page_size=ps, shared_lr=shared_lr,
                     n_phys_pages=n_phys, dtype=dt, sm_scale=sm_scale, k_format=kf, k_scale=ks, v_format=vf)


def _check_tensors(desc: Desc, tensors: dict):
    """Marshalling checks the C ABI cannot make on raw pointers: device, dtype,
    contiguity and shapes."""
    import torch

    dt = torch.bfloat16 if desc.dtype == RATTN_BF16 else torch.float32
    N, QL, HQ, HK, D, r = desc.n_agents, desc.q_len, desc.n_q_heads, desc.n_kv_heads, desc.head_dim, desc.rank
    L, S = desc.prefix_len, desc.priv_len
    nlr = 1 if desc.shared_lr else N
    want = {"q": (N, QL, HQ, D), "lk": (nlr, L, r), "lv": (nlr, L, r), "bk": (N, r, HK * D),
            "bv": (N, r, HK * D), "k_priv": (N, HK, S, D), "v_priv": (N, HK, S, D),
            "out": (N, QL, HQ, D), "lse": (N, QL, HQ)}
    if desc.page_size:
        want["k_base"] = want["v_base"] = (desc.n_phys_pages, HK, desc.page_size, D)
        want["block_table"] = ((L + desc.page_size - 1) // desc.page_size,)
    else:
        want["k_base"] = want["v_base"] = (HK, L, D)
    if desc.v_format == RATTN_VALUES_FWHT3:
        want["v_base"] = (HK, L, 3 * D // 8)
        want["v_scale"] = (HK, L)
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        exp_dt = torch.float32 if name in ("out", "lse") else (torch.int32 if name == "block_table" else dt)
        if name == "k_base" and desc.k_format == RATTN_KEYS_INT8:
            exp_dt = torch.uint8
        if name == "v_base" and desc.v_format == RATTN_VALUES_FWHT3:
            exp_dt = torch.uint8
        if name == "v_scale":
            exp_dt = torch.float32
        if t.dtype != exp_dt:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {exp_dt}")
        if name in want and tuple(t.shape) != want[name]:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want[name]}")


_workspaces = {}


def _ws_key(device, stream) -> tuple:
    """Cache key of a workspace: the device and the HIP stream the call is
    launched on (two streams never share one, since calls that share a
    workspace must not overlap)."""
    return (str(device), int(stream.cuda_stream))


def workspace_for(nbytes: int, device, stream=None):
    """A workspace of at least ``nbytes`` for calls launched on ``stream`` (the
    current stream when None), cached per (device, stream); its contents do not
    matter between calls.  It is allocated while that stream is current, so the
    caching allocator ties it to the stream the kernels run on: a buffer
    replaced by a larger one is reused only by work ordered after them."""
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = _ws_key(device, s)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.empty(max(nbytes, 256), device=device, dtype=torch.uint8)
        _workspaces[key] = ws
    return ws


def _run(fn_name, op, q, k_base, v_base, lk, lv, bk, bv, block_table, k_priv, v_priv, shared_lr, out, lse,
         workspace, sm_scale, prefix_len, stream, desc, stages=None, k_scale=None, v_scale=None):
    import torch

    if desc is None:
        desc = describe(q, k_base, lk, bk, block_table=block_table, k_priv=k_priv, prefix_len=prefix_len,
                        shared_lr=shared_lr, sm_scale=sm_scale, op=op, k_scale=k_scale, v_base=v_base)
    if out is None:
        out = torch.empty(tuple(q.shape), device=q.device, dtype=torch.float32)
    tensors = dict(q=q, k_base=k_base, v_base=v_base, block_table=block_table, lk=lk, lv=lv, bk=bk, bv=bv,
                   k_priv=k_priv, v_priv=v_priv, out=out, lse=lse, v_scale=v_scale)
    _check_tensors(desc, tensors)
    nbytes = workspace_bytes(desc, op)
    if workspace is None:
        workspace = workspace_for(nbytes, q.device, stream)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise RattnError(-4, f"{fn_name}: workspace has {workspace.numel() * workspace.element_size()} bytes, "
                             f"needs {nbytes}")
    args = Args(*[_ptr(tensors.get(n)) for n in ARG_NAMES])
    wsp = ctypes.c_void_p(workspace.data_ptr())
    wsb = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    if stages is None:
        st = getattr(lib(), fn_name)(ctypes.byref(desc), ctypes.byref(args), wsp, wsb, _stream(stream))
    else:
        st = lib().rattn_attention_stages(ctypes.byref(desc), op, ctypes.byref(args), wsp, wsb, _stream(stream),
                                          stages)
        fn_name = f"rattn_attention_stages({stages})"
    if st:
        raise RattnError(st, fn_name)
    return out


def decode(q, k_base, v_base, lk=None, lv=None, bk=None, bv=None, *, block_table=None, k_priv=None,
           v_priv=None, shared_lr=None, out=None, lse=None, workspace=None, sm_scale=0.0, prefix_len=None,
           stream=None, desc: Optional[Desc] = None):
    """rattn_decode: every query token of agent a attends the shared prefix (base +
    agent a's low-rank residual) and all of agent a's private tokens.  Returns out."""
    return _run("rattn_decode", RATTN_OP_DECODE, q, k_base, v_base, lk, lv, bk, bv, block_table, k_priv, v_priv,
                shared_lr, out, lse, workspace, sm_scale, prefix_len, stream, desc)


def prefill_chunk(q, k_base, v_base, lk=None, lv=None, bk=None, bv=None, *, block_table=None, k_priv=None,
                  v_priv=None, shared_lr=None, out=None, lse=None, workspace=None, sm_scale=0.0,
                  prefix_len=None, stream=None, desc: Optional[Desc] = None):
    """rattn_prefill_chunk: chunk query t of agent a attends the prefix and chunk
    tokens 0..t (k_priv/v_priv hold the chunk's own keys and values)."""
    return _run("rattn_prefill_chunk", RATTN_OP_PREFILL, q, k_base, v_base, lk, lv, bk, bv, block_table, k_priv,
                v_priv, shared_lr, out, lse, workspace, sm_scale, prefix_len, stream, desc)


def decode_noalloc(inputs: dict, *, shared_lr=None, prefix_len=None, out, lse=None, stream=None, desc=None):
    """rattn_decode_noalloc on a dict of device tensors (named as in the layouts
    above): rattn_decode with the library's static scratch buffer instead of a
    workspace.  ``out`` (and ``lse``) are the caller's; nothing is allocated."""
    g = inputs.get
    if desc is None:
        desc = describe(inputs["q"], g("k_base"), g("lk"), g("bk"), block_table=g("block_table"),
                        k_priv=g("k_priv"), prefix_len=prefix_len, shared_lr=shared_lr, v_base=g("v_base"))
    tensors = dict(q=inputs["q"], k_base=g("k_base"), v_base=g("v_base"), block_table=g("block_table"), lk=g("lk"),
                   lv=g("lv"), bk=g("bk"), bv=g("bv"), k_priv=g("k_priv"), v_priv=g("v_priv"), out=out, lse=lse,
                   v_scale=g("v_scale"))
    _check_tensors(desc, tensors)
    args = Args(*[_ptr(tensors.get(n)) for n in ARG_NAMES])
    st = lib().rattn_decode_noalloc(ctypes.byref(desc), ctypes.byref(args), _stream(stream))
    if st:
        raise RattnError(st, "rattn_decode_noalloc")
    return out


def decode_reconstruct(inputs: dict, *, rope_theta=None, shared_lr=None, out=None, lse=None, workspace=None,
                       stream=None):
    """rattn_decode_reconstruct: decode with the residual keys rebuilt per token
    in registers, rotated by position when ``rope_theta`` (a [d/2] fp32 GPU
    tensor of frequencies) is given.  Returns out."""
    import torch

    g = inputs.get
    q = inputs["q"]
    desc = describe(q, g("k_base"), g("lk"), g("bk"), shared_lr=shared_lr)
    if out is None:
        out = torch.empty(tuple(q.shape), device=q.device, dtype=torch.float32)
    tensors = dict(q=q, k_base=g("k_base"), v_base=g("v_base"), block_table=None, lk=g("lk"), lv=g("lv"),
                   bk=g("bk"), bv=g("bv"), k_priv=None, v_priv=None, out=out, lse=lse)
    _check_tensors(desc, tensors)
    if rope_theta is not None:
        if not (rope_theta.is_cuda and rope_theta.dtype == torch.float32 and
                rope_theta.numel() == desc.head_dim // 2 and rope_theta.is_contiguous()):
            raise ValueError("rope_theta must be a contiguous fp32 GPU tensor of head_dim / 2 values")
    nbytes = workspace_bytes(desc, RATTN_OP_RECONSTRUCT)
    if workspace is None:
        workspace = workspace_for(nbytes, q.device, stream)
    args = Args(*[_ptr(tensors.get(n)) for n in ARG_NAMES])
    st = lib().rattn_decode_reconstruct(ctypes.byref(desc), ctypes.byref(args), _ptr(rope_theta),
                                        ctypes.c_void_p(workspace.data_ptr()),
                                        ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                        _stream(stream))
    if st:
        raise RattnError(st, "rattn_decode_reconstruct")
    return out


def quantize_keys(k, *, codes=None, scale=None, stream=None):
    """rattn_quantize_keys: int8 codes (uint8, excess-128) of the device tensor k
    (bf16 or fp32, every element covered by the one scale) and the scale as a
    one-element device tensor.  Returns (codes, scale)."""
    import torch

    if not k.is_cuda or not k.is_contiguous():
        raise ValueError("k must be a contiguous GPU tensor")
    if codes is None:
        codes = torch.empty(tuple(k.shape), device=k.device, dtype=torch.uint8)
    if scale is None:
        scale = torch.empty(1, device=k.device, dtype=torch.float32)
    dt = RATTN_BF16 if k.dtype == torch.bfloat16 else RATTN_F32
    if codes.numel() != k.numel() or codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous uint8 tensor of k's size")
    st = lib().rattn_quantize_keys(k.data_ptr(), k.numel(), dt, codes.data_ptr(), scale.data_ptr(),
                                   _stream(stream))
    if st:
        raise RattnError(st, "rattn_quantize_keys")
    return codes, scale


def quantize_values(v, *, codes=None, scale=None, stream=None):
    """rattn_quantize_values: 3-bit codes (uint8, three bit planes of d / 8
    bytes per vector) and fp32 scales of the value vectors in the device tensor
    v [..., d] (bf16 or fp32).  Returns (codes [..., 3 d / 8], scale [...])."""
    import torch

    if not v.is_cuda or not v.is_contiguous():
        raise ValueError("v must be a contiguous GPU tensor")
    d = v.shape[-1]
    n = v.numel() // d
    if codes is None:
        codes = torch.empty(tuple(v.shape[:-1]) + (3 * d // 8,), device=v.device, dtype=torch.uint8)
    if scale is None:
        scale = torch.empty(tuple(v.shape[:-1]), device=v.device, dtype=torch.float32)
    if codes.numel() != n * (3 * d // 8) or codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous uint8 tensor of 3 d / 8 bytes per vector")
    if scale.numel() != n or scale.dtype != torch.float32 or not scale.is_contiguous():
        raise ValueError("scale must be a contiguous fp32 tensor of one value per vector")
    dt = RATTN_BF16 if v.dtype == torch.bfloat16 else RATTN_F32
    st = lib().rattn_quantize_values(v.data_ptr(), n, d, dt, codes.data_ptr(), scale.data_ptr(), _stream(stream))
    if st:
        raise RattnError(st, "rattn_quantize_values")
    return codes, scale


def check_block_table(block_table, prefix_len: int, page_size: int, n_phys_pages: int, *, stream=None) -> int:
    """rattn_check_block_table: the number of the ceil(prefix_len / page_size)
    entries of the int32 device tensor ``block_table`` outside
    [0, n_phys_pages).  Synchronises the stream to read the count."""
    import torch

    desc = make_desc(n_agents=1, n_q_heads=1, n_kv_heads=1, head_dim=128, rank=0, q_len=1, prefix_len=prefix_len,
                     page_size=page_size, n_phys_pages=n_phys_pages)
    n = -(-prefix_len // page_size) if page_size > 0 else 0
    if block_table.dtype != torch.int32 or block_table.numel() < n or not block_table.is_contiguous():
        raise ValueError("block_table: a contiguous int32 tensor of at least ceil(prefix_len / page_size) entries")
    bad = torch.empty(1, device=block_table.device, dtype=torch.int32)
    st = lib().rattn_check_block_table(ctypes.byref(desc), ctypes.c_void_p(block_table.data_ptr()),
                                       ctypes.c_void_p(bad.data_ptr()), _stream(stream))
    if st:
        raise RattnError(st, "rattn_check_block_table")
    return int(bad.cpu().item())


def values_codebook():
    """The library's 8-level quantiser of N(0, 1): (centroids[8], boundaries[7])."""
    c = (ctypes.c_double * 8)()
    b = (ctypes.c_double * 7)()
    st = lib().rattn_values_codebook(c, b)
    if st:
        raise RattnError(st, "rattn_values_codebook")
    return list(c), list(b)


def lr_project(x, ak_t, av_t, lk, lv, *, pos0: int = 0, stream=None):
    """rattn_lr_project: rows pos0 .. pos0 + T - 1 of the low-rank caches,
    lk[n][pos0 + t] = X_n[t] A_k,n and lv likewise (bf16 out of an fp32 sum).
    x [1 or n_sets, T, d_in]; ak_t, av_t [1 or n_sets, r, d_in] (A transposed);
    lk, lv [n_sets, cache_len, r].  Returns (lk, lv)."""
    import torch

    n_sets, cache_len, r = lk.shape
    nx, T, d_in = x.shape
    desc = LrDesc(n_sets, int(nx == 1 and n_sets > 1 or n_sets == 1), int(ak_t.shape[0] == 1 and n_sets > 1 or
                                                                          n_sets == 1),
                  d_in, r, T, pos0, cache_len, RATTN_BF16 if x.dtype == torch.bfloat16 else RATTN_F32)
    want = {"x": (1 if desc.shared_x else n_sets, T, d_in), "ak_t": (1 if desc.shared_a else n_sets, r, d_in),
            "av_t": (1 if desc.shared_a else n_sets, r, d_in), "lv": (n_sets, cache_len, r)}
    for name, t in dict(x=x, ak_t=ak_t, av_t=av_t, lk=lk, lv=lv).items():
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError(f"{name} must be a contiguous GPU tensor of x's dtype")
        if name in want and tuple(t.shape) != want[name]:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want[name]}")
    st = lib().rattn_lr_project(ctypes.byref(desc), x.data_ptr(), ak_t.data_ptr(), av_t.data_ptr(), lk.data_ptr(),
                                lv.data_ptr(), _stream(stream))
    if st:
        raise RattnError(st, "rattn_lr_project")
    return lk, lv


class PagePool:
    """The library's host page allocator (rattn_pagepool_*): reference counts
    and a free list over n_pages physical pages, with copy-on-write appends."""

    def __init__(self, n_pages: int):
        h = ctypes.c_void_p()
        st = lib().rattn_pagepool_create(n_pages, ctypes.byref(h))
        if st:
            raise RattnError(st, "rattn_pagepool_create")
        self._h = h
        self.n_pages = n_pages

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.rattn_pagepool_destroy(self._h)
            self._h = None

    @staticmethod
    def _i32(pages):
        import numpy as np

        a = np.ascontiguousarray(pages, dtype=np.int32)
        return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def free_pages(self) -> int:
        return int(lib().rattn_pagepool_free_pages(self._h))

    def refcount(self, page: int) -> int:
        c = ctypes.c_int32()
        st = lib().rattn_pagepool_refcount(self._h, page, ctypes.byref(c))
        if st:
            raise RattnError(st, "rattn_pagepool_refcount")
        return c.value

    def refcounts(self):
        import numpy as np

        return np.array([self.refcount(p) for p in range(self.n_pages)], np.int64)

    def alloc(self, n: int):
        import numpy as np

        out = np.zeros(max(n, 1), np.int32)
        st = lib().rattn_pagepool_alloc(self._h, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        if st:
            raise RattnError(st, "rattn_pagepool_alloc")
        return out[:n]

    def retain(self, pages):
        a, p = self._i32(pages)
        st = lib().rattn_pagepool_retain(self._h, p, a.size)
        if st:
            raise RattnError(st, "rattn_pagepool_retain")

    def release(self, pages):
        a, p = self._i32(pages)
        st = lib().rattn_pagepool_release(self._h, p, a.size)
        if st:
            raise RattnError(st, "rattn_pagepool_release")

    def plan_append(self, table, cur_len: int, n_new: int, page_size: int):
        """Updates ``table`` (a contiguous int32 numpy array, the sequence's
        block table with room for the new pages) in place; returns the
        copy-on-write pair (cow_src, cow_dst), (-1, -1) without a copy."""
        import numpy as np

        if not (isinstance(table, np.ndarray) and table.dtype == np.int32 and table.flags["C_CONTIGUOUS"]):
            raise TypeError("table must be a contiguous int32 numpy array")
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        st = lib().rattn_pagepool_plan_append(self._h, table.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                              table.size, cur_len, n_new, page_size, ctypes.byref(src),
                                              ctypes.byref(dst))
        if st:
            raise RattnError(st, "rattn_pagepool_plan_append")
        return src.value, dst.value


def append_kv(pool_k, pool_v, table, cur_len: int, k_new, v_new, *, cow=(-1, -1), stream=None):
    """rattn_append_kv: writes k_new/v_new [H_kv, T, d] at logical positions
    cur_len .. cur_len + T - 1 of the sequence whose (updated) device block
    table is ``table``, and fills the copy-on-write page's kept rows."""
    import torch

    n_phys, HK, ps, D = pool_k.shape
    T = k_new.shape[1]
    dt = RATTN_BF16 if pool_k.dtype == torch.bfloat16 else RATTN_F32
    desc = make_desc(n_agents=1, n_q_heads=HK, n_kv_heads=HK, head_dim=D, rank=0, q_len=1, prefix_len=0,
                     page_size=ps, n_phys_pages=n_phys, dtype=dt)
    for name, t in dict(pool_k=pool_k, pool_v=pool_v, k_new=k_new, v_new=v_new).items():
        if not t.is_cuda or not t.is_contiguous() or t.dtype != pool_k.dtype:
            raise ValueError(f"{name} must be a contiguous GPU tensor of the pool's dtype")
    if tuple(pool_v.shape) != tuple(pool_k.shape) or tuple(k_new.shape) != (HK, T, D) or \
            tuple(v_new.shape) != (HK, T, D):
        raise ValueError("pool / new-row shapes disagree")
    if not (table.is_cuda and table.dtype == torch.int32 and table.numel() >= -(-(cur_len + T) // ps)):
        raise ValueError("table must be a GPU int32 tensor covering the new length")
    st = lib().rattn_append_kv(ctypes.byref(desc), pool_k.data_ptr(), pool_v.data_ptr(), table.data_ptr(), cur_len,
                               T, k_new.data_ptr(), v_new.data_ptr(), int(cow[0]), int(cow[1]), _stream(stream))
    if st:
        raise RattnError(st, "rattn_append_kv")


def gather_base(pool, block_table, prefix_len: int, *, out=None, stream=None):
    """rattn_gather_base: logical base cache [H_kv, L, d] from a paged pool."""
    import torch

    n_phys, HK, ps, D = pool.shape
    dt = RATTN_BF16 if pool.dtype == torch.bfloat16 else RATTN_F32
    desc = make_desc(n_agents=1, n_q_heads=HK, n_kv_heads=HK, head_dim=D, rank=0, q_len=1,
                     prefix_len=prefix_len, page_size=ps, n_phys_pages=n_phys, dtype=dt)
    if out is None:
        out = torch.empty((HK, prefix_len, D), device=pool.device, dtype=pool.dtype)
    _check_tensors(desc, dict(k_base=pool, block_table=block_table))
    st = lib().rattn_gather_base(ctypes.byref(desc), ctypes.c_void_p(pool.data_ptr()),
                                 ctypes.c_void_p(block_table.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                 _stream(stream))
    if st:
        raise RattnError(st, "rattn_gather_base")
    return out


def attend(inputs: dict, *, mode: str = "decode", shared_lr=None, prefix_len=None, out=None, lse=None,
           workspace=None, stream=None, desc=None, stages=None, k_scale=None):
    """Runs decode or prefill on a dict of device tensors named as in the layouts above.
    ``stages`` (a mask of STAGE_*) runs only those launches through rattn_attention_stages.
    A uint8 ``k_base`` holds int8 key codes with scale ``k_scale``; a uint8
    ``v_base`` holds 3-bit value codes with their scales in ``inputs["v_scale"]``."""
    if mode == "decode":
        fn_name, op = "rattn_decode", RATTN_OP_DECODE
    else:
        fn_name, op = "rattn_prefill_chunk", RATTN_OP_PREFILL
    g = inputs.get
    return _run(fn_name, op, inputs["q"], g("k_base"), g("v_base"), g("lk"), g("lv"), g("bk"), g("bv"),
                g("block_table"), g("k_priv"), g("v_priv"), shared_lr, out, lse, workspace, 0.0, prefix_len, stream,
                desc, stages, k_scale, g("v_scale"))

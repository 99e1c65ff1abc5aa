"""MI355X-native Kimi Delta Attention (KDA) forward path -- Python binding.

Thin ctypes binding over ``libkda.so`` (HIP, gfx950), whose C ABI is
declared in ``include/kda.h``.  The functions here only marshal arguments:
they check dtypes, shapes, devices and contiguity of torch tensors, allocate
outputs with torch when the caller does not pass them, and call the library
on the current torch stream.  Every arithmetic step runs in the library's
kernels; there is no fallback path -- a missing or unloadable library raises.

Entry points (same names as the C ABI, without the ``kda_`` prefix):
  qk_l2norm(x)                                    -> y
  chunk_prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None)
                                                  -> (o, final_state)
  chunk_prefill_split(...same...)                 -> (o, final_state)
  chunk_prefill_fused(...same...)                 -> (o, final_state)
  chunk_prefill_noalloc(...same...)               -> (o, final_state)
  prefill_partition(B, HV, num_seqs=0)            -> "split" | "fused"
  decode(q, k, v, g, beta, state_pool, state_indices)   -> o
  packed_decode(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_pool,
                state_indices)                    -> o
  state_to_pool(state, state_pool, state_indices)       -> state_pool
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
EXPORTS = ("kda_status_string", "kda_build_id", "kda_qk_l2norm", "kda_chunk_prefill", "kda_chunk_prefill_split",
           "kda_chunk_prefill_fused", "kda_chunk_prefill_noalloc", "kda_chunk_prefill_partition",
           "kda_chunk_prefill_workspace_size", "kda_prefill_overlap_wait_limit", "kda_decode", "kda_packed_decode",
           "kda_state_to_pool", "kda_chunk_backward", "kda_chunk_backward_workspace_size")

_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class KDAError(RuntimeError):
    pass


def load():
    """Load libkda.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KDAError(f"{LIB_PATH} not found; build it with `python -m kda_gated_delta_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_build_id.restype = ctypes.c_char_p
    lib.kda_build_id.argtypes = []
    lib.kda_qk_l2norm.restype = ctypes.c_int
    lib.kda_qk_l2norm.argtypes = [_vp, _vp, _i64, _i32, _vp]
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_chunk_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                      _vp, ctypes.c_size_t, _vp]
    lib.kda_chunk_prefill_split.restype = ctypes.c_int
    lib.kda_chunk_prefill_split.argtypes = lib.kda_chunk_prefill.argtypes
    lib.kda_chunk_prefill_partition.restype = ctypes.c_int
    lib.kda_chunk_prefill_partition.argtypes = [_i32, _i32, _i32]
    lib.kda_chunk_prefill_fused.restype = ctypes.c_int
    lib.kda_chunk_prefill_fused.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                            _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.kda_chunk_prefill_noalloc.restype = ctypes.c_int
    lib.kda_chunk_prefill_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                              _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.kda_chunk_prefill_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_prefill_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.kda_prefill_overlap_wait_limit.restype = _i32
    lib.kda_prefill_overlap_wait_limit.argtypes = [_i32]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                               _i32, _i32, _i32, _i32, _i32, _vp, _vp]
    lib.kda_packed_decode.restype = ctypes.c_int
    lib.kda_packed_decode.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                                      _i32, _i32, _i32, _i32, _vp, _vp]
    lib.kda_state_to_pool.restype = ctypes.c_int
    lib.kda_state_to_pool.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _i64, _i64, _vp, _vp]
    lib.kda_chunk_backward.restype = ctypes.c_int
    lib.kda_chunk_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                       _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, ctypes.c_size_t, _vp]
    lib.kda_chunk_backward_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_backward_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    _lib = lib
    return lib


def build_id():
    """Hash of the sources the loaded library was compiled from."""
    return load().kda_build_id().decode()


def check_build_matches_sources():
    """Raise unless the loaded libkda.so was built from the source files
    in this tree (their hash is compiled into the library)."""
    from .build import source_hash
    want, got = source_hash(), build_id()
    if want != got:
        raise KDAError(f"{LIB_PATH} was built from other sources (library {got}, tree {want}); rebuild it")
    return got


def status_string(code):
    return load().kda_status_string(int(code)).decode()


def _check(code, what):
    if code != 0:
        raise KDAError(f"{what}: {status_string(code)} (status {code})")


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def _need(t, name, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def qk_l2norm(x, out=None):
    """Bit-exact row normalisation of a bf16 tensor whose last dim is 128."""
    lib = load()
    _need(x, "x", torch.bfloat16)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, device=x.device)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    K = x.shape[-1]
    rows = x.numel() // K if K else 0
    _check(lib.kda_qk_l2norm(_ptr(x), _ptr(out), rows, K, _stream()), "kda_qk_l2norm")
    return out


def workspace_size(B, T, H, HV, num_seqs=0, K=128, V=128):
    """Bytes of workspace kda_chunk_prefill needs (num_seqs = 0 without cu_seqlens)."""
    return int(load().kda_chunk_prefill_workspace_size(B, T, H, HV, K, V, num_seqs))


def _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state):
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, T, H, K = q.shape
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 4, dev)
    HV, V = v.shape[2], v.shape[3]
    _need(g, "g", torch.float32, 4, dev)
    _need(beta, "beta", torch.bfloat16, 3, dev)
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, HV, K) \
            or beta.shape != (B, T, HV):
        raise ValueError("inconsistent shapes")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4, dev)
        if initial_state.shape != (N, HV, K, V):
            raise ValueError(f"initial_state must be {(N, HV, K, V)}")
    if out is None:
        out = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=dev)
    if final_state is None:
        final_state = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    _need(final_state, "final_state", torch.float32, 4, dev)
    nseq_arg = N if cu_seqlens is not None else 0
    return dev, (B, T, H, HV, K, V), nseq_arg, out, final_state


def prefill_overlap_wait_limit(polls):
    """Testing hook (kda_prefill_overlap_wait_limit): polls the overlapped
    schedule's carry makes for one ready flag before it leaves the unit to
    the sequential carry; 0 forces that path, negative restores the default.
    Returns the previous value."""
    return int(load().kda_prefill_overlap_wait_limit(int(polls)))


PREFILL_SLOT_BYTES = 66048   # kda.h KDA_PREFILL_SLOT_BYTES: the smallest workspace is HV of these


def prefill_partition(B, HV, num_seqs=0):
    """The form chunk_prefill runs for these sizes on the current device:
    "split" or "fused" (num_seqs = 0 without cu_seqlens)."""
    code = int(load().kda_chunk_prefill_partition(B, HV, num_seqs))
    if code < 0:
        _check(-code, "kda_chunk_prefill_partition")
    return ("split", "fused")[code]


def _prefill_with_workspace(entry, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, workspace):
    lib = load()
    dev, (B, T, H, HV, K, V), nseq_arg, out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    if workspace is None:
        if entry == "kda_chunk_prefill" and prefill_partition(B, HV, nseq_arg) == "fused":
            need = HV * PREFILL_SLOT_BYTES     # checked, never touched by the fused form
        else:
            need = workspace_size(B, T, H, HV, nseq_arg, K, V)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    code = getattr(lib, entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(initial_state), _ptr(cu_seqlens), nseq_arg,
                               B, T, H, HV, K, V, _ptr(out), _ptr(final_state),
                               _ptr(workspace), workspace.numel(), _stream())
    _check(code, entry)
    return out, final_state


def chunk_prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                  out=None, final_state=None, workspace=None):
    """KDA prefill.  q, k [B,T,H,K] bf16; v [B,T,HV,V] bf16; g [B,T,HV,K]
    fp32; beta [B,T,HV] bf16; initial_state [N,HV,K,V] fp32 or None;
    cu_seqlens int32 [N+1] (with B == 1) or None; workspace: a uint8 GPU
    tensor, or None to allocate one (workspace_size(...) bytes, the fastest
    size for the split form; any size from HV * PREFILL_SLOT_BYTES up is
    accepted, the split form then running in more windows).  The library
    picks the split or the fused form (prefill_partition); both give the same
    result bit for bit.  The fused form does not touch the workspace, so for
    it only the minimum is allocated.
    Returns (o, final_state)."""
    return _prefill_with_workspace("kda_chunk_prefill", q, k, v, g, beta, initial_state, cu_seqlens,
                                   out, final_state, workspace)


def chunk_prefill_split(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                        out=None, final_state=None, workspace=None):
    """chunk_prefill in the split form whatever the sizes (workspace-backed
    chunk-parallel kernel plus carry kernel).  Arguments and result as
    chunk_prefill."""
    return _prefill_with_workspace("kda_chunk_prefill_split", q, k, v, g, beta, initial_state, cu_seqlens,
                                   out, final_state, workspace)


def backward_workspace_size(B, T, H, HV, num_seqs=0, K=128, V=128):
    """Bytes of workspace kda_chunk_backward needs (num_seqs = 0 without cu_seqlens)."""
    return int(load().kda_chunk_backward_workspace_size(B, T, H, HV, K, V, num_seqs))


GRAD_FLOAT32 = 0       # kda.h KDA_GRAD_FLOAT32
GRAD_INPUT_DTYPE = 1   # kda.h KDA_GRAD_INPUT_DTYPE


def chunk_backward(q, k, v, g, beta, initial_state, d_out, d_final_state=None, cu_seqlens=None,
                   workspace=None, grad_dtype="input", want_d_initial_state=False):
    """Gradients of sum(o * d_out) + sum(final_state * d_final_state) for
    the prefill with the same inputs.  d_out [B,T,HV,V] bf16; d_final_state
    [N,HV,K,V] fp32 or None (zero).  Returns (dq, dk, dv, dg, dbeta,
    d_initial_state).

    grad_dtype "input" (default): every gradient has its input's dtype --
    dq, dk, dv, dbeta bf16 (the kernels round their float32 values to
    nearest-even), dg and d_initial_state float32.  grad_dtype "float32":
    dq, dk, dv, dbeta float32 as well.  d_initial_state is None when
    initial_state is None, unless want_d_initial_state asks for the
    gradient at a zero initial state."""
    lib = load()
    if grad_dtype not in ("input", "float32"):
        raise ValueError("grad_dtype must be 'input' or 'float32'")
    dev, (B, T, H, HV, K, V), nseq_arg, _, _ = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens, None, None)
    N = nseq_arg if cu_seqlens is not None else B
    _need(d_out, "d_out", torch.bfloat16, 4, dev)
    if d_out.shape != (B, T, HV, V):
        raise ValueError(f"d_out must be {(B, T, HV, V)}")
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", torch.float32, 4, dev)
        if d_final_state.shape != (N, HV, K, V):
            raise ValueError(f"d_final_state must be {(N, HV, K, V)}")
    need = backward_workspace_size(B, T, H, HV, nseq_arg, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    tok = dict(dtype=torch.bfloat16 if grad_dtype == "input" else torch.float32, device=dev)
    dq = torch.empty((B, T, H, K), **tok)
    dk = torch.empty((B, T, H, K), **tok)
    dv = torch.empty((B, T, HV, V), **tok)
    dg = torch.empty((B, T, HV, K), **f32)
    dbeta = torch.empty((B, T, HV), **tok)
    dh0 = torch.empty((N, HV, K, V), **f32) if (initial_state is not None or want_d_initial_state) else None
    code = lib.kda_chunk_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(initial_state), _ptr(cu_seqlens), nseq_arg,
                                  B, T, H, HV, K, V, _ptr(d_out), _ptr(d_final_state),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                  GRAD_INPUT_DTYPE if grad_dtype == "input" else GRAD_FLOAT32,
                                  _ptr(workspace), workspace.numel(), _stream())
    _check(code, "kda_chunk_backward")
    return dq, dk, dv, dg, dbeta, dh0


NOALLOC_WORKSPACE_BYTES = 64 << 20   # kda.h KDA_NOALLOC_WORKSPACE_BYTES


def chunk_prefill_noalloc(q, k, v, g, beta, initial_state=None, cu_seqlens=None, out=None,
                          final_state=None):
    """kda_chunk_prefill_noalloc: the prefill with the library's static
    64 MiB workspace (no workspace argument, nothing allocated by the
    library).  Pass out and final_state to allocate nothing here either.
    Sizes whose workspace exceeds the static one raise (KDA_ERR_WORKSPACE).
    Calls that overlap on one GPU race."""
    lib = load()
    dev, (B, T, H, HV, K, V), nseq_arg, out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    code = lib.kda_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(initial_state), _ptr(cu_seqlens), nseq_arg,
                                         B, T, H, HV, K, V, _ptr(out), _ptr(final_state), _stream())
    _check(code, "kda_chunk_prefill_noalloc")
    return out, final_state


def chunk_prefill_fused(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                        out=None, final_state=None):
    """The same prefill in the fused partition (one workgroup per sequence
    and value head, no workspace).  Arguments and result as chunk_prefill."""
    lib = load()
    dev, (B, T, H, HV, K, V), nseq_arg, out, final_state = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    code = lib.kda_chunk_prefill_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(initial_state), _ptr(cu_seqlens), nseq_arg,
                                       B, T, H, HV, K, V, _ptr(out), _ptr(final_state), _stream())
    _check(code, "kda_chunk_prefill_fused")
    return out, final_state


def decode(q, k, v, g, beta, state_pool, state_indices, out=None):
    """One decode step.  q, k [B,H,K] (or [B,1,H,K]) bf16; v [B,HV,V] bf16;
    g [B,HV,K] fp32; beta [B,HV] bf16; state_pool bf16 [N,HV,K,V] (outer
    stride may be padded, inner dims compact), updated in place;
    state_indices int32 [B].  Returns o [B,1,HV,V] bf16."""
    lib = load()
    if q.dim() == 4:
        q, k, v, g, beta = q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0]
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    B, H, K = q.shape
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    HV, V = v.shape[1], v.shape[2]
    _need(g, "g", torch.float32, 3, dev)
    _need(beta, "beta", torch.bfloat16, 2, dev)
    _need(state_indices, "state_indices", torch.int32, 1, dev)
    if state_pool.dtype != torch.bfloat16 or not state_pool.is_cuda or state_pool.device != dev:
        raise TypeError("state_pool must be a bf16 GPU tensor on q's device")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (HV, K, V):
        raise ValueError(f"state_pool must be [N,{HV},{K},{V}]")
    if state_pool.stride()[1:] != (K * V, V, 1):
        raise ValueError("state_pool inner dims must be compact")
    if out is None:
        out = torch.empty((B, 1, HV, V), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    code = lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                          _ptr(state_pool), state_pool.stride(0), state_pool.shape[0],
                          _ptr(state_indices), B, H, HV, K, V, _ptr(out), _stream())
    _check(code, "kda_decode")
    return out


def state_to_pool(state, state_pool, state_indices):
    """Prefill-to-decode handoff: state fp32 [N,HV,K,V] (e.g. a prefill's
    final_state) is stored, rounded to bf16, into state_pool bf16
    [slots,HV,K,V] (outer stride may be padded, inner dims compact) at slot
    state_indices[n] (int32 [N]; -1 or out of range skips the state).
    Updates state_pool in place and returns it."""
    lib = load()
    _need(state, "state", torch.float32, 4)
    dev = state.device
    N, HV, K, V = state.shape
    _need(state_indices, "state_indices", torch.int32, 1, dev)
    if state_indices.shape[0] != N:
        raise ValueError(f"state_indices must have {N} entries")
    if state_pool.dtype != torch.bfloat16 or not state_pool.is_cuda or state_pool.device != dev:
        raise TypeError("state_pool must be a bf16 GPU tensor on state's device")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (HV, K, V):
        raise ValueError(f"state_pool must be [slots,{HV},{K},{V}]")
    if state_pool.stride()[1:] != (K * V, V, 1):
        raise ValueError("state_pool inner dims must be compact")
    code = lib.kda_state_to_pool(_ptr(state), N, HV, K, V, _ptr(state_pool), state_pool.stride(0),
                                 state_pool.shape[0], _ptr(state_indices), _stream())
    _check(code, "kda_state_to_pool")
    return state_pool


def packed_decode(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_pool, state_indices, out=None):
    """One decode step from packed serving inputs.  mixed_qkv bf16 [B, 3*H*K]
    (rows q | k | v; row stride may be padded to a multiple of 8, last dim
    contiguous); raw_gate bf16 [B, H*K]; raw_beta bf16 [B, H]; A_log fp32
    [H]; dt_bias fp32 [H*K]; state_pool bf16 [N,H,K,V] updated in place;
    state_indices int32 [B].  Returns o [B,1,H,V] bf16."""
    lib = load()
    if not isinstance(mixed_qkv, torch.Tensor) or mixed_qkv.dtype != torch.bfloat16 or not mixed_qkv.is_cuda:
        raise TypeError("mixed_qkv must be a bf16 GPU tensor")
    if mixed_qkv.dim() != 2 or mixed_qkv.stride(1) != 1:
        raise ValueError("mixed_qkv must be [B, 3*H*K] with a contiguous last dim")
    dev = mixed_qkv.device
    _need(A_log, "A_log", torch.float32, 1, dev)
    H = A_log.shape[0]
    B = mixed_qkv.shape[0]
    K = V = 128
    if mixed_qkv.shape[1] != 3 * H * K:
        raise ValueError(f"mixed_qkv rows must hold 3*{H}*{K} elements")
    _need(raw_gate, "raw_gate", torch.bfloat16, 2, dev)
    _need(raw_beta, "raw_beta", torch.bfloat16, 2, dev)
    _need(dt_bias, "dt_bias", torch.float32, 1, dev)
    _need(state_indices, "state_indices", torch.int32, 1, dev)
    if tuple(raw_gate.shape) != (B, H * K) or tuple(raw_beta.shape) != (B, H) or dt_bias.shape[0] != H * K:
        raise ValueError("raw_gate [B,H*K], raw_beta [B,H], dt_bias [H*K] expected")
    if state_pool.dtype != torch.bfloat16 or not state_pool.is_cuda or state_pool.device != dev:
        raise TypeError("state_pool must be a bf16 GPU tensor on mixed_qkv's device")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, K, V):
        raise ValueError(f"state_pool must be [N,{H},{K},{V}]")
    if state_pool.stride()[1:] != (K * V, V, 1):
        raise ValueError("state_pool inner dims must be compact")
    if out is None:
        out = torch.empty((B, 1, H, V), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    row_stride = mixed_qkv.stride(0) if B > 1 else 3 * H * K
    code = lib.kda_packed_decode(_ptr(mixed_qkv), row_stride, _ptr(raw_gate), _ptr(raw_beta), _ptr(A_log),
                                 _ptr(dt_bias), _ptr(state_pool), state_pool.stride(0), state_pool.shape[0],
                                 _ptr(state_indices), B, H, K, V, _ptr(out), _stream())
    _check(code, "kda_packed_decode")
    return out

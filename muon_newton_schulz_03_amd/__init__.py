"""Python binding of libmuon.so, the MI355X (gfx950) Muon optimizer-step library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/muon.h. The functions here carry
the C names; torch tensors supply device pointers, shapes and the current
stream. There is no CPU fallback: if the library is missing, every call
raises.
"""
import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon.so")

MUON_OK = 0
STATUS_NAMES = {
    0: "MUON_OK", 1: "MUON_ERR_INVALID_ARG", 2: "MUON_ERR_SHAPE", 3: "MUON_ERR_DTYPE",
    4: "MUON_ERR_ALIGN", 5: "MUON_ERR_ALIAS", 6: "MUON_ERR_WORKSPACE", 7: "MUON_ERR_HIP",
}
MUON_ERR_INVALID_ARG = 1
MUON_ERR_SHAPE = 2
MUON_ERR_DTYPE = 3
MUON_ERR_ALIGN = 4
MUON_ERR_ALIAS = 5
MUON_ERR_WORKSPACE = 6
MUON_ERR_HIP = 7
MUON_F32 = 0
MUON_BF16 = 1

MUON_NS_FULL = 0x000
MUON_NS_BLOCKWISE = 0x001
MUON_NS_DISTRIBUTED = 0x002
MUON_PACK_RR = 0x000
MUON_PACK_COST = 0x010
MUON_PLACE_RR = 0
MUON_PLACE_LPT = 1
MUON_AA_PLAIN = 0x000
MUON_AA_SPLIT = 0x100

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
DEFAULT_MODE = MUON_NS_FULL | MUON_PACK_COST | MUON_AA_PLAIN

EXPORTED = (
    "muon_ns_batched", "muon_step", "muon_set_stream", "muon_workspace_size",
    "muon_workspace_min_size", "muon_set_workspace", "muon_set_step_options",
    "muon_last_error", "muon_plan_info", "muon_set_phase_timing", "muon_phase_times",
    "muon_place", "muon_adamw_step", "muon_step_noalloc",
)
MUON_NOALLOC_SCRATCH_BYTES = 256 << 20
PHASES = ("prep", "norm", "gram", "aa", "bx", "finish", "adamw", "reduce")


class MuonError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class muon_mat(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("ld", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("col_blocks", ctypes.c_int32),
    ]


_lib = None


def load_library(path=LIB_PATH):
    """Load libmuon.so (built by build.py). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -m muon_newton_schulz_03_amd.build")
    lib = ctypes.CDLL(path)
    mat_p = ctypes.POINTER(muon_mat)
    f3 = ctypes.POINTER(ctypes.c_float)
    sz = ctypes.POINTER(ctypes.c_size_t)
    sigs = {
        "muon_ns_batched": ([mat_p, ctypes.c_int32, ctypes.c_int32, f3, ctypes.c_uint32], ctypes.c_int),
        "muon_step": ([mat_p, mat_p, mat_p, ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_int32],
                      ctypes.c_int),
        "muon_step_noalloc": ([mat_p, mat_p, mat_p, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                               ctypes.c_int32], ctypes.c_int),
        "muon_set_stream": ([ctypes.c_void_p], ctypes.c_int),
        "muon_workspace_size": ([mat_p, ctypes.c_int32, ctypes.c_uint32, sz], ctypes.c_int),
        "muon_workspace_min_size": ([mat_p, ctypes.c_int32, ctypes.c_uint32, sz], ctypes.c_int),
        "muon_set_workspace": ([ctypes.c_void_p, ctypes.c_size_t], ctypes.c_int),
        "muon_set_step_options": ([ctypes.c_int32, f3, ctypes.c_float, ctypes.c_uint32], ctypes.c_int),
        "muon_last_error": ([], ctypes.c_char_p),
        "muon_plan_info": ([mat_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t,
                            ctypes.c_char_p, ctypes.c_size_t, sz], ctypes.c_int),
        "muon_set_phase_timing": ([ctypes.c_int32], ctypes.c_int),
        "muon_phase_times": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
        "muon_adamw_step": ([mat_p, mat_p, mat_p, mat_p, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                             ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int32], ctypes.c_int),
        "muon_place": ([ctypes.POINTER(ctypes.c_double), ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                        ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def lib():
    return load_library()


def muon_last_error():
    return lib().muon_last_error().decode()


def _check(status):
    if status != MUON_OK:
        raise MuonError(status, muon_last_error())


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return MUON_F32
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def mat_of(t, col_blocks=1):
    """Descriptor of a 2-D row-major device tensor (unit column stride)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("expected unit column stride")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    ld = max(ld, t.shape[1])
    return muon_mat(ctypes.c_void_p(t.data_ptr()), t.shape[0], t.shape[1], ld, _dtype_code(t), col_blocks)


def mats(descs):
    """Pack a list of muon_mat (or raw tuples) into a C array."""
    arr = (muon_mat * max(len(descs), 1))()
    for i, d in enumerate(descs):
        arr[i] = d
    return arr


def _coeffs(c):
    if c is None:
        return None
    return (ctypes.c_float * 3)(*[float(x) for x in c])


# ---------------------------------------------------------------------------
# C entry points (same names, raw descriptors)
# ---------------------------------------------------------------------------

def muon_set_stream(stream=None):
    """stream: a torch.cuda.Stream, a raw hipStream_t integer, or None for
    torch's current stream."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _check(lib().muon_set_stream(ctypes.c_void_p(handle)))


def muon_set_workspace(ptr, nbytes):
    _check(lib().muon_set_workspace(ctypes.c_void_p(ptr), ctypes.c_size_t(nbytes)))


def muon_workspace_size(descs, mode=DEFAULT_MODE):
    out = ctypes.c_size_t()
    _check(lib().muon_workspace_size(mats(descs), len(descs), mode, ctypes.byref(out)))
    return out.value


def muon_workspace_min_size(descs, mode=DEFAULT_MODE):
    out = ctypes.c_size_t()
    _check(lib().muon_workspace_min_size(mats(descs), len(descs), mode, ctypes.byref(out)))
    return out.value


def muon_set_step_options(iters=5, coeffs=DEFAULT_COEFFS, eps=1e-7, mode=DEFAULT_MODE):
    _check(lib().muon_set_step_options(iters, _coeffs(coeffs), eps, mode))


def muon_plan_info(descs, iters=5, mode=DEFAULT_MODE, workspace_bytes=0):
    need = ctypes.c_size_t()
    arr = mats(descs)
    _check(lib().muon_plan_info(arr, len(descs), iters, mode, workspace_bytes, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check(lib().muon_plan_info(arr, len(descs), iters, mode, workspace_bytes, buf, need.value,
                                ctypes.byref(need)))
    return json.loads(buf.value.decode())


def muon_set_phase_timing(enable=True):
    _check(lib().muon_set_phase_timing(1 if enable else 0))


def muon_phase_times():
    """{kind: (milliseconds, launches)} since the last query (see muon.h)."""
    ms = (ctypes.c_double * len(PHASES))()
    n = (ctypes.c_int64 * len(PHASES))()
    _check(lib().muon_phase_times(ms, n))
    return {k: (ms[i], n[i]) for i, k in enumerate(PHASES)}


def muon_place(costs, ranks, policy="lpt"):
    """Place matrices with the given costs on `ranks` ranks (see muon.h).
    Returns (owner list, per-rank load list, max/mean imbalance)."""
    n = len(costs)
    c = (ctypes.c_double * max(n, 1))(*[float(x) for x in costs])
    owner = (ctypes.c_int32 * max(n, 1))()
    load = (ctypes.c_double * ranks)()
    imb = ctypes.c_double()
    pol = {"rr": MUON_PLACE_RR, "lpt": MUON_PLACE_LPT}[policy] if isinstance(policy, str) else policy
    _check(lib().muon_place(c, n, ranks, pol, owner, load, ctypes.byref(imb)))
    return list(owner[:n]), list(load), imb.value


# ---------------------------------------------------------------------------
# tensor-level wrappers
# ---------------------------------------------------------------------------

class Workspace:
    """A caller-owned workspace (a torch uint8 buffer) set for this thread."""

    def __init__(self, nbytes, device="cuda"):
        import torch
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)
        muon_set_workspace(self.buf.data_ptr(), self.nbytes)


_ws = None


def ensure_workspace(descs, mode=DEFAULT_MODE, max_bytes=None):
    """Make sure this thread has a workspace large enough for the call:
    everything in flight when it fits under max_bytes, else at least one
    matrix."""
    global _ws
    full = muon_workspace_size(descs, mode)
    want = full
    if max_bytes is not None and full > max_bytes:
        want = max(muon_workspace_min_size(descs, mode), int(max_bytes))
    if _ws is None or _ws.nbytes < want:
        _ws = None
        _ws = Workspace(want)
    else:
        muon_set_workspace(_ws.buf.data_ptr(), _ws.nbytes)
    return _ws


def muon_ns_batched(tensors, iters=5, coeffs=DEFAULT_COEFFS, mode=DEFAULT_MODE, col_blocks=None,
                    workspace=None, max_workspace_bytes=None):
    """Orthogonalize each 2-D device tensor in place (see muon.h)."""
    cb = col_blocks if col_blocks is not None else [1] * len(tensors)
    if isinstance(cb, int):
        cb = [cb] * len(tensors)
    descs = [mat_of(t, c) for t, c in zip(tensors, cb)]
    muon_set_stream(None)
    if workspace is None:
        if descs:
            ensure_workspace(descs, mode, max_workspace_bytes)
    else:
        muon_set_workspace(workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _check(lib().muon_ns_batched(mats(descs), len(descs), iters, _coeffs(coeffs), mode))


def muon_step(params, grads, moms, lr=0.02, beta=0.95, nesterov=False, iters=5, coeffs=DEFAULT_COEFFS,
              eps=1e-7, mode=DEFAULT_MODE, col_blocks=None, workspace=None, max_workspace_bytes=None):
    """One Muon step over lists of 2-D device tensors; params and moms are
    updated in place (see muon.h)."""
    cb = col_blocks if col_blocks is not None else [1] * len(params)
    if isinstance(cb, int):
        cb = [cb] * len(params)
    W = [mat_of(t, c) for t, c in zip(params, cb)]
    G = [mat_of(t) for t in grads]
    M = [mat_of(t) for t in moms]
    muon_set_stream(None)
    muon_set_step_options(iters, coeffs, eps, mode)
    if workspace is None:
        if W:
            ensure_workspace(W, mode, max_workspace_bytes)
    else:
        muon_set_workspace(workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _check(lib().muon_step(mats(W), mats(G), mats(M), len(W), lr, beta, 1 if nesterov else 0))


def muon_step_noalloc(params, grads, moms, lr=0.02, beta=0.95, nesterov=False, iters=5,
                      coeffs=DEFAULT_COEFFS, eps=1e-7, mode=DEFAULT_MODE, col_blocks=None):
    """muon_step with the library's device scratch instead of a workspace
    (see muon.h): no device memory is allocated by the library or here."""
    cb = col_blocks if col_blocks is not None else [1] * len(params)
    if isinstance(cb, int):
        cb = [cb] * len(params)
    W = [mat_of(t, c) for t, c in zip(params, cb)]
    G = [mat_of(t) for t in grads]
    M = [mat_of(t) for t in moms]
    muon_set_stream(None)
    muon_set_step_options(iters, coeffs, eps, mode)
    _check(lib().muon_step_noalloc(mats(W), mats(G), mats(M), len(W), lr, beta, 1 if nesterov else 0))


def muon_adamw_step(params, grads, exp_avg, exp_avg_sq, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                    weight_decay=0.0, step=1):
    """One AdamW step over lists of 2-D device tensors (see muon.h): params
    (bf16 or float32) and the float32 moments are updated in place."""
    W = [mat_of(t) for t in params]
    G = [mat_of(t) for t in grads]
    Mo = [mat_of(t) for t in exp_avg]
    V = [mat_of(t) for t in exp_avg_sq]
    muon_set_stream(None)
    _check(lib().muon_adamw_step(mats(W), mats(G), mats(Mo), mats(V), len(W), lr, beta1, beta2, eps,
                                 weight_decay, step))

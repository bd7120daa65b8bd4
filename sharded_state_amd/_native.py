"""ctypes declarations of libfsdp_shard.so (the C ABI in include/fsdp_shard.h).

The library is built in-tree by ``sharded_state_amd/build.py`` (or
``__graft_entry__.build()``).  There is no fallback: if the library is missing
or fails to load, every entry point raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsdp_shard.so")

F32, F16, BF16 = 0, 1, 2
OK, E_INVAL, E_DTYPE, E_SIZE, E_ALIAS, E_HIP, E_IO, E_FORMAT = 0, -1, -2, -3, -4, -5, -6, -7
MAX_WORLD = 128
ABI_VERSION = 9
OFFLOAD_SCRATCH_BYTES = 32 << 20
OPT_ADAMW, OPT_SGD, OPT_ADAMAX, OPT_ADADELTA = 0, 1, 2, 3


class AdamWHP(ctypes.Structure):
    """fsdp_adamw_hp: one hyper-parameter set per flat unit."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64)]

    def __init__(self, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1):
        super().__init__(lr, beta1, beta2, eps, weight_decay, step)

    def __repr__(self):
        return ("AdamWHP(lr=%g, beta1=%g, beta2=%g, eps=%g, weight_decay=%g, step=%d)"
                % (self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, self.step))


class OptimHP(ctypes.Structure):
    """fsdp_optim_hp: a pointwise optimizer and its hyper-parameters (use the
    constructors sgd / adamax / adadelta / adamw; defaults are torch.optim's,
    with lr 1e-3 for SGD)."""
    _fields_ = [("kind", ctypes.c_int), ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("momentum", ctypes.c_float), ("dampening", ctypes.c_float), ("rho", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("step", ctypes.c_int64)]

    @classmethod
    def sgd(cls, lr=1e-3, momentum=0.0, dampening=0.0, weight_decay=0.0, nesterov=False, step=1):
        return cls(OPT_SGD, lr, weight_decay, 0.0, 0.0, 0.0, momentum, dampening, 0.0, int(bool(nesterov)), step)

    @classmethod
    def adamax(cls, lr=2e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, step=1):
        return cls(OPT_ADAMAX, lr, weight_decay, betas[0], betas[1], eps, 0.0, 0.0, 0.0, 0, step)

    @classmethod
    def adadelta(cls, lr=1.0, rho=0.9, eps=1e-6, weight_decay=0.0, step=1):
        return cls(OPT_ADADELTA, lr, weight_decay, 0.0, 0.0, eps, 0.0, 0.0, rho, 0, step)

    @classmethod
    def adamw(cls, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, step=1):
        return cls(OPT_ADAMW, lr, weight_decay, betas[0], betas[1], eps, 0.0, 0.0, 0.0, 0, step)

    @property
    def n_states(self):
        """State buffers the optimizer keeps (exp_avg, then exp_avg_sq)."""
        if self.kind == OPT_SGD:
            return 1 if self.momentum != 0.0 else 0
        return 2

    @property
    def name(self):
        return {OPT_ADAMW: "adamw", OPT_SGD: "sgd", OPT_ADAMAX: "adamax", OPT_ADADELTA: "adadelta"}[self.kind]

    def at_step(self, step):
        c = OptimHP()
        ctypes.pointer(c)[0] = self
        c.step = step
        return c

    def __repr__(self):
        return "OptimHP(%s, lr=%g, wd=%g, step=%d)" % (self.name, self.lr, self.weight_decay, self.step)


class View(ctypes.Structure):
    """fsdp_view"""
    _fields_ = [("offset", ctypes.c_int64), ("numel", ctypes.c_int64)]


class Unit(ctypes.Structure):
    """fsdp_unit: one unit of a batched step."""
    _fields_ = [("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("rank_grads", ctypes.POINTER(ctypes.c_void_p)),
                ("peer_shards", ctypes.POINTER(ctypes.c_void_p)), ("full_out", ctypes.c_void_p),
                ("compute_shard", ctypes.c_void_p), ("shard_numel", ctypes.c_int64)]


class OffloadUnit(ctypes.Structure):
    """fsdp_offload_unit: one unit of an offloaded step."""
    _fields_ = [("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("rank_grads", ctypes.POINTER(ctypes.c_void_p)), ("grad_shard_dev", ctypes.c_void_p),
                ("grad_shard_host", ctypes.c_void_p), ("compute_host", ctypes.c_void_p),
                ("compute_dev", ctypes.c_void_p), ("shard_numel", ctypes.c_int64)]


class CkptInfo(ctypes.Structure):
    """fsdp_ckpt_info: header of a shard file."""
    _fields_ = [("world", ctypes.c_int32), ("rank", ctypes.c_int32), ("numel", ctypes.c_int64),
                ("padded_numel", ctypes.c_int64), ("shard_numel", ctypes.c_int64), ("state_dt", ctypes.c_int),
                ("compute_dt", ctypes.c_int), ("step", ctypes.c_int64), ("hp", AdamWHP),
                ("n_tensors", ctypes.c_int32)]


class FsdpError(RuntimeError):
    def __init__(self, func, code, msg):
        super().__init__("%s failed (status %d): %s" % (func, code, msg))
        self.code = code


_lib = None


def lib():
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfsdp_shard.so not found at %s: build it first with "
                          "`python -c 'import __graft_entry__ as g; g.build()'` or "
                          "`python sharded_state_amd/build.py`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    vpp = ctypes.POINTER(ctypes.c_void_p)
    i64p = ctypes.POINTER(ctypes.c_int64)
    L.fsdp_abi_version.restype = ctypes.c_int
    L.fsdp_abi_version.argtypes = []
    L.fsdp_last_error.restype = ctypes.c_char_p
    L.fsdp_last_error.argtypes = []
    L.fsdp_time_next_launch.restype = ctypes.c_int
    L.fsdp_time_next_launch.argtypes = [vp, vp]
    L.fsdp_unit_gather_split.restype = ctypes.c_int
    L.fsdp_unit_gather_split.argtypes = [i32, i32, i64]
    L.fsdp_units_in_launch.restype = ctypes.c_int
    L.fsdp_units_in_launch.argtypes = [i32, i64p, i32, i64p]
    L.fsdp_layout.restype = ctypes.c_int
    L.fsdp_layout.argtypes = [i64p, i32, i32, i64p, i64p, i64p]
    L.fsdp_flatten_pad.restype = ctypes.c_int
    L.fsdp_flatten_pad.argtypes = [vpp, i64p, i32, ctypes.c_int, i32, vp, i64, i64p, vp]
    L.fsdp_reduce_scatter_local.restype = ctypes.c_int
    L.fsdp_reduce_scatter_local.argtypes = [vpp, i32, i32, i64, ctypes.c_int, i32, vp, vp]
    L.fsdp_sharded_adamw.restype = ctypes.c_int
    L.fsdp_sharded_adamw.argtypes = [vp, vp, vp, vpp, i32, i32, ctypes.c_int, i32, vp, ctypes.c_int,
                                     i64, ctypes.POINTER(AdamWHP), vp]
    L.fsdp_step_unit.restype = ctypes.c_int
    L.fsdp_step_unit.argtypes = [vp, vp, vp, vpp, i32, i32, ctypes.c_int, i32, vpp, vp, ctypes.c_int,
                                 i64, vp, ctypes.POINTER(AdamWHP), vp]
    L.fsdp_step_units.restype = ctypes.c_int
    L.fsdp_step_units.argtypes = [ctypes.POINTER(Unit), i32, i32, i32, ctypes.c_int, i32, ctypes.c_int,
                                  ctypes.c_int, ctypes.POINTER(AdamWHP), vp]
    L.fsdp_step_units_optim.restype = ctypes.c_int
    L.fsdp_step_units_optim.argtypes = [ctypes.POINTER(Unit), i32, i32, i32, ctypes.c_int, i32, ctypes.c_int,
                                        ctypes.c_int, ctypes.POINTER(OptimHP), vp]
    L.fsdp_unshard_gather.restype = ctypes.c_int
    L.fsdp_unshard_gather.argtypes = [vpp, i32, i64, ctypes.c_int, vp, vp]
    L.fsdp_unflatten_views.restype = ctypes.c_int
    L.fsdp_unflatten_views.argtypes = [i64p, i32, i64, ctypes.POINTER(View), vp, ctypes.c_int, vpp, vp]
    L.fsdp_crc32c.restype = ctypes.c_uint32
    L.fsdp_crc32c.argtypes = [vp, i64]
    L.fsdp_save_shard.restype = ctypes.c_int
    L.fsdp_save_shard.argtypes = [ctypes.c_char_p, ctypes.POINTER(CkptInfo), i64p, vp, vp, vp, i32, vp]
    L.fsdp_shard_info.restype = ctypes.c_int
    L.fsdp_shard_info.argtypes = [ctypes.c_char_p, ctypes.POINTER(CkptInfo), i64p, i32]
    L.fsdp_load_shard.restype = ctypes.c_int
    L.fsdp_load_shard.argtypes = [ctypes.c_char_p, ctypes.POINTER(CkptInfo), vp, vp, vp, i64, i32, vp]
    L.fsdp_host_adamw.restype = ctypes.c_int
    L.fsdp_host_adamw.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, i64, ctypes.POINTER(AdamWHP), i32]
    L.fsdp_offload_step.restype = ctypes.c_int
    L.fsdp_offload_step.argtypes = [vp, vp, vp, vpp, i32, i32, ctypes.c_int, i32, vp, vp, vp, vp, ctypes.c_int,
                                    i64, i64, ctypes.POINTER(AdamWHP), i32, vp, vp]
    L.fsdp_offload_step_units.restype = ctypes.c_int
    L.fsdp_offload_step_units.argtypes = [ctypes.POINTER(OffloadUnit), i32, i32, i32, ctypes.c_int, i32,
                                          ctypes.c_int, i64, ctypes.POINTER(AdamWHP), i32, vp, vp]
    L.fsdp_offload_step_units_noalloc.restype = ctypes.c_int
    L.fsdp_offload_step_units_noalloc.argtypes = L.fsdp_offload_step_units.argtypes
    v = L.fsdp_abi_version()
    if v != ABI_VERSION:
        raise ImportError("libfsdp_shard.so ABI version %d, binding expects %d" % (v, ABI_VERSION))
    _lib = L
    return L


def check(func, code):
    if code != OK:
        raise FsdpError(func, code, lib().fsdp_last_error().decode(errors="replace"))


def ptr_array(ptrs):
    return (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)


def i64_array(vals):
    return (ctypes.c_int64 * max(len(vals), 1))(*[int(v) for v in vals])

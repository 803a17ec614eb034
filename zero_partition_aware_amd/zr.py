"""ctypes binding of libzr.so (the C ABI in include/zr.h).

Argument marshalling only: every function here turns Python/torch arguments
into the plain pointers and sizes of the C call of the same name, calls it,
and raises ``ZrError`` with the library's message when the status is not
ZR_OK.  No step of the computation happens in Python, and there is no
fallback: if the library is missing the import fails.
"""

import ctypes
import operator
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzr.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built: run `python -m zero_partition_aware_amd.build`")

# torch ships its own HIP runtime under the same soname as ROCm's.  Import it
# first so that the library binds to the runtime torch already holds: two HIP
# runtimes in one process do not share devices, streams or memory.
try:
    import torch  # noqa: F401
except ImportError:
    torch = None
_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_loaded():
    try:
        with open("/proc/self/maps") as fh:
            return sorted({ln.split()[-1] for ln in fh
                           if "libamdhip64" in ln and "/" in ln})
    except OSError:
        return []


if len(_hip_runtimes_loaded()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process "
                      f"({_hip_runtimes_loaded()}); import torch before any "
                      "other HIP library")

ZR_OK, ZR_ERR_INVALID, ZR_ERR_OOM, ZR_ERR_HIP, ZR_ERR_UNSUPPORTED = range(5)
ZR_FP32, ZR_BF16 = 0, 1
ZR_MAX_WORLD = 64
STATUS_NAMES = {0: "ZR_OK", 1: "ZR_ERR_INVALID", 2: "ZR_ERR_OOM",
                3: "ZR_ERR_HIP", 4: "ZR_ERR_UNSUPPORTED"}

c_i64, c_i32, c_vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p


class zr_param(ctypes.Structure):
    _fields_ = [("numel", c_i64), ("group", c_i32)]


class zr_group(ctypes.Structure):
    _fields_ = [("world", c_i32), ("sp", c_i32)]


class zr_slice(ctypes.Structure):
    _fields_ = [("bucket", c_i64), ("group", c_i32), ("dst", c_i32),
                ("bucket_offset", c_i64), ("flat_offset", c_i64),
                ("part_offset", c_i64), ("numel", c_i64)]

    def astuple(self):
        return (self.bucket, self.group, self.dst, self.bucket_offset,
                self.flat_offset, self.part_offset, self.numel)


class zr_replica(ctypes.Structure):
    _fields_ = [("ptr", c_vp), ("flat_base", c_i64), ("len", c_i64)]


class zr_adam(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("step", c_i64)]


_P = ctypes.POINTER
_sigs = {
    "zr_plan_buckets": (c_i32, [_P(zr_param), c_i64, _P(zr_group), c_i32, c_i64,
                                c_i32, c_i64, _P(c_vp)]),
    "zr_plan_free": (None, [c_vp]),
    "zr_plan_num_buckets": (c_i32, [c_vp, _P(c_i64)]),
    "zr_plan_num_params": (c_i32, [c_vp, _P(c_i64)]),
    "zr_plan_partition_gradients": (c_i32, [c_vp, _P(c_i32)]),
    "zr_plan_group_info": (c_i32, [c_vp, c_i32, _P(c_i64), _P(c_i64),
                                   _P(c_i64), _P(ctypes.c_float)]),
    "zr_plan_param_offset": (c_i32, [c_vp, c_i64, _P(c_i64)]),
    "zr_plan_param_partitions": (c_i32, [c_vp, c_i64, _P(_P(c_i32)), _P(c_i32)]),
    "zr_plan_grad_start_offset": (c_i32, [c_vp, c_i64, c_i32, _P(c_i64)]),
    "zr_plan_slices": (c_i32, [c_vp, c_i64, _P(_P(zr_slice)), _P(c_i64)]),
    "zr_plan_param_buckets": (c_i32, [c_vp, c_i64, _P(c_i64), _P(c_i64)]),
    "zr_plan_reduce_launches": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                        c_i32, _P(c_i64), _P(c_i64)]),
    "zr_reduce_launch_occupancy": (c_i32, [c_i32, c_i32, c_i32, _P(c_i32), _P(c_i32)]),
    "zr_ipg_accumulate": (c_i32, [c_vp, _P(c_i64), _P(c_vp), c_i64, c_i32, c_vp,
                                  c_i64, c_i64, c_vp]),
    "zr_ipg_accumulate_first": (c_i32, [c_vp, _P(c_i64), _P(c_vp), c_i64, c_i32, c_vp,
                                        c_i64, c_i64, c_vp]),
    "zr_reduce_scatter_local": (c_i32, [c_vp, c_i32, c_i64, c_i32, _P(zr_replica),
                                        c_i32, _P(c_vp), c_vp]),
    "zr_reduce_scatter_local_range": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i32,
                                              _P(zr_replica), c_i32, _P(c_vp), c_vp]),
    "zr_reduce_scatter_adam_range": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i32,
                                             _P(zr_replica), c_i32, _P(zr_adam), c_vp, c_vp,
                                             c_vp, c_vp, c_vp, c_vp]),
    "zr_copy_grads_in_partition": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_vp,
                                           c_vp]),
    "zr_adam_partition": (c_i32, [_P(zr_adam), c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_i64, c_vp]),
    "zr_reduce_scatter_adam": (c_i32, [c_vp, c_i32, c_i64, c_i32, _P(zr_replica),
                                       c_i32, _P(zr_adam), c_vp, c_vp, c_vp, c_vp,
                                       c_vp, c_vp]),
    "zr_reduce_scatter_adam_capped": (c_i32, [c_vp, c_i32, c_i64, c_i32, _P(zr_replica),
                                              c_i32, _P(zr_adam), c_vp, c_vp, c_vp, c_vp,
                                              c_vp, c_i32, c_vp]),
    "zr_reduce_scatter_adam_noalloc": (c_i32, [c_vp, c_i32, c_i64, c_i32, _P(zr_replica),
                                               c_i32, _P(zr_adam), c_vp, c_vp, c_vp, c_vp,
                                               c_vp, c_vp]),
    "zr_ring_rs_step": (c_i32, [_P(c_vp), c_i32, c_i64, c_i32, c_vp]),
    "zr_ring_ag_step": (c_i32, [_P(c_vp), c_i32, c_i64, c_i32, c_vp]),
    "zr_all_gather_params": (c_i32, [c_vp, c_i32, _P(c_vp), c_i32, c_vp, c_i64, c_i64,
                                     c_vp]),
    "zr_last_error": (ctypes.c_char_p, []),
    "zr_version": (c_i32, []),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sigs)


class ZrError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(status):
    if status != ZR_OK:
        raise ZrError(status, _lib.zr_last_error().decode(errors="replace"))


def zr_last_error():
    return _lib.zr_last_error().decode(errors="replace")


def zr_version():
    return _lib.zr_version()


# ------------------------------------------------------------ marshalling

def _int(x, bits, name):
    """A Python integer for a C int32_t / int64_t argument.  ctypes wraps
    out-of-range values silently (2**32 + 5 would arrive as 5), so the range
    is checked here and a violation raises ZrError(ZR_ERR_INVALID)."""
    if isinstance(x, float) and x.is_integer():
        v = int(x)                      # e.g. reduce_bucket_size=5e8
    else:
        try:
            v = operator.index(x)
        except TypeError:
            raise ZrError(ZR_ERR_INVALID, f"{name} must be an integer, not {x!r}") from None
    lim = 1 << (bits - 1)
    if not -lim <= v < lim:
        raise ZrError(ZR_ERR_INVALID, f"{name} = {v} does not fit in int{bits}_t")
    return v


def _i32(x, name):
    return _int(x, 32, name)


def _i64(x, name):
    return _int(x, 64, name)


def _ptr(t):
    """Device (or host) address of a tensor, or None for None."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


_DT_NAME = {ZR_FP32: "fp32", ZR_BF16: "bf16"}


def _buf(t, name, dtype=None, min_numel=None):
    """Checks one buffer argument and returns its address (None for None).

    The C calls see only addresses, so what a pointer cannot carry is checked
    here: a torch tensor must be a contiguous device tensor (a strided view
    would be read as if it were dense), of the element type the call needs,
    and hold at least the elements the call touches.  Violations raise
    ZrError(ZR_ERR_INVALID) before anything is enqueued."""
    if t is None:
        return None
    if torch is not None and isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ZrError(ZR_ERR_INVALID, f"{name} must be contiguous")
        if not t.is_cuda:
            raise ZrError(ZR_ERR_INVALID, f"{name} must be a device tensor")
    if dtype is not None and _dtype_code(t) != dtype:
        raise ZrError(ZR_ERR_INVALID, f"{name} must be {_DT_NAME[dtype]}")
    if min_numel is not None and t.numel() < min_numel:
        raise ZrError(ZR_ERR_INVALID,
                      f"{name} holds {t.numel()} elements; the call touches {min_numel}")
    return ctypes.c_void_p(t.data_ptr())


def _part_numel(plan, group):
    """P_g of the plan's group, queried once per plan and group."""
    P = plan.part_numel.get(group)
    if P is None:
        P = plan.part_numel[group] = zr_plan_group_info(plan, group)[2]
    return P


def _padded_numel(plan, group):
    """L_g = R_g * P_g of the plan's group, queried once per plan and group."""
    key = ("padded", group)
    L = plan.part_numel.get(key)
    if L is None:
        L = plan.part_numel[key] = zr_plan_group_info(plan, group)[1]
    return L


def _world(plan, group):
    """R_g of the plan's group, as given to zr_plan_buckets (an out-of-range
    group is the C call's error: the group query raises it)."""
    g = _i32(group, "group")
    if not 0 <= g < len(plan.worlds):
        zr_plan_group_info(plan, g)
    return plan.worlds[g]


def _expect_len(seq, n, name):
    """The C calls index host arrays by rank: a list shorter (or longer) than
    the group needs would make them read past the array, so its length is
    checked here."""
    if len(seq) != n:
        raise ZrError(ZR_ERR_INVALID, f"{name} has {len(seq)} entries; the call needs {n}")


def _dtype_code(t):
    dt = t.dtype
    if dt is torch.bfloat16:
        return ZR_BF16
    if dt is torch.float32:
        return ZR_FP32
    return -1


def _dtype_name_code(dt):
    """ZR_BF16 / ZR_FP32 for "bf16" / "fp32" or the torch dtype."""
    if dt == "bf16" or (torch is not None and dt is torch.bfloat16):
        return ZR_BF16
    if dt == "fp32" or (torch is not None and dt is torch.float32):
        return ZR_FP32
    raise ZrError(ZR_ERR_INVALID, f"unsupported gradient dtype {dt!r}")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _adam(lr, beta1, beta2, eps, step):
    return zr_adam(float(lr), float(beta1), float(beta2), float(eps), _i64(step, "step"))


class Plan:
    """Owns a zr_plan handle (freed with zr_plan_free)."""

    def __init__(self, handle, numels=(), worlds=()):
        self._h = handle
        self.part_numel = {}      # group -> P_g (the plan is immutable)
        self.numels = tuple(int(n) for n in numels)   # param sizes, list order
        self.worlds = tuple(int(w) for w in worlds)   # R_g per group

    @property
    def handle(self):
        if not self._h:
            raise ValueError("plan already freed")
        return self._h

    def free(self):
        if self._h:
            _lib.zr_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def zr_plan_buckets(numels, param_groups, groups, reduce_bucket_size,
                    partition_gradients=0, align=1):
    """``groups``: list of (world, sp).  Returns a Plan."""
    n = len(numels)
    params = (zr_param * max(n, 1))()
    for i, (ne, g) in enumerate(zip(numels, param_groups)):
        params[i] = zr_param(_i64(ne, f"numels[{i}]"), _i32(g, f"param_groups[{i}]"))
    gs = (zr_group * max(len(groups), 1))()
    for i, (w, sp) in enumerate(groups):
        gs[i] = zr_group(_i32(w, f"groups[{i}].world"), _i32(sp, f"groups[{i}].sp"))
    out = c_vp()
    _check(_lib.zr_plan_buckets(params, n, gs, _i32(len(groups), "len(groups)"),
                                _i64(reduce_bucket_size, "reduce_bucket_size"),
                                _i32(partition_gradients, "partition_gradients"),
                                _i64(align, "align"),
                                ctypes.byref(out)))
    return Plan(out.value, numels, [w for w, _ in groups])


def zr_plan_free(plan):
    plan.free()


def zr_plan_num_buckets(plan):
    v = c_i64()
    _check(_lib.zr_plan_num_buckets(plan.handle, ctypes.byref(v)))
    return v.value


def zr_plan_num_params(plan):
    v = c_i64()
    _check(_lib.zr_plan_num_params(plan.handle, ctypes.byref(v)))
    return v.value


def zr_plan_partition_gradients(plan):
    v = c_i32()
    _check(_lib.zr_plan_partition_gradients(plan.handle, ctypes.byref(v)))
    return v.value


def zr_plan_group_info(plan, g):
    """(total, padded, part_numel, divisor)."""
    t, L, P, d = c_i64(), c_i64(), c_i64(), ctypes.c_float()
    _check(_lib.zr_plan_group_info(plan.handle, _i32(g, "group"), ctypes.byref(t),
                                   ctypes.byref(L), ctypes.byref(P),
                                   ctypes.byref(d)))
    return t.value, L.value, P.value, d.value


def zr_plan_param_offset(plan, p):
    v = c_i64()
    _check(_lib.zr_plan_param_offset(plan.handle, _i64(p, "p"), ctypes.byref(v)))
    return v.value


def zr_plan_param_partitions(plan, p):
    ids, n = _P(c_i32)(), c_i32()
    _check(_lib.zr_plan_param_partitions(plan.handle, _i64(p, "p"), ctypes.byref(ids),
                                         ctypes.byref(n)))
    return [ids[i] for i in range(n.value)]


def zr_plan_grad_start_offset(plan, p, k):
    v = c_i64()
    _check(_lib.zr_plan_grad_start_offset(plan.handle, _i64(p, "p"), _i32(k, "k"),
                                          ctypes.byref(v)))
    return v.value


def zr_plan_param_buckets(plan, p):
    """(first, last) bucket param p feeds."""
    a, b = c_i64(), c_i64()
    _check(_lib.zr_plan_param_buckets(plan.handle, _i64(p, "p"), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def zr_plan_reduce_launches(plan, group, bucket_first, bucket_count, dst, grad_dtype,
                            fused, with_grad_out=False):
    """(tiles, launches) of a reduce call over buckets [bucket_first,
    bucket_first + bucket_count) for ``dst``; grad_dtype is "bf16" or
    "fp32" (or a torch dtype)."""
    dt = _dtype_name_code(grad_dtype)
    t, n = c_i64(), c_i64()
    _check(_lib.zr_plan_reduce_launches(plan.handle, _i32(group, "group"),
                                        _i64(bucket_first, "bucket_first"),
                                        _i64(bucket_count, "bucket_count"), _i32(dst, "dst"),
                                        dt, int(bool(fused)), int(bool(with_grad_out)),
                                        ctypes.byref(t), ctypes.byref(n)))
    return t.value, n.value


def zr_reduce_launch_occupancy(grad_dtype, fused, world):
    """(workgroups per CU, xcd_weighted) of an uncapped reduce call over
    ``world`` replicas of grad_dtype ("bf16", "fp32" or a torch dtype):
    workgroups per CU 0 = as many as the registers allow; xcd_weighted True
    when the odd XCDs take 31/32 of the even XCDs' tiles."""
    dt = _dtype_name_code(grad_dtype)
    k, w = c_i32(), c_i32()
    _check(_lib.zr_reduce_launch_occupancy(dt, int(bool(fused)), _i32(world, "world"),
                                           ctypes.byref(k), ctypes.byref(w)))
    return k.value, bool(w.value)


def zr_plan_slices(plan, bucket=-1):
    """List of slice tuples (bucket, group, dst, bucket_offset, flat_offset,
    part_offset, numel)."""
    s, n = _P(zr_slice)(), c_i64()
    _check(_lib.zr_plan_slices(plan.handle, _i64(bucket, "bucket"), ctypes.byref(s),
                               ctypes.byref(n)))
    return [s[i].astuple() for i in range(n.value)]


def zr_ipg_accumulate(plan, param_ids, grads, main_grad, window_base=0,
                      window_len=None, stream=None):
    """grads[i]: tensor of param param_ids[i] (bf16 or fp32, all one dtype);
    main_grad: fp32 window tensor."""
    _ipg(_lib.zr_ipg_accumulate, plan, param_ids, grads, main_grad, window_base, window_len,
         stream)


def zr_ipg_accumulate_first(plan, param_ids, grads, main_grad, window_base=0,
                            window_len=None, stream=None):
    """The step's first micro-batch: as zr_ipg_accumulate on a zeroed window,
    without reading (or zeroing) main_grad."""
    _ipg(_lib.zr_ipg_accumulate_first, plan, param_ids, grads, main_grad, window_base,
         window_len, stream)


def _ipg(fn, plan, param_ids, grads, main_grad, window_base, window_len, stream):
    n = len(param_ids)
    if len(grads) != n:
        raise ZrError(ZR_ERR_INVALID, "param_ids and grads differ in length")
    ids = (c_i64 * max(n, 1))(*[_i64(p, f"param_ids[{i}]") for i, p in enumerate(param_ids)])
    dt = _dtype_code(grads[0]) if n else ZR_FP32

    def need(i):
        # the param's size; an out-of-range id is left to the C call's check
        p = ids[i]
        return plan.numels[p] if 0 <= p < len(plan.numels) else None

    ptrs = (c_vp * max(n, 1))(*[_buf(g, f"grads[{i}]", dt, need(i)).value
                                for i, g in enumerate(grads)])
    wl = main_grad.numel() if window_len is None else _i64(window_len, "window_len")
    _check(fn(plan.handle, ids, ptrs, n, dt, _buf(main_grad, "main_grad", ZR_FP32, wl),
              _i64(window_base, "window_base"), wl, _stream(stream)))


def _replicas(reps, plan, group):
    """reps: list of R_g tensors (flat_base 0) or (tensor, flat_base) pairs."""
    _expect_len(reps, _world(plan, group), "reps")
    arr = (zr_replica * max(len(reps), 1))()
    dt = None
    for i, r in enumerate(reps):
        t, base = (r, 0) if not isinstance(r, tuple) else r
        dt = _dtype_code(t) if dt is None else dt
        arr[i] = zr_replica(_buf(t, f"replica {i}", dt).value, _i64(base, f"replica {i} flat_base"),
                            t.numel())
    return arr, (ZR_FP32 if dt is None else dt)


def zr_reduce_scatter_local(plan, group, bucket, dst, reps, part_out,
                            stream=None):
    """part_out: list of fp32 tensors (all destinations when dst == -1, else
    the one partition)."""
    arr, dt = _replicas(reps, plan, group)
    P = _part_numel(plan, group)
    R = _world(plan, group)
    if -1 <= _i32(dst, "dst") < R:        # an out-of-range dst is the C call's error
        _expect_len(part_out, R if int(dst) == -1 else 1, "part_out")
    outs = (c_vp * max(len(part_out), 1))(
        *[_buf(t, f"part_out[{i}]", ZR_FP32, P).value if t is not None else None
          for i, t in enumerate(part_out)])
    _check(_lib.zr_reduce_scatter_local(plan.handle, _i32(group, "group"),
                                        _i64(bucket, "bucket"), _i32(dst, "dst"), arr, dt, outs,
                                        _stream(stream)))


def zr_reduce_scatter_local_range(plan, group, bucket_first, bucket_count, dst, reps,
                                  part_out, stream=None):
    """zr_reduce_scatter_local over buckets [bucket_first, bucket_first +
    bucket_count) in one call."""
    arr, dt = _replicas(reps, plan, group)
    P = _part_numel(plan, group)
    R = _world(plan, group)
    if -1 <= _i32(dst, "dst") < R:        # an out-of-range dst is the C call's error
        _expect_len(part_out, R if int(dst) == -1 else 1, "part_out")
    outs = (c_vp * max(len(part_out), 1))(
        *[_buf(t, f"part_out[{i}]", ZR_FP32, P).value if t is not None else None
          for i, t in enumerate(part_out)])
    _check(_lib.zr_reduce_scatter_local_range(plan.handle, _i32(group, "group"),
                                              _i64(bucket_first, "bucket_first"),
                                              _i64(bucket_count, "bucket_count"),
                                              _i32(dst, "dst"), arr, dt, outs, _stream(stream)))


def zr_reduce_scatter_adam_range(plan, group, bucket_first, bucket_count, dst, reps,
                                 master, m, v, param_bf16=None, grad_out=None, lr=1e-3,
                                 beta1=0.9, beta2=0.999, eps=1e-8, step=1, stream=None):
    """zr_reduce_scatter_adam over buckets [bucket_first, bucket_first +
    bucket_count) in one call."""
    arr, dt = _replicas(reps, plan, group)
    h = _adam(lr, beta1, beta2, eps, step)
    P = _part_numel(plan, group) if int(dst) >= 0 else _padded_numel(plan, group)
    _check(_lib.zr_reduce_scatter_adam_range(plan.handle, _i32(group, "group"),
                                             _i64(bucket_first, "bucket_first"),
                                             _i64(bucket_count, "bucket_count"),
                                             _i32(dst, "dst"), arr, dt, ctypes.byref(h),
                                             _buf(master, "master", ZR_FP32, P),
                                             _buf(m, "m", ZR_FP32, P), _buf(v, "v", ZR_FP32, P),
                                             _buf(param_bf16, "param_bf16", ZR_BF16, P),
                                             _buf(grad_out, "grad_out", ZR_FP32, P),
                                             _stream(stream)))


def zr_copy_grads_in_partition(plan, group, bucket, dst, bucket_layout_src,
                               part_out, stream=None):
    need = 0
    if int(bucket) >= 0:
        for s in zr_plan_slices(plan, bucket):
            if s[1] == int(group) and s[2] == int(dst):
                need = max(need, s[3] + s[6])
    _check(_lib.zr_copy_grads_in_partition(
        plan.handle, _i32(group, "group"), _i64(bucket, "bucket"), _i32(dst, "dst"),
        _buf(bucket_layout_src, "bucket_layout_src", ZR_FP32, need),
        _buf(part_out, "part_out", ZR_FP32, _part_numel(plan, group)), _stream(stream)))


def zr_adam_partition(grad, master, m, v, param_bf16=None, lr=1e-3, beta1=0.9,
                      beta2=0.999, eps=1e-8, step=1, n=None, stream=None):
    h = _adam(lr, beta1, beta2, eps, step)
    nn = master.numel() if n is None else _i64(n, "n")
    need = max(nn, 0)
    _check(_lib.zr_adam_partition(ctypes.byref(h), _buf(grad, "grad", ZR_FP32, need),
                                  _buf(master, "master", ZR_FP32, need),
                                  _buf(m, "m", ZR_FP32, need), _buf(v, "v", ZR_FP32, need),
                                  _buf(param_bf16, "param_bf16", ZR_BF16, need), nn,
                                  _stream(stream)))


def zr_reduce_scatter_adam(plan, group, bucket, dst, reps, master, m, v,
                           param_bf16=None, grad_out=None, lr=1e-3, beta1=0.9,
                           beta2=0.999, eps=1e-8, step=1, stream=None):
    arr, dt = _replicas(reps, plan, group)
    h = _adam(lr, beta1, beta2, eps, step)
    # dst == -1: the state buffers hold every partition (L_g elements)
    P = _part_numel(plan, group) if int(dst) >= 0 else _padded_numel(plan, group)
    _check(_lib.zr_reduce_scatter_adam(plan.handle, _i32(group, "group"),
                                       _i64(bucket, "bucket"), _i32(dst, "dst"), arr, dt,
                                       ctypes.byref(h),
                                       _buf(master, "master", ZR_FP32, P),
                                       _buf(m, "m", ZR_FP32, P), _buf(v, "v", ZR_FP32, P),
                                       _buf(param_bf16, "param_bf16", ZR_BF16, P),
                                       _buf(grad_out, "grad_out", ZR_FP32, P),
                                       _stream(stream)))


def zr_reduce_scatter_adam_capped(plan, group, bucket, dst, reps, master, m, v,
                                  param_bf16=None, grad_out=None, max_workgroups=256,
                                  lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=1,
                                  stream=None):
    arr, dt = _replicas(reps, plan, group)
    h = _adam(lr, beta1, beta2, eps, step)
    P = _part_numel(plan, group) if int(dst) >= 0 else _padded_numel(plan, group)
    _check(_lib.zr_reduce_scatter_adam_capped(plan.handle, _i32(group, "group"),
                                              _i64(bucket, "bucket"), _i32(dst, "dst"),
                                              arr, dt, ctypes.byref(h),
                                              _buf(master, "master", ZR_FP32, P),
                                              _buf(m, "m", ZR_FP32, P),
                                              _buf(v, "v", ZR_FP32, P),
                                              _buf(param_bf16, "param_bf16", ZR_BF16, P),
                                              _buf(grad_out, "grad_out", ZR_FP32, P),
                                              _i32(max_workgroups, "max_workgroups"),
                                              _stream(stream)))


def zr_reduce_scatter_adam_noalloc(plan, group, bucket, dst, reps, master, m, v,
                                   param_bf16=None, grad_out=None, lr=1e-3, beta1=0.9,
                                   beta2=0.999, eps=1e-8, step=1, stream=None):
    """zr_reduce_scatter_adam without device allocation: the segment table is
    staged in the library's fixed per-GPU array (calls that overlap on one GPU
    race)."""
    arr, dt = _replicas(reps, plan, group)
    h = _adam(lr, beta1, beta2, eps, step)
    P = _part_numel(plan, group) if int(dst) >= 0 else _padded_numel(plan, group)
    _check(_lib.zr_reduce_scatter_adam_noalloc(plan.handle, _i32(group, "group"),
                                               _i64(bucket, "bucket"), _i32(dst, "dst"), arr,
                                               dt, ctypes.byref(h),
                                               _buf(master, "master", ZR_FP32, P),
                                               _buf(m, "m", ZR_FP32, P),
                                               _buf(v, "v", ZR_FP32, P),
                                               _buf(param_bf16, "param_bf16", ZR_BF16, P),
                                               _buf(grad_out, "grad_out", ZR_FP32, P),
                                               _stream(stream)))


class PreparedReduceScatterAdam:
    """zr_reduce_scatter_adam -- or, with max_workgroups >= 1,
    zr_reduce_scatter_adam_capped -- with its arguments checked and marshalled
    once, for loops that call it per bucket.  Each call passes only the
    bucket, the Adam step and the stream; the C library validates every call
    as usual.  Holds references to the tensors, so their memory stays valid
    while it lives.  One object must not be called from several threads at
    once (the step is written into its argument struct)."""

    def __init__(self, plan, group, dst, reps, master, m, v, param_bf16=None,
                 grad_out=None, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                 max_workgroups=0):
        self._keep = (plan, list(reps), master, m, v, param_bf16, grad_out)
        self._arr, self._dt = _replicas(reps, plan, group)
        self._group = _i32(group, "group")
        self._dst = _i32(dst, "dst")
        P = _part_numel(plan, group) if self._dst >= 0 else _padded_numel(plan, group)
        self._bufs = (_buf(master, "master", ZR_FP32, P), _buf(m, "m", ZR_FP32, P),
                      _buf(v, "v", ZR_FP32, P),
                      _buf(param_bf16, "param_bf16", ZR_BF16, P),
                      _buf(grad_out, "grad_out", ZR_FP32, P))
        self._h = _adam(lr, beta1, beta2, eps, 1)
        self._cap = _i32(max_workgroups, "max_workgroups")
        if self._cap < 0:
            raise ZrError(ZR_ERR_INVALID, "max_workgroups must be >= 0 (0: uncapped)")
        self._handle = plan.handle

    def __call__(self, bucket=-1, step=1, stream=None, count=None):
        """``count`` given: the buckets [bucket, bucket + count) in one call
        (zr_reduce_scatter_adam_range; not with a workgroup cap)."""
        self._h.step = _i64(step, "step")
        b = _i64(bucket, "bucket")
        if count is not None:
            if self._cap:
                raise ZrError(ZR_ERR_INVALID, "a bucket range cannot be capped")
            _check(_lib.zr_reduce_scatter_adam_range(
                self._handle, self._group, b, _i64(count, "count"), self._dst, self._arr,
                self._dt, ctypes.byref(self._h), *self._bufs, _stream(stream)))
            return
        if self._cap:
            _check(_lib.zr_reduce_scatter_adam_capped(
                self._handle, self._group, b, self._dst, self._arr, self._dt,
                ctypes.byref(self._h), *self._bufs, self._cap, _stream(stream)))
        else:
            _check(_lib.zr_reduce_scatter_adam(
                self._handle, self._group, b, self._dst, self._arr, self._dt,
                ctypes.byref(self._h), *self._bufs, _stream(stream)))


def prepare_reduce_scatter_adam(plan, group, dst, reps, master, m, v, param_bf16=None,
                                grad_out=None, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                max_workgroups=0):
    """A PreparedReduceScatterAdam for these arguments."""
    return PreparedReduceScatterAdam(plan, group, dst, reps, master, m, v, param_bf16,
                                     grad_out, lr, beta1, beta2, eps, max_workgroups)


def zr_ring_rs_step(rank_bufs, chunk_numel, step, stream=None):
    n = len(rank_bufs)
    need = max(int(chunk_numel), 0) * n
    arr = (c_vp * max(n, 1))(*[_buf(t, f"rank_bufs[{i}]", ZR_FP32, need).value
                               if t is not None else None for i, t in enumerate(rank_bufs)])
    _check(_lib.zr_ring_rs_step(arr, n, _i64(chunk_numel, "chunk_numel"), _i32(step, "step"),
                                _stream(stream)))


def zr_ring_ag_step(rank_bufs, chunk_numel, step, stream=None):
    n = len(rank_bufs)
    need = max(int(chunk_numel), 0) * n
    arr = (c_vp * max(n, 1))(*[_buf(t, f"rank_bufs[{i}]", ZR_FP32, need).value
                               if t is not None else None for i, t in enumerate(rank_bufs)])
    _check(_lib.zr_ring_ag_step(arr, n, _i64(chunk_numel, "chunk_numel"), _i32(step, "step"),
                                _stream(stream)))


def zr_all_gather_params(plan, group, parts, out, out_base=0, out_len=None,
                         stream=None):
    """parts: list of R_g partition tensors (bf16 or fp32); out: tensor that
    receives flat elements [out_base, out_base + out_len)."""
    n = len(parts)
    _expect_len(parts, _world(plan, group), "parts")
    dt = _dtype_code(out)
    P = _part_numel(plan, group)
    arr = (c_vp * max(n, 1))(*[(_buf(t, f"parts[{i}]", dt, P).value if t is not None else 0)
                               for i, t in enumerate(parts)])
    ol = out.numel() if out_len is None else _i64(out_len, "out_len")
    _check(_lib.zr_all_gather_params(plan.handle, _i32(group, "group"), arr, dt,
                                     _buf(out, "out", dt, ol), _i64(out_base, "out_base"), ol,
                                     _stream(stream)))

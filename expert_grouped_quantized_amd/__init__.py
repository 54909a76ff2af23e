"""Python binding of the MI355X MoE layer library (``libmoe.so``, include/moe.h).

Argument marshalling only: every function here forwards to the C ABI entry of
the same name.  Torch tensors are passed as device pointers and the current
torch stream as the HIP stream; all computation happens in the HIP kernels.
If the library is not built, importing succeeds but every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_OVERRIDE names another build of the same ABI (the host tests point it
# at a sanitizer build of the host side); by default the in-tree libmoe.so.
LIB_PATH = os.environ.get("MOE_LIB_OVERRIDE") or os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EDEVICE = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_I4_G32, MOE_I8_ROW = 0, 1, 2, 3
MOE_I2_G32, MOE_I3_G32, MOE_I5_G32, MOE_I6_G32, MOE_I7_G32, MOE_I8_G32 = 4, 5, 6, 7, 8, 9
MOE_MXFP4 = 10
MOE_BLOB_ROUTED, MOE_BLOB_SHARED = 0, 1
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "i4g32": MOE_I4_G32, "i8row": MOE_I8_ROW,
          "i2g32": MOE_I2_G32, "i3g32": MOE_I3_G32, "i5g32": MOE_I5_G32, "i6g32": MOE_I6_G32,
          "i7g32": MOE_I7_G32, "i8g32": MOE_I8_G32, "mxfp4": MOE_MXFP4}


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d", "n_experts", "ffn", "n_shared", "shared_ffn", "act", "expert_w", "shared_w")]

    def __repr__(self):
        return "Desc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def make_desc(d, n_experts, ffn, n_shared=0, shared_ffn=0, act="bf16", expert_w="bf16",
              shared_w="bf16") -> Desc:
    cv = lambda v: DTYPES[v] if isinstance(v, str) else int(v)
    return Desc(d, n_experts, ffn, n_shared, shared_ffn if n_shared else 0, cv(act),
                cv(expert_w), cv(shared_w))


_lib = None


def lib():
    """Load libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "expert_grouped_quantized_amd.build.build()")
        # torch carries its own HIP runtime (soname libamdhip64.so.7).  Load it
        # first, so that libmoe.so binds to that same runtime instead of
        # loading a second one from the ROCm install, which would not share
        # torch's device memory and streams.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        D = ctypes.POINTER(Desc)
        sig = {
            "moe_abi_version": ([], i32),
            "moe_status_str": ([i32], ctypes.c_char_p),
            "moe_last_error": ([], ctypes.c_char_p),
            "moe_blob_bytes": ([D, i32, ctypes.POINTER(sz)], i32),
            "moe_pack_experts": ([D, i32, vp, vp, vp, vp, vp, vp, vp, sz], i32),
            "moe_unpack_experts": ([D, i32, vp, sz, vp, vp, vp, vp, vp, vp], i32),
            "moe_workspace_bytes": ([D, i32, i32, ctypes.POINTER(sz)], i32),
            "moe_route": ([D, i32, i32, vp, vp, vp, vp, vp, vp, vp], i32),
            "moe_route_from_logits": ([D, i32, i32, vp, vp, vp, vp], i32),
            "moe_permute": ([D, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp], i32),
            "moe_route_plan": ([D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
                               i32),
            "moe_grouped_ffn": ([D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
            "moe_grouped_ffn_noalloc": ([D, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
            "moe_combine": ([D, i32, i32, vp, vp, vp, vp, vp], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(x):
    """Pointer of a torch tensor / numpy array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take a pointer of {type(x)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, fn: str):
    if rc != MOE_OK:
        raise MoeError(rc, fn, (lib().moe_last_error() or b"").decode())


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_last_error() -> str:
    return (lib().moe_last_error() or b"").decode()


def moe_blob_bytes(desc: Desc, kind: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().moe_blob_bytes(ctypes.byref(desc), kind, ctypes.byref(out)), "moe_blob_bytes")
    return out.value


def moe_workspace_bytes(desc: Desc, T: int, k: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(ctypes.byref(desc), T, k, ctypes.byref(out)),
           "moe_workspace_bytes")
    return out.value


def moe_pack_experts(desc: Desc, kind: int, gate, gate_scales, up, up_scales, down, down_scales,
                     blob):
    """Host arrays in, host blob (numpy uint8 of moe_blob_bytes) filled."""
    _check(lib().moe_pack_experts(ctypes.byref(desc), kind, _p(gate), _p(gate_scales), _p(up),
                                  _p(up_scales), _p(down), _p(down_scales), _p(blob),
                                  blob.nbytes), "moe_pack_experts")
    return blob


def moe_unpack_experts(desc: Desc, kind: int, blob, gate, gate_scales, up, up_scales, down,
                       down_scales):
    _check(lib().moe_unpack_experts(ctypes.byref(desc), kind, _p(blob), blob.nbytes, _p(gate),
                                    _p(gate_scales), _p(up), _p(up_scales), _p(down),
                                    _p(down_scales)), "moe_unpack_experts")


def moe_route(desc, T, k, hidden, router_w, bias, logits, topk_ids, topk_w, stream=None):
    _check(lib().moe_route(ctypes.byref(desc), T, k, _p(hidden), _p(router_w), _p(bias),
                           _p(logits), _p(topk_ids), _p(topk_w), _stream(stream)), "moe_route")


def moe_route_from_logits(desc, T, k, logits, topk_ids, topk_w, stream=None):
    _check(lib().moe_route_from_logits(ctypes.byref(desc), T, k, _p(logits), _p(topk_ids),
                                       _p(topk_w), _stream(stream)), "moe_route_from_logits")


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return workspace_bytes
    return workspace.numel() * workspace.element_size()


def moe_permute(desc, T, k, hidden, topk_ids, offsets, perm, inv_perm, workspace,
                workspace_bytes=None, stream=None):
    _check(lib().moe_permute(ctypes.byref(desc), T, k, _p(hidden), _p(topk_ids), _p(offsets),
                             _p(perm), _p(inv_perm), _p(workspace),
                             _ws_bytes(workspace, workspace_bytes), _stream(stream)),
           "moe_permute")


def moe_route_plan(desc, T, k, hidden, router_w, bias, logits, topk_ids, topk_w, offsets, perm,
                   inv_perm, workspace, workspace_bytes=None, stream=None):
    _check(lib().moe_route_plan(ctypes.byref(desc), T, k, _p(hidden), _p(router_w), _p(bias),
                                _p(logits), _p(topk_ids), _p(topk_w), _p(offsets), _p(perm),
                                _p(inv_perm), _p(workspace),
                                _ws_bytes(workspace, workspace_bytes), _stream(stream)),
           "moe_route_plan")


def moe_grouped_ffn(desc, T, k, hidden, topk_w, offsets, perm, routed_blob, shared_blob,
                    out_assign, shared_out, workspace, workspace_bytes=None, stream=None):
    wsb = _ws_bytes(workspace, workspace_bytes)
    _check(lib().moe_grouped_ffn(ctypes.byref(desc), T, k, _p(hidden), _p(topk_w), _p(offsets),
                                 _p(perm), _p(routed_blob), _p(shared_blob), _p(out_assign),
                                 _p(shared_out), _p(workspace), wsb, _stream(stream)),
           "moe_grouped_ffn")


def moe_grouped_ffn_noalloc(desc, T, k, hidden, topk_w, offsets, perm, routed_blob, shared_blob,
                            out_assign, shared_out, stream=None):
    _check(lib().moe_grouped_ffn_noalloc(ctypes.byref(desc), T, k, _p(hidden), _p(topk_w),
                                         _p(offsets), _p(perm), _p(routed_blob),
                                         _p(shared_blob), _p(out_assign), _p(shared_out),
                                         _stream(stream)), "moe_grouped_ffn_noalloc")


def moe_combine(desc, T, k, out_assign, inv_perm, shared_out, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(desc), T, k, _p(out_assign), _p(inv_perm),
                             _p(shared_out), _p(y), _stream(stream)), "moe_combine")


from .layer import MoELayer  # noqa: E402  (buffer holder built on the calls above)

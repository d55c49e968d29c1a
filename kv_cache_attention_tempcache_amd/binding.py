"""ctypes binding of libfastar.so: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI (include/fastar.h).
torch supplies device memory and streams; this module checks tensor shapes,
dtypes and devices, passes raw pointers and the current stream, and turns
non-zero status codes into exceptions.  If the library is not built, every
entry point raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np
import torch  # imported before the library so both share torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfastar.so")

F32, BF16 = 0, 1
_DTYPES = {"f32": (F32, torch.float32), "bf16": (BF16, torch.bfloat16)}

STATUS = {
    0: "FASTAR_OK",
    1: "FASTAR_ERR_INVALID_ARGUMENT",
    2: "FASTAR_ERR_WORKSPACE_TOO_SMALL",
    3: "FASTAR_ERR_CAPACITY",
    4: "FASTAR_ERR_HIP",
    5: "FASTAR_ERR_UNSUPPORTED",
}


class FastarError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("budget_slots", ctypes.c_int32), ("num_tables", ctypes.c_int32),
                ("num_bits", ctypes.c_int32), ("cos_threshold", ctypes.c_float),
                ("dtype", ctypes.c_int), ("pq_subspaces", ctypes.c_int32),
                ("rope_members", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("frame", ctypes.c_int64), ("tokens_seen", ctypes.c_int64),
                ("live_slots", ctypes.c_int64), ("merged_tokens", ctypes.c_int64),
                ("inserted_tokens", ctypes.c_int64), ("evicted_slots", ctypes.c_int64),
                ("evicted_tokens", ctypes.c_int64), ("max_live", ctypes.c_int32),
                ("refused_frames", ctypes.c_int32)]


class State(ctypes.Structure):
    _fields_ = [("k_master", ctypes.c_void_p), ("v_master", ctypes.c_void_p),
                ("k_mirror", ctypes.c_void_p), ("v_mirror", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("last", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("n_live", ctypes.c_void_p),
                ("evicted_tokens", ctypes.c_void_p), ("frame", ctypes.c_int64),
                ("member_frames", ctypes.c_void_p)]

# the array members of State, in order (all but `frame`)
_STATE_ARRAYS = [n for n, _ in State._fields_ if n != "frame"]


# name -> (restype, argtypes); the C ABI of include/fastar.h
_VP, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "fastar_last_error": (ctypes.c_char_p, []),
    "fastar_cache_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(_SZ)]),
    "fastar_cache_create": (ctypes.c_int, [ctypes.POINTER(Config), _VP, _VP, _SZ, _VP,
                                           ctypes.POINTER(_VP)]),
    "fastar_cache_destroy": (ctypes.c_int, [_VP]),
    "fastar_cache_reset": (ctypes.c_int, [_VP, _VP]),
    "fastar_cache_planes": (ctypes.c_int, [_VP, ctypes.POINTER(_VP)]),
    "fastar_hash": (ctypes.c_int, [_VP, ctypes.c_int, _I32, _I32, _I32, _I64, _I64, _VP, _I32,
                                   _I32, _VP, _VP]),
    "fastar_pq_codes": (ctypes.c_int, [_VP, ctypes.c_int, _I32, _I32, _I32, _I64, _I64, _VP, _I32,
                                       _I32, _I32, _VP, _VP]),
    "fastar_match_merge": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _VP, _I32, _I32, _VP, _VP,
                                          _VP]),
    "fastar_attend": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I32, _F, _VP, _I64, _I64, _VP, _VP]),
    "fastar_project_keys": (ctypes.c_int, [_VP, _VP, _I64, _I32, _I32, _VP, _I64, _VP, _I64, _I64,
                                           _VP, _I64, _VP]),
    "fastar_attend_rope": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I32, _I32, _I32, _F, _F, _VP,
                                          _I64, _I64, _VP, _VP]),
    "fastar_attend_with_chunk": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I32, _VP, _VP, _I64, _I64,
                                                _I32, _F, _VP, _I64, _I64, _VP, _VP]),
    "fastar_cache_hash_slots": (ctypes.c_int, [_VP, _VP, _I32, _I32, _VP, _I64, _VP]),
    "fastar_annsa_attend": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I32, _VP, _I32, _F, _VP, _I64,
                                           _I64, _VP, _VP]),
    "fastar_cache_stats": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(Stats)]),
    "fastar_cache_export": (ctypes.c_int, [_VP, _VP, ctypes.POINTER(State)]),
    "fastar_cache_import": (ctypes.c_int, [_VP, ctypes.POINTER(State), _VP]),
    "fastar_annca_select": (ctypes.c_int, [_VP, _I32, _I32, _VP, _I32, _I32, _I32, _VP, _VP,
                                           _VP]),
    "fastar_attend_subset": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _I64, _I64, _VP, _VP,
                                            _I32, _I32, _I32, _I32, _I32, ctypes.c_int, _F, _VP,
                                            _I64, _I64, _VP]),
    "fastar_annca_attend": (ctypes.c_int, [_VP, _I64, _I64, _VP, _I32, _I32, _VP, _VP, _VP,
                                           _VP, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _F,
                                           _VP, _I64, _I64, _VP]),
    "fastar_annca_attend_static": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _I64, _I64,
                                                  _VP, _I32, _I32, _I32, _I32, _I32, _I32,
                                                  ctypes.c_int, _F, _VP, _I64, _I64, _VP]),
}

_lib = None


def library():
    """Load libfastar.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m kv_cache_attention_tempcache_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        msg = library().fastar_last_error().decode(errors="replace")
        raise FastarError(status, msg)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, name: str, dtype=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() >= 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")


def storage_dtype(dtype: str):
    return _DTYPES[dtype]


def planes_to_host(planes, dtype: str) -> np.ndarray:
    """Hyperplanes as a contiguous host array in the storage format."""
    p = torch.as_tensor(np.asarray(planes, dtype=np.float32))
    if dtype == "bf16":
        return p.to(torch.bfloat16).view(torch.int16).numpy().copy()
    return p.numpy().astype(np.float32, copy=True)


def hash_codes(x: torch.Tensor, planes: torch.Tensor, tables: int, bits: int,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """SimHash codes [H][L][N] (uint32 bit patterns in an int32 tensor) of x [H][N][d]."""
    _require(x, "x")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _require(planes, "planes", x.dtype)
    H, N, d = x.shape
    if not planes.is_contiguous() or planes.numel() != tables * bits * d:
        raise ValueError("planes must be contiguous [L][b][d]")
    if out is None:
        out = torch.empty((H, tables, N), dtype=torch.int32, device=x.device)
    _require(out, "out", torch.int32)
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _check(library().fastar_hash(_ptr(x), dt, H, N, d, x.stride(0), x.stride(1), _ptr(planes),
                                 tables, bits, _ptr(out), _stream(stream)))
    return out


def pq_codes(x: torch.Tensor, codebooks: torch.Tensor, tables: int, subspaces: int, bits: int,
             out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Product-quantization codes [H][L][N] (int32 bit patterns) of x [H][N][d]
    under codebooks [L][M][2^(b/M)][d/M]."""
    _require(x, "x")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _require(codebooks, "codebooks", x.dtype)
    H, N, d = x.shape
    if not codebooks.is_contiguous() or subspaces < 1 or bits % subspaces or \
            codebooks.numel() != tables * (1 << (bits // subspaces)) * d:
        raise ValueError("codebooks must be contiguous [L][M][2^(b/M)][d/M]")
    if out is None:
        out = torch.empty((H, tables, N), dtype=torch.int32, device=x.device)
    _require(out, "out", torch.int32)
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _check(library().fastar_pq_codes(_ptr(x), dt, H, N, d, x.stride(0), x.stride(1),
                                     _ptr(codebooks), tables, subspaces, bits, _ptr(out),
                                     _stream(stream)))
    return out


@dataclass
class CacheConfig:
    heads: int
    head_dim: int
    budget: int
    tables: int
    bits: int
    threshold: float
    dtype: str = "bf16"
    subspaces: int = 0   # 0: SimHash; M > 0: product quantization with M slices
    rope_members: int = 0  # frames of each slot's most recent members kept (0..4)

    def c(self) -> Config:
        return Config(self.heads, self.head_dim, self.budget, self.tables, self.bits,
                      float(self.threshold), _DTYPES[self.dtype][0], self.subspaces,
                      self.rope_members)

    def plane_elems(self) -> int:
        """Elements of the hyperplanes [L][b][d] or PQ codebooks [L][M][2^(b/M)][d/M]."""
        if self.subspaces:
            return self.tables * (1 << (self.bits // self.subspaces)) * self.head_dim
        return self.tables * self.bits * self.head_dim


def workspace_bytes(cfg: CacheConfig) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(library().fastar_cache_workspace_bytes(ctypes.byref(c), ctypes.byref(n)))
    return n.value


class Cache:
    """A TempCache over a caller-owned device workspace (a torch uint8 tensor)."""

    def __init__(self, cfg: CacheConfig, planes, device="cuda", stream=None):
        self.cfg = cfg
        self.torch_dtype = _DTYPES[cfg.dtype][1]
        nbytes = workspace_bytes(cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        host = planes_to_host(planes, cfg.dtype)
        if host.size != cfg.plane_elems():
            raise ValueError(f"planes must have {cfg.plane_elems()} elements")
        c = cfg.c()
        h = ctypes.c_void_p(0)
        _check(library().fastar_cache_create(ctypes.byref(c), host.ctypes.data,
                                             _ptr(self.workspace), nbytes, _stream(stream),
                                             ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            library().fastar_cache_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def planes_device(self) -> int:
        p = ctypes.c_void_p(0)
        _check(library().fastar_cache_planes(self._h, ctypes.byref(p)))
        return p.value

    def reset(self, stream=None):
        _check(library().fastar_cache_reset(self._h, _stream(stream)))

    def match_merge(self, k: torch.Tensor, v: torch.Tensor, tokens_per_frame: int,
                    num_frames: int = 1, codes: torch.Tensor | None = None,
                    slot_out: torch.Tensor | None = None, merged_out: torch.Tensor | None = None,
                    stream=None):
        """Merge num_frames frames of new keys/values [H][F*T][d] into the cache."""
        _require(k, "k", self.torch_dtype)
        _require(v, "v", self.torch_dtype)
        if k.shape != v.shape or k.stride() != v.stride():
            raise ValueError("k and v must have the same shape and strides")
        H, N, d = k.shape
        if H != self.cfg.heads or d != self.cfg.head_dim or N != tokens_per_frame * num_frames:
            raise ValueError("k must be [heads][tokens_per_frame*num_frames][head_dim]")
        if codes is not None:
            _require(codes, "codes", torch.int32)
            if tuple(codes.shape) != (H, self.cfg.tables, N) or not codes.is_contiguous():
                raise ValueError("codes must be contiguous [H][L][N]")
        for t, name, dt in ((slot_out, "slot_out", torch.int32), (merged_out, "merged_out", torch.uint8)):
            if t is not None:
                _require(t, name, dt)
                if tuple(t.shape) != (H, N) or not t.is_contiguous():
                    raise ValueError(f"{name} must be contiguous [H][N]")
        _check(library().fastar_match_merge(self._h, _ptr(k), _ptr(v), k.stride(0), k.stride(1),
                                            _ptr(codes), tokens_per_frame, num_frames,
                                            _ptr(slot_out), _ptr(merged_out), _stream(stream)))

    def attend(self, q: torch.Tensor, scale: float = 0.0, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Attention of q [H][Nq][d] over the live slots with the ln(count) bias."""
        _require(q, "q", self.torch_dtype)
        H, Nq, d = q.shape
        if H != self.cfg.heads or d != self.cfg.head_dim:
            raise ValueError("q must be [heads][Nq][head_dim]")
        if out is None:
            out = torch.empty((H, Nq, d), dtype=self.torch_dtype, device=q.device)
        _require(out, "out", self.torch_dtype)
        if lse is not None:
            _require(lse, "lse", torch.float32)
            if tuple(lse.shape) != (H, Nq) or not lse.is_contiguous():
                raise ValueError("lse must be contiguous [H][Nq]")
        _check(library().fastar_attend(self._h, _ptr(q), q.stride(0), q.stride(1), Nq,
                                       float(scale), _ptr(out), out.stride(0), out.stride(1),
                                       _ptr(lse), _stream(stream)))
        return out

    def project_keys(self, x: torch.Tensor, w: torch.Tensor, k_out: torch.Tensor | None = None,
                     codes_out: torch.Tensor | None = None, stream=None):
        """Keys k = x w^T of tokens x [N][D_in] under the key weight w [H*d][D_in]
        (bf16) and their codes under the cache's hyperplanes, in one kernel.
        Returns (k [H][N][d], codes [H][L][N] int32 bit patterns)."""
        _require(x, "x", torch.bfloat16)
        _require(w, "w", torch.bfloat16)
        H, d, L = self.cfg.heads, self.cfg.head_dim, self.cfg.tables
        if x.dim() != 2 or x.stride(1) != 1 or w.dim() != 2 or w.stride(1) != 1:
            raise ValueError("x and w must be 2-D with contiguous rows")
        N, din = x.shape
        if tuple(w.shape) != (H * d, din):
            raise ValueError("w must be [heads*head_dim][D_in]")
        if k_out is None:
            k_out = torch.empty((H, N, d), dtype=torch.bfloat16, device=x.device)
        _require(k_out, "k_out", torch.bfloat16)
        if tuple(k_out.shape) != (H, N, d):
            raise ValueError("k_out must be [heads][N][head_dim]")
        if codes_out is None:
            codes_out = torch.empty((H, L, N), dtype=torch.int32, device=x.device)
        _require(codes_out, "codes_out", torch.int32)
        if tuple(codes_out.shape) != (H, L, N) or not codes_out.is_contiguous():
            raise ValueError("codes_out must be contiguous [heads][tables][N]")
        _check(library().fastar_project_keys(
            self._h, _ptr(x), x.stride(0), N, din, _ptr(w), w.stride(0), _ptr(k_out),
            k_out.stride(0), k_out.stride(1), _ptr(codes_out), N, _stream(stream)))
        return k_out, codes_out

    def attend_rope(self, q: torch.Tensor, m: int, rope_dims: int, rope_base: float = 10000.0,
                    scale: float = 0.0, out: torch.Tensor | None = None,
                    lse: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Attention of rotated queries q [H][Nq][d] with the M-degree
        approximation: each slot's m most recent members' rotations, each
        with logit shift ln(count / min(m, count))."""
        _require(q, "q", self.torch_dtype)
        H, Nq, d = q.shape
        if H != self.cfg.heads or d != self.cfg.head_dim:
            raise ValueError("q must be [heads][Nq][head_dim]")
        if out is None:
            out = torch.empty((H, Nq, d), dtype=self.torch_dtype, device=q.device)
        _require(out, "out", self.torch_dtype)
        if lse is not None:
            _require(lse, "lse", torch.float32)
            if tuple(lse.shape) != (H, Nq) or not lse.is_contiguous():
                raise ValueError("lse must be contiguous [H][Nq]")
        _check(library().fastar_attend_rope(self._h, _ptr(q), q.stride(0), q.stride(1), Nq, m,
                                            rope_dims, float(rope_base), float(scale), _ptr(out),
                                            out.stride(0), out.stride(1), _ptr(lse),
                                            _stream(stream)))
        return out

    def attend_with_chunk(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                          scale: float = 0.0, out: torch.Tensor | None = None,
                          lse: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """One denoising step: q [H][Nq][d] attends over the live slots (ln(count)
        bias) and the chunk's raw tokens k_new, v_new [H][n_new][d] (count 1)."""
        _require(q, "q", self.torch_dtype)
        _require(k_new, "k_new", self.torch_dtype)
        _require(v_new, "v_new", self.torch_dtype)
        H, Nq, d = q.shape
        if H != self.cfg.heads or d != self.cfg.head_dim:
            raise ValueError("q must be [heads][Nq][head_dim]")
        if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or \
                k_new.dim() != 3 or k_new.shape[0] != H or k_new.shape[2] != d:
            raise ValueError("k_new and v_new must be [heads][n_new][head_dim] with equal strides")
        if out is None:
            out = torch.empty((H, Nq, d), dtype=self.torch_dtype, device=q.device)
        _require(out, "out", self.torch_dtype)
        if lse is not None:
            _require(lse, "lse", torch.float32)
            if tuple(lse.shape) != (H, Nq) or not lse.is_contiguous():
                raise ValueError("lse must be contiguous [H][Nq]")
        _check(library().fastar_attend_with_chunk(
            self._h, _ptr(q), q.stride(0), q.stride(1), Nq, _ptr(k_new), _ptr(v_new),
            k_new.stride(0), k_new.stride(1), k_new.shape[1], float(scale), _ptr(out),
            out.stride(0), out.stride(1), _ptr(lse), _stream(stream)))
        return out

    def hash_slots(self, planes: torch.Tensor, tables: int, bits: int,
                   out: torch.Tensor | None = None, stream=None):
        """Hash the slot keys under ``planes`` [L][b][d] and index them for AnnSA;
        the codes [H][L][budget] are also written to ``out`` if given."""
        _require(planes, "planes", self.torch_dtype)
        if not planes.is_contiguous() or planes.numel() != tables * bits * self.cfg.head_dim:
            raise ValueError("planes must be contiguous [L][b][d]")
        ld = self.cfg.budget
        if out is not None:
            _require(out, "out", torch.int32)
            if tuple(out.shape) != (self.cfg.heads, tables, ld) or not out.is_contiguous():
                raise ValueError("out must be contiguous [H][L][budget]")
        _check(library().fastar_cache_hash_slots(self._h, _ptr(planes), tables, bits, _ptr(out),
                                                 ld, _stream(stream)))
        return out

    def annsa_attend(self, q: torch.Tensor, q_codes: torch.Tensor, scale: float = 0.0,
                     out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
        """AnnSA: q [H][Nq][d] attends only to the slots that share a bucket with it;
        q_codes [H][L][Nq] under the hyperplanes of the latest hash_slots."""
        _require(q, "q", self.torch_dtype)
        _require(q_codes, "q_codes", torch.int32)
        H, Nq, d = q.shape
        if H != self.cfg.heads or d != self.cfg.head_dim:
            raise ValueError("q must be [heads][Nq][head_dim]")
        L = q_codes.shape[1]
        if tuple(q_codes.shape) != (H, L, Nq) or not q_codes.is_contiguous():
            raise ValueError("q_codes must be contiguous [H][L][Nq]")
        if out is None:
            out = torch.empty((H, Nq, d), dtype=self.torch_dtype, device=q.device)
        _require(out, "out", self.torch_dtype)
        if lse is not None:
            _require(lse, "lse", torch.float32)
            if tuple(lse.shape) != (H, Nq) or not lse.is_contiguous():
                raise ValueError("lse must be contiguous [H][Nq]")
        _check(library().fastar_annsa_attend(self._h, _ptr(q), q.stride(0), q.stride(1), Nq,
                                             _ptr(q_codes), L, float(scale), _ptr(out),
                                             out.stride(0), out.stride(1), _ptr(lse),
                                             _stream(stream)))
        return out

    def stats(self, stream=None) -> dict:
        st = Stats()
        _check(library().fastar_cache_stats(self._h, _stream(stream), ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in Stats._fields_}

    def export_state(self, stream=None) -> dict:
        c = self.cfg
        H, B, d, L = c.heads, c.budget, c.head_dim, c.tables
        mir = np.uint16 if c.dtype == "bf16" else np.float32
        out = {
            "k_master": np.empty((H, B, d), np.float32), "v_master": np.empty((H, B, d), np.float32),
            "k_mirror": np.empty((H, B, d), mir), "v_mirror": np.empty((H, B, d), mir),
            "count": np.empty((H, B), np.int32), "last": np.empty((H, B), np.int32),
            "codes": np.empty((H, L, B), np.uint32), "n_live": np.empty(H, np.int32),
            "evicted_tokens": np.empty(H, np.int64),
            "member_frames": np.empty((H, B, max(c.rope_members, 1)), np.int32),
        }
        st = State(**{name: out[name].ctypes.data for name in _STATE_ARRAYS}, frame=0)
        _check(library().fastar_cache_export(self._h, _stream(stream), ctypes.byref(st)))
        out["frame"] = int(st.frame)
        if not c.rope_members:
            del out["member_frames"]
        return out

    def import_state(self, state: dict, stream=None):
        c = self.cfg
        H, B, d, L = c.heads, c.budget, c.head_dim, c.tables
        mir = np.uint16 if c.dtype == "bf16" else np.float32
        spec = {"k_master": ((H, B, d), np.float32), "v_master": ((H, B, d), np.float32),
                "k_mirror": ((H, B, d), mir), "v_mirror": ((H, B, d), mir),
                "count": ((H, B), np.int32), "last": ((H, B), np.int32),
                "codes": ((H, L, B), np.uint32), "n_live": ((H,), np.int32),
                "evicted_tokens": ((H,), np.int64),
                "member_frames": ((H, B, c.rope_members), np.int32)}
        keep = {}
        ptrs = {}
        for name in _STATE_ARRAYS:
            arr = state.get(name)
            if arr is None:
                ptrs[name] = None
                continue
            shape, dt = spec[name]
            a = np.ascontiguousarray(arr, dtype=dt)
            if a.shape != shape:
                raise ValueError(f"{name} must have shape {shape}, got {a.shape}")
            keep[name] = a
            ptrs[name] = a.ctypes.data
        # no "frame" key keeps the device's frame counter (-1)
        st = State(**ptrs, frame=int(state.get("frame", -1)))
        _check(library().fastar_cache_import(self._h, ctypes.byref(st), _stream(stream)))


def annca_select(q_codes: torch.Tensor, p_codes: torch.Tensor, frames: int,
                 sel_idx: torch.Tensor | None = None, sel_count: torch.Tensor | None = None,
                 stream=None):
    """Per-frame kept prompt ids: (sel_idx [H][F][Np], sel_count [H][F])."""
    _require(q_codes, "q_codes", torch.int32)
    _require(p_codes, "p_codes", torch.int32)
    H, L, NQ = q_codes.shape
    Hp, Lp, Np = p_codes.shape
    if (Hp, Lp) != (H, L) or NQ % frames:
        raise ValueError("q_codes [H][L][F*Nf] and p_codes [H][L][Np] disagree")
    if not (q_codes.is_contiguous() and p_codes.is_contiguous()):
        raise ValueError("codes must be contiguous")
    if sel_idx is None:
        sel_idx = torch.empty((H, frames, Np), dtype=torch.int32, device=q_codes.device)
    if sel_count is None:
        sel_count = torch.empty((H, frames), dtype=torch.int32, device=q_codes.device)
    _check(library().fastar_annca_select(_ptr(q_codes), NQ // frames, frames, _ptr(p_codes), Np,
                                         H, L, _ptr(sel_idx), _ptr(sel_count), _stream(stream)))
    return sel_idx, sel_count


def attend_subset(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, frames: int,
                  sel_idx: torch.Tensor | None = None, sel_count: torch.Tensor | None = None,
                  scale: float = 0.0, out: torch.Tensor | None = None, stream=None):
    """Each frame's queries attend over its kept prompt keys (or all, if no selection)."""
    _require(q, "q")
    _require(k, "k", q.dtype)
    _require(v, "v", q.dtype)
    H, NQ, d = q.shape
    Np = k.shape[1]
    if k.shape != v.shape or k.stride() != v.stride() or NQ % frames:
        raise ValueError("bad shapes")
    if (sel_idx is None) != (sel_count is None):
        raise ValueError("sel_idx and sel_count go together")
    if sel_idx is not None:
        _require(sel_idx, "sel_idx", torch.int32)
        _require(sel_count, "sel_count", torch.int32)
        if tuple(sel_idx.shape) != (H, frames, Np) or tuple(sel_count.shape) != (H, frames):
            raise ValueError("selection shapes disagree with q/k")
    if out is None:
        out = torch.empty_like(q)
    dt = BF16 if q.dtype == torch.bfloat16 else F32
    _check(library().fastar_attend_subset(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        _ptr(sel_idx), _ptr(sel_count), NQ // frames, frames, Np, H, d, dt, float(scale),
        _ptr(out), out.stride(0), out.stride(1), _stream(stream)))
    return out


def annca_attend_static(q: torch.Tensor, q_codes: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        p_codes: torch.Tensor, frames: int, scale: float = 0.0,
                        out: torch.Tensor | None = None, stream=None):
    """AnnCA select + sparse attention with the selection in the library's
    static device array (no device allocation inside the call; `out` is
    allocated here only when not given)."""
    _require(q, "q")
    _require(k, "k", q.dtype)
    _require(v, "v", q.dtype)
    _require(q_codes, "q_codes", torch.int32)
    _require(p_codes, "p_codes", torch.int32)
    H, NQ, d = q.shape
    Np = k.shape[1]
    L = q_codes.shape[1]
    if k.shape != v.shape or k.stride() != v.stride() or NQ % frames:
        raise ValueError("bad shapes")
    if tuple(q_codes.shape) != (H, L, NQ) or tuple(p_codes.shape) != (H, L, Np):
        raise ValueError("q_codes [H][L][F*Nf] and p_codes [H][L][Np] disagree")
    if not (q_codes.is_contiguous() and p_codes.is_contiguous()):
        raise ValueError("codes must be contiguous")
    if out is None:
        out = torch.empty_like(q)
    dt = BF16 if q.dtype == torch.bfloat16 else F32
    _check(library().fastar_annca_attend_static(
        _ptr(q), q.stride(0), q.stride(1), _ptr(q_codes), _ptr(k), _ptr(v), k.stride(0),
        k.stride(1), _ptr(p_codes), NQ // frames, frames, Np, H, d, L, dt, float(scale),
        _ptr(out), out.stride(0), out.stride(1), _stream(stream)))
    return out


def annca_attend(q: torch.Tensor, q_planes: torch.Tensor, tables: int, bits: int,
                 p_codes: torch.Tensor, k: torch.Tensor, v: torch.Tensor, frames: int,
                 scale: float = 0.0, out: torch.Tensor | None = None,
                 q_codes: torch.Tensor | None = None, stream=None):
    """The AnnCA step in two launches: hash the queries into q_codes ([H][L][NQ]
    int32, allocated when not given), then per frame keep the prompt rows that
    share a bucket with its queries and attend over the kept rows, selection in
    the attention kernel's prologue (bf16, d = 128)."""
    _require(q, "q", torch.bfloat16)
    _require(k, "k", torch.bfloat16)
    _require(v, "v", torch.bfloat16)
    _require(q_planes, "q_planes", torch.bfloat16)
    _require(p_codes, "p_codes", torch.int32)
    H, NQ, d = q.shape
    Np = k.shape[1]
    if k.shape != v.shape or k.stride() != v.stride() or NQ % frames:
        raise ValueError("bad shapes")
    if tuple(p_codes.shape) != (H, tables, Np) or not p_codes.is_contiguous():
        raise ValueError("p_codes must be contiguous [H][L][Np]")
    if not q_planes.is_contiguous() or q_planes.numel() != tables * bits * d:
        raise ValueError("q_planes must be contiguous [L][b][d]")
    if out is None:
        out = torch.empty_like(q)
    if q_codes is None:
        q_codes = torch.empty((H, tables, NQ), dtype=torch.int32, device=q.device)
    _require(q_codes, "q_codes", torch.int32)
    if tuple(q_codes.shape) != (H, tables, NQ) or not q_codes.is_contiguous():
        raise ValueError("q_codes must be contiguous [H][L][NQ]")
    _check(library().fastar_annca_attend(
        _ptr(q), q.stride(0), q.stride(1), _ptr(q_planes), tables, bits, _ptr(q_codes),
        _ptr(p_codes), _ptr(k), _ptr(v), k.stride(0), k.stride(1), NQ // frames, frames, Np, H, d,
        float(scale),
        _ptr(out), out.stride(0), out.stride(1), _stream(stream)))
    return out


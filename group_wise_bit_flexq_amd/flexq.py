"""Python binding of libflexq.so (include/flexq.h): argument marshalling only.

Device memory and streams come from PyTorch; every step of the computation runs in
the library's HIP kernels.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflexq.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_DEVICE = 0, -1, -2, -3

EXPORTED = (
    "flexq_status_string", "flexq_quantize", "flexq_quantize_w4", "flexq_quantize_ex",
    "flexq_dequantize", "flexq_dequantize_ex", "flexq_layernorm",
    "flexq_linear_w4_workspace_size", "flexq_linear_w4", "flexq_linear_w4_f32",
    "flexq_attn_prefill", "flexq_attn_decode_workspace_size", "flexq_attn_decode_kv4",
    "flexq_attn_decode_kv4_static", "flexq_attn_decode_kv4_topk", "flexq_host_attn_decode_kv4",
    "flexq_host_stage_size",
    "flexq_embed", "flexq_argmax", "flexq_pick", "flexq_layer_workspace_size", "flexq_prefill_layer",
    "flexq_decode_layer", "flexq_model_workspace_size", "flexq_prefill", "flexq_decode_step",
    "flexq_probe_mfma",
)


class FlexqError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed: {msg} ({status})")
        self.status = status


# ------------------------------------------------------------------ C structs

class QConfig(C.Structure):
    _fields_ = [("num_bits", C.c_int32), ("group_size", C.c_int32), ("symmetric", C.c_int32)]


class W4Struct(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("params", C.c_void_p), ("rows", C.c_int64),
                ("cols", C.c_int64)]


class KV4Struct(C.Structure):
    _fields_ = [("k_codes", C.c_void_p), ("v_codes", C.c_void_p), ("k_params", C.c_void_p),
                ("v_params", C.c_void_p), ("batch", C.c_int32), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_len", C.c_int32), ("pad", C.c_void_p)]


class LayerStruct(C.Structure):
    _fields_ = [("ln1_g", C.c_void_p), ("ln1_b", C.c_void_p), ("wqkv", W4Struct),
                ("bqkv", C.c_void_p), ("wo", W4Struct), ("bo", C.c_void_p),
                ("ln2_g", C.c_void_p), ("ln2_b", C.c_void_p), ("w1", W4Struct),
                ("b1", C.c_void_p), ("w2", W4Struct), ("b2", C.c_void_p)]


class TraceStruct(C.Structure):
    _fields_ = [("events", C.POINTER(C.c_void_p)), ("kinds", C.POINTER(C.c_int32)),
                ("rows", C.POINTER(C.c_int64)), ("capacity", C.c_int32), ("count", C.c_int32)]


class GenConfig(C.Structure):
    """flexq_gen_config: greedy or temperature sampling, optional stop token."""
    _fields_ = [("do_sample", C.c_int32), ("temperature", C.c_float), ("seed", C.c_uint64),
                ("stop", C.c_int32)]


class HostTierStruct(C.Structure):
    """flexq_host_tier: cache rows >= row0 in host memory, attended on the CPU."""
    _fields_ = [("kv", C.POINTER(KV4Struct)), ("row0", C.c_int32), ("threads", C.c_int32),
                ("host_ws", C.c_void_p), ("host_ws_bytes", C.c_size_t),
                ("stage", C.c_void_p), ("stage_bytes", C.c_size_t)]


class TapStruct(C.Structure):
    """flexq_tap: copies of the hidden state entering listed layers."""
    _fields_ = [("count", C.c_int32), ("layers", C.POINTER(C.c_int32)),
                ("x", C.POINTER(C.c_void_p)), ("rows_cap", C.c_int64)]


class ModelStruct(C.Structure):
    _fields_ = [("layers", C.c_int32), ("hidden", C.c_int32), ("heads", C.c_int32),
                ("ffn", C.c_int32), ("vocab", C.c_int32), ("pos_rows", C.c_int32),
                ("layer", C.POINTER(LayerStruct)), ("kv", C.POINTER(KV4Struct)),
                ("embed", W4Struct), ("pos", C.c_void_p), ("lnf_g", C.c_void_p),
                ("lnf_b", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("trace", C.POINTER(TraceStruct)),
                ("gen", C.POINTER(GenConfig)), ("stopped", C.c_void_p),
                ("attn_sparsity", C.c_float), ("host", C.POINTER(HostTierStruct)),
                ("tap", C.POINTER(TapStruct))]


_lib = None


def lib():
    """Load libflexq.so (after torch, so that torch's HIP runtime is the one in use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (or python group_wise_bit_flexq_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        sig = {
            "flexq_status_string": (C.c_char_p, [C.c_int]),
            "flexq_quantize": (C.c_int, [vp, i64, i64, QConfig, vp, vp, vp]),
            "flexq_quantize_w4": (C.c_int, [vp, i64, i64, QConfig, vp, vp, vp]),
            "flexq_quantize_ex": (C.c_int, [vp, i64, i64, i64, QConfig, vp, vp, vp]),
            "flexq_dequantize_ex": (C.c_int, [vp, vp, i64, i64, i64, QConfig, vp, vp]),
            "flexq_dequantize": (C.c_int, [vp, vp, i64, i64, vp, vp]),
            "flexq_layernorm": (C.c_int, [vp, i64, i64, i64, vp, vp, vp, vp]),
            "flexq_linear_w4_workspace_size": (sz, [i64, i64, i64]),
            "flexq_linear_w4": (C.c_int, [vp, i64, C.POINTER(W4Struct), vp, vp, i32, vp, vp, sz, vp]),
            "flexq_linear_w4_f32": (C.c_int, [vp, i64, C.POINTER(W4Struct), vp, vp, sz, vp]),
            "flexq_attn_prefill": (C.c_int, [vp, i32, i32, i32, C.POINTER(KV4Struct), vp, vp]),
            "flexq_attn_decode_workspace_size": (sz, [i32, i32, i32, i32]),
            "flexq_attn_decode_kv4": (C.c_int, [vp, i32, i32, i32, C.POINTER(KV4Struct), vp, vp,
                                                sz, vp]),
            "flexq_attn_decode_kv4_static": (C.c_int, [vp, i32, i32, i32, C.POINTER(KV4Struct),
                                                       vp, vp]),
            "flexq_attn_decode_kv4_topk": (C.c_int, [vp, i32, i32, i32, C.POINTER(KV4Struct),
                                                     C.c_float, vp, vp]),
            "flexq_host_attn_decode_kv4": (C.c_int, [vp, i32, i32, i32, C.POINTER(KV4Struct),
                                                     vp, i32]),
            "flexq_host_stage_size": (sz, [i32, i32, i32, i32]),
            "flexq_embed": (C.c_int, [vp, i64, i32, i32, vp, C.POINTER(W4Struct), vp, i32, vp,
                                      vp]),
            "flexq_argmax": (C.c_int, [vp, i64, i64, vp, vp]),
            "flexq_pick": (C.c_int, [vp, i64, i64, C.POINTER(GenConfig), i32, i32, vp, vp, vp]),
            "flexq_layer_workspace_size": (sz, [i32, i32, i32, i64, i32]),
            "flexq_prefill_layer": (C.c_int, [C.POINTER(LayerStruct), C.POINTER(KV4Struct), i32,
                                              i32, i32, vp, i32, i32, i32, vp, vp, sz, vp]),
            "flexq_decode_layer": (C.c_int, [C.POINTER(LayerStruct), C.POINTER(KV4Struct), i32,
                                             i32, i32, vp, i32, i32, i32, vp, vp, sz, vp]),
            "flexq_model_workspace_size": (sz, [i32, i32, i32, i32, i64, i32, i32]),
            "flexq_prefill": (C.c_int, [C.POINTER(ModelStruct), vp, i32, i32, i32, vp, vp, vp]),
            "flexq_decode_step": (C.c_int, [C.POINTER(ModelStruct), vp, i32, i32, vp, vp, vp]),
            "flexq_probe_mfma": (C.c_int, [i32, i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(name, status):
    if status != OK:
        msg = lib().flexq_status_string(status).decode()
        raise FlexqError(name, status, msg)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} CUDA tensor")


# ------------------------------------------------------------------ compressed tensors

class Q4:
    """A group-wise 4-bit tensor [rows][cols] in row-major group order (flexq_quantize):
    codes uint8 [rows][cols/2], params fp16 [rows][cols/64][2]."""

    def __init__(self, codes: torch.Tensor, params: torch.Tensor):
        self.codes, self.params = codes, params
        self.rows, self.cols = codes.shape[0], codes.shape[1] * 2

    @staticmethod
    def empty(rows, cols, device="cuda"):
        return Q4(torch.empty(rows, cols // 2, dtype=torch.uint8, device=device),
                  torch.empty(rows, cols // 64, 2, dtype=torch.float16, device=device))


W4_BLOCK_ROWS = 128


class W4:
    """A 4-bit weight [rows][cols] in the weight layout of flexq_w4: rows in blocks of
    128, k-tile major, codes of each 4-byte word with its first four in the low nibbles.
    codes uint8 [rows_pad/128][cols/64][128][32], params fp16 [rows_pad/128][cols/64][128][2]
    (rows_pad = rows rounded up to 128, pad rows zero)."""

    def __init__(self, codes: torch.Tensor, params: torch.Tensor, rows: int):
        if codes.dim() != 4 or codes.shape[2:] != (W4_BLOCK_ROWS, 32):
            raise ValueError("W4 codes: expected [blocks][cols/64][128][32]")
        self.codes, self.params = codes, params
        self.rows, self.cols = rows, codes.shape[1] * 64
        if codes.shape[0] * W4_BLOCK_ROWS < rows:
            raise ValueError("W4 codes: fewer blocks than rows need")

    def c(self) -> W4Struct:
        return W4Struct(self.codes.data_ptr(), self.params.data_ptr(), self.rows, self.cols)

    @staticmethod
    def empty(rows, cols, device="cuda"):
        nb, kt = (rows + W4_BLOCK_ROWS - 1) // W4_BLOCK_ROWS, cols // 64
        return W4(torch.empty(nb, kt, W4_BLOCK_ROWS, 32, dtype=torch.uint8, device=device),
                  torch.empty(nb, kt, W4_BLOCK_ROWS, 2, dtype=torch.float16, device=device), rows)

    @staticmethod
    def from_rowmajor(codes: torch.Tensor, params: torch.Tensor) -> "W4":
        """Reorders row-major codes [rows][cols/2] and params [rows][cols/64][2] (as
        flexq_quantize writes them) into the weight layout; a permutation, no arithmetic."""
        rows, kt = codes.shape[0], codes.shape[1] // 32
        nb = (rows + W4_BLOCK_ROWS - 1) // W4_BLOCK_ROWS
        pad = nb * W4_BLOCK_ROWS - rows
        c = torch.nn.functional.pad(codes, (0, 0, 0, pad)).view(nb, W4_BLOCK_ROWS, kt, 32)
        p = torch.nn.functional.pad(params, (0, 0, 0, 0, 0, pad)).view(nb, W4_BLOCK_ROWS, kt, 2)
        # within each 4-byte word: codes 0..7 of the word, then low nibbles = codes 0..3
        w = c.reshape(nb, W4_BLOCK_ROWS, kt, 8, 4)
        e = torch.stack((w & 15, w >> 4), dim=-1).reshape(nb, W4_BLOCK_ROWS, kt, 8, 8)
        c = (e[..., :4] | (e[..., 4:] << 4)).reshape(nb, W4_BLOCK_ROWS, kt, 32)
        return W4(c.permute(0, 2, 1, 3).contiguous(), p.permute(0, 2, 1, 3).contiguous(), rows)

    def rowmajor(self):
        """(codes [rows][cols/2], params [rows][cols/64][2]) in row-major group order."""
        nb, kt = self.codes.shape[0], self.codes.shape[1]
        w = self.codes.reshape(nb, kt, W4_BLOCK_ROWS, 8, 4)
        e = torch.cat((w & 15, w >> 4), dim=-1)              # codes 0..7 of each word
        w = e[..., 0::2] | (e[..., 1::2] << 4)              # back to the packed order
        c = w.reshape(nb, kt, W4_BLOCK_ROWS, 32).permute(0, 2, 1, 3)
        c = c.reshape(nb * W4_BLOCK_ROWS, kt * 32)[:self.rows]
        p = self.params.permute(0, 2, 1, 3).reshape(nb * W4_BLOCK_ROWS, kt, 2)[:self.rows]
        return c, p

    def nbytes(self):
        return self.codes.numel() + self.params.numel() * 2


class KV4:
    """The 4-bit KV cache of one layer (see flexq_kv4_layer); `pad` is None or a device
    int32 [batch] tensor of left-padding counts."""

    def __init__(self, batch, heads, head_dim, max_len, device="cuda", pad=None, pin=False):
        """device "cuda" for the GPU kernels; "cpu" for a host-memory cache (pinned with
        pin=True, for asynchronous copies) served by flexq_host_attn_decode_kv4."""
        self.batch, self.heads, self.head_dim, self.max_len = batch, heads, head_dim, max_len
        dev = torch.device(device)
        if pad is not None:
            if pad.dtype != torch.int32 or not pad.is_contiguous() or pad.device.type != dev.type:
                raise ValueError(f"pad: expected a contiguous int32 tensor on {dev.type}")
            if pad.numel() < batch:
                raise ValueError("pad: at least one entry per cache row")
        self.pad = pad
        shp = (batch, heads, max_len, head_dim // 2)
        pshp = (batch, heads, max_len, head_dim // 64, 2)
        kw = dict(device=dev, pin_memory=True) if (pin and dev.type == "cpu") else dict(device=dev)
        self.k_codes = torch.zeros(shp, dtype=torch.uint8, **kw)
        self.v_codes = torch.zeros(shp, dtype=torch.uint8, **kw)
        self.k_params = torch.zeros(pshp, dtype=torch.float16, **kw)
        self.v_params = torch.zeros(pshp, dtype=torch.float16, **kw)

    def c(self) -> KV4Struct:
        return KV4Struct(self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                         self.k_params.data_ptr(), self.v_params.data_ptr(), self.batch,
                         self.heads, self.head_dim, self.max_len, _ptr(self.pad))

    def nbytes(self):
        return 2 * (self.k_codes.numel() + self.k_params.numel() * 2)


# ------------------------------------------------------------------ single calls

QCFG = QConfig(4, 64, 0)


def quantize(x: torch.Tensor, out: Q4 | None = None, stream=None) -> Q4:
    """Group-wise 4-bit quantization along the last dimension (row-major groups)."""
    _need(x, torch.float16, "x")
    rows = x.numel() // x.shape[-1]
    cols = x.shape[-1]
    q = out if out is not None else Q4.empty(rows, cols, x.device)
    _check("flexq_quantize", lib().flexq_quantize(x.data_ptr(), rows, cols, QCFG,
                                                  q.codes.data_ptr(), q.params.data_ptr(),
                                                  _stream(stream)))
    return q


def quantize_weight(x: torch.Tensor, out: W4 | None = None, stream=None) -> W4:
    """The same quantization written in the weight layout the GEMMs read (flexq_quantize_w4)."""
    _need(x, torch.float16, "x")
    rows = x.numel() // x.shape[-1]
    cols = x.shape[-1]
    w = out if out is not None else W4.empty(rows, cols, x.device)
    _check("flexq_quantize_w4", lib().flexq_quantize_w4(x.data_ptr(), rows, cols, QCFG,
                                                        w.codes.data_ptr(), w.params.data_ptr(),
                                                        _stream(stream)))
    return w


def dequantize(q: Q4, stream=None) -> torch.Tensor:
    out = torch.empty(q.rows, q.cols, dtype=torch.float16, device=q.codes.device)
    _check("flexq_dequantize", lib().flexq_dequantize(q.codes.data_ptr(), q.params.data_ptr(),
                                                      q.rows, q.cols, out.data_ptr(),
                                                      _stream(stream)))
    return out


def _split_dims(shape, group_dim):
    gd = group_dim % len(shape)
    outer = 1
    for d in shape[:gd]:
        outer *= d
    inner = 1
    for d in shape[gd + 1:]:
        inner *= d
    return gd, outer, shape[gd], inner


def quantize_ex(x: torch.Tensor, num_bits=4, group_size=64, group_dim=-1, symmetric=False,
                stream=None):
    """General compression config (flexq_quantize_ex): returns (codes, params) with codes
    uint8 shape[:gd] + (ng * group_size * num_bits / 8,) + shape[gd+1:] and params fp16
    shape[:gd] + (ng,) + shape[gd+1:] + (2,), ng = ceil(shape[gd] / group_size)."""
    _need(x, torch.float16, "x")
    shape = tuple(x.shape)
    gd, outer, n, inner = _split_dims(shape, group_dim)
    ng = -(-n // group_size)
    gb = group_size * num_bits // 8
    codes = torch.empty(shape[:gd] + (ng * gb,) + shape[gd + 1:], dtype=torch.uint8, device=x.device)
    params = torch.empty(shape[:gd] + (ng,) + shape[gd + 1:] + (2,), dtype=torch.float16,
                         device=x.device)
    cfg = QConfig(num_bits, group_size, 1 if symmetric else 0)
    _check("flexq_quantize_ex", lib().flexq_quantize_ex(x.data_ptr(), outer, n, inner, cfg,
                                                        codes.data_ptr(), params.data_ptr(),
                                                        _stream(stream)))
    return codes, params


def dequantize_ex(codes: torch.Tensor, params: torch.Tensor, n, num_bits=4, group_size=64,
                  group_dim=-1, symmetric=False, stream=None) -> torch.Tensor:
    """fp16 values of `quantize_ex`'s output, the grouped axis back to its n elements."""
    shape = tuple(codes.shape)
    gd, outer, _, inner = _split_dims(shape, group_dim)
    out = torch.empty(shape[:gd] + (n,) + shape[gd + 1:], dtype=torch.float16, device=codes.device)
    cfg = QConfig(num_bits, group_size, 1 if symmetric else 0)
    _check("flexq_dequantize_ex", lib().flexq_dequantize_ex(codes.data_ptr(), params.data_ptr(),
                                                            outer, n, inner, cfg, out.data_ptr(),
                                                            _stream(stream)))
    return out


def layernorm(x, g, b, rows=None, row_stride=None, out=None, stream=None):
    h = g.numel()
    M = rows if rows is not None else x.numel() // h
    stride = row_stride if row_stride is not None else h
    y = out if out is not None else torch.empty(M, h, dtype=torch.float16, device=x.device)
    _check("flexq_layernorm", lib().flexq_layernorm(x.data_ptr(), M, h, stride, g.data_ptr(),
                                                    b.data_ptr(), y.data_ptr(), _stream(stream)))
    return y


def linear_ws_bytes(M, N, K):
    return lib().flexq_linear_w4_workspace_size(M, N, K)


def _ws(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def linear_w4(x, w: W4, bias=None, residual=None, relu=False, out=None, ws=None, stream=None):
    _need(x, torch.float16, "x")
    M = x.numel() // w.cols
    y = out if out is not None else torch.empty(M, w.rows, dtype=torch.float16, device=x.device)
    _need(y, torch.float16, "out")
    if ws is None:
        ws = _ws(linear_ws_bytes(M, w.rows, w.cols), x.device)
    wc = w.c()
    _check("flexq_linear_w4", lib().flexq_linear_w4(
        x.data_ptr(), M, C.byref(wc), _ptr(bias), _ptr(residual), int(relu), y.data_ptr(),
        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return y


def linear_w4_f32(x, w: W4, out=None, ws=None, stream=None):
    _need(x, torch.float16, "x")
    M = x.numel() // w.cols
    y = out if out is not None else torch.empty(M, w.rows, dtype=torch.float32, device=x.device)
    _need(y, torch.float32, "out")
    if ws is None:
        ws = _ws(linear_ws_bytes(M, w.rows, w.cols), x.device)
    wc = w.c()
    _check("flexq_linear_w4_f32", lib().flexq_linear_w4_f32(
        x.data_ptr(), M, C.byref(wc), y.data_ptr(), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream(stream)))
    return y


def attn_prefill(qkv, B, S, kv: KV4, b0=0, out=None, stream=None):
    _need(qkv, torch.float16, "qkv")
    h = kv.heads * kv.head_dim
    y = out if out is not None else torch.empty(B * S, h, dtype=torch.float16, device=qkv.device)
    kc = kv.c()
    _check("flexq_attn_prefill", lib().flexq_attn_prefill(qkv.data_ptr(), B, S, b0, C.byref(kc),
                                                          y.data_ptr(), _stream(stream)))
    return y


def attn_decode_ws_bytes(B, heads, head_dim, pos):
    return lib().flexq_attn_decode_workspace_size(B, heads, head_dim, pos)


def attn_decode(qkv, pos, kv: KV4, b0=0, out=None, ws=None, stream=None):
    _need(qkv, torch.float16, "qkv")
    B = qkv.shape[0]
    h = kv.heads * kv.head_dim
    y = out if out is not None else torch.empty(B, h, dtype=torch.float16, device=qkv.device)
    if ws is None:
        ws = _ws(attn_decode_ws_bytes(B, kv.heads, kv.head_dim, pos), qkv.device)
    kc = kv.c()
    _check("flexq_attn_decode_kv4", lib().flexq_attn_decode_kv4(
        qkv.data_ptr(), B, b0, pos, C.byref(kc), y.data_ptr(), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))
    return y


def host_attn_decode(qkv, pos, kv: KV4, b0=0, out=None, threads=0):
    """Decode attention on the host CPU over a host-memory cache (CPU tensors)."""
    if qkv.device.type != "cpu" or qkv.dtype != torch.float16 or not qkv.is_contiguous():
        raise ValueError("qkv: expected a contiguous float16 CPU tensor")
    if kv.k_codes.device.type != "cpu":
        raise ValueError("kv: expected a host-memory cache")
    B = qkv.shape[0]
    h = kv.heads * kv.head_dim
    y = out if out is not None else torch.empty(B, h, dtype=torch.float16)
    kc = kv.c()
    _check("flexq_host_attn_decode_kv4", lib().flexq_host_attn_decode_kv4(
        qkv.data_ptr(), B, b0, pos, C.byref(kc), y.data_ptr(), int(threads)))
    return y


def attn_decode_topk(qkv, pos, kv: KV4, sparsity, b0=0, out=None, stream=None):
    """Sparse decode attention: each query keeps its ceil(sparsity * n) best positions."""
    _need(qkv, torch.float16, "qkv")
    B = qkv.shape[0]
    h = kv.heads * kv.head_dim
    y = out if out is not None else torch.empty(B, h, dtype=torch.float16, device=qkv.device)
    kc = kv.c()
    _check("flexq_attn_decode_kv4_topk", lib().flexq_attn_decode_kv4_topk(
        qkv.data_ptr(), B, b0, pos, C.byref(kc), float(sparsity), y.data_ptr(),
        _stream(stream)))
    return y


def embed(tokens, pos_base, seq, emb: W4, pos_table, out=None, stream=None, pad=None):
    _need(tokens, torch.int32, "tokens")
    n = tokens.numel()
    y = out if out is not None else torch.empty(n, emb.cols, dtype=torch.float16,
                                                device=tokens.device)
    if pad is not None:
        _need(pad, torch.int32, "pad")
    ec = emb.c()
    _check("flexq_embed", lib().flexq_embed(tokens.data_ptr(), n, pos_base, seq, _ptr(pad),
                                            C.byref(ec),
                                            pos_table.data_ptr(), pos_table.shape[0],
                                            y.data_ptr(), _stream(stream)))
    return y


def probe_mfma(mode, blocks, iters, out=None, stream=None):
    """Matrix-core rate probe (flexq_probe_mfma): returns the checksum tensor."""
    y = out if out is not None else torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    _check("flexq_probe_mfma", lib().flexq_probe_mfma(int(mode), int(blocks), int(iters),
                                                      y.data_ptr(), _stream(stream)))
    return y


def argmax(logits, out=None, stream=None):
    M, N = logits.shape
    y = out if out is not None else torch.empty(M, dtype=torch.int32, device=logits.device)
    _check("flexq_argmax", lib().flexq_argmax(logits.data_ptr(), M, N, y.data_ptr(),
                                              _stream(stream)))
    return y


def gen_config(do_sample=False, temperature=1.0, seed=0, stop=-1):
    return GenConfig(int(bool(do_sample)), float(temperature), int(seed) & (2**64 - 1), int(stop))


def pick(logits, gen=None, step=0, m0=0, stopped=None, out=None, stream=None):
    """Next tokens from fp32 logits [M][N] (flexq_pick); `gen` a GenConfig or None,
    `stopped` None or a device int32 [M] tensor updated in place."""
    M, N = logits.shape
    _need(logits, torch.float32, "logits")
    y = out if out is not None else torch.empty(M, dtype=torch.int32, device=logits.device)
    if stopped is not None:
        _need(stopped, torch.int32, "stopped")
    _check("flexq_pick", lib().flexq_pick(logits.data_ptr(), M, N,
                                          None if gen is None else C.byref(gen), step, m0,
                                          _ptr(stopped), y.data_ptr(), _stream(stream)))
    return y


# ------------------------------------------------------------------ layers and models

class QLayer:
    """fp16 vectors + four W4 matrices of one decoder layer, resident on the device."""

    VECS = ("ln1_g", "ln1_b", "bqkv", "bo", "ln2_g", "ln2_b", "b1", "b2")
    MATS = ("wqkv", "wo", "w1", "w2")

    def __init__(self, vecs: dict, mats: dict, heads: int):
        self.v = vecs
        self.m = mats
        self.heads = heads
        self.hidden = mats["wo"].rows
        self.ffn = mats["w1"].rows
        self.head_dim = self.hidden // heads

    @staticmethod
    def from_fp16(w16: dict, heads: int, device="cuda", stream=None):
        """Quantizes the four matrices with flexq_quantize_w4; vectors stay fp16."""
        vecs = {k: w16[k].to(device).contiguous() for k in QLayer.VECS}
        mats = {k: quantize_weight(w16[k].to(device).contiguous(), stream=stream)
                for k in QLayer.MATS}
        return QLayer(vecs, mats, heads)

    def c(self) -> LayerStruct:
        v, m = self.v, self.m
        return LayerStruct(v["ln1_g"].data_ptr(), v["ln1_b"].data_ptr(), m["wqkv"].c(),
                           v["bqkv"].data_ptr(), m["wo"].c(), v["bo"].data_ptr(),
                           v["ln2_g"].data_ptr(), v["ln2_b"].data_ptr(), m["w1"].c(),
                           v["b1"].data_ptr(), m["w2"].c(), v["b2"].data_ptr())

    def weight_bytes(self):
        return sum(w.nbytes() for w in self.m.values())


def layer_ws_bytes(hidden, heads, ffn, rows, max_len):
    return lib().flexq_layer_workspace_size(hidden, heads, ffn, rows, max_len)


def prefill_layer(layer: QLayer, kv: KV4, x, nb, S, b0=0, out=None, ws=None, stream=None):
    _need(x, torch.float16, "x")
    y = out if out is not None else torch.empty_like(x)
    if ws is None:
        ws = _ws(layer_ws_bytes(layer.hidden, layer.heads, layer.ffn, nb * S, 0), x.device)
    lc, kc = layer.c(), kv.c()
    _check("flexq_prefill_layer", lib().flexq_prefill_layer(
        C.byref(lc), C.byref(kc), layer.hidden, layer.heads, layer.ffn, x.data_ptr(), nb, S, b0,
        y.data_ptr(), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return y


def decode_layer(layer: QLayer, kv: KV4, x, pos, b0=0, out=None, ws=None, stream=None):
    _need(x, torch.float16, "x")
    B = x.shape[0]
    y = out if out is not None else torch.empty_like(x)
    if ws is None:
        ws = _ws(layer_ws_bytes(layer.hidden, layer.heads, layer.ffn, B, pos + 1), x.device)
    lc, kc = layer.c(), kv.c()
    _check("flexq_decode_layer", lib().flexq_decode_layer(
        C.byref(lc), C.byref(kc), layer.hidden, layer.heads, layer.ffn, x.data_ptr(), B, b0, pos,
        y.data_ptr(), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return y


class QModel:
    """An OPT-shaped model with 4-bit weights and per-layer 4-bit KV caches.

    host_rows > 0 keeps the caches of the last host_rows sequences in pinned host
    memory (flexq_host_tier): their decode attention runs on host_threads CPU threads;
    their prefill micro-batches (at most max_prefill_batch sequences) go through a
    device staging area."""

    def __init__(self, layers: list, embed_w4: W4, pos16, lnf_g, lnf_b, heads, batch, max_len,
                 max_prefill_rows, device="cuda", host_rows=0, host_threads=0,
                 max_prefill_batch=None):
        self.layers = layers
        self.embed = embed_w4
        self.pos = pos16
        self.lnf_g, self.lnf_b = lnf_g, lnf_b
        self.heads = heads
        self.hidden = embed_w4.cols
        self.vocab = embed_w4.rows
        self.ffn = layers[0].ffn
        self.batch, self.max_len = batch, max_len
        hd = self.hidden // heads
        if not 0 <= host_rows <= batch:
            raise ValueError("host_rows outside [0, batch]")
        self.row0 = batch - host_rows
        # left padding of each cache row, shared by every layer's cache (0: none); the
        # device array covers every row (the embedding reads it), the host one the host rows
        self.pad = torch.zeros(batch, dtype=torch.int32, device=device)
        self.caches = [KV4(self.row0, heads, hd, max_len, device, pad=self.pad) for _ in layers]
        nbytes = lib().flexq_model_workspace_size(self.hidden, heads, self.ffn, self.vocab,
                                                  max_prefill_rows, batch, max_len)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._layer_arr = (LayerStruct * len(layers))(*[L.c() for L in layers])
        self._kv_arr = (KV4Struct * len(layers))(*[k.c() for k in self.caches])
        self._struct = ModelStruct(len(layers), self.hidden, heads, self.ffn, self.vocab,
                                   pos16.shape[0], self._layer_arr, self._kv_arr, embed_w4.c(),
                                   pos16.data_ptr(), lnf_g.data_ptr(), lnf_b.data_ptr(),
                                   self.workspace.data_ptr(), nbytes)
        self.host_caches = []
        if host_rows > 0:
            self.host_pad = torch.zeros(host_rows, dtype=torch.int32, pin_memory=True)
            self.host_caches = [KV4(host_rows, heads, hd, max_len, "cpu", pad=self.host_pad,
                                    pin=True) for _ in layers]
            self._host_kv_arr = (KV4Struct * len(layers))(*[k.c() for k in self.host_caches])
            self.host_ws = torch.empty(host_rows * 4 * self.hidden, dtype=torch.float16,
                                       pin_memory=True)
            nb = max_prefill_batch or host_rows
            sb = lib().flexq_host_stage_size(heads, hd, nb, max_len)
            self.stage = torch.empty(max(sb, 16), dtype=torch.uint8, device=device)
            self._host = HostTierStruct(self._host_kv_arr, self.row0, int(host_threads),
                                        self.host_ws.data_ptr(), self.host_ws.numel() * 2,
                                        self.stage.data_ptr(), sb)
            self._struct.host = C.pointer(self._host)

    def set_tap(self, layers=None, rows=0):
        """Copy the hidden state entering each listed layer (len(layers) = the output
        head's input) on every following prefill / decode call of up to `rows` rows;
        returns the device buffers [rows][hidden], in the order of `layers`.  None
        removes the tap."""
        if not layers:
            self._tap = self._tap_bufs = None
            self._struct.tap = None
            return []
        dev = self.workspace.device
        self._tap_bufs = [torch.empty(rows, self.hidden, dtype=torch.float16, device=dev)
                          for _ in layers]
        self._tap_layers = (C.c_int32 * len(layers))(*layers)
        self._tap_ptrs = (C.c_void_p * len(layers))(*[b.data_ptr() for b in self._tap_bufs])
        self._tap = TapStruct(len(layers), self._tap_layers, self._tap_ptrs, rows)
        self._struct.tap = C.pointer(self._tap)
        return self._tap_bufs

    def set_attn_sparsity(self, sparsity=0.0):
        """Decode attention keeps each query's ceil(sparsity * n) best positions when
        0 < sparsity < 1; dense otherwise."""
        self._struct.attn_sparsity = float(sparsity)

    def set_generation(self, gen=None):
        """Greedy (None) or a GenConfig for the following prefill / decode calls; with a
        stop token the model keeps device stopped flags, one per cache row."""
        self._gen = gen
        self._struct.gen = None if gen is None else C.pointer(gen)
        self.stopped = None
        if gen is not None and gen.stop >= 0:
            self.stopped = torch.zeros(self.batch, dtype=torch.int32, device=self.workspace.device)
        self._struct.stopped = _ptr(self.stopped)

    def prefill(self, tokens, b0=0, logits=None, next_out=None, stream=None, pad=None):
        """Prefill of cache rows b0.. from tokens [nb][S]; `pad` (None or nb ints): left
        padding of each ragged prompt, recorded for the later decode steps."""
        _need(tokens, torch.int32, "tokens")
        nb, S = tokens.shape
        if b0 < 0 or b0 + nb > self.batch:
            raise ValueError("prefill rows outside the cache")
        p = torch.zeros(nb, dtype=torch.int32) if pad is None else \
            torch.as_tensor(pad, dtype=torch.int32).reshape(nb).cpu()
        self.pad[b0:b0 + nb].copy_(p)
        if self.host_caches and b0 >= self.row0:
            self.host_pad[b0 - self.row0:b0 - self.row0 + nb].copy_(p)
        nxt = next_out if next_out is not None else torch.empty(nb, dtype=torch.int32,
                                                                device=tokens.device)
        _need(nxt, torch.int32, "next_out")
        if logits is not None:
            _need(logits, torch.float32, "logits")
        _check("flexq_prefill", lib().flexq_prefill(C.byref(self._struct), tokens.data_ptr(), nb,
                                                    S, b0, nxt.data_ptr(), _ptr(logits),
                                                    _stream(stream)))
        return nxt

    def decode_step(self, tokens, pos, logits=None, next_out=None, stream=None):
        _need(tokens, torch.int32, "tokens")
        B = tokens.numel()
        nxt = next_out if next_out is not None else torch.empty(B, dtype=torch.int32,
                                                                device=tokens.device)
        _need(nxt, torch.int32, "next_out")
        if logits is not None:
            _need(logits, torch.float32, "logits")
        _check("flexq_decode_step", lib().flexq_decode_step(C.byref(self._struct),
                                                            tokens.data_ptr(), B, pos,
                                                            nxt.data_ptr(), _ptr(logits),
                                                            _stream(stream)))
        return nxt

    def weight_bytes(self):
        return sum(L.weight_bytes() for L in self.layers) + self.embed.nbytes()

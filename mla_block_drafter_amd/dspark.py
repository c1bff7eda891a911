"""ctypes binding of libdspark.so (include/dspark.h), argument marshalling only.

Device memory and streams come from PyTorch (ROCm build); every step of the
draft pass runs in the library's HIP kernels.  Loading fails loudly when the
library has not been built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark.so")

# ---- constants mirrored from include/dspark.h ----
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ENODEVICE, EPLANONLY = 0, -1, -2, -3, -4, -5, -6
DT_F32, DT_BF16, DT_Q8_0, DT_FP8_E4M3, DT_MXFP4 = 0, 1, 2, 3, 4
W_FC, W_FC_NORM, W_FINAL_NORM, W_LM_HEAD = 0, 1, 2, 3
W_MARKOV_W1, W_MARKOV_W2, W_CONF_W, W_CONF_B = 4, 5, 6, 7
W_LAYER_BASE, W_LAYER_STRIDE = 16, 16
L_KEYS = ["in_norm", "q_a", "q_a_norm", "kv_a", "kv_a_norm", "q_b", "kv_b", "o",
          "post_norm", "gate", "up", "down"]
CFG_LAYERS_ONLY, CFG_PLAN_ONLY = 1, 2

FMT_CODE = {"f32": DT_F32, "bf16": DT_BF16, "q8_0": DT_Q8_0, "fp8_e4m3": DT_FP8_E4M3, "mxfp4": DT_MXFP4}
TOP_IDS = {"fc": W_FC, "fc_norm": W_FC_NORM, "final_norm": W_FINAL_NORM, "lm_head": W_LM_HEAD,
           "markov_w1": W_MARKOV_W1, "markov_w2": W_MARKOV_W2, "conf_w": W_CONF_W, "conf_b": W_CONF_B}

EXPORTS = ["dspark_packed_bytes", "dspark_model_create", "dspark_model_destroy",
           "dspark_workspace_bytes", "dspark_draft_block", "dspark_layer_forward",
           "dspark_append_workspace_bytes", "dspark_cache_append",
           "dspark_verify_workspace_bytes", "dspark_verify",
           "dspark_accept_len", "dspark_accept_len_host", "dspark_dequant", "dspark_last_error",
           "dspark_draft_block_static", "dspark_read_probe"]
STATIC_SCRATCH_BYTES = 64 << 20


def layer_id(layer: int, key: str) -> int:
    return W_LAYER_BASE + layer * W_LAYER_STRIDE + L_KEYS.index(key)


def weight_id(name: str) -> int:
    """'fc' / 'L3.q_b' style names -> weight table id."""
    if name in TOP_IDS:
        return TOP_IDS[name]
    head, key = name.split(".", 1)
    return layer_id(int(head[1:]), key)


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ["hidden", "n_layers", "n_heads", "q_lora", "kv_lora", "qk_nope", "qk_rope", "v_head",
                 "inter", "vocab", "markov_rank", "block", "n_captured", "flags"]] + \
               [("rms_eps", C.c_float), ("rope_theta", C.c_float), ("yarn_factor", C.c_float),
                ("yarn_orig_ctx", C.c_int32), ("yarn_beta_fast", C.c_float), ("yarn_beta_slow", C.c_float)]


class Weight(C.Structure):
    _fields_ = [("id", C.c_int32), ("dtype", C.c_int32), ("data", C.c_void_p), ("scales", C.c_void_p),
                ("rows", C.c_int64), ("cols", C.c_int64)]


class BlockIn(C.Structure):
    _fields_ = [("n_seq", C.c_int32), ("act_dtype", C.c_int32), ("kv_dtype", C.c_int32), ("pad_", C.c_int32),
                ("total_ctx", C.c_int64), ("captured", C.c_void_p), ("kv", C.POINTER(C.c_void_p)),
                ("kv_offsets", C.c_void_p), ("prev_token", C.c_void_p), ("forced_prev", C.c_void_p),
                ("page_size", C.c_int32), ("max_pages", C.c_int32), ("block_table", C.c_void_p),
                ("sample_u", C.c_void_p), ("temperature", C.c_float), ("poll_limit", C.c_int32)]


class VerifyIn(C.Structure):
    _fields_ = [("n_seq", C.c_int32), ("block", C.c_int32), ("vocab", C.c_int32), ("method", C.c_int32),
                ("temperature", C.c_float), ("pad_", C.c_int32), ("draft", C.c_void_p),
                ("draft_logits", C.c_void_p), ("target_logits", C.c_void_p), ("u", C.c_void_p)]


VERIFY_TOKEN, VERIFY_BLOCK = 0, 1


class AppendIn(C.Structure):
    _fields_ = [("n_new", C.c_int32), ("act_dtype", C.c_int32), ("kv_dtype", C.c_int32), ("pad_", C.c_int32),
                ("captured", C.c_void_p), ("positions", C.c_void_p), ("slot_mapping", C.c_void_p),
                ("kv", C.POINTER(C.c_void_p))]


APPEND_MAX = 128


class BlockOut(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("conf", C.c_void_p), ("logits", C.c_void_p), ("hidden", C.c_void_p),
                ("stage_events", C.POINTER(C.c_void_p)), ("status", C.c_void_p)]


N_STAGES = 4
STAGES = ["fc", "layers", "lm_head", "markov"]


class DsparkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dspark error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libdspark.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built; run __graft_entry__.build() or "
                          "python mla_block_drafter_amd/build.py")
    L = C.CDLL(LIB_PATH)
    L.dspark_packed_bytes.restype = C.c_size_t
    L.dspark_packed_bytes.argtypes = [C.POINTER(Config), C.POINTER(Weight), C.c_int32]
    L.dspark_model_create.restype = C.c_int32
    L.dspark_model_create.argtypes = [C.POINTER(Config), C.POINTER(Weight), C.c_int32, C.c_void_p, C.c_size_t,
                                      C.c_void_p, C.POINTER(C.c_void_p)]
    L.dspark_model_destroy.restype = C.c_int32
    L.dspark_model_destroy.argtypes = [C.c_void_p]
    L.dspark_workspace_bytes.restype = C.c_size_t
    L.dspark_workspace_bytes.argtypes = [C.c_void_p, C.c_int32, C.c_int64]
    L.dspark_draft_block.restype = C.c_int32
    L.dspark_draft_block.argtypes = [C.c_void_p, C.POINTER(BlockIn), C.POINTER(BlockOut), C.c_void_p, C.c_size_t,
                                     C.c_void_p]
    L.dspark_draft_block_static.restype = C.c_int32
    L.dspark_draft_block_static.argtypes = [C.c_void_p, C.POINTER(BlockIn), C.POINTER(BlockOut), C.c_void_p]
    L.dspark_layer_forward.restype = C.c_int32
    L.dspark_layer_forward.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_int32, C.c_void_p, C.c_int64, C.c_void_p, C.c_size_t,
                                       C.c_void_p]
    L.dspark_append_workspace_bytes.restype = C.c_size_t
    L.dspark_append_workspace_bytes.argtypes = [C.c_void_p, C.c_int32]
    L.dspark_cache_append.restype = C.c_int32
    L.dspark_cache_append.argtypes = [C.c_void_p, C.POINTER(AppendIn), C.c_void_p, C.c_size_t, C.c_void_p]
    L.dspark_verify_workspace_bytes.restype = C.c_size_t
    L.dspark_verify_workspace_bytes.argtypes = [C.c_int32, C.c_int32]
    L.dspark_verify.restype = C.c_int32
    L.dspark_verify.argtypes = [C.POINTER(VerifyIn), C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    L.dspark_accept_len.restype = C.c_int32
    L.dspark_accept_len.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    L.dspark_accept_len_host.restype = C.c_int32
    L.dspark_accept_len_host.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
    L.dspark_dequant.restype = C.c_int32
    L.dspark_dequant.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]
    L.dspark_read_probe.restype = C.c_int32
    L.dspark_read_probe.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]
    L.dspark_last_error.restype = C.c_char_p
    L.dspark_last_error.argtypes = []
    _lib = L
    return L


def last_error() -> str:
    return lib().dspark_last_error().decode()


def check(rc: int) -> None:
    if rc != OK:
        raise DsparkError(rc, last_error())


def make_config(m, layers_only: bool = False, plan_only: bool = False) -> Config:
    """Fill the C config from any object with the ModelConfig attribute names."""
    c = Config()
    for f in ["hidden", "n_layers", "n_heads", "q_lora", "kv_lora", "qk_nope", "qk_rope", "v_head",
              "inter", "vocab", "markov_rank", "block", "n_captured"]:
        setattr(c, f, int(getattr(m, f)))
    c.flags = (CFG_LAYERS_ONLY if layers_only else 0) | (CFG_PLAN_ONLY if plan_only else 0)
    c.rms_eps, c.rope_theta, c.yarn_factor = float(m.rms_eps), float(m.rope_theta), float(m.yarn_factor)
    c.yarn_orig_ctx = int(m.yarn_orig_ctx)
    c.yarn_beta_fast, c.yarn_beta_slow = float(m.yarn_beta_fast), float(m.yarn_beta_slow)
    return c


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Model:
    """Packed model on the device.

    `tensors`: name -> (fmt, data, scales) with data / scales torch device
    tensors in the storage formats of include/dspark.h (scales None unless FP8).
    """

    def __init__(self, m, tensors: Dict[str, tuple], layers_only: bool = False, stream=None):
        import torch
        L = lib()
        self.cfg = make_config(m, layers_only)
        self.geometry = m
        table = (Weight * len(tensors))()
        for i, (name, (fmt, data, scales, rows, cols)) in enumerate(tensors.items()):
            table[i].id = weight_id(name)
            table[i].dtype = FMT_CODE[fmt]
            table[i].data = data.data_ptr()
            table[i].scales = None if scales is None else scales.data_ptr()
            table[i].rows, table[i].cols = int(rows), int(cols)
        nbytes = L.dspark_packed_bytes(C.byref(self.cfg), table, len(tensors))
        if nbytes == 0:
            raise DsparkError(EINVAL, last_error())
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        h = C.c_void_p()
        check(L.dspark_model_create(C.byref(self.cfg), table, len(tensors), self.packed.data_ptr(), nbytes,
                                    _stream_ptr(stream), C.byref(h)))
        self.handle = h
        self.packed_bytes = nbytes

    def close(self):
        if getattr(self, "handle", None):
            lib().dspark_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, n_seq: int, total_ctx: int) -> int:
        n = lib().dspark_workspace_bytes(self.handle, n_seq, total_ctx)
        if n == 0:
            raise DsparkError(EINVAL, last_error())
        return n

    def workspace(self, n_seq: int, total_ctx: int):
        import torch
        return torch.empty(self.workspace_bytes(n_seq, total_ctx), dtype=torch.uint8, device="cuda")

    def draft_block(self, captured, kv: Sequence, kv_offsets, prev_token, total_ctx: int, tokens, conf,
                    workspace, logits=None, hidden=None, forced_prev=None, stream=None,
                    stage_events=None, page_size: int = 0, block_table=None, sample_u=None,
                    temperature: float = 1.0, status=None, poll_limit: int = 0) -> None:
        """stage_events: optional list of 2*N_STAGES torch.cuda.Event (enable_timing).
        page_size > 0: kv holds page pools and block_table (int32 [n_seq][max_pages])
        maps each sequence's pages.  status: optional int32 device tensor [1]
        (1 when the Markov rollout's bounded wait expired; tokens are then -1);
        poll_limit: that wait's bound (0 default, < 0 expire at once).
        workspace None: dspark_draft_block_static (the library's static
        scratch, for callers that cannot allocate)."""
        import torch
        n_seq = int(prev_token.shape[0])
        kv_arr = (C.c_void_p * len(kv))(*[t.data_ptr() if t is not None else None for t in kv])
        bi = BlockIn()
        bi.n_seq = n_seq
        bi.act_dtype = DT_F32 if captured.dtype == torch.float32 else DT_BF16
        bi.kv_dtype = DT_F32 if kv[0] is not None and kv[0].dtype == torch.float32 else DT_BF16
        bi.total_ctx = int(total_ctx)
        bi.captured = captured.data_ptr()
        bi.kv = kv_arr
        bi.kv_offsets = kv_offsets.data_ptr()
        bi.prev_token = prev_token.data_ptr()
        bi.forced_prev = _ptr(forced_prev)
        if sample_u is not None:
            bi.sample_u = sample_u.data_ptr()
            bi.temperature = float(temperature)
        if page_size:
            bi.page_size = int(page_size)
            bi.max_pages = int(block_table.shape[1])
            bi.block_table = block_table.data_ptr()
        bi.poll_limit = int(poll_limit)
        bo = BlockOut(tokens.data_ptr(), conf.data_ptr(), _ptr(logits), _ptr(hidden), None, _ptr(status))
        if stage_events is not None:
            evs = (C.c_void_p * (2 * N_STAGES))(*[e.cuda_event for e in stage_events])
            bo.stage_events = evs
        if workspace is None:   # the library's static scratch (no allocation anywhere)
            check(lib().dspark_draft_block_static(self.handle, C.byref(bi), C.byref(bo), _stream_ptr(stream)))
        else:
            check(lib().dspark_draft_block(self.handle, C.byref(bi), C.byref(bo), workspace.data_ptr(),
                                           workspace.numel(), _stream_ptr(stream)))

    def layer_forward(self, layer: int, with_mlp: bool, x_in, x_out, kv, kv_offsets, total_ctx: int,
                      workspace, stream=None) -> None:
        import torch
        n_seq = int(kv_offsets.shape[0]) - 1
        kdt = DT_F32 if kv.dtype == torch.float32 else DT_BF16
        check(lib().dspark_layer_forward(self.handle, layer, int(with_mlp), n_seq, x_in.data_ptr(),
                                         x_out.data_ptr(), kv.data_ptr(), kdt, kv_offsets.data_ptr(),
                                         int(total_ctx), workspace.data_ptr(), workspace.numel(),
                                         _stream_ptr(stream)))

    def append_workspace(self, n_new: int):
        import torch
        n = lib().dspark_append_workspace_bytes(self.handle, n_new)
        if n == 0:
            raise DsparkError(EINVAL, last_error())
        return torch.empty(n, dtype=torch.uint8, device="cuda")

    def cache_append(self, captured, positions, slot_mapping, kv: Sequence, workspace, stream=None) -> None:
        """Latent rows of n_new verified positions into every layer's cache.
        captured: [n_new][n_captured][hidden] (bf16 or f32); positions: int32
        [n_new]; slot_mapping: int64 [n_new] destination rows; kv: per-layer
        caches or page pools viewed as rows of kv_lora + qk_rope."""
        import torch
        ai = AppendIn()
        ai.n_new = int(positions.shape[0])
        ai.act_dtype = DT_F32 if captured.dtype == torch.float32 else DT_BF16
        ai.kv_dtype = DT_F32 if kv[0].dtype == torch.float32 else DT_BF16
        ai.captured = captured.data_ptr()
        ai.positions = positions.data_ptr()
        ai.slot_mapping = slot_mapping.data_ptr()
        kv_arr = (C.c_void_p * len(kv))(*[t.data_ptr() for t in kv])
        ai.kv = kv_arr
        check(lib().dspark_cache_append(self.handle, C.byref(ai), workspace.data_ptr(), workspace.numel(),
                                        _stream_ptr(stream)))

    def dequant(self, name: str, out, stream=None) -> None:
        check(lib().dspark_dequant(self.handle, weight_id(name), out.data_ptr(), _stream_ptr(stream)))


def verify(draft, draft_logits, target_logits, u, temperature: float, method: int, out_len, out_token,
           stream=None, workspace=None) -> None:
    """Verification of sampled draft blocks (include/dspark.h, dspark_verify).
    draft int32 [n_seq][block]; draft_logits [n_seq][block][vocab];
    target_logits [n_seq][block + 1][vocab]; u [n_seq][block + 1]; workspace: a
    uint8 device tensor of at least verify_workspace_bytes (allocated here if None)."""
    import torch
    n_seq, block = draft.shape
    vi = VerifyIn()
    vi.n_seq, vi.block, vi.vocab, vi.method = int(n_seq), int(block), int(draft_logits.shape[-1]), int(method)
    vi.temperature = float(temperature)
    vi.draft, vi.draft_logits = draft.data_ptr(), draft_logits.data_ptr()
    vi.target_logits, vi.u = target_logits.data_ptr(), u.data_ptr()
    L = lib()
    nb = L.dspark_verify_workspace_bytes(int(n_seq), int(block))
    if nb == 0:
        raise DsparkError(EINVAL, last_error())
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if workspace is None else workspace
    check(L.dspark_verify(C.byref(vi), out_len.data_ptr(), out_token.data_ptr(), ws.data_ptr(), ws.numel(),
                          _stream_ptr(stream)))


def verify_workspace_bytes(n_seq: int, block: int) -> int:
    nb = lib().dspark_verify_workspace_bytes(int(n_seq), int(block))
    if nb == 0:
        raise DsparkError(EINVAL, last_error())
    return int(nb)


def accept_len(draft, verifier, out, stream=None) -> None:
    """Device acceptance length (int32 tensors [n_seq][block] -> [n_seq])."""
    n_seq, block = draft.shape
    check(lib().dspark_accept_len(draft.data_ptr(), verifier.data_ptr(), n_seq, block, out.data_ptr(),
                                  _stream_ptr(stream)))


def accept_len_host(draft, verifier):
    """Host acceptance length on numpy int32 arrays [n_seq][block]."""
    import numpy as np
    d = np.ascontiguousarray(draft, dtype=np.int32)
    v = np.ascontiguousarray(verifier, dtype=np.int32)
    out = np.zeros(d.shape[0], dtype=np.int32)
    check(lib().dspark_accept_len_host(d.ctypes.data, v.ctypes.data, d.shape[0], d.shape[1], out.ctypes.data))
    return out


READ_PROBE_WORDS = 2048


def read_probe(buf, out, stream=None) -> None:
    """Stream-read the device tensor `buf` once (dspark_read_probe); `out`:
    int32 device tensor of READ_PROBE_WORDS entries (one XOR word per
    workgroup)."""
    assert out.numel() >= READ_PROBE_WORDS and out.element_size() == 4
    check(lib().dspark_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                                  _stream_ptr(stream)))


def upload_stored(stored: Dict[str, object], device: str = "cuda") -> Dict[str, tuple]:
    """Host tensors in storage format (objects with fmt, shape, data, scales)
    -> the device tensor table Model() takes."""
    import numpy as np
    import torch
    out = {}
    for name, st in stored.items():
        shape = tuple(st.shape)
        rows, cols = (shape[0], shape[1]) if len(shape) == 2 else (shape[0], 1)
        data = torch.from_numpy(np.ascontiguousarray(st.data).view(np.uint8).reshape(-1)).to(device)
        scales = None if st.scales is None else torch.from_numpy(np.ascontiguousarray(st.scales)).to(device)
        out[name] = (st.fmt, data, scales, rows, cols)
    return out

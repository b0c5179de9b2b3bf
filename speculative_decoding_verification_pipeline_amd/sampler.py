"""Thin ctypes binding of libss_sampler.so (argument marshalling only).

Every computation runs in the HIP library; this module only turns torch device
tensors into the C ABI's pointers and sizes (include/ss_sampler.h) and passes
torch's current stream. It raises if the library is missing: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libss_sampler.so")

SS_OK = 0
SS_ERR_INVALID_ARG = -1
SS_ERR_UNSUPPORTED = -2
SS_ERR_OUT_OF_MEMORY = -3
SS_ERR_HIP = -4
SS_F32 = 0
SS_BF16 = 1

EXPORTED = ("ss_sampler_create", "ss_sampler_destroy", "ss_status_string",
            "ss_sampler_workspace_bytes", "ss_sampler_set_launch_events", "ss_sample",
            "ss_spec_verify", "ss_spec_verify_scatter", "ss_tree_verify", "ss_lmhead_sample",
            "ss_lmhead_sample_params", "ss_sample_noalloc")
NOALLOC_MAX_BATCH = 64
NOALLOC_MAX_ENTRIES = 1 << 23


class Config(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("vocab_size", ctypes.c_int32),
                ("max_draft", ctypes.c_int32), ("hidden_size", ctypes.c_int32),
                ("device", ctypes.c_int32)]


class CParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p),
                ("top_p", ctypes.c_void_p), ("min_p", ctypes.c_void_p),
                ("repetition_penalty", ctypes.c_void_p), ("frequency_penalty", ctypes.c_void_p),
                ("presence_penalty", ctypes.c_void_p), ("history_ids", ctypes.c_void_p),
                ("history_len", ctypes.c_void_p), ("history_stride", ctypes.c_int32),
                ("bias_ids", ctypes.c_void_p), ("bias_values", ctypes.c_void_p),
                ("bias_len", ctypes.c_void_p), ("bias_stride", ctypes.c_int32),
                ("grammar_mask", ctypes.c_void_p), ("mask_stride", ctypes.c_int32),
                ("request_ids", ctypes.c_void_p), ("positions", ctypes.c_void_p),
                ("seed", ctypes.c_uint64)]


class CDebug(ctypes.Structure):
    _fields_ = [("processed_logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_stride", ctypes.c_int32), ("kept_count", ctypes.c_void_p),
                ("probs", ctypes.c_void_p), ("path", ctypes.c_void_p)]


class CSequences(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_void_p), ("stride", ctypes.c_int64),
                ("capacity", ctypes.c_int32), ("len", ctypes.c_void_p)]


class SamplerError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


_lib = None


def load_library(path=None):
    """Load libss_sampler.so and declare its signatures (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = LIB_PATH if path is None else path
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    lib.ss_sampler_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
    lib.ss_sampler_create.restype = i32
    lib.ss_sampler_destroy.argtypes = [vp]
    lib.ss_sampler_destroy.restype = None
    lib.ss_status_string.argtypes = [i32]
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_sampler_workspace_bytes.argtypes = [vp]
    lib.ss_sampler_workspace_bytes.restype = i64
    lib.ss_sampler_set_launch_events.argtypes = [vp, ctypes.POINTER(vp), i32]
    lib.ss_sampler_set_launch_events.restype = i32
    lib.ss_sample.argtypes = [vp, vp, i32, i64, i32, ctypes.POINTER(CParams), vp,
                              ctypes.POINTER(CDebug), vp]
    lib.ss_sample.restype = i32
    lib.ss_spec_verify.argtypes = [vp, vp, i32, i64, vp, i64, vp, i32, i32,
                                   ctypes.POINTER(CParams), vp, vp, vp]
    lib.ss_spec_verify.restype = i32
    lib.ss_spec_verify_scatter.argtypes = [vp, vp, i32, i64, vp, i64, vp, i32, i32,
                                           ctypes.POINTER(CParams), vp, vp,
                                           ctypes.POINTER(CSequences), vp]
    lib.ss_spec_verify_scatter.restype = i32
    lib.ss_tree_verify.argtypes = [vp, vp, i32, i64, vp, vp, i32, i32, ctypes.POINTER(CParams),
                                   vp, vp, vp, vp]
    lib.ss_tree_verify.restype = i32
    lib.ss_lmhead_sample.argtypes = [vp, vp, vp, i32, vp, vp, vp, u64, vp, vp, vp]
    lib.ss_lmhead_sample.restype = i32
    lib.ss_lmhead_sample_params.argtypes = [vp, vp, vp, i32, ctypes.POINTER(CParams), vp, vp, vp]
    lib.ss_lmhead_sample_params.restype = i32
    lib.ss_sample_noalloc.argtypes = [vp, i32, i64, i32, i32, ctypes.POINTER(CParams), vp, vp]
    lib.ss_sample_noalloc.restype = i32
    _lib = lib
    return lib


def _check(fn, st):
    if st != SS_OK:
        raise SamplerError(fn, st, load_library().ss_status_string(st).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_dev(t, name, dtypes, device):
    _require(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _require(t.is_cuda and t.device.index == device, f"{name} must live on cuda:{device}")
    _require(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _check_vec(t, name, n, dtype, device):
    """A per-row array: at least n entries, unit stride (the ABI takes a bare pointer)."""
    if t is None:
        return
    _check_dev(t, name, (dtype,), device)
    _require(t.dim() == 1 and t.shape[0] >= n and (t.shape[0] <= 1 or t.stride(0) == 1),
             f"{name} must be a 1-D array of >= {n} entries with unit stride")


def _check_rows(t, name, n, dtypes, device):
    """A [rows, cols] matrix with unit column stride: the ABI takes its row stride."""
    _check_dev(t, name, dtypes, device)
    _require(t.dim() == 2 and t.shape[0] >= n, f"{name} must be 2-D with >= {n} rows")
    _require(t.shape[1] <= 1 or t.stride(1) == 1, f"{name} must have unit stride along its last dim")


@dataclass
class SamplingParams:
    """Per-request parameters as device tensors (None disables a feature)."""
    temperature: torch.Tensor
    top_k: torch.Tensor | None = None
    top_p: torch.Tensor | None = None
    min_p: torch.Tensor | None = None
    repetition_penalty: torch.Tensor | None = None
    frequency_penalty: torch.Tensor | None = None
    presence_penalty: torch.Tensor | None = None
    history_ids: torch.Tensor | None = None   # [B, H] int32
    history_len: torch.Tensor | None = None   # [B] int32
    bias_ids: torch.Tensor | None = None      # [B, NB] int32
    bias_values: torch.Tensor | None = None   # [B, NB] float32
    bias_len: torch.Tensor | None = None      # [B] int32
    grammar_mask: torch.Tensor | None = None  # [B, W] (or [B, G+1, W]) int32 view of uint32 words
    request_ids: torch.Tensor | None = None
    positions: torch.Tensor | None = None
    seed: int = 0

    def validate(self, B, V, device, mask_rows=None):
        """Check every tensor against what the C ABI can express for B rows of a
        V-entry vocabulary; mask_rows = G + 1 for a per-position [B, G+1, W]
        mask (verification). Raises ValueError; returns the mask row stride."""
        _require(self.temperature is not None, "temperature is required")
        _check_vec(self.temperature, "temperature", B, torch.float32, device)
        _check_vec(self.top_k, "top_k", B, torch.int32, device)
        for name in ("top_p", "min_p", "repetition_penalty", "frequency_penalty",
                     "presence_penalty"):
            _check_vec(getattr(self, name), name, B, torch.float32, device)
        _check_vec(self.request_ids, "request_ids", B, torch.int32, device)
        _check_vec(self.positions, "positions", B, torch.int32, device)
        if self.history_len is not None or self.history_ids is not None:
            _require(self.history_len is not None and self.history_ids is not None,
                     "history_ids and history_len go together")
            _check_rows(self.history_ids, "history_ids", B, (torch.int32,), device)
            _check_vec(self.history_len, "history_len", B, torch.int32, device)
        if self.bias_len is not None or self.bias_ids is not None or self.bias_values is not None:
            _require(self.bias_len is not None and self.bias_ids is not None and
                     self.bias_values is not None, "bias_ids, bias_values and bias_len go together")
            _check_rows(self.bias_ids, "bias_ids", B, (torch.int32,), device)
            _check_rows(self.bias_values, "bias_values", B, (torch.float32,), device)
            _require(self.bias_values.shape[1] >= self.bias_ids.shape[1] and
                     self.bias_values.stride(0) == self.bias_ids.stride(0),
                     "bias_values must share bias_ids' row stride (one stride in the ABI)")
            _check_vec(self.bias_len, "bias_len", B, torch.int32, device)
        mask_stride = 0
        if self.grammar_mask is not None:
            m = self.grammar_mask
            _check_dev(m, "grammar_mask", (torch.int32,), device)
            words = (V + 31) // 32
            _require(m.shape[-1] >= words and (m.shape[-1] <= 1 or m.stride(-1) == 1),
                     f"grammar_mask needs >= {words} unit-stride words per row")
            if mask_rows is None:
                _require(m.dim() == 2 and m.shape[0] >= B, "grammar_mask must be [B, words]")
                mask_stride = m.stride(0)
            else:
                _require(m.dim() == 3 and m.shape[0] >= B and m.shape[1] == mask_rows and
                         (B <= 1 or m.stride(0) == mask_rows * m.stride(1)),
                         "a verification grammar_mask must be [B, G+1, words] with rows "
                         "evenly spaced")
                mask_stride = m.stride(1)
        return mask_stride

    def to_c(self, mask_stride=None):
        c = CParams()
        c.temperature = _ptr(self.temperature)
        c.top_k = _ptr(self.top_k)
        c.top_p = _ptr(self.top_p)
        c.min_p = _ptr(self.min_p)
        c.repetition_penalty = _ptr(self.repetition_penalty)
        c.frequency_penalty = _ptr(self.frequency_penalty)
        c.presence_penalty = _ptr(self.presence_penalty)
        c.history_ids = _ptr(self.history_ids)
        c.history_len = _ptr(self.history_len)
        c.history_stride = 0 if self.history_ids is None else int(self.history_ids.stride(0))
        c.bias_ids = _ptr(self.bias_ids)
        c.bias_values = _ptr(self.bias_values)
        c.bias_len = _ptr(self.bias_len)
        c.bias_stride = 0 if self.bias_ids is None else int(self.bias_ids.stride(0))
        c.grammar_mask = _ptr(self.grammar_mask)
        if mask_stride is None:
            mask_stride = 0 if self.grammar_mask is None else int(self.grammar_mask.stride(-2))
        c.mask_stride = int(mask_stride)
        c.request_ids = _ptr(self.request_ids)
        c.positions = _ptr(self.positions)
        c.seed = int(self.seed) & 0xFFFFFFFFFFFFFFFF
        return c


@dataclass
class Debug:
    """Optional debug outputs of sample() (device tensors, None = not wanted)."""
    processed_logits: torch.Tensor | None = None
    topk_ids: torch.Tensor | None = None
    kept_count: torch.Tensor | None = None
    probs: torch.Tensor | None = None
    path: torch.Tensor | None = None

    @staticmethod
    def full(B, V, device, topk_stride=1024):
        return Debug(torch.empty(B, V, dtype=torch.float32, device=device),
                     torch.empty(B, topk_stride, dtype=torch.int32, device=device),
                     torch.empty(B, dtype=torch.int32, device=device),
                     torch.empty(B, V, dtype=torch.float32, device=device),
                     torch.empty(B, dtype=torch.int32, device=device))

    def to_c(self):
        d = CDebug()
        d.processed_logits = _ptr(self.processed_logits)
        d.topk_ids = _ptr(self.topk_ids)
        d.topk_stride = 0 if self.topk_ids is None else int(self.topk_ids.shape[-1])
        d.kept_count = _ptr(self.kept_count)
        d.probs = _ptr(self.probs)
        d.path = _ptr(self.path)
        return d


class Sampler:
    """Owns one ss_sampler handle (and its device workspace)."""

    def __init__(self, max_batch, vocab_size, max_draft=0, hidden_size=0, device=0):
        self.lib = load_library()
        cfg = Config(max_batch, vocab_size, max_draft, hidden_size, device)
        h = ctypes.c_void_p()
        _check("ss_sampler_create", self.lib.ss_sampler_create(ctypes.byref(cfg), ctypes.byref(h)))
        self.handle = h
        self.vocab_size = vocab_size
        self.hidden_size = hidden_size
        self.max_draft = max_draft
        self.device = device

    def close(self):
        if getattr(self, "handle", None):
            self.lib.ss_sampler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    def workspace_bytes(self):
        return int(self.lib.ss_sampler_workspace_bytes(self.handle))

    def set_launch_events(self, events):
        """Bracket kernel k of the following calls with events[2k] / events[2k+1]
        (torch.cuda.Event objects; None clears). Each event must have been
        recorded once so that its HIP event exists."""
        if not events:
            _check("ss_sampler_set_launch_events",
                   self.lib.ss_sampler_set_launch_events(self.handle, None, 0))
            return
        arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
        _check("ss_sampler_set_launch_events",
               self.lib.ss_sampler_set_launch_events(self.handle, arr, len(events)))

    @staticmethod
    def _dtype(t):
        if t.dtype == torch.float32:
            return SS_F32
        if t.dtype == torch.bfloat16:
            return SS_BF16
        raise TypeError(f"unsupported logits dtype {t.dtype}")

    def sample(self, logits, params: SamplingParams, out=None, debug: Debug | None = None,
               stream=None):
        _check_rows(logits, "logits", 0, (torch.float32, torch.bfloat16), self.device)
        B, V = logits.shape
        _require(V == self.vocab_size, f"logits have {V} columns, the sampler {self.vocab_size}")
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=logits.device)
        _check_vec(out, "out", B, torch.int32, self.device)
        if debug is not None:
            for name, cols in (("processed_logits", V), ("probs", V)):
                t = getattr(debug, name)
                if t is not None:
                    _check_rows(t, f"debug.{name}", B, (torch.float32,), self.device)
                    _require(t.shape[1] == V and (B <= 1 or t.stride(0) == V),
                             f"debug.{name} must be a contiguous [B, V] array")
            if debug.topk_ids is not None:
                _check_rows(debug.topk_ids, "debug.topk_ids", B, (torch.int32,), self.device)
                _require(B <= 1 or debug.topk_ids.stride(0) == debug.topk_ids.shape[1],
                         "debug.topk_ids must be contiguous")
            _check_vec(debug.kept_count, "debug.kept_count", B, torch.int32, self.device)
            _check_vec(debug.path, "debug.path", B, torch.int32, self.device)
        cp = params.to_c(params.validate(B, V, self.device))
        cd = debug.to_c() if debug is not None else None
        st = self.lib.ss_sample(self.handle, _ptr(logits), self._dtype(logits),
                                int(logits.stride(0)), B, ctypes.byref(cp), _ptr(out),
                                ctypes.byref(cd) if cd is not None else None, _stream(stream))
        _check("ss_sample", st)
        return out

    def spec_verify(self, target_logits, draft_probs, draft_tokens, params: SamplingParams,
                    out_tokens=None, out_num_accepted=None, stream=None, seq_tokens=None,
                    seq_len=None):
        """draft_probs None: a greedy draft (q one-hot at each draft token).
        seq_tokens [B, capacity] / seq_len [B] int32: append the emitted tokens
        to these per-request sequences on the device and advance seq_len
        (params.positions may be seq_len itself)."""
        _check_dev(target_logits, "target_logits", (torch.float32, torch.bfloat16), self.device)
        _require(target_logits.dim() == 3, "target_logits must be [B, G+1, V]")
        B, G1, V = target_logits.shape
        G = G1 - 1
        _require(V == self.vocab_size, f"target_logits have {V} columns, the sampler {self.vocab_size}")
        # the ABI addresses row b * (G + 1) + j at one row stride
        _require(target_logits.stride(2) == 1 and
                 (B <= 1 or target_logits.stride(0) == G1 * target_logits.stride(1)),
                 "target_logits rows must be evenly spaced with unit stride along V")
        if draft_probs is not None:
            _check_dev(draft_probs, "draft_probs", (torch.float32,), self.device)
            _require(draft_probs.dim() == 3 and tuple(draft_probs.shape) == (B, G, V) and
                     draft_probs.stride(2) == 1 and
                     (B <= 1 or draft_probs.stride(0) == G * draft_probs.stride(1)),
                     "draft_probs must be [B, G, V] with evenly spaced rows and unit stride "
                     "along V")
        _check_dev(draft_tokens, "draft_tokens", (torch.int32,), self.device)
        _require(tuple(draft_tokens.shape) == (B, G) and draft_tokens.is_contiguous(),
                 "draft_tokens must be a contiguous [B, G] int32 array")
        dev = target_logits.device
        if out_tokens is None:
            out_tokens = torch.empty(B, G1, dtype=torch.int32, device=dev)
        if out_num_accepted is None:
            out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
        _check_dev(out_tokens, "out_tokens", (torch.int32,), self.device)
        _require(tuple(out_tokens.shape) == (B, G1) and out_tokens.is_contiguous(),
                 "out_tokens must be a contiguous [B, G+1] int32 array")
        _check_vec(out_num_accepted, "out_num_accepted", B, torch.int32, self.device)
        cp = params.to_c(params.validate(B, V, self.device, mask_rows=G1))
        seq = None
        if seq_tokens is not None or seq_len is not None:
            _require(seq_tokens is not None and seq_len is not None,
                     "seq_tokens and seq_len go together")
            _check_rows(seq_tokens, "seq_tokens", B, (torch.int32,), self.device)
            _check_vec(seq_len, "seq_len", B, torch.int32, self.device)
            seq = CSequences(_ptr(seq_tokens), int(seq_tokens.stride(0)) if B > 1 else
                             int(seq_tokens.shape[1]), int(seq_tokens.shape[1]), _ptr(seq_len))
        dstride = 0 if draft_probs is None else int(draft_probs.stride(1))
        st = self.lib.ss_spec_verify_scatter(
            self.handle, _ptr(target_logits), self._dtype(target_logits),
            int(target_logits.stride(1)), _ptr(draft_probs), dstride, _ptr(draft_tokens), B, G,
            ctypes.byref(cp), _ptr(out_tokens), _ptr(out_num_accepted),
            ctypes.byref(seq) if seq is not None else None, _stream(stream))
        _check("ss_spec_verify_scatter", st)
        return out_tokens, out_num_accepted

    def tree_verify(self, target_logits, parents, tokens, params: SamplingParams, out_tokens=None,
                    out_nodes=None, out_num_accepted=None, stream=None):
        """Verify one draft tree per request: target_logits [B, N, V] (row n after
        the root path to node n), parents / tokens [B, N] int32. Returns
        (tokens [B, N], nodes [B, N], num_accepted [B])."""
        _check_dev(target_logits, "target_logits", (torch.float32, torch.bfloat16), self.device)
        _require(target_logits.dim() == 3, "target_logits must be [B, N, V]")
        B, N, V = target_logits.shape
        _require(V == self.vocab_size, f"target_logits have {V} columns, the sampler {self.vocab_size}")
        _require(target_logits.stride(2) == 1 and
                 (B <= 1 or target_logits.stride(0) == N * target_logits.stride(1)),
                 "target_logits rows must be evenly spaced with unit stride along V")
        for name, t in (("parents", parents), ("tokens", tokens)):
            _check_dev(t, name, (torch.int32,), self.device)
            _require(tuple(t.shape) == (B, N) and t.is_contiguous(),
                     f"{name} must be a contiguous [B, N] int32 array")
        dev = target_logits.device
        if out_tokens is None:
            out_tokens = torch.empty(B, N, dtype=torch.int32, device=dev)
        if out_nodes is None:
            out_nodes = torch.empty(B, N, dtype=torch.int32, device=dev)
        if out_num_accepted is None:
            out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
        for name, t in (("out_tokens", out_tokens), ("out_nodes", out_nodes)):
            _check_dev(t, name, (torch.int32,), self.device)
            _require(tuple(t.shape) == (B, N) and t.is_contiguous(),
                     f"{name} must be a contiguous [B, N] int32 array")
        _check_vec(out_num_accepted, "out_num_accepted", B, torch.int32, self.device)
        cp = params.to_c(params.validate(B, V, self.device, mask_rows=N))
        st = self.lib.ss_tree_verify(self.handle, _ptr(target_logits), self._dtype(target_logits),
                                     int(target_logits.stride(1)), _ptr(parents), _ptr(tokens), B,
                                     N, ctypes.byref(cp), _ptr(out_tokens), _ptr(out_nodes),
                                     _ptr(out_num_accepted), _stream(stream))
        _check("ss_tree_verify", st)
        return out_tokens, out_nodes, out_num_accepted

    def lmhead_sample_params(self, hidden, weight, params: SamplingParams, out=None, path=None,
                             stream=None):
        """LM-head GEMM with the per-request pipeline (penalties, bias, mask,
        temperature, filters) before Gumbel-max sampling. path: optional [B]
        int32 that receives how each row was decided."""
        _check_dev(hidden, "hidden", (torch.bfloat16, torch.int16), self.device)
        _check_dev(weight, "weight", (torch.bfloat16, torch.int16), self.device)
        _require(hidden.dim() == 2 and hidden.is_contiguous(), "hidden must be a contiguous [B, K] array")
        B, K = hidden.shape
        _require(K == self.hidden_size, f"hidden has K = {K}, the sampler {self.hidden_size}")
        _require(tuple(weight.shape) == (self.vocab_size, K) and weight.is_contiguous(),
                 f"weight must be a contiguous [{self.vocab_size}, {K}] array")
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=hidden.device)
        _check_vec(out, "out", B, torch.int32, self.device)
        _check_vec(path, "path", B, torch.int32, self.device)
        cp = params.to_c(params.validate(B, self.vocab_size, self.device))
        st = self.lib.ss_lmhead_sample_params(self.handle, _ptr(hidden), _ptr(weight), B,
                                              ctypes.byref(cp), _ptr(out), _ptr(path),
                                              _stream(stream))
        _check("ss_lmhead_sample_params", st)
        return out

    def lmhead_sample(self, hidden, weight, temperature, request_ids=None, positions=None,
                      seed=0, out=None, debug_logits=None, stream=None):
        _check_dev(hidden, "hidden", (torch.bfloat16, torch.int16), self.device)
        _check_dev(weight, "weight", (torch.bfloat16, torch.int16), self.device)
        _require(hidden.dim() == 2 and hidden.is_contiguous(), "hidden must be a contiguous [B, K] array")
        B, K = hidden.shape
        _require(K == self.hidden_size, f"hidden has K = {K}, the sampler {self.hidden_size}")
        _require(tuple(weight.shape) == (self.vocab_size, K) and weight.is_contiguous(),
                 f"weight must be a contiguous [{self.vocab_size}, {K}] array")
        _check_vec(temperature, "temperature", B, torch.float32, self.device)
        _check_vec(request_ids, "request_ids", B, torch.int32, self.device)
        _check_vec(positions, "positions", B, torch.int32, self.device)
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=hidden.device)
        _check_vec(out, "out", B, torch.int32, self.device)
        if debug_logits is not None:
            _check_dev(debug_logits, "debug_logits", (torch.float32,), self.device)
            _require(tuple(debug_logits.shape) == (B, self.vocab_size) and debug_logits.is_contiguous(),
                     "debug_logits must be a contiguous [B, V] float32 array")
        st = self.lib.ss_lmhead_sample(self.handle, _ptr(hidden), _ptr(weight), B,
                                       _ptr(temperature), _ptr(request_ids), _ptr(positions),
                                       int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out),
                                       _ptr(debug_logits), _stream(stream))
        _check("ss_lmhead_sample", st)
        return out


def sample_noalloc(logits, params: SamplingParams, out=None, stream=None):
    """ss_sample without a handle: the library's static per-GPU scratch serves
    as workspace, so the call allocates nothing when `out` is given (B rows of
    at most 64, B * V at most 2^23). Calls that overlap on one GPU race."""
    _require(isinstance(logits, torch.Tensor) and logits.is_cuda, "logits must be a device tensor")
    dev = logits.device.index
    _check_rows(logits, "logits", 0, (torch.float32, torch.bfloat16), dev)
    B, V = logits.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    _check_vec(out, "out", B, torch.int32, dev)
    cp = params.to_c(params.validate(B, V, dev))
    with torch.cuda.device(dev):
        st = load_library().ss_sample_noalloc(_ptr(logits), Sampler._dtype(logits),
                                              int(logits.stride(0)), B, V, ctypes.byref(cp),
                                              _ptr(out), _stream(stream))
    _check("ss_sample_noalloc", st)
    return out

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
            "ss_spec_verify", "ss_lmhead_sample")


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
    lib.ss_lmhead_sample.argtypes = [vp, vp, vp, i32, vp, vp, vp, u64, vp, vp, vp]
    lib.ss_lmhead_sample.restype = i32
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

    def to_c(self):
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
        c.mask_stride = 0 if self.grammar_mask is None else int(self.grammar_mask.shape[-1])
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
        B = logits.shape[0]
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=logits.device)
        cp = params.to_c()
        cd = debug.to_c() if debug is not None else None
        st = self.lib.ss_sample(self.handle, _ptr(logits), self._dtype(logits),
                                int(logits.stride(0)), B, ctypes.byref(cp), _ptr(out),
                                ctypes.byref(cd) if cd is not None else None, _stream(stream))
        _check("ss_sample", st)
        return out

    def spec_verify(self, target_logits, draft_probs, draft_tokens, params: SamplingParams,
                    out_tokens=None, out_num_accepted=None, stream=None):
        B, G1, V = target_logits.shape
        G = G1 - 1
        dev = target_logits.device
        if out_tokens is None:
            out_tokens = torch.empty(B, G1, dtype=torch.int32, device=dev)
        if out_num_accepted is None:
            out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
        cp = params.to_c()
        st = self.lib.ss_spec_verify(self.handle, _ptr(target_logits), self._dtype(target_logits),
                                     int(target_logits.stride(1)), _ptr(draft_probs),
                                     int(draft_probs.stride(1)), _ptr(draft_tokens), B, G,
                                     ctypes.byref(cp), _ptr(out_tokens), _ptr(out_num_accepted),
                                     _stream(stream))
        _check("ss_spec_verify", st)
        return out_tokens, out_num_accepted

    def lmhead_sample(self, hidden, weight, temperature, request_ids=None, positions=None,
                      seed=0, out=None, debug_logits=None, stream=None):
        B = hidden.shape[0]
        if out is None:
            out = torch.empty(B, dtype=torch.int32, device=hidden.device)
        st = self.lib.ss_lmhead_sample(self.handle, _ptr(hidden), _ptr(weight), B,
                                       _ptr(temperature), _ptr(request_ids), _ptr(positions),
                                       int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out),
                                       _ptr(debug_logits), _stream(stream))
        _check("ss_lmhead_sample", st)
        return out

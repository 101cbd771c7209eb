"""MI355X (gfx950) WFST Viterbi beam-search decoder: thin Python binding.

Every step of the decode runs in the HIP library ``libwfst_mi355x.so`` (C ABI in
``include/wfst.h``); this module only marshals arguments through ctypes. PyTorch
is used for device memory and the current stream, nothing else. There is no CPU
fallback: importing works without a GPU, but every call needs the built library
and a device, and fails loudly otherwise.
"""

from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass
from types import SimpleNamespace

import numpy as np

__all__ = ["Graph", "Decoder", "DecodeResult", "WfstError", "library_path", "load_library", "decode_noalloc",
           "EXPORTED_SYMBOLS", "LP_F32", "LP_F16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwfst_mi355x.so")

LP_F32, LP_F16 = 0, 1
EXPORTED_SYMBOLS = ("wfst_last_error", "wfst_graph_upload", "wfst_graph_release",
                    "wfst_decoder_create", "wfst_decode", "wfst_decoder_destroy",
                    "wfst_decoder_stats", "wfst_decoder_mem_stats", "wfst_decoder_step_stats", "wfst_decoder_profile",
                    "wfst_decoder_kernel_times", "wfst_create_stream", "wfst_advance_chunk",
                    "wfst_finalize_stream", "wfst_finalize_streams", "wfst_create_streams", "wfst_release_stream", "wfst_lattice_records",
                    "wfst_blank_skip", "wfst_decode_noalloc")
KERNELS = ("clear", "init", "lpmax", "max", "expand", "finalize", "eps_expand", "eps_resolve",
           "eps_apply", "backtrack", "stream_begin", "stream_end", "reclass", "lat_resolve", "lat_init",
           "lat_back", "gc_begin", "gc_mark", "gc_scan", "gc_compact", "gc_commit", "gc_roots", "gc_clear",
           "gc_end", "lat_eps_back", "lat_prune", "lat_eps_round", "eps_apply_expand",
           "lat_prep", "lat_fprep", "lat_sweep", "lat_emit")
LATTICE_FIELDS = ("frame", "src", "dst", "ilabel", "arc", "score_bits", "lane", "flags")
STEP_FIELDS = ("n", "beam", "max", "arcs", "admitted", "distinct", "eps_arcs", "eps_admitted",
               "eps_distinct", "eps_new", "eps_replaced", "eps_passes", "phase", "listed", "_14", "_15")
STAT_FIELDS = ("arcs", "admitted", "distinct", "tokens", "eps_arcs", "eps_admitted",
               "eps_distinct", "eps_changed", "log_entries", "steps", "max_frontier", "device_bytes",
               "lane_frames", "listed", "log_reserved_bytes", "log_committed_bytes", "regrows")


class WfstError(RuntimeError):
    """A call into the decoder library failed (the message is the library's)."""

    def __init__(self, code, msg):
        super().__init__(f"wfst error {code}: {msg}")
        self.code = code


class _GraphDesc(ctypes.Structure):
    _fields_ = [("num_states", ctypes.c_int32), ("num_arcs", ctypes.c_int32),
                ("start_state", ctypes.c_int32), ("vocab_size", ctypes.c_int32),
                ("epsilon_id", ctypes.c_int32),
                ("row_splits", ctypes.c_void_p), ("dest", ctypes.c_void_p),
                ("ilabel", ctypes.c_void_p), ("olabel", ctypes.c_void_p), ("weight", ctypes.c_void_p)]


class _Config(ctypes.Structure):
    _fields_ = [("beam", ctypes.c_float), ("min_active", ctypes.c_int32),
                ("max_active", ctypes.c_int32), ("allow_partial", ctypes.c_int32),
                ("max_lanes", ctypes.c_int32), ("max_frames", ctypes.c_int32),
                ("lp_dtype", ctypes.c_int32), ("eps_iterations", ctypes.c_int32),
                ("use_graphs", ctypes.c_int32), ("frontier_cap", ctypes.c_int32),
                ("claims_cap", ctypes.c_int32), ("grid_blocks", ctypes.c_int32),
                ("arena_entries", ctypes.c_int64), ("slot_cap", ctypes.c_int64),
                ("plain_keys", ctypes.c_int32), ("path_cap", ctypes.c_int32),
                ("lattice", ctypes.c_int32), ("output_beam", ctypes.c_float),
                ("lattice_cap", ctypes.c_int64), ("gc_interval", ctypes.c_int32),
                ("arena_commit", ctypes.c_int64), ("epoch_period", ctypes.c_int32),
                ("lat_prune_interval", ctypes.c_int32), ("recomb_slots", ctypes.c_int64)]


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise WfstError(-4, f"{_LIB_PATH} is missing: build it with "
                                "`python -m wfst_beam_search_amd.build` (there is no CPU fallback)")
        # PyTorch bundles its own HIP runtime under the same soname
        # (libamdhip64.so.7). Loading torch first makes the library bind to that
        # copy, so the process holds one HIP/HSA runtime; loading the system copy
        # first would leave torch unable to open the GPU.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
        lib.wfst_last_error.restype = ctypes.c_char_p
        lib.wfst_graph_upload.argtypes = [ctypes.POINTER(_GraphDesc), ctypes.c_int, ctypes.POINTER(vp)]
        lib.wfst_graph_release.argtypes = [vp]
        lib.wfst_decoder_create.argtypes = [vp, ctypes.POINTER(_Config), ctypes.POINTER(vp)]
        lib.wfst_decoder_destroy.argtypes = [vp]
        lib.wfst_decode.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp]
        lib.wfst_decoder_stats.argtypes = [vp, vp, i32]
        lib.wfst_decoder_mem_stats.argtypes = [vp, vp]
        lib.wfst_decoder_step_stats.argtypes = [vp, i32, vp, i32]
        lib.wfst_decoder_profile.argtypes = [vp, i32]
        lib.wfst_decoder_kernel_times.argtypes = [vp, vp, i32]
        lib.wfst_create_stream.argtypes = [vp, vp, vp]
        lib.wfst_advance_chunk.argtypes = [vp, vp, i32, vp, i32, i32, vp, vp, i32, vp, i32, vp, vp, i32,
                                           vp, vp, vp]
        lib.wfst_finalize_stream.argtypes = [vp, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp]
        lib.wfst_finalize_streams.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp]
        lib.wfst_create_streams.argtypes = [vp, i32, vp, vp, vp]
        lib.wfst_release_stream.argtypes = [vp, i32]
        lib.wfst_lattice_records.argtypes = [vp, i32, vp, ctypes.c_int64, vp]
        lib.wfst_blank_skip.argtypes = [vp, vp, i32, i32, i32, vp, i32, ctypes.c_float, vp, vp, vp]
        lib.wfst_decode_noalloc.argtypes = [vp, ctypes.POINTER(_Config), vp, i32, i32, i32, vp, vp, vp, i32, vp,
                                            vp, i32, vp, vp, vp]
        for name in EXPORTED_SYMBOLS:
            if name != "wfst_last_error":
                getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _check(rc):
    if rc < 0:
        msg = _lib.wfst_last_error().decode(errors="replace")
        raise WfstError(rc, msg)
    return rc


def _ptr(a: np.ndarray):
    return a.ctypes.data if a.size else None


class Graph:
    """A decoding graph uploaded to one device.

    ``g`` has the attributes num_states (including the super-final state, the
    last one), start, vocab, epsilon_id and the arrays row_splits, dest, ilabel,
    olabel, weight (see include/wfst.h for the rules).
    """

    def __init__(self, g, device: int = 0):
        lib = load_library()
        self._arrays = [np.ascontiguousarray(g.row_splits, dtype=np.int32),
                        np.ascontiguousarray(g.dest, dtype=np.int32),
                        np.ascontiguousarray(g.ilabel, dtype=np.int32),
                        np.ascontiguousarray(g.olabel, dtype=np.int32),
                        np.ascontiguousarray(g.weight, dtype=np.float32)]
        rs, dest, il, ol, w = self._arrays
        desc = _GraphDesc(int(g.num_states), int(dest.shape[0]), int(g.start), int(g.vocab),
                          int(g.epsilon_id), _ptr(rs), _ptr(dest), _ptr(il), _ptr(ol), _ptr(w))
        h = ctypes.c_void_p()
        _check(lib.wfst_graph_upload(ctypes.byref(desc), int(device), ctypes.byref(h)))
        self._arrays = None
        self.handle = h
        self.device = device
        self.vocab = int(g.vocab)
        self.epsilon_id = int(g.epsilon_id)

    @classmethod
    def from_arrays(cls, row_splits, dest, ilabel, olabel, weight, start: int, vocab: int,
                    epsilon_id: int = -1, device: int = 0) -> "Graph":
        """Uploads a CSR graph given as plain arrays: row_splits [N + 1] (N states,
        the last one the super-final state), per arc dest, ilabel (-1 final,
        epsilon_id, else [0, vocab)), olabel (0 = no word) and weight (float32
        log-score <= 0); each state's arcs ordered epsilon, emitting, final."""
        g = SimpleNamespace(num_states=len(row_splits) - 1, start=int(start), vocab=int(vocab),
                            epsilon_id=int(epsilon_id), row_splits=row_splits, dest=dest, ilabel=ilabel,
                            olabel=olabel, weight=weight)
        return cls(g, device=device)

    def release(self):
        if self.handle:
            _lib.wfst_graph_release(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


@dataclass
class DecodeResult:
    words: list          # per lane: int32 array of word ids
    arcs: list           # per lane: int32 array of arc ids (forward order)
    scores: np.ndarray   # float32 [B]
    meta: np.ndarray     # int32 [B, 3]: ok, reached_final, overflow bits
    word_lens: np.ndarray
    arc_lens: np.ndarray


def _config(beam, max_active, min_active=0, allow_partial=False, max_lanes=8, max_frames=1024, lp_dtype="f32",
            eps_iterations=0, use_graphs=True, frontier_cap=0, claims_cap=0, arena_entries=0, grid_blocks=0,
            slot_cap=0, plain_keys=0, path_cap=0, lattice=False, output_beam=0.0, lattice_cap=0, gc_interval=0,
            arena_commit=0, epoch_period=0, lat_prune_interval=0, recomb_slots=0) -> _Config:
    return _Config(float(beam), int(min_active), int(max_active), int(bool(allow_partial)),
                   int(max_lanes), int(max_frames), LP_F16 if lp_dtype == "f16" else LP_F32,
                   int(eps_iterations), int(bool(use_graphs)), int(frontier_cap),
                   int(claims_cap), int(grid_blocks), int(arena_entries), int(slot_cap),
                   int(plain_keys), int(path_cap), int(bool(lattice)), float(output_beam),
                   int(lattice_cap), int(gc_interval), int(arena_commit), int(epoch_period),
                   int(lat_prune_interval), int(recomb_slots))


def decode_noalloc(graph: "Graph", log_prob, lengths, beam: float, max_active: int, stream=None,
                   words_cap: int | None = None, arcs_cap: int | None = None, **config) -> "DecodeResult":
    """One decode through ``wfst_decode_noalloc``: no decoder object, the whole
    workspace in the library's static device scratch (no device allocation).
    ``config`` takes Decoder's keyword arguments (capacities must fit the
    scratch); ``log_prob`` and ``lengths`` as Decoder.decode."""
    import torch
    lib = load_library()
    cfg = _config(beam, max_active, **config)
    if not isinstance(log_prob, torch.Tensor) or not log_prob.is_cuda or not log_prob.is_contiguous():
        raise TypeError("log_prob must be a packed torch tensor on the GPU")
    if log_prob.device.index != graph.device:
        raise ValueError(f"log_prob must be on cuda:{graph.device}, the graph's device")
    want = torch.float16 if config.get("lp_dtype", "f32") == "f16" else torch.float32
    if log_prob.dtype != want or log_prob.dim() != 3:
        raise TypeError(f"log_prob must be a [B, T, V] {want} tensor")
    B, T, V = (int(x) for x in log_prob.shape)
    lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32).reshape(-1))
    if lens.shape[0] != B:
        raise ValueError("lengths must have B entries")
    stream = Decoder._stream(stream, log_prob.device)
    P = int(config.get("eps_iterations", 0))
    wcap = int(words_cap) if words_cap is not None else T + 2
    acap = int(arcs_cap) if arcs_cap is not None else (T + 2) * (1 + max(0, P))
    out = Decoder._outputs(B, wcap, acap)
    out_words, wl, out_arcs, al, sc, meta = out
    _check(lib.wfst_decode_noalloc(graph.handle, ctypes.byref(cfg), ctypes.c_void_p(log_prob.data_ptr()), B, T, V,
                                   _ptr(lens), ctypes.c_void_p(int(stream)), _ptr(out_words), wcap, _ptr(wl),
                                   _ptr(out_arcs), acap, _ptr(al), _ptr(sc), _ptr(meta)))
    return Decoder._result(out, wcap, acap)


class Decoder:
    """A decoder instance (workspace on the graph's device)."""

    def __init__(self, graph: Graph, beam: float, max_active: int, min_active: int = 0,
                 allow_partial: bool = False, max_lanes: int = 8, max_frames: int = 1024,
                 lp_dtype: str = "f32", eps_iterations: int = 0, use_graphs: bool = True,
                 frontier_cap: int = 0, claims_cap: int = 0, arena_entries: int = 0,
                 grid_blocks: int = 0, slot_cap: int = 0, plain_keys: int = 0, path_cap: int = 0,
                 lattice: bool = False, output_beam: float = 0.0, lattice_cap: int = 0, gc_interval: int = 0,
                 arena_commit: int = 0, epoch_period: int = 0, lat_prune_interval: int = 0,
                 recomb_slots: int = 0):
        lib = load_library()
        cfg = _config(beam, max_active, min_active, allow_partial, max_lanes, max_frames, lp_dtype,
                      eps_iterations, use_graphs, frontier_cap, claims_cap, arena_entries, grid_blocks,
                      slot_cap, plain_keys, path_cap, lattice, output_beam, lattice_cap, gc_interval,
                      arena_commit, epoch_period, lat_prune_interval, recomb_slots)
        h = ctypes.c_void_p()
        _check(lib.wfst_decoder_create(graph.handle, ctypes.byref(cfg), ctypes.byref(h)))
        self.handle = h
        self.graph = graph
        self.max_lanes = int(max_lanes)
        self.max_frames = int(max_frames)
        self.lp_dtype = lp_dtype
        self.eps_iterations = int(eps_iterations)

    def _check_lp(self, log_prob):
        import torch
        if not isinstance(log_prob, torch.Tensor) or not log_prob.is_cuda:
            raise TypeError("log_prob must be a torch tensor on the GPU")
        if log_prob.device.index != self.graph.device:
            raise ValueError(f"log_prob must be on cuda:{self.graph.device}, the decoder's device")
        if not log_prob.is_contiguous():
            raise ValueError("log_prob must be packed (contiguous)")
        want = torch.float16 if self.lp_dtype == "f16" else torch.float32
        if log_prob.dtype != want:
            raise TypeError(f"log_prob must be {want}")
        if log_prob.dim() != 3:
            raise ValueError("log_prob must be [B, T, V]")

    @staticmethod
    def _stream(stream, device):
        import torch
        return torch.cuda.current_stream(device).cuda_stream if stream is None else stream

    @staticmethod
    def _outputs(n, wcap, acap):
        return (np.zeros((n, max(wcap, 1)), dtype=np.int32), np.zeros(n, dtype=np.int32),
                np.zeros((n, max(acap, 1)), dtype=np.int32), np.zeros(n, dtype=np.int32),
                np.zeros(n, dtype=np.float32), np.zeros((n, 3), dtype=np.int32))

    @staticmethod
    def _result(out, wcap, acap):
        out_words, wl, out_arcs, al, sc, meta = out
        n = sc.shape[0]
        words = [out_words[b, :min(int(wl[b]), wcap)].copy() for b in range(n)]
        arcs = [out_arcs[b, :min(int(al[b]), acap)].copy() for b in range(n)]
        return DecodeResult(words, arcs, sc, meta, wl, al)

    def decode(self, log_prob, lengths, stream=None, words_cap: int | None = None,
               arcs_cap: int | None = None) -> DecodeResult:
        """Decode ``log_prob`` ([B, T, V] torch tensor on the decoder's device, packed,
        in the decoder's dtype) with per-lane ``lengths``; returns host results."""
        self._check_lp(log_prob)
        B, T, V = (int(x) for x in log_prob.shape)
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32).reshape(-1))
        if lens.shape[0] != B:
            raise ValueError("lengths must have B entries")
        stream = self._stream(stream, log_prob.device)
        wcap = int(words_cap) if words_cap is not None else T + 2
        acap = int(arcs_cap) if arcs_cap is not None else (T + 2) * (1 + max(0, self.eps_iterations))
        out = self._outputs(B, wcap, acap)
        out_words, wl, out_arcs, al, sc, meta = out
        _check(_lib.wfst_decode(self.handle, ctypes.c_void_p(log_prob.data_ptr()), B, T, V,
                                _ptr(lens), ctypes.c_void_p(int(stream)),
                                _ptr(out_words), wcap, _ptr(wl), _ptr(out_arcs), acap, _ptr(al),
                                _ptr(sc), _ptr(meta)))
        return self._result(out, wcap, acap)

    # ---- streams (page section 8): one lane per stream, search state kept on the device

    def create_stream(self, stream=None) -> int:
        """Open a stream; returns its channel, or -1 when every lane holds one."""
        import torch
        ch = ctypes.c_int32(-1)
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        _check(_lib.wfst_create_stream(self.handle, ctypes.c_void_p(int(s)), ctypes.byref(ch)))
        return int(ch.value)

    def create_streams(self, n: int, stream=None) -> list:
        """Open up to n streams in one call; returns their channels (fewer when
        fewer lanes are free)."""
        import torch
        out = np.zeros(max(int(n), 1), dtype=np.int32)
        got = ctypes.c_int32(0)
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        _check(_lib.wfst_create_streams(self.handle, int(n), ctypes.c_void_p(int(s)), _ptr(out), ctypes.byref(got)))
        return [int(x) for x in out[:got.value]]

    def advance_chunk(self, channels, log_prob, lengths, want_partial: bool = False, stream=None,
                      words_cap: int = 4096, arcs_cap: int = 4096):
        """Advance each channel by its chunk (row j of ``log_prob`` [C, T, V] for
        channels[j], ``lengths[j]`` frames). Returns the partial hypotheses as a
        DecodeResult (row j for channels[j]) when ``want_partial``, else None."""
        self._check_lp(log_prob)
        C, T, V = (int(x) for x in log_prob.shape)
        chans = np.ascontiguousarray(np.asarray(channels, dtype=np.int32).reshape(-1))
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32).reshape(-1))
        if chans.shape[0] != C or lens.shape[0] != C:
            raise ValueError("channels and lengths must have C entries")
        stream = self._stream(stream, log_prob.device)
        out = self._outputs(C, words_cap, arcs_cap)
        out_words, wl, out_arcs, al, sc, meta = out
        _check(_lib.wfst_advance_chunk(self.handle, _ptr(chans), C, ctypes.c_void_p(log_prob.data_ptr()),
                                       T, V, _ptr(lens), ctypes.c_void_p(int(stream)), int(bool(want_partial)),
                                       _ptr(out_words), words_cap, _ptr(wl), _ptr(out_arcs), arcs_cap,
                                       _ptr(al), _ptr(sc), _ptr(meta)))
        return self._result(out, words_cap, arcs_cap) if want_partial else None

    def finalize_stream(self, channel: int, stream=None, words_cap: int = 1 << 16,
                        arcs_cap: int = 1 << 16) -> DecodeResult:
        """End a stream: final step and best path (a one-row DecodeResult)."""
        import torch
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        out = self._outputs(1, words_cap, arcs_cap)
        out_words, wl, out_arcs, al, sc, meta = out
        _check(_lib.wfst_finalize_stream(self.handle, int(channel), ctypes.c_void_p(int(s)), _ptr(out_words),
                                         words_cap, _ptr(wl), _ptr(out_arcs), arcs_cap, _ptr(al), _ptr(sc),
                                         _ptr(meta)))
        return self._result(out, words_cap, arcs_cap)

    def finalize_streams(self, channels, stream=None, words_cap: int = 1 << 16,
                         arcs_cap: int = 1 << 16) -> DecodeResult:
        """End several streams in one call (row j of the result for channels[j])."""
        import torch
        chans = np.ascontiguousarray(np.asarray(channels, dtype=np.int32).reshape(-1))
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        out = self._outputs(chans.shape[0], words_cap, arcs_cap)
        out_words, wl, out_arcs, al, sc, meta = out
        _check(_lib.wfst_finalize_streams(self.handle, _ptr(chans), chans.shape[0], ctypes.c_void_p(int(s)),
                                          _ptr(out_words), words_cap, _ptr(wl), _ptr(out_arcs), arcs_cap, _ptr(al),
                                          _ptr(sc), _ptr(meta)))
        return self._result(out, words_cap, arcs_cap)

    def release_stream(self, channel: int):
        _check(_lib.wfst_release_stream(self.handle, int(channel)))

    def blank_skip(self, log_prob, lengths, blank_id: int = 0, threshold: float = 0.98, stream=None):
        """Blank-skip pre-slicing on the device: returns (sliced log_prob, same
        shape, kept rows first; kept lengths int32 [B])."""
        import torch
        self._check_lp(log_prob)
        B, T, V = (int(x) for x in log_prob.shape)
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32).reshape(-1))
        if lens.shape[0] != B:
            raise ValueError("lengths must have B entries")
        out = torch.empty_like(log_prob)
        outl = np.zeros(B, dtype=np.int32)
        stream = self._stream(stream, log_prob.device)
        _check(_lib.wfst_blank_skip(self.handle, ctypes.c_void_p(log_prob.data_ptr()), B, T, V, _ptr(lens),
                                    int(blank_id), float(threshold), ctypes.c_void_p(out.data_ptr()), _ptr(outl),
                                    ctypes.c_void_p(int(stream))))
        return out, outl

    def lattice(self, lane: int) -> np.ndarray:
        """Kept lattice arcs of ``lane`` in the last decode (lattice mode): int32
        [n, 8], fields ``LATTICE_FIELDS``, sorted by (frame, src, arc)."""
        n = ctypes.c_int64(0)
        _check(_lib.wfst_lattice_records(self.handle, int(lane), None, 0, ctypes.byref(n)))
        out = np.zeros((max(int(n.value), 1), 8), dtype=np.int32)
        _check(_lib.wfst_lattice_records(self.handle, int(lane), _ptr(out), out.shape[0], ctypes.byref(n)))
        out = out[:int(n.value)]
        return out[np.lexsort((out[:, 4], out[:, 1], out[:, 0]))] if out.shape[0] else out

    def stats(self) -> dict:
        out = np.zeros(len(STAT_FIELDS), dtype=np.int64)
        _check(_lib.wfst_decoder_stats(self.handle, _ptr(out), len(STAT_FIELDS)))
        return dict(zip(STAT_FIELDS, (int(x) for x in out)))

    def mem_stats(self) -> dict:
        """Device bytes: reserved, committed, fixed workspace, winners-log high water."""
        out = np.zeros(4, dtype=np.int64)
        _check(_lib.wfst_decoder_mem_stats(self.handle, _ptr(out)))
        return dict(zip(("reserved", "committed", "fixed", "log_high_water"), (int(x) for x in out)))

    def step_stats(self, lane: int) -> np.ndarray:
        """Per-step records of ``lane`` in the last decode: int64 [n, 16]
        (record 0: start closure; record t + 1: step t)."""
        cap = self.max_frames + 2
        out = np.zeros((cap, len(STEP_FIELDS)), dtype=np.int64)
        n = _check(_lib.wfst_decoder_step_stats(self.handle, int(lane), _ptr(out), cap))
        return out[:n]

    def profile(self, enable: bool = True):
        """Record hipEvents between this decoder's kernel launches (see kernel_times)."""
        _check(_lib.wfst_decoder_profile(self.handle, int(bool(enable))))

    def kernel_times(self) -> dict:
        """{kernel: (total ms, launches)} of the last decode (run with profile on)."""
        out = np.zeros(2 * len(KERNELS), dtype=np.float64)
        _check(_lib.wfst_decoder_kernel_times(self.handle, _ptr(out), out.shape[0]))
        return {k: (float(out[2 * i]), int(out[2 * i + 1])) for i, k in enumerate(KERNELS)}

    def close(self):
        if self.handle:
            _lib.wfst_decoder_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

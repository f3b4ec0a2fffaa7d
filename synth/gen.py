"""ctypes front-end of the synthetic generators (synth_host.c, synth_dev.hip) and
the numpy Zipf-logit generator.  See synth_recipe.md for the exact recipe."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from .configs import Config

_HERE = os.path.dirname(os.path.abspath(__file__))


def host_lib_path() -> str:
    return os.path.join(_HERE, "libsynth_host.so")


def dev_lib_path() -> str:
    return os.path.join(_HERE, "libsynth_dev.so")


def build_libs(verbose: bool = False) -> None:
    """Compile the host (gcc) and device (hipcc, gfx950) generators in place."""
    host = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
            os.path.join(_HERE, "synth_host.c"), "-o", host_lib_path(), "-lm"]
    dev = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "synth_dev.hip"), "-o", dev_lib_path()]
    for cmd in (host, dev):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("synth build failed: %s\n%s" % (" ".join(cmd), r.stderr))
        if verbose:
            print(" ".join(cmd))


def _u64p(a):
    return (ctypes.c_uint64 * 3)(*[int(v) for v in a])


class HostGen:
    """Host generator (synth_host.c)."""

    def __init__(self, path: Optional[str] = None):
        path = path or host_lib_path()
        if not os.path.exists(path):
            raise FileNotFoundError("%s is not built (run __graft_entry__.build())" % path)
        lib = ctypes.CDLL(path)
        lib.synth_expert_blob.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                          ctypes.c_void_p]
        lib.synth_expert_blob_mx.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_x.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p]
        lib.synth_w_router.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
        lib.synth_w_shared_gate.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p]
        lib.synth_global_scale.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.synth_global_scale.restype = ctypes.c_float
        self.lib = lib

    def expert_blob(self, cfg: Config, layer: int, expert: int, layout) -> np.ndarray:
        """uint8 [slot_stride]: the blob of (layer, expert); layout gives the offsets."""
        out = np.zeros(int(layout.slot_stride), dtype=np.uint8)
        self.lib.synth_expert_blob(cfg.seed, cfg.cfg_id, layer, expert, cfg.H, cfg.I,
                                   _u64p(layout.off_codes), _u64p(layout.off_scales), int(layout.off_globals),
                                   out.ctypes.data)
        return out

    def expert_blob_mx(self, cfg: Config, layer: int, expert: int, layout) -> np.ndarray:
        """uint8 [slot_stride]: the MX blob of (layer, expert); layout gives the offsets."""
        out = np.zeros(int(layout.slot_stride), dtype=np.uint8)
        self.lib.synth_expert_blob_mx(cfg.seed, cfg.cfg_id, layer, expert, cfg.H, cfg.I,
                                      _u64p(layout.off_codes), _u64p(layout.off_scales), out.ctypes.data)
        return out

    def x(self, cfg: Config, layer: int, step: int = 0, T: Optional[int] = None) -> np.ndarray:
        T = cfg.T if T is None else T
        out = np.empty((T, cfg.H), dtype=np.uint16)
        self.lib.synth_x(cfg.seed, cfg.cfg_id, layer, step, T, cfg.H, out.ctypes.data)
        return out

    def w_router(self, cfg: Config, layer: int) -> np.ndarray:
        out = np.empty((cfg.H, cfg.E), dtype=np.float32)
        self.lib.synth_w_router(cfg.seed, cfg.cfg_id, layer, cfg.H, cfg.E, out.ctypes.data)
        return out

    def w_shared_gate(self, cfg: Config, layer: int) -> np.ndarray:
        out = np.empty(cfg.H, dtype=np.float32)
        self.lib.synth_w_shared_gate(cfg.seed, cfg.cfg_id, layer, cfg.H, out.ctypes.data)
        return out


class DevGen:
    """Device generator (synth_dev.hip).  Pointers are device addresses (ints),
    streams are hipStream_t handles (ints)."""

    def __init__(self, path: Optional[str] = None):
        path = path or dev_lib_path()
        if not os.path.exists(path):
            raise FileNotFoundError("%s is not built (run __graft_entry__.build())" % path)
        lib = ctypes.CDLL(path)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
        lib.synth_dev_pool.argtypes = [u64, i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, u64, u64, vp, vp]
        lib.synth_dev_pool_mx.argtypes = [u64, i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, u64, vp, vp]
        lib.synth_dev_x.argtypes = [u64, i32, i32, i32, i32, i32, vp, vp]
        lib.synth_dev_w_router.argtypes = [u64, i32, i32, i32, i32, vp, vp]
        lib.synth_dev_w_shared_gate.argtypes = [u64, i32, i32, i32, vp, vp]
        self.lib = lib

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise RuntimeError("synth device generator failed with hipError %d" % rc)

    def pool(self, cfg: Config, layer0: int, n_layers: int, slot_table_ptr: int, n_slots: int, layout,
             pool_ptr: int, stream: int = 0) -> None:
        self._check(self.lib.synth_dev_pool(cfg.seed, cfg.cfg_id, layer0, n_layers, cfg.E1, cfg.H, cfg.I,
                                            slot_table_ptr, n_slots, _u64p(layout.off_codes),
                                            _u64p(layout.off_scales), int(layout.off_globals),
                                            int(layout.slot_stride), pool_ptr, stream))

    def pool_mx(self, cfg: Config, layer0: int, n_layers: int, slot_table_ptr: int, n_slots: int, layout,
                pool_ptr: int, stream: int = 0) -> None:
        self._check(self.lib.synth_dev_pool_mx(cfg.seed, cfg.cfg_id, layer0, n_layers, cfg.E1, cfg.H, cfg.I,
                                               slot_table_ptr, n_slots, _u64p(layout.off_codes),
                                               _u64p(layout.off_scales), int(layout.slot_stride), pool_ptr, stream))

    def x(self, cfg: Config, layer: int, step: int, out_ptr: int, stream: int = 0, T: Optional[int] = None) -> None:
        self._check(self.lib.synth_dev_x(cfg.seed, cfg.cfg_id, layer, step, cfg.T if T is None else T, cfg.H,
                                         out_ptr, stream))

    def w_router(self, cfg: Config, layer: int, out_ptr: int, stream: int = 0) -> None:
        self._check(self.lib.synth_dev_w_router(cfg.seed, cfg.cfg_id, layer, cfg.H, cfg.E, out_ptr, stream))

    def w_shared_gate(self, cfg: Config, layer: int, out_ptr: int, stream: int = 0) -> None:
        self._check(self.lib.synth_dev_w_shared_gate(cfg.seed, cfg.cfg_id, layer, cfg.H, out_ptr, stream))


def zipf_popularity(cfg: Config, layer: int, epoch: int) -> np.ndarray:
    """p_e proportional to (pi(e) + 1)^-s for a per-(layer, epoch) permutation pi."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, cfg.cfg_id, layer, epoch])))
    pi = g.permutation(cfg.E)
    p = (pi + 1.0) ** (-cfg.zipf_s)
    return p / p.sum()


def zipf_logits(cfg: Config, layer: int, step: int = 0, T: Optional[int] = None) -> np.ndarray:
    """fp32 [T, E] logits ln p_e + Gumbel(0,1): top-k is a draw without
    replacement in proportion to the Zipf popularity."""
    T = cfg.T if T is None else T
    p = zipf_popularity(cfg, layer, cfg.epoch(step))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, cfg.cfg_id, layer, step, 7])))
    gumbel = g.gumbel(0.0, 1.0, size=(T, cfg.E))
    return (np.log(p)[None, :] + gumbel).astype(np.float32)

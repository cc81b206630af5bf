"""Seeded synthetic inputs for the MoE-layer workloads.

This package draws the layer's inputs (activations, router weights, expert
bias, expert weights) from counter-based random streams and rounds them into
the storage formats the layer reads (fp32, bf16, int8 blocks of 32 with an fp16
scale).  It performs no step of the MoE method itself: both the CPU oracle
and the GPU library consume the arrays it returns, and neither imports it.

The arithmetic lives in ``synth.c`` (built by :func:`build` with gcc); this
module only marshals numpy buffers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

u64 = ctypes.c_uint64
f64 = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, f64, f64, P]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, f64, f64, P]
        lib.synth_q8b32.argtypes = [u64, u64, u64, u64, u64, f64, P, P]
        lib.synth_uniform_f32.argtypes = [u64, u64, u64, u64, f64, f64, P]
        lib.synth_zipf_bias.argtypes = [u64, u64, ctypes.c_int32, f64, P, P]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_q8b32,
                  lib.synth_uniform_f32, lib.synth_zipf_bias):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f32(seed, stream, n, sigma, mean=0.0, start=0, out=None):
    """Elements [start, start+n) of a stream as fp32 ~ N(mean, sigma^2)."""
    out = np.empty(n, np.float32) if out is None else out
    _load().synth_normal_f32(seed, stream, start, n, mean, sigma, _ptr(out))
    return out


def normal_bf16(seed, stream, n, sigma, mean=0.0, start=0, out=None):
    """Same draws as :func:`normal_f32`, stored as bf16 bit patterns (uint16)."""
    out = np.empty(n, np.uint16) if out is None else out
    _load().synth_normal_bf16(seed, stream, start, n, mean, sigma, _ptr(out))
    return out


def q8b32(seed, stream, n_rows, cols, sigma, row0=0, q_out=None, s_out=None):
    """Rows [row0, row0+n_rows) of a normal matrix quantised to int8/32 + fp16 scale.

    Returns ``(q int8 [n_rows, cols], scale uint16-bits [n_rows, cols//32])``.
    """
    assert cols % 32 == 0
    q = np.empty((n_rows, cols), np.int8) if q_out is None else q_out
    s = np.empty((n_rows, cols // 32), np.uint16) if s_out is None else s_out
    _load().synth_q8b32(seed, stream, row0, n_rows, cols, sigma, _ptr(q), _ptr(s))
    return q, s


def uniform_f32(seed, stream, n, lo, hi, start=0):
    out = np.empty(n, np.float32)
    _load().synth_uniform_f32(seed, stream, start, n, lo, hi, _ptr(out))
    return out


def zipf_bias(seed, stream, n, beta):
    """Skew bias ``-beta * ln(rank)`` over a seeded ranking; returns (bias, rank)."""
    b = np.empty(n, np.float32)
    r = np.empty(n, np.int32)
    _load().synth_zipf_bias(seed, stream, n, beta, _ptr(b), _ptr(r))
    return b, r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (storage-format helper)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float32)

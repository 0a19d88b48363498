"""Test-side helpers: the oracle's pipeline over a workload, storage decoding in numpy.

The numpy decoders here are independent of both the oracle's C codecs and the
HIP kernels; they serve the dense-attention pins.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import poisoned_cache


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of each stored element (numpy/torch route)."""
    if dtype == "f32":
        return x.astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float64)
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    raise ValueError(dtype)


def torch_fp8_quantise(x_src: np.ndarray, src_dtype: str, scale: float) -> np.ndarray:
    """torch's own e4m3fn cast of fl32(x) / fl32(scale): an independent route to the codes."""
    xf = storage_to_f64(x_src, src_dtype).astype(np.float32)
    qf = xf / np.float32(scale)
    return torch.from_numpy(qf).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def oracle_step(orc, w, threads: int = 1, pairs=None):
    """One decode step through the oracle: fill the poisoned cache with the
    history, write the new tokens, attend.  Returns (k_cache, v_cache, new_slots, out)."""
    c = w.cfg
    kc = poisoned_cache(w)
    vc = poisoned_cache(w)
    if w.hist_seq.size:
        hs = orc.slot_mapping(w.hist_seq, w.hist_pos, w.block_tables, c.block_size)
        orc.kv_write(hs, w.hist_k, w.hist_v, c.src_dtype, kc, vc, c.kv_dtype, w.k_scale, w.v_scale)
    ns = orc.slot_mapping(w.new_seq, w.new_pos, w.block_tables, c.block_size)
    orc.kv_write(ns, w.new_k, w.new_v, c.src_dtype, kc, vc, c.kv_dtype, w.k_scale, w.v_scale)
    out = orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype, w.block_tables, w.context_lens, w.scale,
                     w.k_scale, w.v_scale, pairs=pairs, threads=threads)
    return kc, vc, ns, out


def attended_tokens(ctx: int, window: int = 0, sinks: int = 0) -> np.ndarray:
    """Positions a decode of a ctx-token context attends to: all of them (window 0), else
    the last `window` ones and the first `sinks` ones."""
    t = np.arange(ctx)
    if window == 0:
        return t
    return t[(t >= ctx - window) | (t < sinks)]


def free_blocks_outside_window(w, window: int, sinks: int) -> np.ndarray:
    """Block tables in which every block holding no attended token points at the
    NaN-filled sentinel block, as if the engine had freed it."""
    bt = w.block_tables.copy()
    B = w.cfg.block_size
    for s, ctx in enumerate(w.context_lens):
        used = set((attended_tokens(int(ctx), window, sinks) // B).tolist())
        for j in range((int(ctx) + B - 1) // B):
            if j not in used:
                bt[s, j] = w.sentinel_block
    return bt


def dense_causal(w, s: int, q_row: np.ndarray, pos: int) -> np.ndarray:
    """softmax(q K^T * scale) V over tokens 0 .. pos of sequence s's contiguous K/V for one
    query row [H_q][D] in the query dtype (fp64, numpy), per query head."""
    c = w.cfg
    k, v = w.logical_kv(s)
    k, v = k[:pos + 1], v[:pos + 1]
    if c.kv_dtype == "fp8":
        kf = storage_to_f64(torch_fp8_quantise(k, c.src_dtype, w.k_scale), "fp8") * w.k_scale
        vf = storage_to_f64(torch_fp8_quantise(v, c.src_dtype, w.v_scale), "fp8") * w.v_scale
    else:
        kf = storage_to_f64(k, c.kv_dtype)
        vf = storage_to_f64(v, c.kv_dtype)
    q = storage_to_f64(q_row, c.q_dtype)
    G = c.group
    out = np.empty((c.num_q_heads, c.head_dim))
    for h in range(c.num_q_heads):
        z = (kf[:, h // G, :] @ q[h]) * float(w.scale)
        p = np.exp(z - z.max())
        out[h] = (p @ vf[:, h // G, :]) / p.sum()
    return out


def dense_reference(w, s: int, window: int = 0, sinks: int = 0) -> np.ndarray:
    """softmax(q K^T * scale) V per query head on sequence s's contiguous K/V (fp64, numpy),
    over the attended rows (all of them unless a window is given).

    Independent of the paged layout: K and V come in logical order from the
    generator; fp8 values go through torch's e4m3fn cast."""
    c = w.cfg
    k, v = w.logical_kv(s)
    sel = attended_tokens(k.shape[0], window, sinks)
    k, v = k[sel], v[sel]
    if c.kv_dtype == "fp8":
        kf = storage_to_f64(torch_fp8_quantise(k, c.src_dtype, w.k_scale), "fp8") * w.k_scale
        vf = storage_to_f64(torch_fp8_quantise(v, c.src_dtype, w.v_scale), "fp8") * w.v_scale
    else:
        kf = storage_to_f64(k, c.kv_dtype)
        vf = storage_to_f64(v, c.kv_dtype)
    q = storage_to_f64(w.q[s], c.q_dtype)  # [H_q][D]
    G = c.group
    out = np.empty((c.num_q_heads, c.head_dim))
    for h in range(c.num_q_heads):
        K = kf[:, h // G, :]
        V = vf[:, h // G, :]
        z = (K @ q[h]) * float(w.scale)
        z = z - z.max()
        p = np.exp(z)
        out[h] = (p @ V) / p.sum()
    return out

"""Dense fp64 reference used to pin the oracle (test helper, numpy only).

Gathers each sequence's K and V into contiguous [L][Hkv][D] arrays -- the
static contiguous per-request layout that paging replaces -- by reshaping the
pool tensors with numpy, decodes the stored values without the oracle's
codecs (bf16 by bit shift, E4M3 through torch's float8_e4m3fn), and computes
softmax(scale * Q K^T) V with the KV heads repeated over their query group.
"""
import numpy as np
import torch

F32, BF16, E4M3 = 0, 1, 2


def f32(x) -> float:
    """Scales cross the library boundary as fp32; widen that exact value."""
    return float(np.float32(x))


def decode_np(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return a.astype(np.float64)
    if dtype == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def token_major(k_cache: np.ndarray, v_cache: np.ndarray):
    """Pool tensors -> [nb][H][16][D] views in token-major order."""
    nb, H, DX, BS, X = k_cache.shape
    K = k_cache.transpose(0, 1, 3, 2, 4).reshape(nb, H, BS, DX * X)
    V = v_cache.transpose(0, 1, 3, 2)
    return K, V


def gather(k_cache, v_cache, table_row, L):
    K, V = token_major(k_cache, v_cache)
    nblk = -(-L // K.shape[2])
    blocks = np.asarray(table_row[:nblk], dtype=np.int64)
    Ks = K[blocks].transpose(0, 2, 1, 3).reshape(nblk * K.shape[2], K.shape[1], K.shape[3])[:L]
    Vs = V[blocks].transpose(0, 2, 1, 3).reshape(nblk * V.shape[2], V.shape[1], V.shape[3])[:L]
    return Ks, Vs


def dense_attention(q, q_dtype, k_cache, v_cache, cache_dtype, tables, lens, scale,
                    k_scale=1.0, v_scale=1.0):
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale, k_scale, v_scale = (f32(x) for x in (scale, k_scale, v_scale))
    Q = decode_np(q, q_dtype)
    out = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), -np.inf)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        Ks, Vs = gather(k_cache, v_cache, tables[s], L)
        Kf = np.repeat(decode_np(Ks, cache_dtype) * float(k_scale), G, axis=1)  # [L][Hq][D]
        Vf = np.repeat(decode_np(Vs, cache_dtype) * float(v_scale), G, axis=1)
        sc = np.einsum("hd,thd->ht", Q[s], Kf) * float(scale)
        m = sc.max(axis=1, keepdims=True)
        e = np.exp(sc - m)
        w = e / e.sum(axis=1, keepdims=True)
        out[s] = np.einsum("ht,thd->hd", w, Vf)
        lse[s] = (m[:, 0] + np.log(e.sum(axis=1)))
    return out, lse


def sdpa_attention(q, q_dtype, k_cache, v_cache, cache_dtype, tables, lens, scale,
                   k_scale=1.0, v_scale=1.0):
    """Same, through torch.nn.functional.scaled_dot_product_attention (CPU fp64)."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale, k_scale, v_scale = (f32(x) for x in (scale, k_scale, v_scale))
    Q = torch.from_numpy(decode_np(q, q_dtype))
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        Ks, Vs = gather(k_cache, v_cache, tables[s], L)
        K = torch.from_numpy(decode_np(Ks, cache_dtype) * float(k_scale)).permute(1, 0, 2)
        V = torch.from_numpy(decode_np(Vs, cache_dtype) * float(v_scale)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            Q[s][:, None, :], K, V, scale=float(scale))
        out[s] = o[:, 0, :].numpy()
    return out


def dense_prefill(q, q_dtype, k_cache, v_cache, cache_dtype, tables, lens, qstart, scale,
                  k_scale=1.0, v_scale=1.0):
    """Chunked prefill as matrices: for sequence s, Q_s [C][Hq][D] against the
    gathered K/V [L][Hkv][D] with the boolean mask t <= L - C + j."""
    R, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale, k_scale, v_scale = (f32(x) for x in (scale, k_scale, v_scale))
    Q = decode_np(q, q_dtype)
    out = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), -np.inf)
    for s in range(len(lens)):
        L = int(lens[s])
        a, b = int(qstart[s]), int(qstart[s + 1])
        C = b - a
        if C == 0 or L == 0:
            continue
        Ks, Vs = gather(k_cache, v_cache, tables[s], L)
        Kf = np.repeat(decode_np(Ks, cache_dtype) * float(k_scale), G, axis=1)  # [L][Hq][D]
        Vf = np.repeat(decode_np(Vs, cache_dtype) * float(v_scale), G, axis=1)
        pos = L - C + np.arange(C)                                      # [C]
        mask = np.arange(L)[None, :] <= pos[:, None]                     # [C][L]
        sc = np.einsum("jhd,thd->hjt", Q[a:b], Kf) * float(scale)        # [Hq][C][L]
        sc = np.where(mask[None], sc, -np.inf)
        m = sc.max(axis=2, keepdims=True)
        live = np.isfinite(m)
        e = np.where(live, np.exp(sc - np.where(live, m, 0.0)), 0.0)
        z = e.sum(axis=2, keepdims=True)
        w = np.divide(e, z, out=np.zeros_like(e), where=z > 0)
        out[a:b] = np.einsum("hjt,thd->jhd", w, Vf)
        with np.errstate(divide="ignore"):
            lse[a:b] = np.where(z[..., 0] > 0, m[..., 0] + np.log(z[..., 0]), -np.inf).T
    return out, lse

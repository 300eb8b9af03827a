"""Oracle decoders: packed expert weights -> dense float64 matrices.  Test infrastructure.

The pages name a "Q2_0" 2-bit build and 3-bit builds (page "Strata Runs 125B
Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "The numbers, measured by the
author"; page "Strata: a 125B AI model on your gaming PC", model-size table) but
print no bit layout.  The layouts below are this project's own definition, and
this module is the oracle's reading of it:

A weight matrix W has N rows (output features) and K columns (input features),
N a multiple of 64 and K a multiple of 128.  It is cut into tiles of 64 rows x
64 columns, numbered t = (n // 64) * (K // 64) + k // 64.

* Q2 (2-bit, 32-weight blocks): code c in 0..3, weight = s * (c - 2) with s the
  fp16 scale of the row's 32-column block.
    code byte  = t * 1024 + (n % 64) * 16 + (k % 64) // 4,  bits 2 * (k % 4) and up
    scale index (fp16) = ((n // 64) * (K // 128) + (k // 32) // 4) * 256
                         + (n % 64) * 4 + (k // 32) % 4
* Q3 (3-bit, 32-weight blocks): code c = lo + 4 * hi in 0..7, weight = s * (c - 4).
  ``lo`` is a Q2-layout code plane; ``hi`` is a bit plane with 8 bytes per
  (tile, row): writing k % 64 = 16 * w + j (w in 0..3, j in 0..15), the bit sits
  at position  32 * (w // 2) + 8 * (w % 2) + (j % 8) + 16 * (j // 8)  of the
  little-endian 64-bit value at byte t * 512 + (n % 64) * 8.  Scales as Q2.
* BF16 (unquantised): element (n, k) at index
    ((n // 64) * (K // 8) + k // 8) * 512 + (n % 64) * 8 + k % 8.
* Router weight: plain row-major bf16 [E, H].

All conversions here are exact in float64.
"""
import numpy as np


def bf16_to_f64(bits):
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits):
    """fp16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_bf16_bits(a):
    """Round float64 to bf16 (nearest, ties to even) directly, without passing through fp32.

    Normal-range values: round the 52-bit fp64 significand to 7 stored bits at
    bit 45 (add half an ulp minus one plus the kept lsb, then truncate); the
    result is exactly a bf16 value.  Zeros, subnormal-range values, overflow and
    non-finite values go through the scalar definition ``_round_one_to_bf16``."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    u = a.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    v = r.view(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        out = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        special = ~np.isfinite(a) | (np.abs(a) < 2.0 ** -126) | ~(np.abs(v) < 2.0 ** 128)
    for i in np.flatnonzero(special.ravel()):
        out.flat[i] = _round_one_to_bf16(float(a.flat[i]))
    return out


def _round_one_to_bf16(v):
    # bf16 keeps 8 significant bits.  Find the two bf16 neighbours of v by
    # truncating its fp64 significand to 8 bits, then pick the nearer, ties to even.
    if v != v:
        return 0x7FC0
    if v == 0.0:
        return 0x8000 if np.signbit(v) else 0x0000
    sign = 0x8000 if v < 0 else 0
    if abs(v) == float("inf"):
        return sign | 0x7F80
    m, e = np.frexp(abs(v))            # abs(v) = m * 2**e, 0.5 <= m < 1
    e = int(e)
    if e - 1 < -126:                   # subnormal range of bf16: fixed spacing 2**-133
        ulp_exp = -133
    else:
        ulp_exp = e - 8                # 8 significant bits
    q = abs(v) / 2.0 ** ulp_exp        # exact scaling by a power of two
    lo = np.floor(q)
    rem = q - lo
    if rem > 0.5 or (rem == 0.5 and int(lo) % 2 == 1):
        lo += 1
    r = float(lo) * 2.0 ** ulp_exp
    if r >= 2.0 ** 128:                # overflow
        return sign | 0x7F80
    bits = int(np.float32(r).view(np.uint32)) >> 16
    return sign | bits


def _tile_index(N, K):
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    t = (n // 64) * (K // 64) + k // 64
    return n, k, t


def _scale_index(N, K):
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    b = k // 32
    return ((n // 64) * (K // 128) + b // 4) * 256 + (n % 64) * 4 + b % 4


def _check_shape(N, K):
    if N % 64 or K % 128:
        raise ValueError(f"matrix {N}x{K}: rows must be a multiple of 64 and columns of 128")


def q2_codes(codes, N, K):
    """Code c[n, k] in 0..3 from a Q2 code plane."""
    _check_shape(N, K)
    codes = np.asarray(codes, dtype=np.uint8)
    n, k, t = _tile_index(N, K)
    byte = t * 1024 + (n % 64) * 16 + (k % 64) // 4
    return (codes[byte] >> (2 * (k % 4)).astype(np.uint8)) & 3


def q3_hi_bits(hi, N, K):
    """High bit of the 3-bit code of every (n, k) from a Q3 hi plane."""
    _check_shape(N, K)
    hi = np.asarray(hi, dtype=np.uint8)
    n, k, t = _tile_index(N, K)
    w = (k % 64) // 16
    j = k % 16
    pos = 32 * (w // 2) + 8 * (w % 2) + (j % 8) + 16 * (j // 8)
    byte = t * 512 + (n % 64) * 8 + pos // 8
    return (hi[byte] >> (pos % 8).astype(np.uint8)) & 1


def block_scales(scales, N, K):
    """fp16 scale of the block holding (n, k), as float64 [N, K]."""
    _check_shape(N, K)
    return fp16_to_f64(np.asarray(scales, dtype=np.uint16)[_scale_index(N, K)])


def decode_q2(codes, scales, N, K):
    """Dense float64 W[N, K] of a Q2 matrix: s * (c - 2)."""
    c = q2_codes(codes, N, K).astype(np.float64)
    return block_scales(scales, N, K) * (c - 2.0)


def decode_q3(lo, hi, scales, N, K):
    """Dense float64 W[N, K] of a Q3 matrix: s * (lo + 4 * hi - 4)."""
    c = q2_codes(lo, N, K).astype(np.float64) + 4.0 * q3_hi_bits(hi, N, K).astype(np.float64)
    return block_scales(scales, N, K) * (c - 4.0)


def decode_bf16_tiled(w, N, K):
    """Dense float64 W[N, K] of an unquantised matrix in the 64 x 8 tiled bf16 layout."""
    if N % 64 or K % 8:
        raise ValueError(f"matrix {N}x{K}: rows must be a multiple of 64 and columns of 8")
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    idx = ((n // 64) * (K // 8) + k // 8) * 512 + (n % 64) * 8 + k % 8
    return bf16_to_f64(np.asarray(w, dtype=np.uint16)[idx])


def expert_matrices(fmt, tensors, H, I, j=0):
    """(W_gate [I, H], W_up [I, H], W_down [H, I]) of expert j of a bank, dense float64.

    The gate/up matrix W13 has 2I rows: rows [0, I) are the gate projection and
    rows [I, 2I) the up projection; W2 is the down projection [H, I]."""
    n13, n2 = 2 * I * H, H * I
    if fmt == "bf16":
        w13 = decode_bf16_tiled(tensors["w13"][j * n13:(j + 1) * n13], 2 * I, H)
        w2 = decode_bf16_tiled(tensors["w2"][j * n2:(j + 1) * n2], H, I)
    elif fmt == "q2":
        w13 = decode_q2(tensors["w13"][j * n13 // 4:(j + 1) * n13 // 4],
                        tensors["w13_scale"][j * n13 // 32:(j + 1) * n13 // 32], 2 * I, H)
        w2 = decode_q2(tensors["w2"][j * n2 // 4:(j + 1) * n2 // 4],
                       tensors["w2_scale"][j * n2 // 32:(j + 1) * n2 // 32], H, I)
    elif fmt == "q3":
        w13 = decode_q3(tensors["w13"][j * n13 // 4:(j + 1) * n13 // 4],
                        tensors["w13_hi"][j * n13 // 8:(j + 1) * n13 // 8],
                        tensors["w13_scale"][j * n13 // 32:(j + 1) * n13 // 32], 2 * I, H)
        w2 = decode_q3(tensors["w2"][j * n2 // 4:(j + 1) * n2 // 4],
                       tensors["w2_hi"][j * n2 // 8:(j + 1) * n2 // 8],
                       tensors["w2_scale"][j * n2 // 32:(j + 1) * n2 // 32], H, I)
    else:
        raise ValueError(fmt)
    return w13[:I], w13[I:], w2

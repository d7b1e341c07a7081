"""Seeded synthetic GGUF blocks, activations and router logits.

Shared by the tests, the bench and the smoke check as the single source of
inputs for both the HIP path and the oracle.  It only draws random fields and
packs them at their byte offsets in a block; it performs no dequantization,
dot product, activation or routing arithmetic.

Block byte layouts (little-endian, blocks contiguous, rows contiguous):
  Q8_0  34 B / 32 values : f16 d | int8 q[32]
  Q4_0  18 B / 32 values : f16 d | u8 nibbles[16]
  Q4_K 144 B / 256 values: f16 d | f16 dmin | u8 scales[12] | u8 qs[128]
  Q6_K 210 B / 256 values: u8 ql[128] | u8 qh[64] | int8 scales[16] | f16 d
Draw order inside each generator is fixed, so a seed names one input exactly.
f16 fields are encoded with numpy's round-to-nearest-even float16 cast.
"""
import numpy as np

Q4_0, Q8_0, Q4_K, Q6_K = 2, 8, 12, 14
QK = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q6_K: 210}
NAMES = {Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K"}


def rng(seed):
    return np.random.default_rng(seed)


def row_bytes(t, cols):
    assert cols % QK[t] == 0
    return cols // QK[t] * BLOCK_BYTES[t]


def _f16_bytes(v):
    return np.ascontiguousarray(np.asarray(v, np.float32).astype(np.float16)).view(np.uint8)


def _abs_normal_f16(g, n, sigma):
    return _f16_bytes(np.abs(g.normal(0.0, sigma, n))).reshape(n, 2)


def q8_0(g, rows, cols, sigma=0.02):
    """d = f16(|N(0, sigma)|); codes uniform int8 on [-127, 127]."""
    nb = rows * (cols // 32)
    d = _abs_normal_f16(g, nb, sigma)
    q = g.integers(-127, 128, size=(nb, 32), dtype=np.int8).view(np.uint8)
    return np.concatenate([d, q], axis=1).reshape(rows, -1)


def q4_0(g, rows, cols, sigma=0.02):
    """d = f16(|N(0, sigma)|); nibble bytes uniform on 0..255 (nibbles uniform 0..15)."""
    nb = rows * (cols // 32)
    d = _abs_normal_f16(g, nb, sigma)
    q = g.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    return np.concatenate([d, q], axis=1).reshape(rows, -1)


def q4_k(g, rows, cols, sigma=0.01):
    """d, dmin = f16(|N(0, sigma)|); the 12 scale bytes and 128 qs bytes uniform."""
    nb = rows * (cols // 256)
    d = _abs_normal_f16(g, nb, sigma)
    dmin = _abs_normal_f16(g, nb, sigma)
    sc = g.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    return np.concatenate([d, dmin, sc, qs], axis=1).reshape(rows, -1)


def q6_k(g, rows, cols, sigma=0.01):
    """ql, qh bytes uniform; int8 scales uniform over all 256 values; d = f16(|N(0, sigma)|)."""
    nb = rows * (cols // 256)
    ql = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    qh = g.integers(0, 256, size=(nb, 64), dtype=np.uint8)
    sc = g.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    d = _abs_normal_f16(g, nb, sigma)
    return np.concatenate([ql, qh, sc, d], axis=1).reshape(rows, -1)


GEN = {Q8_0: q8_0, Q4_0: q4_0, Q4_K: q4_k, Q6_K: q6_k}
DEFAULT_SIGMA = {Q8_0: 0.02, Q4_0: 0.02, Q4_K: 0.01, Q6_K: 0.01}


def weights(t, g, rows, cols, sigma=None):
    return GEN[t](g, rows, cols, DEFAULT_SIGMA[t] if sigma is None else sigma)


def activations(g, ntok, n):
    """x ~ N(0, 1) f32, token-major [ntok][n]."""
    return g.standard_normal((ntok, n), dtype=np.float32)


def logits(g, ntok, E):
    """router logits ~ N(0, 1) f32 [ntok][E]."""
    return g.standard_normal((ntok, E), dtype=np.float32)


def down_scales(g, E):
    """per-expert down scale ~ U(0.5, 2) f32 [E]."""
    return g.uniform(0.5, 2.0, E).astype(np.float32)


def expert_pool(t, g, E, H, F, sigma=None):
    """E expert records, each [gate||up (2F x H) blocks][down (H x F) blocks].

    Returns (pool bytes [E * record], record, gate_up_offset, down_offset)."""
    gu_b = 2 * F * row_bytes(t, H)
    d_b = H * row_bytes(t, F)
    rec = gu_b + d_b
    pool = np.empty(E * rec, np.uint8)
    for e in range(E):
        pool[e * rec:e * rec + gu_b] = weights(t, g, 2 * F, H, sigma).ravel()
        pool[e * rec + gu_b:(e + 1) * rec] = weights(t, g, H, F, sigma).ravel()
    return pool, rec, 0, gu_b


# ---- the five workloads ------------------------------------------------------
# Each returns a dict of numpy arrays plus shape metadata; drawing order fixed.

def config0(seed=0):
    """Q8_0 GEMV, 1 token: W 1024 x 2048, x [2048]."""
    g = rng(seed)
    W = q8_0(g, 1024, 2048)
    x = activations(g, 1, 2048)
    return dict(name="q8_0_gemv_1024x2048", type=Q8_0, W=W, x=x, rows=1024, cols=2048, ntok=1)


def config1(seed=0, head_rows=151936):
    """Dense Qwen3-style MLP at Q8_0, 1 token: hidden 2560, ff 9728, tied head."""
    g = rng(seed)
    H, F = 2560, 9728
    Wg = q8_0(g, F, H)
    Wu = q8_0(g, F, H)
    Wd = q8_0(g, H, F)
    Wh = q8_0(g, head_rows, H)
    x = activations(g, 1, H)
    return dict(name="q8_0_dense_mlp_2560x9728_head_%d" % head_rows, type=Q8_0, H=H, F=F,
                Wg=Wg, Wu=Wu, Wd=Wd, Wh=Wh, head_rows=head_rows, x=x, ntok=1)


def config2(seed=0, E=128):
    """Qwen3-30B-A3B-shaped MoE at Q8_0, 1 token: H 2048, E experts of ff 768, top-8."""
    g = rng(seed)
    H, F, k = 2048, 768, 8
    pool, rec, gu_off, d_off = expert_pool(Q8_0, g, E, H, F)
    lg = logits(g, 1, E)
    x = activations(g, 1, H)
    return dict(name="q8_0_moe_2048_e%d_ff768_top8" % E, type=Q8_0, H=H, F=F, E=E, k=k,
                pool=pool, record=rec, gu_off=gu_off, d_off=d_off, logits=lg, x=x, ntok=1,
                slots=np.arange(E, dtype=np.int32), down_scale=None)


def config3(seed=0):
    """K-quant dense GEMVs, 1 token: Q4_K 17408 x 5120 and Q6_K 5120 x 17408."""
    g = rng(seed)
    W4 = q4_k(g, 17408, 5120)
    x4 = activations(g, 1, 5120)
    W6 = q6_k(g, 5120, 17408)
    x6 = activations(g, 1, 17408)
    return dict(name="kquant_gemv", W4=W4, x4=x4, W6=W6, x6=x6)


def config4(seed=0, ntok=1, E=128):
    """Gemma4-26B-A4B-shaped Q4_0: dense GELU MLP (H 2816, ff 2112) beside E experts
    (ff 704, fused gate_up), per-expert down scale, top-8; T tokens."""
    g = rng(seed)
    H, Fd, F, k = 2816, 2112, 704, 8
    Wg = q4_0(g, Fd, H)
    Wu = q4_0(g, Fd, H)
    Wd = q4_0(g, H, Fd)
    pool, rec, gu_off, d_off = expert_pool(Q4_0, g, E, H, F)
    ds = down_scales(g, E)
    lg = logits(g, ntok, E)
    x = activations(g, ntok, H)
    return dict(name="q4_0_gemma_moe_2816_e%d_ff704_top8_t%d" % (E, ntok), type=Q4_0, H=H,
                Fd=Fd, F=F, E=E, k=k, Wg=Wg, Wu=Wu, Wd=Wd, pool=pool, record=rec,
                gu_off=gu_off, d_off=d_off, down_scale=ds, logits=lg, x=x, ntok=ntok,
                slots=np.arange(E, dtype=np.int32))


# ---- the same recipes drawn on the GPU (timing-size inputs) ------------------
# Seeded torch generator on the device; same distributions and byte layout as
# the numpy generators above (a different random stream).  Used where only
# the shapes and distributions matter (bandwidth timing), never for parity.

def device_weights(t, rows, cols, gen, device="cuda", sigma=None):
    import torch
    sigma = DEFAULT_SIGMA[t] if sigma is None else sigma
    nb = rows * (cols // QK[t])

    def f16(n):
        return (torch.randn(n, generator=gen, device=device) * sigma).abs().half().view(torch.uint8).view(n, 2)

    def u8(n, k):
        return torch.randint(0, 256, (n, k), generator=gen, device=device, dtype=torch.uint8)

    if t == Q8_0:
        q = torch.randint(-127, 128, (nb, 32), generator=gen, device=device, dtype=torch.int8).view(torch.uint8)
        parts = [f16(nb), q]
    elif t == Q4_0:
        parts = [f16(nb), u8(nb, 16)]
    elif t == Q4_K:
        parts = [f16(nb), f16(nb), u8(nb, 12), u8(nb, 128)]
    else:
        parts = [u8(nb, 128), u8(nb, 64), u8(nb, 16), f16(nb)]
    return torch.cat(parts, dim=1).view(rows, -1)


def device_activations(ntok, n, gen, device="cuda"):
    import torch
    return torch.randn((ntok, n), generator=gen, device=device, dtype=torch.float32)


# ---- whole FFN blocks (the steps around the MoE) -------------------------------

def norm_weights(g, n):
    """a norm's gain vector ~ U(0.5, 1.5) f32 [n] (stand-in for trained gains near 1)."""
    return g.uniform(0.5, 1.5, n).astype(np.float32)


def f32_matrix(g, rows, cols, sigma):
    """plain f32 weights ~ N(0, sigma) [rows][cols] (router, shared-expert gate)."""
    return (g.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def qwen35_block(seed=0, ntok=1, t=Q8_0, H=2048, E=256, F=512, SF=512, k=8):
    """Qwen3.5/3.6-MoE-style FFN block: post-attention RMS norm, f32 router
    [E x H] (sigma 1/sqrt(H), so logits are about N(0, 1)), E routed experts of
    ff F, top-k, and a shared expert of ff SF with an f32 gate row; residual
    stream x ~ N(0, 1)."""
    g = rng(seed)
    pool, rec, gu_off, d_off = expert_pool(t, g, E, H, F)
    sg = weights(t, g, SF, H)
    su = weights(t, g, SF, H)
    sd = weights(t, g, H, SF)
    return dict(name="qwen35_moe_block_h%d_e%d_ff%d_shared%d_top%d_t%d" % (H, E, F, SF, k, ntok), type=t, H=H,
                F=F, SF=SF, E=E, k=k, pool=pool, record=rec, gu_off=gu_off, d_off=d_off,
                sh_gate=sg, sh_up=su, sh_down=sd,
                sh_gate_inp=f32_matrix(g, 1, H, 1.0 / np.sqrt(H))[0],
                router=f32_matrix(g, E, H, 1.0 / np.sqrt(H)), norm=norm_weights(g, H),
                x=activations(g, ntok, H), ntok=ntok, slots=np.arange(E, dtype=np.int32))


def gemma_block(seed=0, ntok=1, E=128):
    """Gemma4-26B-A4B-style FFN block at Q4_0: the dense GELU MLP (ff 2112) and
    the MoE (E experts of ff 704, top-8, per-expert down scale) with their
    norms: ffn_norm, pre_ffw_norm_2, the router's scale (router input
    rmsnorm * 1/sqrt(H) * scale; f32 router [E x H] ~ N(0, 1), so logits are
    about N(0, 1)), post_ffw_norm_1 / _2, post_ffw_norm and the layer's output
    scalar ~ U(0.5, 1); residual stream x ~ N(0, 1)."""
    c = config4(seed, ntok, E)
    g = rng(seed + 7919)
    H = c["H"]
    c.update(name="gemma_ffn_block_2816_e%d_t%d" % (E, ntok), router=f32_matrix(g, E, H, 1.0),
             w_ffn=norm_weights(g, H), w_pre2=norm_weights(g, H), w_rscale=norm_weights(g, H),
             w_post1=norm_weights(g, H), w_post2=norm_weights(g, H), w_post=norm_weights(g, H),
             out_scale=np.array([g.uniform(0.5, 1.0)], np.float32))
    return c

"""Seeded synthetic inputs with the shapes and value distributions of the
five workloads.

The pages evaluate on WikiText/PG19 with Huginn-0125 (RAMP page, section
6.1), GSM8K with Qwen3-0.6B (escalation article) and LLaMA/Qwen2.5 with
perplexity/MMLU (ARCQuant page, experimental results).  None of those
weights or datasets is used: these generators stand in for them with
synthetic tensors of the same shapes (Qwen3-0.6B-shaped linears, 4K-token
prefill) and with outlier channels of the kind the ARCQuant and Day-0 pages
describe.

Seeds: numpy PCG64 seeded from SeedSequence(20261203 + config) with a
spawn key per sub-problem; each sub-problem spawns four streams in a fixed
order: A (activations), W (weights), outlier-channel choice, flags.
Draws are made in float64, cast to float32, then to BF16 (round to nearest
even) by torch's dtype cast.
"""

import numpy as np
import torch

SEED_BASE = 20261203

# Qwen3-0.6B linear shapes (name, K = in_features, N = out_features)
QWEN3_LINEARS = (
    ("q_proj", 1024, 2048),
    ("k_proj", 1024, 1024),
    ("v_proj", 1024, 1024),
    ("o_proj", 2048, 1024),
    ("gate_proj", 1024, 3072),
    ("up_proj", 1024, 3072),
    ("down_proj", 3072, 1024),
)
QWEN3_LAYERS = 28
QWEN3_LM_HEAD = ("lm_head", 1024, 151936)


def streams(config, sub=0):
    """Four generators (A, W, outliers, flags) for (config, sub-problem)."""
    ss = np.random.SeedSequence(entropy=SEED_BASE + config, spawn_key=(sub,))
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def to_bf16_bits(x):
    """float64 draws -> float32 -> BF16 (torch cast) -> uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _outlier_channels(rng, K, count):
    return np.sort(rng.choice(K, size=count, replace=False))


# ------------------------------------------------------------ config 1 --

def c1_gemm_mxfp4(M=128, K=1024, N=1024):
    """Single MXFP4 GEMM: A ~ N(0,1) with 8 outlier channels x20,
    W ~ N(0, 0.02^2)."""
    ra, rw, ro, _ = streams(1)
    a = ra.standard_normal((M, K))
    ch = _outlier_channels(ro, K, 8)
    a[:, ch] *= 20.0
    w = rw.normal(0.0, 0.02, (N, K))
    return dict(a=to_bf16_bits(a), w=to_bf16_bits(w), outliers=ch)


# ------------------------------------------------------------ config 2 --

def c2_linear(i, M=4096):
    """Linear i of the Qwen3-0.6B set at M tokens, MXFP8: A ~ N(0,1) with
    round(0.01 K) channels x15, W ~ N(0, 0.02^2)."""
    name, K, N = QWEN3_LINEARS[i]
    ra, rw, ro, _ = streams(2, i)
    a = ra.standard_normal((M, K))
    ch = _outlier_channels(ro, K, int(round(0.01 * K)))
    a[:, ch] *= 15.0
    w = rw.normal(0.0, 0.02, (N, K))
    return dict(name=name, a=to_bf16_bits(a), w=to_bf16_bits(w), outliers=ch)


# Inputs of one transformer layer: q/k/v read the same (normed) hidden
# state and gate/up the same MLP input, so a layer has four activation
# tensors.  Each group's input is the first member's c2_linear activation;
# its weights are the members' matrices stacked along N.
QWEN3_GROUPS = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))


def c2_layer(M=4096):
    """The linear set of one layer as four GEMMs on shared inputs: list of
    dict(name, members, a [M x K] BF16 bits, w [sum N x K] BF16 bits, Ns)."""
    out = []
    for gname, members in QWEN3_GROUPS:
        ds = [c2_linear(i, M=M) for i in members]
        out.append(dict(name=gname, members=[d["name"] for d in ds], a=ds[0]["a"],
                        w=np.concatenate([d["w"] for d in ds], axis=0), Ns=[d["w"].shape[0] for d in ds]))
    return out


# ------------------------------------------------------------ config 3 --

def c3_arc(M=4096, K=4096, N=4096, n_outliers=64):
    """ARC GEMM: A ~ Student-t(3) with 64 channels x20, W ~ N(0, 0.02^2)."""
    ra, rw, ro, _ = streams(3)
    a = ra.standard_t(3.0, (M, K))
    ch = _outlier_channels(ro, K, n_outliers)
    a[:, ch] *= 20.0
    w = rw.normal(0.0, 0.02, (N, K))
    return dict(a=to_bf16_bits(a), w=to_bf16_bits(w), outliers=ch)


# ------------------------------------------------------------ config 4 --

def _spectral_rescale(w, rng, target=0.9, iters=100):
    """Rescale w so its largest singular value (power iteration) is target."""
    v = rng.standard_normal(w.shape[1])
    v /= np.linalg.norm(v)
    sigma = 0.0
    for _ in range(iters):
        u = w @ v
        u /= np.linalg.norm(u)
        v = w.T @ u
        sigma = np.linalg.norm(v)
        v /= sigma
    return w * (target / sigma)


def c4_ramp(S=4096, D=2048, F=5632, tied=False):
    """Recurrent block h <- h + W2 SiLU(W1 RMSNorm(h)): h0 ~ N(0,1),
    W1 [F, D] and W2 [D, F] ~ N(0,1) rescaled to spectral norm 0.9.
    tied=True uses W2 = -W1^T (a negative-feedback, contractive variant)."""
    ra, rw, ro, _ = streams(4, 1 if tied else 0)
    h0 = ra.standard_normal((S, D))
    w1 = _spectral_rescale(rw.standard_normal((F, D)), ro)
    w2 = -w1.T.copy() if tied else _spectral_rescale(rw.standard_normal((D, F)), ro)
    return dict(h0=to_bf16_bits(h0), w1=to_bf16_bits(w1), w2=to_bf16_bits(w2))


# ------------------------------------------------------------ config 5 --

def int8_weights_fp16_scales(rng, N, K, std=0.02):
    """int8 weights with one FP16 scale per 32 along K: draw W ~ N(0, std^2),
    s = fp16(amax/127) per block (1 for an all-zero block),
    q = clip(rint(w / s), -127, 127)."""
    w = rng.normal(0.0, std, (N, K))
    blocks = w.reshape(N, K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    s16 = np.where(amax > 0, amax / 127.0, 1.0).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    q = np.rint(blocks / s16.astype(np.float64)[..., None])
    q = np.clip(q, -127, 127).astype(np.int8).reshape(N, K)
    return q, s16


def c5_linear_list():
    """(name, K, N) for the 28 x 7 layer linears followed by the LM head."""
    out = []
    for layer in range(QWEN3_LAYERS):
        for name, K, N in QWEN3_LINEARS:
            out.append((f"layers.{layer}.{name}", K, N))
    out.append(QWEN3_LM_HEAD)
    return out


def c5_flags(B=16, frac=0.15):
    """Exactly round(frac * B) flagged tokens, by a seeded permutation."""
    _, _, _, rf = streams(5, 10_000)
    nflag = int(round(frac * B))
    f = np.zeros(B, dtype=np.uint8)
    f[rf.permutation(B)[:nflag]] = 1
    return f


def c5_linear(i, B=16, N=None, K=None):
    """Linear i of the decode sweep (see c5_linear_list), optionally with
    its shape overridden: int8 W with FP16 scales, x ~ N(0,1) BF16 [B, K]."""
    name, K0, N0 = c5_linear_list()[i]
    K = K0 if K is None else K
    N = N0 if N is None else N
    ra, rw, _, _ = streams(5, i)
    w, s = int8_weights_fp16_scales(rw, N, K)
    x = to_bf16_bits(ra.standard_normal((B, K)))
    return dict(name=name, w=w, scales=s, x=x, flags=c5_flags(B))


# ------------------------------------------------------------ KV tiles --

def kv_tiles(T=256, H=8, D=128):
    """K/V vectors ~ N(0,1) BF16 with a few outlier tokens x20."""
    ra, _, ro, _ = streams(6)
    x = ra.standard_normal((T, H, D))
    tok = _outlier_channels(ro, T, max(1, T // 64))
    x[tok] *= 20.0
    return dict(x=to_bf16_bits(x))

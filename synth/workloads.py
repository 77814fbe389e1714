"""Seeded synthetic inputs for the HARP rotated low-bit linear.

This module draws the raw buffers that cross the library boundary and feeds
both the HIP library (through the tests and the bench) and the float64
oracle.  It holds none of the method's arithmetic: no butterfly, no
quantizer, no packing, no dequantization.  Every buffer is drawn directly in
its boundary format:

* rotation: per side, float32 (cos t, sin t) with t = pi/4 + N(0, var 0.05)
  per stage and block (pi/4 is the Hadamard initialisation of the page's
  zero-initialised Givens angle), and a random sign bitmask;
* mixed-radix rotation: per stage and group the learnable parameters
  (Givens angle or Cayley upper triangle) drawn as N(0, 0.1^2) around the
  zero initialisation, a random sign bitmask, and per radix that is not a
  power of two the one fixed standard Gaussian matrix whose QR factor is its
  mixer (the blocks themselves are an offline expansion of these inputs);
* int8-stored rotation: the same angle spread drawn directly as int8 codes
  (a normal rounded to integers, clipped to [-127, 127]) with one float32
  step per side chosen so that +-127 codes span +-4 standard deviations;
* packed weights: uniformly random uint32 words (so every B-bit code is
  uniform on [0, 2^B - 1]), fp16 group scales with the magnitude a min-max
  grid gives for N(0, 0.02^2) weights, and integer fp16 zeros near the middle
  of the grid;
* activations: N(0, 1) with 1 % outlier channels scaled by 20, stored as
  bf16 (or float32 for the tiny layer);
* dense weights (offline-pipeline checks only): N(0, std^2) with the same
  outlier columns scaled by 20.

The layer shapes are those of Llama-2-7B, Qwen3-8B and Llama-2-70B linears
(the models the HARP pages evaluate); no checkpoint or dataset is used.

Seeds: numpy SeedSequence([config id, tensor id, linear index, instance]).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# tensor ids inside a seed sequence
T_W, T_X, T_THETA_V, T_THETA_U, T_SIGN_V, T_SIGN_U, T_OUTLIER = range(7)
T_SCALE, T_ZERO = 7, 8

THETA_VAR = 0.05        # angle perturbation variance around pi/4 (rad^2)
CODE_SPAN_SIGMAS = 4.0  # int8 angle codes: +-127 covers this many std devs
OUTLIER_FRAC = 0.01
OUTLIER_GAIN = 20.0


@dataclass(frozen=True)
class Linear:
    """One linear layer: K inputs -> N outputs, butterfly block per side."""
    name: str
    K: int
    N: int
    b_v: int      # block size on the input side (K)
    b_u: int      # block size on the output side (N)


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    linears: tuple
    bits: tuple
    Ms: tuple
    x_dtype: str = "bf16"       # "bf16" or "f32"
    w_std: float = 0.02
    outliers: bool = True
    notes: str = ""


CONFIGS = {
    "tiny": Config(
        1, "tiny", (Linear("w256", 256, 256, 256, 256),), (2,), (4,),
        x_dtype="f32", w_std=1.0 / 16.0, outliers=False,
        notes="256x256, b=256 both sides, 2-bit, M=4 float32"),
    "l7b_decode": Config(
        2, "l7b_decode", (Linear("attn4096", 4096, 4096, 4096, 4096),),
        (2,), (1,), notes="Llama-2-7B attention projection, decode"),
    "l7b_mlp": Config(
        3, "l7b_mlp",
        (Linear("up4096_11008", 4096, 11008, 4096, 256),
         Linear("down11008_4096", 11008, 4096, 256, 4096)),
        (2,), (1, 16), notes="Llama-2-7B MLP, 11008 = 43 x 256 blocks"),
    "q8b_prefill": Config(
        4, "q8b_prefill",
        (Linear("attn4096", 4096, 4096, 4096, 4096),
         Linear("up4096_12288", 4096, 12288, 4096, 256),
         Linear("down12288_4096", 12288, 4096, 256, 4096)),
        (2, 4), (512,), notes="Qwen3-8B prefill, 12288 = 48 x 256 blocks"),
    "l70b_slice": Config(
        5, "l70b_slice",
        (Linear("attn8192", 8192, 8192, 8192, 8192),
         Linear("up8192_28672", 8192, 28672, 8192, 256),
         Linear("down28672_8192", 28672, 8192, 256, 8192)),
        (2, 3, 4), (1, 32), notes="Llama-2-70B slice, 28672 = 112 x 256"),
}


def rng_for(cid: int, tensor: int, lin: int = 0, inst: int = 0):
    return np.random.default_rng(np.random.SeedSequence([cid, tensor, lin, inst]))


@dataclass
class Rotation:
    """One side's parameters in boundary format."""
    dim: int
    block: int
    cs: np.ndarray          # float32 [dim/b][log2 b][b/2][2] = (cos t, sin t), or None
    sign_bits: np.ndarray   # uint32 [ceil(dim/32)], bit i set -> d_i = -1
    theta: np.ndarray = field(repr=False, default=None)  # float64 angles
    phi_codes: np.ndarray = None  # int8 [dim/b][log2 b][b/2] when cs is None
    phi_step: float = 0.0         # float32 step of the codes


def rotation(dim: int, block: int, rng, theta_var: float = THETA_VAR,
             theta=None) -> Rotation:
    """Draw one side: angles pi/4 + N(0, theta_var), random sign bitmask.

    ``theta`` (shape [dim/b][L][b/2]) overrides the random angles.
    """
    if block < 2 or block & (block - 1) or dim % block:
        raise ValueError("block must be a power of two dividing dim")
    L = block.bit_length() - 1
    if theta is None:
        theta = math.pi / 4 + rng.normal(0.0, math.sqrt(theta_var),
                                         size=(dim // block, L, block // 2))
    theta = np.asarray(theta, dtype=np.float64)
    cs = np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)
    return Rotation(dim, block, np.ascontiguousarray(cs), _sign_bits(dim, rng), theta)


def _sign_bits(dim: int, rng) -> np.ndarray:
    nw = (dim + 31) // 32
    bits = rng.integers(0, 2 ** 32, size=nw, dtype=np.uint64).astype(np.uint32)
    if dim % 32:
        bits[-1] &= np.uint32((1 << (dim % 32)) - 1)
    return bits


def rotation_q8(dim: int, block: int, rng, theta_var: float = THETA_VAR,
                codes=None, step=None) -> Rotation:
    """Draw one side with int8-stored angles and a random sign bitmask.

    Codes are integers drawn from N(0, theta_var / step^2), rounded and
    clipped to [-127, 127]; step = CODE_SPAN_SIGMAS * sqrt(theta_var) / 127
    in float32.  ``codes`` ([dim/b][L][b/2] int8) and ``step`` override.
    """
    if block < 2 or block & (block - 1) or dim % block:
        raise ValueError("block must be a power of two dividing dim")
    L = block.bit_length() - 1
    if step is None:
        step = CODE_SPAN_SIGMAS * math.sqrt(theta_var) / 127.0
    step = np.float32(step)
    if codes is None:
        z = rng.normal(0.0, math.sqrt(theta_var) / float(step),
                       size=(dim // block, L, block // 2))
        codes = np.clip(np.rint(z), -127, 127)
    codes = np.ascontiguousarray(np.asarray(codes).astype(np.int8))
    if codes.shape != (dim // block, L, block // 2):
        raise ValueError("codes must have shape [dim/b][log2 b][b/2]")
    return Rotation(dim, block, None, _sign_bits(dim, rng), None, codes, float(step))


@dataclass
class MixedRotation:
    """One side with a mixed-radix schedule: learnable parameters per stage
    and group (Givens angle for radix 2, the b(b-1)/2 upper-triangle entries
    of the Cayley parameter otherwise), a random sign bitmask, and per stage
    whose radix is not a power of two the fixed b x b standard Gaussian whose
    QR factor is that radix's mixer (None for powers of two)."""
    dim: int
    radices: tuple
    params: list            # [t] -> float64 (dim / b_t, b_t (b_t - 1) / 2)
    sign_bits: np.ndarray
    gaussians: list = None  # [t] -> float64 (b_t, b_t) or None


def mixer_gaussian(b: int, mixer_seed: int = 0) -> np.ndarray:
    """The fixed b x b standard Gaussian of radix b: drawn once with numpy
    default_rng(mixer_seed + b), so every stage and group of that radix
    shares it."""
    return np.random.default_rng(mixer_seed + b).normal(size=(b, b))


def mixer_gaussians(radices, mixer_seed: int = 0) -> list:
    """Per stage: mixer_gaussian(b_t) when b_t is not a power of two, else None."""
    return [None if b & (b - 1) == 0 else mixer_gaussian(int(b), mixer_seed)
            for b in radices]


def mixed_rotation(radices, rng, scale: float = 0.1, mixer_seed: int = 0) -> MixedRotation:
    """Draw the parameters as N(0, scale^2) around the zero initialisation."""
    radices = tuple(int(b) for b in radices)
    dim = int(np.prod(radices))
    params = [rng.normal(0.0, scale, size=(dim // b, b * (b - 1) // 2)) for b in radices]
    return MixedRotation(dim, radices, params, _sign_bits(dim, rng),
                         mixer_gaussians(radices, mixer_seed))


@dataclass
class QWeight:
    """Packed weight in boundary format."""
    N: int
    K: int
    bits: int
    words: np.ndarray       # uint32 [N][K*bits/32]
    scale: np.ndarray       # uint16 fp16 bits [N][K/64]
    zero: np.ndarray        # uint16 fp16 bits [N][K/64], integer-valued


def qweight(N: int, K: int, bits: int, rng, w_std: float = 0.02,
            spread: str = "mid") -> QWeight:
    """Random packed weight with realistic group scales and zeros.

    spread "mid": for N(0, std^2) groups of 64 the min-max range is about
    4.8 std, so s ~ 4.8 std / (2^B - 1), varied by a factor U(0.75, 1.25)
    per group; zeros are the integers nearest the middle of [0, 2^B - 1].

    spread "wide" (edge coverage of the boundary format): zeros uniform over
    the whole grid [0, 2^B - 1], the first and last group of every row pinned
    to 0 and 2^B - 1; scales 2^e with e uniform in [-24, 4], i.e. across the
    fp16 range from its smallest subnormal (2^-24) up, rounded to fp16, with
    the second group of every row pinned to 2^-24 and the third to the
    largest subnormal (1023 * 2^-24).
    """
    if bits not in (2, 3, 4) or K % 64:
        raise ValueError("bits in {2,3,4} and K % 64 == 0")
    if spread not in ("mid", "wide"):
        raise ValueError("spread must be 'mid' or 'wide'")
    qmax = (1 << bits) - 1
    nw = K * bits // 32
    words = rng.integers(0, 2 ** 32, size=(N, nw), dtype=np.uint64).astype(np.uint32)
    G = K // 64
    if spread == "mid":
        s = (4.8 * w_std / qmax) * rng.uniform(0.75, 1.25, size=(N, G))
        z = rng.integers(qmax // 2, qmax // 2 + 2, size=(N, G)).astype(np.float16)
    else:
        s = np.exp2(rng.uniform(-24.0, 4.0, size=(N, G)))
        z = rng.integers(0, qmax + 1, size=(N, G)).astype(np.float16)
        z[:, 0] = 0
        z[:, -1] = qmax
        if G > 1:
            s[:, 1] = 2.0 ** -24
        if G > 2:
            s[:, 2] = 1023 * 2.0 ** -24
    scale = s.astype(np.float16).view(np.uint16)
    return QWeight(N, K, bits, words, scale, z.view(np.uint16))


def outlier_channels(K: int, rng) -> np.ndarray:
    n = int(round(OUTLIER_FRAC * K))
    return np.sort(rng.choice(K, size=n, replace=False))


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Store float32 values as bf16 bit patterns (round to nearest even)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def activations(M: int, K: int, rng, dtype: str = "bf16", outliers=None):
    """x ~ N(0, 1) [M][K], outlier channels x20; bf16 bits or float32."""
    x = rng.normal(0.0, 1.0, size=(M, K))
    if outliers is not None and len(outliers):
        x[:, outliers] *= OUTLIER_GAIN
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


def dense_weight(N: int, K: int, rng, std: float, outliers=None) -> np.ndarray:
    """W ~ N(0, std^2) [N][K] (float64), outlier input columns x20."""
    W = rng.normal(0.0, std, size=(N, K))
    if outliers is not None and len(outliers):
        W[:, outliers] *= OUTLIER_GAIN
    return W


@dataclass
class LayerInputs:
    lin: Linear
    bits: int
    M: int
    x: np.ndarray
    x_dtype: str
    V: Rotation
    U: Rotation
    W: QWeight


def layer_inputs(cfg: Config, lin_idx: int, bits: int, M: int,
                 inst: int = 0, angles: str = "f32") -> LayerInputs:
    """All boundary buffers for one linear of a config, fully seeded.

    angles: "f32" for float32 (cos, sin) pairs, "int8" for int8-stored angles.
    """
    lin = cfg.linears[lin_idx]
    out = outlier_channels(lin.K, rng_for(cfg.cid, T_OUTLIER, lin_idx, inst)) \
        if cfg.outliers else None
    x = activations(M, lin.K, rng_for(cfg.cid, T_X, lin_idx, inst * 1000 + M),
                    cfg.x_dtype, out)
    draw = {"f32": rotation, "int8": rotation_q8}[angles]
    V = draw(lin.K, lin.b_v, rng_for(cfg.cid, T_THETA_V, lin_idx, inst))
    U = draw(lin.N, lin.b_u, rng_for(cfg.cid, T_THETA_U, lin_idx, inst))
    W = qweight(lin.N, lin.K, bits,
                rng_for(cfg.cid, T_W, lin_idx, inst * 16 + bits), cfg.w_std)
    return LayerInputs(lin, bits, M, x, cfg.x_dtype, V, U, W)

"""Seeded synthetic inputs for the SVDQuant linear layer.

This module only draws random numbers and shapes. It holds none of the
method's arithmetic (no smoothing, SVD, quantization or matmul), so both the
CPU oracle and the HIP path can take their inputs from it without sharing
any of the computation.

Every tensor comes from ``numpy.random.default_rng([config, layer, tensor])``
so each one can be regenerated on its own, on any machine.

Distributions (the workloads are DiT- and UNet-shaped linear layers; the
pages describe SVDQuant on DiT and UNet diffusion models such as FLUX.1,
PixArt-Sigma and SDXL: the SVDQuant paper abstract as given on ai-digest.ru,
and the chattools.cn overview, section "SVDQuant的主要功能" (main features),
item on supported architectures):

* activations X ~ N(0, 1), with ``max(1, rint(frac*K))`` input channels,
  drawn without replacement, multiplied by an outlier factor (x20 at 1%);
* weights W ~ N(0, 0.02^2) in fp32, with the same count of input rows
  (drawn independently of X's channels) multiplied by x10;
* pre-activations for a down-projection: N(0, 1) with 0.5% channels x15,
  passed through GELU-tanh (``post_gelu_activation``);
* LoRA factors A (K x rl) and B (rl x N) ~ N(0, 0.01^2), stored as fp16.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

# tensor ids inside one (config, layer) stream
T_X, T_W, T_BIAS, T_LORA_A, T_LORA_B, T_PREACT = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer Y = X @ W (+ b): X is M x K, W is K x N."""
    M: int
    K: int
    N: int
    rank: int
    x_dtype: str = "f16"          # "f16" or "f32"
    y_dtype: str = "f16"
    x_outlier_frac: float = 0.01
    x_outlier_scale: float = 20.0
    w_outlier_frac: float = 0.01
    w_outlier_scale: float = 10.0
    lora_rank: int = 0            # extra rank concatenated onto the SVD factors
    preact: bool = False          # X = post_gelu_activation(...): GELU_tanh of ``preactivation``


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    layers: List[Layer]
    note: str


def _cfgs() -> List[Config]:
    c0 = Config(0, "tiny", [Layer(256, 512, 512, 16, "f32", "f32")],
                "X fp32 256x512, W 512x512, r=16, bias 0 (plus a seeded-bias variant)")
    c1 = Config(1, "dit_qkv", [Layer(4608, 3072, 9216, 32)],
                "DiT fused QKV projection: 4096 image + 512 text tokens, K=3072, N=9216, r=32")
    c2 = Config(2, "dit_mlp", [
        Layer(4608, 3072, 12288, 32),
        Layer(4608, 12288, 3072, 32, x_outlier_frac=0.005, x_outlier_scale=15.0, preact=True),
    ], "DiT MLP: up 3072->12288, GELU-tanh in fp16, down 12288->3072, r=32 on both")
    # UNet-style mixed shapes; "batch 2" doubles the listed token count.
    unet = [(16384, 320, 320), (4096, 640, 640), (4096, 640, 5120),
            (1024, 1280, 1280), (1024, 1280, 10240)]
    c3 = Config(3, "unet_mixed", [Layer(2 * m, k, n, 32) for (m, k, n) in unet],
                "UNet-style linears, batch 2, r=32")
    c4 = Config(4, "dit_lora_stack", [Layer(9216, 3072, 3072, 32, lora_rank=64) for _ in range(19)],
                "19 sequential DiT linears K=N=3072, M=2x4608, SVD rank 32 + LoRA rank 64 -> r=96")
    return [c0, c1, c2, c3, c4]


CONFIGS: List[Config] = _cfgs()


def _rng(cfg: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([int(cfg), int(layer), int(tensor)])


def outlier_count(n: int, frac: float) -> int:
    return max(1, int(np.rint(frac * n)))


def activation(cfg: int, layer: int, M: int, K: int, dtype: str = "f16",
               frac: float = 0.01, scale: float = 20.0, rows: slice | None = None) -> np.ndarray:
    """X (M x K): N(0,1) with ``outlier_count(K, frac)`` channels times ``scale``.

    ``rows`` returns a slice of the same matrix (the full matrix is drawn,
    so a slice equals the corresponding rows of the whole)."""
    g = _rng(cfg, layer, T_X)
    x = g.standard_normal((M, K))
    idx = g.choice(K, outlier_count(K, frac), replace=False)
    x[:, idx] *= scale
    if rows is not None:
        x = x[rows]
    return x.astype(np.float16 if dtype == "f16" else np.float32)


def preactivation(cfg: int, layer: int, M: int, K: int, frac: float = 0.005,
                  scale: float = 15.0) -> np.ndarray:
    """Z (M x K) fp16: N(0,1) pre-activations with a few channels times ``scale``."""
    g = _rng(cfg, layer, T_PREACT)
    z = g.standard_normal((M, K))
    idx = g.choice(K, outlier_count(K, frac), replace=False)
    z[:, idx] *= scale
    return z.astype(np.float16)


def post_gelu_activation(cfg: int, layer: int, M: int, K: int, frac: float = 0.005,
                         scale: float = 15.0) -> np.ndarray:
    """X (M x K) fp16 for the down-projection of an MLP: the seeded pre-activations
    of ``preactivation`` through the tanh form of GELU, evaluated in fp64 and
    rounded once to fp16. This is only the input distribution (a heavy positive
    tail from the outlier channels, negatives bounded near -0.17); the GELU the
    layers run between them is the library's."""
    z = preactivation(cfg, layer, M, K, frac, scale).astype(np.float64)
    u = np.sqrt(2.0 / np.pi) * (z + 0.044715 * z * z * z)
    return (0.5 * z * (1.0 + np.tanh(u))).astype(np.float16)


def weight(cfg: int, layer: int, K: int, N: int, frac: float = 0.01,
           scale: float = 10.0) -> np.ndarray:
    """W (K x N) fp32: N(0, 0.02^2) with ``outlier_count(K, frac)`` input rows times ``scale``."""
    g = _rng(cfg, layer, T_W)
    w = g.standard_normal((K, N)) * 0.02
    idx = g.choice(K, outlier_count(K, frac), replace=False)
    w[idx, :] *= scale
    return w.astype(np.float32)


def bias(cfg: int, layer: int, N: int, std: float = 0.1) -> np.ndarray:
    return (_rng(cfg, layer, T_BIAS).standard_normal(N) * std).astype(np.float32)


def lora(cfg: int, layer: int, K: int, N: int, rl: int = 64, std: float = 0.01):
    """(A, B): A is K x rl, B is rl x N, both N(0, std^2) rounded to fp16."""
    a = (_rng(cfg, layer, T_LORA_A).standard_normal((K, rl)) * std).astype(np.float16)
    b = (_rng(cfg, layer, T_LORA_B).standard_normal((rl, N)) * std).astype(np.float16)
    return a, b


def layer_inputs(cfg: int, layer_idx: int = 0):
    """Convenience: (Layer, X, W) for one layer of a config. For a layer whose
    input is a GELU output, X is ``post_gelu_activation``."""
    L = CONFIGS[cfg].layers[layer_idx]
    W = weight(cfg, layer_idx, L.K, L.N, L.w_outlier_frac, L.w_outlier_scale)
    if L.preact:
        return L, post_gelu_activation(cfg, layer_idx, L.M, L.K, L.x_outlier_frac,
                                       L.x_outlier_scale), W
    X = activation(cfg, layer_idx, L.M, L.K, L.x_dtype, L.x_outlier_frac, L.x_outlier_scale)
    return L, X, W


# --------------------------------------------------------------------------
# UNet convolutions (NHWC), run as implicit GEMMs: M = batch * OH * OW output
# pixels, K = KH * KW * C, N = output channels. Shapes are those of an SDXL-
# style UNet at 128x128 latents, batch 2 (3x3 convolutions at each level, a
# stride-2 downsample); the pages say SVDQuant applies to UNet backbones
# (chattools.cn overview, main features; disruptive-concepts.com post).

@dataclasses.dataclass(frozen=True)
class ConvLayer:
    batch: int
    H: int
    W: int
    C: int
    N: int
    KH: int
    KW: int
    stride: int
    pad: int
    rank: int
    x_dtype: str = "f16"
    y_dtype: str = "f16"
    name: str = ""

    @property
    def OH(self) -> int:
        return (self.H + 2 * self.pad - self.KH) // self.stride + 1

    @property
    def OW(self) -> int:
        return (self.W + 2 * self.pad - self.KW) // self.stride + 1

    @property
    def M(self) -> int:
        return self.batch * self.OH * self.OW

    @property
    def K(self) -> int:
        return self.KH * self.KW * self.C


CONV_LAYERS: List[ConvLayer] = [
    ConvLayer(1, 8, 8, 64, 64, 3, 3, 1, 1, 16, "f32", "f32", "tiny 3x3"),
    ConvLayer(2, 128, 128, 320, 320, 3, 3, 1, 1, 32, name="unet 128x128 3x3 320->320"),
    ConvLayer(2, 64, 64, 640, 640, 3, 3, 1, 1, 32, name="unet 64x64 3x3 640->640"),
    ConvLayer(2, 32, 32, 1280, 1280, 3, 3, 1, 1, 32, name="unet 32x32 3x3 1280->1280"),
    ConvLayer(2, 128, 128, 320, 320, 3, 3, 2, 1, 32, name="unet downsample 128->64 3x3 s2"),
]
CONV_CFG = 10          # seed stream of the convolution layers


def conv_inputs(idx: int):
    """(ConvLayer, X NHWC (batch x H x W x C), Wc (KH x KW x C x N) fp32), seeded like the
    linear layers: X N(0,1) with 1% of channels x20, Wc N(0, 0.02^2) with 1% of its
    KH*KW*C input rows x10."""
    L = CONV_LAYERS[idx]
    X = activation(CONV_CFG, idx, L.batch * L.H * L.W, L.C, L.x_dtype)
    Wc = weight(CONV_CFG, idx, L.K, L.N)
    return L, X.reshape(L.batch, L.H, L.W, L.C), Wc.reshape(L.KH, L.KW, L.C, L.N)

"""Seeded synthetic inputs for the routed-expert MoE feed-forward layer.

This module is shared by the HIP path's tests and bench and by the CPU oracle's
tests. It holds shapes, value distributions and sequence layouts only: none of
the layer's arithmetic lives here.

Where the shapes come from:

* HunyuanImage 3.0 Technical Report, section 3.1.1 "Architecture": 64 routed
  experts, 8 active per token, plus one shared MLP.
* HunyuanImage-3.0 model-coverage page, "Cache Contract": the latent is
  [32, height/16, width/16], so a 1024x1024 image is a 64x64 grid of image
  tokens, and a sample is prefix + <img> * (h*w) + suffix, right-padded
  in a batch.
* nemo_automodel ...hunyuan_image3.layers, init_leaf_weights: linear weights
  are drawn normal with std 0.02, stored [out, in].

Every value is generated from one integer seed through numpy's
SeedSequence / PCG64, in fixed-size chunks with their own child streams, so
the result does not depend on how many threads generate it.

bf16 tensors are returned as numpy uint16 arrays holding the bf16 bit
pattern (fp32 rounded to nearest, ties to even); fp32 tensors as float32.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}

BF16_NAN = np.uint16(0x7FC0)

# Number of rows per generator chunk for activations, and of elements per
# chunk for weights: fixed so results are independent of the thread count.
_X_ROWS_PER_CHUNK = 256
_W_ELEMS_PER_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Sizes of one MoE feed-forward layer."""

    H: int          # hidden size
    E: int          # routed experts
    K: int          # experts selected per token
    I: int          # routed expert intermediate size
    Is: int         # shared expert intermediate size
    dtype: int      # F32 or BF16: activations, expert weights and output


@dataclasses.dataclass(frozen=True)
class Workload:
    """A token batch: which rows are real and which are right padding."""

    name: str
    shape: LayerShape
    seq_lens: tuple          # real tokens per sequence
    padded_len: int          # rows per sequence after right padding
    skew: bool = False       # skewed router weights (load-imbalance stress)
    description: str = ""

    @property
    def T(self) -> int:
        return self.padded_len * len(self.seq_lens)

    @property
    def T_valid(self) -> int:
        return int(sum(self.seq_lens))

    def pad_mask(self) -> np.ndarray:
        """uint8 [T]; 1 at padding rows (the pages' padding_mask polarity)."""
        m = np.ones((len(self.seq_lens), self.padded_len), np.uint8)
        for b, n in enumerate(self.seq_lens):
            m[b, :n] = 0
        return m.reshape(-1)


FULL = LayerShape(H=4096, E=64, K=8, I=3072, Is=3072, dtype=BF16)
TINY = LayerShape(H=256, E=8, K=2, I=128, Is=128, dtype=F32)


def _image_seq(prompt: int, h: int, w: int, specials: int) -> int:
    return prompt + h * w + specials


def _padded_mixed_lens(seed: int):
    """Four right-padded sequences with mixed image grids; prompt lengths are
    drawn uniformly from 64..200 from the seed's 'lengths' stream."""
    grids = [(48, 80), (64, 64), (80, 48), (32, 128)]
    rng = np.random.Generator(np.random.PCG64(_streams(seed)["lengths"]))
    prompts = rng.integers(64, 201, size=len(grids))
    lens = tuple(int(p) + h * w for p, (h, w) in zip(prompts, grids))
    return lens, max(lens)


def workload(name: str, seed: int = 0) -> Workload:
    """The named workloads. 'padded_mixed' depends on the seed (its prompt
    lengths are drawn from it); the others do not."""
    if name == "tiny_f32":
        return Workload(name, TINY, (64,), 64,
                        description="T=64, H=256, E=8, K=2, I=Is=128, fp32")
    if name == "image_1024":
        # 32 prompt + 1 timestep + 64*64 image + 2 suffix tokens.
        n = 32 + 1 + 64 * 64 + 2
        return Workload(name, FULL, (n,), n,
                        description="one 1024x1024 image sequence, T=4131")
    if name == "batch8_512":
        n = _image_seq(96, 32, 32, 3)
        return Workload(name, FULL, (n,) * 8, n,
                        description="8 sequences at 512x512, T=8*1123=8984")
    if name == "skew_16k":
        return Workload(name, FULL, (16384,), 16384, skew=True,
                        description="T=16384 with skewed router weights")
    if name == "padded_mixed":
        lens, L = _padded_mixed_lens(seed)
        return Workload(name, FULL, lens, L,
                        description="4 right-padded sequences, grids 48x80, "
                                    "64x64, 80x48, 32x128, prompts 64..200")
    if name == "image_512":
        # one 512x512 image: 32 prompt + 1 timestep + 32*32 image + 2 suffix
        # tokens; about 132 rows per expert, below the weight-bandwidth ridge
        n = 32 + 1 + 32 * 32 + 2
        return Workload(name, FULL, (n,), n,
                        description="one 512x512 image sequence, T=1059")
    if name == "prompt_512":
        # a text-only sequence of 512 tokens (the causal text path), about 64
        # rows per expert: the layer streams its weights
        return Workload(name, FULL, (512,), 512,
                        description="one 512-token text sequence, T=512")
    raise KeyError(name)


WORKLOADS = ("tiny_f32", "image_1024", "batch8_512", "skew_16k", "padded_mixed",
             "image_512", "prompt_512")


def custom(shape: LayerShape, seq_lens, padded_len=None, skew=False,
           name="custom") -> Workload:
    seq_lens = tuple(int(n) for n in seq_lens)
    if padded_len is None:
        padded_len = max(seq_lens) if seq_lens else 0
    return Workload(name, shape, seq_lens, int(padded_len), skew=skew)


# ---------------------------------------------------------------- helpers

def _streams(seed: int) -> dict:
    names = ("x", "w_router", "w13", "w2", "ws13", "ws2", "lengths", "spare", "dout")
    kids = np.random.SeedSequence(int(seed)).spawn(len(names))
    return dict(zip(names, kids))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite
    inputs; NaN stays NaN)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _normal_fill(ss: np.random.SeedSequence, n: int, scale: float,
                 chunk: int, out_dtype: int) -> np.ndarray:
    """n values of scale*N(0,1), generated in `chunk`-sized pieces each with
    its own child stream; returned as float32 or bf16 bits."""
    nchunks = max(1, -(-n // chunk))
    kids = ss.spawn(nchunks)
    out = np.empty(n, np.uint16 if out_dtype == BF16 else np.float32)

    def job(i):
        lo = i * chunk
        hi = min(n, lo + chunk)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        out[lo:hi] = f32_to_bf16_bits(v) if out_dtype == BF16 else v

    if nchunks == 1:
        job(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, range(nchunks)))
    return out


def make_router_weight(shape: LayerShape, seed: int = 0, skew: bool = False) -> np.ndarray:
    """Router weight [E,H] fp32, N(0, 0.02^2).

    skew=True applies the load-imbalance construction: +0.5 on every
    element of rows 0..3 (those experts then win for roughly half of all
    tokens), and the last four rows scaled by 0.1, 0.1, 0.3, 0.3 so those
    experts receive almost no tokens."""
    s = _streams(seed)
    H, E = shape.H, shape.E
    wr = _normal_fill(s["w_router"], E * H, 0.02, _W_ELEMS_PER_CHUNK, F32).reshape(E, H)
    if skew:
        if E < 8:
            raise ValueError("skewed router needs E >= 8")
        wr[0:4] += np.float32(0.5)
        wr[E - 4:E - 2] *= np.float32(0.1)
        wr[E - 2:E] *= np.float32(0.3)
    return wr


def make_expert_weights(shape: LayerShape, seed: int = 0) -> dict:
    """Fused expert projections W13 [E,2I,H] (rows [0,I) up, [I,2I) gate);
    down projections W2 [E,H,I]; shared expert Ws13 [2Is,H] and Ws2 [H,Is].
    All N(0, 0.02^2), in the layer dtype."""
    s = _streams(seed)
    H, E, I, Is = shape.H, shape.E, shape.I, shape.Is
    dt = shape.dtype
    w13 = _normal_fill(s["w13"], E * 2 * I * H, 0.02, _W_ELEMS_PER_CHUNK, dt)
    w2 = _normal_fill(s["w2"], E * H * I, 0.02, _W_ELEMS_PER_CHUNK, dt)
    ws13 = _normal_fill(s["ws13"], 2 * Is * H, 0.02, _W_ELEMS_PER_CHUNK, dt)
    ws2 = _normal_fill(s["ws2"], H * Is, 0.02, _W_ELEMS_PER_CHUNK, dt)
    return {
        "w13": w13.reshape(E, 2 * I, H),
        "w2": w2.reshape(E, H, I),
        "ws13": ws13.reshape(2 * Is, H),
        "ws2": ws2.reshape(H, Is),
    }


def make_weights(shape: LayerShape, seed: int = 0, skew: bool = False) -> dict:
    """Router weight plus all expert weights (see the two functions above)."""
    d = make_expert_weights(shape, seed)
    d["w_router"] = make_router_weight(shape, seed, skew)
    return d


def make_norm_weight(shape: LayerShape, seed: int = 0) -> np.ndarray:
    """Weight [H] of the block's RMSNorm in front of the layer: 1 + 0.1 N(0,1)
    in the layer dtype (the module initialises it to ones; the spread makes
    the multiply by the weight visible)."""
    s = _streams(seed)
    v = _normal_fill(s["spare"], shape.H, 0.1, shape.H, F32) + np.float32(1.0)
    return f32_to_bf16_bits(v) if shape.dtype == BF16 else v


def make_x(wl: Workload, seed: int = 0) -> tuple:
    """Activations [T,H] ~ N(0,1) (the layer's input after RMSNorm), with
    padding rows set to NaN so that any read of them shows; and the uint8
    padding mask [T] (1 = padding)."""
    s = _streams(seed)
    H = wl.shape.H
    T = wl.T
    x = _normal_fill(s["x"], T * H, 1.0, _X_ROWS_PER_CHUNK * H,
                     wl.shape.dtype).reshape(T, H)
    pad = wl.pad_mask()
    if pad.any():
        x[pad.astype(bool)] = BF16_NAN if wl.shape.dtype == BF16 else np.nan
    return x, pad


def make_dout(wl: Workload, seed: int = 0) -> np.ndarray:
    """Output gradient [T,H] ~ N(0,1) in the layer dtype (the backward's
    input), padding rows NaN like x's."""
    s = _streams(seed)
    H, T = wl.shape.H, wl.T
    g = _normal_fill(s["dout"], T * H, 1.0, _X_ROWS_PER_CHUNK * H, wl.shape.dtype).reshape(T, H)
    pad = wl.pad_mask()
    if pad.any():
        g[pad.astype(bool)] = BF16_NAN if wl.shape.dtype == BF16 else np.nan
    return g


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    d = make_weights(wl.shape, seed, skew=wl.skew)
    x, pad = make_x(wl, seed)
    d["x"] = x
    d["pad_mask"] = pad
    return d


def flop_per_valid_token(shape: LayerShape) -> int:
    """Algorithmic FLOP per real token: K routed SwiGLU experts (three
    projections of H x I each), the shared expert, and the router."""
    return (shape.K * 6 * shape.H * shape.I + 6 * shape.H * shape.Is
            + 2 * shape.H * shape.E)

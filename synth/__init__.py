"""Seeded synthetic inputs for segment-causal attention over a lifelong INT8 KV cache.

This module only draws random numbers and lays them out in the shapes of the
Hy-Nomas workloads.  It holds none of the method's arithmetic (no RoPE, no
quantisation, no attention, no camera normalisation): both the CPU oracle and
the GPU library consume exactly the bytes produced here.

Sources for the shapes (Hy-Nomas pages):
  * comfyui-wiki news page, "模型内部" table: 16 heads x 128, hidden 2048,
    latent patch 1x1x1; DCAE-V f32t4c32 latent (32x spatial, 4x temporal), so
    one 1280x704 latent frame is 40 x 22 = 880 tokens.
  * same page, "相机控制": c2w trajectory [N,4,4], grouped per 4 video frames
    into a 64-d camera token.
  * huaweicloud blog, section 3.5 table: an 18-latent-frame GPU history window.

Random streams.  Every tensor is drawn as float32 from numpy's PCG64, seeded by
``SeedSequence(20261021 + config, spawn_key=(instance, stream, chunk))`` where
``instance`` is the layer (seg4s) or the turn (fiveturns), 0 otherwise, and
``stream`` indexes STREAMS.  Tensors are drawn in chunks of 2**22 values so the
draw can run on several threads and still be identical byte for byte.
BF16 tensors are then rounded to bfloat16 with round-to-nearest-even and kept
as raw uint16 bit patterns.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

STREAMS = ("q", "k_new", "v_new", "k_hist", "v_hist", "outlier_idx",
           "cam_path", "w_k", "w_v", "q_cam", "d_out")
BASE_SEED = 20261021
CHUNK = 1 << 22
D = 128

# 1280x704 frame, 32x spatial compression -> 40 columns x 22 rows of tokens.
HG, WG = 22, 40


@dataclass(frozen=True)
class Seg:
    """One segment: ``n_text`` text tokens, then ``T*Hg*Wg`` video tokens in
    (t, h, w) row-major order with t running over [t0, t0+T)."""
    n_text: int
    t0: int
    T: int
    Hg: int
    Wg: int

    @property
    def ntok(self) -> int:
        return self.n_text + self.T * self.Hg * self.Wg

    def astuple(self):
        return (self.n_text, self.t0, self.T, self.Hg, self.Wg)


def seg_tokens(segs) -> int:
    return sum(s.ntok for s in segs)


@dataclass
class Config:
    """A workload: the current segment(s), the history that forms the INT8
    cache, head count and extras."""
    cid: int
    name: str
    H: int
    new_segs: tuple
    hist_segs: tuple          # positions of the cached history (RoPE before caching)
    outliers: int = 0         # number of hidden channels scaled x20
    outlier_gain: float = 20.0
    layers: int = 1
    steps: int = 1
    turns: int = 1
    cam_frames: int = 0       # video frames in the camera path per turn
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def Lq(self) -> int:
        return seg_tokens(self.new_segs)

    @property
    def Lc(self) -> int:
        return seg_tokens(self.hist_segs)


TINY_SEGS = (Seg(16, 0, 2, 4, 6), Seg(16, 2, 2, 4, 6), Seg(16, 4, 2, 4, 6))

# The workloads by name; cid seeds their random streams.
WORKLOADS = {
    "tiny": Config(1, "tiny", 2, new_segs=(TINY_SEGS[1],), hist_segs=(TINY_SEGS[0],),
              notes="2 segments of 16 text + 2x4x6 video tokens; packed and "
                    "3-segment variants drawn from the same streams"),
    "turn3s": Config(2, "turn3s", 16, new_segs=(Seg(256, 18, 18, HG, WG),),
              hist_segs=(Seg(0, 0, 18, HG, WG),),
              notes="3 s turn: 18 latent frames + 256 text vs 18-frame INT8 history"),
    "seg4s": Config(3, "seg4s", 16, new_segs=(Seg(256, 18, 24, HG, WG),),
              hist_segs=(Seg(0, 0, 18, HG, WG),), outliers=20, layers=54, steps=8,
              notes="4 s segment, 1% of the 2048 hidden channels x20 in Q/K, 54 layers x 8 steps"),
    "fullcache": Config(4, "fullcache", 16, new_segs=(Seg(0, 288, 72, HG, WG),),
              hist_segs=(Seg(0, 0, 288, HG, WG),),
              notes="12 s segment vs 288 cached latent frames (~317K keys)"),
    "fiveturns": Config(5, "fiveturns", 16, new_segs=(Seg(0, 0, 72, HG, WG),), hist_segs=(),
              turns=5, cam_frames=288,
              notes="5 turns of 72 latent frames; cache grows by 63,360 tokens a turn"),
}


def turn_seg(k: int) -> Seg:
    """The k-th 12 s turn of the five-turn workload (72 latent frames)."""
    return Seg(0, 72 * k, 72, HG, WG)


# ----------------------------------------------------------------------------
# raw draws


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _seed(cid: int, inst: int, stream: str, chunk: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(BASE_SEED + cid, spawn_key=(inst, STREAMS.index(stream), chunk))


def normal_f32(cid: int, inst: int, stream: str, n: int, scale: float = 1.0) -> np.ndarray:
    """n float32 draws of N(0, scale^2), chunked and threaded, deterministic."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(_seed(cid, inst, stream, i)))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if scale != 1.0:
            out[lo:hi] *= np.float32(scale)

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(b.shape, dtype=np.uint16)
    n = b.size
    flat_b, flat_o = b.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for lo in range(0, n, step):
        bb = flat_b[lo:lo + step]
        flat_o[lo:lo + step] = ((bb + np.uint32(0x7FFF) + ((bb >> np.uint32(16)) & np.uint32(1)))
                                >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_tensor(cid, inst, stream, shape, scale=1.0, outlier_cols=None, gain=20.0):
    """A bf16 tensor (uint16 bits) of N(0, scale^2) draws; optional columns of
    the flattened [.., H*128] hidden dimension are multiplied by ``gain`` in
    float32 before rounding (the outlier channels of the 4 s workload)."""
    n = int(np.prod(shape))
    x = normal_f32(cid, inst, stream, n, scale).reshape(shape)
    if outlier_cols is not None and len(outlier_cols):
        hidden = x.reshape(shape[0], -1)
        hidden[:, outlier_cols] *= np.float32(gain)
    return to_bf16_bits(x)


def outlier_columns(cfg: Config, inst: int) -> np.ndarray:
    """``cfg.outliers`` distinct hidden channels out of H*128, sorted."""
    if not cfg.outliers:
        return np.zeros(0, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(_seed(cfg.cid, inst, "outlier_idx", 0)))
    return np.sort(g.choice(cfg.H * D, size=cfg.outliers, replace=False)).astype(np.int64)


# ----------------------------------------------------------------------------
# camera path: a random rigid-motion (SE(3)) trajectory of c2w matrices


def _axis_angle_matrix(axis, angle):
    axis = axis / np.linalg.norm(axis)
    x, y, z = axis
    K = np.array([[0, -z, y], [z, 0, -x], [-y, x, 0]], dtype=np.float64)
    return np.eye(3) + math.sin(angle) * K + (1 - math.cos(angle)) * (K @ K)


def camera_path(cid: int, inst: int, n_frames: int) -> np.ndarray:
    """[n_frames, 4, 4] float64 camera-to-world matrices: a random start pose
    followed by small random per-frame rotations and translations."""
    g = np.random.Generator(np.random.PCG64(_seed(cid, inst, "cam_path", 0)))
    c2w = np.zeros((n_frames, 4, 4), dtype=np.float64)
    R = _axis_angle_matrix(g.standard_normal(3), g.uniform(0, math.pi))
    t = g.standard_normal(3) * 2.0
    vel = g.standard_normal(3) * 0.05
    for i in range(n_frames):
        c2w[i, :3, :3] = R
        c2w[i, :3, 3] = t
        c2w[i, 3, 3] = 1.0
        dR = _axis_angle_matrix(g.standard_normal(3), abs(g.normal(0.0, 0.01)))
        R = R @ dR
        vel = 0.9 * vel + g.standard_normal(3) * 0.01
        t = t + vel
    return c2w


# ----------------------------------------------------------------------------
# whole workloads


def tiny_inputs():
    """Tiny: three segments of 64 tokens (16 text + 2x4x6 video), 2 heads.
    q/k/v are drawn for all 192 tokens; cache mode uses segment 0's k/v as the
    history and segment 1 as the new segment, the packed mode takes segments
    0 and 1 as new tokens, the 3-segment mode caches segment 0 and takes 1, 2."""
    cfg = WORKLOADS["tiny"]
    L = seg_tokens(TINY_SEGS)
    shp = (L, cfg.H, D)
    return dict(cfg=cfg, segs=TINY_SEGS,
                q=bf16_tensor(1, 0, "q", shp),
                k=bf16_tensor(1, 0, "k_new", shp),
                v=bf16_tensor(1, 0, "v_new", shp))


def layer_inputs(name: str, inst: int = 0, with_hist: bool = True):
    """q, k_new, v_new [Lq][H][128] and k_hist, v_hist [Lc][H][128] (pre-RoPE
    history keys) as bf16 bits for the turn3s, seg4s (one layer) and
    fullcache workloads."""
    cfg = WORKLOADS[name]
    cid = cfg.cid
    cols = outlier_columns(cfg, inst)
    shp = (cfg.Lq, cfg.H, D)
    out = dict(cfg=cfg, outlier_cols=cols,
               q=bf16_tensor(cid, inst, "q", shp, outlier_cols=cols, gain=cfg.outlier_gain),
               k_new=bf16_tensor(cid, inst, "k_new", shp, outlier_cols=cols, gain=cfg.outlier_gain),
               v_new=bf16_tensor(cid, inst, "v_new", shp))
    if with_hist and cfg.Lc:
        hshp = (cfg.Lc, cfg.H, D)
        out["k_hist"] = bf16_tensor(cid, inst, "k_hist", hshp, outlier_cols=cols, gain=cfg.outlier_gain)
        out["v_hist"] = bf16_tensor(cid, inst, "v_hist", hshp)
    return out


def turn_inputs(k: int, with_cam: bool = True):
    """Turn k of the five-turn workload: new-segment q/k/v, camera queries for
    the video tokens, a 288-frame c2w path and the camera K/V projections."""
    cfg = WORKLOADS["fiveturns"]
    seg = turn_seg(k)
    shp = (seg.ntok, cfg.H, D)
    out = dict(cfg=cfg, seg=seg,
               q=bf16_tensor(5, k, "q", shp),
               k_new=bf16_tensor(5, k, "k_new", shp),
               v_new=bf16_tensor(5, k, "v_new", shp))
    if with_cam:
        out["q_cam"] = bf16_tensor(5, k, "q_cam", shp)
        out["c2w"] = camera_path(5, k, cfg.cam_frames)
        # projection weights are per model, so they do not change with the turn
        out["w_k"] = bf16_tensor(5, 0, "w_k", (64, cfg.H * D), scale=1.0 / 8.0)
        out["w_v"] = bf16_tensor(5, 0, "w_v", (64, cfg.H * D), scale=1.0 / 8.0)
    return out


# Segment-forcing training (huaweicloud blog, section 2.3): sequences packed
# up to 360,000 tokens.  Reading: one packed sequence is one long video cut
# into 3 s turns (18 latent frames of 880 tokens plus 256 text tokens each,
# the turn3s segment shape); 22 turns, 354,112 tokens, fit the packing limit.
TRAIN_CID = 6
TRAIN_TURNS = 22


def train_segs(n: int = TRAIN_TURNS, n_text: int = 256, T: int = 18, Hg: int = HG, Wg: int = WG):
    """n consecutive turns of T latent frames each, t0 = T * turn."""
    return tuple(Seg(n_text, T * i, T, Hg, Wg) for i in range(n))


def train_inputs(segs, H: int, inst: int = 0):
    """q, k, v (pre-RoPE) and the output gradient d_out, [L][H][128] bf16
    bits, N(0, 1), for a packed training sequence of the given segments."""
    shp = (seg_tokens(segs), H, D)
    return dict(segs=tuple(segs), H=H,
                q=bf16_tensor(TRAIN_CID, inst, "q", shp),
                k=bf16_tensor(TRAIN_CID, inst, "k_new", shp),
                v=bf16_tensor(TRAIN_CID, inst, "v_new", shp),
                d_out=bf16_tensor(TRAIN_CID, inst, "d_out", shp))


def random_bf16(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Ad-hoc seeded N(0, scale^2) bf16 tensor (uint16 bits) for edge-case
    shapes that are not one of the named workloads."""
    n = int(np.prod(shape))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = g.standard_normal(n, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_bf16_bits(x).reshape(shape)


def random_int8_cache(seed: int, H: int, L: int):
    """Seeded INT8 cache contents for edge-case sizes: codes [H][L][128]
    uniform in [-127, 127] and one positive fp32 scale per (head, token),
    uniform in [2^-8, 2^-6) (values of the size N(0,1) rows quantise to).
    Any such codes and scales are a valid cache; drawing them directly
    avoids quantising millions of rows."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    codes = g.integers(-127, 128, size=(H, L, D), dtype=np.int8)
    scale = (np.float32(2.0 ** -8) * (1.0 + 3.0 * g.random((H, L), dtype=np.float32))).astype(np.float32)
    return codes, scale

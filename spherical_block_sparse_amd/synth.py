"""Seeded synthetic inputs for the BSA forward pass.

This module is the only code that both the HIP path (tests, bench) and the
float64 oracle consume: it makes the input bits and nothing else.  It holds
none of the attention arithmetic.

Workloads (the resolutions are the HEALPix ladder Nside in {32, 64, 128, 256}
of the papernotes.org ICML2026 notes, 关键设计 › HEALPix + NESTED; the pages'
own data, ERA5 / WeatherBench2, is not available, so these seeded fields stand
in for it):

  tiny   Nside=8:   b1  H2  d32, block 16, top-n 4,  W 32,   i.i.d. N(0,1), fp32
  ns32   Nside=32:  b1  H8  d64, block 64, top-n 16, W 256,  i.i.d. N(0,1), bf16
  ns64   Nside=64:  b4  H8  d64, block 64, top-n 16, W 256,  Fourier field, bf16
  ns128  Nside=128: b24 H8  d64, block 64, top-n 16, W 512,  Fourier field, bf16
  ns256  Nside=256: b2  H16 d64, block 256, top-n 8, W 1024, Fourier field, bf16

Gates are sigmoid(N(0,1)) per token, head and branch, fp32.

Fourier field (per tensor and batch element): 16 modes with wave vectors
omega = f * r_hat (f ~ U[0, 8], r_hat uniform on the sphere), phases
~ U[0, 2*pi) and amplitudes A ~ N(0, 1/8) per channel c = h*d + j;
X[t, c] = sum_modes A[c] cos(omega . u_t + phase) + 0.1 * N(0, 1), where u_t
is the NESTED pixel-centre unit vector of token t.  The channel variance is
16 * (1/8) * (1/2) + 0.01 ~= 1.

Seeding: the config's seed (its Nside) feeds numpy's SeedSequence, whose
four spawned children seed the q, k, v and gate streams in that order; each
stream drives one torch.Generator on the device the inputs are made on.
Bits made on the CPU and on a GPU differ; every comparison hands the same
bits to both sides.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class BSAConfig:
    name: str
    nside: int
    batch: int
    heads: int
    head_dim: int
    block: int
    topn: int
    window: int
    field: str          # "iid" or "fourier"
    seed: int

    @property
    def n_tokens(self) -> int:
        return 12 * self.nside * self.nside

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // self.block

    @property
    def slices(self) -> int:
        return self.batch * self.heads

    @property
    def tokens(self) -> int:
        """Tokens per forward call = batch * N (HEALPix pixels of all members)."""
        return self.batch * self.n_tokens

    def with_(self, **kw) -> "BSAConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": BSAConfig("tiny", 8, 1, 2, 32, 16, 4, 32, "iid", 8),
    "ns32": BSAConfig("ns32", 32, 1, 8, 64, 64, 16, 256, "iid", 32),
    "ns64": BSAConfig("ns64", 64, 4, 8, 64, 64, 16, 256, "fourier", 64),
    "ns128": BSAConfig("ns128", 128, 24, 8, 64, 64, 16, 512, "fourier", 128),
    "ns256": BSAConfig("ns256", 256, 2, 16, 64, 256, 8, 1024, "fourier", 256),
}


# --------------------------------------------------------------------------
# HEALPix NESTED pixel centres (textbook geometry: Gorski et al. 2005,
# ApJ 622:759).  Used only to shape the synthetic fields.
# --------------------------------------------------------------------------

_JRLL = np.array([2, 2, 2, 2, 3, 3, 3, 3, 4, 4, 4, 4], dtype=np.int64)
_JPLL = np.array([1, 3, 5, 7, 0, 2, 4, 6, 1, 3, 5, 7], dtype=np.int64)


def _compact_even_bits(v: np.ndarray) -> np.ndarray:
    """Gather bits 0, 2, 4, ... of v into a contiguous integer."""
    v = v & 0x5555555555555555
    v = (v | (v >> 1)) & 0x3333333333333333
    v = (v | (v >> 2)) & 0x0F0F0F0F0F0F0F0F
    v = (v | (v >> 4)) & 0x00FF00FF00FF00FF
    v = (v | (v >> 8)) & 0x0000FFFF0000FFFF
    v = (v | (v >> 16)) & 0x00000000FFFFFFFF
    return v


def _nest_ring_coords(nside: int):
    """Ring number jr (1 .. 4*nside-1, north to south), pixel-in-ring jp
    (1-based, eastward), pixels in the ring nr/4 (nr) and the belt shift of
    every NESTED pixel."""
    if nside < 1 or nside & (nside - 1):
        raise ValueError("nside must be a power of two")
    npface = nside * nside
    p = np.arange(12 * npface, dtype=np.int64)
    face = p // npface
    ipf = p % npface
    ix = _compact_even_bits(ipf)
    iy = _compact_even_bits(ipf >> 1)
    jr = _JRLL[face] * nside - ix - iy - 1            # ring number, 1 .. 4*nside-1
    north = jr < nside
    south = jr > 3 * nside
    belt = ~(north | south)
    nr = np.where(north, jr, np.where(south, 4 * nside - jr, nside))
    kshift = np.where(belt, (jr - nside) & 1, 0)
    jp = (_JPLL[face] * nr + ix - iy + 1 + kshift) // 2
    jp = np.where(jp > 4 * nside, jp - 4 * nside, jp)
    jp = np.where(jp < 1, jp + 4 * nside, jp)
    return jr, jp, nr, kshift


def nest_ring_order(nside: int) -> np.ndarray:
    """NESTED indices of the pixels in RING order (iso-latitude rings north to
    south, each from azimuth 0 eastward): the layout of a latitude-longitude
    raster on the same mesh, used to compare block locality with NESTED."""
    jr, jp, _, _ = _nest_ring_coords(nside)
    return np.lexsort((jp, jr))


def pix2vec_nest(nside: int) -> np.ndarray:
    """Unit vectors of the centres of all 12*nside^2 NESTED pixels, [N, 3] f64.

    The in-face coordinates (ix, iy) are the even and odd bits of the index
    within the base face; ring number and azimuth follow from the face's
    position (polar caps above/below |z| = 2/3, equatorial belt between)."""
    jr, jp, nr, kshift = _nest_ring_coords(nside)
    npface = nside * nside
    north = jr < nside
    south = jr > 3 * nside
    cap_z = 1.0 - nr.astype(np.float64) ** 2 / (3.0 * npface)
    z = np.where(north, cap_z, np.where(south, -cap_z, (2 * nside - jr) * (2.0 / (3.0 * nside))))
    phi = (jp - (kshift + 1) * 0.5) * (np.pi / (2.0 * nr))
    sth = np.sqrt((1.0 - z) * (1.0 + z))
    return np.stack([sth * np.cos(phi), sth * np.sin(phi), z], axis=1)


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------

def _stream_seeds(seed: int) -> list[int]:
    children = np.random.SeedSequence(seed).spawn(4)
    return [int(c.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF) for c in children]


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _fourier_field(u: torch.Tensor, channels: int, gen: torch.Generator, modes: int = 16,
                   fmax: float = 8.0, noise: float = 0.1) -> torch.Tensor:
    """[N, channels] float32 field: sum of random cosine modes of the pixel
    centre vectors u [N, 3], plus white noise."""
    dev = u.device
    r_hat = torch.randn(modes, 3, generator=gen, device=dev, dtype=torch.float32)
    r_hat = r_hat / r_hat.norm(dim=1, keepdim=True)
    f = torch.rand(modes, 1, generator=gen, device=dev, dtype=torch.float32) * fmax
    phase = torch.rand(modes, generator=gen, device=dev, dtype=torch.float32) * (2.0 * math.pi)
    amp = torch.randn(modes, channels, generator=gen, device=dev, dtype=torch.float32) * math.sqrt(1.0 / 8.0)
    x = torch.cos(u @ (f * r_hat).T + phase) @ amp
    x += noise * torch.randn(x.shape, generator=gen, device=dev, dtype=torch.float32)
    return x


def make_inputs(cfg: BSAConfig, device="cpu", dtype=torch.bfloat16, seed: int | None = None):
    """Return (q, k, v, gates) for ``cfg`` on ``device``.

    q, k, v: [b, H, N, d] in ``dtype`` (bf16 rounding is torch's
    round-to-nearest-even); gates: [b, H, N, 3] float32 = sigmoid(N(0,1))."""
    seeds = _stream_seeds(cfg.seed if seed is None else seed)
    b, h, n, d = cfg.batch, cfg.heads, cfg.n_tokens, cfg.head_dim
    tensors = []
    u = None
    if cfg.field == "fourier":
        u = torch.from_numpy(pix2vec_nest(cfg.nside)).to(device=device, dtype=torch.float32)
    for s in seeds[:3]:
        gen = _generator(device, s)
        out = torch.empty((b, h, n, d), dtype=dtype, device=device)
        for bi in range(b):
            if cfg.field == "iid":
                x = torch.randn((h, n, d), generator=gen, device=device, dtype=torch.float32)
                out[bi].copy_(x)
            elif cfg.field == "fourier":
                x = _fourier_field(u, h * d, gen)                 # [N, H*d]
                out[bi].copy_(x.view(n, h, d).permute(1, 0, 2))
            else:
                raise ValueError(cfg.field)
            del x
        tensors.append(out)
    gen = _generator(device, seeds[3])
    gates = torch.sigmoid(torch.randn((b, h, n, 3), generator=gen, device=device, dtype=torch.float32))
    return tensors[0], tensors[1], tensors[2], gates


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact widening of a (bf16 / fp32) tensor to a float64 numpy array on the host."""
    return x.detach().to("cpu").to(torch.float64).numpy()


def make_layer_inputs(cfg: BSAConfig, channels: int, layers: int = 1, device="cpu", seed: int | None = None):
    """Return (x, w_in, w_out) for an encoder layer on ``cfg``'s mesh.

    x: [b, N, channels] bf16, the config's field ("iid": N(0,1); "fourier":
    the cosine-mode field above with ``channels`` channels) from the first
    stream of seed + 1000.  w_in: [layers, 3*H*d + 3*H, channels] and w_out:
    [layers, channels, H*d], bf16, i.i.d. N(0, 1/fan_in) from the second and
    third streams (fan_in = channels and H*d)."""
    seeds = _stream_seeds((cfg.seed if seed is None else seed) + 1000)
    b, n = cfg.batch, cfg.n_tokens
    hd = cfg.heads * cfg.head_dim
    e = 3 * hd + 3 * cfg.heads
    gen = _generator(device, seeds[0])
    x = torch.empty((b, n, channels), dtype=torch.bfloat16, device=device)
    u = None
    if cfg.field == "fourier":
        u = torch.from_numpy(pix2vec_nest(cfg.nside)).to(device=device, dtype=torch.float32)
    for bi in range(b):
        if cfg.field == "iid":
            x[bi].copy_(torch.randn((n, channels), generator=gen, device=device, dtype=torch.float32))
        elif cfg.field == "fourier":
            x[bi].copy_(_fourier_field(u, channels, gen))
        else:
            raise ValueError(cfg.field)
    gen = _generator(device, seeds[1])
    w_in = (torch.randn((layers, e, channels), generator=gen, device=device, dtype=torch.float32)
            / math.sqrt(channels)).to(torch.bfloat16)
    gen = _generator(device, seeds[2])
    w_out = (torch.randn((layers, channels, hd), generator=gen, device=device, dtype=torch.float32)
             / math.sqrt(hd)).to(torch.bfloat16)
    return x, w_in, w_out


# --------------------------------------------------------------------------
# lat-lon source grid and its stencil around HEALPix targets
# --------------------------------------------------------------------------

def latlon_vectors(n_lat: int, n_lon: int) -> np.ndarray:
    """Unit vectors of a regular latitude-longitude grid with both poles:
    row r at latitude 90 - 180*r/(n_lat-1) degrees, column c at longitude
    360*c/n_lon; [n_lat*n_lon, 3], row-major."""
    lat = np.radians(90.0 - 180.0 * np.arange(n_lat) / (n_lat - 1))
    lon = np.radians(360.0 * np.arange(n_lon) / n_lon)
    cl = np.cos(lat)[:, None]
    return np.stack([np.broadcast_to(cl * np.cos(lon)[None, :], (n_lat, n_lon)),
                     np.broadcast_to(cl * np.sin(lon)[None, :], (n_lat, n_lon)),
                     np.broadcast_to(np.sin(lat)[:, None], (n_lat, n_lon))], axis=-1).reshape(-1, 3)


def latlon_stencil(nside: int, n_lat: int, n_lon: int):
    """The source neighbourhood of every HEALPix NESTED pixel on a lat-lon
    grid: the 4 x 4 grid points around the pixel centre (rows r0-1 .. r0+2
    clamped at the poles, columns c0-1 .. c0+2 wrapped in longitude, with
    (r0, c0) the grid cell holding the centre), and each one's position
    relative to the centre, (u_j - u_i) / spacing with the grid spacing in
    radians.  Returns nbr [N, 16] int32 and rel [N, 16, 3] float32."""
    u = pix2vec_nest(nside)
    lat = np.degrees(np.arcsin(np.clip(u[:, 2], -1.0, 1.0)))
    lon = np.mod(np.degrees(np.arctan2(u[:, 1], u[:, 0])), 360.0)
    dlat, dlon = 180.0 / (n_lat - 1), 360.0 / n_lon
    r0 = np.minimum(np.floor((90.0 - lat) / dlat).astype(np.int64), n_lat - 2)
    c0 = np.floor(lon / dlon).astype(np.int64) % n_lon
    rows = np.clip(r0[:, None] + np.arange(-1, 3)[None, :], 0, n_lat - 1)        # [N, 4]
    cols = (c0[:, None] + np.arange(-1, 3)[None, :]) % n_lon                      # [N, 4]
    nbr = (rows[:, :, None] * n_lon + cols[:, None, :]).reshape(-1, 16)
    src = latlon_vectors(n_lat, n_lon)
    rel = (src[nbr] - u[:, None, :]) / np.radians(dlat)
    return nbr.astype(np.int32), rel.astype(np.float32)


def make_interp_inputs(nside: int, n_lat: int, n_lon: int, slices: int, d: int = 64, dv: int = 64,
                       device="cpu", seed: int = 0):
    """Source keys and values on the lat-lon grid (smooth cosine-mode fields
    of the grid points' unit vectors, bf16 [slices, n_src, d] and
    [slices, n_src, dv]), the relative-position query weights w_q [d, 3]
    (float32, N(0, 1)), and the stencil of ``latlon_stencil``."""
    seeds = _stream_seeds(seed + 2000)
    u = torch.from_numpy(latlon_vectors(n_lat, n_lon)).to(device=device, dtype=torch.float32)
    n_src = u.shape[0]
    out = []
    for s, ch in zip(seeds[:2], (d, dv)):
        gen = _generator(device, s)
        t = torch.empty((slices, n_src, ch), dtype=torch.bfloat16, device=device)
        for i in range(slices):
            t[i].copy_(_fourier_field(u, ch, gen))
        out.append(t)
    gen = _generator(device, seeds[2])
    w_q = torch.randn((d, 3), generator=gen, device=device, dtype=torch.float32)
    nbr, rel = latlon_stencil(nside, n_lat, n_lon)
    return out[0], out[1], w_q, torch.from_numpy(nbr).to(device), torch.from_numpy(rel).to(device)

"""Seeded synthetic inputs for paged decode attention.

Shared by the tests, the smoke check and the benchmark. It draws context lengths, physical
block placements and values, and nothing else: no attention, cache-write or allocator
arithmetic lives here.

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64, in this order: lengths,
placement, then values):

* values are N(0, 1) drawn in float32, then rounded to the cache dtype (round to nearest
  even); the rounded values are the inputs;
* placement: a seeded random permutation of the NB physical blocks is the pool's free order,
  and sequences take consecutive runs of it in sequence order (what a FIFO free list hands
  out when sequences are filled one after another);
* the pool holds ceil(1.1 * blocks needed) blocks unless a config fixes NB.

Large pools are filled on the GPU with a seeded ``torch.Generator`` instead of NumPy
(``device_normal``); the checks then copy back exactly the blocks they need.

The named shapes follow the workloads the method is usually run on:
  tiny            4 seqs, n = {1, 15, 16, 37}, 2 q / 2 kv heads, hd 64, f32, NB 16
  llama2_7b       64 seqs, n ~ U[128, 2048], MHA 32 x 128, f16
  qwen25_7b       256 seqs, n = clip(round(lognormal(ln 1024, 1)), 16, 32768), 28 q / 4 kv x 128, bf16
  prefix_shared   128 seqs sharing a 2000-token prefix (125 blocks) + private tails U[16, 512],
                  MHA 32 x 128, bf16 (and a beam variant: 32 groups x 4 beams)
  long_context    8 seqs at 32768 + 120 seqs U[64, 4096], 32 q / 8 kv x 128, bf16, one new
                  token per sequence written before attention
  prefill         chunked prefill of 16 seqs: a cached prefix of U[0, 1536] tokens plus a new
                  chunk of 512 tokens each (8192 query tokens), MHA 32 x 128, f16
"""

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    B: int
    Hq: int
    Hkv: int
    hd: int
    dtype: str  # "f32" | "f16" | "bf16"
    seed: int


SHAPES = {
    "tiny": Shape("tiny", 4, 2, 2, 64, "f32", 1),
    "llama2_7b": Shape("llama2_7b", 64, 32, 32, 128, "f16", 2),
    "qwen25_7b": Shape("qwen25_7b", 256, 28, 4, 128, "bf16", 3),
    "prefix_shared": Shape("prefix_shared", 128, 32, 32, 128, "bf16", 4),
    "long_context": Shape("long_context", 128, 32, 8, 128, "bf16", 5),
    "beam_search": Shape("beam_search", 128, 32, 32, 128, "bf16", 6),
    "prefill": Shape("prefill", 16, 32, 32, 128, "f16", 7),
}
PREFILL_CHUNK = 512  # new tokens per sequence in the prefill workload
PREFILL_CACHED = (0, 1536)  # cached-prefix tokens before the chunk, inclusive range

TINY_LENGTHS = (1, 15, 16, 37)
TINY_POOL = 16
PREFIX_TOKENS = 2000
BEAMS = 4  # beams per group in the beam-search workload


def rng_for(seed):
    return np.random.default_rng(seed)


def blocks_for(n, bs=BLOCK_SIZE):
    return -(-int(n) // bs)


def draw_lengths(shape, rng, *, B=None):
    """Context lengths (after the current token is written) for a named shape."""
    B = shape.B if B is None else B
    if shape.name == "tiny":
        return np.array(TINY_LENGTHS[:B], dtype=np.int32)
    if shape.name == "llama2_7b":
        return rng.integers(128, 2048, size=B, endpoint=True).astype(np.int32)
    if shape.name == "qwen25_7b":
        x = np.exp(rng.normal(math.log(1024.0), 1.0, size=B))
        return np.clip(np.rint(x), 16, 32768).astype(np.int32)
    if shape.name == "prefix_shared":
        return (PREFIX_TOKENS + rng.integers(16, 512, size=B, endpoint=True)).astype(np.int32)
    if shape.name == "long_context":
        return long_context_lengths(rng, B=B)
    if shape.name == "beam_search":  # B / BEAMS groups; a group's beams share its length
        tails = rng.integers(16, 512, size=B // BEAMS, endpoint=True)
        return np.repeat(PREFIX_TOKENS + tails, BEAMS).astype(np.int32)
    raise KeyError(shape.name)


def prefill_lengths(rng, S, *, chunk=PREFILL_CHUNK, cached=PREFILL_CACHED):
    """Chunked prefill: (context_lens, query_lens), each sequence a cached prefix drawn
    U[cached] followed by ``chunk`` new tokens (context_lens count both)."""
    pre = rng.integers(cached[0], cached[1], size=S, endpoint=True)
    q = np.full(S, chunk, dtype=np.int32)
    return (pre + q).astype(np.int32), q


def long_context_lengths(rng, *, B=128, n_long=8, long_len=32768, lo=64, hi=4096, n_fresh=8):
    """8 sequences at 32768 followed by short ones U[64, 4096]; at least ``n_fresh`` of the
    short ones have (n - 1) % 16 == 0, i.e. their newest token is the first of a block."""
    n_long = min(n_long, B)
    short = rng.integers(lo, hi, size=B - n_long, endpoint=True)
    k = min(n_fresh, B - n_long)
    pick = rng.choice(B - n_long, size=k, replace=False)
    for j in pick:
        short[j] = max(lo, (short[j] - 1) // BLOCK_SIZE * BLOCK_SIZE + 1)
        if (short[j] - 1) % BLOCK_SIZE:
            short[j] += BLOCK_SIZE - (short[j] - 1) % BLOCK_SIZE
    lens = np.concatenate([np.full(n_long, long_len), short]).astype(np.int32)
    return lens


def pool_blocks(lengths, slack=1.1, bs=BLOCK_SIZE):
    need = sum(blocks_for(n, bs) for n in lengths)
    return max(1, math.ceil(slack * need))


def place_sequences(lengths, free_order, max_blocks=None, bs=BLOCK_SIZE):
    """Block tables [B, max_blocks] (pad -1): sequence i takes the next blocks_for(n_i) entries
    of ``free_order``, sequences in order."""
    nblk = [blocks_for(n, bs) for n in lengths]
    if max_blocks is None:
        max_blocks = max(1, max(nblk) if nblk else 1)
    tables = np.full((len(lengths), max_blocks), -1, dtype=np.int32)
    pos = 0
    for i, c in enumerate(nblk):
        assert pos + c <= len(free_order), "pool too small"
        tables[i, :c] = free_order[pos:pos + c]
        pos += c
    return tables


def prefix_shared_tables(lengths, free_order, prefix_tokens=PREFIX_TOKENS, max_blocks=None,
                         bs=BLOCK_SIZE):
    """All sequences point at the same physical blocks for the prefix; tails are private."""
    assert prefix_tokens % bs == 0
    pb = prefix_tokens // bs
    nblk = [blocks_for(n, bs) for n in lengths]
    if max_blocks is None:
        max_blocks = max(nblk)
    tables = np.full((len(lengths), max_blocks), -1, dtype=np.int32)
    prefix = np.asarray(free_order[:pb])
    pos = pb
    for i, c in enumerate(nblk):
        tables[i, :pb] = prefix
        tables[i, pb:c] = free_order[pos:pos + c - pb]
        pos += c - pb
    return tables


def beam_tables(group_tail_lens, free_order, beams=4, prefix_tokens=PREFIX_TOKENS,
                bs=BLOCK_SIZE):
    """Beam variant: groups share the prefix; within a group the beams share every block of
    the group's history except each beam's own last block. Returns (tables, lengths)."""
    pb = prefix_tokens // bs
    lens = []
    rows = []
    pos = pb
    prefix = list(free_order[:pb])
    for tl in group_tail_lens:
        n = prefix_tokens + int(tl)
        tail_blocks = blocks_for(n, bs) - pb
        shared = list(free_order[pos:pos + tail_blocks - 1])
        pos += tail_blocks - 1
        for _ in range(beams):
            rows.append(prefix + shared + [int(free_order[pos])])
            pos += 1
            lens.append(n)
    max_blocks = max(len(r) for r in rows)
    tables = np.full((len(rows), max_blocks), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    return tables, np.asarray(lens, dtype=np.int32)


def beam_parents(rng, groups, beams):
    """Stand-in for beam selection (no model here): for each of ``groups`` groups, the parent
    beam (0..beams-1) of each of its next ``beams`` beams, drawn uniformly with replacement
    and sorted. int array [groups, beams]."""
    return np.sort(rng.integers(0, beams, size=(groups, beams)), axis=1)


def request_stream(rng, n, *, prompt=(1, 60), new=(1, 30), rate=0.5):
    """A seeded stream of n requests for the continuous-batching loop: (id, prompt length,
    max new tokens, arrival step). Lengths uniform in the inclusive ranges; arrivals a
    Poisson process of ``rate`` requests per step (exponential gaps, rounded down)."""
    p = rng.integers(prompt[0], prompt[1], size=n, endpoint=True)
    m = rng.integers(new[0], new[1], size=n, endpoint=True)
    arrival = np.floor(np.cumsum(rng.exponential(1.0 / rate, size=n))).astype(np.int64)
    return [(i, int(p[i]), int(m[i]), int(arrival[i])) for i in range(n)]


def blocks_in_use(tables, lengths, bs=BLOCK_SIZE):
    used = set()
    for row, n in zip(tables, lengths):
        used.update(int(b) for b in row[:blocks_for(n, bs)])
    return used


# ---- values --------------------------------------------------------------------------------

def round_to_dtype(x_f32, dtype):
    """Round float32 values to the storage dtype (nearest even). bf16 is returned as uint16
    bits; f16 as float16; f32 unchanged."""
    x_f32 = np.asarray(x_f32, dtype=np.float32)
    if dtype == "f32":
        return x_f32
    if dtype == "f16":
        return x_f32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise KeyError(dtype)


def normal_values(rng, shape, dtype):
    """N(0,1) float32 draws rounded to ``dtype`` (storage array)."""
    return round_to_dtype(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def device_normal(shape, dtype, seed, device="cuda"):
    """N(0,1) values drawn on the device with a seeded torch generator, in ``dtype``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=g)
    return t.to(torch_dtype(dtype))


def to_storage_numpy(t, dtype):
    """Exact host copy of a torch tensor as a storage array (bf16 -> uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_storage_numpy(a, dtype, device="cuda"):
    """Device tensor holding exactly the bits of a storage array."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)

"""GPU parity for caches of 8-bit and 3-bit per-row codes.

The library quantizes each new (token, KV head) row as it writes it
(paged_cache_write_q8 / _q3) and attends over the codes
(paged_attention_decode_q8 / _q3).
The oracle quantizes the same rows with oracle/quant.py (the course page's
teaching quantizer, float64) into its own host pool built by its own
allocator, and walks the tables in float64 over code * scale. Codes and
scales must match bit for bit; outputs within max-abs 1e-2 (bf16 queries).
Scale arrays start as NaN, so a stale slot that leaked into a result would
show up.
"""

import math
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_202_amd as pkv
from oracle import native
from oracle import quant
from oracle.attention import widen
from oracle.pool import PagedPool
from scenario import TIGHT
from synth import workloads as wl

pytestmark = pytest.mark.gpu


def host_bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# The 4-bit float e2m1 (sign, 2 exponent bits with bias 1, 1 mantissa bit;
# exponent 0 is subnormal: 0.5 x mantissa), by nibble. The 3-bit cache stores
# each code in [-3, 3] as its e2m1 bits; a nibble the quantizer never writes
# (-0, a half, +-4, +-6) decodes to a value no code equals (100 for the
# non-integers and -0).
E2M1_AS_CODE = np.array([0, 100, 1, 100, 2, 3, 4, 6, 100, 100, -1, 100, -2, -3, -4, -6],
                        np.int16)


def test_e2m1_table_is_the_format():
    """Pin the decoding table to the e2m1 definition itself."""
    for n in range(16):
        s, e, m = n >> 3, (n >> 1) & 3, n & 1
        v = (0.5 * m) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        v = -v if s else v
        want = int(v) if v == int(v) and not (s and v == 0) else 100
        assert E2M1_AS_CODE[n] == want, n


def unpack3(codes):
    """int8 codes of a 3-bit cache's bytes (e2m1 nibbles, even dim low)."""
    lo = E2M1_AS_CODE[codes & 0xF]
    hi = E2M1_AS_CODE[codes >> 4]
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (-1,)).astype(np.int8)


class Q8Case:
    def __init__(self, lens, Hq, Hkv, D, nq=1, bs=16, seed=0, in_dtype="bf16", device="cuda:0",
                 bits=8):
        self.bits = bits
        self.lens = [int(n) for n in lens]
        self.B, self.Hq, self.Hkv, self.D, self.nq, self.bs = len(lens), Hq, Hkv, D, nq, bs
        self.device = device
        rng = np.random.default_rng(seed)
        self.num_blocks = sum(-(-n // bs) for n in self.lens) + 4
        stack = rng.permutation(self.num_blocks).astype(np.int32)
        root = wl.root_seed(rng)
        T = sum(self.lens)
        # per-row magnitudes spread over decades, as real K/V rows are
        mag = wl.normal_array(root, 3, (T, Hkv, 1))
        k = wl.normal_array(root, 0, (T, Hkv, D)) * np.exp(mag)
        v = wl.normal_array(root, 1, (T, Hkv, D))
        self.k_new = wl.cast(k.astype(np.float32), in_dtype)
        self.v_new = wl.cast(v.astype(np.float32), in_dtype)
        self.q = wl.cast(wl.normal_array(root, 2, (self.B, nq, Hq, D)), "bf16")
        self.max_blocks = max(-(-n // bs) for n in self.lens)
        self.scale = 1.0 / math.sqrt(D)
        # oracle
        opool = PagedPool(self.num_blocks, bs, stack.tolist())
        slots = []
        for b, n in enumerate(self.lens):
            opool.create(b)
            s, _ = opool.append(b, n)
            slots += s
        shape = (self.num_blocks, Hkv, bs, D)
        self.o_kc = np.zeros(shape, np.int8)
        self.o_vc = np.zeros(shape, np.int8)
        self.o_ks = np.full(shape[:3], np.nan, np.float32)
        self.o_vs = np.full(shape[:3], np.nan, np.float32)
        quant.cache_write_q(self.o_kc, self.o_vc, self.o_ks, self.o_vs,
                            widen(host_bits(self.k_new), in_dtype),
                            widen(host_bits(self.v_new), in_dtype), slots, bs, bits=bits)
        t, l = opool.block_tables(range(self.B), self.max_blocks)
        self.o_tables, self.o_lens = np.array(t, np.int32), np.array(l, np.int32)
        self.o_slots = np.array(slots, np.int32)
        # library
        pool = pkv.PagedKVPool(self.num_blocks, bs, stack)
        for b in range(self.B):
            pool.seq_create(b)
        lslots, _ = pool.alloc_batch(list(range(self.B)), self.lens)
        assert np.array_equal(lslots, self.o_slots)
        tt, ll = pool.block_tables(list(range(self.B)), self.max_blocks)
        assert np.array_equal(tt, self.o_tables)
        self.cache = (pkv.Q8Cache if bits == 8 else pkv.Q3Cache)(self.num_blocks, Hkv, bs, D,
                                                                 device)
        self.cache.k_scales.fill_(float("nan"))
        self.cache.v_scales.fill_(float("nan"))
        # codes the quantizer never writes: -128, or e2m1 nibbles -6
        self.cache.k_codes.fill_(-128 if bits == 8 else 0xFF)
        self.cache.v_codes.fill_(-128 if bits == 8 else 0xFF)
        write = pkv.paged_cache_write_q8 if bits == 8 else pkv.paged_cache_write_q3
        write(self.k_new.to(device), self.v_new.to(device), self.cache,
              torch.from_numpy(lslots).to(device))
        self.d_tables = torch.from_numpy(tt).to(device)
        self.d_lens = torch.from_numpy(ll).to(device)
        self.d_q = self.q.to(device)

    def live_mask(self):
        live = np.zeros((self.num_blocks, self.bs), bool)
        for s in self.o_slots:
            live[s // self.bs, s % self.bs] = True
        return live

    def run_gpu(self, part=0):
        out = torch.full((self.B, self.nq, self.Hq, self.D), float("nan"), device=self.device)
        lse = torch.full((self.B, self.nq, self.Hq), float("nan"), device=self.device)
        n = pkv.paged_attention_workspace_size(self.B, self.nq, self.Hq, self.Hkv, self.D,
                                               self.max_blocks, self.bs, part)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        decode = pkv.paged_attention_decode_q8 if self.bits == 8 else pkv.paged_attention_decode_q3
        decode(out, self.d_q, self.cache, self.d_tables, self.d_lens, self.scale,
               partition_tokens=part, workspace=ws, lse=lse)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    def codes(self):
        """The library's codes as int8 arrays (3-bit ones unpacked)."""
        kc, vc = self.cache.k_codes.cpu().numpy(), self.cache.v_codes.cpu().numpy()
        if self.bits == 3:
            return unpack3(kc), unpack3(vc)
        return kc, vc

    def run_oracle(self, rows=None):
        return native.attention_q8(host_bits(self.q), "bf16", self.o_kc, self.o_vc, self.o_ks,
                                   self.o_vs, self.o_tables, self.o_lens, self.scale, self.bs,
                                   rows=rows, threads=min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D,bits", [(64, 8), (128, 8), (256, 8), (128, 3), (256, 3)])
def test_cache_write_codes_bit_exact(in_dtype, D, bits, device):
    print(f"code cache write: {bits} bits, {in_dtype} D {D}", flush=True)
    c = Q8Case((1, 17, 40, 77), 8, 2, D, seed=D, in_dtype=in_dtype, device=device, bits=bits)
    live = c.live_mask()
    kc, vc = c.codes()
    ks = c.cache.k_scales.cpu().numpy()
    vs = c.cache.v_scales.cpu().numpy()
    for got, want in ((kc, c.o_kc), (vc, c.o_vc)):
        assert np.array_equal(got.transpose(0, 2, 1, 3)[live], want.transpose(0, 2, 1, 3)[live])
    for got, want in ((ks, c.o_ks), (vs, c.o_vs)):
        g = got.transpose(0, 2, 1)[live].view(np.uint32)
        w = want.transpose(0, 2, 1)[live].view(np.uint32)
        assert np.array_equal(g, w)
    # slots nobody wrote keep their fill
    assert (kc.transpose(0, 2, 1, 3)[~live] == (-128 if bits == 8 else -6)).all()
    assert np.isnan(ks.transpose(0, 2, 1)[~live]).all()


def test_cache_write_zero_rows_and_skipped_slots(device):
    T, Hkv, D = 4, 2, 128
    k = torch.zeros((T, Hkv, D), dtype=torch.bfloat16, device=device)
    k[1, 0, 5] = -3.0
    v = torch.ones((T, Hkv, D), dtype=torch.bfloat16, device=device)
    cache = pkv.Q8Cache(2, Hkv, 16, D, device)
    cache.k_scales.fill_(7.0)
    slots = torch.tensor([0, 1, -1, 10 ** 6], dtype=torch.int32, device=device)
    pkv.paged_cache_write_q8(k, v, cache, slots)
    torch.cuda.synchronize()
    kc, ks = cache.k_codes.cpu().numpy(), cache.k_scales.cpu().numpy()
    assert (kc[0, :, 0] == 0).all() and (ks[0, :, 0] == 1.0).all()  # zero row: scale 1
    assert kc[0, 0, 1, 5] == -127 and ks[0, 0, 1] == np.float32(3.0 / 127)
    assert (cache.v_codes.cpu().numpy()[0, :, :2] == 127).all()
    assert (ks[0, :, 2:] == 7.0).all() and (ks[1] == 7.0).all()  # -1 and out of range skipped
    # K and V scales sit side by side per (block, KV head)
    sc = cache.scales.cpu().numpy()
    assert np.array_equal(sc[:, :, 0].view(np.uint32), ks.view(np.uint32))
    assert (sc[0, :, 1, :2] == np.float32(1.0 / 127)).all()  # V rows of ones


@pytest.mark.parametrize("bits", [8, 3])
def test_code_cache_copy_blocks(bits, device):
    """Copy-on-write of a code cache: the codes of K and V and the block's
    whole scale run move from src to dst; pairs naming a block outside the
    pool are skipped; every other block is left alone."""
    print(f"code cache copy_blocks: {bits} bits", flush=True)
    NB, Hkv, bs, D = 6, 2, 16, 128
    cache = (pkv.Q8Cache if bits == 8 else pkv.Q3Cache)(NB, Hkv, bs, D, device)
    g = torch.Generator().manual_seed(11)
    for t in (cache.k_codes, cache.v_codes):
        t.copy_(torch.randint(0, 256, t.shape, generator=g, dtype=torch.uint8).view(t.dtype))
    cache.scales.copy_(torch.rand(cache.scales.shape, generator=g))
    before = [t.cpu().numpy().copy() for t in (cache.k_codes, cache.v_codes, cache.scales)]
    pairs = torch.tensor([[1, 4], [2, 5], [0, NB], [-1, 3]], dtype=torch.int32, device=device)
    cache.copy_blocks(pairs)
    torch.cuda.synchronize()
    after = [t.cpu().numpy() for t in (cache.k_codes, cache.v_codes, cache.scales)]
    for b, a in zip(before, after):
        want = b.copy()
        want[4], want[5] = b[1], b[2]
        assert np.array_equal(a.view(np.uint8), want.view(np.uint8))


CASES = [
    # lens, Hq, Hkv, D, nq, partition_tokens
    ((1, 17, 250, 1000), 32, 8, 128, 1, 0),
    ((33, 700), 8, 8, 64, 1, 64),
    ((129, 300), 16, 2, 256, 1, 0),
    ((515, 47, 2000), 64, 8, 128, 1, -1),   # G = 8: 8 rows per wavefront
    ((90, 600), 32, 8, 128, 4, 0),          # 4 drafts x 4 heads: 16 rows per wavefront
    ((400,), 8, 4, 64, 2, 128),
    # the balanced plan on the stream mode: mixed lengths, G = 4 and 2
    ((1, 15, 16, 17, 100, 333, 2049, 700), 32, 8, 128, 1, -1),
    ((5, 64, 129, 700, 1025, 3), 16, 8, 64, 1, -1),
    (tuple(range(1, 300, 11)), 8, 2, 128, 1, -1),
    # 4096-token partitions: the many-wavefront workgroup split, ragged last tile
    ((8192, 5000), 32, 8, 128, 1, 4096),
    ((4500, 4200), 32, 8, 128, 4, 4096),    # 16 rows per wavefront
]


@pytest.mark.parametrize("bits", [8, 3])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_q8_attention_matches_oracle(ci, bits, device):
    lens, Hq, Hkv, D, nq, part = CASES[ci]
    if bits == 3 and D == 64:
        pytest.skip("3-bit codes are built for D 128 and 256")
    print(f"{bits}-bit attention case {ci}: lens {lens} Hq {Hq} Hkv {Hkv} D {D} nq {nq} "
          f"part {part}", flush=True)
    c = Q8Case(lens, Hq, Hkv, D, nq=nq, seed=100 + ci, device=device, bits=bits)
    out, lse = c.run_gpu(part)
    ref, ref_lse = c.run_oracle()
    err = np.abs(out - ref).max()
    print(f"  max-abs error {err:.3e}", flush=True)
    assert np.isfinite(out).all() and err <= 1e-2
    assert np.abs(lse - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("bits", [8, 3])
@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_q8_negative_and_zero_scale(scale, bits, device):
    """A negative scale (the kernel moves its sign into the query) and scale 0
    (every visible key weighs the same; lse = log of the count), on the split
    plan and on the stream plan."""
    print(f"{bits}-bit attention, scale {scale}", flush=True)
    c = Q8Case((1, 17, 250, 1000), 32, 8, 128, nq=1, seed=77, device=device, bits=bits)
    c.scale = scale
    ref, ref_lse = c.run_oracle()
    for part in (0, -1):
        out, lse = c.run_gpu(part)
        err = np.abs(out - ref).max()
        print(f"  partition {part}: max-abs error {err:.3e}", flush=True)
        assert np.isfinite(out).all() and err <= 1e-2
        assert np.abs(lse - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("bits", [8, 3])
@pytest.mark.parametrize("bs", [32, 64])
def test_q8_larger_blocks(bs, bits, device):
    """Blocks of 32 and 64 tokens: tiles (and their rows' scales) start
    inside a block; the split plan and the stream plan."""
    print(f"{bits}-bit attention, block size {bs}", flush=True)
    c = Q8Case((1, 17, 250, 1000, 2100), 32, 8, 128, bs=bs, seed=40 + bs, device=device,
               bits=bits)
    ref, ref_lse = c.run_oracle()
    for part in (0, -1):
        out, lse = c.run_gpu(part)
        err = np.abs(out - ref).max()
        print(f"  partition {part}: max-abs error {err:.3e}", flush=True)
        assert np.isfinite(out).all() and err <= 1e-2
        assert np.abs(lse - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("bits", [8, 3])
def test_q8_many_partitions_per_workgroup(bits, device):
    """2 sequences x 8 KV heads x 256 partitions of 16 tokens: one wavefront
    streams a run of two consecutive partitions as one partial."""
    c = Q8Case((4096, 2700), 32, 8, 128, nq=1, seed=31, device=device, bits=bits)
    ref, ref_lse = c.run_oracle()
    for part in (16, 0):
        out, lse = c.run_gpu(part)
        err = np.abs(out - ref).max()
        print(f"{bits}-bit, partition {part}: max-abs error {err:.3e}", flush=True)
        assert np.isfinite(out).all() and err <= 1e-2
        assert np.abs(lse - ref_lse).max() <= 1e-2


def test_q8_bad_table_and_short_context_give_nan(device):
    c = Q8Case((50, 60, 70), 8, 2, 128, nq=2, seed=9, device=device)
    tables = c.d_tables.clone()
    tables[1, 2] = c.num_blocks + 5
    lens = c.d_lens.clone()
    lens[2] = 1  # shorter than its 2 queries
    out = torch.zeros((3, 2, 8, 128), device=device)
    pkv.paged_attention_decode_q8(out, c.d_q, c.cache, tables, lens, c.scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    rows = np.arange(0, 2 * 8, dtype=np.int64)  # sequence 0
    ref, _ = c.run_oracle(rows=rows)
    assert np.abs(out[0].reshape(-1, 128) - ref).max() <= 1e-2


@pytest.mark.parametrize("name,bits", [("llama3_8b_b32_8k_q8", 8), ("llama3_8b_b32_8k_q3", 3),
                                       ("llama3_8b_varlen_b256_q8", 8)])
def test_q8_full_size_sampled(name, bits, device):
    """The 8K decode batch (32 sequences, Llama-3-8B layer geometry) over an
    8-bit (3-bit) code cache, and the variable-length batch of 256 over 8-bit
    codes (the stream mode), in the launch configuration bench.py times:
    slots and tables bit for bit, the codes of a few sequences bit for bit,
    and their rows against the C oracle."""
    import bench

    print(f"q8 full size: {name}", flush=True)
    wk = bench.Workload(name, 1, device)
    opool = PagedPool(wk.w.num_blocks, wk.bs, wk.stack.tolist())
    pre = (wk.lens - wk.nq).tolist()
    pre_slots, step_slots = [], []
    for b in range(wk.B):
        opool.create(b)
    for b in range(wk.B):
        pre_slots += opool.append(b, pre[b])[0]
    for b in range(wk.B):
        step_slots += opool.append(b, wk.nq)[0]
    assert np.array_equal(wk.pre_slots, pre_slots)
    assert np.array_equal(wk.step_slots, step_slots)
    tables, lens = opool.block_tables(range(wk.B), wk.max_blocks)
    tables, lens = np.array(tables, np.int32), np.array(lens, np.int32)
    assert np.array_equal(wk.tables_host, tables)
    wk.lse = torch.full((wk.B, wk.nq, wk.Hq), float("nan"), dtype=torch.float32, device=device)
    wk.step(0)
    torch.cuda.synchronize()
    out = wk.out.cpu().numpy()
    lse = wk.lse.cpu().numpy().reshape(-1)
    # the oracle quantizes the rows of a few sequences only (for the
    # variable-length batch also the longest and the last one)
    seqs = [0, 9, 20, 31] if wk.B == 32 else sorted({0, 9, 100, int(np.argmax(wk.lens)),
                                                      wk.B - 1})
    starts = np.concatenate([[0], np.cumsum(wk.lens)[:-1]])
    kbits, vbits = host_bits(wk.host_k), host_bits(wk.host_v)
    shape = (wk.w.num_blocks, wk.Hkv, wk.bs, wk.D)
    kc = np.zeros(shape, np.int8)
    vc = np.zeros(shape, np.int8)
    ks = np.ones(shape[:3], np.float32)
    vs = np.ones(shape[:3], np.float32)
    pre_off = np.concatenate([[0], np.cumsum(pre)])
    for b in seqs:
        tok = np.arange(starts[b], starts[b] + wk.lens[b])
        sl = list(pre_slots[pre_off[b]:pre_off[b + 1]]) + [step_slots[b]]
        quant.cache_write_q(kc, vc, ks, vs, widen(kbits[tok], "bf16"), widen(vbits[tok], "bf16"),
                            sl, wk.bs, bits=bits)
    g = wk.qc[0]
    gk, gks = g.k_codes.cpu().numpy(), g.k_scales.cpu().numpy()
    if bits == 3:
        gk = unpack3(gk)
    for b in seqs:
        for blk in tables[b][:-(-int(lens[b]) // wk.bs)]:
            assert np.array_equal(gk[blk], kc[blk]) and np.array_equal(gks[blk], ks[blk])
    rows = np.concatenate([np.arange(b * wk.Hq, (b + 1) * wk.Hq) for b in seqs]).astype(np.int64)
    ref, ref_lse = native.attention_q8(host_bits(wk.host_q), "bf16", kc, vc, ks, vs, tables,
                                       lens, wk.scale, wk.bs, rows=rows,
                                       threads=min(16, len(os.sched_getaffinity(0))))
    d_out = np.abs(out.reshape(-1, wk.D)[rows] - ref).max(axis=1)
    d_lse = np.abs(lse[rows] - ref_lse)
    err, lerr = d_out.max(), d_lse.max()
    print(f"  max-abs error out {err:.3e}, lse {lerr:.3e} over {len(rows)} rows", flush=True)
    assert np.isfinite(out).all() and err <= 1e-2 and lerr <= 1e-2
    # the tight bounds, by the row's context length (one dropped or repeated
    # tile would break them: tests/test_parity_bounds.py)
    long_row = np.asarray(wk.lens)[rows // wk.Hq] >= 4096
    for sel, key in ((long_row, "codes_long"), (~long_row, "codes_short")):
        if sel.any():
            ob, lb = TIGHT[key]
            assert d_out[sel].max() <= ob and d_lse[sel].max() <= lb, key

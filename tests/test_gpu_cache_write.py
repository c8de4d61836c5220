"""KV-cache write kernels against the oracle's quantiser (MI355X only): every byte of every
written row equal, untouched rows untouched, faults reported.  Calls go through the C ABI."""

import numpy as np
import pytest
import torch

import oracle as O
from tests.packing import bf16_bits

pytestmark = pytest.mark.gpu

M = pytest.importorskip("sparse_attention_decode_dsa_amd.ml4dsa")

DEV = "cuda:0"
FILL = 0xA5


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _values(n, d, seed, dtype):
    """Per-token magnitudes over 12 binades, all-zero tokens, exact E4M3 ties, -0."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, d, generator=g) * torch.exp(torch.empty(n, 1).uniform_(-6, 6, generator=g))
    if n > 1:
        x[1] = 0.0
    if n > 3:
        # amax 448 -> scale exactly 1: the rest are midpoints between E4M3 neighbours (ties)
        pos = np.array(sorted({float(v) for v in O.E4M3_TABLE if np.isfinite(v) and v >= 0}))
        mids = torch.tensor((pos[:-1] + pos[1:]) / 2, dtype=torch.float32)
        x[3] = mids[torch.randint(0, len(mids), (d,), generator=g)] * torch.where(
            torch.rand(d, generator=g) < 0.5, -1.0, 1.0)
        x[3, 0] = 448.0
        x[2, :8] = -0.0
    if dtype == torch.bfloat16:
        x = x.to(torch.bfloat16)
    return x


def _slots(n, capacity, seed):
    g = torch.Generator().manual_seed(seed + 99)
    s = torch.randperm(capacity, generator=g)[:n].to(torch.int64)
    s[::17] = -1                    # padding tokens: skipped
    return s


@pytest.mark.parametrize("n,src", [(1000, torch.bfloat16), (333, torch.float32), (1, torch.bfloat16)])
def test_index_cache_write_matches_quantiser(n, src):
    print(f"[gpu] index cache write n={n} {src}", flush=True)
    bs, nb = 64, (n + 200) // 64 + 2
    k = _values(n, 128, n, src)
    slots = _slots(n, nb * bs, n)
    pool = torch.full((nb, bs, 132), FILL, dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    cache = M.make_cache(pool, M.ML4_IDX_FP8_132)
    dt = M.ML4_BF16 if src == torch.bfloat16 else M.ML4_F32
    kd, sd = k.to(DEV), slots.to(DEV)
    M.ml4_index_cache_write(cache, bs, kd, dt, n, sd, fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    got = pool.cpu().numpy().reshape(-1, 132)
    want = O.quantise_index_rows(k.float().numpy())
    live = slots.numpy() >= 0
    assert np.array_equal(got[slots.numpy()[live]], want[live])
    untouched = np.ones(nb * bs, bool)
    untouched[slots.numpy()[live]] = False
    assert np.all(got[untouched] == FILL)


@pytest.mark.parametrize("n,src,rope", [(700, torch.bfloat16, 64), (129, torch.float32, 64),
                                        (300, torch.bfloat16, 0)])
def test_latent_cache_write_matches_quantiser(n, src, rope):
    print(f"[gpu] latent cache write n={n} {src} rope={rope}", flush=True)
    bs, nb = 64, (n + 100) // 64 + 2
    c = _values(n, 512, n + 7, src)
    kr = torch.randn(n, 64, generator=torch.Generator().manual_seed(n)).to(torch.bfloat16)
    slots = _slots(n, nb * bs, n + 7)
    pool = torch.full((nb, bs, 656), FILL, dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    cache = M.make_cache(pool, M.ML4_LAT_FP8_656)
    dt = M.ML4_BF16 if src == torch.bfloat16 else M.ML4_F32
    M.ml4_latent_cache_write(cache, bs, c.to(DEV), dt, kr.to(DEV) if rope else None, rope, n,
                             slots.to(DEV), fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    got = pool.cpu().numpy().reshape(-1, 656)
    want = O.quantise_latent_rows(c.float().numpy(), bf16_bits(kr.float()) if rope else None)
    live = slots.numpy() >= 0
    rows = slots.numpy()[live]
    assert np.array_equal(got[rows, :528], want[live, :528])
    if rope:
        assert np.array_equal(got[rows, 528:], want[live, 528:])
    else:
        assert np.all(got[rows, 528:] == FILL)          # NoPE: RoPE bytes left as they were
    untouched = np.ones(nb * bs, bool)
    untouched[rows] = False
    assert np.all(got[untouched] == FILL)


def _bf16_ties(d, seed):
    """fp32 values whose low 16 bits are exactly 0x8000 (ties at bf16), both parities."""
    g = np.random.default_rng(seed)
    hi = g.integers(0x3000, 0x4800, d, dtype=np.uint32)
    x = ((hi << 16) | 0x8000).view(np.float32)
    return torch.from_numpy(x * np.where(g.random(d) < 0.5, -1, 1).astype(np.float32))


@pytest.mark.parametrize("n,src,rope", [(700, torch.bfloat16, 64), (129, torch.float32, 64),
                                        (300, torch.float32, 0)])
def test_bf16_latent_cache_write_matches_oracle(n, src, rope):
    """1,152-B bf16 rows: every written bf16 value equals the oracle's round-to-nearest-even
    latents and the given RoPE bits; NoPE leaves the RoPE half untouched."""
    print(f"[gpu] bf16 latent cache write n={n} {src} rope={rope}", flush=True)
    bs, nb = 32, (n + 100) // 32 + 2
    c = _values(n, 512, n + 11, torch.float32)
    if n > 4:
        c[4] = _bf16_ties(512, n)
    c = c.to(src)
    kr = torch.randn(n, 64, generator=torch.Generator().manual_seed(n + 1)).to(torch.bfloat16)
    slots = _slots(n, nb * bs, n + 11)
    pool = torch.full((nb, bs, 1152), FILL, dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    dt = M.ML4_BF16 if src == torch.bfloat16 else M.ML4_F32
    M.ml4_latent_cache_write(M.make_cache(pool, M.ML4_LAT_BF16_1152), bs, c.to(DEV), dt,
                             kr.to(DEV) if rope else None, rope, n, slots.to(DEV), fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    raw = pool.cpu().numpy().reshape(-1, 1152)
    got = raw.view(np.uint16)
    want = O.pack_latent_rows_bf16(c.float().numpy(), bf16_bits(kr.float()) if rope else None)
    live = slots.numpy() >= 0
    rows = slots.numpy()[live]
    assert np.array_equal(got[rows, :512], want[live, :512])
    if rope:
        assert np.array_equal(got[rows, 512:], want[live, 512:])
    else:
        assert np.all(raw[rows, 1024:] == FILL)
    untouched = np.ones(nb * bs, bool)
    untouched[rows] = False
    assert np.all(raw[untouched] == FILL)


@pytest.mark.parametrize("n,src,rope,kv_scale", [(700, torch.bfloat16, 64, 1.0),
                                                 (129, torch.float32, 64, 0.37),
                                                 (300, torch.bfloat16, 0, 3.0)])
def test_e4m3_latent_cache_write_matches_oracle(n, src, rope, kv_scale):
    """576-B plain E4M3 rows: every code equals the oracle's E4M3(x / kv_scale) (ties at
    scale 1, saturation beyond 448 * kv_scale, -0); NoPE leaves the RoPE codes untouched."""
    print(f"[gpu] e4m3 latent cache write n={n} {src} rope={rope} s={kv_scale}", flush=True)
    bs, nb = 64, (n + 100) // 64 + 2
    c = _values(n, 512, n + 13, src)
    kr = (torch.randn(n, 64, generator=torch.Generator().manual_seed(n + 2)) * 40).to(
        torch.bfloat16)
    slots = _slots(n, nb * bs, n + 13)
    pool = torch.full((nb, bs, 576), FILL, dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    dt = M.ML4_BF16 if src == torch.bfloat16 else M.ML4_F32
    M.ml4_latent_cache_write_e4m3(M.make_cache(pool, M.ML4_LAT_E4M3_576), bs, c.to(DEV), dt,
                                  kr.to(DEV) if rope else None, rope, kv_scale, n,
                                  slots.to(DEV), fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    got = pool.cpu().numpy().reshape(-1, 576)
    want = O.quantise_latent_rows_e4m3(c.float().numpy(), kr.float().numpy() if rope else None,
                                       kv_scale)
    live = slots.numpy() >= 0
    rows = slots.numpy()[live]
    assert np.array_equal(got[rows, :512], want[live, :512])
    if rope:
        assert np.array_equal(got[rows, 512:], want[live, 512:])
    else:
        assert np.all(got[rows, 512:] == FILL)
    untouched = np.ones(nb * bs, bool)
    untouched[rows] = False
    assert np.all(got[untouched] == FILL)


def test_e4m3_latent_cache_write_faults():
    """A NaN RoPE value and an out-of-pool slot are both reported; the other rows are the
    oracle's."""
    print("[gpu] e4m3 latent cache write faults", flush=True)
    bs, nb, n = 16, 2, 6
    c = torch.randn(n, 512).to(torch.bfloat16)
    kr = torch.randn(n, 64).to(torch.bfloat16)
    kr[3, 60] = float("nan")
    slots = torch.arange(n, dtype=torch.int64)
    slots[1] = nb * bs
    pool = torch.full((nb, bs, 576), FILL, dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    M.ml4_latent_cache_write_e4m3(M.make_cache(pool, M.ML4_LAT_E4M3_576), bs, c.to(DEV),
                                  M.ML4_BF16, kr.to(DEV), 64, 0.05, n, slots.to(DEV), fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == M.ML4_FAULT_BLOCK_ID | M.ML4_FAULT_RANGE
    got = pool.cpu().numpy().reshape(-1, 576)
    want = O.quantise_latent_rows_e4m3(c.float().numpy(),
                                       np.nan_to_num(kr.float().numpy()), 0.05)
    for i in (0, 2, 4, 5):
        assert np.array_equal(got[i], want[i])
    assert np.all(got[1] == FILL) and np.all(got[nb * bs - 1] == FILL)


def test_cache_write_faults_are_reported_and_contained():
    print("[gpu] cache write faults", flush=True)
    bs, nb, n = 16, 4, 8
    k = torch.randn(n, 128).to(torch.bfloat16)
    k[5, 3] = float("nan")
    slots = torch.arange(n, dtype=torch.int64)
    slots[2] = nb * bs            # one past the pool: skipped, BLOCK_ID
    pool = torch.full((nb, bs, 132), FILL, dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    M.ml4_index_cache_write(M.make_cache(pool, M.ML4_IDX_FP8_132), bs, k.to(DEV), M.ML4_BF16,
                            n, slots.to(DEV), fault)
    torch.cuda.synchronize()
    bits = M.ml4_fault_query(fault)
    assert bits == M.ML4_FAULT_BLOCK_ID | M.ML4_FAULT_RANGE
    got = pool.cpu().numpy().reshape(-1, 132)
    want = O.quantise_index_rows(np.where(np.isfinite(k.float().numpy()), k.float().numpy(), 0))
    for i in range(n):
        if i in (2, 5):
            continue
        assert np.array_equal(got[i], want[i])
    assert np.all(got[nb * bs - 1] == FILL) and np.all(got[2] == FILL)

"""Per-op parity: every C-ABI entry point against the oracle on the same seeded inputs."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from oracle import ops
from oracle.q8_0 import quantize_q8_0
from quantized_transformer_prefill_amd import binding as B
from quantized_transformer_prefill_amd.model import interleave_gate_up
from tests.gpu_util import assert_codes_match, assert_f32_match, need_gpu, say

pytestmark = pytest.mark.gpu
f32 = np.float32


def outlier_acts(m, k, seed, dev):
    x, _ = synth.gen_gemm_inputs(synth.GemmCase(m, k, 32, seed=seed), device=dev)
    return x.contiguous()


# ---------------------------------------------------------------- quantizer
def test_quantize_bit_exact_worked_blocks_and_c2_activations():
    dev = need_gpu()
    from tests.test_oracle_q8_0 import load_worked_blocks
    rows = []
    for case in load_worked_blocks():
        r = np.zeros(32, dtype=f32)
        for i, v in case["x"].items():
            r[i] = v
        rows.append(r)
    x = torch.tensor(np.stack(rows), device=dev)
    gc, gs = B.quantize_q8_0(x)
    oc, os_ = quantize_q8_0(x.cpu().numpy())
    assert_codes_match(gc, gs, oc, os_, what="worked blocks")
    for case in synth.GEMM_SWEEP:  # the activation matrices of the GEMM sweep at full size
        x = outlier_acts(case.m, case.k, case.seed, dev)
        say(f"quantize {case.name}")
        gc, gs = B.quantize_q8_0(x)
        oc, os_ = quantize_q8_0(x.cpu().numpy())
        assert_codes_match(gc, gs, oc, os_, what=case.name)


def test_quantize_extreme_ranges():
    dev = need_gpu()
    g = torch.Generator(device=dev).manual_seed(5)
    parts = [torch.randn(40, 96, generator=g, device=dev) * s for s in (1e-7, 1e-3, 1.0, 1e4)]
    x = torch.cat(parts).contiguous()
    x[3, :32] = 0.0
    gc, gs = B.quantize_q8_0(x)
    oc, os_ = quantize_q8_0(x.cpu().numpy())
    assert_codes_match(gc, gs, oc, os_, what="scales 1e-7..1e4")


# ---------------------------------------------------------------- matmul
def q8_pair(w_dev):
    gc, gs = B.quantize_q8_0(w_dev)
    oc, os_ = quantize_q8_0(w_dev.cpu().numpy())
    return (gc, gs), (oc, os_)


GEMM_CASES = [  # m, k, n, bias, residual, split
    (77, 320, 192, True, False, 1),
    (64, 896, 1152, True, False, 1),
    (130, 4864, 896, False, True, 0),
    (1, 896, 896, False, True, 1),
    (5, 3584, 512, True, True, 0),
    (200, 128, 64, False, False, 1),
    (33, 1024, 256, True, False, 4),
    (256, 512, 16384, True, False, 0),   # 2x2 wave tiles (64 x 128 workgroups)
    (45, 160, 224, False, False, 1),     # one 1-block stage after a full one; row and column tails
    (3, 96, 96, True, False, 1),         # K shorter than one 4-block stage
    (520, 160, 8224, False, True, 0),    # 4x2 wave tiles (128 x 128 workgroups): row, column, K-stage tails
    (520, 160, 16608, True, False, 0),   # 2x2 tiles with row, column and K-stage tails
    (1030, 160, 3936, True, True, 1),    # 4x2 tiles: row, column, K-stage tails
    (1024, 8192, 1024, False, False, 0), # 4x2 tiles, split K chosen by the library
    (600, 8192, 1664, True, True, 0),    # 4x2 tiles for a long reduction over fewer rows, split K, row tail
]


@pytest.mark.parametrize("m,k,n,use_bias,use_res,split", GEMM_CASES,
                         ids=[f"m{c[0]}_k{c[1]}_n{c[2]}_s{c[5]}" for c in GEMM_CASES])
def test_gemm_matches_oracle(m, k, n, use_bias, use_res, split):
    dev = need_gpu()
    say(f"gemm m={m} k={k} n={n} bias={use_bias} res={use_res} split={split}")
    x = outlier_acts(m, k, 11, dev)
    w = synth.gen_normal(12, f"w{n}x{k}", (n, k), std=0.02, device=dev)
    bias = synth.gen_normal(13, f"b{n}", (n,), std=0.02, device=dev) if use_bias else None
    res = synth.gen_normal(14, f"r{m}x{n}", (m, n), device=dev) if use_res else None
    (wc, ws), (owc, ows) = q8_pair(w)
    xc, xs = B.quantize_q8_0(x)
    out = B.gemm_q8_0(xc, xs, wc, ws, bias=bias, residual=res, split_k=split)
    torch.cuda.synchronize()
    want = ops.matmul_q8_0(x.cpu().numpy(), owc, ows, None if bias is None else bias.cpu().numpy())
    if res is not None:
        want = ops.add_f32(res.cpu().numpy(), want)
    assert_f32_match(out.cpu().numpy(), want, what="gemm out")


def _random_gemm_cases(n_cases, seed):
    """Seeded random shapes: rows 1..1200, output columns a multiple of 32 up to 4096, K a multiple of
    32 up to 3072 (odd and even block counts), the library's split or a forced one (1, 2, 3, 7)."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        m = int(rng.integers(1, 1201))
        n = 32 * int(rng.integers(1, 129))
        k = 32 * int(rng.integers(1, 97))
        split = int(rng.choice([0, 0, 1, 2, 3, 7]))
        cases.append((m, k, n, bool(rng.integers(2)), bool(rng.integers(2)), split))
    return cases


RANDOM_GEMM_CASES = _random_gemm_cases(16, 20261203)


@pytest.mark.parametrize("m,k,n,use_bias,use_res,split", RANDOM_GEMM_CASES,
                         ids=[f"m{c[0]}_k{c[1]}_n{c[2]}_s{c[5]}" for c in RANDOM_GEMM_CASES])
def test_gemm_random_shapes_match_oracle(m, k, n, use_bias, use_res, split):
    test_gemm_matches_oracle(m, k, n, use_bias, use_res, split)


RANDOM_SWIGLU_CASES = [(m, k, 32 * max(1, n // 64)) for m, k, n, *_ in _random_gemm_cases(10, 20261204)]


@pytest.mark.parametrize("m,k,f", RANDOM_SWIGLU_CASES, ids=[f"m{c[0]}_k{c[1]}_f{c[2]}" for c in RANDOM_SWIGLU_CASES])
def test_gemm_swiglu_random_shapes_match_oracle(m, k, f):
    dev = need_gpu()
    say(f"gemm+swiglu m={m} k={k} ffn={f}")
    x = synth.gen_normal(34, f"x{m}x{k}", (m, k), device=dev)
    wg = synth.gen_normal(35, f"g{f}x{k}", (f, k), std=0.02, device=dev)
    wu = synth.gen_normal(36, f"u{f}x{k}", (f, k), std=0.02, device=dev)
    (gc, gs), (ogc, ogs) = q8_pair(wg)
    (uc, us), (ouc, ous) = q8_pair(wu)
    wgu_c = interleave_gate_up(gc, uc).contiguous()
    wgu_s = interleave_gate_up(gs, us).contiguous()
    xc, xs = B.quantize_q8_0(x)
    wsp = torch.empty(max(B.lib().mi_gemm_q8_0_workspace_bytes(m, 2 * f, k), 8), dtype=torch.uint8, device=dev)
    sc, ss = B.gemm_swiglu_q8_0(xc, xs, wgu_c, wgu_s, workspace=wsp)
    xh = x.cpu().numpy()
    s = ops.swiglu(ops.matmul_q8_0(xh, ogc, ogs), ops.matmul_q8_0(xh, ouc, ous))
    oc, os_ = quantize_q8_0(s)
    assert_codes_match(sc, ss, oc, os_, max_frac_code_diff=1e-4, what=f"swiglu codes m={m} k={k} f={f}")


def test_gemm_in_place_residual():
    dev = need_gpu()
    x = outlier_acts(40, 896, 21, dev)
    w = synth.gen_normal(22, "w", (896, 896), std=0.02, device=dev)
    h = synth.gen_normal(23, "h", (40, 896), device=dev)
    h0 = h.cpu().numpy()
    (wc, ws), (owc, ows) = q8_pair(w)
    xc, xs = B.quantize_q8_0(x)
    B.gemm_q8_0(xc, xs, wc, ws, residual=h, out=h)
    want = ops.add_f32(h0, ops.matmul_q8_0(x.cpu().numpy(), owc, ows))
    assert_f32_match(h.cpu().numpy(), want, what="h += x W")


@pytest.mark.parametrize("case", synth.GEMM_SWEEP, ids=lambda c: c.name)
def test_gemm_full_size_matches_oracle(case):
    """The GEMM sweep at full size, in the launch configuration the benchmark uses (the library's own
    tile and split choice): every output element against the oracle's f64 matmul of the same Q8_0
    operands (the activations with 1% x20 outliers are quantized by both sides, bit-identically)."""
    dev = need_gpu()
    say(f"gemm full size {case.name}")
    x, w = synth.gen_gemm_inputs(case, device=dev)
    xc, xs = B.quantize_q8_0(x)
    wc, ws = B.quantize_q8_0(w)
    out = B.gemm_q8_0(xc, xs, wc, ws, split_k=0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del out, xc, xs, wc, ws
    oq, od = quantize_q8_0(w.cpu().numpy())
    want = ops.matmul_q8_0(x.cpu().numpy(), oq, od)
    d = got.astype(np.float64) - want
    say(f"  {case.name}: max-abs {np.abs(d).max():.3e} rel-L2 {np.linalg.norm(d) / np.linalg.norm(want):.3e}")
    assert_f32_match(got, want, what=f"{case.name} all outputs")


def test_pack_canonical_blocks():
    """mi_pack_q8_0: canonical 34-byte blocks (fp16 scale, 32 codes), built on the host from the
    oracle's quantization, land in the two planes byte for byte -- the oracle's codes and scales,
    and the library's own quantization of the same f32 values."""
    dev = need_gpu()
    for rows, cols in [(3, 32), (7, 896), (129, 4864)]:
        w = synth.gen_normal(111, f"p{rows}x{cols}", (rows, cols), std=0.02, device=dev)
        w[0, :32] = 0.0                                   # an all-zero block
        oc, os_ = quantize_q8_0(w.cpu().numpy())
        blk = np.zeros(rows * (cols // 32), dtype=np.dtype([("d", "<u2"), ("qs", "i1", 32)], align=False))
        assert blk.dtype.itemsize == 34
        blk["d"] = os_.view(np.uint16).reshape(-1)
        blk["qs"] = oc.reshape(-1, 32)
        raw = torch.as_tensor(np.frombuffer(blk.tobytes(), dtype=np.uint8).copy(), device=dev)
        pc, ps = B.pack_q8_0(raw, rows, cols)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(pc.cpu().numpy(), oc)
        np.testing.assert_array_equal(ps.cpu().numpy().view(np.uint16), os_.view(np.uint16))
        gc, gs = B.quantize_q8_0(w)
        assert torch.equal(gc, pc) and torch.equal(gs, ps)


def test_gemm_swiglu_matches_oracle():
    dev = need_gpu()
    # 1x2 wave tiles for the first three, then 4x2 (128 x 128 workgroups) and 2x2 (64 x 128): the
    # library picks the one that fills the chip's workgroup slots in fewer rounds
    for m, k, f in [(100, 896, 320), (16, 3584, 512), (1, 896, 4864), (512, 256, 8192), (1100, 256, 3680),
                    (1000, 160, 8192),   # 4x2 tiles with a row tail and a 1-block K stage
                    (3, 64, 32), (70, 96, 32)]:  # one 32-wide SwiGLU block: a single column tile
        say(f"gemm+swiglu m={m} k={k} ffn={f}")
        x = synth.gen_normal(31, f"x{m}", (m, k), device=dev)
        wg = synth.gen_normal(32, f"g{f}", (f, k), std=0.02, device=dev)
        wu = synth.gen_normal(33, f"u{f}", (f, k), std=0.02, device=dev)
        (gc, gs), (ogc, ogs) = q8_pair(wg)
        (uc, us), (ouc, ous) = q8_pair(wu)
        wgu_c = interleave_gate_up(gc, uc).contiguous()
        wgu_s = interleave_gate_up(gs, us).contiguous()
        xc, xs = B.quantize_q8_0(x)
        ws_bytes = B.lib().mi_gemm_q8_0_workspace_bytes(m, 2 * f, k)
        wsp = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
        sc, ss = B.gemm_swiglu_q8_0(xc, xs, wgu_c, wgu_s, workspace=wsp)
        xh = x.cpu().numpy()
        s = ops.swiglu(ops.matmul_q8_0(xh, ogc, ogs), ops.matmul_q8_0(xh, ouc, ous))
        oc, os_ = quantize_q8_0(s)
        assert_codes_match(sc, ss, oc, os_, max_frac_code_diff=1e-4, what=f"swiglu codes m={m}")


# ---------------------------------------------------------------- row / elementwise ops
def test_rmsnorm_quant_matches_oracle():
    dev = need_gpu()
    # the last two: full-size row counts of the 7B- and 8B-shaped prompts
    for rows, cols in [(37, 896), (5, 4096), (3, 3584), (2, 18944), (1, 64), (2100, 3584), (2600, 2048)]:
        x = synth.gen_normal(41, f"x{rows}", (rows, cols), std=0.7, device=dev)
        gam = (1 + synth.gen_normal(42, f"g{cols}", (cols,), std=0.02, device=dev)).contiguous()
        gc, gs, y = B.rmsnorm_quant(x, gam, 1e-6, want_y=True)
        want_y = ops.rms_norm(x.cpu().numpy(), gam.cpu().numpy(), 1e-6)
        assert_f32_match(y.cpu().numpy(), want_y, what=f"rmsnorm y {rows}x{cols}")
        oc, os_ = quantize_q8_0(want_y)
        assert_codes_match(gc, gs, oc, os_, max_frac_code_diff=1e-4, what=f"rmsnorm codes {rows}x{cols}")


def test_swiglu_quant_matches_oracle():
    dev = need_gpu()
    g = synth.gen_normal(51, "g", (29, 4864), std=2.0, device=dev)
    u = synth.gen_normal(52, "u", (29, 4864), device=dev)
    gc, gs = B.swiglu_quant(g, u)
    s = ops.swiglu(g.cpu().numpy(), u.cpu().numpy())
    oc, os_ = quantize_q8_0(s)
    assert_codes_match(gc, gs, oc, os_, max_frac_code_diff=1e-4, what="swiglu_quant")


def test_embed_exact():
    dev = need_gpu()
    w = synth.gen_normal(61, "emb", (500, 896), std=0.02, device=dev)
    (wc, ws), (oc, os_) = q8_pair(w)
    ids = np.array([499, 0, 7, 7, 250], dtype=np.int32)
    out = B.embed_q8_0(wc, ws, torch.as_tensor(ids, device=dev))
    np.testing.assert_array_equal(out.cpu().numpy(), ops.embed_q8_0(oc, os_, ids))


def test_qk_norm_matches_oracle():
    dev = need_gpu()
    for nh, hd in [(32, 128), (8, 128), (14, 64)]:
        x = synth.gen_normal(71, f"q{nh}", (19, nh * hd), std=0.5, device=dev)
        gam = (1 + synth.gen_normal(72, f"g{hd}", (hd,), std=0.02, device=dev)).contiguous()
        x0 = x.cpu().numpy()
        B.qk_norm_(x, gam, nh, hd, 1e-6)
        want = ops.qk_norm(x0.reshape(19, nh, hd), gam.cpu().numpy(), 1e-6).reshape(19, nh * hd)
        assert_f32_match(x.cpu().numpy(), want, what=f"qk_norm nh={nh} hd={hd}")


def _rope_table(nh, nkv, hd, rows, dev):
    hp = B.Hparams(1, 64, nh, nkv, hd, 64, 64, 1e-6, 1e6, 0, 0, 0)
    t = torch.empty(B.lib().mi_rope_table_bytes(C.byref(hp), rows) // 8, dtype=torch.float64, device=dev)
    B.check(B.lib().mi_rope_table_init(C.byref(hp), rows, t.data_ptr(), B.stream_ptr()))
    return t


@pytest.mark.parametrize("nh,nkv,hd", [(14, 2, 64), (32, 8, 128)])
def test_rope_kvstore_rows_and_values(nh, nkv, hd):
    dev = need_gpu()
    n_ctx, n = 4096, 23
    rng = np.random.default_rng(hd)
    pos = rng.choice(n_ctx, size=n, replace=False).astype(np.int32)
    pos[0] = n_ctx - 1
    q = synth.gen_normal(81, "q", (n, nh * hd), device=dev)
    k = synth.gen_normal(82, "k", (n, nkv * hd), device=dev)
    v = synth.gen_normal(83, "v", (n, nkv * hd), device=dev)
    q0, k0, v0 = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    sentinel = -12345.5
    kr = torch.full((n_ctx, nkv * hd), sentinel, device=dev)
    vr = torch.full((n_ctx, nkv * hd), sentinel, device=dev)
    table = _rope_table(nh, nkv, hd, n_ctx, dev)
    B.rope_kvstore(q, k, v, torch.as_tensor(pos, device=dev), nh, nkv, hd, table, n_ctx, kr, vr)
    qw = ops.rope_neox(q0.reshape(n, nh, hd), pos, 1e6).reshape(n, nh * hd)
    kw = ops.rope_neox(k0.reshape(n, nkv, hd), pos, 1e6).reshape(n, nkv * hd)
    assert_f32_match(q.cpu().numpy(), qw, what="rope q")
    krh, vrh = kr.cpu().numpy(), vr.cpu().numpy()
    assert_f32_match(krh[pos], kw, what="rope k -> region rows")
    np.testing.assert_array_equal(vrh[pos], v0)
    untouched = np.setdiff1d(np.arange(n_ctx), pos)
    assert np.all(krh[untouched] == sentinel) and np.all(vrh[untouched] == sentinel)
    np.testing.assert_array_equal(k.cpu().numpy(), k0)  # k itself is not modified


# GQA groups of 7, 7, 4, 1, 2 and 16 query heads per KV head; unsorted positions with gaps
@pytest.mark.parametrize("nh,nkv,hd,n,n_ctx", [(14, 2, 64, 37, 300), (28, 4, 128, 21, 200), (32, 8, 128, 50, 700),
                                               (4, 4, 64, 1, 5), (4, 2, 128, 30, 100), (16, 1, 128, 20, 64)])
def test_attention_matches_oracle(nh, nkv, hd, n, n_ctx):
    dev = need_gpu()
    say(f"attention nh={nh} nkv={nkv} hd={hd} n={n} n_ctx={n_ctx}")
    rng = np.random.default_rng(n)
    pos = rng.choice(n_ctx, size=n, replace=False).astype(np.int32)  # unsorted, gaps
    q = synth.gen_normal(91, "q", (n, nh * hd), std=0.6, device=dev)
    kr = synth.gen_normal(92, "k", (n_ctx, nkv * hd), std=0.6, device=dev)
    vr = synth.gen_normal(93, "v", (n_ctx, nkv * hd), device=dev)
    out = B.attention_gqa(q, kr, vr, torch.as_tensor(pos, device=dev), int(pos.max()), nh, nkv, hd)
    want = ops.attention_gqa(q.cpu().numpy(), kr.cpu().numpy(), vr.cpu().numpy(), pos, nh, nkv, hd)
    assert_f32_match(out.cpu().numpy(), want, what="attention")


def _random_attention_cases(n_cases, seed):
    """Seeded random attention calls: head layouts with GQA groups of 1 to 12, head_dim 64 or 128, 1 to
    300 queries over regions of up to 2000 rows, positions either a contiguous run at a random offset
    or a random unsorted subset with gaps."""
    rng = np.random.default_rng(seed)
    layouts = [(14, 2), (28, 4), (32, 8), (16, 16), (12, 1), (8, 2)]
    cases = []
    for _ in range(n_cases):
        nh, nkv = layouts[int(rng.integers(len(layouts)))]
        hd = int(rng.choice([64, 128]))
        n = int(rng.integers(1, 301))
        n_ctx = int(rng.integers(n, 2001))
        contiguous = bool(rng.integers(2))
        cases.append((nh, nkv, hd, n, n_ctx, contiguous, int(rng.integers(1 << 30))))
    return cases


RANDOM_ATTENTION_CASES = _random_attention_cases(12, 20261205)


@pytest.mark.parametrize("nh,nkv,hd,n,n_ctx,contiguous,seed", RANDOM_ATTENTION_CASES,
                         ids=[f"h{c[0]}_{c[1]}_d{c[2]}_n{c[3]}_ctx{c[4]}_{'run' if c[5] else 'set'}"
                              for c in RANDOM_ATTENTION_CASES])
def test_attention_random_calls_match_oracle(nh, nkv, hd, n, n_ctx, contiguous, seed):
    dev = need_gpu()
    say(f"attention nh={nh} nkv={nkv} hd={hd} n={n} n_ctx={n_ctx} contiguous={contiguous}")
    rng = np.random.default_rng(seed)
    if contiguous:
        pos = (int(rng.integers(0, n_ctx - n + 1)) + np.arange(n)).astype(np.int32)
    else:
        pos = rng.choice(n_ctx, size=n, replace=False).astype(np.int32)
    q = synth.gen_normal(seed % 1000, "q", (n, nh * hd), std=0.6, device=dev)
    kr = synth.gen_normal(seed % 1000 + 1, "k", (n_ctx, nkv * hd), std=0.6, device=dev)
    vr = synth.gen_normal(seed % 1000 + 2, "v", (n_ctx, nkv * hd), device=dev)
    out = B.attention_gqa(q, kr, vr, torch.as_tensor(pos, device=dev), int(pos.max()), nh, nkv, hd)
    want = ops.attention_gqa(q.cpu().numpy(), kr.cpu().numpy(), vr.cpu().numpy(), pos, nh, nkv, hd)
    assert_f32_match(out.cpu().numpy(), want, what="attention")


def test_attention_invariants():
    dev = need_gpu()
    nh, nkv, hd, n = 14, 2, 64, 9
    pos = np.arange(n, dtype=np.int32)
    q = synth.gen_normal(95, "q", (n, nh * hd), device=dev)
    kr = synth.gen_normal(96, "k", (16, nkv * hd), device=dev)
    ones = torch.ones(16, nkv * hd, device=dev)
    out = B.attention_gqa(q, kr, ones, torch.as_tensor(pos, device=dev), n - 1, nh, nkv, hd)
    np.testing.assert_array_equal(out.cpu().numpy(), np.ones((n, nh * hd), f32))   # V = 1 gives 1
    vr = synth.gen_normal(97, "v", (16, nkv * hd), device=dev)
    out = B.attention_gqa(q[:1].contiguous(), kr, vr, torch.as_tensor(pos[:1], device=dev), 0, nh, nkv, hd)
    v0 = vr[0].cpu().numpy()
    for h in range(nh):                                                             # one row gives v_0
        g = h // 7
        np.testing.assert_array_equal(out[0, h * hd:(h + 1) * hd].cpu().numpy(), v0[g * hd:(g + 1) * hd])


def test_lm_head_row_matches_oracle():
    dev = need_gpu()
    # row counts that are and are not multiples of the kernel's 4 rows per wave iteration
    for vocab, hidden in [(8192, 896), (151936, 896), (4000, 4096), (3000, 3584), (1001, 896), (4003, 4096)]:
        say(f"lm_head vocab={vocab} hidden={hidden}")
        w = synth.gen_normal(101, f"o{vocab}", (vocab, hidden), std=0.02, device=dev)
        x = synth.gen_normal(102, f"h{hidden}", (hidden,), std=1.5, device=dev)
        gam = (1 + synth.gen_normal(103, f"g{hidden}", (hidden,), std=0.02, device=dev)).contiguous()
        (wc, ws), (oc, os_) = q8_pair(w)
        logits = B.lm_head_row(x, gam, 1e-6, wc, ws)
        xn = ops.rms_norm(x.cpu().numpy()[None, :], gam.cpu().numpy(), 1e-6)
        want = ops.matmul_q8_0(xn, oc, os_)[0]
        assert_f32_match(logits.cpu().numpy(), want, what=f"logits v={vocab}")

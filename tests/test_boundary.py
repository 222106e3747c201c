"""The C-ABI library loads, exports every declared entry point and rejects
invalid arguments on the host, before any HIP call (runs without a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gnf4.h")

gnf4 = pytest.importorskip("bit_mixture_experts_topk_amd.gnf4")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gnf4.LIB_PATH):
        pytest.fail("libgnf4.so is not built (run python -m bit_mixture_experts_topk_amd.build)")
    return gnf4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gnf4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(gnf4.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_build_id(L):
    bid = gnf4.build_id()
    assert bid.startswith("gnf4 ") and bid.endswith("gfx950")


def test_codebook_matches_oracle(L):
    got = np.array(gnf4.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), nf4.codebook().view(np.uint32))


def _bf16_rne(f32):
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_operand_codebook_is_the_least_squares_scale(L):
    """The NF4 contractions use bf16(s * c[q]) with the absmax divided by s.
    Search every float32 s in [1, 2) from the oracle's codebook: the
    library's s is the one whose operand values, divided by s, deviate least
    from the codebook in mean square, and its 16 values are bf16 of
    fp32(s * c[q])."""
    vals, s_lib = gnf4.nf4_codebook_bf16()
    cb = nf4.codebook().astype(np.float32)
    cb64 = cb.astype(np.float64)
    best_m, best_s = np.inf, None
    one = int(np.float32(1.0).view(np.uint32))
    for start in range(0, 1 << 23, 1 << 20):
        s = (np.arange(start, start + (1 << 20), dtype=np.uint32) + one).view(np.float32)
        r = (_bf16_rne((s[:, None] * cb[None, :]).astype(np.float32)).astype(np.uint32) << 16)
        d = r.view(np.float32).astype(np.float64) / s.astype(np.float64)[:, None] - cb64[None, :]
        m = (d * d).mean(axis=1)
        i = int(np.argmin(m))
        if m[i] < best_m:
            best_m, best_s = float(m[i]), s[i]
    assert np.float32(s_lib) == best_s, (s_lib, best_s)
    assert np.array_equal(np.array(vals, dtype=np.uint16), _bf16_rne(np.float32(s_lib) * cb))
    # the unscaled codebook's mean square is larger by more than 2.5x
    d1 = (_bf16_rne(cb).astype(np.uint32) << 16).view(np.float32).astype(np.float64) - cb64
    assert np.mean(d1 * d1) > 2.5 * best_m


def weights(fmt=0, E=4, N=8, K=64, codes=0x1000, scales=0x2000, scales2=None):
    return gnf4.CWeights(fmt, E, N, K, codes, scales, scales2)


INVALID = 1


@pytest.mark.parametrize("kw,msg", [
    (dict(fmt=7), "unknown format"),
    (dict(E=0), "E = 0"),
    (dict(E=2000), "E = 2000"),
    (dict(N=0), "N = 0"),
    (dict(K=96), "K = 96"),
    (dict(fmt=2, K=48), "K = 48"),
    (dict(codes=0), "NULL"),
    (dict(codes=0x1008), "16-byte"),
    (dict(fmt=1), "scales2"),
])
def test_gemm_rejects_bad_weights(L, kw, msg):
    w = weights(**kw)
    st = L.gnf4_grouped_gemm(ctypes.byref(w), 0x3000, 1, 0x4000, 0x4000, 0x4000, 0x4000, 1, 1,
                             0x5000, None)
    assert st == INVALID and msg in gnf4.last_error()


def test_gemm_rejects_bad_call_args(L):
    w = weights()
    st = L.gnf4_grouped_gemm(ctypes.byref(w), 0x3000, 2, 0x4000, 0x4000, 0x4000, 0x4000, 1, 1, 0x5000, None)
    assert st == INVALID and "gather" in gnf4.last_error()
    st = L.gnf4_grouped_gemm(ctypes.byref(w), 0x3008, 1, 0x4000, 0x4000, 0x4000, 0x4000, 1, 1, 0x5000, None)
    assert st == INVALID and "aligned" in gnf4.last_error()
    st = L.gnf4_grouped_gemm(ctypes.byref(w), None, 1, 0x4000, 0x4000, 0x4000, 0x4000, 1, 1, 0x5000, None)
    assert st == INVALID and "NULL" in gnf4.last_error()
    st = L.gnf4_grouped_gemm(ctypes.byref(w), 0x3000, 1, 0x4000, 0x4000, 0x4000, 0x4000, 1, 65, 0x5000, None)
    assert st == INVALID and "k = 65" in gnf4.last_error()
    st = L.gnf4_grouped_gemm(None, 0x3000, 1, 0x4000, 0x4000, 0x4000, 0x4000, 1, 1, 0x5000, None)
    assert st == INVALID and "descriptor" in gnf4.last_error()


def test_gemm_empty_is_ok(L):
    w = weights()
    assert L.gnf4_grouped_gemm(ctypes.byref(w), None, 1, None, None, None, None, 0, 2, None, None) == 0
    assert gnf4.last_error() == ""


def test_route_rejects(L):
    p = 0x1000
    assert L.gnf4_route(p, 4, 8, 0, p, p, p, p, p, p, p, None, 0, None) == INVALID
    assert "E = 0" in gnf4.last_error()
    assert L.gnf4_route(p, 4, 0, 8, p, p, p, p, p, p, p, None, 0, None) == INVALID
    assert L.gnf4_route(p, -1, 2, 8, p, p, p, p, p, p, p, None, 0, None) == INVALID
    assert L.gnf4_route(None, 4, 2, 8, p, p, p, p, p, p, p, None, 0, None) == INVALID
    assert L.gnf4_route(p, 4, 2, 8, p, None, p, p, p, p, p, None, 0, None) == INVALID


WORKSPACE = 3


def test_route_workspace_bytes(L):
    f = L.gnf4_route_workspace_bytes
    # one workgroup routes up to 1024 assignments: no workspace
    assert f(1, 8, 128) == 0 and f(128, 8, 128) == 0 and f(1024, 1, 1024) == 0
    # above: 4 * (E + 1) bytes per chunk of 1024 assignments, rounded up to 256
    assert f(129, 8, 128) == (2 * 129 * 4 + 255) // 256 * 256
    assert f(4096, 8, 128) == 16640                        # 32 chunks
    assert f(512, 8, 64) == (4 * 65 * 4 + 255) // 256 * 256
    # past 256 chunks the chunks grow (whole 1024-assignment tiles)
    n = (1 << 20) + 77
    chunk = -(-(-(-n // 256)) // 1024) * 1024
    assert f(n, 1, 4) == (-(-n // chunk) * 5 * 4 + 255) // 256 * 256
    assert f(-1, 8, 128) == 0 and f(4, 0, 8) == 0 and f(4, 2, 0) == 0 and f(4, 2, 2000) == 0


def test_route_workspace_too_small(L):
    p = 0x1000
    need = L.gnf4_route_workspace_bytes(4096, 8, 128)
    assert L.gnf4_route(p, 4096, 8, 128, p, p, p, p, p, p, p, p, need - 1, None) == WORKSPACE
    assert "workspace" in gnf4.last_error()
    assert L.gnf4_route(p, 4096, 8, 128, p, p, p, p, p, p, p, None, need, None) == INVALID
    assert L.gnf4_route(p, 4096, 8, 128, p, p, p, p, p, p, p, p + 4, need, None) == INVALID
    assert L.gnf4_route_logits(p, 4096, 8, 128, p, p, p, p, p, p, p, p, p, p, 0, None) == WORKSPACE
    w = weights(E=128)
    assert L.gnf4_route_grouped_gemm(p, 4096, 8, p, p, p, p, p, p, p, p, need - 16,
                                     ctypes.byref(w), p, p, None, None) == WORKSPACE
    assert L.gnf4_route_logits_grouped_gemm(p, 4096, 8, p, p, p, p, p, p, p, p, p, None, 0,
                                            ctypes.byref(w), p, p, None, None) == WORKSPACE


def test_route_logits_rejects(L):
    p = 0x1000
    ok_args = [p, 4, 2, 8, p, p, p, p, p, p, p, p, p, None, 0, None]

    def call(**kw):
        a = list(ok_args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.gnf4_route_logits(*a)

    assert call(a3=0) == INVALID and "E = 0" in gnf4.last_error()
    assert call(a2=9) == INVALID and "k = 9" in gnf4.last_error()        # k > E
    assert call(a2=0) == INVALID
    assert call(a2=65, a3=128) == INVALID                                  # k > 64
    assert call(a1=-1) == INVALID
    assert call(a0=None) == INVALID                                        # logits
    assert call(a5=None) == INVALID                                        # topk_w
    assert call(a7=None) == INVALID                                        # offsets


def test_fused_gemm_rejects(L):
    w = weights()
    p = 0x1000
    assert L.gnf4_grouped_gemm_swiglu(ctypes.byref(w), p, 1, p, p, p, p, 2, 2, None, None) == INVALID
    assert L.gnf4_grouped_gemm_swiglu(ctypes.byref(w), p, 1, p, p, p, p, 2, 2, 0x1001, None) == INVALID
    assert "2-byte aligned" in gnf4.last_error()
    assert L.gnf4_grouped_gemm_swiglu(ctypes.byref(w), p, 2, p, p, p, p, 2, 2, p, None) == INVALID
    odd = weights(N=9)
    assert L.gnf4_grouped_gemm_swiglu(ctypes.byref(odd), p, 1, p, p, p, p, 2, 2, p, None) == INVALID
    assert "even N" in gnf4.last_error()


def test_dequant_experts_bf16_rejects(L):
    w = weights()
    p = 0x1000
    assert L.gnf4_dequant_experts_bf16(ctypes.byref(w), p, p, 5, p, None) == INVALID   # > E
    assert "max_experts = 5" in gnf4.last_error()
    assert L.gnf4_dequant_experts_bf16(ctypes.byref(w), p, p, -1, p, None) == INVALID
    assert L.gnf4_dequant_experts_bf16(ctypes.byref(w), None, p, 2, p, None) == INVALID
    assert L.gnf4_dequant_experts_bf16(ctypes.byref(w), p, p, 2, 0x1008, None) == INVALID
    assert L.gnf4_dequant_experts_bf16(ctypes.byref(w), None, None, 0, None, None) == 0


def test_swiglu_rejects(L):
    p = 0x1000
    assert L.gnf4_swiglu(p, 4, 6, p, None) == INVALID and "I = 6" in gnf4.last_error()
    assert L.gnf4_swiglu(p, 4, 0, p, None) == INVALID
    assert L.gnf4_swiglu(p, -1, 8, p, None) == INVALID
    assert L.gnf4_swiglu(0x1004, 4, 8, p, None) == INVALID                # Y alignment
    assert L.gnf4_swiglu(p, 4, 8, 0x1002, None) == INVALID                # H alignment
    assert L.gnf4_swiglu(None, 4, 8, p, None) == INVALID
    assert L.gnf4_swiglu(None, 0, 8, None, None) == 0                     # nothing to do


def test_combine_rejects(L):
    p = 0x1000
    assert L.gnf4_combine(p, p, p, 2, 2, 6, p, None) == INVALID
    assert L.gnf4_combine(p, p, p, 2, 0, 8, p, None) == INVALID
    assert L.gnf4_combine(0x1004, p, p, 2, 2, 8, p, None) == INVALID
    assert L.gnf4_combine(None, p, p, 2, 2, 8, p, None) == INVALID
    assert L.gnf4_combine(None, None, None, 0, 2, 8, None, None) == 0


def test_dequant_and_quantize_reject(L):
    w = weights()
    assert L.gnf4_dequant(ctypes.byref(w), 4, 0x1000, None) == INVALID
    assert "expert 4" in gnf4.last_error()
    assert L.gnf4_dequant(ctypes.byref(w), 0, None, None) == INVALID
    assert L.gnf4_quantize(0, 0x1000, 4, 100, 0x2000, 0x3000, None, None) == INVALID
    assert L.gnf4_quantize(1, 0x1000, 4, 64, 0x2000, 0x3000, None, None) == INVALID
    assert L.gnf4_quantize(5, 0x1000, 4, 64, 0x2000, 0x3000, None, None) == INVALID
    assert L.gnf4_quantize(0, 0x1000, 4, 64, 0x2008, 0x3000, None, None) == INVALID
    assert L.gnf4_quantize(0, None, 0, 64, None, None, None, None) == 0


def test_gemm_dx_rejects(L):
    w = weights()                      # N = 8
    p = 0x1000
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(w), None, p, 2, 2, p, None) == INVALID
    assert "NULL" in gnf4.last_error()
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(w), p, p, 2, 2, 0x1004, None) == INVALID
    assert "16-byte" in gnf4.last_error()
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(w), 0x1008, p, 2, 2, p, None) == INVALID
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(w), p, p, 2, 0, p, None) == INVALID
    assert "k = 0" in gnf4.last_error()
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(w), p, p, -1, 2, p, None) == INVALID
    ragged = weights(N=60)
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(ragged), p, p, 2, 2, p, None) == INVALID
    assert "multiple of 8" in gnf4.last_error()
    assert L.gnf4_grouped_gemm_dx(None, p, p, 2, 2, p, None) == INVALID
    bad = weights(fmt=2, K=48)
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(bad), p, p, 2, 2, p, None) == INVALID
    big = weights(N=65536, K=64)
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(big), p, p, 16384, 2, p, None) == 2        # 4 GiB dY
    assert "4 GiB" in gnf4.last_error()
    assert L.gnf4_grouped_gemm_dx(ctypes.byref(w), None, None, 0, 2, None, None) == 0      # T = 0


def test_route_grouped_gemm_rejects(L):
    w = weights()
    p = 0x1000

    def call(T=1, k=2, ids=p, Y=p, H=None, counts=p, wt=None):
        return L.gnf4_route_grouped_gemm(ids, T, k, counts, p, p, p, p, p, p, None, 0,
                                         ctypes.byref(wt or w), p, Y, H, None)

    assert call(k=0) == INVALID and "k = 0" in gnf4.last_error()
    assert call(k=65) == INVALID
    assert call(T=-1) == INVALID
    assert call(Y=p, H=p) == INVALID and "exactly one" in gnf4.last_error()
    assert call(Y=None, H=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(counts=None) == INVALID
    assert call(wt=weights(E=0)) == INVALID and "E = 0" in gnf4.last_error()


def test_grouped_gemm_combine_rejects(L):
    w = weights()                      # N = 8
    p = 0x1000

    def call(T=1, k=2, X=p, out=p, wt=None, tw=p):
        return L.gnf4_grouped_gemm_combine(ctypes.byref(wt or w), X, p, p, p, p, p, tw, T, k,
                                           None, out, None)

    assert call(k=0) == INVALID
    assert call(T=-1) == INVALID
    assert call(wt=weights(N=6)) == INVALID and "multiple of 4" in gnf4.last_error()
    assert call(out=None) == INVALID and "NULL" in gnf4.last_error()
    assert call(tw=None) == INVALID
    assert call(X=0x1004) == INVALID and "16-byte" in gnf4.last_error()
    assert call(out=0x1008) == INVALID
    assert call(T=0, X=None, out=None) == 0                # nothing to do


def test_expert_cache_sizes(L):
    assert L.gnf4_expert_cache_state_words(64, 16) == 1 + 64 + 32
    assert L.gnf4_expert_cache_state_words(8, 9) == 0                 # S > E
    assert L.gnf4_expert_cache_state_words(0, 1) == 0
    assert L.gnf4_expert_cache_copies_words(1, 8, 64, 16) == 17      # min(8, 64, 16) pairs
    assert L.gnf4_expert_cache_copies_words(4, 8, 64, 16) == 33      # min(32, 64, 16)
    assert L.gnf4_expert_cache_copies_words(0, 8, 64, 16) == 1


def test_expert_cache_stage_rejects(L):
    p = 0x1000

    def call(T=1, k=8, E=64, S=16, ids=p, state=p, slot_ids=p, copies=p):
        return L.gnf4_expert_cache_stage(ids, T, k, E, S, state, slot_ids, copies, None)

    assert call(S=0) == INVALID and "S = 0" in gnf4.last_error()
    assert call(S=65) == INVALID
    assert call(E=2000, S=16) == INVALID
    assert call(k=0) == INVALID
    assert call(T=-1) == INVALID
    assert call(state=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(S=7) == 2 and "distinct" in gnf4.last_error()        # 8 ids may need 8 slots
    assert call(T=3, k=8, E=20, S=19) == 2                             # min(E, T*k) = 20
    assert L.gnf4_expert_cache_reset(None, 64, 16, None) == INVALID
    assert L.gnf4_expert_cache_reset(p, 64, 65, None) == INVALID


def test_expert_cache_fill_rejects(L):
    host = weights(E=8, N=16, K=64)
    cache = weights(E=4, N=16, K=64, codes=0x3000, scales=0x4000)

    def call(h=None, c=None, copies=0x5000, m=2):
        return L.gnf4_expert_cache_fill(ctypes.byref(h or host), ctypes.byref(c or cache), copies, m,
                                        None)

    assert call(c=weights(fmt=2, E=4, N=16, K=64)) == INVALID and "differ" in gnf4.last_error()
    assert call(c=weights(E=4, N=8, K=64)) == INVALID
    assert call(c=weights(E=9, N=16, K=64)) == INVALID and "slots" in gnf4.last_error()
    assert call(m=5) == INVALID and "max_copies" in gnf4.last_error()
    assert call(m=-1) == INVALID
    assert call(copies=None) == INVALID
    # NF4 scales of one expert: 16 rows x 1 block x 4 B = 64 B; N = 3 gives 12 B
    assert call(h=weights(E=8, N=3, K=64), c=weights(E=4, N=3, K=64, codes=0x3000,
                                                      scales=0x4000)) == 2
    assert "multiple of 16" in gnf4.last_error()
    # NF4_DQ: 16 x 1 blocks per expert is not a whole group of 256
    dq = dict(fmt=1, E=8, N=16, K=64, scales2=0x6000)
    assert call(h=weights(**dq), c=weights(**dict(dq, E=4, codes=0x3000, scales=0x4000,
                                                  scales2=0x7000))) == 2
    assert "multiple of 256" in gnf4.last_error()
    assert call(c=weights(E=4, N=16, K=64, codes=0x3000, scales=0x4004)) == INVALID
    assert call(m=0) == 0                                              # nothing to copy


def test_read_probe_rejects(L):
    p = 0x1000
    assert L.gnf4_read_probe(None, 0, 0, None, None) == 0                 # nothing to read
    assert L.gnf4_read_probe(None, 64, 0, p, None) == INVALID
    assert L.gnf4_read_probe(p, 64, 0, None, None) == INVALID
    assert L.gnf4_read_probe(p + 8, 64, 0, p, None) == INVALID            # misaligned
    assert L.gnf4_read_probe(p, 72, 0, p, None) == INVALID                # not whole 16 B
    assert L.gnf4_read_probe(p, 64, -1, p, None) == INVALID


def test_route_noalloc_rejects(L):
    """Host validation of the static-workspace route, before any HIP call:
    the usual argument checks, and a workspace need beyond its 1 MiB array."""
    p = 0x1000
    assert L.gnf4_route_noalloc(p, 4, 2, 0, p, p, p, p, p, p, p, None) == INVALID
    assert L.gnf4_route_noalloc(p, 4, 65, 128, p, p, p, p, p, p, p, None) == INVALID
    assert L.gnf4_route_noalloc(p, -1, 2, 8, p, p, p, p, p, p, p, None) == INVALID
    assert L.gnf4_route_noalloc(None, 4, 2, 8, p, p, p, p, p, p, p, None) == INVALID
    assert L.gnf4_route_noalloc(p, 4, 2, 8, p, p, None, p, p, p, p, None) == INVALID
    T = 261120 // 64 + 1                  # E = 1024: 256 chunks of 1025 words > 1 MiB
    assert L.gnf4_route_workspace_bytes(T, 64, 1024) > (1 << 20)
    assert L.gnf4_route_noalloc(p, T, 64, 1024, p, p, p, p, p, p, p, None) == WORKSPACE
    assert "static" in gnf4.last_error()

"""C-ABI checks that need no GPU: the library loads, exports every function the header declares,
and rejects bad arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest
import torch

import transformer_layer_forward_amd as L
from transformer_layer_forward_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llama_layer.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


def test_header_declares_the_six_layer_entry_points():
    names = _declared_functions()
    for n in ("llama_layer_forward", "rmsnorm", "rope_apply", "gqa_attn_prefill", "gqa_attn_decode", "swiglu_mlp"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    assert set(_lib.EXPORTED) == set(_declared_functions())


def test_library_resolves_all_of_its_own_symbols():
    """Every kernel the host code launches has its host-side stub in the library: no symbol of the
    library's own namespace is left undefined (a missing stub would only fail when the library loads)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    own = [l for l in out.splitlines() if "_ZN2ll" in l]
    assert not own, own[:5]


def test_struct_layouts_match_header():
    # ll_rope: 2 x int32 + 4 x double + int64; ll_layer_cfg: 5 x int64 + double + ll_rope + 2 x int32
    assert ctypes.sizeof(_lib.LLRope) == 48
    assert ctypes.sizeof(_lib.LLLayerCfg) == 104
    assert ctypes.sizeof(_lib.LLLayerWeights) == 48


def _cfg(**kw):
    base = dict(hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=176, dtype=torch.float32)
    base.update(kw)
    return L.LayerConfig(**base).to_c()


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("field,value,status", [
    ("n_heads", 5, _lib.LL_EINVAL),          # not a multiple of n_kv_heads
    ("head_dim", 15, _lib.LL_EINVAL),        # odd
    ("head_dim", 258, _lib.LL_EUNSUPPORTED),
    ("hidden", 0, _lib.LL_EINVAL),
    ("intermediate", -3, _lib.LL_EINVAL),
    ("eps", -1.0, _lib.LL_EINVAL),
    ("dtype", 7, _lib.LL_EINVAL),
    ("reserved", 1, _lib.LL_EINVAL),
])
def test_layer_config_validation(field, value, status):
    lib = L.load()
    c = _cfg()
    setattr(c, field, value)
    w = _lib.LLLayerWeights(*([FAKE.value] * 6))
    st = lib.llama_layer_forward(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 1, 32, 32, None, None, 0, FAKE, FAKE,
                                 1 << 30, None)
    assert st == status, L.last_error()
    assert L.last_error()
    assert lib.llama_layer_workspace_bytes(ctypes.byref(c), 1, 32, 0) == 0


def test_bf16_needs_multiples_of_8():
    lib = L.load()
    c = _cfg(dtype=torch.bfloat16, hidden=60)
    w = _lib.LLLayerWeights(*([FAKE.value] * 6))
    st = lib.llama_layer_forward(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 1, 32, 32, None, None, 0, FAKE, FAKE,
                                 1 << 30, None)
    assert st == _lib.LL_EUNSUPPORTED


@pytest.mark.parametrize("rope_kw", [dict(type="llama3", low_freq_factor=4.0, high_freq_factor=1.0),
                                     dict(type="linear", factor=0.0),
                                     dict(theta=-1.0),
                                     dict(type="dynamic_ntk", original_max_pos=0)])
def test_rope_validation(rope_kw):
    lib = L.load()
    c = _cfg(rope=L.Rope(**rope_kw))
    w = _lib.LLLayerWeights(*([FAKE.value] * 6))
    st = lib.llama_layer_forward(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 1, 32, 32, None, None, 0, FAKE, FAKE,
                                 1 << 30, None)
    assert st == _lib.LL_EINVAL


def test_layer_argument_errors():
    lib = L.load()
    c = _cfg()
    w = _lib.LLLayerWeights(*([FAKE.value] * 6))
    ws = lib.llama_layer_workspace_bytes(ctypes.byref(c), 1, 32, 0)
    assert ws > 0

    def call(**kw):
        a = dict(w=ctypes.byref(w), hidden=FAKE, pos=FAKE, B=1, S=32, L=32, kc=None, vc=None, ctx=0, out=FAKE,
                 ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.llama_layer_forward(ctypes.byref(c), a["w"], a["hidden"], a["pos"], a["B"], a["S"], a["L"], a["kc"],
                                       a["vc"], a["ctx"], a["out"], a["ws"], a["wsb"], None)

    assert call(w=None) == _lib.LL_EINVAL
    assert call(hidden=None) == _lib.LL_EINVAL
    assert call(pos=None) == _lib.LL_EINVAL
    assert call(L=0) == _lib.LL_EINVAL
    assert call(wsb=ws - 1) == _lib.LL_EINVAL
    assert call(kc=FAKE) == _lib.LL_EINVAL                       # only one cache
    assert call(kc=FAKE, vc=FAKE, ctx=0) == _lib.LL_EINVAL      # caches without ctx
    assert call(hidden=ctypes.c_void_p(0x10002)) == _lib.LL_EINVAL  # misaligned
    assert call(B=-1) == _lib.LL_EINVAL
    assert call(B=0) == _lib.LL_OK and call(S=0) == _lib.LL_OK   # empty batch: nothing to do
    bad = _lib.LLLayerWeights(FAKE.value, None, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    assert call(w=ctypes.byref(bad)) == _lib.LL_EINVAL


def test_noalloc_entry_point_checks_before_any_hip_call():
    """llama_layer_forward_noalloc validates like llama_layer_forward and refuses a call whose workspace plus
    RoPE table exceeds its 64 MiB static scratch, all before touching the device."""
    lib = L.load()
    w = _lib.LLLayerWeights(*([FAKE.value] * 6))
    c8 = L.LayerConfig(4096, 32, 8, 128, 14336, dtype=torch.bfloat16).to_c()

    def call(c, B, S, L_, kc=None, vc=None, ctx=0, hidden=FAKE):
        return lib.llama_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(w), hidden, FAKE, B, S, L_, kc, vc, ctx,
                                               FAKE, None)

    assert call(c8, 1, 4096, 4096) == _lib.LL_EINVAL            # 256 MiB of workspace
    assert "static scratch" in L.last_error()
    assert call(c8, 64, 1, 1 << 24, FAKE, FAKE, 1 << 24) == _lib.LL_EINVAL   # a 8 GiB RoPE table
    assert call(c8, 1, 300, 300, hidden=None) == _lib.LL_EINVAL
    assert call(c8, 0, 1, 300) == _lib.LL_OK
    bad = _cfg(head_dim=15)
    assert call(bad, 1, 8, 8) == _lib.LL_EINVAL


def test_kernel_entry_point_errors():
    lib = L.load()
    assert lib.rmsnorm(None, None, None, 4, 64, 1e-5, _lib.LL_BF16, None) == _lib.LL_EINVAL
    assert lib.rmsnorm(FAKE, FAKE, FAKE, 4, 0, 1e-5, _lib.LL_BF16, None) == _lib.LL_EINVAL
    assert lib.rmsnorm(FAKE, FAKE, FAKE, 0, 64, 1e-5, _lib.LL_BF16, None) == _lib.LL_OK
    r = L.Rope().to_c()
    assert lib.rope_apply(None, FAKE, FAKE, 1, 4, 4, 2, 16, 4, _lib.LL_BF16, None) == _lib.LL_EINVAL
    assert lib.rope_apply(ctypes.byref(r), FAKE, FAKE, 1, 4, 4, 2, 15, 4, _lib.LL_BF16, None) == _lib.LL_EINVAL
    assert lib.rope_apply(ctypes.byref(r), FAKE, FAKE, 1, 4, 4, 2, 16, 0, _lib.LL_BF16, None) == _lib.LL_EINVAL
    assert lib.gqa_attn_prefill(FAKE, ctypes.byref(r), None, 8, FAKE, None, None, 0, 1, 4, 4, 2, 64, _lib.LL_BF16,
                                None) == _lib.LL_EINVAL                     # rope without positions
    assert lib.gqa_attn_prefill(FAKE, None, None, 0, FAKE, FAKE, None, 8, 1, 4, 4, 2, 64, _lib.LL_BF16,
                                None) == _lib.LL_EINVAL                     # one cache only
    assert lib.gqa_attn_prefill(FAKE, None, None, 0, FAKE, None, None, 0, 1, 4, 3, 2, 64, _lib.LL_BF16,
                                None) == _lib.LL_EINVAL                     # 3 % 2
    need = lib.gqa_attn_decode_workspace_bytes(2, 4, 64, 1024)
    assert need > 0
    assert lib.gqa_attn_decode(FAKE, None, FAKE, 0, FAKE, FAKE, 1024, FAKE, 2, 4, 2, 64, _lib.LL_BF16, FAKE, need - 1,
                               None) == _lib.LL_EINVAL
    assert lib.gqa_attn_decode(FAKE, None, FAKE, 0, None, None, 1024, FAKE, 2, 4, 2, 64, _lib.LL_BF16, FAKE, need,
                               None) == _lib.LL_EINVAL
    mneed = lib.swiglu_mlp_workspace_bytes(8, 64, 128, _lib.LL_BF16)
    assert lib.swiglu_mlp(FAKE, FAKE, FAKE, None, FAKE, 8, 64, 128, _lib.LL_BF16, FAKE, mneed - 1,
                          None) == _lib.LL_EINVAL
    assert lib.swiglu_mlp(FAKE, FAKE, FAKE, None, FAKE, 8, 60, 128, _lib.LL_BF16, FAKE, mneed,
                          None) == _lib.LL_EUNSUPPORTED
    # out aliasing x is rejected
    assert lib.swiglu_mlp(FAKE, FAKE, FAKE, None, FAKE, 8, 64, 128, _lib.LL_BF16, FAKE, mneed, None) == _lib.LL_EINVAL
    # a workspace off 16-byte alignment is rejected (the projections use 16-byte vector accesses on it)
    other = ctypes.c_void_p(FAKE.value + 4096)
    assert lib.swiglu_mlp(FAKE, FAKE, FAKE, None, other, 8, 64, 128, _lib.LL_BF16,
                          ctypes.c_void_p(FAKE.value + 8192 + 8), mneed, None) == _lib.LL_EINVAL
    assert "aligned" in _lib.last_error()


def test_profile_stage_names():
    lib = L.load()
    names = [lib.ll_profile_stage_name(i).decode() for i in range(7)]
    assert names == ["rmsnorm_attn", "qkv_proj", "attention", "o_proj_residual", "rmsnorm_mlp", "gate_up_silu",
                     "down_residual"]
    assert lib.ll_profile_stage_name(7) == b""


def test_profile_stage_mask_is_validated_before_any_event():
    lib = L.load()
    assert lib.ll_profile_begin_stages(0, 0) == _lib.LL_EINVAL
    assert lib.ll_profile_begin_stages(0, 1 << 7) == _lib.LL_EINVAL
    assert lib.ll_profile_begin_stages(-1, 1) == _lib.LL_EINVAL
    with pytest.raises(ValueError):
        L.profile_begin(0, stages=["no_such_stage"])
    # a valid mask with no reserved events touches no device; ending with no calls timed reports nothing
    assert lib.ll_profile_begin_stages(0, 1 << 5) == _lib.LL_OK
    assert L.profile_end() == {}


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The binding and library sources never reference the oracle or a CPU implementation."""
    pkg = os.path.join(ROOT, "transformer_layer_forward_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "numpy" not in text or f == "build.py", f


def test_workspace_sizes_follow_the_projection_plans():
    """Host-only sizing: a projection with few output tiles splits K and needs fp32 partials beyond the
    activation buffer; one with enough tiles needs none; the key-split area of chunked attention
    appears only when the caller passes the cache length."""
    lib = _lib.load()

    def act(m, i):
        return (m * i * 2 + 255) // 256 * 256

    # M = 256 tokens, Llama-3-8B MLP: down (N = 4096, K = 14336) has 16 tiles of 256 x 256 -> partials
    few = lib.swiglu_mlp_workspace_bytes(256, 4096, 14336, 1)
    assert few > act(256, 14336)
    # M = 8192: every projection has >= 256 tiles -> the activation buffer alone
    assert lib.swiglu_mlp_workspace_bytes(8192, 4096, 14336, 1) == act(8192, 14336)
    # decode-sized M = 64: the down projection streams its weights in K ranges -> partials
    assert lib.swiglu_mlp_workspace_bytes(64, 4096, 14336, 1) > act(64, 14336)
    # fp32 runs its own kernel, no partials
    assert lib.swiglu_mlp_workspace_bytes(256, 4096, 14336, 0) == (256 * 14336 * 4 + 255) // 256 * 256
    cfg = L.LayerConfig(4096, 32, 8, 128, 14336, 1e-5, L.Rope(), torch.bfloat16).to_c()
    no_cache = lib.llama_layer_workspace_bytes(ctypes.byref(cfg), 1, 256, 0)
    with_cache = lib.llama_layer_workspace_bytes(ctypes.byref(cfg), 1, 256, 8192)
    assert with_cache > no_cache > 0

"""The C ABI on the CPU: the library loads, exports what the header declares,
and rejects bad arguments before any HIP call (so these run without a GPU).

Pointers handed to rejected calls are fake (never dereferenced): validation
must fail before a single byte of device memory is touched.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from chunked_prefill_causal_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "chunkattn.h")
FAKE = 1 << 20          # 16-byte aligned, never dereferenced
MISALIGNED = FAKE + 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(L.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_defaults():
    assert L.version() == 3
    o = L.PrefillOpts()
    o.num_splits = 7
    L.lib().ca_prefill_opts_init(ctypes.byref(o))
    assert (o.dtype, o.out_dtype, o.kv_layout, o.num_splits, o.head_dim_v) == (L.CA_BF16, L.CA_BF16,
                                                                                L.CA_KV_CONTIGUOUS, 0, 0)
    assert ctypes.sizeof(L.PrefillOpts) == 104


def test_options_struct_matches_the_header(tmp_path):
    """The ctypes mirror of ca_prefill_opts has the size and field offsets the C header gives."""
    fields = [f for f, _ in L.PrefillOpts._fields_]
    src = tmp_path / "probe.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "chunkattn.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(ca_prefill_opts));\n'
                   + "".join(f'  printf(" %zu", offsetof(ca_prefill_opts, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(L.PrefillOpts)
    assert got[1:] == [getattr(L.PrefillOpts, f).offset for f in fields]


def prefill(q=FAKE, k=FAKE, v=FAKE, past=0, c=4, hq=8, hkv=8, d=128, scale=0.1, out=FAKE, opts=None):
    return L.lib().chunk_prefill_attn(q, k, v, past, c, hq, hkv, d, scale, out,
                                      None if opts is None else ctypes.byref(opts), None)


def opts(**kw):
    o = L.PrefillOpts()
    L.lib().ca_prefill_opts_init(ctypes.byref(o))
    for key, val in kw.items():
        setattr(o, key, val)
    return o


@pytest.mark.parametrize("kwargs,status", [
    (dict(k=None), L.CA_EINVAL),
    (dict(q=None), L.CA_EINVAL),
    (dict(q=MISALIGNED), L.CA_EINVAL),
    (dict(past=-1), L.CA_EINVAL),
    (dict(c=-5), L.CA_EINVAL),
    (dict(hq=8, hkv=3), L.CA_EINVAL),
    (dict(hkv=0), L.CA_EINVAL),
    (dict(scale=0.0), L.CA_EINVAL),
    (dict(scale=float("inf")), L.CA_EINVAL),
    (dict(scale=float("nan")), L.CA_EINVAL),
    (dict(d=96), L.CA_EUNSUPPORTED),
    (dict(d=192), L.CA_EUNSUPPORTED),                                   # needs head_dim_v = 128
    (dict(opts=opts(dtype=L.CA_F32, out_dtype=L.CA_BF16)), L.CA_EUNSUPPORTED),
    (dict(opts=opts(dtype=7)), L.CA_EINVAL),
    (dict(opts=opts(kv_layout=9)), L.CA_EINVAL),
    (dict(opts=opts(kv_capacity=3)), L.CA_ERANGE),
    (dict(opts=opts(k_stride_tok=1028)), L.CA_EINVAL),                   # not a 16-byte multiple (bf16)
    (dict(opts=opts(v_stride_head=-8)), L.CA_EINVAL),
    (dict(opts=opts(dtype=L.CA_F32, out_dtype=L.CA_F32, k_stride_head=130)), L.CA_EINVAL),
    (dict(opts=opts(kv_layout=L.CA_KV_PAGED, block_table=FAKE, block_table_len=1, num_blocks=4,
                    k_stride_tok=2048)), L.CA_EINVAL),                   # strides are contiguous-only
    (dict(past=(1 << 30), c=1), L.CA_ERANGE),
    (dict(opts=opts(kv_layout=L.CA_KV_PAGED)), L.CA_EINVAL),            # no block table
    (dict(opts=opts(kv_layout=L.CA_KV_PAGED, block_table=FAKE, block_table_len=1, num_blocks=4), past=61),
     L.CA_ERANGE),                                                       # 65 tokens, 1 block
    (dict(opts=opts(kv_layout=L.CA_KV_PAGED, block_table=FAKE, block_table_len=1, num_blocks=0)),
     L.CA_EINVAL),
    (dict(opts=opts(num_splits=-1)), L.CA_EINVAL),
    (dict(opts=opts(num_splits=4), past=1000, c=24), L.CA_EWORKSPACE),  # no workspace given
    (dict(opts=opts(num_splits=4, workspace=FAKE, workspace_bytes=16), past=1000, c=24), L.CA_EWORKSPACE),
    (dict(opts=opts(lse_out=FAKE + 2)), L.CA_EINVAL),
])
def test_prefill_rejections(kwargs, status):
    assert prefill(**kwargs) == status
    assert L.lib().chunkattn_last_error().decode()


def test_zero_length_chunk_succeeds_without_touching_memory():
    assert prefill(q=None, out=None, c=0) == L.CA_OK
    assert L.lib().chunkattn_last_error().decode() == ""


def test_workspace_queries():
    assert L.chunkattn_prefill_workspace_size(100, 8, 128, 1) == 0
    need = L.chunkattn_prefill_workspace_size(100, 8, 128, 3)
    assert need >= 3 * 100 * 8 * (128 + 2) * 4
    assert L.chunkattn_prefill_auto_splits(0, 16384, 64, 8) == 1        # big chunk: no split
    assert L.chunkattn_prefill_auto_splits(100000, 64, 8, 2) > 1         # short chunk, long prefix
    assert L.chunkattn_prefill_auto_splits(-1, 4, 8, 8) == 0
    assert L.chunkattn_varlen_workspace_size([0, 1, 3], [100, 50], 8, 2, 128) > 0


def varlen(q=FAKE, cu=(0, 1, 2), kv=(10, 20), hq=8, hkv=2, d=128, dv=128, ws=FAKE, ws_bytes=1 << 30,
           max_blocks=4, num_blocks=8, scale=0.1, out=FAKE, k=FAKE, out_dtype=L.CA_BF16):
    cu_a = (ctypes.c_int32 * len(cu))(*cu)
    kv_a = (ctypes.c_int32 * len(kv))(*kv)
    return L.lib().chunk_attn_varlen(q, k, FAKE, FAKE, max_blocks, num_blocks, FAKE, FAKE,
                                     ctypes.addressof(cu_a), ctypes.addressof(kv_a), len(kv), hq, hkv, d, dv,
                                     scale, out, out_dtype, None, ws, ws_bytes, None)


def test_contiguous_workspace_query():
    """Re-layout room for a bf16 contiguous cache: an identity block table (256-byte aligned) plus
    K and V pools of ceil(kv_len / 64) blocks, then the split partials."""
    past, c, hq, hkv, d = 1000, 100, 8, 2, 128
    blocks = -(-(past + c) // 64)
    relay = -(-blocks * 4 // 256) * 256 + blocks * hkv * (d + d) * 64 * 2
    assert L.chunkattn_prefill_contiguous_workspace_size(past, c, hq, hkv, d, d, 1) == relay
    assert (L.chunkattn_prefill_contiguous_workspace_size(past, c, hq, hkv, d, d, 3)
            == relay + L.chunkattn_prefill_workspace_size(c, hq, d, 3))
    # head-dim pairs the paged kernel does not take get no re-layout room
    assert L.chunkattn_prefill_contiguous_workspace_size(past, c, hq, hkv, 96, 96, 1) == 0
    assert L.chunkattn_prefill_contiguous_workspace_size(past, 0, hq, hkv, d, d, 1) == 0
    assert L.chunkattn_prefill_contiguous_workspace_size(past, c, 8, 3, d, d, 1) == 0
    # fp32 caches are read in place: split partials only
    assert L.chunkattn_prefill_contiguous_workspace_size(past, c, hq, hkv, d, d, 1, L.CA_F32) == 0
    assert (L.chunkattn_prefill_contiguous_workspace_size(past, c, hq, hkv, d, d, 3, L.CA_F32)
            == L.chunkattn_prefill_workspace_size(c, hq, d, 3))


@pytest.mark.parametrize("kwargs,status", [
    (dict(k=None), L.CA_EINVAL),
    (dict(q=None), L.CA_EINVAL),
    (dict(cu=(1, 2, 3)), L.CA_EINVAL),                 # cu[0] != 0
    (dict(cu=(0, 2, 1)), L.CA_EINVAL),                 # decreasing
    (dict(kv=(0, 20)), L.CA_EINVAL),                   # kv_len below q_len
    (dict(kv=(10, 300)), L.CA_ERANGE),                 # 300 tokens > 4 blocks of 64
    (dict(hq=8, hkv=3), L.CA_EINVAL),
    (dict(d=128, dv=64), L.CA_EUNSUPPORTED),
    (dict(ws=None), L.CA_EWORKSPACE),
    (dict(ws_bytes=64), L.CA_EWORKSPACE),
    (dict(ws=FAKE + 16), L.CA_EINVAL),                 # workspace must be 256-byte aligned
    (dict(scale=-1.0), L.CA_EINVAL),
    (dict(max_blocks=0), L.CA_EINVAL),
    (dict(out_dtype=7), L.CA_EINVAL),
])
def test_varlen_rejections(kwargs, status):
    assert varlen(**kwargs) == status


def varlen_noalloc(q=FAKE, cu=(0, 1, 2), kv=(10, 20), hq=8, hkv=2, d=128, dv=128, max_blocks=4, num_blocks=8,
                   scale=0.1, out=FAKE, k=FAKE, out_dtype=L.CA_BF16):
    cu_a = (ctypes.c_int32 * len(cu))(*cu)
    kv_a = (ctypes.c_int32 * len(kv))(*kv)
    return L.lib().chunk_attn_varlen_noalloc(q, k, FAKE, FAKE, max_blocks, num_blocks, FAKE, FAKE,
                                             ctypes.addressof(cu_a), ctypes.addressof(kv_a), len(kv), hq, hkv, d, dv,
                                             scale, out, out_dtype, None, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(k=None), L.CA_EINVAL),
    (dict(cu=(0, 2, 1)), L.CA_EINVAL),
    (dict(kv=(10, 300)), L.CA_ERANGE),
    (dict(d=128, dv=64), L.CA_EUNSUPPORTED),
    (dict(scale=float("nan")), L.CA_EINVAL),
    (dict(out_dtype=-1), L.CA_EINVAL),
])
def test_varlen_noalloc_rejections(kwargs, status):
    """The allocation-free varlen entry validates like chunk_attn_varlen, before any HIP call."""
    assert varlen_noalloc(**kwargs) == status


def test_varlen_noalloc_rejects_batches_beyond_its_scratch():
    """A batch whose partials exceed the static scratch fails with CA_EWORKSPACE before any HIP call;
    the same batch sized just under the limit is accepted by the size query."""
    n = 4096
    cu = tuple(range(n + 1))
    kv = (65536,) * n
    need = L.chunkattn_varlen_workspace_size(cu, kv, 32, 8, 128)
    assert need > L.NOALLOC_SCRATCH_BYTES
    assert varlen_noalloc(cu=cu, kv=kv, hq=32, hkv=8, max_blocks=1024, num_blocks=1 << 20) == L.CA_EWORKSPACE
    assert b"allocation-free" in L.lib().chunkattn_last_error()


def test_varlen_noalloc_empty_batch_succeeds():
    assert varlen_noalloc(q=None, out=None, cu=(0, 0, 0), kv=(5, 9)) == L.CA_OK


def test_varlen_empty_batch_succeeds():
    assert varlen(q=None, out=None, cu=(0, 0, 0), kv=(5, 9), ws=None) == L.CA_OK


def test_kv_append_rejections():
    lib = L.lib()
    f = lambda **kw: lib.chunkattn_kv_append(kw.get("k", FAKE), FAKE, kw.get("start", 0), kw.get("n", 10), 2,
                                             kw.get("d", 128), 128, kw.get("dt", L.CA_BF16), FAKE,
                                             kw.get("tl", 1), 4, FAKE, FAKE, kw.get("st"), None)
    strides = lambda *v: (ctypes.c_int64 * 4)(*v)
    assert f(k=None) == L.CA_EINVAL
    assert f(start=-1) == L.CA_EINVAL
    assert f(d=100) == L.CA_EUNSUPPORTED
    assert f(dt=5) == L.CA_EINVAL
    assert f(start=60, n=10) == L.CA_ERANGE
    assert f(n=0) == L.CA_OK
    assert f(n=0, st=strides(2048, 128, 2048, 128)) == L.CA_OK
    assert f(st=strides(2048, 128, 2052, 128)) == L.CA_EINVAL        # not a 16-byte multiple
    assert f(st=strides(2048, 0, 2048, 128)) == L.CA_EINVAL


def test_mla_block_bytes_follow_the_per_token_record():
    # 64 tokens per block of 1152 B (bf16) and 656 B (fp8 latent) records
    assert L.chunkattn_mla_block_bytes(L.CA_MLA_BF16) == 64 * 1152
    assert L.chunkattn_mla_block_bytes(L.CA_MLA_FP8) == 64 * 656
    assert L.chunkattn_mla_block_bytes(2) == 0
    assert L.chunkattn_mla_decode_workspace_size([100, 5000], 16, L.CA_MLA_FP8) > 2 * 16 * 512 * 4
    assert L.chunkattn_mla_decode_workspace_size([100], 15, L.CA_MLA_BF16) == 0
    assert L.chunkattn_mla_decode_workspace_size([0], 16, L.CA_MLA_BF16) == 0
    assert L.chunkattn_mla_decode_workspace_size([10], 16, 4) == 0


def mla_decode(q=FAKE, fmt=L.CA_MLA_BF16, kv=(10, 300), heads=16, max_blocks=8, num_blocks=8, scale=0.1,
               out=FAKE, out_dtype=L.CA_BF16, ws=FAKE, ws_bytes=1 << 30, lse=None):
    kv_a = (ctypes.c_int32 * len(kv))(*kv)
    return L.lib().chunk_mla_decode(q, FAKE, fmt, FAKE, max_blocks, num_blocks, FAKE, ctypes.addressof(kv_a),
                                    len(kv), heads, scale, out, out_dtype, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=2), L.CA_EINVAL),
    (dict(heads=8), L.CA_EUNSUPPORTED),
    (dict(heads=2048), L.CA_EUNSUPPORTED),
    (dict(kv=(0, 5)), L.CA_EINVAL),
    (dict(kv=(10, 600)), L.CA_ERANGE),                   # 600 tokens > 8 blocks of 64
    (dict(scale=0.0), L.CA_EINVAL),
    (dict(scale=float("nan")), L.CA_EINVAL),
    (dict(q=None), L.CA_EINVAL),
    (dict(q=MISALIGNED), L.CA_EINVAL),
    (dict(lse=FAKE + 2), L.CA_EINVAL),
    (dict(ws=None), L.CA_EWORKSPACE),
    (dict(ws_bytes=1024), L.CA_EWORKSPACE),
    (dict(ws=FAKE + 16), L.CA_EINVAL),
    (dict(max_blocks=0), L.CA_EINVAL),
    (dict(num_blocks=0), L.CA_EINVAL),
    (dict(out_dtype=5), L.CA_EINVAL),
])
def test_mla_decode_rejections(kwargs, status):
    assert mla_decode(**kwargs) == status
    assert L.lib().chunkattn_last_error().decode()


def test_mla_decode_empty_batch_succeeds():
    assert mla_decode(q=None, out=None, kv=(), ws=None) == L.CA_OK


def mla_prefill(q=FAKE, fmt=L.CA_MLA_BF16, table_len=8, num_blocks=8, past=100, chunk=300, heads=16, scale=0.1,
                out=FAKE, out_dtype=L.CA_BF16, lse=None, ws=None, ws_bytes=0):
    return L.lib().chunk_mla_prefill(q, FAKE, fmt, FAKE, table_len, num_blocks, past, chunk, heads, scale, out,
                                     out_dtype, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=2), L.CA_EINVAL),
    (dict(fmt=L.CA_MLA_FP8), L.CA_EWORKSPACE),           # fp8 widens the prefix into the workspace
    (dict(fmt=L.CA_MLA_FP8, ws=FAKE, ws_bytes=7 * 73728 - 1), L.CA_EWORKSPACE),   # 400 tokens: 7 blocks
    (dict(fmt=L.CA_MLA_FP8, ws=FAKE + 16, ws_bytes=1 << 30), L.CA_EINVAL),
    (dict(heads=8), L.CA_EUNSUPPORTED),
    (dict(heads=2048), L.CA_EUNSUPPORTED),
    (dict(past=-1), L.CA_EINVAL),
    (dict(chunk=-5), L.CA_EINVAL),
    (dict(past=300, chunk=213), L.CA_ERANGE),           # 513 tokens > 8 blocks of 64
    (dict(past=1 << 30, chunk=1), L.CA_ERANGE),
    (dict(scale=0.0), L.CA_EINVAL),
    (dict(scale=float("inf")), L.CA_EINVAL),
    (dict(q=None), L.CA_EINVAL),
    (dict(out=None), L.CA_EINVAL),
    (dict(q=MISALIGNED), L.CA_EINVAL),
    (dict(lse=FAKE + 2), L.CA_EINVAL),
    (dict(num_blocks=0), L.CA_EINVAL),
    (dict(out_dtype=5), L.CA_EINVAL),
])
def test_mla_prefill_rejections(kwargs, status):
    assert mla_prefill(**kwargs) == status
    assert L.lib().chunkattn_last_error().decode()


def test_mla_prefill_workspace_size():
    assert L.lib().chunkattn_mla_prefill_workspace_size(100, 300, L.CA_MLA_BF16) == 0
    assert L.lib().chunkattn_mla_prefill_workspace_size(100, 300, L.CA_MLA_FP8) == 7 * 73728
    assert L.lib().chunkattn_mla_prefill_workspace_size(0, 64, L.CA_MLA_FP8) == 73728
    assert L.lib().chunkattn_mla_prefill_workspace_size(0, 65, L.CA_MLA_FP8) == 2 * 73728
    assert L.lib().chunkattn_mla_prefill_workspace_size(-1, 65, L.CA_MLA_FP8) == 0
    assert L.lib().chunkattn_mla_prefill_workspace_size(0, 65, 7) == 0


def test_mla_prefill_empty_chunk_succeeds():
    # 512 tokens fill the 8 blocks exactly: in range; an empty chunk launches nothing
    assert mla_prefill(q=None, out=None, chunk=0) == L.CA_OK


def test_mla_append_rejections():
    lib = L.lib()
    f = lambda **kw: lib.chunkattn_mla_kv_append(kw.get("lat", FAKE), FAKE, kw.get("start", 0), kw.get("n", 10),
                                                 kw.get("fmt", L.CA_MLA_FP8), FAKE, kw.get("tl", 1),
                                                 kw.get("nb", 4), FAKE, None)
    assert f(fmt=3) == L.CA_EINVAL
    assert f(start=-1) == L.CA_EINVAL
    assert f(lat=None) == L.CA_EINVAL
    assert f(lat=MISALIGNED) == L.CA_EINVAL
    assert f(nb=0) == L.CA_EINVAL
    assert f(start=60, n=10) == L.CA_ERANGE
    assert f(n=0, lat=None) == L.CA_OK


def test_stride_of_cache_views():
    """Strides the binding passes for strided cache views (torch CPU views, no library call)."""
    t, hq, hkv, d = 7, 8, 1, 128
    qkv = torch.empty((t, hq + 2 * hkv, d), dtype=torch.bfloat16)
    k = qkv[:, hq:hq + hkv]                                # one KV head sliced out of a fused QKV
    assert k.shape == (t, 1, d)
    assert (L._stride(k, 0), L._stride(k, 1)) == ((hq + 2) * d, d)
    one = torch.empty((4, 1, d), dtype=torch.bfloat16).transpose(0, 1)   # one token, odd strides
    assert one.shape == (1, 4, d)
    assert (L._stride(one, 0), L._stride(one, 1)) == (4 * d, d)
    pad = torch.empty((t, 4, 256), dtype=torch.bfloat16)[:, :, :192]    # d = 192 in heads padded to 256
    assert (L._stride(pad, 0), L._stride(pad, 1)) == (4 * 256, 256)
    one_pad = pad[2:3]
    assert (L._stride(one_pad, 0), L._stride(one_pad, 1)) == (4 * 192, 256)


def test_broadcast_cache_view_is_refused_before_the_library():
    """An expanded (stride-0) view would read as "dense" through the ABI; the binding refuses it."""
    base = torch.empty((9, 1, 64), dtype=torch.bfloat16)
    k = base.expand(9, 4, 64)
    assert k.stride(1) == 0
    with pytest.raises(ValueError, match="broadcast"):
        L._stride(k, 1)
    q = torch.empty((3, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="broadcast"):
        L.chunk_prefill_attn(q, k, k, 6, relayout=False)


def test_binding_refuses_mislaid_tensors_before_the_library():
    """The C calls take bare pointers, so the binding checks every tensor's shape, dtype and layout against
    what the call assumes, and refuses a host tensor, before the library is called (torch CPU tensors)."""
    bf, f32 = torch.bfloat16, torch.float32
    c, hq, hkv, d = 8, 8, 2, 128
    q = torch.zeros((c, hq, d), dtype=bf)
    kp, vp = L.paged_pool(4, hkv, d, d, bf, device="cpu")
    table = torch.zeros(4, dtype=torch.int32)
    run = lambda **kw: L.chunk_prefill_attn(**{**dict(q=q, k_cache=kp, v_cache=vp, past_len=0,
                                                      kv_layout="paged", block_table=table), **kw})
    with pytest.raises(ValueError, match="q: expected"):
        run(q=q[0])
    with pytest.raises(ValueError, match="k_pool: shape"):
        run(k_cache=L.paged_pool(4, hkv, 64, d, bf, device="cpu")[0])          # head dim 64 against q's 128
    with pytest.raises(ValueError, match="k_pool must be contiguous"):
        run(k_cache=torch.empty((4, 4, 16, 64, 8), dtype=bf)[:, ::2])
    with pytest.raises(ValueError, match="v_pool: dtype"):
        run(v_cache=vp.float())
    with pytest.raises(ValueError, match="block_table: dtype"):
        run(block_table=table.long())
    with pytest.raises(ValueError, match="out: shape"):
        run(out=torch.empty((c, hq, 64), dtype=bf))
    with pytest.raises(ValueError, match="out must be contiguous"):
        run(out=torch.empty((hq, c, d), dtype=bf).transpose(0, 1))
    with pytest.raises(ValueError, match="lse: dtype"):
        run(lse=torch.empty((hq, c), dtype=bf))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        run()
    kc = torch.zeros((c, hkv, d), dtype=bf)
    with pytest.raises(ValueError, match="k_cache: dtype"):
        L.chunk_prefill_attn(q, kc.float(), kc, 0, relayout=False)
    with pytest.raises(ValueError, match="disagree"):
        L.chunk_prefill_attn(q, kc[:, :, :64], kc, 0, relayout=False)
    # mixed batch
    cu, kv = [0, 4, 5], [4, 70]
    tables = torch.zeros((2, 2), dtype=torch.int32)
    qv = torch.zeros((5, hq, d), dtype=bf)
    with pytest.raises(ValueError, match="block_tables: shape"):
        L.chunk_attn_varlen(qv, kp, vp, tables[:1], cu, kv)
    with pytest.raises(ValueError, match="one more entry"):
        L.chunk_attn_varlen(qv, kp, vp, tables, cu[:2], kv)
    with pytest.raises(ValueError, match="q: dtype"):
        L.chunk_attn_varlen(qv.float(), kp, vp, tables, cu, kv)
    # cache writes
    with pytest.raises(ValueError, match="disagree"):
        L.chunkattn_kv_append(kc, kc[:4], 0, table, kp, vp)
    with pytest.raises(ValueError, match="k_pool: shape"):                     # fp32 rows against a bf16 pool
        L.chunkattn_kv_append(kc.float(), kc.float(), 0, table, kp, vp)
    # MLA latent calls
    pool = L.mla_pool(4, L.CA_MLA_BF16, device="cpu")
    qm = torch.zeros((c, 16, L.MLA_LATENT + L.MLA_ROPE), dtype=bf)
    with pytest.raises(ValueError, match="q: shape"):
        L.chunk_mla_prefill(qm[:, :, :L.MLA_LATENT], pool, L.CA_MLA_BF16, table, 0, 0.1)
    with pytest.raises(ValueError, match="pool: shape"):
        L.chunk_mla_prefill(qm, pool, L.CA_MLA_FP8, table, 0, 0.1)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        L.chunk_mla_prefill(qm, pool, L.CA_MLA_BF16, table, 0, 0.1)
    with pytest.raises(ValueError, match="kv_lens has"):
        L.chunk_mla_decode(qm, pool, L.CA_MLA_BF16, tables, [4], 0.1)
    with pytest.raises(ValueError, match="rope: shape"):
        L.chunkattn_mla_kv_append(torch.zeros((3, L.MLA_LATENT), dtype=bf), torch.zeros((3, 32), dtype=bf), 0,
                                  table, pool, L.CA_MLA_BF16)


# ---- the build's check of the split direct-to-LDS loads --------------------------------------------------

_M0_OK = """\
kernel:
\t;;#ASMSTART
\ts_mov_b32 m0, s9
\t;;#ASMEND
\tv_mfma_f32_16x16x32_bf16 v[94:97], v[118:121], v[106:109], v[94:97]
\t;;#ASMSTART
\tglobal_load_lds_dwordx4 v148, s[6:7]
\t;;#ASMEND
\t;;#ASMSTART
\ts_mov_b32 m0, s10
\ts_nop 0
\tglobal_load_lds_dwordx4 v149, s[6:7]
\t;;#ASMEND
\ts_endpgm
"""


def test_m0_check_accepts_the_split_and_the_combined_load():
    from chunked_prefill_causal_amd import build as B
    assert B.check_m0(_M0_OK, "ok") == 2


def test_m0_check_rejects_a_compiler_m0_write():
    from chunked_prefill_causal_amd import build as B
    bad = _M0_OK.replace("\tv_mfma_f32_16x16x32_bf16", "\ts_mov_b32 m0, -1\n\tv_mfma_f32_16x16x32_bf16")
    with pytest.raises(RuntimeError, match="the compiler writes m0"):
        B.check_m0(bad, "bad")


def test_m0_check_rejects_a_load_right_after_the_m0_write():
    from chunked_prefill_causal_amd import build as B
    bad = _M0_OK.replace("\ts_nop 0\n", "")
    with pytest.raises(RuntimeError, match="right after an m0 write"):
        B.check_m0(bad, "bad")
    # the split form with nothing between the two statements
    bad = _M0_OK.replace("\tv_mfma_f32_16x16x32_bf16 v[94:97], v[118:121], v[106:109], v[94:97]\n", "")
    with pytest.raises(RuntimeError, match="right after an m0 write"):
        B.check_m0(bad, "bad")


def test_m0_check_holds_on_the_built_kernels():
    """The device assembly the last build checked (written beside the objects) passes again, and holds
    the loads of both kernels."""
    import os
    from chunked_prefill_causal_amd import build as B
    for src, at_least in (("prefill_paged", 100), ("mla_prefill", 20)):
        path = os.path.join(B.BUILD_DIR, src + ".s")
        if not os.path.exists(path):
            pytest.skip("no build under _build/ yet")
        with open(path) as f:
            assert B.check_m0(f.read(), src) >= at_least


def test_kernel_hash_ignores_comments_but_not_code():
    """The counter summary stays valid across comment edits and goes stale on any code edit."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    src = 'int f(int a) {  // the sum\n  return a + 1; /* one\n more */ }\nasm("s_nop 0\\n");\n'
    same = 'int f(int a) {\n  // the sum, said differently\n  return a + 1;\n}\nasm("s_nop 0\\n");\n'
    other = 'int f(int a) {  // the sum\n  return a + 2; /* one\n more */ }\nasm("s_nop 0\\n");\n'
    assert bench.strip_comments(src) == bench.strip_comments(same)
    assert bench.strip_comments(src) != bench.strip_comments(other)
    assert "s_nop 0" in bench.strip_comments(src)


def _mla_plan_bytes(kv_lens, heads, units):
    """Workspace of the MLA decode plan with `units` work units, as the header lays it out: step prefix
    sums, each unit's first sequence, then (m, l) and O per head and slot (one slot per sequence and unit)."""
    up = lambda x: (x + 255) // 256 * 256
    n = len(kv_lens)
    slots = n + units
    unit_off = up((n + 1) * 8)
    ml_off = unit_off + up(units * 4)
    o_off = ml_off + up(heads * slots * 2 * 4)
    return o_off + heads * slots * 512 * 4


@pytest.mark.parametrize("kv_lens, heads, units", [
    ([40000] * 300, 16, 1024),     # 375000 steps: two rounds of 512 units, 367 steps each (at most 383)
    ([17000] * 256, 16, 512),      # 136192 steps: one round of 512 units, 266 steps each
    ([300, 77, 1], 1024, 8),       # 64 head blocks: the minimum of 8 units per head block
    ([5] * 100, 16, 100),          # fewer steps than a round: one unit per step
])
def test_mla_decode_plan_units(kv_lens, heads, units):
    """The host plan cuts the batch's 32-key steps into a whole number of rounds of the workgroups the chip
    holds (two per CU, shared by the head blocks), each unit at most 383 steps; the workspace query pins it."""
    for fmt in (L.CA_MLA_BF16, L.CA_MLA_FP8):
        assert L.chunkattn_mla_decode_workspace_size(kv_lens, heads, fmt) == _mla_plan_bytes(kv_lens, heads, units)

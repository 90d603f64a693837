"""Helpers shared by the GPU parity tests: device pools in the interleaved
layout, readback into the oracle's flat-array form, and tolerance checks."""

import sys

import numpy as np

import paged_kv_cache_inject_amd as pkv
from oracle.layout import PoolSpec

ATOL = 1e-3
RTOL = 2e-3
ELEM = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
            "fp8": torch.uint8}[dtype]


def raw_view(t):
    """numpy raw view of a CPU tensor: float32, uint16 bits for 16-bit types,
    uint8 codes for fp8."""
    import torch
    if t.dtype in (torch.float32, torch.uint8):
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def to_device_raw(arr, dtype, device="cuda"):
    """Upload a raw numpy array (float32 or uint16 bits) as a typed device tensor."""
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if dtype == "fp8":
        return torch.from_numpy(a.astype(np.uint8)).to(device)
    t = torch.from_numpy(a.view(np.int16)).to(device)
    return t.view(torch_dtype(dtype))


class DevicePool:
    """A paged pool whose blocks hold [K planes of all heads][V planes]:
    buffer[layer][block][K|V][head][16*d]."""

    def __init__(self, n_layers, num_blocks, n_kv_heads, head_dim, dtype, fill_bits=None,
                 device="cuda"):
        import torch
        self.n_layers, self.num_blocks = n_layers, num_blocks
        self.n_kv_heads, self.head_dim, self.dtype = n_kv_heads, head_dim, dtype
        plane = 16 * head_dim
        self.head_stride = plane
        self.block_stride = 2 * n_kv_heads * plane
        self.layer_stride = num_blocks * self.block_stride
        self.v_off = n_kv_heads * plane
        self.total = n_layers * self.layer_stride
        self.buf = torch.empty(self.total, dtype=torch_dtype(dtype), device=device)
        self.k_scale = self.v_scale = None        # float32 [layers][heads] (fp8 pools)
        self.scale_mode = 0                       # 1: scales [layers][blocks][heads]
        if fill_bits is not None:
            if dtype == "fp8":
                self.buf.fill_(int(fill_bits) & 0xFF)
            elif dtype == "f32":
                self.buf.view(torch.int32).fill_(int(np.int32(np.uint32(fill_bits))))
            else:
                self.buf.view(torch.int16).fill_(int(np.int16(np.uint16(fill_bits))))

    def desc(self, layer_offset=0):
        e = ELEM[self.dtype]
        base = self.buf.data_ptr() + layer_offset * self.layer_stride * e
        return pkv.pkv_pool(self.n_layers - layer_offset, self.num_blocks, self.n_kv_heads,
                            self.head_dim, pkv.DTYPE_CODES[self.dtype], self.scale_mode, base,
                            base + self.v_off * e, self.layer_stride, self.block_stride,
                            self.head_stride,
                            None if self.k_scale is None else self._scale_ptr(self.k_scale, layer_offset),
                            None if self.v_scale is None else self._scale_ptr(self.v_scale, layer_offset))

    def _scale_ptr(self, t, layer_offset):
        """Address of layer `layer_offset`'s scales (the pool view starts there)."""
        per_layer = t[0].numel()
        return t.data_ptr() + layer_offset * per_layer * 4

    def spec(self):
        return PoolSpec(self.n_layers, self.num_blocks, self.n_kv_heads, self.head_dim,
                        self.dtype, self.layer_stride, self.block_stride, self.head_stride)

    def host_copy(self):
        """Raw numpy copy of the whole buffer."""
        return raw_view(self.buf.cpu()).copy()

    def set_scales(self, k_scale, v_scale):
        """float32 scales of an fp8 pool (host arrays): [layers][heads], or
        [layers][blocks][heads] for per-block scales."""
        import torch
        self.scale_mode = 1 if np.ndim(k_scale) == 3 else 0
        self.k_scale = torch.from_numpy(np.ascontiguousarray(k_scale, np.float32)).cuda()
        self.v_scale = torch.from_numpy(np.ascontiguousarray(v_scale, np.float32)).cuda()

    def oracle_arrays(self, flat):
        """(k_pool, v_pool) views of one flat buffer, as the oracle indexes them."""
        return flat, flat[self.v_off:]

    def host_layers(self, layers):
        """Raw copy holding only the given layers (others zero), for sampling."""
        flat = np.zeros(self.total, dtype=np.float32 if self.dtype == "f32" else np.uint16)
        for l in layers:
            a, b = l * self.layer_stride, (l + 1) * self.layer_stride
            flat[a:b] = raw_view(self.buf[a:b].cpu())
        return flat


def host_planes_for(dp: DevicePool, layer, tables, seqs, heads):
    """Raw copy holding only the blocks of `seqs` (all heads) in `layer`.

    Returns a flat buffer the size of the whole pool (zeros elsewhere) built
    from per-block device slices, so huge pools can be sampled cheaply.
    """
    import torch
    flat = np.zeros(dp.total, dtype={"f32": np.float32, "fp8": np.uint8}.get(dp.dtype, np.uint16))
    blocks = sorted({int(b) for s in seqs for b in tables[s] if b >= 0})
    idx = torch.tensor(blocks, dtype=torch.long, device=dp.buf.device)
    view = dp.buf[layer * dp.layer_stride:(layer + 1) * dp.layer_stride].view(
        dp.num_blocks, dp.block_stride)
    got = raw_view(view.index_select(0, idx).cpu())
    for i, b in enumerate(blocks):
        a = layer * dp.layer_stride + b * dp.block_stride
        flat[a:a + dp.block_stride] = got[i]
    return flat


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    err = np.abs(got - ref)
    bad = ~both_inf & ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d/%d elements out of tolerance; first at %s: got %r ref %r"
                             % (what, bad.sum(), bad.size, tuple(i), got[tuple(i)], ref[tuple(i)]))
    return float(np.max(np.where(both_inf, 0, err))) if err.size else 0.0


def assert_bytes_equal(got, ref, what):
    g = np.ascontiguousarray(got).view(np.uint8)
    r = np.ascontiguousarray(ref).view(np.uint8)
    if not np.array_equal(g, r):
        gw = np.ascontiguousarray(got).view(np.uint16 if got.dtype == np.uint16 else np.uint32)
        rw = np.ascontiguousarray(ref).view(np.uint16 if ref.dtype == np.uint16 else np.uint32)
        diff = np.nonzero(gw != rw)[0]
        raise AssertionError("%s: %d elements differ; first at %d: got %#x ref %#x"
                             % (what, len(diff), diff[0], int(gw[diff[0]]), int(rw[diff[0]])))


def rope_tables(head_dim, max_pos, base=10000.0):
    """Library-built rotary table (host) and its device copy."""
    import torch
    cos, sin = pkv.pkv_rope_table(head_dim, base, max_pos)
    return cos, sin, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()


def workspace(n_bytes):
    import torch
    return torch.empty(max(int(n_bytes), 256), dtype=torch.uint8, device="cuda")


def decode(dp: DevicePool, layer, q_dev, tables_dev, lens, n_q_heads, part_tokens=0,
           with_lse=True, q_dtype=None, window=0):
    """Plan + upload + decode one layer; returns (out, lse) device tensors."""
    import torch
    plan = pkv.pkv_decode_plan_create(lens, n_q_heads, dp.n_kv_heads, dp.head_dim, part_tokens,
                                      window=window)
    try:
        ws = workspace(pkv.pkv_decode_workspace_bytes(plan))
        pkv.pkv_decode_plan_upload(plan, ws)
        b = len(lens)
        out = torch.full((b, n_q_heads, dp.head_dim), float("nan"), device="cuda")
        lse = torch.full((b, n_q_heads), float("nan"), device="cuda") if with_lse else None
        pkv.pkv_decode_attention(plan, dp.desc(), layer, q_dev, tables_dev, out, lse, ws,
                                 q_dtype=q_dtype)
        torch.cuda.synchronize()
    finally:
        pkv.pkv_decode_plan_destroy(plan)
    return out, lse

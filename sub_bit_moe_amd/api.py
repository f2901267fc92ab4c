"""Python front end of libsbm: argument marshalling only.

Every step of the codec and of the fused decode + matvec runs in libsbm.so
(host C++ for dictionary/encoding, HIP kernels on the GPU).  numpy arrays are
used for host buffers, torch tensors for device memory and streams.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np

from . import _native as N
from ._native import check, lib


def _ptr(a) -> int:
    if a is None:
        return 0
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return int(a.data_ptr())


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)

# ------------------------------------------------------------------ dictionary

def build_dictionary(p0: float = 0.885):
    """(words uint32[131072], checksum) of the canonical dictionary."""
    words = np.zeros(N.SBM_DICT_WORDS, np.uint32)
    cs = C.c_uint64()
    check(lib().sbm_build_dictionary(C.c_double(p0), words.ctypes.data, C.addressof(cs)))
    return words, int(cs.value)


def dictionary_checksum(words: np.ndarray) -> int:
    words = np.ascontiguousarray(words, np.uint32)
    cs = C.c_uint64()
    check(lib().sbm_dictionary_checksum(words.ctypes.data, C.addressof(cs)))
    return int(cs.value)


def dict_tag(words: np.ndarray) -> int:
    """Dictionary identity carried by every matrix descriptor: the low 32 bits
    of the dictionary's FNV-1a 64 checksum (also in the decode image header)."""
    return dictionary_checksum(words) & 0xFFFFFFFF


def dict_image(words: np.ndarray, slots: int = 3) -> np.ndarray:
    """Compact decode image (uint8 bytes) for the fused kernel: slots=3 for
    tables whose entries hold at most 3 nonzeros (the page's static table),
    slots=4 for tables built for other data (entries with 4 nonzeros)."""
    words = np.ascontiguousarray(words, np.uint32)
    if slots not in (3, 4):
        raise ValueError("slots must be 3 or 4")
    n = int(lib().sbm_dict_image_bytes() if slots == 3 else lib().sbm_dict_image4_bytes())
    out = np.zeros(n, np.uint8)
    fn = lib().sbm_dict_image if slots == 3 else lib().sbm_dict_image4
    check(fn(words.ctypes.data, out.ctypes.data, n))
    return out

# ------------------------------------------------------------------ host codec

def encode_matrix(sym: np.ndarray, words: np.ndarray):
    """Greedy trie encoding of a symbol matrix uint8 [rows, cols] (0/1/2).
    Returns (codes uint16[n], row_off uint32[rows+1], bstart uint32[nblk])."""
    sym = np.ascontiguousarray(sym, np.uint8)
    rows, cols = sym.shape
    words = np.ascontiguousarray(words, np.uint32)
    n = C.c_uint64()
    check(lib().sbm_encode_size(sym.ctypes.data, rows, cols, words.ctypes.data, C.addressof(n)))
    codes = np.zeros(max(int(n.value), 1), np.uint16)
    row_off = np.zeros(rows + 1, np.uint32)
    nblk = (int(n.value) + N.SBM_BLOCK - 1) // N.SBM_BLOCK
    bstart = np.zeros(max(nblk, 1), np.uint32)
    check(lib().sbm_encode_matrix(sym.ctypes.data, rows, cols, words.ctypes.data, codes.ctypes.data,
                                  codes.size, row_off.ctypes.data, bstart.ctypes.data, C.addressof(n)))
    return codes[:int(n.value)], row_off, bstart[:nblk]


def encode_experts(syms, words: np.ndarray):
    """One projection's matrices (same shape, uint8 0/1/2) encoded natively into
    the stack layout: (codes uint16 with aligned bases, row_off uint32
    [E*(rows+1)], bstart uint32, list of MatrixDesc with scale_base = e*rows)."""
    words = np.ascontiguousarray(words, np.uint32)
    syms = [np.ascontiguousarray(m, np.uint8) for m in syms]
    E = len(syms)
    rows, cols = (syms[0].shape if E else (0, 2))
    if any(m.shape != (rows, cols) for m in syms):
        raise ValueError("all matrices of a projection share one shape")
    ptrs = (C.c_void_p * max(E, 1))(*[m.ctypes.data for m in syms])
    nc, nb = C.c_uint64(), C.c_uint64()
    st = lib().sbm_encode_experts(E, ptrs, rows, cols, words.ctypes.data, None, 0, None, None, 0, None,
                                  C.addressof(nc), C.addressof(nb))
    if st not in (0, -6):          # -6: SBM_ENOSPACE, the size query
        check(st)
    codes = np.zeros(max(int(nc.value), 1), np.uint16)
    row_off = np.zeros(max(E * (rows + 1), 1), np.uint32)
    bstart = np.zeros(max(int(nb.value), 1), np.uint32)
    desc = (N.MatrixDesc * max(E, 1))()
    check(lib().sbm_encode_experts(E, ptrs, rows, cols, words.ctypes.data, codes.ctypes.data, codes.size,
                                   row_off.ctypes.data, bstart.ctypes.data, bstart.size, C.addressof(desc),
                                   C.addressof(nc), C.addressof(nb)))
    return codes[:int(nc.value)], row_off[:E * (rows + 1)], bstart[:int(nb.value)], list(desc)[:E]


def block_starts(codes: np.ndarray, words: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint16)
    nblk = (codes.size + N.SBM_BLOCK - 1) // N.SBM_BLOCK
    out = np.zeros(max(nblk, 1), np.uint32)
    check(lib().sbm_block_starts(codes.ctypes.data, codes.size,
                                 np.ascontiguousarray(words, np.uint32).ctypes.data, out.ctypes.data))
    return out[:nblk]


def validate_stream(codes, row_off, rows: int, cols: int, words) -> None:
    codes = np.ascontiguousarray(codes, np.uint16)
    row_off = np.ascontiguousarray(row_off, np.uint32)
    check(lib().sbm_validate_stream(codes.ctypes.data, codes.size, row_off.ctypes.data, rows, cols,
                                    np.ascontiguousarray(words, np.uint32).ctypes.data))

# ------------------------------------------------------------------ device data

@dataclass
class ExpertStack:
    """Encoded matrices of one shape (one projection of all experts), resident
    on the device in the layout the fused kernel reads."""
    rows: int
    cols: int
    n_experts: int
    codes: object      # torch.int16 [total codes] (uint16 bit patterns)
    row_off: object    # torch.int32 [E*(rows+1)] (uint32 values)
    bstart: object     # torch.int32 [total blocks]
    scales: object     # torch.float16 [E*rows]
    desc: object       # torch.uint8 [E*sizeof(MatrixDesc)]
    host_desc: list
    code_bytes: int    # bytes of codes actually used (without alignment padding)

    def matrix_bytes(self, e: int) -> int:
        """Bytes the fused kernel must read for expert e: codes + block starts
        + scales (row offsets are read once per slice)."""
        d = self.host_desc[e]
        nblk = (d.n_codes + N.SBM_BLOCK - 1) // N.SBM_BLOCK
        per_row = max(1, int(self.scales.numel()) // max(1, self.n_experts * self.rows))   # 1, or 2 (min/max)
        return 2 * d.n_codes + 4 * nblk + 2 * per_row * self.rows

    @staticmethod
    def from_symbols(syms, scales, words, device="cuda"):
        """Matrices of one shape (uint8 0/1/2) encoded by sbm_encode_experts and
        uploaded; scales: per matrix, rows fp16 (or [rows, 2] for the min/max
        grid, whose descriptors then get doubled scale bases)."""
        codes, row_off, bstart, descs = encode_experts(syms, words)
        rows, cols = syms[0].shape
        sc = [np.asarray(s, np.float16).reshape(-1) for s in scales]
        per_row = sc[0].size // rows
        assert all(s.size == per_row * rows for s in sc) and per_row in (1, 2)
        for d in descs:
            d.scale_base *= per_row
        used = 2 * sum(int(d.n_codes) for d in descs)
        return ExpertStack._upload(rows, cols, descs, codes, row_off, bstart, np.concatenate(sc), used, device)

    @staticmethod
    def _upload(rows, cols, descs, codes, row_off, bstart, scales, used, device):
        import torch
        if codes.size == 0:
            codes = np.zeros(8, np.uint16)
        if bstart.size == 0:
            bstart = np.zeros(1, np.uint32)
        desc_arr = (N.MatrixDesc * len(descs))(*descs)
        desc_bytes = np.frombuffer(bytes(desc_arr), np.uint8).copy()
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        return ExpertStack(rows, cols, len(descs), t(codes, np.int16), t(row_off, np.int32),
                           t(bstart, np.int32), t(scales, np.float16), t(desc_bytes, np.uint8), descs, used)

    @staticmethod
    def assemble(mats, rows: int, cols: int, dict_tag: int):
        """Host stack layout from per-matrix encodings made with the dictionary
        whose tag is dict_tag (api.dict_tag(words)): (descs, codes, row_off,
        bstart, scales, used bytes)."""
        descs = []
        code_parts, off_parts, blk_parts, sc_parts = [], [], [], []
        cb = ob = sb = bb = 0
        used = 0
        for codes, row_off, bstart, scales in mats:
            n = int(codes.size)
            # one scale per row, or (w_min, w_max) per row for the min/max grid
            assert row_off.size == rows + 1 and scales.size in (rows, 2 * rows)
            d = N.MatrixDesc(code_base=cb, off_base=ob, scale_base=sb, blk_base=bb, n_codes=n,
                             rows=rows, cols=cols, dict_tag=dict_tag)
            descs.append(d)
            pad = (-n) % N.SBM_CODE_ALIGN
            code_parts.append(np.concatenate([codes.astype(np.uint16), np.zeros(pad, np.uint16)]))
            off_parts.append(row_off.astype(np.uint32))
            blk_parts.append(bstart.astype(np.uint32))
            sc_parts.append(scales.astype(np.float16))
            cb += n + pad
            ob += rows + 1
            sb += scales.size
            bb += bstart.size
            used += 2 * n
        codes = np.concatenate(code_parts) if code_parts else np.zeros(0, np.uint16)
        bstart = np.concatenate(blk_parts) if blk_parts else np.zeros(0, np.uint32)
        return descs, codes, np.concatenate(off_parts), bstart, np.concatenate(sc_parts), used

    @staticmethod
    def from_host(mats, rows: int, cols: int, device="cuda", *, dict_tag: int):
        """mats: list of (codes uint16, row_off uint32, bstart uint32, scales fp16),
        encoded with the dictionary whose tag is dict_tag (api.dict_tag(words))."""
        descs, codes, row_off, bstart, scales, used = ExpertStack.assemble(mats, rows, cols, dict_tag)
        return ExpertStack._upload(rows, cols, descs, codes, row_off, bstart, scales, used, device)


def device_image(words: np.ndarray, device="cuda", slots: int = 3):
    import torch
    return torch.from_numpy(dict_image(words, slots)).to(device)

# ------------------------------------------------------------------ GPU calls

def decode_ref(codes_t, row_off_t, rows: int, cols: int, words_t, stream=None, out=None, bad=None):
    """GPU reference decode of one matrix -> (symbols uint8 [rows, cols], bad_rows)."""
    import torch
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=codes_t.device)
    if bad is None:
        bad = torch.zeros(1, dtype=torch.int32, device=codes_t.device)
    check(lib().sbm_decode_ref(_ptr(codes_t), _ptr(row_off_t), rows, cols, _ptr(words_t), _ptr(out),
                               _ptr(bad), _stream(stream)))
    return out, bad


def decode_dense(stack: "ExpertStack", e: int, image_t, out=None, bad=None, stream=None):
    """Expert e's matrix of a stack decoded to dense fp16 {-1, 0, +1}
    [rows, cols] (sbm_decode_dense; the row scales are not applied)."""
    import torch
    d = stack.host_desc[e]
    if out is None:
        out = torch.empty((stack.rows, stack.cols), dtype=torch.float16, device=stack.codes.device)
    if bad is None:
        bad = torch.zeros(1, dtype=torch.int32, device=stack.codes.device)
    check(lib().sbm_decode_dense(_ptr(stack.codes[d.code_base:]), int(d.n_codes), _ptr(stack.bstart[d.blk_base:]),
                                 stack.rows, stack.cols, _ptr(image_t), int(d.dict_tag), _ptr(out), _ptr(bad),
                                 _stream(stream)))
    return out, bad


def workspace_bytes(n_experts: int, n_tokens: int) -> int:
    return int(lib().sbm_workspace_bytes(n_experts, n_tokens))


def alloc_workspace(n_experts: int, n_tokens: int, device="cuda"):
    import torch
    return torch.empty(max(workspace_bytes(n_experts, n_tokens), 16), dtype=torch.uint8, device=device)


def _x_flag(x) -> int:
    """Activation dtype flag: fp16 (none) or bf16 (SBM_F_IN_BF16)."""
    import torch
    if x is None or x.dtype == torch.float16:
        return 0
    if x.dtype == torch.bfloat16:
        return N.SBM_F_IN_BF16
    raise TypeError(f"activations must be float16 or bfloat16, not {x.dtype}")


def moe_fused_decode_matvec(stack: ExpertStack, image_t, x, expert_ids, relu: bool = False,
                            out_f32: bool = False, workspace=None, y=None, stream=None, in_rms: bool = False,
                            mfma: bool = False, minmax: bool = False, image4=None,
                            deterministic: bool = False):
    """y[t] = act(W_{expert_ids[t]} x[t]) for one projection of an MoE layer
    (in_rms: x[t] is first scaled to unit RMS, as rms_glue does; mfma=True
    sends experts with 16 or more tokens to the dense-tile MFMA path; minmax:
    the stack's scales are (w_min, w_max) per row, the page's grid; image4:
    image_t is a 4-slot image, by default told from its byte size;
    deterministic: fixed-point row accumulators, bit-reproducible outputs)."""
    import torch
    T = int(x.shape[0]) if x is not None else 0
    if y is None:
        y = torch.empty((T, stack.rows), dtype=torch.float32 if out_f32 else torch.float16,
                        device=stack.codes.device)
    if workspace is None:
        workspace = alloc_workspace(stack.n_experts, T, device=stack.codes.device)
    flags = (N.SBM_F_RELU if relu else 0) | (N.SBM_F_OUT_F32 if out_f32 else 0) | (N.SBM_F_IN_RMS if in_rms else 0)
    flags |= N.SBM_F_MFMA if mfma else 0
    flags |= N.SBM_F_MINMAX if minmax else 0
    flags |= N.SBM_F_DETERMINISTIC if deterministic else 0
    flags |= _x_flag(x)
    n4 = int(lib().sbm_dict_image4_bytes())
    if image4 is None:
        image4 = int(image_t.numel()) == n4
    need = n4 if image4 else int(lib().sbm_dict_image_bytes())
    if int(image_t.numel()) * image_t.element_size() < need:
        raise ValueError(f"image buffer holds {image_t.numel() * image_t.element_size()} bytes; the kernel copies {need}")
    flags |= N.SBM_F_IMAGE4 if image4 else 0
    check(lib().sbm_moe_fused_decode_matvec(
        _ptr(stack.codes), _ptr(stack.row_off), _ptr(stack.bstart), _ptr(stack.scales), _ptr(stack.desc),
        stack.n_experts, stack.rows, stack.cols, _ptr(image_t), _ptr(x), _ptr(expert_ids), T, _ptr(y),
        flags, _ptr(workspace), int(workspace.numel()), _stream(stream)))
    return y


def ffn_workspace_bytes(n_experts: int, n_tokens: int) -> int:
    return int(lib().sbm_ffn_workspace_bytes(n_experts, n_tokens))


def alloc_ffn_workspace(n_experts: int, n_tokens: int, device="cuda"):
    """Zeroed workspace of the layer call (it must start zeroed; every call
    leaves it ready for the next)."""
    import torch
    return torch.zeros(max(ffn_workspace_bytes(n_experts, n_tokens), 64), dtype=torch.uint8, device=device)


def _projection(st: ExpertStack):
    return N.Projection(codes=_ptr(st.codes), row_off=_ptr(st.row_off), bstart=_ptr(st.bstart),
                        scales=_ptr(st.scales), experts=_ptr(st.desc), n_experts=st.n_experts, rows=st.rows,
                        cols=st.cols)


def moe_fused_ffn(up: ExpertStack, down: ExpertStack, image_t, x, expert_ids, h=None, y=None, workspace=None,
                  in_rms: bool = False, out_f32: bool = False, stream=None):
    """One MoE expert FFN in one launch (sbm_moe_fused_ffn): h = relu(W_up x),
    y = W_down h for every token's expert.  Returns (y, h)."""
    import torch
    T = int(x.shape[0])
    dev = up.codes.device
    if h is None:
        h = torch.empty((T, up.rows), dtype=torch.float16, device=dev)
    if y is None:
        y = torch.empty((T, down.rows), dtype=torch.float32 if out_f32 else torch.float16, device=dev)
    if workspace is None:
        workspace = alloc_ffn_workspace(up.n_experts, T, dev)
    flags = (N.SBM_F_IN_RMS if in_rms else 0) | (N.SBM_F_OUT_F32 if out_f32 else 0) | _x_flag(x)
    pu, pd = _projection(up), _projection(down)
    check(lib().sbm_moe_fused_ffn(C.addressof(pu), C.addressof(pd), _ptr(image_t), _ptr(x), _ptr(expert_ids), T,
                                  _ptr(h), _ptr(y), flags, _ptr(workspace), int(workspace.numel()), _stream(stream)))
    return y, h


def layers_workspace_bytes(n_layers: int, n_experts: int, n_tokens: int) -> int:
    return int(lib().sbm_layers_workspace_bytes(n_layers, n_experts, n_tokens))


def alloc_layers_workspace(n_layers: int, n_experts: int, n_tokens: int, device="cuda"):
    """Zeroed workspace of the multi-layer call (it must start zeroed; every
    call leaves it ready for the next)."""
    import torch
    return torch.zeros(max(layers_workspace_bytes(n_layers, n_experts, n_tokens), 64), dtype=torch.uint8,
                       device=device)


def moe_fused_layers(ups, downs, image_t, x, expert_ids, h=None, y=None, workspace=None, in_rms: bool = False,
                     stream=None):
    """len(ups) MoE layers in one launch (sbm_moe_fused_layers): per layer l,
    h_l = relu(W_up x_l), y_l = W_down h_l with x_0 = x and x_l = y_{l-1}
    scaled to unit RMS per token; expert_ids: int32 [n_layers, T].  Returns
    (y, h): every layer's outputs, fp16 [n_layers, T, width]."""
    import torch
    L = len(ups)
    assert L == len(downs) and L >= 1
    T = int(x.shape[0])
    dev = ups[0].codes.device
    if h is None:
        h = torch.empty((L, T, ups[0].rows), dtype=torch.float16, device=dev)
    if y is None:
        y = torch.empty((L, T, downs[0].rows), dtype=torch.float16, device=dev)
    assert h.numel() >= L * T * ups[0].rows and y.numel() >= L * T * downs[0].rows
    if workspace is None:
        workspace = alloc_layers_workspace(L, ups[0].n_experts, T, dev)
    flags = (N.SBM_F_IN_RMS if in_rms else 0) | _x_flag(x)
    pu = (N.Projection * L)(*[_projection(u) for u in ups])
    pd = (N.Projection * L)(*[_projection(d) for d in downs])
    check(lib().sbm_moe_fused_layers(C.addressof(pu), C.addressof(pd), L, _ptr(image_t), _ptr(x), _ptr(expert_ids),
                                     T, _ptr(h), _ptr(y), flags, _ptr(workspace), int(workspace.numel()),
                                     _stream(stream)))
    return y, h


def workspace_error(workspace, stream=None) -> int:
    v = C.c_uint32()
    check(lib().sbm_workspace_error(_ptr(workspace), C.addressof(v), _stream(stream)))
    return int(v.value)

# ------------------------------------------------------------------ synthetic stacks

def build_trie(words: np.ndarray) -> np.ndarray:
    """Host trie child table (int32[(65536+1)*9]) of a dictionary."""
    out = np.zeros(int(lib().sbm_trie_words()), np.int32)
    check(lib().sbm_build_trie(np.ascontiguousarray(words, np.uint32).ctypes.data, out.ctypes.data))
    return out


def generate_stack(seed: int, layer: int, n_experts: int, mat: int, rows: int, cols: int, p0: float,
                   trie_t, scale_table_t, stream=None, *, dict_checksum: int) -> ExpertStack:
    """Generate and encode n_experts counter-based matrices on the GPU
    (count pass, row offsets, descriptors, write pass) as an ExpertStack;
    dict_checksum: the checksum of the dictionary the trie was built from."""
    import torch
    from . import synth
    dev = trie_t.device
    z = synth.zero_threshold16(p0)
    s = _stream(stream)
    counts = torch.empty(n_experts * rows, dtype=torch.int32, device=dev)
    check(lib().sbm_gen_count(seed, layer, n_experts, mat, rows, cols, z, _ptr(trie_t), _ptr(counts), s))
    row_off = torch.empty(n_experts * (rows + 1), dtype=torch.int32, device=dev)
    desc = torch.empty(n_experts * C.sizeof(N.MatrixDesc), dtype=torch.uint8, device=dev)
    totals = torch.zeros(2, dtype=torch.int64, device=dev)
    check(lib().sbm_gen_layout(_ptr(counts), n_experts, rows, cols, _ptr(row_off), _ptr(desc), _ptr(totals),
                               C.c_uint64(dict_checksum), s))
    tot = totals.cpu().tolist()
    codes = torch.empty(max(int(tot[0]), 8), dtype=torch.int16, device=dev)
    bstart = torch.empty(max(int(tot[1]), 1), dtype=torch.int32, device=dev)
    scales = torch.empty(n_experts * rows, dtype=torch.float16, device=dev)
    check(lib().sbm_gen_write(seed, layer, n_experts, mat, rows, cols, z, _ptr(trie_t), _ptr(row_off),
                              _ptr(desc), _ptr(codes), _ptr(bstart), _ptr(scale_table_t), _ptr(scales), s))
    del counts
    host_desc = list((N.MatrixDesc * n_experts).from_buffer_copy(desc.cpu().numpy().tobytes()))
    used = 2 * sum(int(d.n_codes) for d in host_desc)
    return ExpertStack(rows, cols, n_experts, codes, row_off, bstart, scales, desc, host_desc, used)


def stream_read(buf, sink, stream=None) -> None:
    """Bandwidth probe: read every byte of the device tensor buf (sbm_stream_read)."""
    check(lib().sbm_stream_read(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(sink), int(sink.numel()),
                                _stream(stream)))


def rms_glue(y, out=None, stream=None):
    """Stack glue (not the method): x_next = y / rms(y) per token, fp16."""
    import torch
    if out is None:
        out = torch.empty_like(y)
    check(lib().sbm_rms_glue(_ptr(y), int(y.shape[0]), int(y.shape[1]), _ptr(out), _stream(stream)))
    return out

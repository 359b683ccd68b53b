"""Host-side checks of libfckl.so: it loads, exports what include/fckl.h declares, and
its scheduler and argument checks behave -- all without touching a GPU (the calls
here return before any HIP call)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import chunked_top_kl_chunk_amd as fckl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fckl.h")
GiB = 1 << 30


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fckl_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fckl.load()
    names = declared_functions()
    assert set(names) == set(fckl.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


# Writable data that the toolchain puts into any HIP shared library: the C runtime's and
# the dynamic linker's bookkeeping and the registration of the embedded GPU code.
TOOLCHAIN_DATA = re.compile(
    r"^(?:_DYNAMIC|_GLOBAL_OFFSET_TABLE_|__dso_handle|__init|__fini|__TMC_END__|DW\.ref\..*"
    r"|__do_init\..*|__do_fini\..*|completed\.\d+|__hip_fatbin_wrapper|__hip_gpubin_handle_\w+"
    r"|__hip_cuid_\w+|__do_global_dtors_aux_fini_array_entry|__frame_dummy_init_array_entry)$")
# The host-side handle of each kernel: an object whose address names the kernel at launch.
KERNEL_HANDLE = re.compile(r"^(?:void )?fckl::\(anonymous namespace\)::\w+_kernel(?:<.*>)?\(.*\)$")
# The allocation-free forward's device array and its per-device address table.
NOALLOC_STATE = {"fckl::scratch", "fckl::g_scratch_once", "fckl::g_scratch_ptr", "fckl::g_scratch_err"}


def test_no_writable_global_state_beyond_the_noalloc_table():
    """The library keeps no mutable globals: no cached device properties, default
    budgets or handles that one call could leave for the next.  Its writable data
    symbols are the toolchain's, the kernels' host handles, and the allocation-free
    forward's device array with its per-device address table."""
    fckl.load()
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm (binutils) is not installed")
    out = subprocess.run([nm, "-C", "--defined-only", fckl.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    writable, noalloc = [], set()
    for line in out.splitlines():
        parts = line.split(None, 2)
        if len(parts) != 3 or parts[1] not in "bBdDvVu":
            continue
        name = parts[2]
        if TOOLCHAIN_DATA.match(name) or KERNEL_HANDLE.match(name):
            continue
        if name in NOALLOC_STATE:
            noalloc.add(name)
            continue
        writable.append(line)
    assert not writable, "writable globals in libfckl.so:\n" + "\n".join(writable)
    assert noalloc == NOALLOC_STATE


def test_status_strings_and_version():
    assert fckl.status_string(fckl.OK) == "success"
    assert "workspace" in fckl.status_string(fckl.ERR_WORKSPACE)
    assert "index" in fckl.status_string(fckl.ERR_INDEX)
    assert fckl.status_string(99) == "unknown status"
    assert fckl.version() >= 100


C3 = dict(N=32768, H=2880, V=201088, K=100, T=1.0)
DEFAULT_BUDGET = 12 * GiB


def test_plan_fits_budget_and_is_even():
    d = fckl.make_desc(**C3)
    for budget in (0, 2 * GiB, 3 * GiB, 8 * GiB):
        chunk, ws = fckl.plan(d, budget)
        assert ws <= (budget or DEFAULT_BUDGET)
        assert chunk % 256 == 0 and 256 <= chunk <= 8192
        nchunks = -(-C3["N"] // chunk)
        assert nchunks * chunk - C3["N"] < 256 * nchunks


def test_workspace_independent_of_tokens():
    sizes = set()
    for N in (4096, 32768, 262144, 2 ** 31 - 1):
        d = fckl.make_desc(N, 2880, 201088, 100, 1.0)
        sizes.add(fckl.workspace_size(d, 4096))
    assert len(sizes) == 1


VPAD3 = (C3["V"] + 255) // 256 * 256


def test_workspace_grows_with_chunk():
    # one backward slab (the whole vocabulary): the workspace grows with the chunk
    d = fckl.make_desc(**C3, vocab_slab=VPAD3)
    w = [fckl.workspace_size(d, c) for c in (256, 1024, 4096, 8192, 16384)]
    assert all(a < b for a, b in zip(w, w[1:]))
    # dominated by the bf16 chunk gradient, kept once (2*C*V bytes), and the transposed
    # LM head (2*V*H bytes)
    C, V, H = 4096, 201088, 2880
    assert 2 * C * V + 2 * V * H < w[2] < 3 * C * V + 2 * V * H
    # the single call also keeps the chunk's exponentials (2*C*V bytes) and their
    # half-tile maxima (8*C*ceil(V/256) bytes)
    d.chunk = C
    chunk, single = fckl.single_plan(d, 0)
    assert chunk == C
    assert single == w[2] + 2 * C * ((V + 255) // 256 * 256) + 8 * C * ((V + 255) // 256)


def test_backward_slabs_bound_the_gradient_buffer():
    # The planner's slabs at 8192 tokens per chunk: 256, 256 and 274 of the 786
    # vocabulary tiles.  g^T is held for the largest slab only; each slab takes 2 dH
    # splits, 6 partial sums in all as for one slab.
    C, H, nVt = 8192, C3["H"], VPAD3 // 256
    auto = fckl.workspace_size(fckl.make_desc(**C3), C)
    whole = fckl.workspace_size(fckl.make_desc(**C3, vocab_slab=VPAD3), C)
    assert whole - auto == 2 * C * 256 * (nVt - 274)
    # at 4096 tokens the whole vocabulary's g^T is within the slab size: one slab
    assert fckl.workspace_size(fckl.make_desc(**C3), 4096) == fckl.workspace_size(
        fckl.make_desc(**C3, vocab_slab=VPAD3), 4096)
    # a slab set by the caller: 512 rows, the last slab takes the remainder (3 tiles)
    small = dict(N=3000, H=264, V=1800, K=20, T=1.0)
    one = fckl.workspace_size(fckl.make_desc(**small, vocab_slab=2048), 1024)
    two = fckl.workspace_size(fckl.make_desc(**small, vocab_slab=512), 1024)
    assert two < one
    # not a multiple of 256, or negative: refused before any HIP call
    for bad in (100, -256):
        with pytest.raises(fckl.FCKLError) as e:
            fckl.workspace_size(fckl.make_desc(**small, vocab_slab=bad), 1024)
        assert e.value.status == fckl.ERR_INVALID_ARG


def test_plan_explicit_chunk_and_small_budget():
    d = fckl.make_desc(**dict(C3, chunk=1000))
    chunk, ws = fckl.plan(d, 0)
    assert chunk == 1000 and ws == fckl.workspace_size(d, 1000)
    d = fckl.make_desc(**C3)
    with pytest.raises(fckl.FCKLError) as e:
        fckl.plan(d, 1 << 20)
    assert e.value.status == fckl.ERR_WORKSPACE
    # a small N plans a single chunk covering it
    chunk, _ = fckl.plan(fckl.make_desc(300, 256, 4096, 10, 1.0), 0)
    assert chunk == 512


@pytest.mark.parametrize("bad,status", [
    (dict(N=0), fckl.ERR_INVALID_ARG),
    (dict(T=0.0), fckl.ERR_INVALID_ARG),
    (dict(T=-1.0), fckl.ERR_INVALID_ARG),
    (dict(T=float("nan")), fckl.ERR_INVALID_ARG),
    (dict(T=float("inf")), fckl.ERR_INVALID_ARG),
    (dict(K=0), fckl.ERR_INVALID_ARG),
    (dict(K=5000, V=4096), fckl.ERR_INVALID_ARG),
    (dict(chunk=-3), fckl.ERR_INVALID_ARG),
    (dict(logit_dtype=7), fckl.ERR_INVALID_ARG),
    (dict(flags=64), fckl.ERR_INVALID_ARG),
    (dict(H=260), fckl.ERR_UNSUPPORTED),
    (dict(K=129), fckl.ERR_UNSUPPORTED),
    # past the kernels' 32-bit tile offsets (pitch 2^24) and grid sizes (2^23 tiles of 256 x 256)
    (dict(V=2 ** 24 + 1), fckl.ERR_UNSUPPORTED),
    (dict(V=2 ** 23, H=65536), fckl.ERR_UNSUPPORTED),
    (dict(N=2 ** 25, chunk=2 ** 24 + 1), fckl.ERR_UNSUPPORTED),
    (dict(N=2 ** 21, H=65536, chunk=2 ** 20), fckl.ERR_UNSUPPORTED),
])
def test_invalid_descriptions_rejected(bad, status):
    args = dict(N=512, H=256, V=4096, K=10, T=1.0)
    args.update(bad)
    d = fckl.make_desc(**args)
    with pytest.raises(fckl.FCKLError) as e:
        fckl.plan(d, 0)
    assert e.value.status == status


def test_limits_at_their_edges_are_planned():
    """The largest supported vocabulary and chunk sizes still plan (given the memory)."""
    budget = 1 << 44          # sizes only: W^T alone is 1.1 TB in the second case
    for args in (dict(N=512, H=256, V=2 ** 24, K=10),                  # 65536 x 1 tiles
                 dict(N=512, H=65536, V=(2 ** 23 - 1) // 256 * 256, K=10),  # 32767 x 256 tiles
                 dict(N=2 ** 20, H=8192, V=4096, K=10, chunk=2 ** 20)):     # C * H = 2^33
        d = fckl.make_desc(T=1.0, **args)
        chunk, ws = fckl.plan(d, budget)
        assert chunk >= 256 and ws > 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The tests below pass fake device addresses that every case must refuse before any HIP
# call.  On a machine with a GPU they are skipped, so that a check that regressed could
# never launch a kernel on those addresses.
fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="host-only check with fake device addresses")


@fake_addresses
def test_entry_points_reject_before_any_hip_call():
    """Null or misaligned pointers and a short workspace are refused up front.

    The pointers are never dereferenced: every case returns before a kernel launch,
    so this runs without a GPU.
    """
    lib = fckl.load()
    d = fckl.make_desc(512, 256, 4096, 10, 1.0, chunk=128)
    need = fckl.workspace_size(d, 128)
    P = 1 << 40  # a 256-aligned address that is never touched
    ok = [_fake(P), _fake(P), _fake(P), _fake(P)]
    # null input
    st = lib.fckl_forward(ctypes.byref(d), None, *ok[1:], _fake(P), _fake(P), None, _fake(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    # null outputs
    st = lib.fckl_forward(ctypes.byref(d), *ok, None, _fake(P), None, _fake(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_backward(ctypes.byref(d), *ok, _fake(P), ctypes.c_float(1.0), None, _fake(P), _fake(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    # misaligned workspace
    st = lib.fckl_forward(ctypes.byref(d), *ok, _fake(P), _fake(P), None, _fake(P + 8), need, None)
    assert st == fckl.ERR_INVALID_ARG
    # workspace too small
    st = lib.fckl_forward(ctypes.byref(d), *ok, _fake(P), _fake(P), None, _fake(P), need - 1, None)
    assert st == fckl.ERR_WORKSPACE
    st = lib.fckl_backward(ctypes.byref(d), *ok, _fake(P), ctypes.c_float(1.0), _fake(P), _fake(P), _fake(P),
                           need - 256, None)
    assert st == fckl.ERR_WORKSPACE
    # bad description through the entry point
    bad = fckl.make_desc(512, 256, 4096, 10, 0.0, chunk=128)
    st = lib.fckl_forward(ctypes.byref(bad), *ok, _fake(P), _fake(P), None, _fake(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_forward(None, *ok, _fake(P), _fake(P), None, _fake(P), need, None)
    assert st == fckl.ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    tl = torch.zeros(4, 2, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fckl.forward(h, W, idx, tl)


@fake_addresses
def test_weighted_and_single_call_entry_points_reject_before_any_hip_call():
    """The weighted passes and the single-call path check their arguments up front too."""
    lib = fckl.load()
    d = fckl.make_desc(512, 256, 4096, 10, 1.0, chunk=128)
    need = fckl.workspace_size(d, 128)
    P = 1 << 40
    ok = [_fake(P), _fake(P), _fake(P), _fake(P)]
    size = ctypes.c_size_t
    # fckl_forward_ex: weights may be NULL, outputs may not
    st = lib.fckl_forward_ex(ctypes.byref(d), *ok, None, None, _fake(P), None, _fake(P), size(need), None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_forward_ex(ctypes.byref(d), *ok, _fake(P), _fake(P), _fake(P), None, _fake(P), size(need - 1), None)
    assert st == fckl.ERR_WORKSPACE
    # fckl_backward_ex
    st = lib.fckl_backward_ex(ctypes.byref(d), *ok, None, _fake(P), ctypes.c_float(1.0), None, None, _fake(P),
                              _fake(P), size(need), None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_backward_ex(ctypes.byref(d), *ok, _fake(P), _fake(P), ctypes.c_float(1.0), None, _fake(P),
                              _fake(P), _fake(P + 8), size(need), None)
    assert st == fckl.ERR_INVALID_ARG
    # fckl_forward_backward: every output is required; its workspace (fckl_single_plan)
    # also holds the kept exponentials
    need = fckl.single_plan(d, 0)[1]
    args = [_fake(P)] * 5
    for missing in range(5):
        outs = list(args)
        outs[missing] = None
        if missing == 2:        # loss_mean may be NULL
            continue
        st = lib.fckl_forward_backward(ctypes.byref(d), *ok, None, ctypes.c_float(1.0), *outs, _fake(P), size(need),
                                       None)
        assert st == fckl.ERR_INVALID_ARG, missing
    st = lib.fckl_forward_backward(ctypes.byref(d), *ok, None, ctypes.c_float(1.0), *args, _fake(P), size(need - 256),
                                   None)
    assert st == fckl.ERR_WORKSPACE
    bad = fckl.make_desc(512, 256, 4096, 10, -1.0, chunk=128)
    st = lib.fckl_forward_backward(ctypes.byref(bad), *ok, None, ctypes.c_float(1.0), *args, _fake(P), size(need), None)
    assert st == fckl.ERR_INVALID_ARG


@fake_addresses
def test_noalloc_forward_rejects_before_any_hip_call():
    """fckl_forward_noalloc checks its arguments, and that the chunk's forward buffers fit
    the library's 64 MiB device array, before any HIP call (the addresses here are fake)."""
    lib = fckl.load()
    P = 1 << 40
    f = _fake
    d = fckl.make_desc(512, 256, 4096, 10, 1.0)
    ok = [f(P)] * 4
    for missing in (0, 1, 2, 3, 5, 6):     # h, W, idx, tl, loss_tok, lse (weights and loss_mean may be NULL)
        args = ok + [None, f(P), f(P), None]
        args[missing] = None
        assert lib.fckl_forward_noalloc(ctypes.byref(d), *args, None) == fckl.ERR_INVALID_ARG, missing
    assert lib.fckl_forward_noalloc(ctypes.byref(d), f(P + 8), *ok[1:], None, f(P), f(P), None,
                                    None) == fckl.ERR_INVALID_ARG
    bad = fckl.make_desc(512, 256, 4096, 10, 0.0)
    assert lib.fckl_forward_noalloc(ctypes.byref(bad), *ok, None, f(P), f(P), None, None) == fckl.ERR_INVALID_ARG
    # ~68 MB of forward buffers at 8192 tokens of a 201088-entry vocabulary: over the array
    big = fckl.make_desc(32768, 2880, 201088, 100, 1.0, chunk=8192)
    assert lib.fckl_forward_noalloc(ctypes.byref(big), *ok, None, f(P), f(P), None, None) == fckl.ERR_WORKSPACE
    # a vocabulary whose 256-token chunk alone does not fit
    huge = fckl.make_desc(1000, 64, 1 << 24, 10, 1.0)
    assert lib.fckl_forward_noalloc(ctypes.byref(huge), *ok, None, f(P), f(P), None, None) == fckl.ERR_WORKSPACE


@fake_addresses
def test_misaligned_pointers_are_refused():
    """h, W (and the teacher's h_t, W_t) are read and dH is written in 16-byte pieces: a
    pointer off that alignment is refused before any HIP call."""
    lib = fckl.load()
    d = fckl.make_desc(512, 256, 4096, 10, 1.0, chunk=128)
    need = ctypes.c_size_t(fckl.workspace_size(d, 128))
    P, odd = 1 << 40, (1 << 40) + 4
    f = _fake
    st = lib.fckl_forward(ctypes.byref(d), f(P + 8), f(P), f(P), f(P), f(P), f(P), None, f(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_forward(ctypes.byref(d), f(P), f(P + 8), f(P), f(P), f(P), f(P), None, f(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_backward(ctypes.byref(d), f(P), f(P), f(P), f(P), f(P), ctypes.c_float(1.0), f(odd), f(P), f(P),
                           need, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_backward_ex(ctypes.byref(d), f(P), f(P), f(P), f(P), None, f(P), ctypes.c_float(1.0), None,
                              f(odd), f(P), f(P), need, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_forward_backward(ctypes.byref(d), f(P), f(P), f(P), f(P), None, ctypes.c_float(1.0), f(P), f(P),
                                   None, f(odd), f(P), f(P), ctypes.c_size_t(fckl.single_plan(d, 0)[1]), None)
    assert st == fckl.ERR_INVALID_ARG
    # dW is written element by element: any 4-byte alignment is fine (the same call with an
    # aligned dH would only fail later, on the fake addresses, so it is not made here)
    small = fckl.make_desc(512, 256, 4096, 1, 1.0, chunk=256)
    _, fneed = fckl.full_plan(small, 384)
    for i_bad in (2, 3, 7):     # h_t, W_t, dH (after loss_tok, lse, loss_mean)
        args = [f(P)] * 4 + [f(P)] * 5
        args[i_bad] = f(odd)
        st = lib.fckl_full_forward_backward(ctypes.byref(small), 384, *args[:4], None, ctypes.c_float(1.0),
                                            *args[4:], f(P), ctypes.c_size_t(fneed), None)
        assert st == fckl.ERR_INVALID_ARG, i_bad


@fake_addresses
def test_full_teacher_plan_and_argument_checks():
    """fckl_full_plan: its workspace holds the teacher's fp32 logits of a chunk on top of the
    loss workspace, never depends on N, fits the budget; bad sizes are refused before any
    HIP call."""
    lib = fckl.load()
    d = fckl.make_desc(C3["N"], C3["H"], C3["V"], 1, 1.0)
    chunk, ws = fckl.full_plan(d, 2880)
    assert ws <= DEFAULT_BUDGET and chunk % 256 == 0
    base = fckl.workspace_size(fckl.make_desc(C3["N"], C3["H"], C3["V"], 1, 1.0), chunk)
    assert ws >= base + 4 * chunk * C3["V"]
    sizes = {fckl.full_plan(fckl.make_desc(N, 2880, 201088, 1, 1.0, 4096), 2880)[1] for N in (4096, 2 ** 31 - 1)}
    assert len(sizes) == 1
    # K and logit_dtype are not read
    d_any = fckl.make_desc(C3["N"], C3["H"], C3["V"], 0, 1.0, 0, 7)
    assert fckl.full_plan(d_any, 2880) == (chunk, ws)
    for Ht, status in ((12, fckl.ERR_UNSUPPORTED), (0, fckl.ERR_INVALID_ARG), (-8, fckl.ERR_INVALID_ARG),
                       (65544, fckl.ERR_UNSUPPORTED)):
        with pytest.raises(fckl.FCKLError) as e:
            fckl.full_plan(d, Ht)
        assert e.value.status == status, Ht
    with pytest.raises(fckl.FCKLError) as e:
        fckl.full_plan(d, 2880, budget_bytes=1 << 20)
    assert e.value.status == fckl.ERR_WORKSPACE
    small = fckl.make_desc(512, 256, 4096, 1, 1.0, chunk=256)
    _, need = fckl.full_plan(small, 384)
    P = 1 << 40
    ins = [_fake(P)] * 4
    outs = [_fake(P)] * 5
    size = ctypes.c_size_t
    for missing in range(9):
        args = ins + outs
        if missing == 6:        # loss_mean may be NULL
            continue
        args[missing] = None
        st = lib.fckl_full_forward_backward(ctypes.byref(small), 384, *args[:4], None, ctypes.c_float(1.0), *args[4:],
                                            _fake(P), size(need), None)
        assert st == fckl.ERR_INVALID_ARG, missing
    st = lib.fckl_full_forward_backward(ctypes.byref(small), 384, *ins, None, ctypes.c_float(1.0), *outs, _fake(P),
                                        size(need - 256), None)
    assert st == fckl.ERR_WORKSPACE
    st = lib.fckl_full_forward_backward(ctypes.byref(small), 384, *ins[:3], _fake(P + 8), None, ctypes.c_float(1.0),
                                        *outs, _fake(P), size(need), None)
    assert st == fckl.ERR_INVALID_ARG


def test_module_validates_arguments_without_a_gpu():
    import torch
    from chunked_top_kl_chunk_amd.loss import FusedChunkedKLLoss
    with pytest.raises(ValueError):
        FusedChunkedKLLoss(temperature=0.0)
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    tl = torch.zeros(4, 2, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        FusedChunkedKLLoss()(h, W, idx, tl)
    with pytest.raises(ValueError):
        fckl.forward_backward(h, W, idx, tl)


@fake_addresses
def test_topk_async_requires_a_status_word():
    lib = fckl.load()
    d = fckl.make_desc(512, 256, 4096, 10, 1.0)
    need = fckl.topk_workspace_size(d)
    P = 1 << 40
    st = lib.fckl_topk_async(ctypes.byref(d), _fake(P), _fake(P), _fake(P), _fake(P), _fake(P), ctypes.c_size_t(need),
                             None, None)
    assert st == fckl.ERR_INVALID_ARG
    st = lib.fckl_topk_async(ctypes.byref(d), _fake(P), _fake(P), _fake(P), _fake(P), _fake(P),
                             ctypes.c_size_t(need - 1), _fake(P), None)
    assert st == fckl.ERR_WORKSPACE


@fake_addresses
def test_scale_rejects_bad_arguments_before_any_hip_call():
    lib = fckl.load()
    P = 1 << 40
    assert lib.fckl_scale(None, 10, _fake(P), None) == fckl.ERR_INVALID_ARG
    assert lib.fckl_scale(_fake(P), 10, None, None) == fckl.ERR_INVALID_ARG
    assert lib.fckl_scale(_fake(P), -1, _fake(P), None) == fckl.ERR_INVALID_ARG
    assert lib.fckl_scale(_fake(P + 4), 10, _fake(P), None) == fckl.ERR_INVALID_ARG
    assert lib.fckl_scale(_fake(P), 0, _fake(P), None) == fckl.OK      # nothing to do: no launch


def test_missing_library_fails_loudly():
    """Without libfckl.so every entry point raises: there is no CPU or eager fallback."""
    saved_lib, saved_path = fckl._lib, fckl.LIB_PATH
    try:
        fckl._lib = None
        fckl.LIB_PATH = os.path.join(ROOT, "no-such-dir", "libfckl.so")
        d = fckl.make_desc(64, 64, 256, 4, 1.0)
        calls = [lambda: fckl.plan(d), lambda: fckl.single_plan(d), lambda: fckl.workspace_size(d, 256),
                 lambda: fckl.full_plan(d, 64),
                 lambda: fckl.topk_workspace_size(d), lambda: fckl.version(), lambda: fckl.load()]
        for call in calls:
            with pytest.raises(ImportError):
                call()
    finally:
        fckl._lib, fckl.LIB_PATH = saved_lib, saved_path


def test_product_code_does_not_reach_the_oracle():
    """The oracle is test infrastructure: nothing in the package or the C ABI names it."""
    pkg = os.path.join(ROOT, "chunked_top_kl_chunk_amd")
    files = [os.path.join(dp, f) for dp, _, fs in os.walk(pkg) for f in fs
             if f.endswith((".py", ".cpp", ".hip", ".h"))] + [HEADER]
    assert len(files) >= 6
    for path in files:
        text = open(path).read()
        assert not re.search(r"\boracle\b|fckl_oracle", text), path

"""ctypes loader for libpkv.so: argument and result types of every C entry point.

Loading fails loudly when the library has not been built; there is no
fallback implementation.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_OUT_OF_BLOCKS = 0, 1, 2, 3
PKV_ERR_REFCOUNT, PKV_ERR_HIP, PKV_ERR_WORKSPACE = 4, 5, 6
PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_INT8 = 0, 1, 2, 3, 4
PKV_ALGO_AUTO, PKV_ALGO_VECTOR, PKV_ALGO_MFMA = 0, 1, 2

P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
SZ, U64 = ctypes.c_size_t, ctypes.c_uint64

# name -> (restype, argtypes)
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_status_string": (ctypes.c_char_p, [I32]),
    "pkv_version": (I32, []),
    "pkv_set_stream_workgroups": (I32, [I32]),
    "pkv_kv_bytes_per_token": (U64, [I32, I32, I32, I32]),
    "pkv_paged_cache_append": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32, F32, P]),
    "pkv_decode_partition_size": (I32, [I32, I32, I32, I32, I32, I32, I32]),
    "pkv_decode_partition_size_for_lengths": (I32, [P, I32, I32, I32, I32, I32, I32]),
    "pkv_decode_workspace_size": (SZ, [I32, I32, I32, I32, I32, I32, I32]),
    "pkv_decode_algo_for": (I32, [I32, I32, I32, I32, I32]),
    "pkv_paged_decode_attention": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32,
                                         I32, I32, F32, F32, I32, P, SZ, P]),
    "pkv_paged_decode_attention_algo": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                              F32, I32, I32, F32, F32, I32, P, SZ, I32, P]),
    "pkv_paged_decode_attention_profiled": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                  I32, F32, I32, I32, F32, F32, I32, P, SZ, I32, P,
                                                  P, P, P]),
    "pkv_paged_decode_attention_appending": (I32, [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32,
                                                   I32, I32, I32, F32, I32, I32, F32, F32, I32, P,
                                                   SZ, I32, P, P, P, P]),
    "pkv_paged_decode_attention_noalloc": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                 I32, F32, I32, I32, F32, F32, I32, I32, P]),
    "pkv_multiquery_partition_size": (I32, [I32, I32, I32, I32, I32, I32]),
    "pkv_multiquery_partition_size_for_lengths": (I32, [P, I32, I32, I32, I32, I32, I32]),
    "pkv_multiquery_workspace_size": (SZ, [I32, I32, I32, I32, I32, I32, I32, I32]),
    "pkv_paged_multiquery_attention": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                             I32, I32, I32, F32, I32, I32, F32, F32, I32, P, SZ,
                                             P]),
    "pkv_paged_multiquery_attention_profiled": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                                      I32, I32, I32, I32, F32, I32, I32, F32, F32,
                                                      I32, P, SZ, P, P, P, P]),
    "pkv_paged_cache_append_per_channel": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                 I32, P, P, P]),
    "pkv_paged_decode_attention_per_channel": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                                     I32, I32, F32, I32, I32, P, P, I32, P, SZ,
                                                     I32, P, P, P, P]),
    "pkv_copy_blocks": (I32, [P, P, P, I32, I32, I64, P]),
    "pkv_swap_blocks": (I32, [P, P, I32, P, P, I32, P, I32, I64, P]),
    "pkv_stream_read_probe": (I32, [P, I64, P, I32, P, I32, P, P, P]),
    "pkv_seq_swap": (I32, [P, P, P, I32, P, P]),
    "pkv_seq_create_cached": (I32, [P, P, I32, P, I32, P, P]),
    "pkv_pool_register_blocks": (I32, [P, P, I32, P, I32]),
    "pkv_pool_cached_blocks": (I32, [P]),
    "pkv_pool_create": (I32, [I32, I32, P, ctypes.POINTER(P)]),
    "pkv_pool_destroy": (None, [P]),
    "pkv_pool_alloc": (I32, [P, P]),
    "pkv_pool_incref": (I32, [P, I32]),
    "pkv_pool_decref": (I32, [P, I32]),
    "pkv_pool_refcount": (I32, [P, I32]),
    "pkv_pool_num_free": (I32, [P]),
    "pkv_pool_num_blocks": (I32, [P]),
    "pkv_pool_block_size": (I32, [P]),
    "pkv_pool_free_list": (I32, [P, P, I32, P]),
    "pkv_seq_create": (I32, [P, I32, P, I32, P]),
    "pkv_seq_fork": (I32, [P, P, I32]),
    "pkv_seq_append_slots": (I32, [P, P, P, I32, I32, I32, P, P, I32, P]),
    "pkv_batch_append_slots": (I32, [P, P, I32, P, P, P, I32, P, P, I32, P, P]),
    "pkv_seq_free": (I32, [P, P, I32]),
}

_lib = None


class PkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"[{status}] {message}")
        self.status = status


class InvalidArg(PkvError):
    pass


class Unsupported(PkvError):
    pass


class OutOfBlocks(PkvError):
    pass


class RefcountError(PkvError):
    pass


class HipError(PkvError):
    pass


class WorkspaceError(PkvError):
    pass


_ERR = {PKV_ERR_INVALID_ARG: InvalidArg, PKV_ERR_UNSUPPORTED: Unsupported,
        PKV_ERR_OUT_OF_BLOCKS: OutOfBlocks, PKV_ERR_REFCOUNT: RefcountError,
        PKV_ERR_HIP: HipError, PKV_ERR_WORKSPACE: WorkspaceError}


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_363_amd.build`")
    l = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    _lib = l
    return l


def check(status):
    if status != PKV_OK:
        msg = lib().pkv_last_error().decode(errors="replace")
        raise _ERR.get(status, PkvError)(status, msg)

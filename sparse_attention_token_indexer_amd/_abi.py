"""ctypes signatures of libdsa_indexer.so's exported functions (argument
marshalling table of the binding; no torch import, so host-only tools can load
the library with the same signatures)."""
import ctypes

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

_SIGS = {
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_abi_version": ([], ctypes.c_int),
    "indexer_score_topk_workspace_size": ([_i32, _i32, _i32, _i32, _i64, _i32, _i32], _sz),
    "indexer_score_topk": ([_c_p, _c_p, _c_p, _i32, _c_p, _c_p, _i32, _i32, _i32, _i32, _i64, _i32,
                            _c_p, _c_p, _c_p, _sz, _c_p], ctypes.c_int),
    "indexer_score_topk_noalloc": ([_c_p, _c_p, _c_p, _i32, _c_p, _c_p, _i32, _i32, _i32, _i32,
                                    _i64, _i32, _c_p, _c_p, _c_p], ctypes.c_int),
    "indexer_certified_topk_workspace_size": ([_i32, _i32, _i32, _i32, _i64, _i32, _i32], _sz),
    "indexer_certified_topk": ([_c_p, _c_p, _c_p, _i32, _c_p, _c_p, _i32, _i32, _i32, _i32, _i64,
                                _i32, _i32, _c_p, _c_p, _c_p, _c_p, _sz, _c_p], ctypes.c_int),
    "indexer_mean_pool_keys": ([_c_p, _i32, _i32, _i64, _i32, _i32, _c_p, _c_p], ctypes.c_int),
    "misa_route_score_topk_workspace_size": ([_i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32,
                                              _i32], _sz),
    "misa_route_score_topk": ([_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _i32, _i32, _i32, _i32,
                               _i64, _i32, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                               _sz, _c_p], ctypes.c_int),
    "hisa_block_filter_topk_workspace_size": ([_i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                               _i32], _sz),
    "hisa_block_filter_topk": ([_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _i32, _i32, _i32, _i32,
                                _i64, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz,
                                _c_p], ctypes.c_int),
    "misa_hisa_topk_workspace_size": ([_i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _i32,
                                       _i32], _sz),
    "misa_hisa_topk": ([_c_p, _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _i32, _i32, _i32, _i32, _i64,
                        _i32, _i32, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                        _sz, _c_p], ctypes.c_int),
    "dsa_hisa_wait_limit": ([_i64], ctypes.c_int),
    "sparse_mla_workspace_size": ([_i32, _i32, _i32, _i32, _i32], _sz),
    "sparse_mla_attention": ([_c_p, _c_p, _i32, _c_p, _c_p, _c_p, _i32, _i32, _i32, _i32, _i32,
                              _i64, _i32, ctypes.c_float, _c_p, _c_p, _sz, _c_p], ctypes.c_int),
    "indexer_selection_iou": ([_c_p, _c_p, _i32, _i32, _c_p, _c_p], ctypes.c_int),
    "dsa_kernel_timing": ([ctypes.c_int], ctypes.c_int),
    "dsa_kernel_timing_read": ([_i32, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)],
                               ctypes.c_int),
}

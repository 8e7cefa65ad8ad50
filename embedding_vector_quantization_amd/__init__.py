"""TurboQuant online vector quantiser for AMD MI355X (gfx950).

The quantiser runs in the HIP kernels of libtq.so behind the C ABI of
include/tq.h; this package is its ctypes binding."""

from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, TQ_BF16, TQ_ERR_ALIGN, TQ_ERR_ARG, TQ_ERR_BITS, TQ_ERR_DIM,
    TQ_ERR_HIP, TQ_ERR_NOCONV, TQ_ERR_WORKSPACE, TQ_F16, TQ_F32, TQ_MSE, TQ_OK, TQ_PROD,
    Quantizer, SplitQuantizer, TQError, TqCodes, TqParams, decode, encode, lib, score, status_string,
    tq_decode, tq_encode_mse, tq_encode_prod, tq_attend, tq_attend_workspace, tq_make_codebook, tq_rht,
    tq_score, tq_score_accumulate, tq_score_grouped, tq_score_workspace, tq_topk, tq_topk_workspace,
)

// Host-only entry points of the library: the ABI version and the text of each
// status code.

#include "bsa_fp8.h"

extern "C" {

int bsa_fp8_abi_version(void) { return 4; }

const char* bsa_fp8_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case BSA_ERR_HEAD_DIM: return "head_dim must be 128";
    case BSA_ERR_PAGE_SIZE: return "page_size must be 32 or 64 (a decode cache: at least 1)";
    case BSA_ERR_GQA: return "num_heads_q must be a multiple of num_heads_kv with ratio 1..16";
    case BSA_ERR_QUANT_TYPE: return "unknown quant_type";
    case BSA_ERR_KV_LAYOUT: return "unknown kv_layout";
    case BSA_ERR_SIZE: return "a size is negative or inconsistent";
    case BSA_ERR_MASK_SHAPE: return "block_mask shape does not cover max_seqlen_q";
    case BSA_ERR_SOFTMAX_SCALE: return "softmax_scale must be finite (and not negative for the prefill)";
    case BSA_ERR_TOO_LARGE: return "problem exceeds a supported limit";
    case BSA_ERR_LAUNCH: return "kernel launch failed";
    case BSA_ERR_Q_LAYOUT: return "unknown q_layout";
    case BSA_ERR_P_SCALE: return "p_scale must be 0 (default 256) or in (0, 448]";
    case BSA_ERR_SPARSE_FORM: return "give block_mask or sparse_indices with sparse_seq_len, not both";
    case BSA_ERR_SCHEDULE: return "schedule_len must equal the task count";
    case BSA_ERR_SCALE_MODE: return "unknown scale_mode";
    case BSA_ERR_QK_PRECISION: return "unknown qk_precision";
    case BSA_ERR_SCRATCH: return "the partial results exceed the library's static decode scratch";
    default: return "unknown status";
  }
}

}  // extern "C"

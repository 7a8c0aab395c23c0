// Helpers shared by the prefill and the scheduling pre-pass: the rule that
// bounds the KV tiles a Q tile can see, and the host-side validation of the
// static arguments.
#ifndef BSA_INTERNAL_H
#define BSA_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "bsa_fp8.h"

namespace bsa {

constexpr int kTile = 128;
constexpr int kHeadDim = 128;
constexpr float kDefaultPScale = 256.0f;  // P-scale when none is given
constexpr float kMaxPScale = 448.0f;      // largest finite E4M3 value
constexpr int kFormDense = 0;             // no sparsity array: every candidate tile
constexpr int kFormMask = 1;              // uint8 block_mask
constexpr int kFormList = 2;              // sparse_indices + sparse_seq_len

// KV tiles 0 .. candidate_end-1 can hold a key that some query of Q tile m
// sees: below the KV length and, in causal mode (bottom-right aligned), at or
// below the largest query position lkv - lq + min(128m + 127, lq - 1).
__host__ __device__ __forceinline__ int candidate_end(int lq, int lkv, int m, int causal) {
  int n_end = (lkv + kTile - 1) / kTile;
  if (causal) {
    const int last = m * kTile + kTile - 1 < lq - 1 ? m * kTile + kTile - 1 : lq - 1;
    const int p_max = lkv - lq + last;
    n_end = p_max >= 0 ? (n_end < p_max / kTile + 1 ? n_end : p_max / kTile + 1) : 0;
  }
  return n_end;
}

// Static arguments after validation.
struct Resolved {
  bsa_fp8_dims d;
  int group;         // Hq / Hkv
  int mt_grid;       // ceil(max_seqlen_q / 128)
  int64_t tasks;     // B * Hq * mt_grid
  int form;          // kFormDense / kFormMask / kFormList
  const int32_t* sidx;
  const int32_t* slen;
  int q_layout;
  float p_scale;
  const int32_t* schedule;
  int qk;            // Q.K^T matrix path: BSA_QK_F16, BSA_QK_FP8 or BSA_QK_FP8_SPLIT
};

inline bool finite_float(float x) {
  uint32_t bits;
  memcpy(&bits, &x, sizeof(bits));
  return (bits & 0x7f800000u) != 0x7f800000u;
}

// Checks every static argument except the quantisation type, page size and
// data pointers.  Returns BSA_OK and fills `r`, or the first error found.
inline int resolve(const bsa_fp8_dims* dims, const uint8_t* block_mask, const bsa_fp8_options* opts,
                   Resolved* r) {
  if (dims == nullptr) return BSA_ERR_NULL_POINTER;
  const bsa_fp8_dims d = *dims;
  if (d.head_dim != kHeadDim) return BSA_ERR_HEAD_DIM;
  if (d.kv_layout != BSA_KV_NHD && d.kv_layout != BSA_KV_HND) return BSA_ERR_KV_LAYOUT;
  if (d.batch < 0 || d.total_q < 0 || d.num_pages < 0 || d.max_pages_per_seq < 0 ||
      d.max_seqlen_q < 0 || d.num_heads_q <= 0 || d.num_heads_kv <= 0)
    return BSA_ERR_SIZE;
  if (d.num_heads_q % d.num_heads_kv != 0) return BSA_ERR_GQA;
  if (d.num_heads_kv > 65536) return BSA_ERR_TOO_LARGE;  // page offsets are 32-bit
  const int group = d.num_heads_q / d.num_heads_kv;
  if (group < 1 || group > 16) return BSA_ERR_GQA;
  // The kernels keep the score constant strictly positive (a masked score of
  // -inf must turn into a probability of exactly 0), so a negative scale is
  // refused rather than silently clamped; 0 gives uniform weights.
  if (!finite_float(d.softmax_scale) || d.softmax_scale < 0.0f) return BSA_ERR_SOFTMAX_SCALE;
  if (d.causal != 0 && d.causal != 1) return BSA_ERR_SIZE;

  bsa_fp8_options o;
  memset(&o, 0, sizeof(o));
  if (opts != nullptr) o = *opts;
  if (o.q_layout != BSA_Q_TND && o.q_layout != BSA_Q_NTD) return BSA_ERR_Q_LAYOUT;
  float ps = o.p_scale;
  if (ps == 0.0f) ps = kDefaultPScale;
  if (!finite_float(ps) || !(ps > 0.0f) || ps > kMaxPScale) return BSA_ERR_P_SCALE;
  if ((o.sparse_indices == nullptr) != (o.sparse_seq_len == nullptr)) return BSA_ERR_SPARSE_FORM;
  if (o.sparse_indices != nullptr && block_mask != nullptr) return BSA_ERR_SPARSE_FORM;

  const int mt_grid = (d.max_seqlen_q + kTile - 1) / kTile;
  const int form = o.sparse_indices != nullptr ? kFormList : block_mask != nullptr ? kFormMask : kFormDense;
  if (form != kFormDense) {
    if (d.mask_tiles_q <= 0 || d.mask_tiles_kv <= 0) return BSA_ERR_MASK_SHAPE;
    if ((int64_t)d.mask_tiles_q * kTile < d.max_seqlen_q) return BSA_ERR_MASK_SHAPE;
    if (d.mask_tiles_kv > BSA_MAX_KV_TILES) return BSA_ERR_TOO_LARGE;
  }
  const int64_t tasks = (int64_t)d.batch * d.num_heads_q * mt_grid;
  if (tasks > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;
  if (o.schedule != nullptr && o.schedule_len != tasks) return BSA_ERR_SCHEDULE;
  if (o.qk_precision != BSA_QK_DEFAULT && o.qk_precision != BSA_QK_F16 && o.qk_precision != BSA_QK_FP8 &&
      o.qk_precision != BSA_QK_FP8_SPLIT)
    return BSA_ERR_QK_PRECISION;

  r->d = d;
  r->group = group;
  r->mt_grid = mt_grid;
  r->tasks = tasks;
  r->form = form;
  r->sidx = o.sparse_indices;
  r->slen = o.sparse_seq_len;
  r->q_layout = o.q_layout;
  r->p_scale = ps;
  r->schedule = o.schedule;
  r->qk = o.qk_precision == BSA_QK_DEFAULT ? BSA_QK_FP8_SPLIT : o.qk_precision;
  return BSA_OK;
}

}  // namespace bsa

#endif  // BSA_INTERNAL_H

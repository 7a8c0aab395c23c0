// FP8 (E4M3) quantisation of the prefill's inputs, gfx950: Q rows with their
// per-(token, head) descales, and the chunk's K and V rows appended to the
// paged cache at the tail of every sequence.
//
// Method (FlashMLA FP8 KV-cache article, "Quant/dequant source"): a row of 128
// values gets the descale d = amax / 448, optionally rounded up to a power of
// two, and each value is stored as E4M3(x / d).  Rows whose descale is given
// (K for quant type 0, V for both types) use it in the same formula.  The
// descale is an IEEE float32 division and every quotient x / d equals the
// correctly rounded float32 one (computed from one reciprocal per row, see
// encode8), the E4M3 rounding is to nearest even and saturates at 448, so
// every code and descale is a pure function of the bfloat16 input.
//
// One row per 16 lanes: each lane loads 8 bfloat16 values (16 bytes), the row
// maximum is reduced over the 16 lanes with cross-lane shuffles, and each lane
// stores its 8 codes (8 bytes).  Each 16-lane group handles four rows, whose
// loads are all issued before the first is used, so that enough bytes are in
// flight per CU to cover the memory latency; a workgroup of 256 threads covers
// 64 rows (at each of the four steps its 16 groups take 16 consecutive rows,
// so every load instruction of a wave reads 1 KB of contiguous input).  The
// grid covers the Q rows, then the K rows, then the V rows.  The whole kernel
// streams HBM: 256 bytes read and 128 (+4) written per row, each touched once,
// so inputs and codes use non-temporal loads and stores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_fp8.h"
#include "bsa_internal.h"

namespace {

using bsa::kHeadDim;

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kGroups = kThreads / kLanesPerRow;  // 16-lane groups per workgroup
constexpr int kRowSteps = 4;                       // rows per group
constexpr int kRowsPerBlock = kGroups * kRowSteps;
constexpr float kFp8Max = 448.0f;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

struct QuantParams {
  const uint16_t* q_in;   // bf16 [T, Hq, 128]
  const uint16_t* k_in;   // bf16 [T, Hkv, 128]
  const uint16_t* v_in;   // bf16 [T, Hkv, 128]
  const int32_t* cu_q;
  const int32_t* seqlens_kv;
  const int32_t* block_table;
  const float* kscale;    // quant 0: [1]
  const float* vscale;    // [1] or [Hkv]
  uint8_t* q_out;
  float* qscale_out;
  uint8_t* kc;
  uint8_t* vc;
  float* kscale_cache;    // quant 1: cache-shaped, no head dimension
  int64_t rows_q, rows_kv;  // T*Hq (0 without Q), T*Hkv (0 without K/V)
  int B, Hkv, quant, pow2;
  int page_size, page_shift, max_pages;
  uint32_t page_bytes;
  int slot_stride, head_stride;
};

// Smallest power of two >= d, for a positive finite float (exact).
__device__ __forceinline__ float round_up_pow2(float d) {
  const uint32_t u = __float_as_uint(d);
  const uint32_t e = u >> 23;
  const uint32_t m = u & 0x7fffffu;
  if (e == 0) {  // subnormal: m * 2^-149
    uint32_t p = 1;
    while (p < m) p <<= 1;
    return __uint_as_float(p);  // p == 2^23 is 2^-126, the smallest normal
  }
  return m == 0 ? d : __uint_as_float((e + 1) << 23);
}

// E4M3 codes of fp32(x[i] / d), packed little-endian into two dwords.
//
// For descales in [2^-80, 2^100] the quotients come from one reciprocal per
// row instead of eight divisions: with r = 1/d correctly rounded and
// q0 = RN(x*r) within an ulp of x/d, the remainder x - q0*d is exact in one
// fma and RN(q0 + remainder*r) is the correctly rounded x/d (Markstein's
// theorem for quotients; the range keeps the remainder of every x whose
// quotient reaches the E4M3 grid clear of underflow).  q0 is first clamped to
// [-1024, 1024]: a quotient beyond that saturates to 448 whatever its rounding,
// and the clamp keeps the remainder finite.  The sign is taken from x so that
// -0 stays -0.  tests/quotient_check.c compares the resulting codes with those
// of the IEEE quotient for every descale amax/448 and every bfloat16 x.  Other
// descales use IEEE division per value.
__device__ __forceinline__ v2i encode8(const float* x, float d) {
  float y[8];
  if (d >= 0x1p-80f && d <= 0x1p100f) {
    const float r = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = __builtin_amdgcn_fmed3f(x[i] * r, -1024.0f, 1024.0f);
      const float q = fmaf(fmaf(-q0, d, x[i]), r, q0);
      y[i] = __builtin_amdgcn_fmed3f(copysignf(q, x[i]), -kFp8Max, kFp8Max);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fmaxf(fminf(x[i] / d, kFp8Max), -kFp8Max);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], __builtin_nondeterministic_value(0), false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], __builtin_nondeterministic_value(0), false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return v2i{lo, hi};
}

// Which part a row belongs to (0 = Q, 1 = K, 2 = V) and its index there.
__device__ __forceinline__ int split_row(const QuantParams& p, int64_t row, int64_t* r) {
  if (row < p.rows_q) {
    *r = row;
    return 0;
  }
  if (row < p.rows_q + p.rows_kv) {
    *r = row - p.rows_q;
    return 1;
  }
  *r = row - p.rows_q - p.rows_kv;
  return 2;
}

__device__ __forceinline__ void quantize_row(const QuantParams& p, int part, int64_t r, int sub, v4i raw) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
    x[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xffff0000u);
  }

  // Descale: computed from the row maximum (Q; K of quant type 1) or given.
  float d;
  const bool computed = part == 0 || (part == 1 && p.quant == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD);
  const int g = part == 0 ? 0 : (int)(r % p.Hkv);
  if (computed) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int m = 1; m < kLanesPerRow; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kLanesPerRow));
    d = amax == 0.0f ? 1.0f : amax / kFp8Max;
    if (p.pow2) d = round_up_pow2(d);
  } else if (part == 1) {
    d = p.kscale[0];
  } else {
    d = p.quant == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD ? p.vscale[g] : p.vscale[0];
  }
  const v2i codes = encode8(x, d);

  if (part == 0) {
    __builtin_nontemporal_store(codes, reinterpret_cast<v2i*>(p.q_out + r * kHeadDim + sub * 8));
    if (sub == 0) p.qscale_out[r] = d;
    return;
  }
  // Token t of the chunk belongs to the sequence b with cu_q[b] <= t < cu_q[b+1]
  // (binary search; empty sequences are skipped by the strict upper bound) and
  // goes to position Lkv_b - Lq_b + (t - cu_q[b]) of that sequence.
  const int t = (int)(r / p.Hkv);
  int lo = 0, hi = p.B;  // invariant: cu_q[lo] <= t < cu_q[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cu_q[mid] <= t) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int t0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - t0;
  const int pos = p.seqlens_kv[b] - lq + (t - t0);
  const int page = p.block_table[(int64_t)b * p.max_pages + (pos >> p.page_shift)];
  const int slot = pos & (p.page_size - 1);
  const uint32_t in_page = (uint32_t)(slot * p.slot_stride + g * p.head_stride);
  uint8_t* dst = (part == 1 ? p.kc : p.vc) + (uint64_t)(uint32_t)page * p.page_bytes + in_page * kHeadDim;
  __builtin_nontemporal_store(codes, reinterpret_cast<v2i*>(dst + sub * 8));
  if (part == 1 && computed && sub == 0)
    p.kscale_cache[(uint64_t)(uint32_t)page * (p.page_bytes / kHeadDim) + in_page] = d;
}

__global__ void __launch_bounds__(kThreads) bsa_fp8_quantize_kernel(QuantParams p) {
  const int sub = threadIdx.x & (kLanesPerRow - 1);
  const int grp = threadIdx.x >> 4;
  const int64_t total = p.rows_q + 2 * p.rows_kv;
  const int64_t base = (int64_t)blockIdx.x * kRowsPerBlock + grp;
  // All four loads first; a row past the end is skipped by its whole group.
  v4i raw[kRowSteps];
  int part[kRowSteps];
  int64_t r[kRowSteps];
#pragma unroll
  for (int j = 0; j < kRowSteps; ++j) {
    const int64_t row = base + j * kGroups;
    part[j] = split_row(p, row < total ? row : 0, &r[j]);
    const uint16_t* src = part[j] == 0 ? p.q_in : (part[j] == 1 ? p.k_in : p.v_in);
    raw[j] = row < total ? __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + r[j] * kHeadDim + sub * 8)) : v4i{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < kRowSteps; ++j)
    if (base + j * kGroups < total) quantize_row(p, part[j], r[j], sub, raw[j]);
}

}  // namespace

extern "C" {

int bsa_fp8_quantize_append(const void* q_in, const void* k_in, const void* v_in,
                            const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                            const int32_t* block_table, const float* kscale, const float* vscale,
                            int quant_type, int page_size, int scale_mode, const bsa_fp8_dims* dims,
                            void* q_out, float* qscale_out, void* kcache, void* vcache,
                            float* kscale_cache, void* stream) {
  bsa::Resolved r;
  const int st = bsa::resolve(dims, nullptr, nullptr, &r);
  if (st != BSA_OK) return st;
  if (page_size != 32 && page_size != 64) return BSA_ERR_PAGE_SIZE;
  if (quant_type != BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR &&
      quant_type != BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD)
    return BSA_ERR_QUANT_TYPE;
  if (scale_mode != BSA_SCALE_AMAX && scale_mode != BSA_SCALE_AMAX_POW2) return BSA_ERR_SCALE_MODE;
  if ((k_in == nullptr) != (v_in == nullptr)) return BSA_ERR_NULL_POINTER;
  const bsa_fp8_dims& d = r.d;
  const int64_t rows_q = q_in != nullptr ? (int64_t)d.total_q * d.num_heads_q : 0;
  const int64_t rows_kv = k_in != nullptr ? (int64_t)d.total_q * d.num_heads_kv : 0;
  const int64_t total = rows_q + 2 * rows_kv;
  if ((total + kRowsPerBlock - 1) / kRowsPerBlock > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;
  if (rows_q > 0 && (q_out == nullptr || qscale_out == nullptr)) return BSA_ERR_NULL_POINTER;
  if (rows_kv > 0) {
    if (cu_seqlens_q == nullptr || seqlens_kv == nullptr || block_table == nullptr ||
        kcache == nullptr || vcache == nullptr || vscale == nullptr)
      return BSA_ERR_NULL_POINTER;
    if (quant_type == BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR && kscale == nullptr) return BSA_ERR_NULL_POINTER;
    if (quant_type == BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD && kscale_cache == nullptr)
      return BSA_ERR_NULL_POINTER;
    if (d.batch <= 0) return BSA_ERR_SIZE;
  }
  if (total == 0) return BSA_OK;

  QuantParams p;
  p.q_in = static_cast<const uint16_t*>(q_in);
  p.k_in = static_cast<const uint16_t*>(k_in);
  p.v_in = static_cast<const uint16_t*>(v_in);
  p.cu_q = cu_seqlens_q;
  p.seqlens_kv = seqlens_kv;
  p.block_table = block_table;
  p.kscale = kscale;
  p.vscale = vscale;
  p.q_out = static_cast<uint8_t*>(q_out);
  p.qscale_out = qscale_out;
  p.kc = static_cast<uint8_t*>(kcache);
  p.vc = static_cast<uint8_t*>(vcache);
  p.kscale_cache = kscale_cache;
  p.rows_q = rows_q;
  p.rows_kv = rows_kv;
  p.B = d.batch;
  p.Hkv = d.num_heads_kv;
  p.quant = quant_type;
  p.pow2 = scale_mode == BSA_SCALE_AMAX_POW2;
  p.page_size = page_size;
  p.page_shift = page_size == 64 ? 6 : 5;
  p.max_pages = d.max_pages_per_seq;
  p.page_bytes = (uint32_t)page_size * (uint32_t)d.num_heads_kv * kHeadDim;
  p.slot_stride = d.kv_layout == BSA_KV_NHD ? d.num_heads_kv : 1;
  p.head_stride = d.kv_layout == BSA_KV_NHD ? 1 : page_size;

  const unsigned blocks = (unsigned)((total + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(bsa_fp8_quantize_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_LAUNCH;
  return BSA_OK;
}

}  // extern "C"
